// Top-k selection: per query head, the k largest scores, lowest index among
// equal scores, returned in ascending index order (ai-feeds digest, Method /
// key module 5 and Output: the scan outputs top-k key indices per query).
//
// Scores are mapped to order-preserving 32-bit keys
//   key(f) = f >= +0 ? bits | 0x80000000 : ~bits      (-0 folded onto +0)
// and everything after that is integer work, with two passes over the scores.
// The head histograms and the per-head state start at zero: cleared by the
// scan that writes the scores, or by sel_init.
//   1. hist     LDS histogram of the top 12 key bits per 4096-key chunk, added
//               to the head's histogram (or built by the scan itself);
//   2. collect  every workgroup finds, from its head's histogram, the bin b
//               holding the k-th largest key; every key of its 4096-key chunk in
//               bin b or above is written, as (key, index), to the chunk's slot
//               in index order (ballot ranks per wavefront, no atomics), with the
//               slot's count;
//   3. resolve  one workgroup per head concatenates the slots in chunk order in
//               LDS -- all kept keys, in index order -- radix-selects the exact
//               k-th key T among them (10 + 10 more bits) and how many keys equal
//               to T still belong to the top k, and compacts in order: keys above
//               T and the lowest-index keys equal to T.  No sorting is needed.
// A chunk whose kept keys overflow its slot writes them, still in index order,
// to a segment of its head's spill area (claimed with one atomic), so kept keys
// concentrated in a few chunks stay on the fast path.  A head whose candidates
// (the keys in bin b or above) exceed the resolve's LDS buffer (16384) is known
// from the histogram: in rows of 262144 keys or more the collect counts its bin
// b keys by their next 10 bits and a recollect keeps the keys whose top 22 bits
// reach the refined threshold; otherwise, or if those still overflow, the
// resolve takes an exact in-order fallback: radix passes over the whole row
// find T, then one ordered pass writes the selection.  Rows of at most 16384
// keys skip all of this: sel_small selects each in LDS in one launch.
#include <algorithm>

#include "fathom_internal.h"
#include "select_parts.h"

namespace fathom {
namespace {

using namespace sel;


__global__ __launch_bounds__(kSelThreads) void sel_init(uint32_t* hist, uint32_t* state, uint32_t* hist2) {
  const int h = blockIdx.x;
  for (int b = threadIdx.x; b < kBins; b += kSelThreads) hist[(int64_t)h * kBins + b] = 0u;
  if (threadIdx.x < kStateWords) state[h * kStateWords + threadIdx.x] = 0u;
  if (hist2)
    for (int b = threadIdx.x; b < k2ndBins; b += kSelThreads) hist2[(int64_t)h * k2ndBins + b] = 0u;
}

// First-digit histogram of `per` consecutive chunks per workgroup (long rows
// take several, so that fewer workgroups flush their bins to the global one).
__global__ __launch_bounds__(kSelThreads) void sel_hist(const float* __restrict__ scores, int64_t ld,
                                                        int64_t n, uint32_t* __restrict__ hist, int per) {
  __shared__ uint32_t lh[kBins];
  const int h = blockIdx.y;
  for (int b = threadIdx.x; b < kBins; b += kSelThreads) lh[b] = 0u;
  __syncthreads();
  const float* row = scores + (int64_t)h * ld;   // rows are 256-byte aligned, padded to 64 keys
  for (int sc = 0; sc < per; ++sc) {
    const int64_t j0 = ((int64_t)blockIdx.x * per + sc) * kChunk;
    if (j0 >= n) break;
    // 16-byte loads: thread t counts keys j0 + 4 (t + 256 i) + e (the order does not matter here)
    constexpr int kQuads = kPerThread / 4;
    float4 v[kQuads];
#pragma unroll
    for (int i = 0; i < kQuads; ++i) {
      const int64_t j = j0 + 4 * ((int64_t)i * kSelThreads + threadIdx.x);
      v[i] = j < n ? *reinterpret_cast<const float4*>(row + j) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < kQuads; ++i) {
      const int64_t j = j0 + 4 * ((int64_t)i * kSelThreads + threadIdx.x);
      const float e4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (j + e < n) atomicAdd(&lh[order_key(e4[e]) >> kDigit0], 1u);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += kSelThreads) {
    const uint32_t v = lh[b];
    if (v) atomicAdd(&hist[(int64_t)h * kBins + b], v);
  }
}

// The 16-byte loads of chunk c of a row (rows are 256-byte aligned and padded
// to 64 keys, so a quad that starts inside the row is readable whole).
template <int NQ>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int64_t n, int64_t c, float4 (&f)[NQ]) {
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int64_t j = c * kChunk + 4 * ((int64_t)i * kSelThreads + threadIdx.x);
    f[i] = j < n ? *reinterpret_cast<const float4*>(row + j) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// One pass over the scores: the keys of a chunk in bin b or above go to the
// chunk's slot (compact_chunk).  Every workgroup finds b itself from the head's
// histogram (read while its own scores are in flight); the first chunk's
// records it for the resolve.  With hist2 (rows long enough for the refinement
// stage), each workgroup also clears its slice of the head's second-digit
// histogram.
__global__ __launch_bounds__(kSelThreads) void sel_collect(const float* __restrict__ scores, int64_t ld,
                                                           int64_t n, int k, const uint32_t* __restrict__ hist,
                                                           uint32_t* __restrict__ state,
                                                           uint64_t* __restrict__ kept,
                                                           uint32_t* __restrict__ counts,
                                                           uint32_t* __restrict__ soff,
                                                           uint64_t* __restrict__ spill, int64_t spill_cap,
                                                           int64_t nchunks, uint32_t* __restrict__ hist2) {
  constexpr int NW = kSelThreads / 64;
  constexpr int kPer = kBins / kSelThreads;   // 16 bins per thread
  constexpr int kQuads = kPerThread / 4;
  __shared__ uint32_t cnt[kQuads][NW];
  __shared__ uint64_t* dst_sh;
  __shared__ uint32_t cap_sh;
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t sh[2];
  __shared__ uint32_t lh2[k2ndBins];
  const int h = blockIdx.y;
  const float* row = scores + (int64_t)h * ld;
  float4 f[kQuads];
  load_chunk(row, n, blockIdx.x, f);
  // bin b of the k-th largest key
  {
    const uint32_t* hh = hist + (int64_t)h * kBins;
    uint32_t hv[kPer];
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      hv[i] = hh[threadIdx.x * kPer + i];
      mine += hv[i];
    }
    uint32_t above = block_suffix_inclusive<kSelThreads>(mine, wsum) - mine;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) {
      if (above < (uint32_t)k && above + hv[i] >= (uint32_t)k) {
        sh[0] = threadIdx.x * kPer + i;
        sh[1] = above;
      }
      above += hv[i];
    }
    __syncthreads();
  }
  const uint32_t bin = sh[0];
  uint32_t* st = state + h * kStateWords;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    st[0] = bin;
    st[1] = sh[1];
  }
  if (sh[1] + hist[(int64_t)h * kBins + bin] > (uint32_t)kKeep) {
    // more candidates than the resolve holds: nothing to compact.  Rows long
    // enough for the refinement stage count the chunk's keys of bin b by their
    // next 10 bits instead (the recollect's histogram); shorter rows take the
    // resolve's full-row path.
    if (blockIdx.x == 0 && threadIdx.x == 0) st[2] = 1u;
    if (hist2) {
      uint32_t* lh = reinterpret_cast<uint32_t*>(lh2);
      for (int b = threadIdx.x; b < k2ndBins; b += kSelThreads) lh[b] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kQuads; ++i) {
        const int64_t j = (int64_t)blockIdx.x * kChunk + 4 * ((int64_t)i * kSelThreads + threadIdx.x);
        const float e4[4] = {f[i].x, f[i].y, f[i].z, f[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = order_key(e4[e]);
          if (j + e < n && (key >> kDigit0) == bin) atomicAdd(&lh[(key >> 10) & (k2ndBins - 1)], 1u);
        }
      }
      __syncthreads();
      for (int b = threadIdx.x; b < k2ndBins; b += kSelThreads) {
        const uint32_t v = lh[b];
        if (v) atomicAdd(&hist2[h * k2ndBins + b], v);
      }
    }
    return;
  }
  compact_chunk<NW>(f, n, (int64_t)blockIdx.x * kChunk, kDigit0, bin, &st[3], &st[2],
                    (int64_t)h * nchunks + blockIdx.x, kept, counts, soff, spill + (int64_t)h * spill_cap, spill_cap,
                    cnt, &dst_sh, &cap_sh);
}

// Refinement stage, for long rows whose first-digit bin b holds more candidates
// than the resolve keeps on chip (scores in a narrow band: one or two bins of
// 1/8 octave): the collect has counted the keys of bin b by their next 10 bits;
// here the second digit b2 of the k-th key comes from that histogram, then
// every chunk's keys whose top 22 bits are at least (b, b2) are compacted
// (compact_chunk, with the state's second spill counter and flag).  The first
// chunk's workgroup records b2 (marked refined) and the keys of bin b above it
// for the resolve.  Heads without that need return at once.
__global__ __launch_bounds__(kSelThreads) void sel_recollect(const float* __restrict__ scores, int64_t ld,
                                                             int64_t n, int k, const uint32_t* __restrict__ hist,
                                                             uint32_t* __restrict__ state,
                                                             const uint32_t* __restrict__ hist2,
                                                             uint64_t* __restrict__ kept,
                                                             uint32_t* __restrict__ counts,
                                                             uint32_t* __restrict__ soff,
                                                             uint64_t* __restrict__ spill, int64_t spill_cap,
                                                             int64_t nchunks, int per) {
  constexpr int NW = kSelThreads / 64;
  constexpr int kPer = k2ndBins / kSelThreads;   // 4 bins per thread
  constexpr int kQuads = kPerThread / 4;
  __shared__ uint32_t cnt[kQuads][NW];
  __shared__ uint64_t* dst_sh;
  __shared__ uint32_t cap_sh;
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t sh[2];
  const int h = blockIdx.y;
  uint32_t* st = state + h * kStateWords;
  const uint32_t bin = st[0];
  const uint32_t above = st[1];
  if (above + hist[(int64_t)h * kBins + bin] <= (uint32_t)kKeep) return;
  const float* row = scores + (int64_t)h * ld;
  const int64_t c0 = (int64_t)blockIdx.x * per;
  const int64_t c1 = min<int64_t>(c0 + per, nchunks);
  float4 f[kQuads];
  load_chunk(row, n, c0, f);
  {
    const uint32_t need = (uint32_t)k - above;
    uint32_t hv[kPer];
    uint32_t mine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      hv[i] = hist2[h * k2ndBins + threadIdx.x * kPer + i];
      mine += hv[i];
    }
    uint32_t ab = block_suffix_inclusive<kSelThreads>(mine, wsum) - mine;
#pragma unroll
    for (int i = kPer - 1; i >= 0; --i) {
      if (ab < need && ab + hv[i] >= need) {
        sh[0] = threadIdx.x * kPer + i;
        sh[1] = ab;
      }
      ab += hv[i];
    }
    __syncthreads();
  }
  const uint32_t b2 = sh[0];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    st[4] = b2 | kRefined;
    st[5] = sh[1];
  }
  for (int64_t c = c0; c < c1; ++c) {
    if (c > c0) {
      __syncthreads();   // the previous chunk's counts and destination are read
      load_chunk(row, n, c, f);
    }
    compact_chunk<NW>(f, n, c * kChunk, 10, (bin << 10) | b2, &st[7], &st[6], (int64_t)h * nchunks + c, kept, counts,
                      soff, spill + (int64_t)h * spill_cap, spill_cap, cnt, &dst_sh, &cap_sh);
  }
}

// Streams wavefront w's contiguous part of a row -- the w-th of NW parts, each a
// multiple of 256 keys -- in sweeps of 256 keys, lane l taking keys 4l .. 4l+3 of
// each (so lane-major order within a sweep is index order), U sweeps of loads in
// flight.  f(j, v, valid) gets a lane's first key index, its 4 scores and how
// many of them lie in the row.
template <int NW, class Fn>
__device__ __forceinline__ void stream_part(const float* __restrict__ row, int64_t n, Fn&& f) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t seg = ((n + NW - 1) / NW + 255) / 256 * 256;
  const int64_t j_lo = (int64_t)w * seg;
  const int64_t j_hi = min(n, j_lo + seg);
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  for (int64_t s0 = j_lo; s0 < j_hi; s0 += 256 * U) {
    float v[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = s0 + 256 * u + 4 * lane;
      if (vec && j + 3 < j_hi) {
        const float4 x = *reinterpret_cast<const float4*>(row + j);
        v[u][0] = x.x;
        v[u][1] = x.y;
        v[u][2] = x.z;
        v[u][3] = x.w;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[u][i] = j + i < j_hi ? row[j + i] : 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = s0 + 256 * u + 4 * lane;
      const int valid = (int)max<int64_t>(0, min<int64_t>(4, j_hi - j));
      f(j, v[u], valid);
    }
  }
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  const uint32_t b = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(b);
}

// Exact in-order selection of one head from its whole row by one workgroup:
// the path for heads whose kept keys do not fit the on-chip buffer (keys
// concentrated in one chunk beyond the spill area, or a first-digit bin that
// holds too many of them, e.g. massive ties or scores far from zero).  The
// threshold bin b and the keys above it come from the head's histogram; two
// passes over the row count the keys of bin b by their next 10, then last 10
// bits and give the exact k-th key T; then each wavefront counts, over its own
// part of the row, the keys above T and equal to T, and a second pass writes the
// keys above T and the first `need` keys equal to T in index order.  Barriers:
// a handful in all, none per sweep.
__device__ void resolve_row(const float* __restrict__ row, int64_t n, int k, uint32_t bin, uint32_t above,
                            int32_t* __restrict__ out, float* __restrict__ outv, uint32_t* lh, uint32_t* wsum,
                            uint32_t* sh) {
  constexpr int NT = kResolveThreads;
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t prefix = bin, need = (uint32_t)k - above;
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 10 : 0;
    const int hi_shift = pass == 0 ? kDigit0 : 10;
    lh[threadIdx.x] = 0u;
    __syncthreads();
    stream_part<NW>(row, n, [&](int64_t, const float (&v)[4], int valid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t key = order_key(v[i]);
        const bool act = i < valid && (key >> hi_shift) == prefix;
        const uint32_t b = (key >> shift) & 1023u;
        // one atomic for the wavefront when all its keys share a bin (ties)
        const uint64_t m = __ballot(act);
        if (m == 0ull) continue;
        const int leader = __builtin_ctzll(m);
        const uint32_t lb = (uint32_t)__shfl((int)b, leader, 64);
        if (__ballot(act && b == lb) == m) {
          if (lane == leader) atomicAdd(&lh[lb], (uint32_t)__popcll(m));
        } else if (act) {
          atomicAdd(&lh[b], 1u);
        }
      }
    });
    __syncthreads();
    find_bin<NT, 1024>(lh, need, wsum, sh);
    prefix = (prefix << 10) | sh[0];
    need -= sh[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  // per wavefront: keys above T and equal to T in its part
  uint32_t gt = 0, eq = 0;
  stream_part<NW>(row, n, [&](int64_t, const float (&v)[4], int valid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t key = order_key(v[i]);
      gt += (uint32_t)__popcll(__ballot(i < valid && key > T));
      eq += (uint32_t)__popcll(__ballot(i < valid && key == T));
    }
  });
  uint32_t* wgt = lh;          // the histogram is no longer needed
  uint32_t* weq = lh + NW;
  if (lane == 0) {
    wgt[w] = gt;
    weq[w] = eq;
  }
  __syncthreads();
  uint32_t pos = 0, ties = 0;
  for (int x = 0; x < w; ++x) {
    pos += wgt[x];
    ties += weq[x];
  }
  pos += min(ties, need);
  // ordered writes: ranks from ballots, lane-major within a sweep
  stream_part<NW>(row, n, [&](int64_t j, const float (&v)[4], int valid) {
    uint32_t key[4];
    uint64_t mg[4], me[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      key[i] = order_key(v[i]);
      mg[i] = __ballot(i < valid && key[i] > T);
      me[i] = __ballot(i < valid && key[i] == T);
    }
    if (((mg[0] | mg[1] | mg[2] | mg[3]) | (me[0] | me[1] | me[2] | me[3])) == 0ull) return;
    uint32_t rank = ties;   // equal keys before this lane's first key
#pragma unroll
    for (int i = 0; i < 4; ++i) rank += (uint32_t)__popcll(me[i] & lt);
    bool take[4];
    uint64_t mt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool e = (me[i] >> lane) & 1ull;
      take[i] = ((mg[i] >> lane) & 1ull) || (e && rank < need);
      if (e) ++rank;
      mt[i] = __ballot(take[i]);
    }
    uint32_t p = pos;
#pragma unroll
    for (int i = 0; i < 4; ++i) p += (uint32_t)__popcll(mt[i] & lt);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (take[i]) {
        if (p < (uint32_t)k) {
          out[p] = (int32_t)(j + i);
          if (outv) outv[p] = v[i];
        }
        ++p;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pos += (uint32_t)__popcll(mt[i]);
      ties += (uint32_t)__popcll(me[i]);
    }
  });
}


__global__ __launch_bounds__(kResolveThreads) void sel_resolve(const float* __restrict__ scores, int64_t ld,
                                                               int64_t n, int k,
                                                               const uint32_t* __restrict__ state,
                                                               const uint64_t* __restrict__ kept,
                                                               const uint32_t* __restrict__ counts,
                                                               const uint32_t* __restrict__ soff,
                                                               const uint64_t* __restrict__ spill, int64_t spill_cap,
                                                               int64_t nchunks, int32_t* __restrict__ idx,
                                                               float* __restrict__ val) {
  constexpr int NT = kResolveThreads;
  __shared__ uint64_t buf[kKeep];          // kept (key, index) of the head, in index order
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t coff[kResolveThreads + 1];   // offsets of the chunk slots in buf
  __shared__ uint32_t wsum[NT / 64];
  __shared__ uint32_t sh[2];
  const int h = blockIdx.x;
  const float* row = scores + (int64_t)h * ld;
  int32_t* out = idx + (int64_t)h * k;
  float* outv = val ? val + (int64_t)h * k : nullptr;
  const uint32_t* st = state + h * kStateWords;
  const uint32_t bin = st[0];
  const uint32_t above = st[1];
  const uint32_t r2 = st[4];
  const bool refined = (r2 & kRefined) != 0u;   // the recollect's kept keys replaced the collect's
  bool fallback = st[refined ? 6 : 2] != 0u;
  uint32_t total = 0;
  static_assert(NT == 1024, "one of the 1024 bins of a 10-bit digit per thread");
  lh[threadIdx.x] = 0u;   // the first 10-bit digit's histogram, counted during the gather
  // Chunk offsets in the concatenation: up to NT chunks one per thread (kept in
  // LDS for the parallel gather), beyond that a consecutive range per thread,
  // which gathers its own chunks.
  const uint32_t* cnt_h = counts + (int64_t)h * nchunks;
  const bool wide = nchunks > NT;
  const int64_t per = wide ? (nchunks + NT - 1) / NT : 1;
  const int64_t c0 = min<int64_t>((int64_t)threadIdx.x * per, nchunks);
  const int64_t c1 = min<int64_t>(c0 + per, nchunks);
  uint32_t off = 0;
  uint32_t mine = 0;   // read beside the state, not after it (the counts are always written)
  for (int64_t c = c0; c < c1; ++c) mine += cnt_h[c];
  if (!fallback) {
    off = block_exclusive<NT>(mine, wsum, &total);
    if (!wide) {
      coff[threadIdx.x] = off;
      if (threadIdx.x == 0) coff[nchunks] = total;
    }
    fallback = total > (uint32_t)kKeep;
  }
  if (fallback) {
    resolve_row(row, n, k, bin, above, out, outv, lh, wsum, sh);
    return;
  }
  __syncthreads();
  // a chunk's kept keys: its slot, or its spill segment when they overflowed it
  auto src_of = [&](int64_t c, uint32_t cn) -> const uint64_t* {
    return cn <= (uint32_t)kSlot ? kept + ((int64_t)h * nchunks + c) * kSlot
                                 : spill + (int64_t)h * spill_cap + soff[(int64_t)h * nchunks + c];
  };
  // gather in chunk order, every load of a batch issued before its stores; keys
  // of bin b are counted by their next 10 bits on the way
  constexpr int kBatch = 16;
  auto put = [&](uint32_t at, uint64_t v) {
    buf[at] = v;
    const uint32_t key = (uint32_t)(v >> 32);
    if ((key >> kDigit0) == bin) atomicAdd(&lh[(key >> 10) & 1023u], 1u);
  };
  if (wide) {
    uint32_t at = off;
    for (int64_t c = c0; c < c1; ++c) {
      const uint32_t cn = cnt_h[c];
      if (cn == 0) continue;
      const uint64_t* src = src_of(c, cn);
      for (uint32_t x0 = 0; x0 < cn; x0 += kBatch) {
        uint64_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) v[u] = x0 + u < cn ? src[x0 + u] : 0ull;
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (x0 + u < cn) put(at + x0 + u, v[u]);
      }
      at += cn;
    }
  } else {
    // TPC threads per chunk
    int tpc = 1;
    while (tpc * 2 * nchunks <= NT) tpc *= 2;
    const int c = threadIdx.x / tpc;
    const int r = threadIdx.x % tpc;
    if (c < nchunks) {
      const uint32_t cn = coff[c + 1] - coff[c];
      const uint64_t* src = src_of(c, cn);
      for (uint32_t x0 = r; x0 < cn; x0 += kBatch * tpc) {
        uint64_t v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t x = x0 + u * tpc;
          v[u] = x < cn ? src[x] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const uint32_t x = x0 + u * tpc;
          if (x < cn) put(coff[c] + x, v[u]);
        }
      }
    }
  }
  // the k-th key among the kept ones: keys above bin b are all in; among the keys
  // of bin b find the (k - above)-th largest by the next 10, then the last 10 bits
  // (refined: the next 10 bits are b2 already, and keys of bin b above b2 are in)
  uint32_t prefix = bin, need = (uint32_t)k - above;
  int pass0 = 0;
  if (refined) {
    prefix = (bin << 10) | (r2 & (uint32_t)(k2ndBins - 1));
    need -= st[5];
    pass0 = 1;
  }
  __syncthreads();
  for (int pass = pass0; pass < 2; ++pass) {
    if (pass == 1) {
      lh[threadIdx.x] = 0u;
      __syncthreads();
      for (uint32_t x = threadIdx.x; x < total; x += NT) {
        const uint32_t key = (uint32_t)(buf[x] >> 32);
        if ((key >> 10) == prefix) atomicAdd(&lh[key & 1023u], 1u);
      }
      __syncthreads();
    }
    find_bin<NT, 1024>(lh, need, wsum, sh);
    prefix = (prefix << 10) | sh[0];
    need -= sh[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  // ordered compaction: thread t owns kept items [span t, span (t+1)), span as small
  // as the kept count allows (short strides keep the LDS reads conflict-light)
  const uint32_t span = (total + NT - 1) / NT;   // <= kKeepPer
  const uint32_t x0 = threadIdx.x * span;
  uint32_t gt = 0, eq = 0;
  uint64_t kv[kKeepPer];
#pragma unroll
  for (int r = 0; r < kKeepPer; ++r) {
    const uint32_t x = x0 + r;
    const bool in = (uint32_t)r < span && x < total;
    kv[r] = in ? buf[x] : 0ull;
    const uint32_t key = (uint32_t)(kv[r] >> 32);
    gt += in && key > T;
    eq += in && key == T;
  }
  // both counts in one scan, as 16-bit halves (each total is at most kKeep)
  static_assert(kKeep < 65536, "16-bit halves");
  uint32_t tot = 0;
  const uint32_t before = block_exclusive<NT>((gt << 16) | eq, wsum, &tot);
  const uint32_t eq_before = before & 0xffffu;
  const uint32_t gt_before = before >> 16;
  uint32_t ties = eq_before;
  uint32_t pos = gt_before + min(eq_before, need);
#pragma unroll
  for (int r = 0; r < kKeepPer; ++r) {
    if ((uint32_t)r >= span || x0 + r >= total) break;
    const uint32_t key = (uint32_t)(kv[r] >> 32);
    bool take = key > T;
    if (key == T) {
      take = ties < need;
      ++ties;
    }
    if (take) {
      if (pos < (uint32_t)k) {
        out[pos] = (int32_t)(kv[r] & 0xffffffffu);
        if (outv) outv[pos] = key_to_float(key);
      }
      ++pos;
    }
  }
}

// Rows of at most kSmallRow keys: one workgroup per head holds the row's keys
// in LDS and runs the whole radix select there (first 12-bit digit, then two
// 10-bit digits, each counted over LDS), then the ordered compaction: one
// launch instead of histogram, collect and resolve.
__global__ __launch_bounds__(kResolveThreads) void sel_small(const float* __restrict__ scores, int64_t ld,
                                                             int n, int k, int32_t* __restrict__ idx,
                                                             float* __restrict__ val) {
  constexpr int NT = kResolveThreads;
  constexpr int kSpan = kSmallRow / NT;
  __shared__ uint32_t keys[kSmallRow];
  __shared__ uint32_t lh[kBins];
  __shared__ uint32_t wsum[NT / 64];
  __shared__ uint32_t sh[2];
  const int h = blockIdx.x;
  const float* row = scores + (int64_t)h * ld;   // 256-byte aligned rows padded to 64 keys
  int32_t* out = idx + (int64_t)h * k;
  float* outv = val ? val + (int64_t)h * k : nullptr;
  for (int q = threadIdx.x; 4 * q < n; q += NT) {
    const float4 v = *reinterpret_cast<const float4*>(row + 4 * q);
    const float e4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * q + e < n) keys[4 * q + e] = order_key(e4[e]);
  }
  for (int b = threadIdx.x; b < kBins; b += NT) lh[b] = 0u;
  __syncthreads();
  for (int x = threadIdx.x; x < n; x += NT) atomicAdd(&lh[keys[x] >> kDigit0], 1u);
  __syncthreads();
  find_bin<NT, kBins>(lh, (uint32_t)k, wsum, sh);
  uint32_t prefix = sh[0], need = (uint32_t)k - sh[1];
  __syncthreads();
  // two 10-bit digits among the keys that share the prefix found so far
  for (int shift = 10; shift >= 0; shift -= 10) {
    lh[threadIdx.x] = 0u;
    __syncthreads();
    for (int x = threadIdx.x; x < n; x += NT) {
      const uint32_t key = keys[x];
      if ((key >> (shift + 10)) == prefix) atomicAdd(&lh[(key >> shift) & 1023u], 1u);
    }
    __syncthreads();
    find_bin<NT, 1024>(lh, need, wsum, sh);
    prefix = (prefix << 10) | sh[0];
    need -= sh[1];
    __syncthreads();
  }
  const uint32_t T = prefix;
  // ordered compaction: thread t owns keys [span t, span (t+1))
  const int span = (n + NT - 1) / NT;   // <= kSpan
  const int x0 = threadIdx.x * span;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int r = 0; r < kSpan; ++r) {
    const int x = x0 + r;
    if (r < span && x < n) {
      gt += keys[x] > T;
      eq += keys[x] == T;
    }
  }
  uint32_t tot = 0;
  const uint32_t before = block_exclusive<NT>((gt << 16) | eq, wsum, &tot);
  const uint32_t eq_before = before & 0xffffu;
  uint32_t ties = eq_before;
  uint32_t pos = (before >> 16) + min(eq_before, need);
#pragma unroll
  for (int r = 0; r < kSpan; ++r) {
    const int x = x0 + r;
    if (r >= span || x >= n) break;
    const uint32_t key = keys[x];
    bool take = key > T;
    if (key == T) {
      take = ties < need;
      ++ties;
    }
    if (take) {
      if (pos < (uint32_t)k) {
        out[pos] = x;
        if (outv) outv[pos] = key_to_float(key);
      }
      ++pos;
    }
  }
}

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

int64_t select_chunks(int64_t n) { return (n + kChunk - 1) / kChunk; }



// Spill entries per head: the resolve holds at most kKeep kept keys (rows of at
// most kSmallRow keys are selected by sel_small and need none).
int64_t spill_entries(int64_t n) { return n <= kSmallRow ? 0 : kKeep; }

// The words that must be zero when the selection starts lead the workspace:
// histograms, state, and for long rows the second-digit histograms.
static size_t hist2_bytes(int h_q, int64_t n) { return n >= kRefineMin ? al256((size_t)h_q * k2ndBins * 4) : 0; }

size_t select_workspace_bytes(int h_q, int64_t n, int k) {
  (void)k;
  const size_t nc = (size_t)select_chunks(n);
  return al256((size_t)h_q * kBins * 4) + al256((size_t)h_q * kStateWords * 4) +
         hist2_bytes(h_q, n) +
         2 * al256((size_t)h_q * nc * 4) + al256((size_t)h_q * nc * kSlot * 8) +
         al256((size_t)h_q * (size_t)spill_entries(n) * 8);
}

size_t select_clear_words(const SelectWorkspace& ws, int h_q) {
  return (al256((size_t)h_q * kBins * 4) + al256((size_t)h_q * kStateWords * 4) +
          (ws.hist2 ? al256((size_t)h_q * k2ndBins * 4) : 0)) / 4;
}

SelectWorkspace carve_select(void* base, int h_q, int64_t n, int k) {
  (void)k;
  uint8_t* p = static_cast<uint8_t*>(base);
  SelectWorkspace ws;
  ws.nchunks = select_chunks(n);
  ws.hist = reinterpret_cast<uint32_t*>(p);
  p += al256((size_t)h_q * kBins * 4);
  ws.state = reinterpret_cast<uint32_t*>(p);
  p += al256((size_t)h_q * kStateWords * 4);
  ws.hist2 = n >= kRefineMin ? reinterpret_cast<uint32_t*>(p) : nullptr;
  p += hist2_bytes(h_q, n);
  ws.counts = reinterpret_cast<uint32_t*>(p);
  p += al256((size_t)h_q * (size_t)ws.nchunks * 4);
  ws.soff = reinterpret_cast<uint32_t*>(p);
  p += al256((size_t)h_q * (size_t)ws.nchunks * 4);
  ws.kept = reinterpret_cast<uint64_t*>(p);
  p += al256((size_t)h_q * (size_t)ws.nchunks * kSlot * 8);
  ws.spill = reinterpret_cast<uint64_t*>(p);
  ws.spill_cap = spill_entries(n);

  ws.small = n <= kSmallRow;
  return ws;
}

hipError_t launch_select_clear(const SelectWorkspace& ws, int h_q, hipStream_t s) {
  sel_init<<<h_q, kSelThreads, 0, s>>>(ws.hist, ws.state, ws.hist2);
  return hipGetLastError();
}

hipError_t launch_select(const float* scores, int64_t ld, int h_q, int64_t n, int k, int32_t* idx,
                         float* val, const SelectWorkspace& ws, bool cleared, bool hist_done, hipStream_t s) {
  if (k == 0 || n == 0 || h_q == 0) return hipSuccess;
  if (n <= kSmallRow) {
    sel_small<<<h_q, kResolveThreads, 0, s>>>(scores, ld, (int)n, k, idx, val);
    return hipGetLastError();
  }
  dim3 grid((unsigned)ws.nchunks, (unsigned)h_q);
  if (!hist_done) {
    if (!cleared) sel_init<<<h_q, kSelThreads, 0, s>>>(ws.hist, ws.state, ws.hist2);
    // chunks per histogram workgroup: 1, or more while the grid keeps >= 1024 workgroups
    // (4 per CU); fewer workgroups flush fewer partial histograms
    int per = 1;
    while (per < 8 && (ws.nchunks + 2 * per - 1) / (2 * per) * h_q >= 1024) per *= 2;
    const dim3 hgrid((unsigned)((ws.nchunks + per - 1) / per), (unsigned)h_q);
    sel_hist<<<hgrid, kSelThreads, 0, s>>>(scores, ld, n, ws.hist, per);
  }
  const bool refine = n >= kRefineMin;
  sel_collect<<<grid, kSelThreads, 0, s>>>(scores, ld, n, k, ws.hist, ws.state, ws.kept, ws.counts, ws.soff,
                                           ws.spill, ws.spill_cap, ws.nchunks, refine ? ws.hist2 : nullptr);
  if (refine) {   // returns at once for heads whose candidates fit on chip
    int rper = 1;   // chunks per workgroup: up to 8 while the grid keeps >= 1024 workgroups
    while (rper < 8 && (ws.nchunks + 2 * rper - 1) / (2 * rper) * h_q >= 1024) rper *= 2;
    const dim3 rgrid((unsigned)((ws.nchunks + rper - 1) / rper), (unsigned)h_q);
    sel_recollect<<<rgrid, kSelThreads, 0, s>>>(scores, ld, n, k, ws.hist, ws.state, ws.hist2, ws.kept, ws.counts,
                                                ws.soff, ws.spill, ws.spill_cap, ws.nchunks, rper);
  }
  sel_resolve<<<h_q, kResolveThreads, 0, s>>>(scores, ld, n, k, ws.state, ws.kept, ws.counts, ws.soff, ws.spill,
                                              ws.spill_cap, ws.nchunks, idx, val);
  return hipGetLastError();
}

}  // namespace fathom
