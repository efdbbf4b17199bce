// Pieces of the top-k selection: constants, the per-head state layout,
// workgroup scans, the threshold-bin search and the ordered compaction of kept
// keys.
#pragma once

#include "fathom_internal.h"

namespace fathom {
namespace sel {

constexpr int kSelThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kSelThreads * kPerThread;   // keys per hist/collect workgroup
constexpr int kBins = kSelBins;                    // first digit: top 12 key bits
constexpr int kDigit0 = kSelDigit0;                // shift of the first digit
constexpr int kResolveThreads = 1024;
constexpr int kSlot = 512;                         // kept keys per 4096-key chunk
constexpr int kKeep = 16384;                       // kept keys per head resolved in LDS (128 KB)
constexpr int kKeepPer = kKeep / kResolveThreads;
constexpr int k2ndBins = 1024;                     // second digit: the next 10 key bits
constexpr int64_t kRefineMin = 262144;             // rows at least this long get the refinement stage
// State per head: [0] first-digit bin b of the k-th key, [1] keys above bin b,
// [2] spill overflow of the collect, [3] its spill counter, [4] the refined
// second digit b2 | kRefined, [5] keys of bin b above b2, [6] spill overflow
// of the recollect, [7] its spill counter.
constexpr int kStateWords = 8;
constexpr int kSmallRow = 16384;                   // rows up to this long are selected by sel_small
constexpr uint32_t kRefined = 0x80000000u;

// inclusive suffix sum over the workgroup's threads (thread t gets sum over t' >= t)
template <int NT>
__device__ __forceinline__ uint32_t block_suffix_inclusive(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_sum(v);
  const uint32_t s = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63) - inc + v;   // lanes >= this one
  __syncthreads();
  if (lane == 0) wsum[w] = s;
  __syncthreads();
  uint32_t above = 0;
  for (int x = w + 1; x < NT / 64; ++x) above += wsum[x];
  return s + above;
}

// exclusive prefix sum over the workgroup's threads, in thread order; *total = sum
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_sum(v);
  __syncthreads();
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t base = 0, all = 0;
  for (int x = 0; x < NT / 64; ++x) {
    if (x < w) base += wsum[x];
    all += wsum[x];
  }
  *total = all;
  return base + inc - v;
}

// The bin of an NB-bin histogram holding the need-th largest key: sh[0] = bin,
// sh[1] = keys in higher bins.  Called by every thread; needs 1 <= need <= total.
template <int NT, int NB = kBins>
__device__ __forceinline__ void find_bin(const uint32_t* lh, uint32_t need, uint32_t* wsum, uint32_t* sh) {
  static_assert(NB % NT == 0, "whole bins per thread");
  constexpr int kPer = NB / NT;
  uint32_t v[kPer];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    v[i] = lh[threadIdx.x * kPer + i];
    mine += v[i];
  }
  uint32_t above = block_suffix_inclusive<NT>(mine, wsum) - mine;
#pragma unroll
  for (int i = kPer - 1; i >= 0; --i) {
    if (above < need && above + v[i] >= need) {
      sh[0] = threadIdx.x * kPer + i;
      sh[1] = above;
    }
    above += v[i];
  }
  __syncthreads();
}

// Compacts the keys of chunk c of a head (its scores f, first key j0) whose
// key >> shift is at least thr, in index order, into the chunk's slot or, if
// they do not fit there, a segment of the head's spill area claimed with one
// atomic on *ctr (all of the head's kept keys must fit the resolve's on-chip
// buffer, so the area has that size; beyond it *overflow is set and the head
// takes the resolve's full-row path).  Quad i of wavefront w holds keys
// j0 + 4 (256 i + 64 w + lane) + e, e < 4, so (i, w, lane, e) order is index
// order.  Called by every thread of the workgroup.
template <int NW, int NQ>
__device__ __forceinline__ void compact_chunk(const float4 (&f)[NQ], int64_t n, int64_t j0, int shift, uint32_t thr,
                                              uint32_t* ctr, uint32_t* overflow, int64_t c, uint64_t* kept,
                                              uint32_t* counts, uint32_t* soff, uint64_t* spill_h,
                                              int64_t spill_cap, uint32_t (*cnt)[NW], uint64_t** dst_sh,
                                              uint32_t* cap_sh) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  uint32_t key[NQ][4];
  uint64_t mask[NQ][4];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int64_t j = j0 + 4 * ((int64_t)i * kSelThreads + threadIdx.x);
    const float e4[4] = {f[i].x, f[i].y, f[i].z, f[i].w};
    uint32_t cc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      key[i][e] = order_key(e4[e]);
      mask[i][e] = __ballot(j + e < n && (key[i][e] >> shift) >= thr);
      cc += (uint32_t)__popcll(mask[i][e]);
    }
    if (lane == 0) cnt[i][w] = cc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tot = 0;
    for (int i = 0; i < NQ; ++i)
      for (int x = 0; x < NW; ++x) tot += cnt[i][x];
    uint64_t* dst = kept + c * kSlot;
    uint32_t cap = (uint32_t)kSlot;
    if (tot > (uint32_t)kSlot) {
      const uint32_t base = atomicAdd(ctr, tot);
      if ((int64_t)base + tot <= spill_cap) {
        dst = spill_h + base;
        cap = tot;
        soff[c] = base;
      } else {
        *overflow = 1u;
        cap = 0;
      }
    }
    counts[c] = tot;
    *dst_sh = dst;
    *cap_sh = cap;
  }
  __syncthreads();
  // offset of (i, w): keys kept by the (i', w') pairs before it
  uint64_t* dst = *dst_sh;
  const uint32_t cap = *cap_sh;
  const uint64_t lt = (1ull << lane) - 1ull;
  uint32_t run = 0;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    uint32_t off = run;   // kept keys of the quads before (i, w, lane)
    for (int x = 0; x < w; ++x) off += cnt[i][x];
#pragma unroll
    for (int e = 0; e < 4; ++e) off += (uint32_t)__popcll(mask[i][e] & lt);
    const int64_t j = j0 + 4 * ((int64_t)i * kSelThreads + threadIdx.x);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((mask[i][e] >> lane) & 1ull) {
        if (off < cap) store_global(dst + off, ((uint64_t)key[i][e] << 32) | (uint32_t)(j + e));
        ++off;
      }
    }
    for (int x = 0; x < NW; ++x) run += cnt[i][x];
  }
}

}  // namespace sel
}  // namespace fathom
