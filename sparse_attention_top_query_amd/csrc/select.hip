// Top-k selection: per query head, the k largest scores, lowest index among
// equal scores, returned in ascending index order (ai-feeds digest, Method /
// key module 5 and Output: the scan outputs top-k key indices per query).
//
// Radix select on order-preserving 32-bit keys, integer-only, LDS histograms:
//   key(f) = f >= +0 ? bits | 0x80000000 : ~bits   (-0 folded onto +0)
//   passes over digits [31:21], [20:10], [9:0] narrow the k-th largest key T and
//   the number `need` of keys equal to T that still belong to the top k;
//   a count pass gives every chunk its (> T, == T) counts, and the write pass
//   places the selected keys of each chunk after those of earlier chunks, so the
//   output is in index order and ties at T go to the lowest indices.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kSelThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kSelThreads * kPerThread;   // keys per workgroup
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct Digit {
  int shift;       // position of this digit
  int bits;        // width of this digit
  int hi_shift;    // keys must match the prefix in bits [31:hi_shift]; 32 = no filter
};

__device__ __forceinline__ Digit digit_of(int pass) {
  if (pass == 0) return {21, 11, 32};
  if (pass == 1) return {10, 11, 21};
  return {0, 10, 10};
}

__global__ __launch_bounds__(kSelThreads) void select_init(uint32_t* hist, uint32_t* state, int k) {
  const int h = blockIdx.x;
  for (int b = threadIdx.x; b < kBins; b += kSelThreads) hist[(int64_t)h * kBins + b] = 0u;
  if (threadIdx.x == 0) {
    state[h * 4 + 0] = 0u;               // prefix
    state[h * 4 + 1] = (uint32_t)k;      // need
  }
}

__global__ __launch_bounds__(kSelThreads) void select_hist(const float* __restrict__ scores, int64_t ld,
                                                           int64_t n, int pass,
                                                           uint32_t* __restrict__ hist,
                                                           const uint32_t* __restrict__ state) {
  __shared__ uint32_t lh[kBins];
  const int h = blockIdx.y;
  const Digit dg = digit_of(pass);
  for (int b = threadIdx.x; b < kBins; b += kSelThreads) lh[b] = 0u;
  __syncthreads();
  const uint32_t prefix = state[h * 4 + 0];
  const uint32_t mask = (1u << dg.bits) - 1u;
  const float* row = scores + (int64_t)h * ld;
  const int64_t j0 = (int64_t)blockIdx.x * kChunk;
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = j0 + (int64_t)i * kSelThreads + threadIdx.x;
    if (j < n) {
      const uint32_t key = order_key(row[j]);
      if (dg.hi_shift == 32 || (key >> dg.hi_shift) == prefix) atomicAdd(&lh[(key >> dg.shift) & mask], 1u);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += kSelThreads) {
    const uint32_t v = lh[b];
    if (v) atomicAdd(&hist[(int64_t)h * kBins + b], v);
  }
}

// One workgroup per head: find the bin holding the need-th largest key, extend
// the prefix by it, reduce `need` by the keys in higher bins, clear the histogram.
__global__ __launch_bounds__(kSelThreads) void select_find(uint32_t* __restrict__ hist,
                                                           uint32_t* __restrict__ state, int pass) {
  constexpr int kPer = kBins / kSelThreads;   // 8 bins per thread
  __shared__ uint32_t tot[kSelThreads];
  const int h = blockIdx.x;
  const Digit dg = digit_of(pass);
  const int nbins = 1 << dg.bits;
  uint32_t* hh = hist + (int64_t)h * kBins;
  uint32_t v[kPer];
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = threadIdx.x * kPer + i;
    v[i] = b < nbins ? hh[b] : 0u;
    mine += v[i];
  }
  tot[threadIdx.x] = mine;
  __syncthreads();
  // keys in bins above this thread's range
  uint32_t above = 0;
  for (int t = threadIdx.x + 1; t < kSelThreads; ++t) above += tot[t];
  const uint32_t need = state[h * 4 + 1];
  const uint32_t prefix = state[h * 4 + 0];
  __syncthreads();
#pragma unroll
  for (int i = kPer - 1; i >= 0; --i) {
    const int b = threadIdx.x * kPer + i;
    if (b < nbins && above < need && above + v[i] >= need) {
      state[h * 4 + 0] = (prefix << dg.bits) | (uint32_t)b;
      state[h * 4 + 1] = need - above;
    }
    above += v[i];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) hh[threadIdx.x * kPer + i] = 0u;
}

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t s = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) s += red[w];
  return s;
}

__global__ __launch_bounds__(kSelThreads) void select_count(const float* __restrict__ scores, int64_t ld,
                                                            int64_t n, const uint32_t* __restrict__ state,
                                                            uint32_t* __restrict__ counts, int64_t nchunks) {
  __shared__ uint32_t red[kSelThreads / 64];
  const int h = blockIdx.y;
  const uint32_t T = state[h * 4 + 0];
  const float* row = scores + (int64_t)h * ld;
  const int64_t j0 = (int64_t)blockIdx.x * kChunk;
  uint32_t gt = 0, eq = 0;
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = j0 + (int64_t)i * kSelThreads + threadIdx.x;
    if (j < n) {
      const uint32_t key = order_key(row[j]);
      gt += key > T;
      eq += key == T;
    }
  }
  gt = block_sum(gt, red);
  eq = block_sum(eq, red);
  if (threadIdx.x == 0) {
    counts[((int64_t)h * nchunks + blockIdx.x) * 2 + 0] = gt;
    counts[((int64_t)h * nchunks + blockIdx.x) * 2 + 1] = eq;
  }
}

// exclusive scan of one value per thread over the workgroup (thread order)
__device__ __forceinline__ uint32_t block_exclusive(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t x = __shfl_up(inc, off, 64);
    if (lane >= off) inc += x;
  }
  __syncthreads();
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t base = 0;
  for (int x = 0; x < w; ++x) base += wsum[x];
  return base + inc - v;
}

__global__ __launch_bounds__(kSelThreads) void select_write(const float* __restrict__ scores, int64_t ld,
                                                            int64_t n, int k,
                                                            const uint32_t* __restrict__ state,
                                                            const uint32_t* __restrict__ counts,
                                                            int64_t nchunks, int32_t* __restrict__ idx,
                                                            float* __restrict__ val) {
  __shared__ uint32_t red[kSelThreads / 64];
  __shared__ uint32_t wsum[kSelThreads / 64];
  const int h = blockIdx.y;
  const int64_t chunk = blockIdx.x;
  const uint32_t T = state[h * 4 + 0];
  const uint32_t need = state[h * 4 + 1];
  const uint32_t* cnt = counts + (int64_t)h * nchunks * 2;
  uint32_t gsum = 0, esum = 0;
  for (int64_t x = threadIdx.x; x < chunk; x += kSelThreads) {
    gsum += cnt[2 * x];
    esum += cnt[2 * x + 1];
  }
  const uint32_t Gb = block_sum(gsum, red);
  const uint32_t Eb = block_sum(esum, red);

  // this thread's keys: kPerThread consecutive indices
  const float* row = scores + (int64_t)h * ld;
  const int64_t j0 = chunk * kChunk + (int64_t)threadIdx.x * kPerThread;
  uint32_t keys[kPerThread];
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = j0 + i;
    const bool valid = j < n;
    keys[i] = valid ? order_key(row[j]) : 0u;
    gt += valid && keys[i] > T;
    eq += valid && keys[i] == T;
  }
  const uint32_t gt_before = block_exclusive(gt, wsum);
  const uint32_t eq_before = block_exclusive(eq, wsum);
  const uint32_t room = need > Eb ? need - Eb : 0u;         // ties still to take in this chunk
  const uint32_t ties_taken_before = min(room, eq_before);
  uint32_t pos = Gb + min(Eb, need) + gt_before + ties_taken_before;
  uint32_t tie_rank = Eb + eq_before;
  int32_t* out = idx + (int64_t)h * k;
  float* outv = val ? val + (int64_t)h * k : nullptr;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int64_t j = j0 + i;
    if (j >= n) break;
    bool take = false;
    if (keys[i] > T) {
      take = true;
    } else if (keys[i] == T) {
      take = tie_rank < need;
      ++tie_rank;
    }
    if (take) {
      if (pos < (uint32_t)k) {   // always true when the threshold search is right
        out[pos] = (int32_t)j;
        if (outv) outv[pos] = row[j];
      }
      ++pos;
    }
  }
}

}  // namespace

int64_t select_chunks(int64_t n) { return (n + kChunk - 1) / kChunk; }

size_t select_workspace_bytes(int h_q, int64_t n) {
  const size_t hist = (size_t)h_q * kBins * 4;
  const size_t state = (size_t)h_q * 4 * 4;
  const size_t counts = (size_t)h_q * (size_t)select_chunks(n) * 2 * 4;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return al(hist) + al(state) + al(counts);
}

SelectWorkspace carve_select(void* base, int h_q, int64_t n) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(base);
  SelectWorkspace ws;
  ws.nchunks = select_chunks(n);
  ws.hist = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)h_q * kBins * 4);
  ws.state = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)h_q * 4 * 4);
  ws.counts = reinterpret_cast<uint32_t*>(p);
  return ws;
}

hipError_t launch_select(const float* scores, int64_t ld, int h_q, int64_t n, int k, int32_t* idx,
                         float* val, const SelectWorkspace& ws, hipStream_t s) {
  if (k == 0 || n == 0 || h_q == 0) return hipSuccess;
  select_init<<<h_q, kSelThreads, 0, s>>>(ws.hist, ws.state, k);
  dim3 grid((unsigned)ws.nchunks, (unsigned)h_q);
  for (int pass = 0; pass < 3; ++pass) {
    select_hist<<<grid, kSelThreads, 0, s>>>(scores, ld, n, pass, ws.hist, ws.state);
    select_find<<<h_q, kSelThreads, 0, s>>>(ws.hist, ws.state, pass);
  }
  select_count<<<grid, kSelThreads, 0, s>>>(scores, ld, n, ws.state, ws.counts, ws.nchunks);
  select_write<<<grid, kSelThreads, 0, s>>>(scores, ld, n, k, ws.state, ws.counts, ws.nchunks, idx, val);
  return hipGetLastError();
}

}  // namespace fathom
