// Exact scores of the open tail block.
//
// The block scale is shared by a whole 128-key block (evolve.pub review,
// "Strengths", paper Sec 3.2), so the newest keys of a growing cache cannot be
// quantised before their block is full.  Reading: they stay in fp32 and are
// scored exactly, s = sum_c q_c k_c, then ranked with the scanned keys.
//
// One wavefront per (tail key, KV head): the lanes read the key's row (d <= 256,
// lane owns channels lane + 64 i), and for each query head of the group form
// the d products and a fixed-order butterfly sum.  With `hist`, each score is
// also counted into the selection's first-digit histogram of its head (when the
// scan of the sealed keys built those histograms).
#include "append.h"

namespace fathom {
namespace {

constexpr int kTailWaves = 4;

__global__ __launch_bounds__(64 * kTailWaves) void tail_kernel(const float* __restrict__ tail_k,
                                                               const float* __restrict__ q, int g, int64_t m,
                                                               int d, float* __restrict__ scores, int64_t ld,
                                                               int64_t first, uint32_t* __restrict__ hist) {
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kTailWaves + (threadIdx.x >> 6);
  const int64_t kv = blockIdx.y;
  if (i >= m) return;   // whole wavefronts; no barriers below
  const float* row = tail_k + (kv * m + i) * d;
  float kr[kMaxD / 64];
#pragma unroll
  for (int x = 0; x < kMaxD / 64; ++x) {
    const int c = lane + 64 * x;
    kr[x] = c < d ? row[c] : 0.0f;
  }
  for (int h = 0; h < g; ++h) {
    const int64_t hq = kv * g + h;
    const float* qh = q + hq * d;
    float acc = 0.0f;
#pragma unroll
    for (int x = 0; x < kMaxD / 64; ++x) {
      const int c = lane + 64 * x;
      if (c < d) acc = fmaf(qh[c], kr[x], acc);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) {
      scores[hq * ld + first + i] = acc;
      if (hist) atomicAdd(&hist[hq * kSelBins + (order_key(acc) >> kSelDigit0)], 1u);
    }
  }
}

}  // namespace

hipError_t launch_tail_scores(const float* tail_k, const float* q, int h_kv, int g, int64_t m, int d,
                              float* scores, int64_t ld, int64_t first, uint32_t* hist, hipStream_t s) {
  if (m == 0) return hipSuccess;
  dim3 grid((unsigned)((m + kTailWaves - 1) / kTailWaves), (unsigned)h_kv);
  tail_kernel<<<grid, 64 * kTailWaves, 0, s>>>(tail_k, q, g, m, d, scores, ld, first, hist);
  return hipGetLastError();
}

}  // namespace fathom
