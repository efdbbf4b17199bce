// allocate_depths kernel: per-query read depth by reverse water-filling.
//
// Fathom abstract; ai-feeds digest, Method / key module 2: each query spreads
// its bit budget over channels by reverse water-filling on variance-weighted
// importance, so important channels are read deeper and unimportant ones
// not at all.  Review "Strengths" (paper Sec 3.3): the rule follows from each
// extra plane cutting the channel's error 4x, i.e. it minimises
// sum_c w_c 4^(-t_c) subject to sum_c t_c = B, t_c in {0..4}.
//
// One workgroup per KV head, one wavefront per query head of its group.  A
// lane owns channels lane, lane+64, lane+128, lane+192.  Each of the B greedy
// steps finds the channel of largest marginal gain w_c 4^(-t_c) with a
// wave-wide max over a single 64-bit key:
//   key = bits(double(w_c) * 4^(-t_c)) | (256 - c).
// w_c is an fp32 value, so as a double its low 29 significand bits are zero
// and scaling by 4^(-t) is exact: the key orders by exact gain first, then
// by lowest channel, which is the tie rule.  Non-negative doubles order like
// their bit patterns, and 256 - c >= 1 keeps every real candidate above 0.
#include "fathom_internal.h"

namespace fathom {
namespace {

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ inline uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v |= __shfl_xor(v, off, 64);
  return v;
}

__global__ __launch_bounds__(1024) void allocate_kernel(const float* __restrict__ q,
                                                        const float* __restrict__ sigma2, int g,
                                                        int d, int mode, int budget,
                                                        uint8_t* __restrict__ depth,
                                                        uint8_t* __restrict__ uni,
                                                        uint32_t* __restrict__ status) {
  __shared__ uint8_t sdep[kMaxG][kMaxD];
  __shared__ float sabs[kMaxG][kMaxD];
  __shared__ uint32_t sflag[kMaxG];

  const int kv = blockIdx.x;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = kv * g + wv;

  float w[4];
  float aq[4];
  int t[4];
  uint32_t flag = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    t[i] = 0;
    w[i] = 0.0f;
    aq[i] = 0.0f;
    if (c < d) {
      const float qv = q[(int64_t)h * d + c];
      const float sv = sigma2[(int64_t)kv * d + c];
      if (!isfinite(qv)) flag |= 4u;                         // FATHOM_FLAG_Q_NONFINITE
      if (!(isfinite(sv) && sv >= 0.0f)) flag |= 8u;         // FATHOM_FLAG_SIGMA2_INVALID
      // two fp32 round-to-nearest products, never fused
      w[i] = __fmul_rn(__fmul_rn(qv, qv), sv);
      if (!flag && !isfinite(w[i])) flag |= 16u;             // FATHOM_FLAG_IMPORTANCE_OVERFLOW
      aq[i] = fabsf(qv);
    }
  }
  flag = wave_or(flag);

  // |q| of every channel, for the fixed-depth mode (written by all waves so the
  // barrier below is reached uniformly)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    if (c < d) sabs[wv][c] = aq[i];
  }
  __syncthreads();

  if (flag == 0 && mode == 0) {
    for (int step = 0; step < budget; ++step) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = lane + 64 * i;
        if (c < d && t[i] < kPlanes) {
          const double gain = ldexp((double)w[i], -2 * t[i]);
          const uint64_t key = ((uint64_t)__double_as_longlong(gain)) | (uint64_t)(256 - c);
          best = key > best ? key : best;
        }
      }
      best = wave_max_u64(best);   // > 0: step < budget <= 4d leaves a channel with room
      const int cw = 256 - (int)(best & 511u);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == cw) t[i] += 1;
    }
  } else if (flag == 0) {
    // fixed-depth comparison mode: 4 planes on the m channels of largest |q_c|
    const int m = budget / kPlanes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = lane + 64 * i;
      if (c < d) {
        int rank = 0;
        for (int c2 = 0; c2 < d; ++c2) {
          const float a2 = sabs[wv][c2];
          rank += (a2 > aq[i]) || (a2 == aq[i] && c2 < c);
        }
        t[i] = rank < m ? kPlanes : 0;
      }
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    if (c < d) {
      depth[(int64_t)h * d + c] = (uint8_t)t[i];
      sdep[wv][c] = (uint8_t)t[i];
    }
  }
  if (lane == 0) sflag[wv] = flag;
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += blockDim.x) {
    int u = 0;
    for (int x = 0; x < g; ++x) u = max(u, (int)sdep[x][c]);
    uni[(int64_t)kv * d + c] = (uint8_t)u;
  }
  if (threadIdx.x == 0 && status) {
    uint32_t f = 0;
    for (int x = 0; x < g; ++x) f |= sflag[x];
    status[kv] = f;
  }
}

}  // namespace

hipError_t launch_allocate(const float* q, const float* sigma2, int h_kv, int g, int d,
                           int mode, int budget, uint8_t* depth, uint8_t* uni,
                           uint32_t* status, hipStream_t s) {
  allocate_kernel<<<h_kv, 64 * g, 0, s>>>(q, sigma2, g, d, mode, budget, depth, uni, status);
  return hipGetLastError();
}

}  // namespace fathom
