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
// lane owns channels lane + 64 i, i < CPL (2 for d <= 128, else 4).
//
// The greedy is computed in closed form rather than step by step.  Plane t of
// channel c (t = 0..3) is an item with marginal gain w_c 4^(-t); gains fall
// with t, so the greedy takes items in the order (gain desc, channel asc,
// plane asc) and after B steps holds exactly the B first items of that order.
// Each item gets a distinct integer key that sorts in that order:
//   key = bits(double(w_c) * 4^(-t)) >> 29 << 11 | (256 - c) << 2 | (3 - t).
// w_c is an fp32 value, so as a double its low 29 significand bits are zero and
// scaling by 4^(-t) is exact (no double underflow for t <= 3); non-negative
// doubles order like their bit patterns, and dropping the 29 zero bits keeps
// the key within 45 bits.  The B-th largest key K is found by a bitwise search
// from bit 44 down (each step counts the keys >= a candidate, one wave ballot
// per item), and t_c is the number of channel c's items with key >= K.  The
// fixed top-|q| mode selects m channels the same way with
// key = bits(|q_c|) << 8 | (255 - c).
//
// Static mode (mode 3) selects the same way with key = bits(sigma2_c) << 8 |
// (255 - c); sigma2 >= 0, so its bits order like its values.
//
// Group-shared mode (mode 2): one allocation per KV head on the fp32 sum, in
// head order, of the group's importances w_h,c; all query heads of the group
// get the same depths, so the scan reads exactly B bits per KV-head key.
#include "fathom_internal.h"

namespace fathom {
namespace {

__device__ inline uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v |= __shfl_xor(v, off, 64);
  return v;
}

// Largest K such that at least `want` of the wave's keys are >= K (the want-th
// largest key when keys are distinct); `want` >= 1 and at most the key count.
template <int N>
__device__ __forceinline__ uint64_t wave_kth_key(const uint64_t (&key)[N], uint32_t want, int top_bit) {
  uint64_t T = 0;
  for (int bit = top_bit; bit >= 0; --bit) {
    const uint64_t cand = T | (1ull << bit);
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) cnt += (uint32_t)__popcll(__ballot(key[i] >= cand));
    if (cnt >= want) T = cand;
  }
  return T;
}

template <int CPL>
__global__ __launch_bounds__(1024) void allocate_kernel(const float* __restrict__ q,
                                                        const float* __restrict__ sigma2, int g,
                                                        int d, int mode, int budget,
                                                        uint8_t* __restrict__ depth,
                                                        uint8_t* __restrict__ uni,
                                                        uint32_t* __restrict__ status) {
  __shared__ uint8_t sdep[kMaxG][kMaxD];
  __shared__ uint32_t sflag[kMaxG];

  const int kv = blockIdx.x;
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = kv * g + wv;

  float w[CPL];
  float aq[CPL];
  int t[CPL];
  uint32_t flag = 0;
  // the group-shared mode sums the importances of all g query heads of the KV
  // head, in head order; every wavefront of the group forms the same sum
  const int h_lo = mode == 2 ? kv * g : h;
  const int h_hi = mode == 2 ? kv * g + g : h + 1;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + 64 * i;
    t[i] = 0;
    w[i] = 0.0f;
    aq[i] = 0.0f;
    if (c < d) {
      const float sv = sigma2[(int64_t)kv * d + c];
      if (!(isfinite(sv) && sv >= 0.0f)) flag |= 8u;         // FATHOM_FLAG_SIGMA2_INVALID
      for (int x = h_lo; x < h_hi; ++x) {
        const float qv = q[(int64_t)x * d + c];
        if (!isfinite(qv)) flag |= 4u;                       // FATHOM_FLAG_Q_NONFINITE
        // two fp32 round-to-nearest products, never fused; sums in fp32, in order
        w[i] = __fadd_rn(w[i], __fmul_rn(__fmul_rn(qv, qv), sv));
        if (x == h) aq[i] = fabsf(qv);
      }
      if (!flag && !isfinite(w[i])) flag |= 16u;             // FATHOM_FLAG_IMPORTANCE_OVERFLOW
    }
  }
  flag = wave_or(flag);

  if (flag == 0 && (mode == 0 || mode == 2) && budget > 0) {
    uint64_t key[kPlanes * CPL];   // item (channel lane + 64 i, plane t) at 4 i + t; 0 = no item
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
#pragma unroll
      for (int t = 0; t < kPlanes; ++t) {
        const uint64_t gain = (uint64_t)__double_as_longlong(ldexp((double)w[i], -2 * t)) >> 29;
        key[4 * i + t] = c < d ? (gain << 11 | (uint64_t)(256 - c) << 2 | (uint64_t)(3 - t)) : 0ull;
      }
    }
    const uint64_t K = wave_kth_key(key, (uint32_t)budget, 44);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      int tc = 0;
#pragma unroll
      for (int t = 0; t < kPlanes; ++t) tc += key[4 * i + t] >= K;
      t[i] = lane + 64 * i < d ? tc : 0;
    }
  } else if (flag == 0 && (mode == 1 || mode == 3) && budget > 0) {
    // fixed-depth comparison modes: 4 planes on the m channels of largest |q_c|
    // (mode 1) or of largest offline variance sigma2_c (mode 3, the same for
    // every query head of the KV head)
    const uint32_t m = (uint32_t)(budget / kPlanes);
    uint64_t key[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      const float v = mode == 1 ? aq[i] : (c < d ? sigma2[(int64_t)kv * d + c] : 0.0f);
      key[i] = c < d ? ((uint64_t)__float_as_uint(v) << 8 | (uint64_t)(255 - c)) : 0ull;
    }
    // a channel with |q| = +0 and c = 255 has key 0: count it via the >= test only
    // when something else is smaller, so search over keys + 1
#pragma unroll
    for (int i = 0; i < CPL; ++i) key[i] = lane + 64 * i < d ? key[i] + 1 : 0ull;
    const uint64_t K = wave_kth_key(key, m, 40);
#pragma unroll
    for (int i = 0; i < CPL; ++i) t[i] = (lane + 64 * i < d && key[i] >= K) ? kPlanes : 0;
  }

#pragma unroll
  for (int i = 0; i < CPL; ++i) {
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
  if (d <= 128)
    allocate_kernel<2><<<h_kv, 64 * g, 0, s>>>(q, sigma2, g, d, mode, budget, depth, uni, status);
  else
    allocate_kernel<4><<<h_kv, 64 * g, 0, s>>>(q, sigma2, g, d, mode, budget, depth, uni, status);
  return hipGetLastError();
}

}  // namespace fathom
