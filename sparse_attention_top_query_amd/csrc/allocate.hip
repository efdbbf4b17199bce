// allocate_depths kernel: per-query read depth by reverse water-filling.
//
// Sources: the Fathom arXiv abstract and the ai-feeds digest (Method, key
// module 2).  A query decides per channel how many planes to read; channels of
// large importance w_c = q_c^2 sigma_c^2 get more planes, channels of small
// importance few or none.  The evolve.pub review, "Strengths" (paper Sec 3.3),
// derives the rule from the 4x drop in squared error per extra plane: the
// depths minimise sum_c w_c 4^(-t_c) subject to sum_c t_c = B, t_c in {0..4}.
//
// One workgroup per KV head, one wavefront per query head of its group.  A
// lane owns channels lane + 64 i, i < CPL (2 for d <= 128, else 4).
//
// The greedy is computed in closed form rather than step by step.  Plane t of
// channel c (t = 0..3) is an item with marginal gain w_c 4^(-t); gains fall
// with t, so the greedy takes items in the order (gain desc, channel asc,
// plane asc) and after B steps holds exactly the B first items of that order.
// Gains are compared exactly through the bits of w_c as a double (w_c is an
// fp32 value, so its low 29 significand bits are zero and scaling by 4^(-t)
// only lowers the exponent by 2t, never underflowing): with x_c = bits >> 29,
// the item (c, t) of a nonzero channel has the level L_c - t, L_c = x_c >> 24,
// and the fraction F_c = x_c mod 2^24, and items order by (level, fraction,
// lower channel).  So the B-th item is found in two short searches:
//   1. its level m, the largest m with A(m) = sum_c clamp(L_c - m + 1, 0, 4)
//      >= B (A(m) counts the items of level >= m), bit by bit over 10 bits,
//      each count one wave sum;
//   2. among the channels with an item at level m (L_c - m in 0..3), the
//      r = B - A(m + 1) largest keys F_c << 8 | (255 - c), by a bitwise search
//      over 32 bits with one ballot per channel slot.
// Then t_c = clamp(L_c - m, 0, 4), plus one for the r chosen channels.  Items
// of zero importance come after every other item, channel by channel in
// ascending order, so when B exceeds the nonzero items the lowest zero
// channels take the rest, 4 planes each.  The fixed top-|q| mode selects m
// channels by a bitwise search over the 41-bit keys bits(|q_c|) << 8 |
// (255 - c).
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
    const uint32_t B = (uint32_t)budget;
    int lvl[CPL];          // L_c of a nonzero channel, else 0 (which counts no item at any level >= 1)
    uint32_t frac[CPL];    // F_c << 8 | (255 - c)
    uint64_t nzm[CPL];     // lanes whose channel lane + 64 i has nonzero importance
    uint64_t zm[CPL];      // ... zero importance
    uint32_t nz = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      const uint64_t x = (uint64_t)__double_as_longlong((double)w[i]) >> 29;
      const bool valid = c < d;
      const bool pos = valid && w[i] > 0.0f;
      lvl[i] = pos ? (int)(x >> 24) : 0;
      frac[i] = (uint32_t)(x & 0xffffffu) << 8 | (uint32_t)(255 - c);
      nzm[i] = __ballot(pos);
      zm[i] = __ballot(valid && !pos);
      nz += 4u * (uint32_t)__popcll(nzm[i]);
    }
    if (B <= nz) {
      // items of level >= m, summed over the wave
      auto count_from = [&](int m) -> uint32_t {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) v += (uint32_t)min(max(lvl[i] - m + 1, 0), 4);
        return (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum(v), 63);
      };
      int m = 0;   // A(0) = nz >= B
      for (int bit = 9; bit >= 0; --bit) {
        const int cand = m | (1 << bit);
        if (count_from(cand) >= B) m = cand;
      }
      const uint32_t r = B - count_from(m + 1);   // >= 1 items still to take at level m
      uint64_t cm[CPL];
#pragma unroll
      for (int i = 0; i < CPL; ++i) cm[i] = __ballot(lvl[i] - m >= 0 && lvl[i] - m <= 3) & nzm[i];
      uint32_t T = 0;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) cnt += (uint32_t)__popcll(__ballot(frac[i] >= cand) & cm[i]);
        if (cnt >= r) T = cand;
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const bool chosen = ((cm[i] >> lane) & 1ull) && frac[i] >= T;
        t[i] = ((nzm[i] >> lane) & 1ull) ? min(max(lvl[i] - m, 0), 4) + (chosen ? 1 : 0) : 0;
      }
    } else {
      // every nonzero channel reads 4 planes; the B - nz remaining items go to the
      // zero channels in ascending order, 4 each
      const uint32_t rest = B - nz;
      uint32_t before = 0;   // zero channels in earlier slots
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t rank = before + (uint32_t)__popcll(zm[i] & ((1ull << lane) - 1ull));
        const int fill = (int)min<uint32_t>(rest - min(rest, 4u * rank), 4u);
        t[i] = ((nzm[i] >> lane) & 1ull) ? 4 : (((zm[i] >> lane) & 1ull) ? fill : 0);
        before += (uint32_t)__popcll(zm[i]);
      }
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
      // (sigma2 >= 0 here, so fabsf only folds -0 onto +0: the key orders values,
      // not bit patterns)
      const float v = mode == 1 ? aq[i] : (c < d ? fabsf(sigma2[(int64_t)kv * d + c]) : 0.0f);
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
