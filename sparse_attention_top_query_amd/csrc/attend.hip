// attend_topk kernels: attention of every query head over its selected keys.
//
// ai-feeds digest, Output: the scan yields top-k key indices per query, and
// real attention is then computed over those keys; evolve.pub review, FAQ:
// the scan picks the top-k for sparse attention.  The pages give no formula,
// so the reading is the standard one: s_j = scale (q . K_j) over the query's
// index set, o = sum_j softmax(s)_j V_j, lse = log sum_j exp(s_j).  K and V are
// the serving stack's bf16 cache rows, token-major [h_kv][n][d], in HBM or in
// pinned host memory read in place.
//
// Work decomposition (flash-decoding style).  A workgroup of 4 wavefronts takes
// KW consecutive entries of one query head's index list.  A row of d bf16
// channels is d/8 lanes of 16 bytes, so a wavefront gathers 64/(d/8) rows per
// load step; every lane issues all of its K and V row loads before using any,
// which keeps many independent host-link or HBM requests in flight.  Logits
// are reduced across the row's lanes, the workgroup max M and weight sum l
// follow, and sum_j exp(s_j - M) V_j is reduced across rows, wavefronts in a
// fixed order.  With one split per head the workgroup writes o and lse; with
// more, it writes (o, M, l) and a merge kernel combines the splits.
// Workgroup ids are mapped XCD-aware so that the query heads of one KV head
// share an XCD and its L2: rows selected by several heads of the group are
// then fetched over the link once.
#include "attend.h"

namespace fathom {
namespace {

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kXcdCount = 8;
constexpr uint32_t kFlagIndexRange = 32u;   // FATHOM_FLAG_INDEX_RANGE

struct AttArgs {
  const uint16_t* kc;     // [h_kv][n][d] bf16
  const uint16_t* vc;     // [h_kv][n][d] bf16
  const float* q;         // [h_q][d]
  const int32_t* idx;     // [h_q][k]
  int64_t n;
  int d, k, g, splits;
  float scale;
  float* part;            // [h_q][splits][d + 2]
  uint32_t* pflag;        // [h_q][splits]
  float* out;             // [h_q][d]
  float* lse;             // [h_q] or null
  uint32_t* status;       // [h_q] or null
};

__device__ __forceinline__ void bf16x8(const uint4& v, float (&f)[8]) {
  f[0] = __uint_as_float(v.x << 16);
  f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16);
  f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16);
  f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16);
  f[7] = __uint_as_float(v.w & 0xffff0000u);
}

// LPK = d / 8 lanes per row; KPI = 64 / LPK rows per wavefront step; KW rows per
// workgroup; IT = load steps per wavefront.
template <int LPK>
struct AttCfg {
  static constexpr int KPI = 64 / LPK;
  static constexpr int KW = (4096 / LPK) < 256 ? (4096 / LPK) : 256;
  static constexpr int IT = KW / (kAttWaves * KPI);
  static_assert(IT >= 1 && IT * kAttWaves * KPI == KW, "row split");
};

template <int LPK>
__global__ __launch_bounds__(kAttThreads) void attend_kernel(AttArgs a, int64_t total) {
  using C = AttCfg<LPK>;
  constexpr int D = 8 * LPK;
  __shared__ float sm_o[kAttWaves][D];
  __shared__ float sm_m[kAttWaves];
  __shared__ float sm_l[kAttWaves];
  __shared__ uint32_t sm_f[kAttWaves];

  const int64_t w = blockIdx.x;
  const int64_t per = (total + kXcdCount - 1) / kXcdCount;
  const int64_t L = (w % kXcdCount) * per + w / kXcdCount;
  if (L >= total) return;
  const int h = (int)(L / a.splits);
  const int sp = (int)(L % a.splits);
  const int gk = h / a.g;

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int sub = lane % LPK;        // channels 8 sub .. 8 sub + 7
  const int row = lane / LPK;        // row within the load step

  float qf[8];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.q + (int64_t)h * D + 8 * sub);
    const float4 q0 = qp[0], q1 = qp[1];
    qf[0] = q0.x; qf[1] = q0.y; qf[2] = q0.z; qf[3] = q0.w;
    qf[4] = q1.x; qf[5] = q1.y; qf[6] = q1.z; qf[7] = q1.w;
  }
  const uint16_t* kbase = a.kc + (int64_t)gk * a.n * D + 8 * sub;
  const uint16_t* vbase = a.vc + (int64_t)gk * a.n * D + 8 * sub;
  const int32_t* ids = a.idx + (int64_t)h * a.k;
  const int i0 = sp * C::KW + wv * (C::IT * C::KPI) + row;

  // all row loads first
  uint4 kr[C::IT], vr[C::IT];
  bool ok[C::IT];
  uint32_t bad = 0;
#pragma unroll
  for (int it = 0; it < C::IT; ++it) {
    const int i = i0 + it * C::KPI;
    int64_t j = -1;
    if (i < a.k) {
      j = ids[i];
      if (j < 0 || j >= a.n) {
        bad = 1;
        j = -1;
      }
    }
    ok[it] = j >= 0;
    if (ok[it]) {
      kr[it] = *reinterpret_cast<const uint4*>(kbase + j * D);
      vr[it] = *reinterpret_cast<const uint4*>(vbase + j * D);
    } else {
      kr[it] = make_uint4(0u, 0u, 0u, 0u);
      vr[it] = make_uint4(0u, 0u, 0u, 0u);
    }
  }

  // logits, reduced over the row's lanes
  float s[C::IT];
  float mx = -INFINITY;
#pragma unroll
  for (int it = 0; it < C::IT; ++it) {
    float kf[8];
    bf16x8(kr[it], kf);
    float dot = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = fmaf(qf[e], kf[e], dot);
#pragma unroll
    for (int off = 1; off < LPK; off <<= 1) dot += __shfl_xor(dot, off, 64);
    s[it] = ok[it] ? dot * a.scale : -INFINITY;
    mx = fmaxf(mx, s[it]);
  }
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  bad = __ballot(bad) != 0ull ? 1u : 0u;
  if (lane == 0) {
    sm_m[wv] = mx;
    sm_f[wv] = bad;
  }
  __syncthreads();
  float M = sm_m[0];
  uint32_t flag = sm_f[0];
#pragma unroll
  for (int x = 1; x < kAttWaves; ++x) {
    M = fmaxf(M, sm_m[x]);
    flag |= sm_f[x];
  }

  // weights, their sum and the weighted value rows
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  float lsum = 0.0f;
#pragma unroll
  for (int it = 0; it < C::IT; ++it) {
    const float p = ok[it] ? expf(s[it] - M) : 0.0f;
    lsum += p;
    float vf[8];
    bf16x8(vr[it], vf);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
  }
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    lsum += __shfl_xor(lsum, off, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  }
  if (row == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[wv][8 * sub + e] = acc[e];
  }
  if (lane == 0) sm_l[wv] = lsum;
  __syncthreads();

  if (tid < D) {
    float o = sm_o[0][tid];
    float l = sm_l[0];
#pragma unroll
    for (int x = 1; x < kAttWaves; ++x) {
      o += sm_o[x][tid];
      l += sm_l[x];
    }
    if (a.splits == 1) {
      a.out[(int64_t)h * D + tid] = l > 0.0f ? o / l : 0.0f;
      if (tid == 0) {
        if (a.lse) a.lse[h] = l > 0.0f ? M + logf(l) : -INFINITY;
        if (a.status) a.status[h] = flag ? kFlagIndexRange : 0u;
      }
    } else {
      float* pp = a.part + ((int64_t)h * a.splits + sp) * (D + 2);
      pp[tid] = o;
      if (tid == 0) {
        pp[D] = M;
        pp[D + 1] = l;
        a.pflag[(int64_t)h * a.splits + sp] = flag;
      }
    }
  }
}

// One workgroup per query head: o = sum_s o_s e^(M_s - M) / sum_s l_s e^(M_s - M).
// The factors e^(M_s - M) are formed once per split in LDS; sums run in split
// order.
constexpr int kMergeSplits = 1024;   // splits merged per pass through LDS

__global__ __launch_bounds__(kAttThreads) void attend_merge(AttArgs a) {
  __shared__ float fac[kMergeSplits];
  __shared__ float red[kAttThreads];
  const int h = blockIdx.x;
  const int d = a.d;
  const int tid = threadIdx.x;
  const float* pp = a.part + (int64_t)h * a.splits * (d + 2);
  // M = max over splits (threads stride the splits, then a tree in LDS)
  float m = -INFINITY;
  for (int sp = tid; sp < a.splits; sp += kAttThreads) m = fmaxf(m, pp[(int64_t)sp * (d + 2) + d]);
  red[tid] = m;
  __syncthreads();
  for (int w = kAttThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float o = 0.0f, l = 0.0f;
  for (int base = 0; base < a.splits; base += kMergeSplits) {
    const int cnt = min(kMergeSplits, a.splits - base);
    for (int x = tid; x < cnt; x += kAttThreads) {
      const float* q = pp + (int64_t)(base + x) * (d + 2);
      fac[x] = q[d + 1] > 0.0f ? expf(q[d] - M) : 0.0f;
    }
    __syncthreads();
    for (int x = 0; x < cnt; ++x) {
      const float f = fac[x];
      const float* q = pp + (int64_t)(base + x) * (d + 2);
      if (tid < d) o = fmaf(q[tid], f, o);
      l = fmaf(q[d + 1], f, l);
    }
    __syncthreads();
  }
  if (tid < d) a.out[(int64_t)h * d + tid] = l > 0.0f ? o / l : 0.0f;
  if (tid == 0) {
    if (a.lse) a.lse[h] = l > 0.0f ? M + logf(l) : -INFINITY;
    if (a.status) {
      uint32_t f = 0;
      for (int sp = 0; sp < a.splits; ++sp) f |= a.pflag[(int64_t)h * a.splits + sp];
      a.status[h] = f ? kFlagIndexRange : 0u;
    }
  }
}

template <int LPK>
hipError_t launch_lpk(const AttArgs& a, int h_q, hipStream_t s) {
  const int64_t total = (int64_t)h_q * a.splits;
  const int64_t per = (total + kXcdCount - 1) / kXcdCount;
  attend_kernel<LPK><<<(unsigned)(per * kXcdCount), kAttThreads, 0, s>>>(a, total);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  attend_merge<<<h_q, kAttThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attend(const uint16_t* kc, const uint16_t* vc, const float* q, const int32_t* idx,
                         int h_q, int h_kv, int64_t n, int d, int k, float scale, float* out, float* lse,
                         uint32_t* status, void* workspace, hipStream_t s) {
  AttArgs a;
  a.kc = kc;
  a.vc = vc;
  a.q = q;
  a.idx = idx;
  a.n = n;
  a.d = d;
  a.k = k;
  a.g = h_q / h_kv;
  a.splits = (int)attend_splits(d, k);
  a.scale = scale;
  const size_t parts = (size_t)h_q * (size_t)a.splits;
  a.part = static_cast<float*>(workspace);
  a.pflag = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) +
                                        (parts * (size_t)(d + 2) * 4 + 255) / 256 * 256);
  a.out = out;
  a.lse = lse;
  a.status = status;
  switch (d) {
    case 8: return launch_lpk<1>(a, h_q, s);
    case 16: return launch_lpk<2>(a, h_q, s);
    case 32: return launch_lpk<4>(a, h_q, s);
    case 64: return launch_lpk<8>(a, h_q, s);
    case 128: return launch_lpk<16>(a, h_q, s);
    case 256: return launch_lpk<32>(a, h_q, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fathom
