// The "free path": the per-query variable-depth scan run directly over the
// token-major 4-bit K copy a quantized serving stack holds, with no bit-plane
// index (Fathom abstract: the store is the serving stack's 4-bit K copy;
// evolve.pub review, weaknesses: the free path is unbuilt).
//
// Layout (a reading; the pages give none; d a multiple of 32 up to 128): codes
// [h_kv][n][d/2] bytes, channel
// 2i in the low nibble of byte i, 2i+1 in the high nibble; scales [h_kv][nb][d]
// fp16, one per (128-key block, channel) -- the same quantiser as the records.
// A key's codes are one contiguous row, so reading any bit of a channel means
// reading the whole row: the scan moves d/2 + (d/64) bytes per key whatever the
// budget, against the bit-plane prefix runs of the records.
//
// pack_nibbles: one workgroup per (128-key block, KV head), one thread per
// channel, the same threshold search as pack_bitplanes; an even channel's
// thread takes its odd neighbour's code by a lane shuffle and writes the byte.
//
// nibble_scan_kernel<G>: a workgroup scores 512 keys (4 blocks) of one KV head
// for all G query heads.  The tile's rows are staged into LDS (each row padded
// by one word so that lanes reading their own rows hit distinct banks), with
// the blocks' scales.  Lane l of wavefront w owns keys 128 w + l and 128 w + l
// + 64 (both in block w).  Channels are visited in order; for a union channel c
// read to depth t by some head, u = code >> (4 - t) is one bit-field extract,
// r = u - 2^(t-1), z = 2^(7-t) (2 r + 1), and the term a z (a = [q Delta / 16])
// joins the score of every head reading t planes: the same fp32 operations in
// the same order as the bit-plane scan, so the scores are bit-identical to it.
#include <hip/hip_fp16.h>

#include "fathom_internal.h"
#include "freepath.h"

namespace fathom {
namespace {

constexpr int kNibThreads = 256;
constexpr int kNibBlocks = 4;                       // 128-key blocks per workgroup
constexpr int kNibKeys = kNibBlocks * kBlock;       // 512
constexpr int kXcdN = 8;
constexpr int kNibMaxD = 128;                       // channels supported (rows of <= 64 bytes)

__global__ __launch_bounds__(256) void pack_nibbles_kernel(const float* __restrict__ k, int64_t n, int d,
                                                           int64_t nb, uint8_t* __restrict__ codes,
                                                           __half* __restrict__ scales,
                                                           uint32_t* __restrict__ status) {
  const int c = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int64_t g = blockIdx.y;
  const int64_t j0 = b * kBlock;
  const int cnt = (int)min<int64_t>(kBlock, n - j0);
  const bool act = c < d;
  const float* col = k + (g * n + j0) * d + c;
  float mx = 0.0f;
  bool finite = true;
  for (int j = 0; j < cnt; ++j) {
    const float v = act ? col[(int64_t)j * d] : 0.0f;
    finite &= isfinite(v);
    mx = fmaxf(mx, fabsf(v));
  }
  const __half dh = __float2half_rn(mx * 0.125f);
  const float dl = __half2float(dh);
  if (act) {
    uint32_t flags = 0;
    if (!finite) flags |= 1u;                      // FATHOM_FLAG_KEY_NONFINITE
    else if (!isfinite(dl)) flags |= 2u;           // FATHOM_FLAG_SCALE_OVERFLOW
    if (flags && status) atomicOr(status, flags);
    scales[(g * nb + b) * d + c] = dh;
  }
  const int64_t rowb = d / 2;
  for (int j = 0; j < cnt; ++j) {
    const float v = act ? col[(int64_t)j * d] : 0.0f;
    int code = 8;
    if (dl != 0.0f) {
      code = 0;
#pragma unroll
      for (int step = 8; step >= 1; step >>= 1) {
        const int cand = code + step;
        if (v >= (float)(cand - 8) * dl) code = cand;
      }
    }
    const int hi = __shfl_down(code, 1, 64);       // the odd neighbour (d is even)
    if (act && (c & 1) == 0) codes[(g * n + j0 + j) * rowb + c / 2] = (uint8_t)(code | (hi << 4));
  }
}

template <int G>
struct NibSmem {
  uint32_t rows[kNibKeys][kNibMaxD / 8 + 1];   // codes of the tile's keys, 8 channels per word, padded
  float coef[kNibBlocks][kNibMaxD][G];         // [q_h Delta / 16] of each block and channel
  float cq[kNibMaxD][G];                       // q_h / 16 per channel (0 when not read)
  uint64_t cw[kNibMaxD];                       // union depth | depths in use | head depths
  uint32_t wmask[kNibMaxD / 8];                // channels of the union per code word
};

__device__ __forceinline__ int nword_th(uint64_t w, int h) { return (int)((w >> (8 + 3 * h)) & 7); }

template <int G>
__global__ __launch_bounds__(kNibThreads) void nibble_scan_kernel(
    const uint8_t* __restrict__ codes, const __half* __restrict__ scales, const float* __restrict__ q,
    const uint8_t* __restrict__ depth, const uint8_t* __restrict__ uni, int64_t n, int d, int64_t nb,
    int64_t tiles, int64_t total, float* __restrict__ scores, int64_t ld) {
  __shared__ NibSmem<G> sm;
  const int64_t w = blockIdx.x;
  const int64_t per = (total + kXcdN - 1) / kXcdN;
  const int64_t L = (w % kXcdN) * per + w / kXcdN;
  if (L >= total) return;
  const int64_t g = L / tiles;
  const int64_t tile = L % tiles;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int64_t key0 = tile * kNibKeys;
  const int nkeys = (int)min<int64_t>(kNibKeys, n - key0);
  const int rw = d / 8;                       // code words per row
  const int64_t rowb = d / 2;

  // channel table
  if (tid < d) {
    const int c = tid;
    const int u = uni[g * d + c];
    uint64_t word = (uint64_t)u;
    for (int h = 0; h < G; ++h) {
      const int64_t row = (g * G + h) * d + c;
      const int th = u > 0 ? depth[row] : 0;
      if (th > 0) word |= (uint64_t)1 << (2 + th);
      word |= (uint64_t)th << (8 + 3 * h);
      sm.cq[c][h] = u > 0 ? ldexpf(q[row], -4) : 0.0f;   // exact power-of-two scaling
    }
    sm.cw[c] = u > 0 ? word : 0ull;
  }
  if (tid < rw) {
    uint32_t m = 0;
    for (int x = 0; x < 8; ++x) m |= (uni[g * d + 8 * tid + x] > 0 ? 1u : 0u) << x;
    sm.wmask[tid] = m;
  }
  // rows of the tile (16-byte pieces; rows are d/2 bytes, a multiple of 16)
  {
    const int pieces_per_row = d / 32;
    const int total_pieces = nkeys * pieces_per_row;
    const uint8_t* src = codes + (g * n + key0) * rowb;
    for (int i = tid; i < total_pieces; i += kNibThreads) {
      const int r = i / pieces_per_row;
      const int pc = i % pieces_per_row;
      const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)r * rowb + 16 * pc);
      uint32_t* dst = &sm.rows[r][4 * pc];
      dst[0] = v.x;
      dst[1] = v.y;
      dst[2] = v.z;
      dst[3] = v.w;
    }
  }
  __syncthreads();
  // coefficients per block of the tile, channel and head
  for (int i = tid; i < kNibBlocks * d; i += kNibThreads) {
    const int bl = i / d;
    const int c = i % d;
    const int64_t b = tile * kNibBlocks + bl;
    const float dl = b < nb ? __half2float(scales[(g * nb + b) * d + c]) : 0.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) sm.coef[bl][c][h] = sm.cq[c][h] * dl;   // one rounding
  }
  __syncthreads();

  float acc[2][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int s = 0; s < 2; ++s) acc[s][h] = 0.0f;
  }
  const int r0 = kBlock * wv + lane;          // rows of this lane's two keys
  const int r1 = r0 + 64;
  if (kBlock * wv < nkeys) {
    for (int wi = 0; wi < rw; ++wi) {
      const uint32_t m = __builtin_amdgcn_readfirstlane(sm.wmask[wi]);
      if (m == 0) continue;
      const uint32_t c0 = sm.rows[r0][wi];
      const uint32_t c1 = sm.rows[r1][wi];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        if (!(m & (1u << x))) continue;
        const int c = 8 * wi + x;
        const uint64_t cwv = sm.cw[c];
        uint64_t word = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)cwv);
        if (8 + 3 * G > 32)
          word |= (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(cwv >> 32)) << 32;
        float cf[G];
#pragma unroll
        for (int h = 0; h < G; ++h) cf[h] = sm.coef[wv][c][h];
#pragma unroll
        for (int t = 1; t <= kPlanes; ++t) {
          if (!(word & (8u << (t - 1)))) continue;
          // u = code >> (4 - t): the top t bits of the nibble; z = 2^(7-t) (2 (u - 2^(t-1)) + 1)
          const int u0 = (int)__builtin_amdgcn_ubfe(c0, 4 * x + 4 - t, t);
          const int u1 = (int)__builtin_amdgcn_ubfe(c1, 4 * x + 4 - t, t);
          const float f0 = (float)((2 * u0 + 1 - (1 << t)) * (1 << (7 - t)));
          const float f1 = (float)((2 * u1 + 1 - (1 << t)) * (1 << (7 - t)));
#pragma unroll
          for (int h = 0; h < G; ++h) {
            if (nword_th(word, h) != t) continue;
            acc[0][h] = fmaf(cf[h], f0, acc[0][h]);
            acc[1][h] = fmaf(cf[h], f1, acc[1][h]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int r = s == 0 ? r0 : r1;
    const int64_t j = key0 + r;
    if (r < nkeys) {
#pragma unroll
      for (int h = 0; h < G; ++h) scores[(g * G + h) * ld + j] = acc[s][h];
    }
  }
}

template <int G>
hipError_t launch_nib_g(const uint8_t* codes, const __half* scales, const float* q, const uint8_t* depth,
                        const uint8_t* uni, int h_kv, int64_t n, int d, float* scores, int64_t ld, hipStream_t s) {
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t tiles = (n + kNibKeys - 1) / kNibKeys;
  const int64_t total = tiles * h_kv;
  const int64_t per = (total + kXcdN - 1) / kXcdN;
  nibble_scan_kernel<G><<<(unsigned)(per * kXcdN), kNibThreads, 0, s>>>(codes, scales, q, depth, uni, n, d, nb,
                                                                        tiles, total, scores, ld);
  return hipGetLastError();
}

__global__ void clear_status(uint32_t* p) { *p = 0u; }

}  // namespace

hipError_t launch_pack_nibbles(const float* k, int h_kv, int64_t n, int d, uint8_t* codes, uint16_t* scales,
                               uint32_t* status, hipStream_t s) {
  if (status) {
    clear_status<<<1, 1, 0, s>>>(status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nb = (n + kBlock - 1) / kBlock;
  if (nb == 0) return hipSuccess;
  dim3 grid((unsigned)nb, (unsigned)h_kv);
  pack_nibbles_kernel<<<grid, ((d + 63) / 64) * 64, 0, s>>>(k, n, d, nb, codes, reinterpret_cast<__half*>(scales),
                                                           status);
  return hipGetLastError();
}

hipError_t launch_nibble_scan(const uint8_t* codes, const uint16_t* scales, const float* q, const uint8_t* depth,
                              const uint8_t* uni, int h_kv, int g, int64_t n, int d, float* scores, int64_t ld,
                              hipStream_t s) {
  if (n == 0) return hipSuccess;
  const __half* sc = reinterpret_cast<const __half*>(scales);
  switch (g) {
    case 1: return launch_nib_g<1>(codes, sc, q, depth, uni, h_kv, n, d, scores, ld, s);
    case 2: return launch_nib_g<2>(codes, sc, q, depth, uni, h_kv, n, d, scores, ld, s);
    case 4: return launch_nib_g<4>(codes, sc, q, depth, uni, h_kv, n, d, scores, ld, s);
    case 8: return launch_nib_g<8>(codes, sc, q, depth, uni, h_kv, n, d, scores, ld, s);
    case 16: return launch_nib_g<16>(codes, sc, q, depth, uni, h_kv, n, d, scores, ld, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fathom
