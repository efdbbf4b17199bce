// Scan kernel: reconstruct every key from its budgeted plane prefixes and
// accumulate q . k_hat for the query heads of one KV head.
//
// ai-feeds digest, Method / key modules 4-5: the scan reads only the planes
// the budget asks for and rebuilds each channel's value from the read prefix
// (the paper's Sec 3.5 rule; its formula is not in the text, the reading here
// is the midpoint of the prefix's cell of the t-bit mid-rise quantizer).
// Fathom abstract: the prefix of t planes is exactly the channel's t-bit
// quantizer, so k_hat_t = Delta 2^(4-t) (r_t + 1/2) with
// r_t = (code >> (4-t)) - 2^(t-1), a signed integer of t bits.
//
// Work decomposition (one workgroup = 4 wavefronts = 2048 keys of one KV head):
//  1. The union depths of the KV head give the list of channels to read; every
//     query head of the group is scored from the one read of the longest prefix.
//  2. Staging, channel group by channel group (at most 64 plane chunks, 16 KB):
//     the tile's plane bytes (256 contiguous bytes per channel-plane, 16 per
//     128-key block) and fp16 scales are loaded into registers with 16-byte
//     loads, all issued before any LDS write so many requests are in flight,
//     then stored to LDS.  The same code reads HBM or, for host-resident
//     records, pinned host memory over the host link, where contiguous runs of
//     >= 256 bytes are what keeps the link near its peak.
//  3. Compute: lane = key.  A 64-key plane word is wave-uniform, so it lives in
//     an SGPR pair and every lane takes its own bit from it.  The signed prefix
//     integer is built MSB first: r_1 = b_0 - 1, r_{t+1} = 2 r_t + b_t, which
//     yields every shorter prefix on the way, so heads reading fewer planes of
//     the same channel reuse it.  Per head: s += c_h * float(r_t) with
//     c_h = q_h * Delta * 2^(4-t) (one rounding), and the +1/2 term is summed
//     per block into a wave-uniform bias c_h / 2.
//     Error: |c r| <= 2 |c (r + 1/2)| for every integer r, so the fp32 sums stay
//     within ~(3m + 3) 2^-24 sum_c |q_c k_hat_c| for m channels.
#include <hip/hip_fp16.h>

#include "fathom_internal.h"

namespace fathom {
namespace {

#ifndef FATHOM_TILE_BLOCKS
#define FATHOM_TILE_BLOCKS 16
#endif
constexpr int kTileBlocks = FATHOM_TILE_BLOCKS;   // 128-key blocks per tile
#ifndef FATHOM_WAVE_BLOCKS
#define FATHOM_WAVE_BLOCKS 4
#endif
constexpr int kWaveBlocks = FATHOM_WAVE_BLOCKS;   // blocks per wavefront
constexpr int kThreads = 64 * kTileBlocks / kWaveBlocks;
constexpr int kSub = kWaveBlocks * 2;          // 64-key sub-chunks per wavefront
constexpr int kGroupChunks = 64;               // (entry, plane) chunks staged at once
constexpr int kGroupEntries = 64;              // entries staged at once (scales)
constexpr int kScalePieces = kTileBlocks * 2 / 16;   // 16-byte pieces of a tile's scales
static_assert(kTileBlocks % 8 == 0 && kThreads >= kMaxD, "tile must hold whole 16-byte scale pieces and one thread per channel");
constexpr int kMaxPieces = kGroupChunks * kTileBlocks + kGroupEntries * kScalePieces;
constexpr int kPiecesPerThread = (kMaxPieces + kThreads - 1) / kThreads;
constexpr int kMaxChunks = kPlanes * kMaxD;

template <int G>
struct ScanSmem {
  uint4 planes[kGroupChunks][kTileBlocks];     // staged plane bits (16 KB)
  uint4 scales[kGroupEntries][kScalePieces];   // staged fp16 scales
  float ent_q[kMaxD][G];                       // q of each query head
  uint8_t ent_th[kMaxD][G];                    // depth of each query head
  uint16_t ent_base[kMaxD + 1];                // first chunk of entry e (prefix sum)
  uint8_t ent_c[kMaxD];                        // channel of list entry e
  uint8_t ent_tb[kMaxD];                       // union depth of entry e
  uint16_t grp[kMaxD + 1];                     // first entry of each channel group
  uint8_t chunk_e[kMaxChunks];
  uint8_t chunk_p[kMaxChunks];
  int wsum[2][kThreads / 64];
  int n_grp;
};

__device__ __forceinline__ bool lane_bit(uint64_t m) { return __builtin_amdgcn_inverse_ballot_w64(m); }

template <int G>
__global__ __launch_bounds__(kThreads) void scan_kernel(const uint8_t* __restrict__ rec,
                                                        const float* __restrict__ q,
                                                        const uint8_t* __restrict__ depth,
                                                        const uint8_t* __restrict__ uni, int64_t n,
                                                        int64_t nb, int64_t S, int64_t P, int64_t R,
                                                        int d, float* __restrict__ scores,
                                                        int64_t ld) {
  __shared__ ScanSmem<G> sm;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t g = blockIdx.y;
  const int64_t blk0 = (int64_t)blockIdx.x * kTileBlocks;
  const int nvalid = (int)min<int64_t>(kTileBlocks, nb - blk0);

  // ---- 1. list of union channels, in channel order ----
  const int c = tid;
  const int u = (c < d) ? (int)uni[g * d + c] : 0;
  const int act = u > 0;
  int a_inc = act, t_inc = u;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int xa = __shfl_up(a_inc, off, 64);
    const int xt = __shfl_up(t_inc, off, 64);
    if (lane >= off) {
      a_inc += xa;
      t_inc += xt;
    }
  }
  if (lane == 63) {
    sm.wsum[0][wv] = a_inc;
    sm.wsum[1][wv] = t_inc;
  }
  __syncthreads();
  int a_off = 0, t_off = 0, n_ent = 0, n_chunk = 0;
#pragma unroll
  for (int x = 0; x < kThreads / 64; ++x) {
    if (x < wv) {
      a_off += sm.wsum[0][x];
      t_off += sm.wsum[1][x];
    }
    n_ent += sm.wsum[0][x];
    n_chunk += sm.wsum[1][x];
  }
  if (act) {
    const int e = a_off + a_inc - 1;
    const int base = t_off + t_inc - u;
    sm.ent_c[e] = (uint8_t)c;
    sm.ent_tb[e] = (uint8_t)u;
    sm.ent_base[e] = (uint16_t)base;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t row = (g * G + h) * d + c;
      sm.ent_th[e][h] = depth[row];
      sm.ent_q[e][h] = q[row];
    }
    for (int p = 0; p < u; ++p) {
      sm.chunk_e[base + p] = (uint8_t)e;
      sm.chunk_p[base + p] = (uint8_t)p;
    }
  }
  if (tid == 0) sm.ent_base[n_ent] = (uint16_t)n_chunk;
  __syncthreads();
  if (tid == 0) {
    // channel groups: consecutive entries with at most kGroupChunks chunks and
    // kGroupEntries entries each (an entry has at most 4 chunks)
    int ng = 0, e0 = 0;
    sm.grp[0] = 0;
    for (int e = 0; e < n_ent; ++e) {
      if (sm.ent_base[e + 1] - sm.ent_base[e0] > kGroupChunks || e + 1 - e0 > kGroupEntries) {
        sm.grp[++ng] = (uint16_t)e;
        e0 = e;
      }
    }
    if (n_ent > 0) sm.grp[++ng] = (uint16_t)n_ent;
    sm.n_grp = ng;
  }
  __syncthreads();

  float acc[kSub][G];
  float bias[kWaveBlocks][G];
#pragma unroll
  for (int s = 0; s < kSub; ++s)
#pragma unroll
    for (int h = 0; h < G; ++h) acc[s][h] = 0.0f;
#pragma unroll
  for (int x = 0; x < kWaveBlocks; ++x)
#pragma unroll
    for (int h = 0; h < G; ++h) bias[x][h] = 0.0f;

  const uint8_t* recg = rec + g * d * R;
  const int n_grp = sm.n_grp;

  // ---- 2. staging, software-pipelined: the loads of channel group gi+1 are in
  // flight (in registers) while group gi is computed from LDS ----
  uint4 v[kPiecesPerThread];
  auto issue = [&](int gi) {
    const int e_lo = sm.grp[gi], e_hi = sm.grp[gi + 1];
    const int ch_lo = sm.ent_base[e_lo];
    const int n_plane_pieces = (sm.ent_base[e_hi] - ch_lo) * kTileBlocks;
    const int total = n_plane_pieces + (e_hi - e_lo) * kScalePieces;
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int i = tid + r * kThreads;
      const uint4* src = nullptr;
      if (i < n_plane_pieces) {
        const int ch = ch_lo + i / kTileBlocks;
        const int b = i % kTileBlocks;
        if (b < nvalid) {
          const int e = sm.chunk_e[ch];
          src = reinterpret_cast<const uint4*>(recg + (int64_t)sm.ent_c[e] * R + S +
                                               sm.chunk_p[ch] * P + (blk0 + b) * 16);
        }
      } else if (i < total) {
        const int j = i - n_plane_pieces;
        const int e = e_lo + j / kScalePieces;
        const int piece = j % kScalePieces;          // blocks 8*piece .. 8*piece+7
        if (piece * 8 < nvalid)
          src = reinterpret_cast<const uint4*>(recg + (int64_t)sm.ent_c[e] * R + blk0 * 2 + piece * 16);
      }
      v[r] = src ? *src : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto commit = [&](int gi) {
    const int e_lo = sm.grp[gi], e_hi = sm.grp[gi + 1];
    const int ch_lo = sm.ent_base[e_lo];
    const int n_plane_pieces = (sm.ent_base[e_hi] - ch_lo) * kTileBlocks;
    const int total = n_plane_pieces + (e_hi - e_lo) * kScalePieces;
    uint4* const dst_planes = &sm.planes[0][0];
    uint4* const dst_scales = &sm.scales[0][0];
#pragma unroll
    for (int r = 0; r < kPiecesPerThread; ++r) {
      const int i = tid + r * kThreads;
      if (i < n_plane_pieces) dst_planes[i] = v[r];
      else if (i < total) dst_scales[i - n_plane_pieces] = v[r];
    }
  };

  if (n_grp > 0) issue(0);
  for (int gi = 0; gi < n_grp; ++gi) {
    const int e_lo = sm.grp[gi], e_hi = sm.grp[gi + 1];
    const int ch_lo = sm.ent_base[e_lo];
    commit(gi);
    __syncthreads();
    if (gi + 1 < n_grp) issue(gi + 1);

    // ---- 3. reconstruct and accumulate; wave wv owns kWaveBlocks blocks from kWaveBlocks*wv ----
    if (kWaveBlocks * wv < nvalid) {
      for (int e = e_lo; e < e_hi; ++e) {
        const int tb = sm.ent_tb[e];
        const int cb = sm.ent_base[e] - ch_lo;
        const __half* sc = reinterpret_cast<const __half*>(&sm.scales[e - e_lo][0]);
        int th[G];
        float coef[kWaveBlocks][G];
        int used = 0;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          th[h] = sm.ent_th[e][h];
          used |= 1 << th[h];
          const float qs = ldexpf(sm.ent_q[e][h], kPlanes - th[h]);   // exact power-of-two scaling
#pragma unroll
          for (int x = 0; x < kWaveBlocks; ++x) {
            coef[x][h] = qs * __half2float(sc[kWaveBlocks * wv + x]);
            if (th[h] > 0) bias[x][h] += 0.5f * coef[x][h];
          }
        }
        // plane p of sub-chunk s: 64-bit word pw[p * 2 * kTileBlocks + s]
        const uint64_t* pw = reinterpret_cast<const uint64_t*>(&sm.planes[cb][kWaveBlocks * wv]);
#pragma unroll
        for (int s = 0; s < kSub; ++s) {
          const int r1 = lane_bit(pw[s]) ? 0 : -1;
          int r2 = 0, r3 = 0, r4 = 0;
          if (tb >= 2) r2 = 2 * r1 + (int)lane_bit(pw[2 * kTileBlocks + s]);
          if (tb >= 3) r3 = 2 * r2 + (int)lane_bit(pw[4 * kTileBlocks + s]);
          if (tb >= 4) r4 = 2 * r3 + (int)lane_bit(pw[6 * kTileBlocks + s]);
          float f1 = 0.f, f2 = 0.f, f3 = 0.f, f4 = 0.f;
          if (used & 2) f1 = (float)r1;
          if (used & 4) f2 = (float)r2;
          if (used & 8) f3 = (float)r3;
          if (used & 16) f4 = (float)r4;
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const float cf = coef[s >> 1][h];
            if (th[h] == 1) acc[s][h] = fmaf(cf, f1, acc[s][h]);
            else if (th[h] == 2) acc[s][h] = fmaf(cf, f2, acc[s][h]);
            else if (th[h] == 3) acc[s][h] = fmaf(cf, f3, acc[s][h]);
            else if (th[h] == 4) acc[s][h] = fmaf(cf, f4, acc[s][h]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- 4. scores ----
#pragma unroll
  for (int s = 0; s < kSub; ++s) {
    const int64_t j = (blk0 + kWaveBlocks * wv + (s >> 1)) * kBlock + (s & 1) * 64 + lane;
    if (j < n) {
#pragma unroll
      for (int h = 0; h < G; ++h) scores[(g * G + h) * ld + j] = acc[s][h] + bias[s >> 1][h];
    }
  }
}

template <int G>
hipError_t launch_g(const uint8_t* rec, const float* q, const uint8_t* depth, const uint8_t* uni,
                    int h_kv, const Layout& L, int d, float* scores, int64_t ld, hipStream_t s) {
  dim3 grid((unsigned)((L.nb + kTileBlocks - 1) / kTileBlocks), (unsigned)h_kv);
  scan_kernel<G><<<grid, kThreads, 0, s>>>(rec, q, depth, uni, L.n, L.nb, L.S, L.P, L.R, d,
                                           scores, ld);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const uint8_t* rec, const float* q, const uint8_t* depth,
                       const uint8_t* uni, int h_kv, int g, const Layout& L, int d,
                       float* scores, int64_t ld, hipStream_t s) {
  if (L.nb == 0) return hipSuccess;
  switch (g) {
    case 1: return launch_g<1>(rec, q, depth, uni, h_kv, L, d, scores, ld, s);
    case 2: return launch_g<2>(rec, q, depth, uni, h_kv, L, d, scores, ld, s);
    case 4: return launch_g<4>(rec, q, depth, uni, h_kv, L, d, scores, ld, s);
    case 8: return launch_g<8>(rec, q, depth, uni, h_kv, L, d, scores, ld, s);
    case 16: return launch_g<16>(rec, q, depth, uni, h_kv, L, d, scores, ld, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fathom
