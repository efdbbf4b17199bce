// Scan kernels: reconstruct every key from its budgeted plane prefixes and
// accumulate q . k_hat for the query heads of one KV head.
//
// ai-feeds digest, Method / key modules 4-5: the scan reads only the planes
// the budget asks for and rebuilds each channel's value from the read prefix
// (the paper's Sec 3.5 rule; its formula is not in the text, the reading here
// is the midpoint of the prefix's cell of the t-bit mid-rise quantizer).
// Fathom abstract: the prefix of t planes is exactly the channel's t-bit
// quantizer, so with r_t = (code >> (4-t)) - 2^(t-1), a signed t-bit integer,
//   q * k_hat_t = q Delta 2^(4-t) (r_t + 1/2) = c (2 r_t + 1),  c = [q 2^(3-t) Delta],
// and the scan accumulates it as (2c) r_t per key plus, once per block, c: with
// c one fp32 rounding (2c exact), every term is bounded by |2 c r_t| <= 2 |q k_hat|
// and |c| <= |q k_hat| (|2 r_t + 1| >= 1), so the fp32 sum over m channels stays
// within about 3 (m + 2) 2^-24 sum_c |q_c k_hat_c|.
//
// Work decomposition: one workgroup scores a tile of TB 128-key blocks of one KV
// head for all of its G query heads; each wavefront owns 2 blocks (256 keys):
// lanes 0-31 one block, lanes 32-63 the other, and lane l scores the 4
// consecutive keys 4 (l%32) .. 4 (l%32) + 3 of its block, which one 32-bit
// word of each plane row holds.
//  1. The union depths of the KV head list the channels to read; every query
//     head of the group is scored from the one read of the longest prefix.
//  2. Staging, channel group by channel group (about 64 channel-planes): the
//     tile's slice of each channel's record head (its units' fp16 scales and
//     plane-0 bits) and of planes 1..t-1 are loaded with 16-byte loads into
//     registers -- all issued before any LDS write, and those of the next group
//     while the current group is computed -- then stored to LDS, the most
//     significant plane complemented.  The same code reads HBM, an HBM staging
//     mirror, or pinned host memory over the host link; the tile size sets the
//     contiguous run per channel-plane (16 B per block).
//  3. Per (channel, block) the doubled coefficients 2 c = 2 [q_h 2^(3-t_h) Delta]
//     are formed once in LDS.  Per key, each lane reads its own plane words and
//     builds the signed prefix MSB first: r_1 = -(complemented bit) = b_0 - 1,
//     then r_{t+1} = 2 r_t + b_t, which yields every shorter prefix on the way
//     for heads that read fewer planes; float(r_t) once per depth in use, and
//     per head one fma with 2c and one add of 2c to the lane's per-head sum,
//     half of which joins every score at the end.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>

#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kGroupChunks = 64;               // channel-planes per staging group (+3 slack)
constexpr int kSlackChunks = kPlanes - 1;      // an entry starting in a group ends in it
constexpr int kStageChunks = kGroupChunks + kSlackChunks;
constexpr int kStageEntries = kStageChunks;    // entries have >= 1 chunk
constexpr int kMaxChunks = kPlanes * kMaxD;
constexpr int kWaveBlocks = 2;                 // 128-key blocks per wavefront
constexpr int kSub = kBlock / 32;              // 32-key words per block; a lane scores one key of each

template <int G, int TB>
struct Cfg {
  static constexpr int threads = 64 * TB / kWaveBlocks;
  static constexpr int units = TB / kUnitBlocks;      // 1024-key record units per tile
  static constexpr int slots = TB + units;            // 16-byte pieces per chunk slot
  static constexpr int ppt = (kStageChunks * slots + threads - 1) / threads;
  static_assert(threads >= kMaxD && threads <= 1024, "one thread per channel in the list build");
  static_assert(TB % kUnitBlocks == 0, "tiles hold whole 1024-key units");
};

template <int G, int TB>
struct ScanSmem {
  uint4 planes[kStageChunks + kPlanes - 1][TB];    // staged plane bits (plane 0 complemented); the last
                                                   // rows pad reads of a prefix's unread planes
  uint4 scales[kStageEntries][TB / kUnitBlocks];   // staged fp16 scales per entry of the group
  float coef[kStageChunks][TB][G];                 // 2 [q_h 2^(3-t_h) Delta_b] per block and head, in the
                                                   // row of the entry's first chunk (for G = 4 a row has the
                                                   // planes' stride: one address serves both)
  float ent_q[kMaxD][G];                           // q_h 2^(3-t_h) of each list entry
  uint64_t ent_word[kMaxD + 1];                    // level masks: bit (t-1) G + h iff head h reads t planes
  uint16_t ent_base[kMaxD + 1];                    // first chunk of entry e (prefix sum)
  uint16_t grp[kMaxChunks / kGroupChunks + 2];     // first entry of each staging group
  uint32_t chunk_meta[kMaxChunks];                 // entry | channel << 8 | plane << 16 of each chunk
  int wsum[2][16];
  int n_grp;
};

struct ScanArgs {
  const uint8_t* rec;        // records, device-visible
  const float* q;
  const uint8_t* depth;
  const uint8_t* uni;
  int64_t n, nb, H, P, R;
  int d;
  float* scores;
  int64_t ld;
  uint32_t* zero;            // words to clear on the way (may be null)
  int64_t zero_words;
  uint32_t* hist;            // selection histograms [h_q][kSelBins] to add to (fused scans)
  // paged records (may be null): pages[g * npages + p] is the device-visible
  // base of page p of KV head g, [d][R] bytes for page_tiles tiles of keys,
  // laid out as whole records of those keys (H, P, R are the page's)
  const uint8_t* const* pages;
  int64_t npages;
  int64_t page_tiles;
};

// Entry word: one G-bit mask per depth t = 1..4, bit (t - 1) G + h set iff head h
// reads exactly t planes of the channel (at most 64 bits for G <= 16).  The
// union depth is the entry's chunk count.


// The fused first-digit histograms live in the tile's staging memory, which is
// dead once the last group is scored: 16-bit counts, two bins per word (a tile
// holds at most 4096 keys), for as many heads per round as fit.
constexpr int kHistWords = kSelBins / 2;
template <int G, int TB>
constexpr int kHistHeads = (int)(sizeof(ScanSmem<G, TB>) / 4 / kHistWords) < G
                               ? (int)(sizeof(ScanSmem<G, TB>) / 4 / kHistWords) : G;

// Scores of tile `tile` (TB blocks) of KV head g, all its query heads.  With
// FUSE, the tile's scores are also counted into a.hist by their first
// selection digit (an LDS histogram per round of heads, then one global atomic
// per non-empty bin).
template <int G, int TB, bool FUSE = false>
__device__ __forceinline__ void scan_tile(const ScanArgs& a, int64_t g, int64_t tile, ScanSmem<G, TB>& sm) {
  using C = Cfg<G, TB>;
  constexpr int SLOTS = C::slots;
  constexpr int NT = C::threads;
  constexpr int PPT = C::ppt;
  static_assert(4 * G <= 64, "the level masks must fit the entry word");
  const uint8_t* __restrict__ rec = a.rec;
  const int64_t nb = a.nb, H = a.H, P = a.P, R = a.R;
  const int d = a.d;

  const int tid = threadIdx.x;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int64_t blk0 = tile * TB;
  const int bl = kWaveBlocks * wv + (lane >> 5);   // block of this lane within the tile
  const int nvalid = (int)min<int64_t>(TB, nb - blk0);

  // ---- 1. list of union channels, in channel order, and staging groups ----
  {
    const int c = tid;
    // every input of the list in one round trip, without branches: threads past
    // the last channel read channel d-1 and drop it
    const int cs = c < d ? c : d - 1;
    const int u0 = (int)a.uni[g * d + cs];
    int th[G];
    float qc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t row = (g * G + h) * d + cs;
      th[h] = (int)a.depth[row];
      qc[h] = a.q[row];
    }
    const int u = c < d ? u0 : 0;
    const int act = u > 0;
    // entry and chunk counts in one scan (16-bit halves: at most 64 and 256 per wave)
    const uint32_t both = wave_inclusive_sum((uint32_t)act | (uint32_t)u << 16);
    const int a_inc = (int)(both & 0xffffu), t_inc = (int)(both >> 16);
    if (lane == 63) {
      sm.wsum[0][wv] = a_inc;
      sm.wsum[1][wv] = t_inc;
    }
    __syncthreads();
    int a_off = 0, t_off = 0, n_ent = 0;
#pragma unroll
    for (int x = 0; x < NT / 64; ++x) {
      if (x < wv) {
        a_off += sm.wsum[0][x];
        t_off += sm.wsum[1][x];
      }
      n_ent += sm.wsum[0][x];
    }
    const int e = a_off + a_inc - 1;
    const int base = t_off + t_inc - u;
    if (act) {
      uint64_t word = 0;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (th[h] > 0) word |= (uint64_t)1 << ((th[h] - 1) * G + h);
        sm.ent_q[e][h] = ldexpf(qc[h], 3 - th[h]);   // exact power-of-two scaling
      }
      sm.ent_word[e] = word;
      sm.ent_base[e] = (uint16_t)base;
      if (e == n_ent - 1) {
        sm.ent_base[n_ent] = (uint16_t)(base + u);
        // an entry joins the group holding its first chunk; first chunks are at
        // most 4 apart, so groups 0 .. base/64 are all non-empty
        sm.n_grp = base / kGroupChunks + 1;
        sm.grp[base / kGroupChunks + 1] = (uint16_t)n_ent;
      }
#pragma unroll
      for (int p = 0; p < kPlanes; ++p)
        if (p < u) sm.chunk_meta[base + p] = (uint32_t)e | (uint32_t)c << 8 | (uint32_t)p << 16;
    }
    if (tid == 0 && n_ent == 0) sm.n_grp = 0;
    __syncthreads();
    if (act) {
      const int gi = base / kGroupChunks;
      if (e == 0 || sm.ent_base[e - 1] / kGroupChunks != gi) sm.grp[gi] = (uint16_t)e;
    }
    __syncthreads();
  }

  float acc[kSub][G];
  float half_sum[G];   // per head: the sum of its coefficients 2 c over the channels it reads
#pragma unroll
  for (int h = 0; h < G; ++h) {
    half_sum[h] = 0.0f;
#pragma unroll
    for (int s = 0; s < kSub; ++s) acc[s][h] = 0.0f;
  }

  // the tile's records: the KV head's own, or its page (addressed page-locally)
  const uint8_t* recg;
  int64_t ablk0;   // first block of the tile within those records
  if (a.pages) {
    recg = a.pages[g * a.npages + tile / a.page_tiles];
    ablk0 = (tile % a.page_tiles) * TB;
  } else {
    recg = rec + g * d * R;
    ablk0 = blk0;
  }
  const int64_t unit0 = ablk0 / kUnitBlocks;
  const int n_grp = sm.n_grp;

  // ---- 2. staging.  Piece i of a group is slot i % SLOTS of chunk i / SLOTS.  A
  // record-head chunk walks the tile's head slice in memory order (per unit: 1
  // scale piece, then 8 plane-0 pieces); a chunk of plane p >= 1 uses its first
  // TB slots.  A thread's pieces sit at the same (chunk, slot) of every group, so
  // their slot offsets are fixed; issue keeps each piece's chunk meta for commit.
  uint4 v[PPT];
  uint32_t meta[PPT];
  const uint32_t R32 = (uint32_t)R, H32 = (uint32_t)H, P32 = (uint32_t)P;
  auto issue = [&](int gi) {
    const int ch_lo = sm.ent_base[sm.grp[gi]];
    const int n_pieces = (sm.ent_base[sm.grp[gi + 1]] - ch_lo) * SLOTS;
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int i = tid + r * NT;
      const int k = i % SLOTS;
      const int un = k / (kUnitBlocks + 1);
      const int w = k % (kUnitBlocks + 1);
      const uint4* src = nullptr;
      meta[r] = 0u;
      if (i < n_pieces) {
        const uint32_t m = sm.chunk_meta[i / SLOTS + ch_lo];
        const uint32_t p = m >> 16;
        meta[r] = m;
        // byte offset within the channel's record (records hold at most 2^30 keys,
        // so R < 2^32): the unit's head slice, or the blocks' slice of plane p
        // (the second test also skips the unused slots k >= TB)
        const bool ok = p == 0u ? un * kUnitBlocks + (w == 0 ? 0 : w - 1) < nvalid : k < nvalid;
        const uint32_t at = p == 0u ? kUnitHead * (uint32_t)(unit0 + un) + 16u * w
                                    : H32 + (p - 1u) * P32 + 16u * (uint32_t)(ablk0 + k);
        if (ok) src = reinterpret_cast<const uint4*>(recg + (uint64_t)((m >> 8) & 0xffu) * R32 + at);
      }
      v[r] = src ? load_global(src) : make_uint4(0u, 0u, 0u, 0u);   // not flat: the loop's LDS waits stay short
    }
  };
  auto commit = [&](int gi) {
    const int e_lo = sm.grp[gi];
    const int ch_lo = sm.ent_base[e_lo];
    const int n_pieces = (sm.ent_base[sm.grp[gi + 1]] - ch_lo) * SLOTS;
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int i = tid + r * NT;
      if (i < n_pieces) {
        const int chl = i / SLOTS;
        const int k = i % SLOTS;
        if ((meta[r] >> 16) == 0u) {
          const int un = k / (kUnitBlocks + 1);
          const int w = k % (kUnitBlocks + 1);
          if (w == 0) {
            sm.scales[(int)(meta[r] & 0xffu) - e_lo][un] = v[r];
          } else {
            const uint4 x = v[r];
            sm.planes[chl][un * kUnitBlocks + w - 1] = make_uint4(~x.x, ~x.y, ~x.z, ~x.w);
          }
        } else if (k < TB) {
          sm.planes[chl][k] = v[r];
        }
      }
    }
  };

  if (n_grp > 0) issue(0);
  for (int gi = 0; gi < n_grp; ++gi) {
    const int e_lo = __builtin_amdgcn_readfirstlane(sm.grp[gi]);
    const int e_hi = __builtin_amdgcn_readfirstlane(sm.grp[gi + 1]);
    const int ch_lo = __builtin_amdgcn_readfirstlane(sm.ent_base[e_lo]);
    commit(gi);
    __syncthreads();
    // coefficients q_h 2^(3-t_h) Delta_b for every entry, block and head of the group
    for (int i = tid; i < (e_hi - e_lo) * TB; i += NT) {   // one (entry, block) per thread, all heads
      const int el = i / TB;
      const int b = i % TB;
      const float dl = __half2float(reinterpret_cast<const __half*>(&sm.scales[el][0])[b]);
      const int row = sm.ent_base[e_lo + el] - ch_lo;
      float qh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) qh[h] = sm.ent_q[e_lo + el][h];
#pragma unroll
      for (int h = 0; h < G; ++h) sm.coef[row][b][h] = 2.0f * (qh[h] * dl);   // rounded, then doubled
    }
    __syncthreads();
    if (gi + 1 < n_grp) issue(gi + 1);

    // ---- 3. reconstruct and accumulate.  Lane l owns block bl = 2wv + l/32 and,
    // in it, keys 4 (l%32) .. 4 (l%32) + 3, bits 4 (l%8) .. of the block's word
    // (l%32)/8: a lane reads one 32-bit word per plane row (a quarter of the
    // row), which keeps the loop's LDS reads to what it uses.
    if (kWaveBlocks * wv < nvalid) {
      const int bit0 = 4 * (lane & 7);
      // the group's entries (at most 64: each starts in one of its 64 chunk
      // slots), one per lane; the loop reads them lane by lane into scalars
      // Per lane: chunk base within the group (< 128) | union depth << 8, and
      // for G <= 4 the level masks in bits 12 .. 27 of the same word.
      constexpr int MB = 4 * G;
      const bool mine = e_lo + lane < e_hi;
      const uint64_t lword = mine ? sm.ent_word[e_lo + lane] : 0ull;
      int linfo = 0;
      if (mine) {
        const int b0 = sm.ent_base[e_lo + lane], b1 = sm.ent_base[e_lo + lane + 1];
        linfo = (b0 - ch_lo) | (b1 - b0) << 8;
        if (MB <= 16) linfo |= (int)lword << 12;
      }
      // a 32-bit word where the masks fit, so a mask test sets the branch condition
      using Word = std::conditional_t<(MB <= 32), uint32_t, uint64_t>;
      for (int e = e_lo; e < e_hi; ++e) {
        const uint32_t info = (uint32_t)__builtin_amdgcn_readlane(linfo, e - e_lo);
        Word word;
        if constexpr (MB <= 16) {
          word = info >> 12;
        } else if constexpr (MB <= 32) {
          word = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lword, e - e_lo);
        } else {
          word = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lword, e - e_lo) |
                 (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lword >> 32), e - e_lo) << 32;
        }
        const int cb = (int)(info & 0xffu);
        const int tb = (int)((info >> 8) & 0xfu);
        const uint32_t* pp = reinterpret_cast<const uint32_t*>(&sm.planes[cb][bl]) + ((lane & 31) >> 3);
        // the lane's word of each plane row: all four rows are read (within the
        // padded array), only tb of them used
        const uint32_t w0 = pp[0], w1 = pp[4 * TB], w2 = pp[8 * TB], w3 = pp[12 * TB];
        float cf[G];
#pragma unroll
        for (int h = 0; h < G; ++h) cf[h] = sm.coef[cb][bl][h];
        int r[kSub];
        // one depth t: float(r_t) once, then every head that reads exactly t planes
        // adds (2c) r_t per key and 2c to its per-lane sum (c (2 r_t + 1) in total)
        auto level = [&](int t) {
          float f[kSub];
#pragma unroll
          for (int s2 = 0; s2 < kSub; ++s2) f[s2] = (float)r[s2];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            if (!(word & ((Word)1 << ((t - 1) * G + h)))) continue;
#pragma unroll
            for (int s2 = 0; s2 < kSub; ++s2) acc[s2][h] = fmaf(cf[h], f[s2], acc[s2][h]);
            half_sum[h] += cf[h];
          }
        };
        // signed prefixes MSB first (plane 0 is stored complemented): r_1 = b_0 - 1,
        // r_{t+1} = 2 r_t + b_t
#pragma unroll
        for (int s2 = 0; s2 < kSub; ++s2) r[s2] = __builtin_amdgcn_sbfe((int)w0, bit0 + s2, 1);
        constexpr Word kHeads = (Word)((1ull << G) - 1ull);
        if (word & kHeads) level(1);
        if (tb > 1) {
#pragma unroll
          for (int s2 = 0; s2 < kSub; ++s2) r[s2] = 2 * r[s2] + (int)__builtin_amdgcn_ubfe(w1, bit0 + s2, 1);
          if (word & (kHeads << G)) level(2);
          if (tb > 2) {
#pragma unroll
            for (int s2 = 0; s2 < kSub; ++s2) r[s2] = 2 * r[s2] + (int)__builtin_amdgcn_ubfe(w2, bit0 + s2, 1);
            if (word & (kHeads << (2 * G))) level(3);
            if (tb > 3) {
#pragma unroll
              for (int s2 = 0; s2 < kSub; ++s2) r[s2] = 2 * r[s2] + (int)__builtin_amdgcn_ubfe(w3, bit0 + s2, 1);
              level(4);
            }
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- 4. scores: sum_c (2c) r + (1/2) sum_c 2c = sum_c c (2 r + 1) ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int s = 0; s < kSub; ++s) acc[s][h] += 0.5f * half_sum[h];
  }
  if (bl < nvalid) {
    // a lane's 4 keys are consecutive: one 16-byte store per head where the rows
    // allow it (so a wavefront writes 1 KB runs), else one store per key
    const int64_t j0 = (blk0 + bl) * kBlock + 4 * (lane & 31);
    const bool vec = (a.ld & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
    if (vec && j0 + 3 < a.n) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        store_global(reinterpret_cast<float4*>(a.scores + (g * G + h) * a.ld + j0),
                     make_float4(acc[0][h], acc[1][h], acc[2][h], acc[3][h]));
    } else {
#pragma unroll
      for (int s2 = 0; s2 < kSub; ++s2) {
        if (j0 + s2 < a.n) {
#pragma unroll
          for (int h = 0; h < G; ++h) a.scores[(g * G + h) * a.ld + j0 + s2] = acc[s2][h];
        }
      }
    }
  }

  // ---- 5. fused first-digit histogram of the selection ----
  if constexpr (FUSE) {
    constexpr int HR = kHistHeads<G, TB>;
    static_assert(HR >= 1 && TB * kBlock < 65536, "16-bit counts of at least one head must fit");
    uint32_t* lh = reinterpret_cast<uint32_t*>(&sm);
#pragma unroll
    for (int h0 = 0; h0 < G; h0 += HR) {
      __syncthreads();   // every wave is past the staging memory (or the previous round's flush)
      for (int i = tid; i < HR * kHistWords; i += NT) lh[i] = 0u;
      __syncthreads();
      if (bl < nvalid) {
#pragma unroll
        for (int s2 = 0; s2 < kSub; ++s2) {
          const int64_t j = (blk0 + bl) * kBlock + 4 * (lane & 31) + s2;
          if (j < a.n) {
#pragma unroll
            for (int hh = 0; hh < HR; ++hh) {
              if (h0 + hh < G) {
                const uint32_t b = order_key(acc[s2][h0 + hh]) >> kSelDigit0;
                atomicAdd(&lh[hh * kHistWords + (b >> 1)], 1u << (16 * (b & 1u)));
              }
            }
          }
        }
      }
      __syncthreads();
      for (int i = tid; i < HR * kHistWords; i += NT) {
        const int hh = h0 + i / kHistWords;
        const uint32_t v = lh[i];
        if (hh < G && v) {
          uint32_t* gh = a.hist + (g * G + hh) * kSelBins + 2 * (i % kHistWords);
          if (v & 0xffffu) atomicAdd(gh, v & 0xffffu);
          if (v >> 16) atomicAdd(gh + 1, v >> 16);
        }
      }
    }
  }
}

// Tile size per residency: device memory likes many small tiles (occupancy);
// reading pinned host memory in place wants long contiguous runs per
// channel-plane (>= 512 bytes keeps the host link near its streaming rate).
constexpr int kTileDevice = 8;    // 1024 keys, 256 threads
template <int G>
struct HostTile {
  static constexpr int TB = G <= 4 ? 32 : 16;   // LDS for the coefficients bounds it for large G
};

// Workgroup ids are dealt round-robin to the 8 XCDs, each with its own L2.  The
// kernel gives XCD x = w % 8 the x-th eighth of every KV head's tiles (t8 =
// ceil(tiles / 8) of them), head after head: neighbouring tiles, whose head runs
// can share a cache line at their boundary, mostly meet in the same L2, and
// every XCD gets the same mix of heads (whose union depths, and so work, differ).
constexpr int kXcds = 8;

template <int G, int TB, bool FUSE>
__global__ __launch_bounds__((Cfg<G, TB>::threads)) void scan_kernel(ScanArgs a, int64_t tiles, int64_t total) {
  __shared__ ScanSmem<G, TB> sm;
  const int64_t w = blockIdx.x;
  const int64_t t8 = (tiles + kXcds - 1) / kXcds;
  const int64_t j = w / kXcds;
  const int64_t g = j / t8;
  const int64_t tile = (w % kXcds) * t8 + j % t8;
  if (tile >= tiles) return;
  const int64_t L = g * tiles + tile;   // distinct in [0, total)
  if (a.zero) {   // the selection's counters: one slice per workgroup
    const int64_t slice = (a.zero_words + total - 1) / total;
    const int64_t z1 = min((L + 1) * slice, a.zero_words);
    for (int64_t i = L * slice + threadIdx.x; i < z1; i += Cfg<G, TB>::threads) a.zero[i] = 0u;
  }
  scan_tile<G, TB, FUSE>(a, g, tile, sm);
}

// ---------------------------------------------------------------------------
// Host-resident records, staged: the scan's input is first gathered from
// pinned host memory into an HBM mirror of the records with long contiguous
// reads (each channel's prefix run of the union depth, split into 32 KB
// pieces), which keeps the host link at its streaming rate.  Launch i copies
// KV heads [i*hb, (i+1)*hb) while the same launch's other workgroups scan the
// heads staged by launch i-1, so the copy of one head overlaps the compute of
// the previous one; kernel boundaries order the copy before its scan.
// ---------------------------------------------------------------------------

constexpr int64_t kCopyPiece = 32768;   // bytes per copy workgroup

inline int64_t copy_pieces_per_head(const Layout& L, int d) {
  return (int64_t)d * ((L.R + kCopyPiece - 1) / kCopyPiece);
}

template <int G, int TB>
__device__ __forceinline__ void copy_piece(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                           const uint8_t* __restrict__ uni, int64_t g, int d,
                                           int64_t H, int64_t P, int64_t R, int64_t piece,
                                           ScanSmem<G, TB>& sm) {
  constexpr int NT = Cfg<G, TB>::threads;
  constexpr int PER = (int)(kCopyPiece / 16 / NT);
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  // pieces of channel c's run [0, H + (t-1) P), t = union depth
  const int c = tid;
  const int t = c < d ? (int)uni[g * d + c] : 0;
  const int64_t bytes = t > 0 ? H + (int64_t)(t - 1) * P : 0;
  const int np = (int)((bytes + kCopyPiece - 1) / kCopyPiece);
  const int inc = (int)wave_inclusive_sum((uint32_t)np);
  if (lane == 63) sm.wsum[0][wv] = inc;
  if (tid == 0) sm.n_grp = -1;
  __syncthreads();
  int base = 0;
  for (int x = 0; x < wv; ++x) base += sm.wsum[0][x];
  const int first = base + inc - np;
  if (np > 0 && piece >= first && piece < first + np) {
    sm.n_grp = c;                                    // owner channel of this piece
    sm.wsum[1][0] = (int)(piece - first);            // piece index within the run
    sm.wsum[1][1] = (int)((bytes + 15) / 16);        // run length in 16-byte units
  }
  __syncthreads();
  const int owner = sm.n_grp;
  if (owner < 0) return;                             // past the last piece of this head
  const int64_t u0 = (int64_t)sm.wsum[1][0] * (kCopyPiece / 16);
  const int64_t units = sm.wsum[1][1];
  const uint4* s4 = reinterpret_cast<const uint4*>(src + (g * d + owner) * R);
  uint4* d4 = reinterpret_cast<uint4*>(dst + (g * d + owner) * R);
  uint4 v[PER];
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int64_t i = u0 + (int64_t)r * NT + tid;
    v[r] = i < units ? s4[i] : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int64_t i = u0 + (int64_t)r * NT + tid;
    if (i < units) d4[i] = v[r];
  }
}

template <int G, int TB>
__global__ __launch_bounds__((Cfg<G, TB>::threads)) void stage_scan_kernel(
    ScanArgs a, const uint8_t* __restrict__ host, int64_t copy_g0, int copy_heads, int64_t ncopy,
    int64_t scan_g0, int scan_heads, int64_t tiles) {
  __shared__ ScanSmem<G, TB> sm;
  const int64_t b = blockIdx.x;
  const int64_t scan_blocks = tiles * scan_heads;
  if (b < scan_blocks) {
    scan_tile<G, TB>(a, scan_g0 + b / tiles, b % tiles, sm);
  } else {
    const int64_t cb = b - scan_blocks;
    if (cb < ncopy * copy_heads)
      copy_piece<G, TB>(host, const_cast<uint8_t*>(a.rec), a.uni, copy_g0 + cb / ncopy, a.d, a.H, a.P,
                        a.R, cb % ncopy, sm);
  }
}

// Paging of a scan: the page table and the keys per page (0: contiguous records).
struct Paging {
  const uint8_t* const* table;
  int64_t npages;
  int64_t page_keys;
};

template <int G, int TB>
hipError_t launch_g(const uint8_t* rec, const float* q, const uint8_t* depth, const uint8_t* uni,
                    int h_kv, const Layout& L, int d, float* scores, int64_t ld, uint32_t* zero,
                    int64_t zero_words, uint32_t* hist, const Paging& pg, hipStream_t s) {
  ScanArgs a{rec, q, depth, uni, L.n, L.nb, L.H, L.P, L.R, d, scores, ld, zero, zero_words, hist, nullptr, 0, 1};
  if (pg.table) {
    // page records are laid out for page_keys keys; tiles never straddle pages
    const Layout P = make_layout(pg.page_keys);
    if (pg.page_keys % (TB * kBlock) != 0) return hipErrorInvalidValue;
    a.H = P.H;
    a.P = P.P;
    a.R = P.R;
    a.pages = pg.table;
    a.npages = pg.npages;
    a.page_tiles = pg.page_keys / (TB * kBlock);
  }
  const int64_t tiles = (L.nb + TB - 1) / TB;
  const int64_t total = tiles * h_kv;
  const int64_t grid = kXcds * h_kv * ((tiles + kXcds - 1) / kXcds);
  if (hist) {
    scan_kernel<G, TB, true><<<(unsigned)grid, Cfg<G, TB>::threads, 0, s>>>(a, tiles, total);
    return hipGetLastError();
  }
  scan_kernel<G, TB, false><<<(unsigned)grid, Cfg<G, TB>::threads, 0, s>>>(a, tiles, total);
  return hipGetLastError();
}

template <int G>
hipError_t launch_staged_g(const uint8_t* host, uint8_t* staging, const float* q, const uint8_t* depth,
                           const uint8_t* uni, int h_kv, const Layout& L, int d, float* scores,
                           int64_t ld, hipStream_t s) {
  constexpr int TB = kTileDevice;
  const ScanArgs a{staging, q, depth, uni, L.n, L.nb, L.H, L.P, L.R, d, scores, ld, nullptr, 0, nullptr,
                   nullptr, 0, 1};
  const int64_t tiles = (L.nb + TB - 1) / TB;
  const int64_t ncopy = copy_pieces_per_head(L, d);
  // heads per launch: about 64 MB of records per launch
  const int64_t head_bytes = (int64_t)d * L.R;
  const int hb = (int)std::max<int64_t>(
      1, std::min<int64_t>(h_kv, (int64_t(64) << 20) / std::max<int64_t>(head_bytes, 1)));
  const int steps = (h_kv + hb - 1) / hb;
  for (int i = 0; i <= steps; ++i) {
    const int64_t cg0 = (int64_t)i * hb;
    const int ch = i < steps ? (int)std::min<int64_t>(hb, h_kv - cg0) : 0;
    const int64_t sg0 = (int64_t)(i - 1) * hb;
    const int sh = i > 0 ? (int)std::min<int64_t>(hb, h_kv - sg0) : 0;
    const int64_t blocks = ncopy * ch + tiles * sh;
    stage_scan_kernel<G, TB><<<(unsigned)blocks, Cfg<G, TB>::threads, 0, s>>>(a, host, cg0, ch, ncopy, sg0,
                                                                               sh, tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int G>
hipError_t launch_any(const uint8_t* rec, bool host, const float* q, const uint8_t* depth,
                      const uint8_t* uni, int h_kv, const Layout& L, int d, float* scores, int64_t ld,
                      uint32_t* zero, int64_t zero_words, uint32_t* hist, const Paging& pg, hipStream_t s) {
  if (host)
    return launch_g<G, HostTile<G>::TB>(rec, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words, hist, pg, s);
  return launch_g<G, kTileDevice>(rec, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words, hist, pg, s);
}

}  // namespace

hipError_t launch_scan(const uint8_t* rec, bool host, const float* q, const uint8_t* depth,
                       const uint8_t* uni, int h_kv, int g, const Layout& L, int d,
                       float* scores, int64_t ld, uint32_t* zero, int64_t zero_words, uint32_t* hist,
                       hipStream_t s) {
  return launch_scan_paged(rec, nullptr, 0, 0, host, q, depth, uni, h_kv, g, L, d, scores, ld, zero, zero_words,
                           hist, s);
}

hipError_t launch_scan_paged(const uint8_t* rec, const uint8_t* const* table, int64_t npages, int64_t page_keys,
                             bool host, const float* q, const uint8_t* depth, const uint8_t* uni, int h_kv, int g,
                             const Layout& L, int d, float* scores, int64_t ld, uint32_t* zero, int64_t zero_words,
                             uint32_t* hist, hipStream_t s) {
  if (L.nb == 0) return hipSuccess;
  const Paging pg{table, npages, page_keys};
  switch (g) {
    case 1: return launch_any<1>(rec, host, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words, hist, pg, s);
    case 2: return launch_any<2>(rec, host, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words, hist, pg, s);
    case 4: return launch_any<4>(rec, host, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words, hist, pg, s);
    case 8: return launch_any<8>(rec, host, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words, hist, pg, s);
    case 16: return launch_any<16>(rec, host, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words, hist, pg, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_scan_staged(const uint8_t* host, uint8_t* staging, const float* q, const uint8_t* depth,
                              const uint8_t* uni, int h_kv, int g, const Layout& L, int d, float* scores,
                              int64_t ld, hipStream_t s) {
  if (L.nb == 0) return hipSuccess;
  switch (g) {
    case 1: return launch_staged_g<1>(host, staging, q, depth, uni, h_kv, L, d, scores, ld, s);
    case 2: return launch_staged_g<2>(host, staging, q, depth, uni, h_kv, L, d, scores, ld, s);
    case 4: return launch_staged_g<4>(host, staging, q, depth, uni, h_kv, L, d, scores, ld, s);
    case 8: return launch_staged_g<8>(host, staging, q, depth, uni, h_kv, L, d, scores, ld, s);
    case 16: return launch_staged_g<16>(host, staging, q, depth, uni, h_kv, L, d, scores, ld, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fathom
