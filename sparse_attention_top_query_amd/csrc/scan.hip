// Scan kernels: reconstruct every key from its budgeted plane prefixes and
// accumulate q . k_hat for the query heads of one KV head.
//
// Sources: the ai-feeds digest, Method, key modules 4-5 (only the budgeted
// planes are read, and each channel's value is rebuilt from what was read; the
// paper's Sec 3.5 rule itself is not in the text, so the value taken is the
// midpoint of the prefix's cell of the t-bit mid-rise quantizer), and the
// Fathom arXiv abstract (a t-plane prefix is the t-bit quantizer of the
// channel).  With r_t = (code >> (4-t)) - 2^(t-1), a signed t-bit integer,
//   q * k_hat_t = q Delta 2^(4-t) (r_t + 1/2) = a z_t,
//   a = [q Delta / 16] (one fp32 rounding),  z_t = 2^(7-t) (2 r_t + 1),
// where z_t is an integer in [-127, 127] (a signed byte) and a does not depend
// on the depth.  Each term a z_t is an exact product in the fma, within one
// rounding of q k_hat, so the fp32 sum over m channels stays within about
// (m + 1) 2^-24 sum_c |q_c k_hat_c|.
//
// Work decomposition: one workgroup scores a tile of TB 128-key blocks of one KV
// head for all of its G query heads; each wavefront owns 2 KW blocks, 32 / KW
// lanes per block (KW = 1 from device memory; KW = 2 and 8192-key tiles for
// reading pinned host memory in place).  With KW = 1, lane l owns the keys
// 32 i + jj + 8 s (s = 0..3) of its block, i = (l%32)/8, jj = l%8: the bits
// jj + 8 s of 32-bit word i of each plane row of the block; with KW = 2 it owns
// two such groups of 4 keys, 4 bits apart in the same word.
//  1. The union depths of the KV head list the channels to read; every query
//     head of the group is scored from the one read of the longest prefix.
//  2. Staging, channel group by channel group (64 channel-planes from device
//     memory, 4 from pinned host memory): the tile's slice of each channel's
//     record head (its units' fp16 scales and plane-0 bits) and of planes
//     1..t-1 are loaded with 16-byte loads into registers -- all issued before
//     any LDS write, and those of the next group while the current group is
//     computed -- then stored to LDS, the most significant plane complemented.
//     The same code reads HBM, an HBM staging ring, or pinned host memory over
//     the host link; the tile size sets the contiguous run per channel-plane
//     (16 B per block).
//  3. Per (channel, block) the coefficients a = [q_h Delta / 16] are formed once
//     in LDS.  Per channel, each lane reads its word of each plane row and
//     builds each group of 4 keys' prefixes side by side, one per byte of a
//     register y: plane p's word rotated right by jj + p - 7 puts the group's 4
//     bits at bit 7 - p of bytes 0..3, and one and-or adds them to y (two
//     operations per plane for 4 keys).  The complemented MSB is the byte's sign bit, so after
//     t planes byte s of y is 2^(8-t) r_t of key s; setting bit 7 - t of every
//     byte makes it z_t.  Per depth in use: that one or, then 4 signed-byte
//     conversions to float; per head reading the channel: one fma per key.
#include <hip/hip_fp16.h>

#include <algorithm>
#include <type_traits>

#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kSlackChunks = kPlanes - 1;      // an entry starting in a group ends in it
constexpr int kTileDevice = 8;                 // blocks per tile from device memory: 1024 keys, 256 threads
// Channel-planes per staging group (GS, +3 slack).  For the 1024-key tiles
// that read device memory: 64 as a rule, since each group boundary costs the
// arithmetic two barriers; 32 for rows of more than 8 tiles per CU in all when
// 2 to 8 query heads share a KV head, where the smaller staging memory and
// registers raise the workgroups a CU holds at once (for 4 heads 71 against 82
// VGPRs, 7 workgroups instead of 5), so fewer generations of tiles start up in
// turn (10-14% faster scans from 393216 keys up; with 1 or 16 heads the
// occupancy does not change and 64 stays).  For the longer tiles that read
// pinned host memory: 4, the least that keeps every group non-empty (an
// entry's first chunk is at most 4 past the previous one's).  The link then
// sees each workgroup's reads as a stream of small batches from a few channels
// at a time, which it serves at up to 99% of the copy engine's rate, against
// 96% with 32-plane batches (the arithmetic is idle enough to take the extra
// group boundaries).
template <int TB>
constexpr int kStageGroup = TB > kTileDevice ? 4 : 64;
constexpr int kDeviceRunGroup = 32;
constexpr int64_t kDeviceRunTiles = 2048;     // 8 per CU
template <int GS>
struct Stage {
  static_assert(GS >= kPlanes, "first chunks of consecutive entries are at most 4 apart: groups of >= 4 are never empty");
  static constexpr int group = GS;
  static constexpr int chunks = group + kSlackChunks;
  static constexpr int entries = chunks;        // entries have >= 1 chunk
};
constexpr int kMaxChunks = kPlanes * kMaxD;
constexpr int kSub = kBlock / 32;              // 32-key words per block, keys per byte register

// KW byte registers of 4 keys per lane: a wavefront covers 2 KW blocks, 32 / KW
// lanes per block.  One (KW = 1, 4 wavefronts per SIMD at 131k keys) where
// the arithmetic must hide latency; two where the tile must be long (the
// host-link scan: 8192-key tiles, 1-KB runs per channel-plane, still 1024
// threads).
template <int G, int TB, int KW = 1, int GS = kStageGroup<TB>>
struct Cfg {
  static constexpr int keys = kSub * KW;              // keys per lane
  static constexpr int wave_blocks = 2 * KW;          // 128-key blocks per wavefront
  static constexpr int threads = 64 * TB / wave_blocks;
  static constexpr int units = TB / kUnitBlocks;      // 1024-key record units per tile
  static constexpr int slots = TB + units;            // 16-byte pieces per chunk slot
  static constexpr int ppt = (Stage<GS>::chunks * slots + threads - 1) / threads;
  static_assert(threads >= kMaxD && threads <= 1024, "one thread per channel in the list build");
  static_assert(TB % kUnitBlocks == 0, "tiles hold whole 1024-key units");
};

template <int G, int TB, int GS = kStageGroup<TB>>
struct ScanSmem {
  uint4 planes[Stage<GS>::chunks + kPlanes - 1][TB];   // staged plane bits (plane 0 complemented); the last
                                                   // rows pad reads of a prefix's unread planes
  uint4 scales[Stage<GS>::entries][TB / kUnitBlocks];  // staged fp16 scales per entry of the group
  float coef[Stage<GS>::chunks][TB][G];            // a = [q_h Delta_b / 16] per block and head, in the
                                                   // row of the entry's first chunk (for G = 4 a row has the
                                                   // planes' stride)
  float ent_q[kMaxD][G];                           // q_h / 16 of each list entry
  uint64_t ent_word[kMaxD + 1];                    // level masks: bit (t-1) G + h iff head h reads t planes
  uint16_t ent_base[kMaxD + 1];                    // first chunk of entry e (prefix sum)
  uint16_t grp[kMaxChunks / Stage<GS>::group + 2];  // first entry of each staging group
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
  int64_t zero_slice;        // words per workgroup: ceil(zero_words / workgroups)
  uint32_t* hist;            // selection histograms [h_q][kSelBins] to add to (fused scans)
  // paged records (may be null): pages[g * npages + p] is the device-visible
  // base of page p of KV head g, [d][R] bytes for page_tiles tiles of keys,
  // laid out as whole records of those keys (H, P, R are the page's)
  const uint8_t* const* pages;
  int64_t npages;
  int64_t page_tiles;
  // ring of staged heads (0: none): KV head g's records are at slot g % ring
  int64_t ring;
};

// Entry word: one G-bit mask per depth t = 1..4, bit (t - 1) G + h set iff head h
// reads exactly t planes of the channel (at most 64 bits for G <= 16).  The
// union depth is the entry's chunk count.

// The fused first-digit histograms live in the tile's staging memory, which is
// dead once the last group is scored: 16-bit counts, two bins per word (a tile
// holds at most 8192 keys), for as many heads per round as fit.
constexpr int kHistWords = kSelBins / 2;
template <int G, int TB, int GS = kStageGroup<TB>>
constexpr int kHistHeads = (int)(sizeof(ScanSmem<G, TB, GS>) / 4 / kHistWords) < G
                               ? (int)(sizeof(ScanSmem<G, TB, GS>) / 4 / kHistWords) : G;

// Scores of tile `tile` (TB blocks) of KV head g for all its query heads, left
// in acc: acc[s][h] is the score for query head g G + h of the key
// tile_key(s) of the tile.
template <int G, int TB, int KW, int GS>
__device__ __forceinline__ void scan_tile_acc(const ScanArgs& a, int64_t g, int64_t tile, ScanSmem<G, TB, GS>& sm,
                                              float (&acc)[Cfg<G, TB, KW>::keys][G]) {
  using C = Cfg<G, TB, KW, GS>;
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
  constexpr int LB = 32 / KW;                        // lanes per block
  const int bl = C::wave_blocks * wv + lane / LB;    // block of this lane within the tile
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
        sm.ent_q[e][h] = ldexpf(qc[h], -4);   // exact power-of-two scaling
      }
      sm.ent_word[e] = word;
      sm.ent_base[e] = (uint16_t)base;
      if (e == n_ent - 1) {
        sm.ent_base[n_ent] = (uint16_t)(base + u);
        // an entry joins the group holding its first chunk; first chunks are at
        // most 4 apart, so every group up to this one is non-empty
        sm.n_grp = base / Stage<GS>::group + 1;
        sm.grp[base / Stage<GS>::group + 1] = (uint16_t)n_ent;
      }
#pragma unroll
      for (int p = 0; p < kPlanes; ++p)
        if (p < u) sm.chunk_meta[base + p] = (uint32_t)e | (uint32_t)c << 8 | (uint32_t)p << 16;
    }
    if (tid == 0 && n_ent == 0) sm.n_grp = 0;
    __syncthreads();
    if (act) {
      const int gi = base / Stage<GS>::group;
      if (e == 0 || sm.ent_base[e - 1] / Stage<GS>::group != gi) sm.grp[gi] = (uint16_t)e;
    }
    __syncthreads();
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int s = 0; s < C::keys; ++s) acc[s][h] = 0.0f;
  }

  // the tile's records: the KV head's own, or its page (addressed page-locally)
  const uint8_t* recg;
  int64_t ablk0;   // first block of the tile within those records
  if (a.pages) {
    const uint32_t pt = (uint32_t)a.page_tiles;
    const uint32_t pg = (uint32_t)tile / pt;
    recg = a.pages[g * a.npages + pg];
    ablk0 = (int64_t)((uint32_t)tile - pg * pt) * TB;
  } else {
    recg = rec + (a.ring ? (int64_t)((uint32_t)g % (uint32_t)a.ring) : g) * d * R;
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
    // coefficients a = [q_h Delta_b / 16] for every entry, block and head of the group
    for (int i = tid; i < (e_hi - e_lo) * TB; i += NT) {   // one (entry, block) per thread, all heads
      const int el = i / TB;
      const int b = i % TB;
      const float dl = __half2float(reinterpret_cast<const __half*>(&sm.scales[el][0])[b]);
      const int row = sm.ent_base[e_lo + el] - ch_lo;
      float qh[G];
#pragma unroll
      for (int h = 0; h < G; ++h) qh[h] = sm.ent_q[e_lo + el][h];
#pragma unroll
      for (int h = 0; h < G; ++h) sm.coef[row][b][h] = qh[h] * dl;   // one rounding
    }
    __syncthreads();
    if (gi + 1 < n_grp) issue(gi + 1);
    // A CU runs several tiles at once and its arbiter favours the oldest
    // wavefronts, so the youngest tile would finish alone with the VALU half
    // idle.  Lowering a wavefront's priority as its tile advances lets the
    // laggards catch up, group by group.
    if (gi == 0) __builtin_amdgcn_s_setprio(3);
    else if (gi == 1) __builtin_amdgcn_s_setprio(2);
    else if (gi == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);

    // ---- 3. reconstruct and accumulate.  Lane l owns block bl = 2 KW wv + l/LB
    // and, in it, the keys 32 i + jj + JS k + 8 s (k < KW, s = 0..3) of its
    // block's 32-key word i = (l%LB)/JS, jj = l%JS, JS = 8/KW: bits jj + JS k +
    // 8 s of that word of each plane row, so a lane reads one 32-bit word per
    // plane row and finds its KW groups of 4 bits at a stride of 8.  Rotating
    // the word right by jj + JS k + p - 7 brings group k to bit 7 - p of bytes
    // 0..3, where plane p belongs in the byte-wise signed prefix y[k].
    if (C::wave_blocks * wv < nvalid) {
      constexpr int JS = 8 / KW;
      const int jj = lane % JS;
      uint32_t rot[kPlanes][KW];
#pragma unroll
      for (int p = 0; p < kPlanes; ++p)
#pragma unroll
        for (int k = 0; k < KW; ++k) rot[p][k] = (uint32_t)(jj + JS * k + 25 + p) & 31u;
      // the group's entries (at most 64: each starts in one of its <= 64 chunk
      // slots), one per lane; the loop reads them lane by lane into scalars.
      // Per lane: chunk base within the group (< 128) in bits 0..7; for G <= 4
      // the level masks in bits 8..23, a flag per depth read by some head in
      // bits 24..27 and flags for union depth > 1, > 2, > 3 in bits 28..30, so
      // every test of the loop is one scalar bit test; for larger G the union
      // depth in bits 8..11 and the masks read separately.
      constexpr int MB = 4 * G;
      const bool mine = e_lo + lane < e_hi;
      const uint64_t lword = mine ? sm.ent_word[e_lo + lane] : 0ull;
      int linfo = 0;
      if (mine) {
        const int b0 = sm.ent_base[e_lo + lane], b1 = sm.ent_base[e_lo + lane + 1];
        const int u = b1 - b0;
        if constexpr (MB <= 16) {
          int any = 0;
#pragma unroll
          for (int t = 0; t < kPlanes; ++t) any |= ((lword >> (G * t)) & ((1u << G) - 1u)) ? 1 << t : 0;
          linfo = (b0 - ch_lo) | (int)lword << 8 | any << 24 | (u > 1) << 28 | (u > 2) << 29 | (u > 3) << 30;
        } else {
          linfo = (b0 - ch_lo) | u << 8;
        }
      }
      // a 32-bit word where the masks fit, so a mask test sets the branch condition
      using Word = std::conditional_t<(MB <= 32), uint32_t, uint64_t>;
      for (int e = e_lo; e < e_hi; ++e) {
        const uint32_t info = (uint32_t)__builtin_amdgcn_readlane(linfo, e - e_lo);
        Word word;
        if constexpr (MB <= 16) {
          word = info >> 8;
        } else if constexpr (MB <= 32) {
          word = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lword, e - e_lo);
        } else {
          word = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lword, e - e_lo) |
                 (uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lword >> 32), e - e_lo) << 32;
        }
        // some head reads exactly t planes; the union depth exceeds t
        auto has_level = [&](int t) -> bool {
          if constexpr (MB <= 16) return (info >> (23 + t)) & 1u;
          else return (word & ((Word)((1ull << G) - 1ull) << (G * (t - 1)))) != 0;
        };
        auto deeper = [&](int t) -> bool {
          if constexpr (MB <= 16) return (info >> (27 + t)) & 1u;
          else return (int)((info >> 8) & 0xfu) > t;
        };
        const int cb = (int)(info & 0xffu);
        const uint32_t* pp = reinterpret_cast<const uint32_t*>(&sm.planes[cb][bl]) + (lane % LB) / JS;
        // the lane's word of each plane row: all four rows are read (within the
        // padded array), only tb of them used
        const uint32_t w0 = pp[0], w1 = pp[4 * TB], w2 = pp[8 * TB], w3 = pp[12 * TB];
        float cf[G];
#pragma unroll
        for (int h = 0; h < G; ++h) cf[h] = sm.coef[cb][bl][h];
        // y[k]: byte s holds the signed prefix of key (k, s) read so far, MSB at
        // bit 7 (plane 0 is stored complemented, so bit 7 is the sign); one
        // depth t: z = y | 2^(7-t) per byte is 2^(7-t) (2 r_t + 1), converted
        // once (signed byte to float), then every head that reads exactly t
        // planes adds a z per key
        uint32_t y[KW];
#pragma unroll
        for (int k = 0; k < KW; ++k) y[k] = __builtin_amdgcn_alignbit(w0, w0, rot[0][k]) & 0x80808080u;
        auto plane = [&](uint32_t w, int p) {
#pragma unroll
          for (int k = 0; k < KW; ++k) y[k] |= __builtin_amdgcn_alignbit(w, w, rot[p][k]) & (0x80808080u >> p);
        };
        auto level = [&](int t) {
          float f[C::keys];
#pragma unroll
          for (int k = 0; k < KW; ++k) {
            const uint32_t z = y[k] | (0x01010101u << (7 - t));
#pragma unroll
            for (int s2 = 0; s2 < kSub; ++s2) f[kSub * k + s2] = (float)(int)(int8_t)(z >> (8 * s2));
          }
#pragma unroll
          for (int h = 0; h < G; ++h) {
            if (!(word & ((Word)1 << ((t - 1) * G + h)))) continue;
#pragma unroll
            for (int s2 = 0; s2 < C::keys; ++s2) acc[s2][h] = fmaf(cf[h], f[s2], acc[s2][h]);
          }
        };
        if (has_level(1)) level(1);
        if (deeper(1)) {
          plane(w1, 1);
          if (has_level(2)) level(2);
          if (deeper(2)) {
            plane(w2, 2);
            if (has_level(3)) level(3);
            if (deeper(3)) {
              plane(w3, 3);
              level(4);
            }
          }
        }
      }
    }
    __syncthreads();
  }

}

// Key of acc[s] of this thread within its tile: block 2 KW w + l/LB, word
// (l%LB)/JS, bit l%JS + JS (s/4) + 8 (s%4) of that word (LB = 32/KW, JS = 8/KW).
template <int TB, int KW>
__device__ __forceinline__ int tile_key(int s) {
  constexpr int LB = 32 / KW, JS = 8 / KW;
  const int lane = threadIdx.x & 63;
  return (2 * KW * (int)(threadIdx.x >> 6) + lane / LB) * kBlock + 32 * ((lane % LB) / JS) + lane % JS +
         JS * (s / kSub) + 8 * (s % kSub);
}

// Scores of the tile to a.scores, one store per key and head.
template <int G, int TB, int KW>
__device__ __forceinline__ void store_tile(const ScanArgs& a, int64_t g, int64_t tile,
                                           const float (&acc)[Cfg<G, TB, KW>::keys][G]) {
  const int64_t key0 = tile * TB * kBlock;
#pragma unroll
  for (int s2 = 0; s2 < Cfg<G, TB, KW>::keys; ++s2) {
    const int64_t j = key0 + tile_key<TB, KW>(s2);
    if (j < a.n) {
#pragma unroll
      for (int h = 0; h < G; ++h) store_global(a.scores + (g * G + h) * a.ld + j, acc[s2][h]);
    }
  }
}

// The tile's scores counted into hist[h][kSelBins] by their first selection
// digit: an LDS histogram per round of heads (16-bit counts in the staging
// memory, dead once the tile is scored), then one global atomic per non-empty
// bin.
template <int G, int TB, int KW, int GS>
__device__ __forceinline__ void hist_tile(const ScanArgs& a, uint32_t* hist, int64_t g, int64_t tile,
                                          const float (&acc)[Cfg<G, TB, KW>::keys][G], ScanSmem<G, TB, GS>& sm) {
  constexpr int NT = Cfg<G, TB, KW>::threads;
  constexpr int HR = kHistHeads<G, TB, GS>;
  static_assert(HR >= 1 && TB * kBlock < 65536, "16-bit counts of at least one head must fit");
  const int tid = threadIdx.x;
  const int64_t key0 = tile * TB * kBlock;
  uint32_t* lh = reinterpret_cast<uint32_t*>(&sm);
#pragma unroll
  for (int h0 = 0; h0 < G; h0 += HR) {
    __syncthreads();   // every wave is past the staging memory (or the previous round's flush)
    for (int i = tid; i < HR * kHistWords; i += NT) lh[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < Cfg<G, TB, KW>::keys; ++s2) {
      if (key0 + tile_key<TB, KW>(s2) < a.n) {
#pragma unroll
        for (int hh = 0; hh < HR; ++hh) {
          if (h0 + hh < G) {
            const uint32_t b = order_key(acc[s2][h0 + hh]) >> kSelDigit0;
            atomicAdd(&lh[hh * kHistWords + (b >> 1)], 1u << (16 * (b & 1u)));
          }
        }
      }
    }
    __syncthreads();
    for (int i = tid; i < HR * kHistWords; i += NT) {
      const int hh = h0 + i / kHistWords;
      const uint32_t v = lh[i];
      if (hh < G && v) {
        uint32_t* gh = hist + (g * G + hh) * kSelBins + 2 * (i % kHistWords);
        if (v & 0xffffu) atomicAdd(gh, v & 0xffffu);
        if (v >> 16) atomicAdd(gh + 1, v >> 16);
      }
    }
  }
}

// Scores of tile `tile` (TB blocks) of KV head g, all its query heads.  With
// FUSE, the tile's scores are also counted into a.hist by their first
// selection digit.
template <int G, int TB, int KW = 1, bool FUSE = false, int GS = kStageGroup<TB>>
__device__ __forceinline__ void scan_tile(const ScanArgs& a, int64_t g, int64_t tile, ScanSmem<G, TB, GS>& sm) {
  float acc[Cfg<G, TB, KW>::keys][G];
  scan_tile_acc<G, TB, KW, GS>(a, g, tile, sm, acc);
  store_tile<G, TB, KW>(a, g, tile, acc);
  if constexpr (FUSE) hist_tile<G, TB, KW, GS>(a, a.hist, g, tile, acc, sm);
}

// Tile size per residency: device memory likes many small tiles (occupancy);
// reading pinned host memory in place wants long contiguous runs per
// channel-plane (>= 512 bytes keeps the host link near its streaming rate; 1 KB
// runs, 8192-key tiles at 8 keys per lane, scan 1% faster than 512-byte ones).
// Paged host records keep 4096-key tiles so that pages of any multiple of 4096
// keys hold whole tiles.
template <int G>
struct HostTile {
  // 8 keys per lane needs twice the accumulators; the coefficients' LDS bounds
  // the tile for larger G
  static constexpr int KW = G <= 4 ? 2 : 1;
  static constexpr int TB = G <= 4 ? 64 : 16;
};
template <int G>
struct PagedHostTile {
  static constexpr int KW = 1;
  static constexpr int TB = G <= 4 ? 32 : 16;
};

// Workgroup ids are dealt round-robin to the 8 XCDs, each with its own L2.  The
// kernel gives XCD x = w % 8 the x-th eighth of every KV head's tiles (t8 =
// ceil(tiles / 8) of them), head after head: neighbouring tiles, whose head runs
// can share a cache line at their boundary, mostly meet in the same L2, and
// every XCD gets the same mix of heads (whose union depths, and so work, differ).
constexpr int kXcds = 8;

template <int G, int TB, int KW, bool FUSE, int GS = kStageGroup<TB>>
__global__ __launch_bounds__((Cfg<G, TB, KW>::threads)) void scan_kernel(ScanArgs a, int64_t tiles, int64_t total) {
  __shared__ ScanSmem<G, TB, GS> sm;
  // 32-bit index arithmetic (tiles and grids stay far below 2^31): a 64-bit
  // division by a run-time value is a long scalar sequence at every start
  const uint32_t w = blockIdx.x;
  const uint32_t t8 = (uint32_t)((tiles + kXcds - 1) / kXcds);
  const uint32_t j = w / kXcds;
  const uint32_t g = j / t8;
  const int64_t tile = (int64_t)((w % kXcds) * t8 + (j - g * t8));
  if (tile >= tiles) return;
  const int64_t L = (int64_t)g * tiles + tile;   // distinct in [0, total)
  if (a.zero) {   // the selection's counters: one slice of zero_slice words per workgroup
    const int64_t z1 = min((L + 1) * a.zero_slice, a.zero_words);
    for (int64_t i = L * a.zero_slice + threadIdx.x; i < z1; i += Cfg<G, TB, KW>::threads) a.zero[i] = 0u;
  }
  scan_tile<G, TB, KW, FUSE, GS>(a, g, tile, sm);
}

// ---------------------------------------------------------------------------
// Host-resident records, staged: the scan's input is first gathered from
// pinned host memory into HBM with contiguous reads (each channel's prefix run
// of the union depth, split into 4 KB pieces, one per copy workgroup: the link
// serves many small batches better than fewer large ones, 54.5 GB/s against
// 52.3 with 32 KB pieces).  The HBM side is a ring of two KV heads'
// records: launch i copies KV head i into slot i % 2 while the same launch's
// other workgroups scan head i - 1 from slot (i - 1) % 2, so the copy of one
// head overlaps the compute of the previous one; kernel boundaries order each
// copy before its scan, and the scan of head i - 2 (launch i - 1) before the
// copy that reuses its slot.
// ---------------------------------------------------------------------------

constexpr int64_t kCopyPiece = 4096;    // bytes per copy workgroup: one 16-byte piece per thread

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
  static_assert(PER >= 1 && (int64_t)PER * 16 * NT == kCopyPiece, "whole 16-byte pieces per thread");
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
  uint4* d4 = reinterpret_cast<uint4*>(dst + ((g % kStageRing) * d + owner) * R);
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
  const uint32_t b = blockIdx.x;
  const uint32_t scan_blocks = (uint32_t)(tiles * scan_heads);
  if (b < scan_blocks) {
    const uint32_t hb = b / (uint32_t)tiles;
    scan_tile<G, TB>(a, scan_g0 + hb, (int64_t)(b - hb * (uint32_t)tiles), sm);
  } else {
    const uint32_t cb = b - scan_blocks;
    if (cb < (uint32_t)(ncopy * copy_heads)) {
      const uint32_t hc = cb / (uint32_t)ncopy;
      copy_piece<G, TB>(host, const_cast<uint8_t*>(a.rec), a.uni, copy_g0 + hc, a.d, a.H, a.P,
                        a.R, (int64_t)(cb - hc * (uint32_t)ncopy), sm);
    }
  }
}

// Paging of a scan: the page table and the keys per page (0: contiguous records).
struct Paging {
  const uint8_t* const* table;
  int64_t npages;
  int64_t page_keys;
};

template <int G, int TB, int KW, int GS = kStageGroup<TB>>
hipError_t launch_g(const uint8_t* rec, const float* q, const uint8_t* depth, const uint8_t* uni,
                    int h_kv, const Layout& L, int d, float* scores, int64_t ld, uint32_t* zero,
                    int64_t zero_words, uint32_t* hist, const Paging& pg, hipStream_t s) {
  ScanArgs a{rec, q, depth, uni, L.n, L.nb, L.H, L.P, L.R, d, scores, ld, zero, zero_words, 0, hist, nullptr, 0, 1};
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
  a.zero_slice = (zero_words + total - 1) / total;
  if (hist) {
    scan_kernel<G, TB, KW, true, GS><<<(unsigned)grid, Cfg<G, TB, KW>::threads, 0, s>>>(a, tiles, total);
    return hipGetLastError();
  }
  scan_kernel<G, TB, KW, false, GS><<<(unsigned)grid, Cfg<G, TB, KW>::threads, 0, s>>>(a, tiles, total);
  return hipGetLastError();
}

template <int G>
hipError_t launch_staged_g(const uint8_t* host, uint8_t* staging, const float* q, const uint8_t* depth,
                           const uint8_t* uni, int h_kv, const Layout& L, int d, float* scores,
                           int64_t ld, hipStream_t s) {
  constexpr int TB = kTileDevice;
  const ScanArgs a{staging, q, depth, uni, L.n, L.nb, L.H, L.P, L.R, d, scores, ld, nullptr, 0, 0, nullptr,
                   nullptr, 0, 1, kStageRing};
  const int64_t tiles = (L.nb + TB - 1) / TB;
  const int64_t ncopy = copy_pieces_per_head(L, d);
  for (int i = 0; i <= h_kv; ++i) {
    const int ch = i < h_kv ? 1 : 0;   // copy head i (none in the last launch)
    const int sh = i > 0 ? 1 : 0;      // scan head i - 1 (none in the first)
    const int64_t blocks = ncopy * ch + tiles * sh;
    stage_scan_kernel<G, TB><<<(unsigned)blocks, Cfg<G, TB>::threads, 0, s>>>(a, host, i, ch, ncopy, i - 1, sh,
                                                                               tiles);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int G>
hipError_t launch_any(const uint8_t* rec, bool host, const float* q, const uint8_t* depth,
                      const uint8_t* uni, int h_kv, const Layout& L, int d, float* scores, int64_t ld,
                      uint32_t* zero, int64_t zero_words, uint32_t* hist, const Paging& pg, hipStream_t s) {
  if (host && pg.table)
    return launch_g<G, PagedHostTile<G>::TB, PagedHostTile<G>::KW>(rec, q, depth, uni, h_kv, L, d, scores, ld, zero,
                                                                     zero_words, hist, pg, s);
  if (host)
    return launch_g<G, HostTile<G>::TB, HostTile<G>::KW>(rec, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words,
                                                         hist, pg, s);
  // long rows take the smaller staging groups (more workgroups resident at once)
  if constexpr (G >= 2 && G <= 8) {
    const int64_t tiles = (L.nb + kTileDevice - 1) / kTileDevice;
    if (tiles * h_kv > kDeviceRunTiles)
      return launch_g<G, kTileDevice, 1, kDeviceRunGroup>(rec, q, depth, uni, h_kv, L, d, scores, ld, zero,
                                                           zero_words, hist, pg, s);
  }
  return launch_g<G, kTileDevice, 1>(rec, q, depth, uni, h_kv, L, d, scores, ld, zero, zero_words, hist, pg, s);
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
