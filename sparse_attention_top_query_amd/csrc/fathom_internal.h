// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fathom {

constexpr int kBlock = 128;       // keys per shared scale
constexpr int kPlanes = 4;        // 4-bit codes
constexpr int kMaxD = 256;        // channels supported (one wave covers 64, 4 per lane)
constexpr int kMaxG = 16;         // query heads per KV head

constexpr int kUnitBlocks = 8;    // blocks per interleave unit (1024 keys)
constexpr int kUnitHead = 144;    // head bytes per unit: 16 B scales + 128 B plane-0 bits

// Byte geometry of one (KV head, channel) record:
//   head [0, H): per 1024-key unit u, at 144u: 8 fp16 scales (16 B) then the
//                unit's plane-0 bits (128 B);
//   plane p in 1..3 at H + (p-1) P, one bit per key (key j: bit j%8 of byte j/8).
// A prefix of t >= 1 planes is the single run [0, H + (t-1) P).
struct Layout {
  int64_t n;     // keys
  int64_t nb;    // 128-key blocks
  int64_t U;     // 1024-key units
  int64_t H;     // head bytes = 144 U
  int64_t P;     // bytes of plane 1, 2 or 3 = 128 U
  int64_t R;     // record bytes = H + 3P
};

inline Layout make_layout(int64_t n) {
  Layout L;
  L.n = n;
  L.nb = (n + kBlock - 1) / kBlock;
  L.U = (L.nb + kUnitBlocks - 1) / kUnitBlocks;
  L.H = kUnitHead * L.U;
  L.P = 16 * kUnitBlocks * L.U;
  L.R = L.H + (kPlanes - 1) * L.P;
  return L;
}

inline int64_t prefix_bytes(const Layout& L, int t) { return t <= 0 ? 0 : L.H + (t - 1) * L.P; }

// Selection keys: an order-preserving map of fp32 scores to uint32 (-0 folded
// onto +0), and the first digit of the selection's histogram (its top 12 bits).
constexpr int kSelBins = 4096;
constexpr int kSelDigit0 = 20;
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Loads and stores through the global address space, for pointers whose origin
// the compiler cannot see (chosen at run time, passed through LDS).  A generic
// (flat) access also counts against the LDS wait counter, so any later LDS wait
// would stall until it completed.
template <typename T>
__device__ __forceinline__ T load_global(const T* p) {
  return *(const __attribute__((address_space(1))) T*)p;
}
template <typename T>
__device__ __forceinline__ void store_global(T* p, T v) {
  *(__attribute__((address_space(1))) T*)p = v;
}
// (the HIP vector types' copies take generic references: move them as vectors)
__device__ __forceinline__ uint4 load_global(const uint4* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u x = *(const __attribute__((address_space(1))) v4u*)p;
  return make_uint4(x.x, x.y, x.z, x.w);
}
__device__ __forceinline__ void store_global(float4* p, float4 v) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  v4f x;
  x.x = v.x;
  x.y = v.y;
  x.z = v.z;
  x.w = v.w;
  *(__attribute__((address_space(1))) v4f*)p = x;
}

// Inclusive prefix sum over the 64 lanes of a wavefront, in lane order, with DPP
// moves (no LDS round trips): shifts by 1, 2, 4, 8 within each row of 16 lanes
// (zero fill), then lane 15 of rows 0 and 2 is added to rows 1 and 3, and lane
// 31 to rows 2 and 3.  Every lane must be active.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Size of the fixed device scratch of scan_topk_noalloc (one copy per GPU).
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
// The current device's address of that scratch (looked up on the first call
// per device, then cached).
hipError_t noalloc_scratch(void** out);

// ---- launchers (each returns hipSuccess or the launch error) ----
hipError_t launch_pack(const float* k, int h_kv, const Layout& L, int d, uint8_t* rec,
                       uint32_t* status, hipStream_t s);
hipError_t launch_allocate(const float* q, const float* sigma2, int h_kv, int g, int d,
                           int mode, int budget, uint8_t* depth, uint8_t* uni,
                           uint32_t* status, hipStream_t s);
// Scores of every key from device memory (host = false) or read in place from
// pinned host memory (host = true, larger tiles for long contiguous runs).
// The kernel also zeroes `zero_words` words at `zero` (the selection's
// histograms and state; may be null).  With `hist` (may be null; not together
// with `zero`) it also adds every score's first selection digit to
// hist[h][kSelBins], which must be zero beforehand (launch_select_clear).
hipError_t launch_scan(const uint8_t* rec, bool host, const float* q, const uint8_t* depth,
                       const uint8_t* uni, int h_kv, int g, const Layout& L, int d,
                       float* scores, int64_t ld, uint32_t* zero, int64_t zero_words, uint32_t* hist,
                       hipStream_t s);
// The same over paged records: table[g * npages + p] is the device-visible base
// of page p of KV head g, [d][R(page_keys)] bytes laid out as whole records of
// the page's page_keys keys (a multiple of 4096); L describes the keys scanned.
hipError_t launch_scan_paged(const uint8_t* rec, const uint8_t* const* table, int64_t npages, int64_t page_keys,
                             bool host, const float* q, const uint8_t* depth, const uint8_t* uni, int h_kv, int g,
                             const Layout& L, int d, float* scores, int64_t ld, uint32_t* zero, int64_t zero_words,
                             uint32_t* hist, hipStream_t s);
// Host-resident records: gather the union prefix runs into `staging` (a ring of
// kStageRing KV heads' records in HBM, min(h_kv, kStageRing) * d * R bytes) and
// scan them there, the copy of one KV head overlapped with the scan of the
// previous.
constexpr int64_t kStageRing = 2;
hipError_t launch_scan_staged(const uint8_t* host, uint8_t* staging, const float* q,
                              const uint8_t* depth, const uint8_t* uni, int h_kv, int g,
                              const Layout& L, int d, float* scores, int64_t ld, hipStream_t s);

// Top-k selection over scores [h_q][ld], first n entries per row.
struct SelectWorkspace {
  uint32_t* hist;     // [h_q][4096] histogram of the top 12 key bits
  uint32_t* state;    // [h_q][8]: threshold bin, keys above it, overflow flag, spill fill, and the same
                      // four for the refinement stage's second digit
  uint32_t* counts;   // [h_q][nchunks] kept keys per 4096-key chunk
  uint32_t* soff;     // [h_q][nchunks] spill offset of a chunk whose kept keys overflow its slot
  uint64_t* kept;     // [h_q][nchunks][512] (key, index) at or above the threshold bin
  uint64_t* spill;    // [h_q][spill_cap] kept keys of overflowing chunks, one segment per chunk
  int64_t spill_cap;  // spill entries per head: 16384 (0 for rows of at most 16384 keys)
  uint32_t* hist2;    // [h_q][1024] second-digit histogram of the refinement stage (long rows), or null
  int64_t nchunks;
  bool small;         // rows of at most 16384 keys: one launch, selecting in LDS, needs none of the above
};
int64_t select_chunks(int64_t n);
size_t select_workspace_bytes(int h_q, int64_t n, int k);
SelectWorkspace carve_select(void* base, int h_q, int64_t n, int k);
// Words from ws.hist that must be zero when the selection starts (histograms,
// state, and for rows long enough for the refinement stage its second-digit
// histograms); `cleared` says a previous kernel on the stream zeroed them.
size_t select_clear_words(const SelectWorkspace& ws, int h_q);
// `hist_done`: earlier kernels on the stream built ws.hist (after zeroing it
// and the per-head state); otherwise the selection builds it first, clearing
// it unless `cleared`.
hipError_t launch_select(const float* scores, int64_t ld, int h_q, int64_t n, int k,
                         int32_t* idx, float* val, const SelectWorkspace& ws, bool cleared, bool hist_done,
                         hipStream_t s);
hipError_t launch_select_clear(const SelectWorkspace& ws, int h_q, hipStream_t s);
}  // namespace fathom
