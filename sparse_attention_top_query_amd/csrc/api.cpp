// C ABI of the Fathom key scan: argument validation and launch sequencing.
// The declarations, with their citations and contracts, are in include/fathom.h.
#include "fathom.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "append.h"
#include "attend.h"
#include "fathom_internal.h"
#include "freepath.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return FATHOM_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(FATHOM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

int check_heads(int h_q, int h_kv, int d) {
  if (h_kv < 1 || h_kv > 65535) return fail(FATHOM_ESHAPE, "h_kv=%d outside [1, 65535]", h_kv);
  if (h_q < h_kv || h_q % h_kv != 0)
    return fail(FATHOM_ESHAPE, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  if (h_q > 65535) return fail(FATHOM_ESHAPE, "h_q=%d exceeds 65535 (one grid row per query head)", h_q);
  if (!valid_group(h_q / h_kv))
    return fail(FATHOM_ESHAPE, "query heads per KV head %d not in {1,2,4,8,16}", h_q / h_kv);
  if (d < 1 || d > fathom::kMaxD) return fail(FATHOM_ESHAPE, "d=%d outside [1, %d]", d, fathom::kMaxD);
  return FATHOM_OK;
}

int64_t score_ld(int64_t n) { return (n + 63) / 64 * 64; }

// Size limits that keep every launch grid within 2^32 work-items per dimension:
// keys per head, keys times KV heads (the scan's threads are n h_kv / 4), and
// the open tail.
constexpr int64_t kMaxN = int64_t(1) << 30;
constexpr int64_t kMaxKeyHeads = int64_t(1) << 33;
constexpr int64_t kMaxTail = int64_t(1) << 20;

int check_n(int64_t n, int h_kv, const char* what) {
  if (n < 0 || n > kMaxN) return fail(FATHOM_ESHAPE, "%s=%lld outside [0, 2^30]", what, (long long)n);
  if (n * h_kv > kMaxKeyHeads)
    return fail(FATHOM_ESHAPE, "%s * h_kv = %lld exceeds 2^33", what, (long long)(n * h_kv));
  return FATHOM_OK;
}

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// Resolve the device-visible address of a buffer (`what`: records, k_cache, ...)
// for the claimed residency.
int resolve_view(const void* buf, int residency, const char* what, const uint8_t** dev) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, buf);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // not a pointer HIP knows: pageable host memory
    return fail(FATHOM_ERESIDENCY, "%s pointer is not HIP device or pinned host memory", what);
  }
  if (residency == FATHOM_HBM) {
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
      return fail(FATHOM_ERESIDENCY, "FATHOM_HBM %s must be device memory", what);
    *dev = static_cast<const uint8_t*>(buf);
    return FATHOM_OK;
  }
  if (residency == FATHOM_HOST_DIRECT || residency == FATHOM_HOST_STAGED) {
    if (attr.type != hipMemoryTypeHost)
      return fail(FATHOM_ERESIDENCY, "host-resident %s must be pinned host memory", what);
    const uint8_t* p = static_cast<const uint8_t*>(attr.devicePointer);
    if (!p) return fail(FATHOM_ERESIDENCY, "pinned host %s has no device mapping", what);
    *dev = p + (static_cast<const uint8_t*>(buf) - static_cast<const uint8_t*>(attr.hostPointer));
    return FATHOM_OK;
  }
  return fail(FATHOM_EINVAL, "unknown residency %d", residency);
}

int resolve_records(const void* records, int residency, const uint8_t** dev) {
  return resolve_view(records, residency, "records", dev);
}

int check_scan_args(const void* records, int residency, const float* q, const uint8_t* depth,
                    const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d,
                    const uint8_t** dev) {
  int st = check_heads(h_q, h_kv, d);
  if (st) return st;
  st = check_n(n, h_kv, "n");
  if (st) return st;
  if (!q || !depth || !union_depth) return fail(FATHOM_EINVAL, "null q/depth/union_depth");
  if (!aligned(q, 4)) return fail(FATHOM_EINVAL, "q must be 4-byte aligned");
  if (n == 0) return FATHOM_OK;
  if (!records) return fail(FATHOM_EINVAL, "null records");
  if (!aligned(records, 16)) return fail(FATHOM_EINVAL, "records must be 16-byte aligned");
  return resolve_records(records, residency, dev);
}

}  // namespace

extern "C" {

int fathom_version(void) { return 100; }

const char* fathom_last_error(void) { return g_last_error.c_str(); }

size_t fathom_record_bytes(int64_t n) { return n <= 0 ? 0 : (size_t)fathom::make_layout(n).R; }
size_t fathom_prefix_bytes(int64_t n, int t) {
  if (n <= 0 || t <= 0) return 0;
  return (size_t)fathom::prefix_bytes(fathom::make_layout(n), t > fathom::kPlanes ? fathom::kPlanes : t);
}

int pack_bitplanes(const float* k, int h_kv, int64_t n, int d, void* records, uint32_t* status,
                   void* stream) {
  if (h_kv < 1 || h_kv > 65535) return fail(FATHOM_ESHAPE, "h_kv=%d outside [1, 65535]", h_kv);
  if (d < 1 || d > fathom::kMaxD) return fail(FATHOM_ESHAPE, "d=%d outside [1, %d]", d, fathom::kMaxD);
  int st = check_n(n, h_kv, "n");
  if (st) return st;
  if (n > 0 && (!k || !records)) return fail(FATHOM_EINVAL, "null k or records");
  if (n > 0 && (!aligned(k, 4) || !aligned(records, 16)))
    return fail(FATHOM_EINVAL, "k must be 4-byte and records 16-byte aligned");
  if (fathom::make_layout(n).nb > 0x7fffffff) return fail(FATHOM_ESHAPE, "too many blocks");
  hipError_t e = fathom::launch_pack(k, h_kv, fathom::make_layout(n), d, static_cast<uint8_t*>(records),
                                     status, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return ok();
}

int allocate_depths(const float* q, const float* sigma2, int h_q, int h_kv, int d, int mode,
                    int budget, uint8_t* depth, uint8_t* union_depth, uint32_t* status,
                    void* stream) {
  int st = check_heads(h_q, h_kv, d);
  if (st) return st;
  if (!q || !sigma2 || !depth || !union_depth) return fail(FATHOM_EINVAL, "null pointer argument");
  if (!aligned(q, 4) || !aligned(sigma2, 4)) return fail(FATHOM_EINVAL, "q/sigma2 must be 4-byte aligned");
  if (mode != FATHOM_WATERFILL && mode != FATHOM_TOPQ && mode != FATHOM_WATERFILL_GROUP && mode != FATHOM_STATIC)
    return fail(FATHOM_EINVAL, "unknown mode %d", mode);
  if (budget < 0 || budget > fathom::kPlanes * d)
    return fail(FATHOM_EBUDGET, "budget=%d outside [0, %d]", budget, fathom::kPlanes * d);
  if ((mode == FATHOM_TOPQ || mode == FATHOM_STATIC) && budget % fathom::kPlanes != 0)
    return fail(FATHOM_EBUDGET, "fixed-depth mode needs budget %% 4 == 0 (got %d)", budget);
  hipError_t e = fathom::launch_allocate(q, sigma2, h_kv, h_q / h_kv, d, mode, budget, depth,
                                         union_depth, status, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "allocate launch");
  return ok();
}

size_t fathom_workspace_bytes(int h_q, int h_kv, int64_t n, int d, int k, int residency) {
  (void)k;
  if (h_q <= 0 || h_kv <= 0 || d <= 0 || n <= 0) return 0;
  size_t bytes = al256((size_t)h_q * (size_t)score_ld(n) * 4) + fathom::select_workspace_bytes(h_q, n, k > 0 ? k : 1);
  if (residency == FATHOM_HOST_STAGED)
    bytes += al256((size_t)std::min<int64_t>(h_kv, fathom::kStageRing) * (size_t)d * (size_t)fathom::make_layout(n).R);
  return bytes;
}

}  // extern "C"

namespace {

// Launches the scan of the sealed keys described by L (contiguous records at
// `dev`, or pages through `table`) and prepares the selection on the way: the
// link-bound host-direct scan builds the first-digit histograms itself after a
// clearing launch (*hist_done), where the extra work hides behind the link; the
// arithmetic-bound HBM scan only zeroes them (*cleared).
hipError_t scan_for_select(const uint8_t* dev, const uint8_t* const* table, int64_t npages, int64_t page_keys,
                           bool host, const float* q, const uint8_t* depth, const uint8_t* union_depth, int h_q,
                           int h_kv, const fathom::Layout& L, int d, float* scores, int64_t ld,
                           const fathom::SelectWorkspace& sel, bool* cleared, bool* hist_done, hipStream_t s) {
  const int g = h_q / h_kv;
  hipError_t e;
  if (sel.small) {   // the selection builds no histogram and needs no clearing
    *cleared = *hist_done = false;
    return fathom::launch_scan_paged(dev, table, npages, page_keys, host, q, depth, union_depth, h_kv, g, L, d, scores,
                                     ld, nullptr, 0, nullptr, s);
  }
  if (host) {
    e = fathom::launch_select_clear(sel, h_q, s);
    if (e == hipSuccess)
      e = fathom::launch_scan_paged(dev, table, npages, page_keys, true, q, depth, union_depth, h_kv, g, L, d, scores,
                                    ld, nullptr, 0, sel.hist, s);
    *cleared = *hist_done = e == hipSuccess;
  } else {
    e = fathom::launch_scan_paged(dev, table, npages, page_keys, false, q, depth, union_depth, h_kv, g, L, d, scores,
                                  ld, sel.hist, (int64_t)fathom::select_clear_words(sel, h_q), nullptr, s);
    *cleared = e == hipSuccess;
  }
  return e;
}

// How the selection continues after run_scan: with what the scan prepared.
struct ScanOutcome {
  bool cleared = false;
  bool hist_done = false;
};

// Scores of every key into `scores` [h_q][ld]; staging comes from the workspace.
// With a selection to follow (`sel`), the direct scans also prepare it.
int run_scan(const uint8_t* dev, int residency, const float* q, const uint8_t* depth,
             const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d, float* scores, int64_t ld,
             uint8_t* staging, const fathom::SelectWorkspace* sel, ScanOutcome* out, hipStream_t s) {
  const fathom::Layout L = fathom::make_layout(n);
  const int g = h_q / h_kv;
  const bool host = residency == FATHOM_HOST_DIRECT;
  hipError_t e;
  bool* cleared = &out->cleared;
  bool* hist_done = &out->hist_done;
  *out = ScanOutcome();
  if (residency == FATHOM_HOST_STAGED) {
    e = fathom::launch_scan_staged(dev, staging, q, depth, union_depth, h_kv, g, L, d, scores, ld, s);
  } else if (sel && L.nb > 0) {
    e = scan_for_select(dev, nullptr, 0, 0, host, q, depth, union_depth, h_q, h_kv, L, d, scores, ld, *sel, cleared,
                        hist_done, s);
  } else {
    e = fathom::launch_scan(dev, host, q, depth, union_depth, h_kv, g, L, d, scores, ld, nullptr, 0, nullptr, s);
  }
  if (e != hipSuccess) return hip_fail(e, "scan launch");
  return FATHOM_OK;
}

size_t staging_offset(int h_q, int64_t n, int k) {
  return al256((size_t)h_q * (size_t)score_ld(n) * 4) + fathom::select_workspace_bytes(h_q, n, k > 0 ? k : 1);
}

}  // namespace

extern "C" {

int fathom_scan_scores(const void* records, int residency, const float* q, const uint8_t* depth,
                       const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d,
                       float* scores, int64_t ld, void* workspace, size_t workspace_bytes,
                       void* stream) {
  const uint8_t* dev = nullptr;
  int st = check_scan_args(records, residency, q, depth, union_depth, h_q, h_kv, n, d, &dev);
  if (st) return st;
  if (n == 0) return ok();
  if (!scores) return fail(FATHOM_EINVAL, "null scores");
  if (ld < n) return fail(FATHOM_ESHAPE, "ld=%lld < n=%lld", (long long)ld, (long long)n);
  uint8_t* staging = nullptr;
  if (residency == FATHOM_HOST_STAGED) {
    const size_t need = fathom_workspace_bytes(h_q, h_kv, n, d, 1, residency);
    if (!workspace || workspace_bytes < need)
      return fail(FATHOM_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(FATHOM_EINVAL, "workspace must be 256-byte aligned");
    staging = static_cast<uint8_t*>(workspace) + staging_offset(h_q, n, 1);
  }
  ScanOutcome out;
  st = run_scan(dev, residency, q, depth, union_depth, h_q, h_kv, n, d, scores, ld, staging, nullptr, &out,
                static_cast<hipStream_t>(stream));
  if (st) return st;
  return ok();
}

int scan_topk(const void* records, int residency, const float* q, const uint8_t* depth,
              const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d, int k,
              int32_t* topk_idx, float* topk_score, void* workspace, size_t workspace_bytes,
              void* stream) {
  const uint8_t* dev = nullptr;
  int st = check_scan_args(records, residency, q, depth, union_depth, h_q, h_kv, n, d, &dev);
  if (st) return st;
  if (k < 0 || k > n) return fail(FATHOM_ESHAPE, "k=%d outside [0, n=%lld]", k, (long long)n);
  if (k == 0) return ok();
  if (!topk_idx) return fail(FATHOM_EINVAL, "null topk_idx");
  const size_t need = fathom_workspace_bytes(h_q, h_kv, n, d, k, residency);
  if (!workspace || workspace_bytes < need)
    return fail(FATHOM_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(FATHOM_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ld = score_ld(n);
  float* scores = static_cast<float*>(workspace);
  uint8_t* sel_base = static_cast<uint8_t*>(workspace) + al256((size_t)h_q * (size_t)ld * 4);
  uint8_t* staging = static_cast<uint8_t*>(workspace) + staging_offset(h_q, n, k);
  const fathom::SelectWorkspace sel = fathom::carve_select(sel_base, h_q, n, k);
  ScanOutcome out;
  st = run_scan(dev, residency, q, depth, union_depth, h_q, h_kv, n, d, scores, ld, staging, &sel, &out, s);
  if (st) return st;
  hipError_t e = fathom::launch_select(scores, ld, h_q, n, k, topk_idx, topk_score, sel, out.cleared,
                                       out.hist_done, s);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

size_t fathom_noalloc_scratch_bytes(void) { return fathom::kNoallocScratchBytes; }

int scan_topk_noalloc(const void* records, int residency, const float* q, const uint8_t* depth,
                      const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d, int k, int32_t* topk_idx,
                      float* topk_score, void* stream) {
  if (residency != FATHOM_HBM && residency != FATHOM_HOST_DIRECT)
    return fail(FATHOM_ERESIDENCY, "scan_topk_noalloc reads records from HBM or in place from pinned host memory");
  int st = check_heads(h_q, h_kv, d);
  if (st) return st;
  st = check_n(n, h_kv, "n");
  if (st) return st;
  const size_t need = fathom_workspace_bytes(h_q, h_kv, n, d, k, residency);
  if (need > fathom::kNoallocScratchBytes)
    return fail(FATHOM_EWORKSPACE,
                "scan_topk_noalloc: h_q=%d, n=%lld, k=%d needs %zu bytes of workspace, more than the %zu bytes "
                "of the library's fixed scratch (use scan_topk with a caller workspace)",
                h_q, (long long)n, k, need, fathom::kNoallocScratchBytes);
  void* scratch = nullptr;
  hipError_t e = fathom::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  return scan_topk(records, residency, q, depth, union_depth, h_q, h_kv, n, d, k, topk_idx, topk_score, scratch,
                   fathom::kNoallocScratchBytes, stream);
}

size_t fathom_attend_workspace_bytes(int h_q, int d, int k) {
  if (h_q <= 0 || d <= 0 || k <= 0) return 0;
  return fathom::attend_workspace_bytes(h_q, d, k);
}

int attend_topk(const void* k_cache, const void* v_cache, int residency, const float* q,
                const int32_t* topk_idx, int h_q, int h_kv, int64_t n, int d, int k, float scale,
                float* out, float* lse, uint32_t* status, void* workspace, size_t workspace_bytes,
                void* stream) {
  if (h_kv < 1 || h_kv > 65535) return fail(FATHOM_ESHAPE, "h_kv=%d outside [1, 65535]", h_kv);
  if (h_q < h_kv || h_q % h_kv != 0)
    return fail(FATHOM_ESHAPE, "h_q=%d is not a multiple of h_kv=%d", h_q, h_kv);
  if (h_q > 65535) return fail(FATHOM_ESHAPE, "h_q=%d exceeds 65535 (one grid row per query head)", h_q);
  if (d != 8 && d != 16 && d != 32 && d != 64 && d != 128 && d != 256)
    return fail(FATHOM_ESHAPE, "attend_topk needs d in {8, 16, 32, 64, 128, 256} (got %d)", d);
  if (n < 1 || n > kMaxN) return fail(FATHOM_ESHAPE, "n=%lld outside [1, 2^30]", (long long)n);
  if (k < 1 || k > (1 << 28)) return fail(FATHOM_ESHAPE, "k=%d outside [1, 2^28]", k);
  if ((int64_t)h_q * fathom::attend_splits(d, k) > (int64_t(1) << 23))
    return fail(FATHOM_ESHAPE, "h_q * ceil(k / %d) exceeds 2^23 workgroups", fathom::attend_keys_per_group(d));
  if (!std::isfinite(scale)) return fail(FATHOM_EINVAL, "scale must be finite");
  if (!k_cache || !v_cache || !q || !topk_idx || !out) return fail(FATHOM_EINVAL, "null pointer argument");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(q, 16))
    return fail(FATHOM_EINVAL, "k_cache, v_cache and q must be 16-byte aligned");
  if (!aligned(topk_idx, 4) || !aligned(out, 4) || (lse && !aligned(lse, 4)) || (status && !aligned(status, 4)))
    return fail(FATHOM_EINVAL, "topk_idx/out/lse/status must be 4-byte aligned");
  if (residency != FATHOM_HBM && residency != FATHOM_HOST_DIRECT)
    return fail(FATHOM_ERESIDENCY, "attend_topk reads its caches from HBM or in place from pinned host memory");
  const size_t need = fathom::attend_workspace_bytes(h_q, d, k);
  if (!workspace || workspace_bytes < need)
    return fail(FATHOM_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(FATHOM_EINVAL, "workspace must be 256-byte aligned");
  const uint8_t* kd = nullptr;
  const uint8_t* vd = nullptr;
  int st = resolve_view(k_cache, residency, "k_cache", &kd);
  if (st) return st;
  st = resolve_view(v_cache, residency, "v_cache", &vd);
  if (st) return st;
  hipError_t e = fathom::launch_attend(reinterpret_cast<const uint16_t*>(kd), reinterpret_cast<const uint16_t*>(vd),
                                       q, topk_idx, h_q, h_kv, n, d, k, scale, out, lse, status, workspace,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attend launch");
  return ok();
}

int pack_blocks(const float* k, int h_kv, int64_t n_cap, int64_t block0, int64_t nblocks, int d,
                void* records, uint32_t* status, void* stream) {
  if (h_kv < 1 || h_kv > 65535) return fail(FATHOM_ESHAPE, "h_kv=%d outside [1, 65535]", h_kv);
  if (d < 1 || d > fathom::kMaxD) return fail(FATHOM_ESHAPE, "d=%d outside [1, %d]", d, fathom::kMaxD);
  if (n_cap < 1) return fail(FATHOM_ESHAPE, "n_cap=%lld must be positive", (long long)n_cap);
  int st = check_n(n_cap, h_kv, "n_cap");
  if (st) return st;
  const fathom::Layout cap = fathom::make_layout(n_cap);
  if (block0 < 0 || nblocks < 0 || block0 + nblocks > cap.nb)
    return fail(FATHOM_ESHAPE, "blocks [%lld, %lld) outside the %lld blocks of capacity %lld", (long long)block0,
                (long long)(block0 + nblocks), (long long)cap.nb, (long long)n_cap);
  if (nblocks > 0x7fffffff) return fail(FATHOM_ESHAPE, "too many blocks");
  if (nblocks > 0 && (!k || !records)) return fail(FATHOM_EINVAL, "null k or records");
  if (nblocks > 0 && (!aligned(k, 4) || !aligned(records, 16)))
    return fail(FATHOM_EINVAL, "k must be 4-byte and records 16-byte aligned");
  hipError_t e = fathom::launch_pack_blocks(k, h_kv, cap, block0, nblocks, d, static_cast<uint8_t*>(records),
                                            status, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return ok();
}

int scan_topk_append(const void* records, int residency, int64_t n_cap, int64_t n_sealed, const float* tail_k,
                     int64_t n_tail, const float* q, const uint8_t* depth, const uint8_t* union_depth, int h_q,
                     int h_kv, int d, int k, int32_t* topk_idx, float* topk_score, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int st = check_heads(h_q, h_kv, d);
  if (st) return st;
  st = check_n(n_cap, h_kv, "n_cap");
  if (st) return st;
  if (n_sealed < 0 || n_sealed > n_cap || (n_sealed % fathom::kBlock != 0 && n_sealed != n_cap))
    return fail(FATHOM_ESHAPE, "n_sealed=%lld must be a multiple of 128 (or n_cap) within [0, n_cap=%lld]",
                (long long)n_sealed, (long long)n_cap);
  if (n_tail < 0 || n_tail > kMaxTail) return fail(FATHOM_ESHAPE, "n_tail=%lld outside [0, 2^20]", (long long)n_tail);
  const int64_t n = n_sealed + n_tail;
  if (k < 0 || k > n) return fail(FATHOM_ESHAPE, "k=%d outside [0, n_sealed + n_tail = %lld]", k, (long long)n);
  if (residency != FATHOM_HBM && residency != FATHOM_HOST_DIRECT)
    return fail(FATHOM_ERESIDENCY, "scan_topk_append reads records from HBM or in place from pinned host memory");
  if (!q || !depth || !union_depth) return fail(FATHOM_EINVAL, "null q/depth/union_depth");
  if (!aligned(q, 4)) return fail(FATHOM_EINVAL, "q must be 4-byte aligned");
  if (n_tail > 0 && (!tail_k || !aligned(tail_k, 4))) return fail(FATHOM_EINVAL, "tail_k must be non-null, 4-byte aligned");
  if (k == 0) return ok();
  if (!topk_idx) return fail(FATHOM_EINVAL, "null topk_idx");
  const uint8_t* dev = nullptr;
  if (n_sealed > 0) {
    if (!records) return fail(FATHOM_EINVAL, "null records");
    if (!aligned(records, 16)) return fail(FATHOM_EINVAL, "records must be 16-byte aligned");
    st = resolve_records(records, residency, &dev);
    if (st) return st;
  }
  const size_t need = fathom_workspace_bytes(h_q, h_kv, n, d, k, FATHOM_HBM);
  if (!workspace || workspace_bytes < need)
    return fail(FATHOM_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(FATHOM_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ld = score_ld(n);
  float* scores = static_cast<float*>(workspace);
  uint8_t* sel_base = static_cast<uint8_t*>(workspace) + al256((size_t)h_q * (size_t)ld * 4);
  const fathom::SelectWorkspace sel = fathom::carve_select(sel_base, h_q, n, k);
  const int g = h_q / h_kv;
  hipError_t e;
  bool cleared = false, hist_done = false;
  if (n_sealed > 0) {
    // the capacity's geometry, cut to the sealed blocks; where the scan builds
    // the histograms, the tail kernel adds its keys
    fathom::Layout L = fathom::make_layout(n_cap);
    L.n = n_sealed;
    L.nb = (n_sealed + fathom::kBlock - 1) / fathom::kBlock;
    e = scan_for_select(dev, nullptr, 0, 0, residency == FATHOM_HOST_DIRECT, q, depth, union_depth, h_q, h_kv, L, d,
                        scores, ld, sel, &cleared, &hist_done, s);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
  }
  e = fathom::launch_tail_scores(tail_k, q, h_kv, g, n_tail, d, scores, ld, n_sealed, hist_done ? sel.hist : nullptr,
                                 s);
  if (e != hipSuccess) return hip_fail(e, "tail launch");
  e = fathom::launch_select(scores, ld, h_q, n, k, topk_idx, topk_score, sel, cleared, hist_done, s);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

int fathom_device_address(const void* p, int residency, void** out) {
  if (!p || !out) return fail(FATHOM_EINVAL, "null pointer argument");
  if (residency != FATHOM_HBM && residency != FATHOM_HOST_DIRECT)
    return fail(FATHOM_ERESIDENCY, "addresses are resolved for FATHOM_HBM or FATHOM_HOST_DIRECT memory");
  const uint8_t* dev = nullptr;
  int st = resolve_view(p, residency, "buffer", &dev);
  if (st) return st;
  *out = const_cast<uint8_t*>(dev);
  return ok();
}

int scan_topk_paged(const void* const* page_table, int residency, int64_t page_keys, int64_t n_sealed,
                    const float* tail_k, int64_t n_tail, const float* q, const uint8_t* depth,
                    const uint8_t* union_depth, int h_q, int h_kv, int d, int k, int32_t* topk_idx,
                    float* topk_score, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_heads(h_q, h_kv, d);
  if (st) return st;
  if (page_keys < 4096 || page_keys % 4096 != 0 || page_keys > kMaxN)
    return fail(FATHOM_ESHAPE, "page_keys=%lld must be a positive multiple of 4096 up to 2^30", (long long)page_keys);
  st = check_n(n_sealed, h_kv, "n_sealed");
  if (st) return st;
  if (n_sealed % fathom::kBlock != 0)
    return fail(FATHOM_ESHAPE, "n_sealed=%lld must be a multiple of 128", (long long)n_sealed);
  if (n_tail < 0 || n_tail > kMaxTail) return fail(FATHOM_ESHAPE, "n_tail=%lld outside [0, 2^20]", (long long)n_tail);
  const int64_t n = n_sealed + n_tail;
  if (k < 0 || k > n) return fail(FATHOM_ESHAPE, "k=%d outside [0, n_sealed + n_tail = %lld]", k, (long long)n);
  if (residency != FATHOM_HBM && residency != FATHOM_HOST_DIRECT)
    return fail(FATHOM_ERESIDENCY, "scan_topk_paged reads pages from HBM or in place from pinned host memory");
  if (!q || !depth || !union_depth) return fail(FATHOM_EINVAL, "null q/depth/union_depth");
  if (!aligned(q, 4)) return fail(FATHOM_EINVAL, "q must be 4-byte aligned");
  if (n_tail > 0 && (!tail_k || !aligned(tail_k, 4))) return fail(FATHOM_EINVAL, "tail_k must be non-null, 4-byte aligned");
  if (n_sealed > 0 && (!page_table || !aligned(page_table, 8)))
    return fail(FATHOM_EINVAL, "page_table must be non-null and 8-byte aligned");
  if (k == 0) return ok();
  if (!topk_idx) return fail(FATHOM_EINVAL, "null topk_idx");
  const size_t need = fathom_workspace_bytes(h_q, h_kv, n, d, k, FATHOM_HBM);
  if (!workspace || workspace_bytes < need)
    return fail(FATHOM_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(FATHOM_EINVAL, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ld = score_ld(n);
  float* scores = static_cast<float*>(workspace);
  uint8_t* sel_base = static_cast<uint8_t*>(workspace) + al256((size_t)h_q * (size_t)ld * 4);
  const fathom::SelectWorkspace sel = fathom::carve_select(sel_base, h_q, n, k);
  const int g = h_q / h_kv;
  const bool host = residency == FATHOM_HOST_DIRECT;
  hipError_t e = hipSuccess;
  bool cleared = false, hist_done = false;
  if (n_sealed > 0) {
    fathom::Layout L = fathom::make_layout(n_sealed);
    const int64_t npages = (n_sealed + page_keys - 1) / page_keys;
    const auto* table = reinterpret_cast<const uint8_t* const*>(page_table);
    e = scan_for_select(nullptr, table, npages, page_keys, host, q, depth, union_depth, h_q, h_kv, L, d, scores, ld,
                        sel, &cleared, &hist_done, s);
    if (e != hipSuccess) return hip_fail(e, "scan launch");
  }
  e = fathom::launch_tail_scores(tail_k, q, h_kv, g, n_tail, d, scores, ld, n_sealed, hist_done ? sel.hist : nullptr,
                                 s);
  if (e != hipSuccess) return hip_fail(e, "tail launch");
  e = fathom::launch_select(scores, ld, h_q, n, k, topk_idx, topk_score, sel, cleared, hist_done, s);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

int pack_nibbles(const float* k, int h_kv, int64_t n, int d, void* codes, void* scales, uint32_t* status,
                 void* stream) {
  if (h_kv < 1 || h_kv > 65535) return fail(FATHOM_ESHAPE, "h_kv=%d outside [1, 65535]", h_kv);
  if (d < 32 || d > 128 || d % 32 != 0) return fail(FATHOM_ESHAPE, "the 4-bit token-major copy needs d in {32, 64, 96, 128} (got %d)", d);
  int st = check_n(n, h_kv, "n");
  if (st) return st;
  if (n > 0 && (!k || !codes || !scales)) return fail(FATHOM_EINVAL, "null k, codes or scales");
  if (n > 0 && (!aligned(k, 4) || !aligned(codes, 16) || !aligned(scales, 2)))
    return fail(FATHOM_EINVAL, "k must be 4-byte, codes 16-byte and scales 2-byte aligned");
  hipError_t e = fathom::launch_pack_nibbles(k, h_kv, n, d, static_cast<uint8_t*>(codes),
                                             static_cast<uint16_t*>(scales), status, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "pack launch");
  return ok();
}

int scan_topk_nibbles(const void* codes, const void* scales, int residency, const float* q, const uint8_t* depth,
                      const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d, int k, int32_t* topk_idx,
                      float* topk_score, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_heads(h_q, h_kv, d);
  if (st) return st;
  if (d < 32 || d > 128 || d % 32 != 0) return fail(FATHOM_ESHAPE, "the 4-bit token-major copy needs d in {32, 64, 96, 128} (got %d)", d);
  st = check_n(n, h_kv, "n");
  if (st) return st;
  if (k < 0 || k > n) return fail(FATHOM_ESHAPE, "k=%d outside [0, n=%lld]", k, (long long)n);
  if (residency != FATHOM_HBM && residency != FATHOM_HOST_DIRECT)
    return fail(FATHOM_ERESIDENCY, "scan_topk_nibbles reads HBM or pinned host memory in place");
  if (!q || !depth || !union_depth) return fail(FATHOM_EINVAL, "null q/depth/union_depth");
  if (!aligned(q, 4)) return fail(FATHOM_EINVAL, "q must be 4-byte aligned");
  if (k == 0) return ok();
  if (!topk_idx) return fail(FATHOM_EINVAL, "null topk_idx");
  if (!codes || !scales) return fail(FATHOM_EINVAL, "null codes or scales");
  if (!aligned(codes, 16) || !aligned(scales, 2)) return fail(FATHOM_EINVAL, "codes must be 16-byte, scales 2-byte aligned");
  const size_t need = fathom_workspace_bytes(h_q, h_kv, n, d, k, FATHOM_HBM);
  if (!workspace || workspace_bytes < need)
    return fail(FATHOM_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!aligned(workspace, 256)) return fail(FATHOM_EINVAL, "workspace must be 256-byte aligned");
  const uint8_t* cdev = nullptr;
  const uint8_t* sdev = nullptr;
  st = resolve_view(codes, residency, "codes", &cdev);
  if (st) return st;
  st = resolve_view(scales, residency, "scales", &sdev);
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ld = score_ld(n);
  float* scores = static_cast<float*>(workspace);
  uint8_t* sel_base = static_cast<uint8_t*>(workspace) + al256((size_t)h_q * (size_t)ld * 4);
  hipError_t e = fathom::launch_nibble_scan(cdev, reinterpret_cast<const uint16_t*>(sdev), q, depth, union_depth, h_kv,
                                            h_q / h_kv, n, d, scores, ld, s);
  if (e != hipSuccess) return hip_fail(e, "scan launch");
  e = fathom::launch_select(scores, ld, h_q, n, k, topk_idx, topk_score, fathom::carve_select(sel_base, h_q, n, k),
                            false, false, s);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return ok();
}

}  // extern "C"
