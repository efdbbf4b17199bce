// Internal declarations shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fathom {

constexpr int kBlock = 128;       // keys per shared scale
constexpr int kPlanes = 4;        // 4-bit codes
constexpr int kMaxD = 256;        // channels supported (one wave covers 64, 4 per lane)
constexpr int kMaxG = 16;         // query heads per KV head

// Byte geometry of one (KV head, channel) record.
struct Layout {
  int64_t n;     // keys
  int64_t nb;    // 128-key blocks
  int64_t S;     // scale section bytes (multiple of 16)
  int64_t P;     // bytes per plane (16 per block)
  int64_t R;     // record bytes = S + 4P
};

inline Layout make_layout(int64_t n) {
  Layout L;
  L.n = n;
  L.nb = (n + kBlock - 1) / kBlock;
  L.S = ((2 * L.nb + 15) / 16) * 16;
  L.P = 16 * L.nb;
  L.R = L.S + kPlanes * L.P;
  return L;
}

// ---- launchers (each returns hipSuccess or the launch error) ----
hipError_t launch_pack(const float* k, int h_kv, const Layout& L, int d, uint8_t* rec,
                       uint32_t* status, hipStream_t s);
hipError_t launch_allocate(const float* q, const float* sigma2, int h_kv, int g, int d,
                           int mode, int budget, uint8_t* depth, uint8_t* uni,
                           uint32_t* status, hipStream_t s);
hipError_t launch_scan(const uint8_t* rec, const float* q, const uint8_t* depth,
                       const uint8_t* uni, int h_kv, int g, const Layout& L, int d,
                       float* scores, int64_t ld, hipStream_t s);

// Top-k selection over scores [h_q][ld], first n entries per row.
struct SelectWorkspace {
  uint32_t* hist;     // [h_q][2048]
  uint32_t* state;    // [h_q][4]: prefix, need, -, -
  uint32_t* counts;   // [h_q][nchunks][2]: (greater, equal) per chunk
  int64_t nchunks;
};
int64_t select_chunks(int64_t n);
size_t select_workspace_bytes(int h_q, int64_t n);
SelectWorkspace carve_select(void* base, int h_q, int64_t n);
hipError_t launch_select(const float* scores, int64_t ld, int h_q, int64_t n, int k,
                         int32_t* idx, float* val, const SelectWorkspace& ws, hipStream_t s);

}  // namespace fathom
