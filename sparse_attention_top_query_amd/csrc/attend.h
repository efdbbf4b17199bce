// Internal declarations of the attention over the selected keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fathom {

// Selected keys per workgroup for rows of d channels (d / 8 lanes per row):
// at most 16 row loads per lane and per cache.
inline int attend_keys_per_group(int d) {
  const int lpk = d / 8;
  const int kw = 4096 / lpk;
  return kw < 256 ? kw : 256;
}
inline int64_t attend_splits(int d, int k) {
  const int kw = attend_keys_per_group(d);
  return (k + kw - 1) / kw;
}
// Workspace: per (query head, split) the unnormalised output, the running max
// and the sum of weights (d + 2 floats), then a flag word.
inline size_t attend_workspace_bytes(int h_q, int d, int k) {
  const size_t parts = (size_t)h_q * (size_t)attend_splits(d, k);
  const size_t a = (parts * (size_t)(d + 2) * 4 + 255) / 256 * 256;
  return a + (parts * 4 + 255) / 256 * 256;
}

hipError_t launch_attend(const uint16_t* kc, const uint16_t* vc, const float* q, const int32_t* idx,
                         int h_q, int h_kv, int64_t n, int d, int k, float scale, float* out, float* lse,
                         uint32_t* status, void* workspace, hipStream_t s);

}  // namespace fathom
