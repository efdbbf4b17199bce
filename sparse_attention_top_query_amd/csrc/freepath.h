// Internal declarations of the scan over a serving stack's token-major 4-bit
// K copy (codes [h_kv][n][d/2], scales [h_kv][nb][d] fp16), d a multiple of 32
// up to 128.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fathom {

hipError_t launch_pack_nibbles(const float* k, int h_kv, int64_t n, int d, uint8_t* codes, uint16_t* scales,
                               uint32_t* status, hipStream_t s);
hipError_t launch_nibble_scan(const uint8_t* codes, const uint16_t* scales, const float* q, const uint8_t* depth,
                              const uint8_t* uni, int h_kv, int g, int64_t n, int d, float* scores, int64_t ld,
                              hipStream_t s);

}  // namespace fathom
