// Internal declarations for keys appended during decoding: sealing whole
// 128-key blocks into capacity-sized records, and exact scores of the open
// tail block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fathom_internal.h"

namespace fathom {

// Pack blocks [block0, block0 + nblocks) of records laid out for `cap` (its n
// is the capacity); `k` holds those blocks' rows, token-major, per KV head.
hipError_t launch_pack_blocks(const float* k, int h_kv, const Layout& cap, int64_t block0, int64_t nblocks,
                              int d, uint8_t* rec, uint32_t* status, hipStream_t s);

// Exact fp32 scores of m tail keys (tail_k [h_kv][m][d]) for every query head,
// written to scores[h][first + i]; with `hist` also counted into the
// selection's first-digit histograms hist[h][kSelBins].
hipError_t launch_tail_scores(const float* tail_k, const float* q, int h_kv, int g, int64_t m, int d,
                              float* scores, int64_t ld, int64_t first, uint32_t* hist, hipStream_t s);

}  // namespace fathom
