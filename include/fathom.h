/*
 * fathom.h -- C ABI of the Fathom per-query variable-depth key scan on MI355X (gfx950).
 *
 * Method: "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
 * Caches" (arXiv 2609.17652).  Page citations below:
 *   [Abstract]  the arXiv abstract;
 *   [Review]    the evolve.pub review ("Summary", "Strengths" -> paper Sec 3.2,
 *               3.3, 3.6, "Frequently asked questions");
 *   [Digest]    the ai-feeds.com summary (Method: Inputs, Key modules 1-5, Output).
 *
 * A top-k step is three calls:
 *   pack_bitplanes   once per cache: 4-bit codes as channel-major bit planes;
 *   allocate_depths  per query step: read depth t_c of every channel per query head;
 *   scan_topk        per query step: score every key from its read prefix, return top-k.
 * and the attention that consumes the selection is a fourth:
 *   attend_topk      per query step: attention of each query head over its top-k keys.
 * A cache that grows during decoding uses pack_blocks and scan_topk_append, or
 * paged records and scan_topk_paged.
 *
 * Conventions shared by every call:
 *   - Device pointers are HIP device memory unless stated; every call is
 *     asynchronous on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns after validating its arguments and enqueueing work.
 *   - The caller owns every buffer.  No call allocates device or host memory
 *     and none keeps state between calls (scan_topk_noalloc aside, whose fixed
 *     scratch array lives in the library).  There is no context object to
 *     create or destroy: the library owns no streams or events, every
 *     call enqueues on the caller's stream only (the host-staged residency too:
 *     its copies and scans are kernels on that stream), and the device is the
 *     one current on the calling thread.
 *   - Non-finite inputs are reported through device status words (the
 *     FATHOM_FLAG_* bits below), written by the kernels that read the values,
 *     not by a return code: checking q or sigma2 on the host would need a
 *     device-to-host copy and a synchronisation in every decode step.
 *   - Return value: FATHOM_OK or a negative fathom_status.  On a negative
 *     status nothing was enqueued and no output was written;
 *     fathom_last_error() gives a message (per calling thread).
 *   - Shapes: h_kv KV heads, G = h_q / h_kv query heads per KV head
 *     (G in {1, 2, 4, 8, 16}, h_q <= 65535), d channels (1..256), n keys
 *     (0 <= n <= 2^30, n * h_kv <= 2^33; these keep every launch grid within
 *     its limits).
 *     Query head h belongs to KV head h / G.  Independent sessions are passed
 *     as extra KV heads (session-major), since sessions never mix.
 */
#ifndef FATHOM_H
#define FATHOM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fathom_status {
  FATHOM_OK = 0,
  FATHOM_EINVAL = -1,     /* null pointer, bad mode/residency, misaligned pointer      */
  FATHOM_ESHAPE = -2,     /* h_kv, h_q, d, n or k outside the supported range          */
  FATHOM_EBUDGET = -3,    /* budget outside [0, 4d], or fixed mode with budget % 4 != 0 */
  FATHOM_EWORKSPACE = -5, /* workspace smaller than fathom_workspace_bytes()           */
  FATHOM_EHIP = -6,       /* a HIP runtime call or kernel launch failed                 */
  FATHOM_ERESIDENCY = -7  /* records pointer does not match the residency it claims    */
} fathom_status;

/* Where scan_topk finds the records. */
enum fathom_residency {
  FATHOM_HBM = 0,          /* records in device memory                                  */
  FATHOM_HOST_DIRECT = 1,  /* records in pinned host memory (hipHostMalloc or torch
                              pin_memory); the scan kernel reads the budgeted plane
                              prefixes of each tile straight over the host link          */
  FATHOM_HOST_STAGED = 2   /* records in pinned host memory; each channel's budgeted prefix
                              run is gathered with long contiguous reads into a ring of two
                              KV heads' records in the workspace, and the copy of one KV head
                              overlaps the scan of the previous one ([Review] Strengths, paper
                              Sec 3.6: partial reads as contiguous host-link runs)          */
};

/* How allocate_depths spends the budget. */
enum fathom_depth_mode {
  FATHOM_WATERFILL = 0,    /* reverse water-filling (the method)                         */
  FATHOM_TOPQ = 1,         /* fixed-depth comparison scan: 4 planes on the budget/4
                              channels of largest |q_c| (ties: lowest channel)           */
  FATHOM_WATERFILL_GROUP = 2, /* one reverse water-filling per KV head on the group's summed
                              importance; every query head of the group gets the same
                              depths, so the scan reads exactly `budget` bits per
                              KV-head key (a GQA variant the pages leave open)           */
  FATHOM_STATIC = 3        /* fixed-depth comparison scan with static channels: 4 planes on
                              the budget/4 channels of largest sigma2_c (offline statistics,
                              as Double Sparsity calibrates its channels offline; ties:
                              lowest channel), the same for every query of a KV head     */
};

/* Flags OR-ed into the device status words. */
#define FATHOM_FLAG_KEY_NONFINITE 1u        /* pack: a key is NaN or +-Inf              */
#define FATHOM_FLAG_SCALE_OVERFLOW 2u       /* pack: max|k|/8 rounds past fp16 range    */
#define FATHOM_FLAG_Q_NONFINITE 4u          /* allocate: q is NaN or +-Inf              */
#define FATHOM_FLAG_SIGMA2_INVALID 8u       /* allocate: sigma2 negative or non-finite  */
#define FATHOM_FLAG_IMPORTANCE_OVERFLOW 16u /* allocate: q^2 sigma2 overflows fp32      */
#define FATHOM_FLAG_INDEX_RANGE 32u         /* attend: an index outside [0, n), skipped */

/* ---------------------------------------------------------------------------
 * Record layout.  [Digest] Inputs and key module 1, [Review] FAQ: the 4-bit K
 * cache is stored channel-major as bit planes, the 4 planes of a channel
 * contiguous, so the first t planes are the channel's t-bit quantizer;
 * [Review] Strengths (paper Sec 3.6): a partial read is one contiguous run.
 *
 * records = [h_kv][d] records of R = fathom_record_bytes(n) bytes each.  With
 * U = ceil(n / 1024) units of 1024 keys (8 blocks of 128):
 *   head, bytes [0, 144 U): unit u at 144 u holds the fp16 scales Delta of
 *        blocks 8u..8u+7 (16 bytes, little-endian) followed by the plane-0 bits
 *        of keys 1024u..1024u+1023 (128 bytes);
 *   plane p in 1..3 at 144 U + (p-1) 128 U: 128 U bytes.
 * Plane 0 is the most significant bit; key j is bit (j % 8) of byte (j % 1024)/8
 * of its unit's plane-0 bits, and of byte j/8 of planes 1..3.  Padding is 0.
 * The scales and the first t >= 1 planes form the single contiguous run of
 * fathom_prefix_bytes(n, t) = 144 U + (t-1) 128 U bytes at the record start,
 * and every key's scale is read together with its most significant plane.
 * For n a multiple of 1024: R = n/64 + n/2 and the t-prefix is n/64 + t n/8.
 * ------------------------------------------------------------------------- */
size_t fathom_record_bytes(int64_t n);
size_t fathom_prefix_bytes(int64_t n, int t);

/* pack_bitplanes -- quantise and pack the K cache (once per cache or layer).
 * [Review] Strengths (paper Sec 3.2) and FAQ: 4-bit uniform codes under one
 * shared block scale; prefix of t planes = the t-bit mid-rise quantizer.
 *   k        device, float32 [h_kv][n][d] (token-major, as a serving stack holds K).
 *   records  device, [h_kv][d][fathom_record_bytes(n)] bytes, written completely.
 *   status   device, one uint32; cleared by the call, then FATHOM_FLAG_KEY_NONFINITE /
 *            FATHOM_FLAG_SCALE_OVERFLOW are OR-ed in (asynchronously).  The
 *            affected records are then unspecified.  May be NULL.
 * Per (KV head, channel, 128-key block): Delta = fp16_RNE(max|k| / 8); per key:
 * code = clamp(floor(k / Delta) + 8, 0, 15), evaluated exactly (code 8 when
 * Delta = 0); plane p holds bit (3 - p) of the code.
 * Alignment: k 4-byte, records 16-byte aligned.  n = 0 is a no-op. */
int pack_bitplanes(const float* k, int h_kv, int64_t n, int d, void* records,
                   uint32_t* status, void* stream);

/* allocate_depths -- per-query read depths ([Abstract]; [Digest] key module 2;
 * [Review] Strengths, paper Sec 3.3: each extra plane cuts the error 4x).
 * One wavefront per query head.
 *   q            device, float32 [h_q][d].
 *   sigma2       device, float32 [h_kv][d] per-channel key variance (offline
 *                statistics, [Digest] Inputs).
 *   mode         FATHOM_WATERFILL: w_c = fl32(fl32(q_c*q_c)*sigma2_c); `budget`
 *                greedy steps each give one plane to the channel with t_c < 4 of
 *                largest w_c * 4^-t_c (compared exactly), lowest channel on ties --
 *                the minimiser of sum_c w_c 4^-t_c with sum_c t_c = budget.
 *                FATHOM_TOPQ: t_c = 4 on the budget/4 channels of largest |q_c|.
 *                FATHOM_STATIC: t_c = 4 on the budget/4 channels of largest sigma2_c.
 *                FATHOM_WATERFILL_GROUP: the same greedy once per KV head on
 *                W_c = fl32(... fl32(w_0,c + w_1,c) ... + w_G-1,c), the fp32 sum in
 *                head order of the group's w_h,c; all G query heads get its depths
 *                (a non-finite q in the group zeroes the whole group's depths).
 *   budget       bits per key and query head, 0..4d (multiple of 4 for TOPQ, STATIC).
 *   depth        device, uint8 [h_q][d] output.
 *   union_depth  device, uint8 [h_kv][d] output: max over the KV head's query heads
 *                (the longest prefix, which contains every head's prefix).
 *   status       device, uint32 [h_kv], written (not OR-ed) by the call: the OR of
 *                FATHOM_FLAG_Q_NONFINITE / _SIGMA2_INVALID / _IMPORTANCE_OVERFLOW
 *                over the KV head's query heads; a flagged query head gets all-zero
 *                depths.  May be NULL. */
int allocate_depths(const float* q, const float* sigma2, int h_q, int h_kv, int d,
                    int mode, int budget, uint8_t* depth, uint8_t* union_depth,
                    uint32_t* status, void* stream);

/* Bytes of device workspace scan_topk (and fathom_scan_scores) needs for this
 * shape and residency: the fp32 scores and selection state, plus for
 * FATHOM_HOST_STAGED a ring of two KV heads' records in HBM
 * (min(h_kv, 2) * d * R bytes) through which the prefix runs are staged. */
size_t fathom_workspace_bytes(int h_q, int h_kv, int64_t n, int d, int k, int residency);

/* scan_topk -- score every key from its read prefix and select the top k
 * ([Abstract]; [Digest] key modules 4-5 and Output: the scan pulls only the
 * budgeted planes and outputs top-k indices per query).
 *   records      packed records (layout above), device memory (FATHOM_HBM) or
 *                pinned host memory (FATHOM_HOST_DIRECT read in place,
 *                FATHOM_HOST_STAGED copied through the workspace); read-only.
 *   q, depth, union_depth   as for allocate_depths (device).
 *   k            0..n keys to return per query head.
 *   topk_idx     device, int32 [h_q][k]: the k keys of largest score, lowest index
 *                among equal scores, in ascending index order.
 *   topk_score   device, float32 [h_q][k] or NULL: the scores of topk_idx.
 *   workspace    device, >= fathom_workspace_bytes(h_q, h_kv, n, d, k) bytes,
 *                256-byte aligned; contents on entry ignored, on exit unspecified.
 * Score of key j for query head h (fp32 accumulation):
 *   s = sum over channels with t_c > 0 of q_c * Delta_c,b(j) * 2^(4-t) *
 *       ((code >> (4-t)) - 2^(t-1) + 1/2),
 * the midpoint of the key's cell of the t-bit mid-rise quantizer ([Digest] key
 * module 4; the paper's Sec 3.5 rule is not in the text, this is the reading).
 * Within 1e-4 * sum_c |q_c * k_hat_c| of the exact value. */
int scan_topk(const void* records, int residency, const float* q, const uint8_t* depth,
              const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d, int k,
              int32_t* topk_idx, float* topk_score, void* workspace,
              size_t workspace_bytes, void* stream);

/* fathom_scan_scores -- the scan stage alone (for tests and profiling): the same
 * scores scan_topk ranks, written to device float32 [h_q][ld] (ld >= n; the
 * first n entries of each row are written).  The workspace is used only by
 * FATHOM_HOST_STAGED (for its HBM ring of staged records) and may be NULL
 * otherwise. */
int fathom_scan_scores(const void* records, int residency, const float* q,
                       const uint8_t* depth, const uint8_t* union_depth, int h_q,
                       int h_kv, int64_t n, int d, float* scores, int64_t ld,
                       void* workspace, size_t workspace_bytes, void* stream);

/* scan_topk_noalloc -- scan_topk with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The workspace is a fixed device
 * array inside the library, fathom_noalloc_scratch_bytes() (32 MiB) on every
 * GPU the library runs on, held until the process ends; the call allocates
 * nothing and frees nothing.
 *   residency   FATHOM_HBM or FATHOM_HOST_DIRECT (not the staged residency,
 *               whose HBM ring of staged records does not fit the scratch).
 *   all other arguments and results as for scan_topk (bit-identical output).
 * A shape whose fathom_workspace_bytes(...) exceeds the scratch returns
 * FATHOM_EWORKSPACE and enqueues nothing (e.g. 32 query heads of 131072 keys
 * fit; 32 heads of 1M keys do not).  Every call on a GPU uses that GPU's one
 * scratch, which keeps the last call's contents (each call clears what it
 * needs): calls that overlap on one GPU -- on different streams, or from
 * different threads -- race on it and must be serialised by the caller. */
size_t fathom_noalloc_scratch_bytes(void);
int scan_topk_noalloc(const void* records, int residency, const float* q, const uint8_t* depth,
                      const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d, int k,
                      int32_t* topk_idx, float* topk_score, void* stream);

/* ---------------------------------------------------------------------------
 * Appending keys during decoding.  The block scale is shared by a whole
 * 128-key block ([Review] Strengths, paper Sec 3.2), so a key can only be
 * quantised once its block is full.  Records are allocated for a capacity
 * n_cap (fathom_record_bytes(n_cap) bytes per (KV head, channel)); full blocks
 * are sealed into them with pack_blocks, and the newest keys -- the open tail
 * block -- stay in fp32 and are scored exactly by scan_topk_append (a reading:
 * the pages say nothing of the newest keys).
 * ------------------------------------------------------------------------- */

/* pack_blocks -- seal blocks [block0, block0 + nblocks) of records with capacity
 * n_cap: the same quantisation and layout as pack_bitplanes applied to the
 * whole cache, for those blocks only (other blocks are not touched, except that
 * sealing the last block of the capacity zeroes the padding after it).
 *   k        device, float32 [h_kv][rows][d], the rows of those blocks:
 *            rows = min(128 nblocks, n_cap - 128 block0).
 *   records  device, [h_kv][d][fathom_record_bytes(n_cap)] bytes.
 *   status   as for pack_bitplanes (cleared, then flags OR-ed in); may be NULL.
 * Sealing blocks one call at a time or all at once gives identical bytes. */
int pack_blocks(const float* k, int h_kv, int64_t n_cap, int64_t block0, int64_t nblocks, int d,
                void* records, uint32_t* status, void* stream);

/* scan_topk_append -- scan_topk over a growing cache: keys 0 .. n_sealed - 1 are
 * the sealed blocks of records with capacity n_cap (n_sealed a multiple of 128,
 * or n_cap), keys n_sealed .. n_sealed + n_tail - 1 are the open tail, scored
 * exactly in fp32 as sum_c q_c k_c from tail_k (device float32
 * [h_kv][n_tail][d]).  The top k over all n_sealed + n_tail keys follow the
 * scan_topk rules.  Residency FATHOM_HBM or FATHOM_HOST_DIRECT.  Workspace:
 * fathom_workspace_bytes(h_q, h_kv, n_sealed + n_tail, d, k, FATHOM_HBM). */
int scan_topk_append(const void* records, int residency, int64_t n_cap, int64_t n_sealed,
                     const float* tail_k, int64_t n_tail, const float* q, const uint8_t* depth,
                     const uint8_t* union_depth, int h_q, int h_kv, int d, int k,
                     int32_t* topk_idx, float* topk_score, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Paged records: a cache that grows without reallocating or copying.  A page
 * holds page_keys keys (a multiple of 4096) of one KV head, laid out exactly as
 * the records of a page_keys-key cache: [d][fathom_record_bytes(page_keys)]
 * bytes, so pack_bitplanes or pack_blocks (h_kv = 1, n = n_cap = page_keys)
 * write it, and any t-prefix of a channel is one contiguous run inside it.
 * Page p of KV head g holds keys p page_keys .. (p + 1) page_keys - 1.
 * ------------------------------------------------------------------------- */

/* fathom_device_address -- the address a kernel uses for `p`: `p` itself for
 * device memory (FATHOM_HBM), the mapped device address of pinned host memory
 * (FATHOM_HOST_DIRECT).  For building page tables.  Synchronous, no GPU work. */
int fathom_device_address(const void* p, int residency, void** out);

/* scan_topk_paged -- scan_topk_append over paged records.
 *   page_table   device, [h_kv][ceil(n_sealed / page_keys)] device addresses
 *                (fathom_device_address) of the pages, all in `residency`
 *                (FATHOM_HBM or FATHOM_HOST_DIRECT); 8-byte aligned.
 *   n_sealed     sealed keys, a multiple of 128; the blocks past n_sealed in the
 *                last page are not read.
 *   tail_k, n_tail, q, depth, union_depth, k, topk_idx, topk_score, workspace
 *                as for scan_topk_append (workspace: fathom_workspace_bytes(h_q,
 *                h_kv, n_sealed + n_tail, d, k, FATHOM_HBM)).
 * The scores, and so the selection, are bit-identical to those of the same
 * keys in contiguous records. */
int scan_topk_paged(const void* const* page_table, int residency, int64_t page_keys, int64_t n_sealed,
                    const float* tail_k, int64_t n_tail, const float* q, const uint8_t* depth,
                    const uint8_t* union_depth, int h_q, int h_kv, int d, int k, int32_t* topk_idx,
                    float* topk_score, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * The "free path": the same scan over the token-major 4-bit K copy a quantized
 * serving stack holds, with no bit-plane index ([Abstract]: the store is the
 * serving stack's 4-bit K copy; [Review] weaknesses: the free path is unbuilt).
 * Layout (a reading; the pages give none), d in {32, 64, 96, 128}:
 *   codes   [h_kv][n][d/2] bytes: channel 2i in the low nibble of byte i,
 *           2i+1 in the high nibble;
 *   scales  [h_kv][ceil(n/128)][d] fp16, one per (128-key block, channel).
 * Codes and scales are those of pack_bitplanes.  A key's codes are one row, so
 * the scan reads every row whole: d/2 + d/64 bytes per key whatever the budget.
 * ------------------------------------------------------------------------- */

/* pack_nibbles -- the token-major 4-bit copy of K (device float32 [h_kv][n][d],
 * 4-byte aligned) into codes (device, 16-byte aligned) and scales (device,
 * 2-byte aligned), both written whole; the last block of a head may be short.
 * The codes and scales are the ones pack_bitplanes stores for the same K (the
 * same threshold search and fp16 block scale).  d outside {32, 64, 96, 128} or
 * n beyond the record limits: FATHOM_ESHAPE; null or misaligned buffers with
 * n > 0: FATHOM_EINVAL; n = 0 writes nothing.  status: as for pack_bitplanes
 * (non-finite keys, scale overflow), OR-ed, may be NULL. */
int pack_nibbles(const float* k, int h_kv, int64_t n, int d, void* codes, void* scales, uint32_t* status,
                 void* stream);

/* scan_topk_nibbles -- scan_topk over the token-major copy: the same depths,
 * the same scores bit for bit, the same selection.  codes and scales in device
 * memory (FATHOM_HBM) or pinned host memory read in place (FATHOM_HOST_DIRECT);
 * codes 16-byte aligned.  Workspace: fathom_workspace_bytes(h_q, h_kv, n, d, k,
 * FATHOM_HBM). */
int scan_topk_nibbles(const void* codes, const void* scales, int residency, const float* q, const uint8_t* depth,
                      const uint8_t* union_depth, int h_q, int h_kv, int64_t n, int d, int k, int32_t* topk_idx,
                      float* topk_score, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attend_topk needs: per query head and split of its
 * k keys, a partial output (d + 2 floats) and a flag word. */
size_t fathom_attend_workspace_bytes(int h_q, int d, int k);

/* attend_topk -- attention of every query head over its selected keys
 * ([Digest] Output: top-k key indices per query, then real attention over those
 * keys; [Review] FAQ: the scan picks the top-k for sparse attention).  The pages
 * give no formula; the reading is the standard softmax attention:
 *   s_j = scale * (q_h . K_j) for j in topk_idx[h],
 *   out[h] = sum_j exp(s_j - M) V_j / sum_j exp(s_j - M),  M = max_j s_j,
 *   lse[h] = M + log sum_j exp(s_j - M),
 * with K, V the rows of KV head h / G.
 *   k_cache, v_cache  bf16 (uint16 bit patterns) [h_kv][n][d], token-major, as the
 *                     serving stack holds its cache; device memory (FATHOM_HBM) or
 *                     pinned host memory read in place (FATHOM_HOST_DIRECT); both
 *                     in the same residency; 16-byte aligned; read-only.
 *   q                 device, float32 [h_q][d], 16-byte aligned.
 *   topk_idx          device, int32 [h_q][k] (scan_topk's output, or any list;
 *                     order does not matter, repeats count repeatedly).  Entries
 *                     outside [0, n) are skipped and flagged.
 *   d                 8, 16, 32, 64, 128 or 256.
 *   out               device, float32 [h_q][d].
 *   lse               device, float32 [h_q] or NULL.  A head with no valid entry
 *                     gets out = 0 and lse = -inf.
 *   status            device, uint32 [h_q] or NULL, written (not OR-ed):
 *                     FATHOM_FLAG_INDEX_RANGE if the head's list held an entry
 *                     outside [0, n).
 *   workspace         device, >= fathom_attend_workspace_bytes(h_q, d, k) bytes,
 *                     256-byte aligned.
 * fp32 arithmetic: logits as fused multiply-adds reduced across lanes, expf of
 * s_j - M, sums along chains of at most 16 + 6 + 4 + S additions, S = ceil(k / 256)
 * (ceil(k / 128) for d = 256) splits of the list. */
int attend_topk(const void* k_cache, const void* v_cache, int residency, const float* q,
                const int32_t* topk_idx, int h_q, int h_kv, int64_t n, int d, int k,
                float scale, float* out, float* lse, uint32_t* status, void* workspace,
                size_t workspace_bytes, void* stream);

/* Message for the last failing call on this thread ("" if none). */
const char* fathom_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int fathom_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FATHOM_H */
