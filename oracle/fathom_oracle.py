"""Plain CPU oracle for the Fathom per-query variable-depth key scan.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product path: the two share no code.

Everything here is written from the definitions on the pages about
"Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches"
(arXiv 2609.17652), cited by page and section:

* [Abstract]  the arXiv abstract (aiqbench reprint).
* [Review]    the evolve.pub review: "Summary", "Key claims under review",
              "Strengths" (which points at the paper's Sec 3.2, 3.3, 3.6 and
              App. A) and "Frequently asked questions".
* [Digest]    the ai-feeds.com Chinese summary: Method -> Inputs, Key modules
              1-5, Output.

Where the pages leave a step open, the reading taken is stated next to the
code that implements it.  The 128-token block and the max|x|/8 block scale
come from the workload definition; the pages only say "one shared block
scale".

Precision: integer and byte work is exact; importance weights are formed in
fp32 exactly as the method defines them; gains are compared exactly in fp64;
scores are accumulated in fp64, where every product q*k_hat is exact (24 + 11 +
5 significant bits < 53), so the only rounding is the fp64 summation.

Parity status of each function (what pins it, in tests/test_oracle_*.py):
  block_scales, quantize_codes   pinned: exact floor(K/Delta) via Fractions,
                                 nesting identity, hand examples.
  pack_records, unpack_codes     pinned: bit-by-bit decoding of the layout
                                 definition, round trip, hand example.
  importance, waterfill_depths   pinned: brute force over all depth vectors
                                 (d=4, B<=16) with exact rationals, exchange
                                 (KKT) certificate at d=128, sum t = B,
                                 monotone in B.
  topq_depths                    pinned: independent sort by (-|q|, c).
  static_depths                  pinned: selection loop over (-sigma2, c),
                                 ties and zeros.
  group_importance               pinned: one head equals importance; the
                                 shared allocation equals brute force over all
                                 depth vectors of sum_h sum_c w_hc 4^-t_c
                                 (exact rationals, d=4, B<=16); sequential
                                 fp32 summation checked with Fractions.
  union_depths                   pinned: prefix nesting (union prefix contains
                                 every head's prefix).
  reconstruct, scores            pinned: B=4d equals full 4-bit dequant
                                 (q . (kappa-7.5)Delta) computed by a matmul,
                                 the t-bit quantizer identity, the
                                 4x-per-bit error bound.
  topk                           pinned: brute-force sort on small n.
  pack_nibbles, unpack_nibbles   pinned: hand-decoded bytes, round trip, sizes
                                 (the free path's scores are ``scores``).
  tail_scores, step_append       pinned: tail scores equal exact rational
                                 sums; an empty tail reduces to step(); an
                                 all-tail cache gives the brute-force top-k of
                                 the exact q . k.
The pages' own six-key worked example (the review's App. A) is referenced
but its values are not in the text we have, so it cannot serve as a pin.
"""

from __future__ import annotations

import numpy as np

BLOCK = 128          # tokens per shared scale (workload definition)
PLANES = 4           # 4-bit codes -> 4 bit planes ([Abstract]; [Digest] module 1)
CODE_MID = 8         # offset-binary zero point of a 4-bit mid-rise code
TOL_REL = 1e-4       # score tolerance factor applied to sum_c |q_c * k_hat_c|


# ---------------------------------------------------------------------------
# Record layout (our own; the pages fix only "channel-major, 4 contiguous
# planes per channel" -- [Digest] Inputs / module 1, [Review] FAQ on the
# bit-plane cache -- and that a partial read is a contiguous run, [Review]
# Strengths citing paper Sec 3.6).
# ---------------------------------------------------------------------------

UNIT_BLOCKS = 8                      # 128-key blocks per interleave unit (1024 keys)
UNIT_SCALE_BYTES = 2 * UNIT_BLOCKS   # 16: fp16 scales of one unit
UNIT_PLANE_BYTES = 16 * UNIT_BLOCKS  # 128: one plane's bits of one unit


def n_blocks(n: int) -> int:
    """Number of 128-token scale blocks covering n keys (last one may be partial)."""
    return (n + BLOCK - 1) // BLOCK


def n_units(n: int) -> int:
    """Number of 1024-key units covering n keys."""
    return (n_blocks(n) + UNIT_BLOCKS - 1) // UNIT_BLOCKS


def record_layout(n: int) -> tuple[int, int, int, int]:
    """(units U, head bytes H, plane bytes P, record bytes R) of one (KV head, channel) record.

    A record is   [ head: U units of (16 B fp16 scales of the unit's 8 blocks,
                                     128 B plane-0 bits of the unit's 1024 keys) ]
                  [ plane 1: P = 128 U bytes ] [ plane 2 ] [ plane 3 ]
    Plane 0 is the most significant bit.  Every key's scale travels with its
    plane-0 bits, and reading the first t >= 1 planes is the single contiguous
    run [0, H + (t - 1) P).  For n a multiple of 1024, R = n/64 + n/2.
    Padding (blocks or keys past n) is zero.
    """
    u = n_units(n)
    h = u * (UNIT_SCALE_BYTES + UNIT_PLANE_BYTES)
    p = u * UNIT_PLANE_BYTES
    return u, h, p, h + (PLANES - 1) * p


def prefix_bytes(n: int, t: int) -> int:
    """Bytes of the contiguous run holding the scales and the first t planes."""
    _, h, p, _ = record_layout(n)
    return 0 if t == 0 else h + (t - 1) * p


# ---------------------------------------------------------------------------
# Quantisation: 4-bit uniform mid-rise codes under one shared block scale.
# [Review] Strengths (paper Sec 3.2) and FAQ: 4-bit uniform per-channel codes,
# one shared scale per block, prefix of t planes = the t-bit mid-rise
# quantizer.  Offset-binary codes are the reading: code 8 is the cell
# [0, Delta), plane 0 holds the most significant bit.
# ---------------------------------------------------------------------------

def _blocked(k: np.ndarray) -> np.ndarray:
    """View float32 [n, d] keys as [n_blocks, 128, d], zero-padding the last block.

    Zero padding never changes a block maximum of |k| (which is >= 0)."""
    n, d = k.shape
    nb = n_blocks(n)
    if nb * BLOCK == n:
        return k.reshape(nb, BLOCK, d)
    kp = np.zeros((nb * BLOCK, d), dtype=np.float32)
    kp[:n] = k
    return kp.reshape(nb, BLOCK, d)


def block_scales(k: np.ndarray) -> np.ndarray:
    """Delta[c, b] = fp16_RNE(max_{j in block b} |k[j, c]| / 8).

    k: float32 [n, d] keys of one KV head, token-major.
    Returns float16 [d, n_blocks(n)].  Raises ValueError on NaN/Inf input or if
    a scale overflows fp16 (the GPU path reports both through a status word).
    """
    k = np.asarray(k)
    assert k.dtype == np.float32 and k.ndim == 2
    if not np.all(np.isfinite(k)):
        raise ValueError("non-finite key")
    mx = np.max(np.abs(_blocked(k)), axis=1)          # [nb, d], exact in fp32
    eighth = mx / np.float32(8.0)                     # power-of-two scaling
    with np.errstate(over="ignore"):
        out = eighth.astype(np.float16).T.copy()      # IEEE round-to-nearest-even
    if not np.all(np.isfinite(out)):
        raise ValueError("block scale overflows fp16")
    return out


def quantize_codes(k: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """kappa[j, c] = clamp(floor(k / Delta) + 8, 0, 15); kappa = 8 where Delta = 0.

    Evaluated as a count of thresholds, kappa = #{i in 1..15 : k >= (i - 8) * Delta},
    which equals the clamped floor exactly: each (i-8)*Delta is exact in fp32
    (Delta has 11 significant bits) and the comparison is exact.
    """
    n, d = k.shape
    kb = _blocked(np.asarray(k, dtype=np.float32))    # [nb, 128, d]
    dl = delta.T.astype(np.float32)[:, None, :]       # [nb, 1, d], exact widening
    cnt = np.zeros(kb.shape, dtype=np.uint8)
    for i in range(1, 16):
        cnt += kb >= np.float32(i - CODE_MID) * dl
    cnt[np.broadcast_to(dl == 0, kb.shape)] = CODE_MID
    return cnt.reshape(-1, d)[:n].copy()


def _plane_bits(kappa: np.ndarray, plane: int, units: int) -> np.ndarray:
    """Bits of one plane packed per channel: uint8 [d, 128 * units]; key j is bit
    (j mod 8) of byte j // 8; keys past n are 0."""
    n, d = kappa.shape
    bits = ((kappa >> (PLANES - 1 - plane)) & 1).astype(np.uint8)       # [n, d]
    padded = np.zeros((units * UNIT_BLOCKS * BLOCK, d), dtype=np.uint8)
    padded[:n] = bits
    return np.packbits(padded.T, axis=1, bitorder="little")


def pack_records(kappa: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """Channel-major bit-plane records of one KV head: uint8 [d, R] (layout in
    record_layout).  Plane p holds bit (3 - p) of every key's code; scales are
    little-endian fp16."""
    n, d = kappa.shape
    u, h, p, r = record_layout(n)
    rec = np.zeros((d, r), dtype=np.uint8)
    if u == 0:
        return rec
    sc = np.zeros((d, u * UNIT_BLOCKS), dtype="<f2")
    sc[:, : delta.shape[1]] = delta
    sc_bytes = sc.view(np.uint8).reshape(d, u, UNIT_SCALE_BYTES)
    p0 = _plane_bits(kappa, 0, u).reshape(d, u, UNIT_PLANE_BYTES)
    rec[:, :h] = np.concatenate([sc_bytes, p0], axis=2).reshape(d, h)
    for plane in range(1, PLANES):
        rec[:, h + (plane - 1) * p: h + plane * p] = _plane_bits(kappa, plane, u)
    return rec


def unpack_codes(rec: np.ndarray, n: int, depth: int = PLANES) -> tuple[np.ndarray, np.ndarray]:
    """Read back (delta [d, nb] fp16, t-bit prefix codes [n, d]) from records.

    Reads only bytes [0, prefix_bytes(n, depth)) of each record -- the run the
    scan pulls -- and returns kappa >> (4 - depth) (the scales need depth >= 1;
    with depth 0 they are returned as zeros, as nothing is read).
    """
    d = rec.shape[0]
    u, h, p, _ = record_layout(n)
    nb = n_blocks(n)
    run = rec[:, : prefix_bytes(n, depth)]
    code = np.zeros((n, d), dtype=np.uint8)
    delta = np.zeros((d, nb), dtype=np.float16)
    if depth == 0 or u == 0:
        return delta, code
    head = np.ascontiguousarray(run[:, :h]).reshape(d, u, UNIT_SCALE_BYTES + UNIT_PLANE_BYTES)
    delta = np.ascontiguousarray(head[:, :, :UNIT_SCALE_BYTES]).view("<f2").reshape(d, -1)[:, :nb]
    delta = delta.astype(np.float16)
    planes = [np.ascontiguousarray(head[:, :, UNIT_SCALE_BYTES:]).reshape(d, p)]
    for plane in range(1, depth):
        planes.append(run[:, h + (plane - 1) * p: h + plane * p])
    for bits_packed in planes:
        bits = np.unpackbits(bits_packed, axis=1, bitorder="little")
        code = (code << 1) | bits[:, :n].T
    return delta, code


def pack_nibbles(kappa: np.ndarray, delta: np.ndarray):
    """The same 4-bit copy, token-major as a quantized serving stack holds it (the
    "free path" the review's weaknesses name: scanning that copy directly, with
    no bit-plane index; [Abstract]: the store is the serving stack's 4-bit K).

    Reading of the layout (the pages give none; KIVI-style per-channel scales
    over 128-token groups): codes [n][ceil(d/2)] bytes, channel 2i in the low
    nibble of byte i and channel 2i+1 in the high nibble (0 past d); scales
    [n_blocks][d] fp16, little-endian, the same Delta as the records.
    ``delta`` is block_scales' [d, n_blocks].
    Returns (codes uint8 [n, ceil(d/2)], scales uint8 [n_blocks, 2d])."""
    kappa = np.asarray(kappa, dtype=np.int64)
    n, d = kappa.shape
    nib = np.zeros((n, 2 * ((d + 1) // 2)), dtype=np.int64)
    nib[:, :d] = kappa
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    dt = np.asarray(delta).T                                   # [n_blocks, d]
    scales = np.ascontiguousarray(dt.astype("<f2")).view(np.uint8).reshape(dt.shape[0], 2 * d)
    return codes, scales


def unpack_nibbles(codes: np.ndarray, d: int) -> np.ndarray:
    """Codes [n, d] back from the token-major nibbles."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.empty((c.shape[0], 2 * c.shape[1]), dtype=np.int64)
    out[:, 0::2] = c & 15
    out[:, 1::2] = c >> 4
    return out[:, :d]


def pack_head(k: np.ndarray):
    """Convenience: (delta, kappa, records) for one KV head's float32 [n, d] keys."""
    delta = block_scales(k)
    kappa = quantize_codes(k, delta)
    return delta, kappa, pack_records(kappa, delta)


# ---------------------------------------------------------------------------
# Per-query read depth: reverse water-filling of the bit budget.
# [Abstract]; [Digest] Insights and key module 2; [Review] Strengths (paper
# Sec 3.3: each extra bit cuts the channel's error by 4x).  The objective is
# sum_c w_c * 4^(-t_c) with w_c = q_c^2 * sigma_c^2 (variance-weighted
# importance, [Review] Summary; offline statistics, [Digest] Inputs), subject
# to sum_c t_c = B and t_c in {0..4}.
# ---------------------------------------------------------------------------

def importance(q: np.ndarray, sigma2: np.ndarray) -> np.ndarray:
    """w_c = fl32(fl32(q_c * q_c) * sigma2_c): two fp32 round-to-nearest products."""
    q = np.asarray(q, dtype=np.float32)
    sigma2 = np.asarray(sigma2, dtype=np.float32)
    if not (np.all(np.isfinite(q)) and np.all(np.isfinite(sigma2)) and np.all(sigma2 >= 0)):
        raise ValueError("q must be finite and sigma2 finite and non-negative")
    with np.errstate(over="ignore"):
        w = (q * q).astype(np.float32) * sigma2
    if not np.all(np.isfinite(w)):
        raise ValueError("importance overflows fp32")
    return w.astype(np.float32)


def waterfill_depths(w: np.ndarray, budget: int) -> np.ndarray:
    """Greedy marginal-gain allocation, one bit at a time.

    Each of the ``budget`` steps gives one more plane to the channel whose next
    plane removes the most weighted error, i.e. the channel with t_c < 4 that
    maximises w_c * 4^(-t_c); ties go to the lowest channel index.  Gains are
    compared exactly: w_c is fp32, scaling by 4^(-t) is exact in fp64.
    """
    w64 = np.asarray(w, dtype=np.float32).astype(np.float64)
    d = w64.shape[0]
    if not 0 <= budget <= PLANES * d:
        raise ValueError("budget out of range")
    t = np.zeros(d, dtype=np.int64)
    for _ in range(budget):
        gain = np.where(t < PLANES, w64 * np.power(4.0, -t.astype(np.float64)), -np.inf)
        c = int(np.argmax(gain))                      # first maximum -> lowest channel
        t[c] += 1
    return t


def group_importance(qs: np.ndarray, sigma2: np.ndarray) -> np.ndarray:
    """Group-shared importance of a GQA group (a variant the pages leave open:
    the review's FAQ on GQA and the group's shared K): one allocation per KV
    head on w_c = sum_h q_h,c^2 sigma_c^2, so every query head of the group
    reads the same B bits per key.  Reading of the arithmetic: each term is
    ``importance`` of one head, and the terms are added in fp32 in head order,
    w = fl32(...fl32(fl32(w_0 + w_1) + w_2)... + w_{G-1})."""
    qs = np.asarray(qs, dtype=np.float32)
    acc = np.zeros(qs.shape[1], dtype=np.float32)
    for h in range(qs.shape[0]):
        with np.errstate(over="ignore"):
            acc = (acc + importance(qs[h], sigma2)).astype(np.float32)
    if not np.all(np.isfinite(acc)):
        raise ValueError("group importance overflows fp32")
    return acc


def topq_depths(q: np.ndarray, m: int) -> np.ndarray:
    """Fixed-depth comparison mode: all 4 planes of the m channels with the largest |q_c|.

    Stands for the fixed 136-bit (34 x 4) and 68-bit (17 x 4) scans the pages
    compare against ([Abstract]); the channel rule "largest |q_c|, lowest index
    on ties" is the reading.
    """
    d = q.shape[0]
    if not 0 <= m <= d:
        raise ValueError("m out of range")
    order = sorted(range(d), key=lambda c: (-abs(float(q[c])), c))
    t = np.zeros(d, dtype=np.int64)
    t[order[:m]] = PLANES
    return t


def static_depths(sigma2: np.ndarray, m: int) -> np.ndarray:
    """Static fixed-depth comparison mode: all 4 planes of the m channels with the
    largest offline variance sigma2_c, the same for every query of the KV head.

    Stands for Double Sparsity's offline-calibrated channels ([Abstract] lists
    it among the 136-bit scans); choosing by sigma2 with lowest index on ties is
    the reading, sigma2 being the offline statistic the method itself uses.
    """
    s2 = np.asarray(sigma2, dtype=np.float32)
    d = s2.shape[0]
    if not 0 <= m <= d:
        raise ValueError("m out of range")
    order = sorted(range(d), key=lambda c: (-float(s2[c]), c))
    t = np.zeros(d, dtype=np.int64)
    t[order[:m]] = PLANES
    return t


def union_depths(depths: np.ndarray) -> np.ndarray:
    """Union prefix of a GQA group: max over the group's query heads.

    Prefixes nest, so the longest prefix contains every shorter one; reading
    it once serves all heads of the group (a bandwidth choice; each head still
    scores with its own depths).
    """
    return np.max(np.asarray(depths), axis=0)


# ---------------------------------------------------------------------------
# Reconstruction and scores.  [Digest] key module 4 (a rule applied on the
# read prefix to rebuild each channel's value; paper Sec 3.5, formula not in
# the text).  Reading: the t-bit prefix is reconstructed at the midpoint of
# its cell of the t-bit mid-rise quantizer, and an unread channel (t = 0)
# contributes the midpoint of the whole range, 0.
# ---------------------------------------------------------------------------

def reconstruct(kappa_col: np.ndarray, t: int, delta_per_key: np.ndarray) -> np.ndarray:
    """k_hat = Delta * 2^(4-t) * ((kappa >> (4-t)) - 2^(t-1) + 1/2) in fp64; 0 for t = 0."""
    if t == 0:
        return np.zeros(kappa_col.shape[0], dtype=np.float64)
    step = delta_per_key.astype(np.float64) * float(2 ** (PLANES - t))
    prefix = (kappa_col.astype(np.int64) >> (PLANES - t)).astype(np.float64)
    return step * (prefix - float(2 ** (t - 1)) + 0.5)


def scores(q: np.ndarray, kappa: np.ndarray, delta: np.ndarray, t: np.ndarray):
    """s_j = sum_c q_c * k_hat_{j,c} and A_j = sum_c |q_c * k_hat_{j,c}| in fp64.

    q: float32 [d] one query head; kappa: uint8 [n, d] codes of its KV head;
    delta: float16 [d, nb]; t: depths [d].  Computed from the codes (not from
    packed planes), so a GPU path that reads planes is checked end to end.
    """
    n, d = kappa.shape
    active = [c for c in range(d) if t[c] > 0]
    blk = np.arange(n) // BLOCK
    khat = np.zeros((n, len(active)), dtype=np.float64)
    for i, c in enumerate(active):
        khat[:, i] = reconstruct(kappa[:, c], int(t[c]), delta[c, blk])
    qa = np.asarray(q, dtype=np.float32).astype(np.float64)[active]
    s = khat @ qa
    a = np.abs(khat) @ np.abs(qa)
    return s, a


def tolerance(a: np.ndarray) -> np.ndarray:
    """Per-score tolerance 1e-4 * sum_c |q_c * k_hat_c|."""
    return TOL_REL * np.asarray(a, dtype=np.float64)


def topk(s: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, lowest index first among equal scores,
    returned in ascending index order ([Digest] key module 5 and Output: the
    scan outputs top-k key indices per query)."""
    n = s.shape[0]
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    order = np.lexsort((np.arange(n), -np.asarray(s, dtype=np.float64)))
    return np.sort(order[:k])


# ---------------------------------------------------------------------------
# Appending keys during decoding.  The pages fix the block scale over a whole
# 128-key block ([Review] Strengths, paper Sec 3.2), so a block can only be
# quantised once it is full; they say nothing about the newest keys.  Reading:
# full blocks are sealed (scaled and packed) as they fill, and the open tail
# block, fewer than 128 keys, is kept exact in fp32 and scored exactly.
# ---------------------------------------------------------------------------

def tail_scores(q: np.ndarray, tail_k: np.ndarray):
    """Exact scores of unquantised tail keys: s_j = sum_c q_c k_jc in fp64 (each
    product of two fp32 values is exact in fp64), and A_j = sum_c |q_c k_jc|.
    tail_k float32 [m, d]."""
    qq = np.asarray(q, dtype=np.float32).astype(np.float64)
    kk = np.asarray(tail_k, dtype=np.float32).astype(np.float64)
    return kk @ qq, np.abs(kk) @ np.abs(qq)


def step_append(k_sealed, tail_k, q, sigma2, budget, k, mode="waterfill"):
    """One top-k step over n_sealed quantised keys plus an exact open tail.

    k_sealed float32 [h_kv, n_sealed, d] (the keys of the sealed blocks);
    tail_k float32 [h_kv, m, d] (keys n_sealed .. n_sealed + m - 1).  Scores of
    sealed keys are the scan's (``scores``), of tail keys ``tail_scores``; the
    top k over all n_sealed + m keys as in ``topk``."""
    h_kv, n_s, d = k_sealed.shape
    m = tail_k.shape[1]
    h_q = q.shape[0]
    g = h_q // h_kv
    base = step(k_sealed, q, sigma2, budget, min(k, n_s), mode=mode) if n_s > 0 else None
    idx = np.zeros((h_q, k), dtype=np.int64)
    s_all, a_all = [], []
    for h in range(h_q):
        st, at = tail_scores(q[h], tail_k[h // g])
        if base is not None:
            s = np.concatenate([base["scores"][h], st])
            a = np.concatenate([base["sums"][h], at])
        else:
            s, a = st, at
        idx[h] = topk(s, k)
        s_all.append(s)
        a_all.append(a)
    depth = base["depth"] if base is not None else None
    union = base["union"] if base is not None else None
    return {"depth": depth, "union": union, "idx": idx, "scores": s_all, "sums": a_all}


# ---------------------------------------------------------------------------
# One whole step for a GQA layer, the way the scan runs it.
# ---------------------------------------------------------------------------

def step(k_heads, q, sigma2, budget, k, mode="waterfill", packed=None):
    """Reference result of one top-k step over a layer.

    k_heads: float32 [h_kv, n, d]; q: float32 [h_q, d]; sigma2: float32 [h_kv, d].
    mode "waterfill": reverse water-filling with ``budget`` bits per key;
    mode "topq": 4 planes on budget // 4 channels of largest |q_c|;
    mode "group": one water-filling per KV head on the group importance;
    mode "static": 4 planes on budget // 4 channels of largest sigma2.
    ``packed`` may hold precomputed (delta, kappa) per KV head.
    Returns dict with depth [h_q, d], union [h_kv, d], idx [h_q, k], and the
    fp64 scores/sums per query head.
    """
    h_kv, n, d = k_heads.shape
    h_q = q.shape[0]
    g = h_q // h_kv
    depth = np.zeros((h_q, d), dtype=np.int64)
    for h in range(h_q):
        if mode == "waterfill":
            depth[h] = waterfill_depths(importance(q[h], sigma2[h // g]), budget)
        elif mode == "group":
            kv = h // g
            depth[h] = waterfill_depths(group_importance(q[kv * g:(kv + 1) * g], sigma2[kv]), budget)
        elif mode == "static":
            if budget % PLANES:
                raise ValueError("fixed mode needs budget % 4 == 0")
            depth[h] = static_depths(sigma2[h // g], budget // PLANES)
        else:
            if budget % PLANES:
                raise ValueError("fixed mode needs budget % 4 == 0")
            depth[h] = topq_depths(q[h], budget // PLANES)
    union = np.stack([union_depths(depth[kv * g:(kv + 1) * g]) for kv in range(h_kv)])
    idx = np.zeros((h_q, k), dtype=np.int64)
    s_all, a_all = [], []
    for kv in range(h_kv):
        if packed is not None:
            delta, kappa = packed[kv]
        else:
            delta = block_scales(k_heads[kv])
            kappa = quantize_codes(k_heads[kv], delta)
        for h in range(kv * g, (kv + 1) * g):
            s, a = scores(q[h], kappa, delta, depth[h])
            idx[h] = topk(s, k)
            s_all.append(s)
            a_all.append(a)
    return {"depth": depth, "union": union, "idx": idx,
            "scores": s_all, "sums": a_all}
