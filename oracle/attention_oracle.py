"""Plain CPU oracle for sparse attention over the selected keys.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
never imports, calls or links it, and it imports nothing from the product path.

What it follows.  On the pages about "Fathom: Per-Query Read Depth for Sparse
Decoding over Offloaded KV Caches" (arXiv 2609.17652), the scan produces the
top-k key indices of each query and real attention is then computed over those
keys only ([Digest] Output; [Review] "Frequently asked questions": the scan
picks the top-k for sparse attention).  The pages give no formula for that
attention, so the reading taken is the standard one:

    s_j = scale * (q . K_j)                   for j in the query's index set S
    M   = max_j s_j
    o   = sum_j exp(s_j - M) V_j / sum_j exp(s_j - M)
    lse = M + log sum_j exp(s_j - M)          (= log sum_j exp(s_j))

with K and V the cache rows as the serving stack holds them (bf16, token-major
[n][d]), one query head at a time; a query head of a GQA group uses the rows of
its KV head.  Index entries outside [0, n) are skipped; with none left, o = 0
and lse = -inf.

Precision: bf16 values and fp32 q are exact in fp64, every product q_c K_jc is
exact (24 + 8 significant bits), and the rest is fp64.

Parity status (what pins it, in tests/test_oracle_attention.py):
  bf16_to_f64           pinned: hand-decoded bit patterns (normal, negative,
                        largest finite, subnormal, signed zero).
  sparse_attention      pinned: the full index set equals dense softmax
                        attention from scipy.special.softmax and a matmul;
                        one key gives V_j and lse = s_j exactly; q = 0 gives
                        the mean of the rows (exact rationals) and lse = log k;
                        two keys follow the logistic closed form; invariance
                        to the order of the index set; huge common logits do
                        not overflow; skipped indices equal the valid subset.
  topk_recall           pinned: identical, disjoint and half-overlapping sets
                        (exact fractions), order independence.
  attention_error       pinned: 0 for the full index set and for constant
                        value rows; the two-key closed form (one key kept:
                        error = p_1 |V_1 - V_0| / |o|, p from scipy's
                        softmax); value rows e_0 on the kept keys and e_1 on
                        the others at q = 0, where the error is
                        sqrt(2) (1 - m) / sqrt(m^2 + (1 - m)^2) for the kept
                        share m = |S| / n.

Fidelity metrics.  The pages report "attention error" against full attention
and the recovery of the exact top-k (every per-token scan matching exact top-k
decoding on RULER-style tasks), measured on a real model ([Abstract];
[Digest] Experiments: design and key findings), without formulas.  Readings taken, for seeded synthetic
caches: attention error is the relative L2 distance of the query's attention
over the selected keys from its attention over all n keys, both with the same
bf16 K/V rows; recall is the fraction of the exact top-k (largest q . K_j with
K the unquantised fp32 keys, lowest index first on ties) that the selection
contains.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns (uint16): a bf16 value is the fp32 value whose
    upper 16 bits are the pattern and whose lower 16 bits are zero."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def logits(q: np.ndarray, k_rows: np.ndarray, idx: np.ndarray, scale: float) -> np.ndarray:
    """s_j = scale * (q . K_j) in fp64 for the entries of idx (already valid)."""
    kk = bf16_to_f64(k_rows[idx])                       # [m, d]
    return np.float64(np.float32(scale)) * (kk @ np.asarray(q, np.float32).astype(np.float64))


def sparse_attention(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, idx: np.ndarray,
                     scale: float):
    """Attention of one query over the keys idx of one KV head.

    q float32 [d]; k_rows, v_rows uint16 (bf16) [n, d]; idx integer [k].
    Returns (o float64 [d], lse float64, p float64 [m] weights of the valid
    entries, valid int64 [m] their indices in idx order)."""
    n, d = k_rows.shape
    idx = np.asarray(idx, dtype=np.int64)
    valid = idx[(idx >= 0) & (idx < n)]
    if valid.size == 0:
        return np.zeros(d), -np.inf, np.zeros(0), valid
    s = logits(q, k_rows, valid, scale)
    m = s.max()
    w = np.exp(s - m)
    total = w.sum()
    p = w / total
    o = p @ bf16_to_f64(v_rows[valid])
    return o, m + np.log(total), p, valid


def topk_recall(idx: np.ndarray, exact_idx: np.ndarray) -> float:
    """|S & S*| / |S*|: the share of the exact top-k index set S* that the
    selection S contains (both index sets, duplicates not allowed)."""
    exact = np.asarray(exact_idx, dtype=np.int64)
    if exact.size == 0:
        return 1.0
    hit = np.intersect1d(np.asarray(idx, dtype=np.int64), exact, assume_unique=True)
    return hit.size / exact.size


def attention_error(q: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, idx: np.ndarray,
                    scale: float, full=None) -> float:
    """|o_S - o_all| / |o_all| (Euclidean norms over the d channels): o_S is the
    attention of q over the keys idx, o_all over all n keys of the same rows.
    ``full`` may pass a precomputed o_all."""
    n = k_rows.shape[0]
    o_all = sparse_attention(q, k_rows, v_rows, np.arange(n), scale)[0] if full is None else full
    o_s = sparse_attention(q, k_rows, v_rows, idx, scale)[0]
    return float(np.linalg.norm(o_s - o_all) / np.linalg.norm(o_all))
