"""Selection fidelity of the Fathom scan on seeded synthetic caches, from the oracle.

For each selection mode it reports, over the query heads of the 8 KV x 4 query
head, n = 131072, k = 2048 workload (same generator as the HBM-resident
workload: log-normal channel std, 4 outlier channels at 10x):

  recall      share of the exact top-k (largest q . K_j over the unquantised
              fp32 keys) that the mode's top-k contains;
  attn error  |o_S - o_all| / |o_all|, attention over the selected keys
              against attention over all n keys, both on the same bf16 K/V
              rows, softmax scale 1/sqrt(d).

Modes: reverse water-filling at B = 46, 68, 92 bits per key and at B = 4d
(every plane: the exact 4-bit scores), the group-shared allocation, and the
fixed-depth comparison scans that read 4 planes of the m channels of largest
|q_c| (m = 17: 68 bits, m = 34: 136 bits) or of largest offline sigma_c^2.
The pages measure these quantities on a real model; on synthetic keys the
numbers describe the allocation rule on this generator only.

Everything here is the oracle's arithmetic (allocation, fp64 scores, top-k,
fp64 attention); the GPU path selects the same keys (its parity tests), so the
figures hold for it.  CPU only:

    python -m tests.fidelity_report [--n 131072] [--kv-heads 8] [--k 2048]
    python -m tests.fidelity_report --workload w3_host_1m_B92 --n 1048576 --kv-heads 1

(``--workload`` picks whose seeded keys and queries are drawn; the modes and
k stay as above.)
"""

from __future__ import annotations

import argparse
import time

import numpy as np

from oracle import attention_oracle as A
from oracle import fathom_oracle as O
import synthetic

MODES = (
    ("water-filling, B = 46", "waterfill", 46),
    ("water-filling, B = 68", "waterfill", 68),
    ("water-filling, B = 92", "waterfill", 92),
    ("water-filling, B = 4d (all planes)", "waterfill", None),
    ("group-shared water-filling, B = 92", "group", 92),
    ("fixed top-|q|, 17 ch x 4 planes (68 bits)", "topq", 68),
    ("fixed top-|q|, 34 ch x 4 planes (136 bits)", "topq", 136),
    ("fixed top-sigma^2, 17 ch x 4 planes (68 bits)", "static", 68),
    ("fixed top-sigma^2, 34 ch x 4 planes (136 bits)", "static", 136),
)


def measure(n: int = 131072, kv_heads: int = 8, k: int = 2048, modes=MODES,
            workload: str = "w2_hbm_131k_B92"):
    """Per mode: (label, bits, recall [h_q], attention error [h_q]); the first
    row is the exact top-k (fp32 keys, 32 d bits)."""
    wl = synthetic.workloads()[workload]
    wl_key = wl.key
    d, g = wl.d, wl.g
    scale = 1.0 / np.sqrt(d)
    kh = np.empty((kv_heads, n, d), np.float32)
    s2 = np.empty((kv_heads, d), np.float32)
    q = np.empty((kv_heads * g, d), np.float32)
    rows = []
    for v in range(kv_heads):
        kh[v], s2[v] = synthetic.kv_head(wl_key, 0, 0, v, n, d, wl.outliers)
        q[v * g:(v + 1) * g] = synthetic.queries(wl_key, 0, 0, v, g, d)
        rows.append((synthetic.to_bf16_bits(kh[v]),
                     synthetic.to_bf16_bits(synthetic.values(wl_key, 0, 0, v, n, d))))
    packed = []
    for v in range(kv_heads):
        delta = O.block_scales(kh[v])
        packed.append((delta, O.quantize_codes(kh[v], delta)))
    # exact references: top-k of the fp32 keys, attention over all n keys
    exact_idx, full = [], []
    for h in range(kv_heads * g):
        v = h // g
        s = kh[v].astype(np.float64) @ q[h].astype(np.float64)
        exact_idx.append(O.topk(s, k))
        full.append(A.sparse_attention(q[h], rows[v][0], rows[v][1], np.arange(n), scale)[0])
    # the floor: the exact top-k itself, whose error is the mass of the other n - k keys
    out = [("exact top-k of the fp32 keys", 32 * d, np.ones(kv_heads * g),
            np.array([A.attention_error(q[h], rows[h // g][0], rows[h // g][1], exact_idx[h], scale,
                                        full=full[h]) for h in range(kv_heads * g)]))]
    for label, mode, budget in modes:
        b = O.PLANES * d if budget is None else budget
        res = O.step(kh, q, s2, b, k, mode=mode, packed=packed)
        rec = np.array([A.topk_recall(res["idx"][h], exact_idx[h]) for h in range(kv_heads * g)])
        err = np.array([A.attention_error(q[h], rows[h // g][0], rows[h // g][1], res["idx"][h], scale,
                                          full=full[h]) for h in range(kv_heads * g)])
        out.append((label, b, rec, err))
    return out


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--n", type=int, default=131072)
    ap.add_argument("--kv-heads", type=int, default=8)
    ap.add_argument("--k", type=int, default=2048)
    ap.add_argument("--workload", default="w2_hbm_131k_B92",
                    choices=["w2_hbm_131k_B92", "w3_host_1m_B92", "w5_sessions_262k_B68"])
    a = ap.parse_args(argv)
    t0 = time.time()
    res = measure(a.n, a.kv_heads, a.k, workload=a.workload)
    print(f"{a.workload} keys: n = {a.n}, {a.kv_heads} KV heads x 4 query heads, k = {a.k} "
          f"({time.time() - t0:.0f} s)")
    print("| mode | bits per key | recall of the exact top-k: mean (min) | attention error: mean (max) |")
    print("|---|---|---|---|")
    for label, b, rec, err in res:
        print(f"| {label} | {b} | {rec.mean():.3f} ({rec.min():.3f}) | {err.mean():.4f} ({err.max():.4f}) |")


if __name__ == "__main__":
    main()
