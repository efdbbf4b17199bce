"""Parity helpers shared by the GPU tests: run the HIP path on numpy inputs and
compare with the oracle by the acceptance rules.

Rules (all from the method's definition):
  * records and depths: bit-exact;
  * scores: |s_gpu - s_oracle| <= 1e-4 * sum_c |q_c k_hat_c| per (head, key);
  * top-k: k distinct in-range indices in ascending order; the GPU set equals
    the exact top-k of the GPU's own scores (selection is exact); and against
    the oracle's set, every index in the symmetric difference lies within the
    score tolerance of the oracle's k-th score (boundary ties only).
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import fathom_oracle as O


def dev(a, device="cuda:0"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def gpu_pack(k_np, device="cuda:0"):
    from sparse_attention_top_query_amd import fathom
    k = dev(k_np, device)
    status = torch.full((1,), -1, dtype=torch.int32, device=device)
    rec = fathom.pack(k, status=status)
    return rec, int(status.item())


def oracle_pack(k_np):
    """Per KV head (delta, kappa, records) from the oracle."""
    return [O.pack_head(k_np[g]) for g in range(k_np.shape[0])]


def oracle_depths(q, s2, budget, mode="waterfill"):
    h_q, d = q.shape
    g = h_q // s2.shape[0]
    dep = np.zeros((h_q, d), np.int64)
    for h in range(h_q):
        if mode == "waterfill":
            dep[h] = O.waterfill_depths(O.importance(q[h], s2[h // g]), budget)
        elif mode == "group":
            kv = h // g
            dep[h] = O.waterfill_depths(O.group_importance(q[kv * g:(kv + 1) * g], s2[kv]), budget)
        elif mode == "static":
            dep[h] = O.static_depths(s2[h // g], budget // 4)
        else:
            dep[h] = O.topq_depths(q[h], budget // 4)
    uni = np.stack([O.union_depths(dep[v * g:(v + 1) * g]) for v in range(s2.shape[0])])
    return dep, uni


def check_scores(s_gpu, s_or, a_or, where=""):
    err = np.abs(s_gpu.astype(np.float64) - s_or)
    tol = O.tolerance(a_or)
    bad = err > tol
    assert not bad.any(), (f"{where}: {int(bad.sum())} scores out of tolerance; worst excess "
                           f"{float(np.max(err - tol)):.3e} at {int(np.argmax(err - tol))}")
    return float(np.max(err / np.maximum(a_or, 1e-300)))


def check_topk(idx_gpu, s_or, a_or, k, s_gpu=None, where=""):
    idx_gpu = np.asarray(idx_gpu, dtype=np.int64)
    n = s_or.shape[0]
    assert idx_gpu.shape == (k,), where
    assert np.all(np.diff(idx_gpu) > 0), f"{where}: indices not strictly ascending"
    assert idx_gpu.min(initial=0) >= 0 and idx_gpu.max(initial=0) < n, f"{where}: index out of range"
    if s_gpu is not None:
        # selection itself is exact on the GPU's scores (ties: lowest index)
        assert np.array_equal(idx_gpu, O.topk(s_gpu.astype(np.float64), k)), f"{where}: select not exact"
    want = O.topk(s_or, k)
    gs, os_ = set(idx_gpu.tolist()), set(want.tolist())
    extra, missing = sorted(gs - os_), sorted(os_ - gs)
    if not extra:
        return 0
    theta = np.min(s_or[want])
    tau = O.tolerance(a_or)
    t_missing = max(tau[j] for j in missing)
    t_extra = max(tau[j] for j in extra)
    for j in extra:
        assert theta - s_or[j] <= tau[j] + t_missing, f"{where}: extra key {j} not a boundary tie"
    for j in missing:
        assert s_or[j] - theta <= tau[j] + t_extra, f"{where}: missing key {j} not a boundary tie"
    return len(extra)
