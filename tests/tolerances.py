"""Acceptance tolerances of the GPU attention against the oracle's fp64 values.

These are test criteria, not the method's arithmetic, so they live with the
tests.  The oracle (``oracle/attention_oracle.py``) supplies the exact values;
the functions here only bound how far an fp32 evaluation may stray from them.

``attention_tolerance`` assumes nothing about how a kernel blocks its work: any
fp32 evaluation of the attention of one query over m listed keys, whatever the
order of its sums, stays within it.  ``attention_tolerance(..., logit_chain=L,
sum_chain=C)`` gives the tighter bound of a kernel whose sums are known to be
at most L and C roundings deep; the GPU tests check that one as well, as a
second, stricter criterion.

Derivation (u = 2^-24, the fp32 unit roundoff; A_j = |scale| sum_c |q_c K_jc|):
  * a logit s_j = scale * sum_c q_c K_jc formed with products, fused or not,
    and additions in any order carries at most L roundings on its path, so
    |ds_j| <= L u A_j =: e_s with L = d + 2 in general (d products and adds,
    the scale), and 2 e_s on s_j - M (M a computed logit);
  * exp(s_j - M) then has relative error eta <= 2 e_s + u + (a few u for
    expf), the u |s_j - M| of the subtraction being weighted by
    p_j <= e^-(M - s_j), i.e. at most u/e per unit of weight;
  * the numerator sum_j w_j V_jc and the denominator sum_j w_j, summed along
    chains of at most C additions (C = m, the list length, for any order),
    add C u relative to their sums of absolute terms, so
      |do_c| <= (2 eta + 2 C u) sum_j p_j |V_jc|,
      |dlse| <= e_s + eta + C u + 2 u |lse|;
  * a factor 4 covers expf's few-ulp error and the second-order terms.
"""

from __future__ import annotations

import numpy as np

from oracle import attention_oracle as A


def attention_tolerance(q, k_rows, v_rows, idx, scale, logit_chain: int | None = None,
                        sum_chain: int | None = None):
    """(tau_o float64 [d], tau_lse) for the attention of q over the keys idx.

    logit_chain: roundings on a logit's path (default d + 2: any order).
    sum_chain:   additions on the numerator's and denominator's paths
                 (default: the number of valid listed keys, any order)."""
    n, d = k_rows.shape
    o, lse, p, valid = A.sparse_attention(q, k_rows, v_rows, idx, scale)
    if valid.size == 0:
        return np.zeros(d), 0.0
    L = d + 2 if logit_chain is None else logit_chain
    C = valid.size if sum_chain is None else sum_chain
    u = 2.0 ** -24
    kk = A.bf16_to_f64(k_rows[valid])
    a = abs(float(np.float32(scale))) * (np.abs(kk) @ np.abs(np.asarray(q, np.float32).astype(np.float64)))
    e_s = L * u * a.max()
    eta = 2 * e_s + u + 4 * u
    pv = p @ np.abs(A.bf16_to_f64(v_rows[valid]))
    tau_o = 4 * (2 * eta + 2 * C * u) * pv
    tau_lse = 4 * (e_s + eta + C * u + 2 * u * abs(lse))
    return tau_o, tau_lse
