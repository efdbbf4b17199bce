"""Seeded synthetic workloads for the Fathom key scan.

This module only draws random inputs; it holds none of the method's
arithmetic (no quantisation, allocation, scoring or selection).  Both the CPU
oracle (through the tests and the benchmark) and the GPU path consume what it
returns, so the two sides always see identical inputs.

Recipe (one numpy ``Generator`` per (workload, layer, session, KV head)):
  sigma   = exp(N(0, 1)) per channel  (log-normal per-channel std)
  outliers: 4 channels with 10x std (Qwen3-8B-shaped workloads only)
  K       = N(0, 1) * sigma, float32, token-major [n, d]
  q       = N(0, 1), float32 [G, d], from a separate stream of the same seed
  sigma2  = float32(sigma) ** 2 in float32 (the "offline statistics" input)
The pages time synthetic contexts beyond 128k tokens at batch 1; these
arrays stand in for them.  No dataset or model weights are used.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED = 0


@dataclass(frozen=True)
class Workload:
    """Shape and budget of one synthetic workload."""
    key: int                  # workload id used in the seed
    name: str
    h_kv: int
    g: int                    # query heads per KV head
    d: int
    n: int
    budgets: tuple            # per-layer bit budgets (one entry per layer)
    k: int
    residency: str            # "hbm" or "host"
    outliers: int             # channels with 10x std
    sessions: int = 1
    mode: str = "waterfill"   # or "topq" for the fixed-depth comparison scans
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def layers(self) -> int:
        return len(self.budgets)

    @property
    def h_q(self) -> int:
        return self.h_kv * self.g


def layer_budgets(count: int = 36, lo: int = 46, hi: int = 92) -> tuple:
    """Per-layer budgets drawn uniformly from [lo, hi] (a fixed seeded draw)."""
    rng = np.random.default_rng([SEED, 4, 999])
    return tuple(int(b) for b in rng.integers(lo, hi + 1, count))


def workloads() -> dict:
    """The five workloads: small single head; 131072-key HBM layer; 1M-key host
    layer; 36-layer 1M-key host decode step; 8 sessions of 262144 keys."""
    w = {}
    w["w1_single_head_4k"] = Workload(1, "single head, n=4096, HBM", 1, 1, 128, 4096, (64,), 64, "hbm", 0)
    for b in (46, 68, 92):
        w[f"w2_hbm_131k_B{b}"] = Workload(2, f"8x4 heads, n=131072, HBM, B={b}", 8, 4, 128, 131072, (b,), 2048, "hbm", 4)
    w["w3_host_1m_B92"] = Workload(3, "8x4 heads, n=1048576, host, B=92", 8, 4, 128, 1 << 20, (92,), 2048, "host", 4)
    w["w4_host_1m_36layers"] = Workload(4, "36 layers x 8x4 heads, n=1048576, host", 8, 4, 128, 1 << 20,
                                        layer_budgets(), 2048, "host", 4)
    w["w5_sessions_262k_B68"] = Workload(5, "8 sessions x 8x4 heads, n=262144, host, B=68", 8, 4, 128, 262144,
                                         (68,), 2048, "host", 4, sessions=8)
    w["w5_sessions_262k_fixed136"] = Workload(5, "8 sessions, fixed 34 ch x 4 bits", 8, 4, 128, 262144,
                                              (136,), 2048, "host", 4, sessions=8, mode="topq")
    w["w5_sessions_262k_fixed68"] = Workload(5, "8 sessions, fixed 17 ch x 4 bits", 8, 4, 128, 262144,
                                             (68,), 2048, "host", 4, sessions=8, mode="topq")
    return w


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([SEED, *key]))


def _sigma(rng: np.random.Generator, d: int, outliers: int) -> np.ndarray:
    """Per-channel std of one KV head: the first draws of its stream."""
    sigma = np.exp(rng.standard_normal(d)).astype(np.float32)
    if outliers:
        idx = rng.choice(d, outliers, replace=False)
        sigma[idx] *= np.float32(10.0)
    return sigma


def kv_head(wl_key: int, layer: int, session: int, g: int, n: int, d: int, outliers: int):
    """(K float32 [n, d], sigma2 float32 [d]) of one KV head."""
    rng = _rng(wl_key, layer, session, g)
    sigma = _sigma(rng, d, outliers)
    k = rng.standard_normal((n, d), dtype=np.float32)
    k *= sigma
    sigma2 = (sigma * sigma).astype(np.float32)
    return k, sigma2


def kv_sigma2(wl_key: int, layer: int, session: int, g: int, d: int, outliers: int) -> np.ndarray:
    """sigma2 float32 [d] of one KV head, the same values kv_head() returns,
    without drawing its keys."""
    sigma = _sigma(_rng(wl_key, layer, session, g), d, outliers)
    return (sigma * sigma).astype(np.float32)


def layer_queries(wl: "Workload", layer: int = 0):
    """(q [S*h_q, d], sigma2 [S*h_kv, d]) of one layer, equal to those of
    layer_inputs(), without drawing any keys."""
    hk = wl.sessions * wl.h_kv
    s2 = np.empty((hk, wl.d), dtype=np.float32)
    q = np.empty((hk * wl.g, wl.d), dtype=np.float32)
    for v in range(hk):
        s, g = divmod(v, wl.h_kv)
        s2[v] = kv_sigma2(wl.key, layer, s, g, wl.d, wl.outliers)
        q[v * wl.g:(v + 1) * wl.g] = queries(wl.key, layer, s, g, wl.g, wl.d)
    return q, s2


def queries(wl_key: int, layer: int, session: int, g: int, count: int, d: int) -> np.ndarray:
    """float32 [count, d] query heads that share KV head g."""
    return _rng(wl_key, layer, session, g, 1).standard_normal((count, d), dtype=np.float32)


def layer_inputs(wl: Workload, layer: int = 0, n: int | None = None, threads: int = 8):
    """All inputs of one layer: K [S*h_kv, n, d], q [S*h_q, d], sigma2 [S*h_kv, d].

    Sessions are laid out as extra KV heads (session-major), since sessions
    never mix: session s, KV head g is virtual KV head s*h_kv + g.
    ``n`` may shrink the key count for a cheaper variant of the same recipe.
    KV heads are drawn in parallel threads (each from its own seeded stream,
    so the result does not depend on the thread count).
    """
    from concurrent.futures import ThreadPoolExecutor
    n = wl.n if n is None else n
    hk = wl.sessions * wl.h_kv
    k = np.empty((hk, n, wl.d), dtype=np.float32)
    s2 = np.empty((hk, wl.d), dtype=np.float32)
    q = np.empty((hk * wl.g, wl.d), dtype=np.float32)

    def one(v):
        s, g = divmod(v, wl.h_kv)
        k[v], s2[v] = kv_head(wl.key, layer, s, g, n, wl.d, wl.outliers)
        q[v * wl.g:(v + 1) * wl.g] = queries(wl.key, layer, s, g, wl.g, wl.d)

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(one, range(hk)))
    return k, q, s2


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Storage format of a bf16 cache: the fp32 values rounded to bf16 (round to
    nearest, ties to even) and returned as uint16 bit patterns.  Inputs are
    finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + r) >> np.uint32(16)).astype(np.uint16)


def values(wl_key: int, layer: int, session: int, g: int, n: int, d: int) -> np.ndarray:
    """float32 [n, d] value rows of one KV head: N(0, 1) from the stream [..., 2]."""
    return _rng(wl_key, layer, session, g, 2).standard_normal((n, d), dtype=np.float32)


def kv_rows_bf16(wl_key: int, layer: int, session: int, g: int, n: int, d: int, outliers: int):
    """(K bf16 [n, d], V bf16 [n, d]) cache rows of one KV head: K is the same
    draw as kv_head() rounded to bf16, V is values() rounded to bf16."""
    k, _ = kv_head(wl_key, layer, session, g, n, d, outliers)
    return to_bf16_bits(k), to_bf16_bits(values(wl_key, layer, session, g, n, d))


def small_case(seed: int, h_kv: int, g: int, n: int, d: int, outliers: int = 0):
    """A small seeded case with the same recipe, for parity tests at odd shapes."""
    rng = _rng(1000 + seed)
    k = np.empty((h_kv, n, d), dtype=np.float32)
    s2 = np.empty((h_kv, d), dtype=np.float32)
    for v in range(h_kv):
        sigma = np.exp(rng.standard_normal(d)).astype(np.float32)
        if outliers:
            sigma[rng.choice(d, min(outliers, d), replace=False)] *= np.float32(10.0)
        k[v] = rng.standard_normal((n, d), dtype=np.float32) * sigma
        s2[v] = sigma * sigma
    q = rng.standard_normal((h_kv * g, d), dtype=np.float32)
    return k, q, s2
