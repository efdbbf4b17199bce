"""GPU parity of the top-k selection on its own: on every case scan_topk returns
exactly the top k of the GPU's own scores (lowest index among equal scores,
ascending) with those scores bit for bit, from HBM and pinned host records.
The cases include rows whose candidates overflow a chunk's slot (all scores
equal; scores rising with the index), which take the exact in-order
fallback, and rows long enough for many chunks."""

import numpy as np
import pytest
import torch

from oracle import fathom_oracle as O
from synthetic import small_case
from tests.parity import dev, gpu_pack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    from sparse_attention_top_query_amd import fathom
    fathom.load()
    assert torch.cuda.is_available()
    return fathom


def select(F, rec, dq, dep, uni, n, k):
    idx, val = F.scan_topk(rec, dq, dep, uni, n, k, want_scores=True)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def check_exact(idx, val, sg, k, where):
    for h in range(sg.shape[0]):
        want = O.topk(sg[h].astype(np.float64), k)
        assert np.array_equal(idx[h], want), f"{where} head {h}: not the exact top {k} of the GPU scores"
        assert np.array_equal(val[h].view(np.uint32), sg[h][idx[h]].view(np.uint32)), f"{where} head {h}"


CASES = [  # (h_kv, g, n, d, budget, ks)
    (2, 4, 5000, 128, 92, (1, 300, 5000)),
    (1, 1, 4096, 64, 64, (1, 64, 4095)),
    (1, 2, 777, 32, 40, (777,)),
    (4, 1, 65536 + 5, 128, 92, (2048,)),
    (1, 16, 3000, 128, 68, (1000,)),
    (2, 8, 20000 + 37, 64, 46, (2048, 7000)),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("residency", ["hbm", "host"])
def test_select_is_exact(F, case, residency):
    h_kv, g, n, d, budget, ks = case
    print(f"select case={case} residency={residency}", flush=True)
    kk, q, s2 = small_case(sum(case[:5]), h_kv, g, n, d, outliers=min(4, d))
    rec, st = gpu_pack(kk)
    assert st == 0
    if residency == "host":
        rec = rec.cpu().pin_memory()
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    sg = F.scan_scores(rec, dq, dep, uni, n).cpu().numpy()
    for k in ks:
        idx, val = select(F, rec, dq, dep, uni, n, k)
        check_exact(idx, val, sg, k, where=f"{case} k={k}")


def rising_case(n, d=64, seed=5):
    """Keys whose scores rise with the index: every candidate lies in the last
    chunks of the row, more than a chunk's slot holds."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d).astype(np.float32)
    ramp = (np.arange(n, dtype=np.float32) / n + 0.05)[:, None]
    k = (ramp * u[None, :] + 0.01 * rng.standard_normal((n, d))).astype(np.float32)[None]
    q = u[None, :].copy()
    s2 = np.ones((1, d), np.float32)
    return k, q, s2


@pytest.mark.parametrize("n,k", [(40000, 2048), (40000, 1500), (70001, 4000)])
def test_rising_scores_overflow_a_slot(F, n, k):
    kk, q, s2 = rising_case(n)
    rec, _ = gpu_pack(kk)
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), 4 * q.shape[1])
    sg = F.scan_scores(rec, dq, dep, uni, n).cpu().numpy()
    idx, val = select(F, rec, dq, dep, uni, n, k)
    check_exact(idx, val, sg, k, where=f"rising n={n}")
    assert idx[0].min() > n // 2          # the selection really sits at the end of the row


@pytest.mark.parametrize("n", [3000, 20000])
def test_all_equal_scores(F, n):
    """Budget 0: every score is 0, every key is a candidate; the lowest indices win
    (the exact in-order fallback)."""
    kk, q, s2 = small_case(3, 1, 4, n, 32)
    rec, _ = gpu_pack(kk)
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), 0)
    for k in (1, 1024, n):
        idx, val = select(F, rec, dq, dep, uni, n, k)
        assert np.array_equal(idx, np.tile(np.arange(k), (4, 1)))
        assert np.all(val == 0)


def test_workspace_reuse_across_shapes_and_residencies(F):
    """One workspace serves calls of different n, k and residency in turn (the
    HBM scan zeroes the selection counters, the host scan clears and fills
    them): no state of an earlier call leaks into a later one."""
    h_kv, g, d = 2, 4, 64
    kk, q, s2 = small_case(41, h_kv, g, 40000, d, outliers=4)
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), 40)
    recs = {}
    for n in (40000, 9000, 40000 - 77):
        rec, st = gpu_pack(np.ascontiguousarray(kk[:, :n]))
        assert st == 0
        recs[(n, "hbm")] = rec
        recs[(n, "host")] = rec.cpu().pin_memory()
    ws = torch.full((F.workspace_bytes(h_q=h_kv * g, h_kv=h_kv, n=40000, d=d, k=3000, residency=F.HOST_STAGED),),
                    0x7F, dtype=torch.uint8, device="cuda:0")      # garbage to start from
    order = [(40000, "hbm", 3000), (9000, "host", 50), (40000 - 77, "hbm", 1), (40000, "host", 2048),
             (9000, "hbm", 9000), (40000 - 77, "staged", 700), (40000, "hbm", 3000)]
    for n, res, k in order:
        rec = recs[(n, "hbm" if res == "hbm" else "host")]
        residency = {"hbm": F.HBM, "host": F.HOST_DIRECT, "staged": F.HOST_STAGED}[res]
        sg = F.scan_scores(rec, dq, dep, uni, n, residency=residency).cpu().numpy()
        idx, val = F.scan_topk(rec, dq, dep, uni, n, k, residency=residency, workspace=ws, want_scores=True)
        torch.cuda.synchronize()
        check_exact(idx.cpu().numpy(), val.cpu().numpy(), sg, k, where=f"n={n} {res} k={k}")


@pytest.mark.parametrize("n", [1, 2, 5, 127, 128, 129, 1023, 1025])
@pytest.mark.parametrize("residency", ["hbm", "host", "staged"])
def test_tiny_rows(F, n, residency):
    """Rows shorter than one tile, one block or one 32-key word: scores match the
    oracle and every k from 1 to n selects exactly."""
    h_kv, g, d, budget = 2, 4, 32, 20
    kk, q, s2 = small_case(n, h_kv, g, n, d, outliers=2)
    rec, st = gpu_pack(kk)
    assert st == 0
    if residency != "hbm":
        rec = rec.cpu().pin_memory()
    res = {"hbm": F.HBM, "host": F.HOST_DIRECT, "staged": F.HOST_STAGED}[residency]
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    sg = F.scan_scores(rec, dq, dep, uni, n, residency=res).cpu().numpy()
    rd = dep.cpu().numpy()
    for h in range(h_kv * g):
        delta = O.block_scales(kk[h // g])
        kappa = O.quantize_codes(kk[h // g], delta)
        s, a = O.scores(q[h], kappa, delta, rd[h])
        assert np.all(np.abs(sg[h].astype(np.float64) - s) <= O.tolerance(a)), f"head {h}"
    for k in sorted({1, (n + 1) // 2, n}):
        idx, val = F.scan_topk(rec, dq, dep, uni, n, k, residency=res, want_scores=True)
        torch.cuda.synchronize()
        check_exact(idx.cpu().numpy(), val.cpu().numpy(), sg, k, where=f"n={n} {residency} k={k}")


@pytest.mark.parametrize("rising", [False, True])
def test_rows_of_more_than_1024_chunks(F, rising):
    """Rows of more than 1024 select chunks (over 4M keys): the resolve gathers
    chunk ranges per thread; with rising scores the kept keys also sit in spill
    segments of the last chunks."""
    n, d = 4_300_000, 16
    if rising:
        kk, q, s2 = rising_case(n, d=d, seed=8)
    else:
        kk, q, s2 = small_case(13, 1, 2, n, d, outliers=2)
    rec, st = gpu_pack(kk)
    assert st == 0
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), 4 * d if rising else 24)
    sg = F.scan_scores(rec, dq, dep, uni, n).cpu().numpy()
    for k in (1, 2048, 5000):
        idx, val = select(F, rec, dq, dep, uni, n, k)
        check_exact(idx, val, sg, k, where=f"n={n} rising={rising} k={k}")


@pytest.mark.parametrize("n,k", [(50000, 2048), (50000, 20000), (262143, 2048), (262144, 2048), (300000, 2048),
                                 (300000, 30000), (1 << 20, 2048)])
def test_scores_in_a_narrow_band(F, n, k):
    """One dominant channel puts every score within a few percent of the same
    value (one or two first-digit bins of 1/8 octave, so more candidates than
    the resolve holds on chip), while 15 small channels keep them apart.  Short
    rows resolve over the whole row; rows of 262144 keys or more take the
    refinement stage (a second-digit histogram and a second collect), and k =
    30000 keeps more than the resolve holds even then.  Every case selects
    exactly."""
    rng = np.random.default_rng(n + k)
    d = 16
    kk = rng.standard_normal((1, n, d)).astype(np.float32)
    kk[0, :, 0] = 1.0
    q = np.concatenate([[1.0], 0.001 * rng.standard_normal(d - 1)]).astype(np.float32)[None]
    s2 = np.ones((1, d), np.float32)
    rec, _ = gpu_pack(kk)
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), 4 * d)
    sg = F.scan_scores(rec, dq, dep, uni, n).cpu().numpy()
    assert np.ptp(sg[0]) < 0.1 * abs(float(np.median(sg[0])))   # one narrow band
    idx, val = select(F, rec, dq, dep, uni, n, k)
    check_exact(idx, val, sg, k, where=f"narrow band n={n} k={k}")


def test_all_equal_scores_long_row(F):
    """Budget 0 on a row long enough for the refinement stage: every key ties,
    the refined candidates still overflow, and the full-row path takes the
    lowest indices."""
    n = 300000
    kk, q, s2 = small_case(4, 1, 2, n, 16)
    rec, _ = gpu_pack(kk)
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), 0)
    for k in (1, 2048, 20000):
        idx, val = select(F, rec, dq, dep, uni, n, k)
        assert np.array_equal(idx, np.tile(np.arange(k), (2, 1)))
        assert np.all(val == 0)


@pytest.mark.parametrize("n", [16384, 16385])
@pytest.mark.parametrize("residency", ["hbm", "host"])
def test_rows_at_the_one_launch_limit(F, n, residency):
    """Rows of 16384 keys are selected in one launch per head with the row in
    LDS, rows of 16385 by the chunked kernels: both select exactly, k from 1 to
    n."""
    h_kv, g, d, budget = 2, 4, 64, 40
    kk, q, s2 = small_case(n + 3, h_kv, g, n, d, outliers=2)
    rec, st = gpu_pack(kk)
    assert st == 0
    if residency == "host":
        rec = rec.cpu().pin_memory()
    res = F.HBM if residency == "hbm" else F.HOST_DIRECT
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    sg = F.scan_scores(rec, dq, dep, uni, n, residency=res).cpu().numpy()
    for k in (1, 2048, 5000, n):
        idx, val = F.scan_topk(rec, dq, dep, uni, n, k, residency=res, want_scores=True)
        torch.cuda.synchronize()
        check_exact(idx.cpu().numpy(), val.cpu().numpy(), sg, k, where=f"n={n} {residency} k={k}")
