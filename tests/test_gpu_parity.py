"""GPU parity of every stage against the oracle, at small and medium shapes
(several 1024-key tiles plus ragged tails) and at the method's edge cases.
Calls go through the C ABI (libfathom.so) via the thin ctypes binding."""

import zlib

import numpy as np
import pytest
import torch

from oracle import fathom_oracle as O
from synthetic import small_case
from tests.parity import check_scores, check_topk, dev, gpu_pack, oracle_depths, oracle_pack

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    from sparse_attention_top_query_amd import fathom
    fathom.load()
    assert torch.cuda.is_available()
    return fathom


# ---------------------------------------------------------------- pack ----

def crafted():
    from tests.test_oracle_quant import crafted_keys
    return crafted_keys()[None]


@pytest.mark.parametrize("shape", [(1, 1, 7), (1, 128, 256), (1, 129, 64), (3, 4096 + 37, 128),
                                   (2, 3000, 5)])
def test_pack_bit_exact(F, shape):
    h_kv, n, d = shape
    print(f"pack shape={shape}", flush=True)
    k, _, _ = small_case(zlib.crc32(repr(shape).encode()) % 97, h_kv, 1, n, d, outliers=min(4, d))
    rec, st = gpu_pack(k)
    assert st == 0
    ref = np.stack([r for _, _, r in oracle_pack(k)])
    assert np.array_equal(rec.cpu().numpy(), ref)


def test_pack_crafted_thresholds_and_subnormals(F):
    k = crafted()
    # fp32 subnormal keys next to the zero threshold of a block with Delta = 1
    k[0, 20, 0] = np.float32(-1e-40)
    k[0, 21, 0] = np.float32(1e-40)
    rec, st = gpu_pack(k)
    assert st == 0
    _, kappa, ref = O.pack_head(k[0])
    assert kappa[20, 0] == 7 and kappa[21, 0] == 8
    assert np.array_equal(rec.cpu().numpy()[0], ref)


def test_pack_status_flags(F):
    k = np.zeros((2, 256, 4), np.float32)
    _, st = gpu_pack(k)
    assert st == 0
    k[1, 200, 3] = np.nan
    _, st = gpu_pack(k)
    assert st & F.FLAG_KEY_NONFINITE
    k[1, 200, 3] = np.float32(1e6)
    _, st = gpu_pack(k)
    assert st == F.FLAG_SCALE_OVERFLOW
    k[1, 200, 3] = np.inf
    _, st = gpu_pack(k)
    assert st & F.FLAG_KEY_NONFINITE


def test_pack_empty_is_noop(F):
    k = torch.zeros((1, 0, 8), dtype=torch.float32, device="cuda:0")
    rec = F.pack(k)
    assert rec.numel() == 0


# ------------------------------------------------------------ allocate ----

ALLOC_SHAPES = [(8, 4, 128), (2, 16, 256), (3, 1, 5), (1, 2, 64), (2, 8, 100)]


@pytest.mark.parametrize("shape", ALLOC_SHAPES)
@pytest.mark.parametrize("budget_frac", [0.0, 0.09, 0.18, 0.36, 0.5, 1.0])
def test_allocate_waterfill_bit_exact(F, shape, budget_frac):
    h_kv, g, d = shape
    budget = int(round(budget_frac * 4 * d))
    _, q, s2 = small_case(7, h_kv, g, 1, d, outliers=min(4, d))
    dep, uni = F.allocate(dev(q), dev(s2), budget)
    rd, ru = oracle_depths(q, s2, budget)
    assert np.array_equal(dep.cpu().numpy(), rd)
    assert np.array_equal(uni.cpu().numpy(), ru)


@pytest.mark.parametrize("budget", [46, 68, 92])
def test_allocate_qwen_shape_budgets(F, budget):
    for seed in range(5):
        _, q, s2 = small_case(100 + seed, 8, 4, 1, 128, outliers=4)
        dep, uni = F.allocate(dev(q), dev(s2), budget)
        rd, ru = oracle_depths(q, s2, budget)
        assert np.array_equal(dep.cpu().numpy(), rd)
        assert np.array_equal(uni.cpu().numpy(), ru)
        assert np.all(dep.cpu().numpy().sum(axis=1) == budget)


def test_allocate_ties_zeros_and_subnormals(F):
    d = 128
    q = np.zeros((4, d), np.float32)
    q[0] = 0.0                                   # all-zero importance: fill lowest channels
    q[1, ::3] = np.float32(0.5)                  # many exact ties
    q[1, 1::3] = np.float32(-0.5)
    q[2] = np.float32(1e-20)                     # q^2 underflows to a subnormal / zero
    q[2, ::5] = np.float32(3e-20)
    q[3] = np.random.default_rng(3).standard_normal(d).astype(np.float32)
    s2 = np.ones((1, d), np.float32)
    s2[0, 10:20] = 0.0
    s2[0, 40:50] = np.float32(4.0)
    for budget in (0, 1, 5, 46, 92, 257, 511, 512):
        dep, uni = F.allocate(dev(q), dev(s2), budget)
        rd, ru = oracle_depths(q, s2, budget)
        assert np.array_equal(dep.cpu().numpy(), rd), budget
        assert np.array_equal(uni.cpu().numpy(), ru), budget


@pytest.mark.parametrize("budget", [0, 68, 136, 512])
def test_allocate_topq_bit_exact(F, budget):
    _, q, s2 = small_case(11, 8, 4, 1, 128, outliers=4)
    q[0, ::4] = np.float32(0.75)                 # |q| ties, resolved by lowest channel
    q[0, 2::4] = np.float32(-0.75)
    dep, uni = F.allocate(dev(q), dev(s2), budget, mode=F.TOPQ)
    rd, ru = oracle_depths(q, s2, budget, mode="topq")
    assert np.array_equal(dep.cpu().numpy(), rd)
    assert np.array_equal(uni.cpu().numpy(), ru)


@pytest.mark.parametrize("budget", [0, 68, 136, 512])
def test_allocate_static_bit_exact(F, budget):
    _, q, s2 = small_case(19, 8, 4, 1, 128, outliers=4)
    s2[1, ::5] = np.float32(2.0)                 # variance ties, resolved by lowest channel
    s2[2, :40] = 0.0
    s2[2, :40:2] = np.float32(-0.0)              # -0 ranks as 0, not by its bit pattern
    dep, uni = F.allocate(dev(q), dev(s2), budget, mode=F.STATIC)
    rd, ru = oracle_depths(q, s2, budget, mode="static")
    assert np.array_equal(dep.cpu().numpy(), rd)
    assert np.array_equal(uni.cpu().numpy(), ru)


def test_allocate_status_flags(F):
    _, q, s2 = small_case(12, 3, 2, 1, 32)
    q[1, 5] = np.nan          # KV head 0, query head 1
    s2[1, 7] = -1.0           # KV head 1
    q[5, 2] = np.float32(1e20)  # KV head 2: q^2 overflows
    st = torch.full((3,), -1, dtype=torch.int32, device="cuda:0")
    dep, uni = F.allocate(dev(q), dev(s2), 40, status=st)
    st = st.cpu().numpy()
    assert st[0] == 4 and st[1] == 8 and st[2] == 16
    dep = dep.cpu().numpy()
    assert np.all(dep[1] == 0) and np.all(dep[2] == 0) and np.all(dep[3] == 0) and np.all(dep[5] == 0)
    assert dep[0].sum() == 40 and dep[4].sum() == 40


@pytest.mark.parametrize("shape", ALLOC_SHAPES)
@pytest.mark.parametrize("budget_frac", [0.0, 0.09, 0.18, 0.5, 1.0])
def test_allocate_group_shared_bit_exact(F, shape, budget_frac):
    h_kv, g, d = shape
    budget = int(round(budget_frac * 4 * d))
    _, q, s2 = small_case(17, h_kv, g, 1, d, outliers=min(4, d))
    dep, uni = F.allocate(dev(q), dev(s2), budget, mode=F.WATERFILL_GROUP)
    rd, ru = oracle_depths(q, s2, budget, mode="group")
    dep, uni = dep.cpu().numpy(), uni.cpu().numpy()
    assert np.array_equal(dep, rd)
    assert np.array_equal(uni, ru)
    for v in range(h_kv):   # one shared vector per group, exactly B bits
        assert np.all(dep[v * g:(v + 1) * g] == uni[v])
        assert int(uni[v].sum()) == budget


def test_allocate_group_status_zeroes_the_group(F):
    _, q, s2 = small_case(18, 2, 4, 1, 64)
    q[6, 3] = np.inf           # KV head 1, query head 2
    st = torch.full((2,), -1, dtype=torch.int32, device="cuda:0")
    dep, uni = F.allocate(dev(q), dev(s2), 50, mode=F.WATERFILL_GROUP, status=st)
    assert list(st.cpu().numpy()) == [0, 4]
    dep = dep.cpu().numpy()
    assert np.all(dep[4:] == 0) and np.all(dep[:4].sum(axis=1) == 50)


def test_allocate_rejects_bad_budget(F):
    _, q, s2 = small_case(13, 1, 4, 1, 16)
    with pytest.raises(F.FathomError):
        F.allocate(dev(q), dev(s2), 65)
    with pytest.raises(F.FathomError):
        F.allocate(dev(q), dev(s2), 6, mode=F.TOPQ)


# ---------------------------------------------------------------- scan ----

SCAN_CASES = [
    # (h_kv, g, n, d, budget)
    (2, 4, 3 * 1024 + 300, 128, 92),
    (1, 1, 4096, 128, 64),
    (3, 8, 2048 + 5, 64, 40),
    (1, 16, 1500, 256, 1024),
    (2, 2, 777, 100, 0),
    (1, 4, 9 * 1024, 128, 46),
]


def run_case(F, case, residency="hbm", mode="waterfill"):
    h_kv, g, n, d, budget = case
    print(f"scan case={case} residency={residency} mode={mode}", flush=True)
    k, q, s2 = small_case(sum(case), h_kv, g, n, d, outliers=min(4, d))
    rec, st = gpu_pack(k)
    assert st == 0
    if residency == "host":
        rec = rec.cpu().pin_memory()
    dq = dev(q)
    modes = {"waterfill": F.WATERFILL, "topq": F.TOPQ, "group": F.WATERFILL_GROUP, "static": F.STATIC}
    dep, uni = F.allocate(dq, dev(s2), budget, mode=modes[mode])
    scores = F.scan_scores(rec, dq, dep, uni, n)
    torch.cuda.synchronize()
    return k, q, s2, rec, dq, dep, uni, scores.cpu().numpy()


@pytest.mark.parametrize("case", SCAN_CASES)
def test_scan_scores_within_tolerance(F, case):
    h_kv, g, n, d, budget = case
    k, q, s2, rec, dq, dep, uni, sg = run_case(F, case)
    packed = oracle_pack(k)
    rd, _ = oracle_depths(q, s2, budget)
    assert np.array_equal(dep.cpu().numpy(), rd)
    worst = 0.0
    for h in range(h_kv * g):
        delta, kappa, _ = packed[h // g]
        s, a = O.scores(q[h], kappa, delta, rd[h])
        worst = max(worst, check_scores(sg[h], s, a, where=f"head {h}"))
    print(f"worst |err|/A = {worst:.2e}")


@pytest.mark.parametrize("case", SCAN_CASES)
def test_topk_parity(F, case):
    h_kv, g, n, d, budget = case
    k, q, s2, rec, dq, dep, uni, sg = run_case(F, case)
    packed = oracle_pack(k)
    rd, _ = oracle_depths(q, s2, budget)
    ref = []
    for h in range(h_kv * g):
        delta, kappa, _ = packed[h // g]
        ref.append(O.scores(q[h], kappa, delta, rd[h]))
    for kk in sorted({1, min(64, n), n // 3, n}):
        idx, val = F.scan_topk(rec, dq, dep, uni, n, kk, want_scores=True)
        idx, val = idx.cpu().numpy(), val.cpu().numpy()
        for h in range(h_kv * g):
            s, a = ref[h]
            check_topk(idx[h], s, a, kk, s_gpu=sg[h], where=f"k={kk} head {h}")
            assert np.array_equal(val[h], sg[h][idx[h]])


def test_budget_zero_selects_lowest_indices(F):
    case = (2, 2, 5000, 32, 0)
    *_, rec, dq, dep, uni, sg = run_case(F, case)
    assert np.all(sg == 0)
    idx = F.scan_topk(rec, dq, dep, uni, 5000, 100).cpu().numpy()
    assert np.array_equal(idx, np.tile(np.arange(100), (4, 1)))


def test_empty_rows_and_selections(F):
    """n = 0 keys and k = 0 selections succeed and write nothing."""
    case = (1, 2, 700, 16, 20)
    *_, rec, dq, dep, uni, sg = run_case(F, case)
    out = torch.full((2, 64), 7.0, device="cuda:0")
    assert F.scan_scores(rec, dq, dep, uni, 0, out=out).shape == (2, 0)
    idx = torch.full((2, 8), -3, dtype=torch.int32, device="cuda:0")
    for n in (700, 0):
        F.scan_topk(rec, dq, dep, uni, n, 0, idx=idx)
        F.scan_topk(rec.cpu().pin_memory(), dq, dep, uni, n, 0, idx=idx)
        F.scan_topk_noalloc(rec, dq, dep, uni, n, 0, idx=idx)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(idx == -3)


def test_budget_zero_large_n_takes_row_fallback(F):
    """All scores equal (B = 0): every key is a candidate, more than the LDS sort
    holds, so selection runs the exact in-order fallback; lowest indices win."""
    case = (1, 4, 40000, 16, 0)
    *_, rec, dq, dep, uni, sg = run_case(F, case)
    for kk in (1, 2048, 9000, 40000):
        idx = F.scan_topk(rec, dq, dep, uni, 40000, kk).cpu().numpy()
        assert np.array_equal(idx, np.tile(np.arange(kk), (4, 1))), kk


def test_select_many_ties(F):
    """Exact selection among massive score ties (a one-channel cache whose keys take
    three values), across several select chunks."""
    n = 3 * 4096 + 11
    k = np.zeros((1, n, 1), np.float32)
    k[0, ::2, 0] = 1.0          # block max 1 -> codes alternate between 8 (k = 0) and 15 (k = 1)
    k[0, 1::4, 0] = -1.0
    q = np.array([[1.0]], np.float32)
    s2 = np.ones((1, 1), np.float32)
    rec, _ = gpu_pack(k)
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), 4)
    sg = F.scan_scores(rec, dq, dep, uni, n).cpu().numpy()
    _, kappa, _ = O.pack_head(k[0])
    delta = O.block_scales(k[0])
    s, a = O.scores(q[0], kappa, delta, np.array([4]))
    check_scores(sg[0], s, a)
    for kk in (1, 100, n // 2, n - 1, n):
        idx = F.scan_topk(rec, dq, dep, uni, n, kk).cpu().numpy()[0]
        assert np.array_equal(idx, O.topk(s, kk))


@pytest.mark.parametrize("case", [SCAN_CASES[0], SCAN_CASES[2], SCAN_CASES[3], SCAN_CASES[5]])
def test_host_residencies_match_hbm_bit_for_bit(F, case):
    """The same scan over pinned host records, read in place or staged through
    HBM, gives bit-identical scores and indices to the HBM-resident scan."""
    h_kv, g, n, d, budget = case
    k, q, s2, rec, dq, dep, uni, sg = run_case(F, case)
    host = rec.cpu().pin_memory()
    for res in (F.HOST_DIRECT, F.HOST_STAGED):
        sh = F.scan_scores(host, dq, dep, uni, n, residency=res).cpu().numpy()
        assert np.array_equal(sh.view(np.uint32), sg.view(np.uint32)), res
    a = F.scan_topk(rec, dq, dep, uni, n, 64).cpu().numpy()
    for res in (F.HOST_DIRECT, F.HOST_STAGED):
        b = F.scan_topk(host, dq, dep, uni, n, 64, residency=res).cpu().numpy()
        assert np.array_equal(a, b), res


@pytest.mark.parametrize("case", [(2, 4, 3 * 1024 + 300, 128, 92), (1, 1, 4096, 128, 64), (3, 2, 9000, 64, 40),
                                  (1, 8, 5000, 128, 100), (2, 4, 2048, 128, 0), (1, 4, 300, 16, 20)])
def test_host_direct_topk_equals_hbm(F, case):
    # host-direct scans build the selection's histogram inside the scan where it
    # fits (G <= 4); the selection must come out exactly as from HBM records
    h_kv, g, n, d, budget = case
    k_np, q, s2, rec, dq, dep, uni, sg = run_case(F, case)
    k = min(n, 333)
    ih, sh = F.scan_topk(rec, dq, dep, uni, n, k, residency=F.HBM, want_scores=True)
    host = rec.cpu().pin_memory()
    idd, sd = F.scan_topk(host, dq, dep, uni, n, k, residency=F.HOST_DIRECT, want_scores=True)
    torch.cuda.synchronize()
    assert np.array_equal(ih.cpu().numpy(), idd.cpu().numpy())
    assert np.array_equal(sh.cpu().numpy().view(np.uint32), sd.cpu().numpy().view(np.uint32))
    for h in range(h_kv * g):
        assert np.array_equal(idd.cpu().numpy()[h], O.topk(sg[h].astype(np.float64), k))


def test_staged_ring_of_many_heads(F):
    """13 KV heads of ~10 MB of records each staged through the ring of two KV
    heads' slots (every slot reused six or seven times, odd head count): staged
    must still equal HBM-resident, bit for bit."""
    case = (13, 4, 160000, 128, 68)
    h_kv, g, n, d, budget = case
    k, q, s2, rec, dq, dep, uni, sg = run_case(F, case)
    host = rec.cpu().pin_memory()
    sh = F.scan_scores(host, dq, dep, uni, n, residency=F.HOST_STAGED).cpu().numpy()
    assert np.array_equal(sh.view(np.uint32), sg.view(np.uint32))


@pytest.mark.parametrize("case", [(2, 2, 1_100_001, 32, 40), (1, 8, 2_200_000, 16, 24)])
def test_long_hbm_rows_match_oracle_and_host(F, case):
    """HBM rows of more than 2048 tiles in all (2 and 8 query heads per KV head,
    where such rows stage 32 channel-planes per group instead of 64): scores
    of the first and last query head within the tolerance of the oracle over
    the whole row, selection exact, and scores and selection bit-identical to
    the same records read in place from pinned host memory."""
    h_kv, g, n, d, budget = case
    k, q, s2, rec, dq, dep, uni, sg = run_case(F, case)
    host = rec.cpu().pin_memory()
    sh = F.scan_scores(host, dq, dep, uni, n, residency=F.HOST_DIRECT).cpu().numpy()
    assert np.array_equal(sh.view(np.uint32), sg.view(np.uint32))
    idx = F.scan_topk(rec, dq, dep, uni, n, 2048).cpu().numpy()
    assert np.array_equal(F.scan_topk(host, dq, dep, uni, n, 2048).cpu().numpy(), idx)
    rd, _ = oracle_depths(q, s2, budget)
    for h in (0, h_kv * g - 1):
        delta, kappa, _ = O.pack_head(k[h // g])
        s, a = O.scores(q[h], kappa, delta, rd[h])
        check_scores(sg[h], s, a, where=f"head {h}")
        check_topk(idx[h], s, a, 2048, s_gpu=sg[h], where=f"head {h}")


def test_topq_scan_parity(F):
    case = (2, 4, 4096, 128, 68)
    k, q, s2, rec, dq, dep, uni, sg = run_case(F, case, mode="topq")
    packed = oracle_pack(k)
    rd, _ = oracle_depths(q, s2, 68, mode="topq")
    assert np.array_equal(dep.cpu().numpy(), rd)
    idx = F.scan_topk(rec, dq, dep, uni, 4096, 256).cpu().numpy()
    for h in range(8):
        delta, kappa, _ = packed[h // 4]
        s, a = O.scores(q[h], kappa, delta, rd[h])
        check_scores(sg[h], s, a)
        check_topk(idx[h], s, a, 256, s_gpu=sg[h])


def test_group_shared_scan_parity(F):
    case = (2, 4, 5000, 128, 92)
    k, q, s2, rec, dq, dep, uni, sg = run_case(F, case, mode="group")
    packed = oracle_pack(k)
    rd, _ = oracle_depths(q, s2, 92, mode="group")
    assert np.array_equal(dep.cpu().numpy(), rd)
    idx = F.scan_topk(rec, dq, dep, uni, 5000, 300).cpu().numpy()
    for h in range(8):
        delta, kappa, _ = packed[h // 4]
        s, a = O.scores(q[h], kappa, delta, rd[h])
        check_scores(sg[h], s, a)
        check_topk(idx[h], s, a, 300, s_gpu=sg[h])


def test_static_scan_parity(F):
    case = (2, 4, 4096, 128, 136)
    k, q, s2, rec, dq, dep, uni, sg = run_case(F, case, mode="static")
    packed = oracle_pack(k)
    rd, _ = oracle_depths(q, s2, 136, mode="static")
    assert np.array_equal(dep.cpu().numpy(), rd)
    idx = F.scan_topk(rec, dq, dep, uni, 4096, 256).cpu().numpy()
    for h in range(8):
        delta, kappa, _ = packed[h // 4]
        s, a = O.scores(q[h], kappa, delta, rd[h])
        check_scores(sg[h], s, a)
        check_topk(idx[h], s, a, 256, s_gpu=sg[h])


def test_scan_rejects_bad_residency_and_workspace(F):
    case = (1, 4, 1024, 32, 20)
    *_, rec, dq, dep, uni, sg = run_case(F, case)
    for res in (F.HOST_DIRECT, F.HOST_STAGED):
        with pytest.raises(F.FathomError) as e:
            F.scan_topk(rec, dq, dep, uni, 1024, 8, residency=res)
        assert e.value.status == -7
        pageable = rec.cpu()
        with pytest.raises(F.FathomError) as e:
            F.scan_topk(pageable, dq, dep, uni, 1024, 8, residency=res)
        assert e.value.status == -7
    host = rec.cpu().pin_memory()
    small = torch.empty(1024, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(F.FathomError) as e:       # no room for the staging ring
        F.scan_scores(host, dq, dep, uni, 1024, residency=F.HOST_STAGED, workspace=small)
    assert e.value.status == -5
    small = torch.empty(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(F.FathomError) as e:
        F.scan_topk(rec, dq, dep, uni, 1024, 8, workspace=small)
    assert e.value.status == -5
    with pytest.raises(F.FathomError):
        F.scan_topk(rec, dq, dep, uni, 1024, 1025)


def test_repeat_runs_are_deterministic(F):
    case = SCAN_CASES[0]
    h_kv, g, n, d, budget = case
    *_, rec, dq, dep, uni, sg = run_case(F, case)
    runs = [F.scan_topk(rec, dq, dep, uni, n, 500, want_scores=True) for _ in range(3)]
    for i, v in runs[1:]:
        assert torch.equal(i, runs[0][0]) and torch.equal(v, runs[0][1])
