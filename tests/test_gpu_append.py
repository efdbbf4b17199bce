"""GPU parity of the appending path (pack_blocks, scan_topk_append) against the
oracle, through the C ABI: piecewise sealing equals packing the whole cache,
the scan of sealed blocks plus the exact open tail matches step_append, and a
small decode loop that appends keys and seals blocks as they fill."""

import numpy as np
import pytest
import torch

from oracle import fathom_oracle as O
from synthetic import small_case
from tests.parity import check_scores, check_topk, dev, oracle_depths

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    from sparse_attention_top_query_amd import fathom
    fathom.load()
    assert torch.cuda.is_available()
    return fathom


def block_bytes(rec, n_cap, b):
    """(scale bytes, plane-0 bytes, planes 1..3 bytes) of block b in one record."""
    U, H, P, R = O.record_layout(n_cap)
    unit, w = divmod(b, O.UNIT_BLOCKS)
    base = 144 * unit
    sc = rec[base + 2 * w: base + 2 * w + 2]
    p0 = rec[base + 16 + 16 * w: base + 32 + 16 * w]
    rest = [rec[H + (p - 1) * P + 16 * b: H + (p - 1) * P + 16 * b + 16] for p in (1, 2, 3)]
    return sc, p0, rest


def empty_records(F, h_kv, d, n_cap, fill=0xAB):
    return torch.full((h_kv, d, F.record_bytes(n_cap)), fill, dtype=torch.uint8, device="cuda:0")


def test_piecewise_sealing_equals_whole_pack(F):
    h_kv, n_cap, d = 2, 5000, 64          # 40 blocks, the last one 8 keys long
    k, _, _ = small_case(41, h_kv, 1, n_cap, d, outliers=4)
    want = np.stack([O.pack_head(k[g])[2] for g in range(h_kv)])
    rec = empty_records(F, h_kv, d, n_cap)
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    sealed = 0
    for nbl in (3, 1, 6, 30):
        rows = min(128 * nbl, n_cap - 128 * sealed)
        F.pack_blocks(dev(np.ascontiguousarray(k[:, 128 * sealed:128 * sealed + rows])), rec, n_cap, sealed, status=st)
        sealed += nbl
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        got = rec.cpu().numpy()
        for g in range(h_kv):
            for c in (0, 17, d - 1):
                for b in range(sealed):
                    a, bb = block_bytes(got[g, c], n_cap, b), block_bytes(want[g, c], n_cap, b)
                    assert np.array_equal(a[0], bb[0]) and np.array_equal(a[1], bb[1]), (g, c, b)
                    assert all(np.array_equal(x, y) for x, y in zip(a[2], bb[2])), (g, c, b)
    assert sealed == 40
    assert np.array_equal(rec.cpu().numpy(), want)   # padding included once the last block is sealed


APPEND_CASES = [  # (h_kv, g, n_cap, n_sealed, n_tail, d, budget, k)
    (2, 4, 8192, 4480, 77, 128, 92, 300),
    (1, 1, 4096, 0, 100, 128, 64, 20),        # all tail
    (1, 4, 3000, 2944, 0, 64, 40, 100),       # no tail
    (2, 2, 3000, 3000, 5, 128, 68, 64),       # full ragged capacity plus a tail
    (1, 8, 2048, 1024, 127, 256, 200, 1151),  # k = every key
]


@pytest.mark.parametrize("case", APPEND_CASES)
@pytest.mark.parametrize("residency", ["hbm", "host"])
def test_scan_topk_append_matches_oracle(F, case, residency):
    h_kv, g, n_cap, n_s, n_t, d, budget, k = case
    print(f"append case={case} residency={residency}", flush=True)
    kk, q, s2 = small_case(sum(case), h_kv, g, n_cap, d, outliers=min(4, d))
    rec = empty_records(F, h_kv, d, n_cap)
    if n_s > 0:
        F.pack_blocks(dev(np.ascontiguousarray(kk[:, :n_s])), rec, n_cap, 0)
    if residency == "host":
        pinned = torch.empty(rec.shape, dtype=torch.uint8, pin_memory=True)
        pinned.copy_(rec)
        rec = pinned
    tail = np.ascontiguousarray(kk[:, n_s:n_s + n_t])
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    idx, sc = F.scan_topk_append(rec, n_cap, n_s, dev(tail) if n_t else None, dq, dep, uni, k,
                                 residency=F.HBM if residency == "hbm" else F.HOST_DIRECT, want_scores=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    ref = O.step_append(np.ascontiguousarray(kk[:, :n_s]), tail, q, s2, budget, k)
    if n_s:
        rd, _ = oracle_depths(q, s2, budget)
        assert np.array_equal(dep.cpu().numpy(), rd)
    for h in range(h_kv * g):
        s_or, a_or = ref["scores"][h], ref["sums"][h]
        check_topk(idx[h], s_or, a_or, k, where=f"head {h}")
        check_scores(sc[h], s_or[idx[h]], a_or[idx[h]], where=f"head {h} selected scores")


def test_decode_loop_appends_and_seals(F):
    # keys arrive a few at a time; whole blocks are sealed as they fill, the rest
    # stays in the exact tail; every step's top-k matches the oracle
    h_kv, g, d, budget, k, n_cap = 2, 4, 128, 92, 96, 2048
    kk, q, s2 = small_case(55, h_kv, g, n_cap, d, outliers=4)
    rec = empty_records(F, h_kv, d, n_cap)
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    n, sealed = 1000, 0
    for step_no, grow in enumerate((0, 1, 23, 5, 128, 77, 200, 1, 300)):
        n += grow
        new_sealed = n // 128 * 128
        if new_sealed > sealed:
            F.pack_blocks(dev(np.ascontiguousarray(kk[:, sealed:new_sealed])), rec, n_cap, sealed // 128)
            sealed = new_sealed
        tail = np.ascontiguousarray(kk[:, sealed:n])
        idx = F.scan_topk_append(rec, n_cap, sealed, dev(tail) if n > sealed else None, dq, dep, uni, k)
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        ref = O.step_append(np.ascontiguousarray(kk[:, :sealed]), tail, q, s2, budget, k)
        print(f"decode step {step_no}: n={n} sealed={sealed}", flush=True)
        for h in range(h_kv * g):
            check_topk(idx[h], ref["scores"][h], ref["sums"][h], k, where=f"step {step_no} head {h}")


@pytest.mark.parametrize("case", APPEND_CASES)
def test_append_host_direct_equals_hbm(F, case):
    # the host-direct path counts scan and tail scores into the selection's
    # histograms inside its kernels (G <= 4); the selection must equal HBM's
    h_kv, g, n_cap, n_s, n_t, d, budget, k = case
    kk, q, s2 = small_case(sum(case) + 1, h_kv, g, n_cap, d, outliers=min(4, d))
    rec = empty_records(F, h_kv, d, n_cap)
    if n_s > 0:
        F.pack_blocks(dev(np.ascontiguousarray(kk[:, :n_s])), rec, n_cap, 0)
    pinned = torch.empty(rec.shape, dtype=torch.uint8, pin_memory=True)
    pinned.copy_(rec)
    tail = dev(np.ascontiguousarray(kk[:, n_s:n_s + n_t])) if n_t else None
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    a = F.scan_topk_append(rec, n_cap, n_s, tail, dq, dep, uni, k, residency=F.HBM, want_scores=True)
    b = F.scan_topk_append(pinned, n_cap, n_s, tail, dq, dep, uni, k, residency=F.HOST_DIRECT, want_scores=True)
    torch.cuda.synchronize()
    assert np.array_equal(a[0].cpu().numpy(), b[0].cpu().numpy())
    assert np.array_equal(a[1].cpu().numpy().view(np.uint32), b[1].cpu().numpy().view(np.uint32))
