"""GPU parity of the free path (the scan over the token-major 4-bit copy):
pack_nibbles is bit-exact against the oracle's layout, and scan_topk_nibbles
gives the bit-plane scan's scores and selection bit for bit (and so the
oracle's), from HBM and from pinned host memory."""

import zlib

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


@pytest.mark.parametrize("shape", [(2, 1000, 128), (1, 4096, 64), (3, 300, 32), (1, 129, 96)])
def test_pack_nibbles_bit_exact(F, shape):
    h_kv, n, d = shape
    k, _, _ = small_case(zlib.crc32(repr(shape).encode()) % 50, h_kv, 1, n, d, outliers=min(4, d))
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    codes, scales = F.pack_nibbles(dev(k), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for g in range(h_kv):
        delta = O.block_scales(k[g])
        kappa = O.quantize_codes(k[g], delta)
        want_c, want_s = O.pack_nibbles(kappa, delta)
        assert np.array_equal(codes[g].cpu().numpy(), want_c)
        assert np.array_equal(scales[g].cpu().numpy().view(np.uint8).reshape(want_s.shape), want_s)


def test_pack_nibbles_flags(F):
    k, _, _ = small_case(3, 1, 1, 300, 64)
    k[0, 7, 5] = np.nan
    st = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    F.pack_nibbles(dev(k), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 1


FREE_CASES = [  # (h_kv, g, n, d, budget, k)
    (2, 4, 3 * 1024 + 300, 128, 92, 200),
    (1, 1, 4096, 128, 64, 64),
    (3, 8, 2000, 64, 40, 100),
    (1, 16, 1500, 128, 300, 1500),        # k = n: every score compared
    (2, 2, 777, 32, 0, 50),               # budget 0
]


@pytest.mark.parametrize("case", FREE_CASES)
@pytest.mark.parametrize("residency", ["hbm", "host"])
def test_free_path_equals_bit_plane_scan(F, case, residency):
    h_kv, g, n, d, budget, k = case
    print(f"free path case={case} residency={residency}", flush=True)
    kk, q, s2 = small_case(sum(case), h_kv, g, n, d, outliers=min(4, d))
    dk = dev(kk)
    rec = F.pack(dk)
    codes, scales = F.pack_nibbles(dk)
    if residency == "host":
        pc = torch.empty(codes.shape, dtype=torch.uint8, pin_memory=True)
        pc.copy_(codes)
        ps = torch.empty(scales.shape, dtype=torch.float16, pin_memory=True)
        ps.copy_(scales)
        codes, scales = pc, ps
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    a = F.scan_topk(rec, dq, dep, uni, n, k, residency=F.HBM, want_scores=True)
    b = F.scan_topk_nibbles(codes, scales, dq, dep, uni, k, want_scores=True)
    torch.cuda.synchronize()
    assert np.array_equal(a[0].cpu().numpy(), b[0].cpu().numpy())
    assert np.array_equal(a[1].cpu().numpy().view(np.uint32), b[1].cpu().numpy().view(np.uint32))


def test_free_path_matches_oracle(F):
    h_kv, g, n, d, budget, k = FREE_CASES[0]
    kk, q, s2 = small_case(9, h_kv, g, n, d, outliers=4)
    codes, scales = F.pack_nibbles(dev(kk))
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    idx, sc = F.scan_topk_nibbles(codes, scales, dq, dep, uni, k, want_scores=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    rd, _ = oracle_depths(q, s2, budget)
    for h in range(h_kv * g):
        delta = O.block_scales(kk[h // g])
        kappa = O.quantize_codes(kk[h // g], delta)
        s, a = O.scores(q[h], kappa, delta, rd[h])
        check_topk(idx[h], s, a, k, where=f"head {h}")
        check_scores(sc[h], s[idx[h]], a[idx[h]], where=f"head {h}")


def test_free_path_rejects_unsupported_d(F):
    kk, q, s2 = small_case(1, 1, 1, 256, 100)
    with pytest.raises(F.FathomError):
        F.pack_nibbles(dev(kk))
