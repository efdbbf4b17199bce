"""GPU parity of paged records (scan_topk_paged): pages at arbitrary places in a
pool, in HBM or pinned host memory, give the same selection as contiguous
records bit for bit, match the oracle, and support a decode loop that takes a
new page when the last one is full."""

import numpy as np
import pytest
import torch

from oracle import fathom_oracle as O
from synthetic import small_case
from tests.parity import check_scores, check_topk, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    from sparse_attention_top_query_amd import fathom
    fathom.load()
    assert torch.cuda.is_available()
    return fathom


def build_pages(F, kk, n_sealed, page_keys, host, seed):
    """Pack the sealed keys page by page into shuffled slots of one pool; return
    (pool, pages[g][p] views, table)."""
    h_kv, _, d = kk.shape
    rp = F.record_bytes(page_keys)
    npages = -(-n_sealed // page_keys)
    slots = np.random.default_rng(seed).permutation(h_kv * npages + 3)   # spare slots too
    if host:
        # one pinned allocation per page (pages from a pinned pool would be
        # addressed the same way; separate allocations keep the test simple)
        pool = []
        for _ in range(len(slots)):
            t = torch.empty((d, rp), dtype=torch.uint8, pin_memory=True)
            t.fill_(0x5A)
            pool.append(t)
    else:
        pool = torch.full((len(slots), d, rp), 0x5A, dtype=torch.uint8, device="cuda:0")
    stage = torch.empty((1, d, rp), dtype=torch.uint8, device="cuda:0")
    pages = []
    for g in range(h_kv):
        row = []
        for p in range(npages):
            view = pool[int(slots[g * npages + p])]
            lo, hi = p * page_keys, min(n_sealed, (p + 1) * page_keys)
            target = stage if host else view[None]
            F.pack_blocks(dev(np.ascontiguousarray(kk[g:g + 1, lo:hi])), target, page_keys, 0)
            if host:
                view.copy_(stage[0])
            row.append(view)
        pages.append(row)
    torch.cuda.synchronize()
    return pool, pages, F.page_table(pages, residency=F.HOST_DIRECT if host else F.HBM)


PAGED_CASES = [  # (h_kv, g, n_sealed, n_tail, page_keys, d, budget, k)
    (2, 4, 3 * 8192 + 1280, 77, 8192, 128, 92, 300),
    (1, 1, 4096, 0, 4096, 128, 64, 50),
    (2, 8, 12288 + 128, 5, 4096, 64, 40, 200),
    (1, 4, 20480, 127, 16384, 128, 68, 2048),
    # more than 2048 tiles of 1024 keys in all: the long-row HBM staging
    (2, 4, (1 << 20) + 4096, 33, 65536, 32, 40, 2048),
]


@pytest.mark.parametrize("case", PAGED_CASES)
@pytest.mark.parametrize("residency", ["hbm", "host"])
def test_paged_equals_contiguous(F, case, residency):
    h_kv, g, n_s, n_t, page_keys, d, budget, k = case
    print(f"paged case={case} residency={residency}", flush=True)
    host = residency == "host"
    kk, q, s2 = small_case(sum(case), h_kv, g, n_s + n_t, d, outliers=min(4, d))
    pool, pages, table = build_pages(F, kk, n_s, page_keys, host, seed=sum(case))
    rec = F.pack(dev(np.ascontiguousarray(kk[:, :n_s])))        # contiguous records of the sealed keys
    if host:
        pinned = torch.empty(rec.shape, dtype=torch.uint8, pin_memory=True)
        pinned.copy_(rec)
        rec = pinned
    tail = dev(np.ascontiguousarray(kk[:, n_s:])) if n_t else None
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    res = F.HOST_DIRECT if host else F.HBM
    a = F.scan_topk_append(rec, n_s, n_s, tail, dq, dep, uni, k, residency=res, want_scores=True)
    b = F.scan_topk_paged(table, page_keys, n_s, tail, dq, dep, uni, k, residency=res, want_scores=True)
    torch.cuda.synchronize()
    assert np.array_equal(a[0].cpu().numpy(), b[0].cpu().numpy())
    assert np.array_equal(a[1].cpu().numpy().view(np.uint32), b[1].cpu().numpy().view(np.uint32))
    # the pages themselves are the oracle's records of each page's keys
    for p, view in enumerate(pages[0]):
        keys = kk[0, p * page_keys:min(n_s, (p + 1) * page_keys)]
        if keys.shape[0] == page_keys:
            want = O.pack_head(np.ascontiguousarray(keys))[2]
            got = view.cpu().numpy() if not host else view.numpy()
            assert np.array_equal(got, want), f"page {p}"


def test_paged_matches_oracle(F):
    h_kv, g, n_s, n_t, page_keys, d, budget, k = PAGED_CASES[0]
    kk, q, s2 = small_case(7, h_kv, g, n_s + n_t, d, outliers=4)
    pool, pages, table = build_pages(F, kk, n_s, page_keys, True, seed=3)
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    tail = np.ascontiguousarray(kk[:, n_s:])
    idx, sc = F.scan_topk_paged(table, page_keys, n_s, dev(tail), dq, dep, uni, k, want_scores=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    ref = O.step_append(np.ascontiguousarray(kk[:, :n_s]), tail, q, s2, budget, k)
    for h in range(h_kv * g):
        check_topk(idx[h], ref["scores"][h], ref["sums"][h], k, where=f"head {h}")
        check_scores(sc[h], ref["scores"][h][idx[h]], ref["sums"][h][idx[h]], where=f"head {h}")


def test_paged_decode_loop_takes_pages_on_demand(F):
    h_kv, g, d, budget, k, page_keys = 2, 4, 128, 92, 128, 4096
    n_final = 3 * page_keys + 900
    kk, q, s2 = small_case(91, h_kv, g, n_final, d, outliers=4)
    rp = F.record_bytes(page_keys)
    pool = torch.full((8, d, rp), 0x33, dtype=torch.uint8, device="cuda:0")
    free = [5, 2, 7, 0, 3, 6, 1, 4]                  # pages come from the pool in this order
    pages = [[] for _ in range(h_kv)]
    dq = dev(q)
    dep, uni = F.allocate(dq, dev(s2), budget)
    n, sealed = 0, 0
    for step_no, grow in enumerate((1000, 3000, 200, 4096, 1, 3000, 900, 1000)):
        n = min(n_final, n + grow)
        new_sealed = n // 128 * 128
        while sealed < new_sealed:
            p = sealed // page_keys
            if p == len(pages[0]):
                for gg in range(h_kv):
                    pages[gg].append(pool[free.pop(0)])
            hi = min(new_sealed, (p + 1) * page_keys)
            for gg in range(h_kv):
                F.pack_blocks(dev(np.ascontiguousarray(kk[gg:gg + 1, sealed:hi])), pages[gg][p][None], page_keys,
                              (sealed - p * page_keys) // 128)
            sealed = hi
        tail = np.ascontiguousarray(kk[:, sealed:n])
        table = F.page_table(pages) if pages[0] else None
        idx = F.scan_topk_paged(table, page_keys, sealed, dev(tail) if n > sealed else None, dq, dep, uni, k,
                                residency=F.HBM)
        torch.cuda.synchronize()
        idx = idx.cpu().numpy()
        ref = O.step_append(np.ascontiguousarray(kk[:, :sealed]), tail, q, s2, budget, k)
        print(f"paged decode step {step_no}: n={n} sealed={sealed} pages={len(pages[0])}", flush=True)
        for h in range(h_kv * g):
            check_topk(idx[h], ref["scores"][h], ref["sums"][h], k, where=f"step {step_no} head {h}")
