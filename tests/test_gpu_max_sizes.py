"""The size limits the C ABI accepts, run on the GPU: 2^30 keys in one row
(with a ragged tail), 2^33 (KV head, key) pairs in one call, and 65535 query
heads in one call.

Keys come from a seeded device generator (the oracle gets the exact values it
checks, copied back).  At these sizes the oracle checks samples:
  * depths and union depths: whole, bit-exact;
  * records: every channel of sampled 128-key blocks (the first, the last and
    random ones), bit-exact against the oracle's quantisation;
  * scores: every key of those blocks and of the blocks holding the selected
    keys, within 1e-4 * sum|q k_hat|;
  * selection, on the GPU's own scores of the whole row: k strictly ascending
    in-range indices whose returned scores are the row's, every key above the
    k-th score selected, and among the keys equal to it the lowest indices;
  * the longest row read from pinned host memory, in place and staged
    through HBM: scores and selection bit-identical to the HBM scan's.
"""

import numpy as np
import pytest
import torch

from oracle import fathom_oracle as O
from tests.parity import check_scores, oracle_depths

pytestmark = pytest.mark.gpu

CASES = {
    # (h_kv, g, n, d, budget, k, host copy too)
    "longest_row": (1, 1, (1 << 30) - 77, 2, 6, 2048, True),
    "most_key_heads": (8, 1, 1 << 30, 1, 3, 2048, False),
}


@pytest.fixture(scope="module")
def F():
    from sparse_attention_top_query_amd import fathom
    fathom.load()
    assert torch.cuda.is_available()
    return fathom


def block_rows(x_dev, blocks, n):
    """Rows of the given 128-key blocks of x_dev (keys [n, d] or scores [n]),
    gathered on the GPU and copied back at once: (array, rows per block)."""
    b = torch.as_tensor(np.asarray(blocks, np.int64), device=x_dev.device)
    rows = (b[:, None] * O.BLOCK + torch.arange(O.BLOCK, device=x_dev.device)[None]).clamp_(max=n - 1)
    cnt = np.minimum(O.BLOCK, n - np.asarray(blocks, np.int64) * O.BLOCK)
    return x_dev[rows.flatten()].cpu().numpy(), cnt


def oracle_block_scores(q_h, t_h, kb, cnt):
    """The oracle's (scores, sum|q k_hat|) of whole blocks laid end to end (a
    ragged block last, cut to its rows)."""
    full = int(np.sum(cnt == O.BLOCK))
    parts = []
    if full:
        kf = kb[:full * O.BLOCK]
        delta = O.block_scales(kf)
        parts.append(O.scores(q_h, O.quantize_codes(kf, delta), delta, t_h))
    for i in range(full, len(cnt)):
        kr = kb[i * O.BLOCK:i * O.BLOCK + int(cnt[i])]
        delta = O.block_scales(kr)
        parts.append(O.scores(q_h, O.quantize_codes(kr, delta), delta, t_h))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def check_block_records(rec_v, b, kb, layout):
    """Every channel of block b of one KV head's records against the oracle."""
    u, hbytes, p, r = layout
    delta = O.block_scales(kb)
    kappa = O.quantize_codes(kb, delta)
    d = kb.shape[1]
    so = 144 * (b // 8) + 2 * (b % 8)
    got = rec_v[:, so:so + 2].cpu().numpy().copy().view("<u2")[:, 0]
    assert np.array_equal(got, delta[:, 0].astype("<f2").view(np.uint16)), f"scales of block {b}"
    for plane in range(4):
        bits = ((kappa >> (3 - plane)) & 1).astype(np.uint8)
        padded = np.zeros((O.BLOCK, d), np.uint8)
        padded[:bits.shape[0]] = bits
        want = np.packbits(padded.T, axis=1, bitorder="little")
        off = 144 * (b // 8) + 16 + 16 * (b % 8) if plane == 0 else hbytes + (plane - 1) * p + 16 * b
        assert np.array_equal(rec_v[:, off:off + 16].cpu().numpy(), want), f"block {b} plane {plane}"


@pytest.mark.parametrize("case", list(CASES))
def test_size_limits(F, case):
    h_kv, g, n, d, budget, k, host_too = CASES[case]
    h_q = h_kv * g
    print(f"max-size case {case}: h_kv={h_kv} g={g} n={n} d={d} B={budget} k={k}", flush=True)
    rng = np.random.default_rng(4242 + h_kv)
    sigma = np.exp(rng.standard_normal((h_kv, d))).astype(np.float32)
    q_np = rng.standard_normal((h_q, d)).astype(np.float32)
    s2_np = (sigma * sigma).astype(np.float32)
    nb = O.n_blocks(n)
    layout = O.record_layout(n)
    r = F.record_bytes(n)
    assert r == layout[3]

    keys, rec = [], torch.empty((h_kv, d, r), dtype=torch.uint8, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    gen = torch.Generator(device="cuda:0")
    for v in range(h_kv):
        gen.manual_seed(97 + v)
        kv = torch.randn((n, d), generator=gen, dtype=torch.float32, device="cuda:0")
        kv *= torch.from_numpy(sigma[v]).to("cuda:0")
        F.pack(kv[None], records=rec[v:v + 1], status=status)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        keys.append(kv)
    sampled = sorted({0, nb - 1, *rng.choice(nb, size=6, replace=False).tolist()})
    for v in range(h_kv):
        kb, cnt = block_rows(keys[v], sampled, n)
        for i, b in enumerate(sampled):
            check_block_records(rec[v], b, kb[i * O.BLOCK:i * O.BLOCK + int(cnt[i])], layout)
    print("  records checked", flush=True)

    q = torch.from_numpy(q_np).to("cuda:0")
    dep, uni = F.allocate(q, torch.from_numpy(s2_np).to("cuda:0"), budget)
    rd, ru = oracle_depths(q_np, s2_np, budget)
    assert np.array_equal(dep.cpu().numpy(), rd) and np.array_equal(uni.cpu().numpy(), ru)

    scores = F.scan_scores(rec, q, dep, uni, n)
    idx, val = F.scan_topk(rec, q, dep, uni, n, k, want_scores=True)
    torch.cuda.synchronize()
    print("  scanned and selected", flush=True)
    if host_too:
        pinned = torch.empty(rec.shape, dtype=torch.uint8, pin_memory=True)
        pinned.copy_(rec)
        for res in (F.HOST_DIRECT, F.HOST_STAGED):
            s_host = F.scan_scores(pinned, q, dep, uni, n, residency=res)
            idx_host = F.scan_topk(pinned, q, dep, uni, n, k, residency=res)
            torch.cuda.synchronize()
            assert torch.equal(s_host.view(torch.int32), scores.view(torch.int32)), f"residency {res}: scores"
            assert torch.equal(idx_host, idx), f"residency {res}: selection"
            del s_host, idx_host
        del pinned
        print("  pinned host records, in place and staged: bit-identical", flush=True)

    for h in range(h_q):
        v = h // g
        s = scores[h]
        sel = idx[h].long()
        assert sel.numel() == k
        assert bool((sel[1:] > sel[:-1]).all()) and int(sel[0]) >= 0 and int(sel[-1]) < n, f"head {h}: indices"
        vals = s[sel]
        assert torch.equal(vals, val[h]), f"head {h}: returned scores differ from the row's"
        t = vals.min()
        n_above = int((s > t).sum())
        above_sel = int((vals > t).sum())
        assert n_above == above_sel, f"head {h}: {n_above - above_sel} keys above the k-th score left out"
        tie_sel = sel[vals == t]
        assert above_sel + tie_sel.numel() == k
        first_ties = torch.nonzero(s == t).flatten()[:tie_sel.numel()]
        assert torch.equal(first_ties, tie_sel), f"head {h}: ties not taken lowest index first"
        # the oracle's scores of the sampled blocks and of every block holding a
        # selected key (ascending, so a ragged last block comes last)
        blocks = sorted(set(sampled) | set((sel // O.BLOCK).cpu().numpy().tolist()))
        kb, cnt = block_rows(keys[v], blocks, n)
        sb, _ = block_rows(s, blocks, n)
        valid = (np.arange(O.BLOCK)[None, :] < cnt[:, None]).flatten()
        so, ao = oracle_block_scores(q_np[h], rd[h], kb[valid], cnt)
        check_scores(sb[valid], so, ao, where=f"{case} head {h} ({len(blocks)} blocks)")
    print("  checked", flush=True)


def test_most_query_heads(F):
    """65535 query heads (the most one call takes; the attention launches one
    grid row per query head), as 65535 KV heads of 200 keys: every head's
    depths bit-exact, every head's selection exact on the GPU's own scores,
    and the oracle's scores and attention on heads spread over the range."""
    from oracle import attention_oracle as A
    from synthetic import to_bf16_bits
    from tests.parity import dev, gpu_pack
    from tests.tolerances import attention_tolerance
    h_kv, n, d, budget, k = 65535, 200, 8, 12, 5
    print(f"most query heads: h_kv={h_kv} g=1 n={n} d={d} B={budget} k={k}", flush=True)
    rng = np.random.default_rng(65535)
    sigma = np.exp(rng.standard_normal((h_kv, 1, d))).astype(np.float32)
    kk = (rng.standard_normal((h_kv, n, d), dtype=np.float32) * sigma).astype(np.float32)
    q_np = rng.standard_normal((h_kv, d), dtype=np.float32)
    s2_np = (sigma[:, 0] * sigma[:, 0]).astype(np.float32)
    rec, st = gpu_pack(kk)
    assert st == 0
    q = dev(q_np)
    dep, uni = F.allocate(q, dev(s2_np), budget)
    rd, ru = oracle_depths(q_np, s2_np, budget)
    assert np.array_equal(dep.cpu().numpy(), rd) and np.array_equal(uni.cpu().numpy(), ru)
    scores = F.scan_scores(rec, q, dep, uni, n)
    idx = F.scan_topk(rec, q, dep, uni, n, k)
    torch.cuda.synchronize()
    sg, ig = scores.cpu().numpy(), idx.cpu().numpy()
    # the selection of every head: the k largest, lowest index first among
    # equal scores (a stable sort of the negated scores), in ascending order
    want = np.sort(np.argsort(-sg.astype(np.float64), axis=1, kind="stable")[:, :k], axis=1)
    assert np.array_equal(ig, want), f"{int(np.sum(np.any(ig != want, axis=1)))} heads select differently"
    heads = sorted({0, 1, h_kv - 1, *rng.choice(h_kv, size=9, replace=False).tolist()})
    for h in heads:
        delta, kappa, recs = O.pack_head(kk[h])
        assert np.array_equal(rec[h].cpu().numpy(), recs), f"records of KV head {h}"
        so, ao = O.scores(q_np[h], kappa, delta, rd[h])
        check_scores(sg[h], so, ao, where=f"head {h}")
    print("  scan checked", flush=True)
    kc = to_bf16_bits(kk)
    vc = to_bf16_bits(rng.standard_normal((h_kv, n, d), dtype=np.float32))
    scale = float(1 / np.sqrt(d))
    out, lse = F.attend(dev(kc.view(np.int16)), dev(vc.view(np.int16)), q, idx, scale)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for h in heads:
        o, l, _, _ = A.sparse_attention(q_np[h], kc[h], vc[h], ig[h], scale)
        tau_o, tau_l = attention_tolerance(q_np[h], kc[h], vc[h], ig[h], scale)
        assert np.all(np.abs(out[h].astype(np.float64) - o) <= tau_o), f"attention of head {h}"
        assert abs(float(lse[h]) - l) <= tau_l, f"lse of head {h}"
    print("  attention checked", flush=True)
