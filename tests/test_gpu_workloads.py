"""The five workloads at their full sizes, through the C ABI, against the oracle.

Everything the oracle can afford is compared in full; the rest on samples the
oracle computes one by one:
  * depths and union depths: every query head, bit-exact;
  * records: full KV heads where affordable, else every channel of sampled
    128-key blocks, bit-exact against the oracle's quantisation of those blocks;
  * scores and top-k: sampled query heads over all n keys, scores within
    1e-4 * sum|q k_hat|, exact selection on the GPU's own scores, top-k equal
    to the oracle's up to boundary ties inside the tolerance;
  * host residencies (in place and staged): bit-identical to each other.
"""

import numpy as np
import pytest
import torch

from oracle import fathom_oracle as O
from synthetic import layer_inputs, workloads
from tests.parity import check_scores, check_topk, oracle_depths

pytestmark = pytest.mark.gpu

WL = workloads()


@pytest.fixture(scope="module")
def F():
    from sparse_attention_top_query_amd import fathom
    fathom.load()
    assert torch.cuda.is_available()
    return fathom


def pack_layer(F, k_np, host):
    """Pack every KV head on the GPU (one head resident at a time)."""
    hk, n, d = k_np.shape
    r = F.record_bytes(n)
    rec = torch.empty((hk, d, r), dtype=torch.uint8, pin_memory=True) if host else \
        torch.empty((hk, d, r), dtype=torch.uint8, device="cuda:0")
    stage = torch.empty((1, d, r), dtype=torch.uint8, device="cuda:0")
    status = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for v in range(hk):
        kd = torch.from_numpy(k_np[v:v + 1]).to("cuda:0")
        F.pack(kd, records=stage, status=status)
        assert int(status.item()) == 0
        rec[v:v + 1].copy_(stage)
    torch.cuda.synchronize()
    return rec


def check_records(rec_np, k_np, codes, blocks_per_head=6, seed=0):
    """Full records of the KV heads in `codes` (oracle (delta, kappa) per head);
    every channel of sampled 128-key blocks for the others."""
    hk, n, d = k_np.shape
    u, hbytes, p, r = O.record_layout(n)
    nb = O.n_blocks(n)
    rng = np.random.default_rng(seed)
    for v in range(hk):
        if v in codes:
            delta, kappa = codes[v]
            assert np.array_equal(rec_np[v], O.pack_records(kappa, delta)), f"records of KV head {v}"
            continue
        for b in rng.choice(nb, size=min(blocks_per_head, nb), replace=False):
            blk = k_np[v, b * 128:min(n, b * 128 + 128)]
            delta = O.block_scales(blk)
            kappa = O.quantize_codes(blk, delta)
            so = 144 * (b // 8) + 2 * (b % 8)       # fp16 scale of block b in its unit's head slot
            got = np.ascontiguousarray(rec_np[v, :, so:so + 2]).view("<f2")[:, 0]
            assert np.array_equal(got.view(np.uint16), delta[:, 0].astype("<f2").view(np.uint16)), (v, b)
            for plane in range(4):
                bits = ((kappa >> (3 - plane)) & 1).astype(np.uint8)
                padded = np.zeros((128, d), np.uint8)
                padded[:bits.shape[0]] = bits
                want = np.packbits(padded.T, axis=1, bitorder="little")
                off = 144 * (b // 8) + 16 + 16 * (b % 8) if plane == 0 else hbytes + (plane - 1) * p + 16 * b
                assert np.array_equal(rec_np[v, :, off:off + 16], want), (v, b, plane)


def run_and_check(F, wl, layer=0, sample_heads=(0, 1, 2, 3), host_modes=None, full_record_heads=(0,)):
    budget = wl.budgets[layer]
    mode = F.WATERFILL if wl.mode == "waterfill" else F.TOPQ
    print(f"workload {wl.name} layer {layer} budget {budget}", flush=True)
    k_np, q_np, s2_np = layer_inputs(wl, layer)
    hk, n, d = k_np.shape
    g = wl.g
    host = wl.residency == "host"
    rec = pack_layer(F, k_np, host)
    codes = {}
    for v in sorted(set(full_record_heads) | {h // g for h in sample_heads}):
        delta = O.block_scales(k_np[v])
        codes[v] = (delta, O.quantize_codes(k_np[v], delta))
    check_records(rec.numpy() if host else rec.cpu().numpy(), k_np, codes)
    q = torch.from_numpy(q_np).to("cuda:0")
    dep, uni = F.allocate(q, torch.from_numpy(s2_np).to("cuda:0"), budget, mode=mode)
    rd, ru = oracle_depths(q_np, s2_np, budget, mode=wl.mode)
    assert np.array_equal(dep.cpu().numpy(), rd) and np.array_equal(uni.cpu().numpy(), ru)
    residencies = [F.HBM] if not host else (host_modes or [F.HOST_DIRECT, F.HOST_STAGED])
    results = {}
    for res in residencies:
        sg = F.scan_scores(rec, q, dep, uni, n, residency=res)
        idx = F.scan_topk(rec, q, dep, uni, n, wl.k, residency=res)
        torch.cuda.synchronize()
        results[res] = (sg.cpu().numpy(), idx.cpu().numpy())
    first = results[residencies[0]]
    for res in residencies[1:]:
        assert np.array_equal(results[res][0].view(np.uint32), first[0].view(np.uint32)), res
        assert np.array_equal(results[res][1], first[1]), res
    sg, idx = first
    for h in sample_heads:
        delta, kappa = codes[h // g]
        s, a = O.scores(q_np[h], kappa, delta, rd[h])
        check_scores(sg[h], s, a, where=f"{wl.name} head {h}")
        check_topk(idx[h], s, a, wl.k, s_gpu=sg[h], where=f"{wl.name} head {h}")
    # every head: the selection is exact on the GPU's own scores
    for h in range(idx.shape[0]):
        assert np.array_equal(idx[h], O.topk(sg[h].astype(np.float64), wl.k)), f"select head {h}"


def test_w1_single_head_4k(F):
    wl = WL["w1_single_head_4k"]
    run_and_check(F, wl, sample_heads=(0,))


@pytest.mark.parametrize("name", ["w2_hbm_131k_B46", "w2_hbm_131k_B68", "w2_hbm_131k_B92"])
def test_w2_hbm_131k(F, name):
    wl = WL[name]
    run_and_check(F, wl, sample_heads=(0, 5, 13, 31), full_record_heads=(0, 7))


def test_w3_host_1m(F):
    wl = WL["w3_host_1m_B92"]
    run_and_check(F, wl, sample_heads=(0, 3))


@pytest.mark.parametrize("layer", [int(np.argmin(WL["w4_host_1m_36layers"].budgets)),
                                   int(np.argmax(WL["w4_host_1m_36layers"].budgets))])
def test_w4_decode_layers(F, layer):
    """Two layers of the 36-layer decode step (smallest and largest budget)."""
    wl = WL["w4_host_1m_36layers"]
    run_and_check(F, wl, layer=layer, sample_heads=(0,), host_modes=[F.HOST_DIRECT])


@pytest.mark.parametrize("name", ["w5_sessions_262k_B68", "w5_sessions_262k_fixed136",
                                  "w5_sessions_262k_fixed68"])
def test_w5_sessions(F, name):
    wl = WL[name]
    # sessions 0 and 7 (virtual KV heads 0 and 56): query heads 0 and 224
    run_and_check(F, wl, sample_heads=(0, 224), full_record_heads=(0,))
