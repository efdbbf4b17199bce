"""The five workloads at their full sizes, through the C ABI, against the oracle.

Everything the oracle can afford is compared in full; the rest on samples the
oracle computes one by one:
  * depths and union depths: every query head, bit-exact;
  * records: whole KV heads (all of them at 131072 keys), else every channel of
    sampled 128-key blocks, bit-exact against the oracle's quantisation;
  * scores and top-k over all n keys: every query head at 4096, 131072 and 1M
    keys and of all 8 sessions of the 8-session workload (one session's 32 and
    one more in its fixed-depth modes), one KV head's 4 heads in each of six
    layers of the 36-layer step; scores within 1e-4 * sum|q k_hat|, exact
    selection on the GPU's own scores, top-k equal to the oracle's up to
    boundary ties inside the tolerance;
  * host residencies (in place and staged): bit-identical to each other, and
    at 1M keys to the same records scanned from HBM (the HBM scan's long-row
    case: eight generations of tiles per CU).
"""

import time

import numpy as np
import pytest
import torch

from oracle import fathom_oracle as O
from synthetic import layer_inputs, layer_queries, workloads
from tests.parity import check_scores, check_topk, dev, oracle_depths

pytestmark = pytest.mark.gpu

WL = workloads()


@pytest.fixture(scope="module")
def F():
    from sparse_attention_top_query_amd import fathom
    fathom.load()
    assert torch.cuda.is_available()
    return fathom


def oracle_codes(k_head, threads=8):
    """The oracle's scales and codes of one KV head.  The codes of a 128-key
    block depend only on that block's keys and scale, so long heads are cut into
    block-aligned ranges quantised by the oracle side by side (numpy drops the
    interpreter lock inside its loops); the result is the same array."""
    from concurrent.futures import ThreadPoolExecutor
    delta = O.block_scales(k_head)
    n = k_head.shape[0]
    nb = delta.shape[1]
    per = -(-nb // threads)
    if n < 131072:
        return delta, O.quantize_codes(k_head, delta)
    spans = [(b0, min(b0 + per, nb)) for b0 in range(0, nb, per)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda sp: O.quantize_codes(k_head[sp[0] * O.BLOCK:sp[1] * O.BLOCK],
                                                        delta[:, sp[0]:sp[1]]), spans))
    return delta, np.concatenate(parts, axis=0)


_PINNED = {}


def pinned_records(shape):
    """A pinned host buffer of this shape, allocated once per module (pinning
    half a gigabyte takes seconds; the full-size layers reuse one buffer)."""
    if shape not in _PINNED:
        _PINNED.clear()
        _PINNED[shape] = torch.empty(shape, dtype=torch.uint8, pin_memory=True)
    return _PINNED[shape]


def pack_layer(F, k_np, host, fresh=False):
    """Pack every KV head on the GPU (one head resident at a time); host records
    go to a reused pinned buffer unless `fresh`."""
    hk, n, d = k_np.shape
    r = F.record_bytes(n)
    if host:
        rec = torch.empty((hk, d, r), dtype=torch.uint8, pin_memory=True) if fresh else pinned_records((hk, d, r))
    else:
        rec = torch.empty((hk, d, r), dtype=torch.uint8, device="cuda:0")
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


def run_and_check(F, wl, layer=0, sample_heads=(0, 1, 2, 3), host_modes=None, full_record_heads=(0,),
                  select_heads=None, hbm_too=False):
    budget = wl.budgets[layer]
    mode = F.WATERFILL if wl.mode == "waterfill" else F.TOPQ
    t0 = time.perf_counter()

    def mark(what):
        print(f"  {what}: {time.perf_counter() - t0:.1f} s", flush=True)

    print(f"workload {wl.name} layer {layer} budget {budget}", flush=True)
    k_np, q_np, s2_np = layer_inputs(wl, layer)
    mark("inputs drawn")
    hk, n, d = k_np.shape
    g = wl.g
    host = wl.residency == "host"
    rec = pack_layer(F, k_np, host)
    mark("packed")
    codes = {}
    for v in sorted(set(full_record_heads) | {h // g for h in sample_heads}):
        codes[v] = oracle_codes(k_np[v])
    mark("oracle codes")
    check_records(rec.numpy() if host else rec.cpu().numpy(), k_np,
                  {v: codes[v] for v in full_record_heads})
    mark("records checked")
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
    if host and hbm_too:   # the same records copied to HBM
        rec_dev = rec.to("cuda:0")
        sg = F.scan_scores(rec_dev, q, dep, uni, n, residency=F.HBM)
        idx = F.scan_topk(rec_dev, q, dep, uni, n, wl.k, residency=F.HBM)
        torch.cuda.synchronize()
        results[F.HBM] = (sg.cpu().numpy(), idx.cpu().numpy())
        del rec_dev, sg, idx
        residencies = residencies + [F.HBM]
    first = results[residencies[0]]
    for res in residencies[1:]:
        assert np.array_equal(results[res][0].view(np.uint32), first[0].view(np.uint32)), res
        assert np.array_equal(results[res][1], first[1]), res
    sg, idx = first
    mark("scanned")
    # the oracle's scores of the sampled heads, side by side on 8 threads
    from concurrent.futures import ThreadPoolExecutor

    def oracle_head(h):
        delta, kappa = codes[h // g]
        return O.scores(q_np[h], kappa, delta, rd[h])

    with ThreadPoolExecutor(max_workers=8) as ex:
        oracle_scores = list(ex.map(oracle_head, sample_heads))
    for h, (s, a) in zip(sample_heads, oracle_scores):
        check_scores(sg[h], s, a, where=f"{wl.name} head {h}")
        check_topk(idx[h], s, a, wl.k, s_gpu=sg[h], where=f"{wl.name} head {h}")
    # every head (or those named): the selection is exact on the GPU's own scores
    for h in (range(idx.shape[0]) if select_heads is None else select_heads):
        assert np.array_equal(idx[h], O.topk(sg[h].astype(np.float64), wl.k)), f"select head {h}"
    mark("checked")


def test_w1_single_head_4k(F):
    wl = WL["w1_single_head_4k"]
    run_and_check(F, wl, sample_heads=(0,))


@pytest.mark.parametrize("name", ["w2_hbm_131k_B46", "w2_hbm_131k_B68", "w2_hbm_131k_B92"])
def test_w2_hbm_131k(F, name):
    wl = WL[name]
    run_and_check(F, wl, sample_heads=tuple(range(wl.h_q)), full_record_heads=tuple(range(wl.h_kv)))


def test_w3_host_1m(F):
    wl = WL["w3_host_1m_B92"]
    run_and_check(F, wl, sample_heads=tuple(range(wl.h_q)), full_record_heads=(0, 7), hbm_too=True)


W4 = WL["w4_host_1m_36layers"]


def spread_layers(budgets, count=6):
    """`count` layers whose budgets span the range: the smallest, the largest and
    evenly spaced ranks between (lowest layer index among equal budgets)."""
    order = sorted(range(len(budgets)), key=lambda layer: (budgets[layer], layer))
    return [order[round(i * (len(order) - 1) / (count - 1))] for i in range(count)]


def test_w4_every_layer_depths(F):
    """All 36 layers of the decode step: every query head's depths and every KV
    head's union depths bit-exact, and each head's depths spend its layer's
    budget (the per-layer budgets of the ai-feeds digest, Method, key module 3).
    Allocation reads only q and sigma2, so no keys are drawn."""
    for layer in range(W4.layers):
        budget = W4.budgets[layer]
        q_np, s2_np = layer_queries(W4, layer)
        dep, uni = F.allocate(dev(q_np), dev(s2_np), budget)
        rd, ru = oracle_depths(q_np, s2_np, budget)
        assert np.array_equal(dep.cpu().numpy(), rd), f"depths of layer {layer}"
        assert np.array_equal(uni.cpu().numpy(), ru), f"union depths of layer {layer}"
        assert np.all(rd.sum(axis=1) == budget), layer


@pytest.mark.slow
@pytest.mark.parametrize("layer", spread_layers(W4.budgets))
def test_w4_decode_layer_full_size(F, layer):
    """Six layers of the 36-layer step at full size (1M keys, pinned host records),
    budgets from the smallest to the largest: records, depths and selection as in
    the other workloads, oracle scores and top-k of the 4 query heads of one KV
    head per layer (a different KV head in each), exact selection on the GPU's
    own scores for every head."""
    v = (5 * layer + 3) % W4.h_kv
    heads = tuple(range(v * W4.g, (v + 1) * W4.g))
    run_and_check(F, W4, layer=layer, sample_heads=heads, host_modes=[F.HOST_DIRECT], full_record_heads=(v,),
                  select_heads=None)


def test_w4_decode_step_loop(F):
    """The whole 36-layer decode step as the benchmark runs it, at a reduced key
    count (50152 keys per layer, a ragged last block; every layer's records
    resident in pinned host memory together): one depth buffer and one
    workspace reused by every layer, a union-depth buffer and an index buffer
    per layer, the step run twice.  Every layer's selection: for all 32 query
    heads exact on the GPU's own scores of that layer, for the 4 query heads of
    one KV head (a different one per layer) equal to the oracle's top-k up to
    boundary ties, and identical in both runs."""
    n, k, hq, hk, d = 50152, W4.k, W4.h_q, W4.h_kv, W4.d
    g = W4.g
    layers, oracle_kv = [], []
    for layer in range(W4.layers):
        k_np, q_np, s2_np = layer_inputs(W4, layer, n=n)
        rec = pack_layer(F, k_np, host=True, fresh=True)
        v = layer % hk
        delta = O.block_scales(k_np[v])
        oracle_kv.append((v, delta, O.quantize_codes(k_np[v], delta)))
        layers.append((rec, dev(q_np), dev(s2_np), q_np, s2_np))
        del k_np
    print(f"decode step loop: {W4.layers} layers of {n} keys packed", flush=True)
    depth = torch.empty((hq, d), dtype=torch.uint8, device="cuda:0")
    uni = [torch.empty((hk, d), dtype=torch.uint8, device="cuda:0") for _ in range(W4.layers)]
    ws = torch.empty(F.workspace_bytes(hq, hk, n, d, k, F.HOST_DIRECT), dtype=torch.uint8, device="cuda:0")
    runs = []
    for _ in range(2):
        idx = torch.empty((W4.layers, hq, k), dtype=torch.int32, device="cuda:0")
        for layer, (rec, q, s2, _, _) in enumerate(layers):
            F.allocate(q, s2, W4.budgets[layer], depth=depth, union_depth=uni[layer])
            F.scan_topk(rec, q, depth, uni[layer], n, k, residency=F.HOST_DIRECT, workspace=ws, idx=idx[layer])
        torch.cuda.synchronize()
        runs.append(idx.cpu().numpy())
    assert np.array_equal(runs[0], runs[1]), "the two runs of the step differ"
    idx = runs[0]
    for layer, (rec, q, s2, q_np, s2_np) in enumerate(layers):
        rd, ru = oracle_depths(q_np, s2_np, W4.budgets[layer])
        assert np.array_equal(uni[layer].cpu().numpy(), ru), f"union depths kept for layer {layer}"
        sg = F.scan_scores(rec, q, dev(rd.astype(np.uint8)), uni[layer], n, residency=F.HOST_DIRECT)
        sg = sg.cpu().numpy()
        for h in range(hq):
            assert np.array_equal(idx[layer, h], O.topk(sg[h].astype(np.float64), k)), f"layer {layer} head {h}"
        v, delta, kappa = oracle_kv[layer]
        for h in range(v * g, (v + 1) * g):
            s, a = O.scores(q_np[h], kappa, delta, rd[h])
            check_scores(sg[h], s, a, where=f"layer {layer} head {h}")
            check_topk(idx[layer, h], s, a, k, where=f"layer {layer} head {h}")


@pytest.mark.parametrize("name", ["w5_sessions_262k_B68", "w5_sessions_262k_fixed136",
                                  "w5_sessions_262k_fixed68"])
def test_w5_sessions(F, name):
    wl = WL[name]
    if wl.mode == "waterfill":
        # the method: every query head of all 8 sessions
        heads = tuple(range(wl.sessions * wl.h_q))
    else:
        # the fixed-depth comparison modes: every query head of session 0
        # (virtual KV heads 0-7) and query head 224 of session 7 (virtual KV head 56)
        heads = tuple(range(wl.h_q)) + (224,)
    run_and_check(F, wl, sample_heads=heads, full_record_heads=(0,))


@pytest.mark.parametrize("name", ["w2_hbm_131k_B92", "w3_host_1m_B92"])
def test_attention_at_full_size(F, name):
    """attend_topk at the benchmark's shapes: the method's own top-2048 of each of
    the 32 query heads (scan_topk over the full records), attention over those
    rows of the workload's bf16 K/V caches (HBM at 131072 keys, pinned host
    memory at 1M keys), every head against the oracle's attention within the
    order-independent fp32 bound."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import attention_oracle as A
    from synthetic import to_bf16_bits, values
    from tests.tolerances import attention_tolerance
    wl = WL[name]
    host = wl.residency == "host"
    print(f"attention at full size: {wl.name}", flush=True)
    k_np, q_np, s2_np = layer_inputs(wl, 0)
    hk, n, d = k_np.shape
    rec = pack_layer(F, k_np, host)
    q = dev(q_np)
    dep, uni = F.allocate(q, dev(s2_np), wl.budgets[0])
    idx = F.scan_topk(rec, q, dep, uni, n, wl.k, residency=F.HOST_DIRECT if host else F.HBM)
    kc = to_bf16_bits(k_np)
    del k_np
    vc = np.stack([to_bf16_bits(values(wl.key, 0, 0, v, n, d)) for v in range(hk)])

    def cache(a):
        t = torch.from_numpy(a.view(np.int16))
        if not host:
            return t.to("cuda:0")
        p = torch.empty(t.shape, dtype=torch.int16, pin_memory=True)
        p.copy_(t)
        return p

    scale = float(1 / np.sqrt(d))
    out, lse = F.attend(cache(kc), cache(vc), q, idx, scale)
    torch.cuda.synchronize()
    out, lse, idx = out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()

    def one(h):
        v = h // wl.g
        o, l, _, _ = A.sparse_attention(q_np[h], kc[v], vc[v], idx[h], scale)
        tau_o, tau_l = attention_tolerance(q_np[h], kc[v], vc[v], idx[h], scale)
        return o, l, tau_o, tau_l

    with ThreadPoolExecutor(max_workers=8) as ex:
        ref = list(ex.map(one, range(wl.h_q)))
    for h, (o, l, tau_o, tau_l) in enumerate(ref):
        err = np.abs(out[h].astype(np.float64) - o)
        assert np.all(err <= tau_o), f"{wl.name} head {h}: worst excess {float(np.max(err - tau_o)):.3e}"
        assert abs(float(lse[h]) - l) <= tau_l, f"{wl.name} head {h}: lse {lse[h]} vs {l}"
