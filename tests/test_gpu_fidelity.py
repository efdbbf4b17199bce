"""The GPU path's selection fidelity on one KV head of the 131072-key workload
(k = 2048): pack -> allocate -> scan_topk -> attend_topk on the GPU give the
recall of the exact top-k and the attention error against attention over all
n keys that the oracle gives for the same mode."""

import numpy as np
import pytest
import torch

from oracle import attention_oracle as A
from oracle import fathom_oracle as O
import synthetic
from tests.parity import dev

pytestmark = pytest.mark.gpu

N, K, D, G = 131072, 2048, 128, 4


@pytest.fixture(scope="module")
def F():
    from sparse_attention_top_query_amd import fathom
    fathom.load()
    assert torch.cuda.is_available()
    return fathom


@pytest.fixture(scope="module")
def head():
    wl = synthetic.workloads()["w2_hbm_131k_B92"]
    kf, s2 = synthetic.kv_head(wl.key, 0, 0, 0, N, D, wl.outliers)
    q = synthetic.queries(wl.key, 0, 0, 0, G, D)
    kc = synthetic.to_bf16_bits(kf)
    vc = synthetic.to_bf16_bits(synthetic.values(wl.key, 0, 0, 0, N, D))
    scale = 1.0 / np.sqrt(D)
    exact = [O.topk(kf.astype(np.float64) @ q[h].astype(np.float64), K) for h in range(G)]
    full = [A.sparse_attention(q[h], kc, vc, np.arange(N), scale)[0] for h in range(G)]
    delta = O.block_scales(kf)
    packed = [(delta, O.quantize_codes(kf, delta))]
    return dict(kf=kf, s2=s2, q=q, kc=kc, vc=vc, scale=scale, exact=exact, full=full, packed=packed)


@pytest.mark.parametrize("mode,budget", [("waterfill", 68), ("waterfill", 92), ("topq", 68), ("static", 136)])
def test_fidelity_matches_the_oracle(F, head, mode, budget):
    print(f"fidelity mode={mode} B={budget}", flush=True)
    fmode = {"waterfill": F.WATERFILL, "topq": F.TOPQ, "static": F.STATIC}[mode]
    kf, q, s2, scale = head["kf"], head["q"], head["s2"], head["scale"]
    rec = F.pack(dev(kf[None]))
    depth, uni = F.allocate(dev(q), dev(s2[None]), budget, mode=fmode)
    idx = F.scan_topk(rec, dev(q), depth, uni, N, K)
    kt = torch.from_numpy(head["kc"][None].view(np.int16)).to("cuda:0")
    vt = torch.from_numpy(head["vc"][None].view(np.int16)).to("cuda:0")
    out, _ = F.attend(kt, vt, dev(q), idx, float(scale))
    torch.cuda.synchronize()
    idx_g, out_g = idx.cpu().numpy(), out.cpu().numpy().astype(np.float64)
    ref = O.step(kf[None], q, s2[None], budget, K, mode=mode, packed=head["packed"])
    for h in range(G):
        r_gpu = A.topk_recall(idx_g[h], head["exact"][h])
        r_or = A.topk_recall(ref["idx"][h], head["exact"][h])
        # selections agree up to boundary ties inside the score tolerance
        assert abs(r_gpu - r_or) <= 4 / K, f"head {h}: recall {r_gpu} vs oracle {r_or}"
        full = head["full"][h]
        e_gpu = float(np.linalg.norm(out_g[h] - full) / np.linalg.norm(full))
        e_or = A.attention_error(q[h], head["kc"], head["vc"], ref["idx"][h], scale, full=full)
        assert abs(e_gpu - e_or) <= 1e-3 * max(1.0, e_or), f"head {h}: error {e_gpu} vs oracle {e_or}"
