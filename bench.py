"""Benchmark of the Fathom top-k step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one pass of the whole hot path over one batch: allocate_depths
(reverse water-filling for every query head) then scan_topk (read the budgeted
plane prefixes, score every key, select the top k) for one layer.  The default
workload is 8 KV heads x 4 query heads, d = 128, n = 1,048,576 keys, B = 92,
k = 2048, with the packed records in pinned host memory read over the host
link.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PCIE5_X16_GBPS = 64.0      # published host-link rate per direction (PCIe 5.0 x16)
HBM_PEAK_GBPS = 8000.0     # MI355X HBM3E
# VALU lane-operations per second: 256 CUs x 64 lanes x 2.4 GHz (packed FP32 is
# not used, so one lane-op per lane and clock)
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12
# The pages' own figures (NVIDIA A100, Qwen3-8B, 4-bit K cache), quoted for
# context only: the Fathom arXiv abstract and the thedatum.uk "Key facts".
PAGES_CONTEXT = {
    "hardware": "A100 (the pages' setup; not this machine)",
    "decode_step_speedup_vs_136bit_scans_at_1M": 1.67,
    "fewer_bytes_than_68bit_sparq_r16_at_equal_gpu_time": 0.18,
    "bits_reaching_the_136bit_step_agreement": 92,
    "index_resident_in_gpu_memory": "no speedup (the kernel is arithmetic-bound)",
}

# rocprofv3 summaries whose FETCH_SIZE / WRITE_SIZE figures give the measured
# traffic of the dominant kernel, keyed by (workload, residency)
PROFILES = {
    ("w3_host_1m_B92", "direct"): "scan_host_1m_B92_direct.md",
    ("w2_hbm_131k_B92", "hbm"): "scan_hbm_131k_B92.md",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="w3_host_1m_B92")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-attend", action="store_true",
                    help="skip the attention over the selected keys (bf16 K/V caches are not built)")
    ap.add_argument("--no-append", action="store_true",
                    help="skip the growing-cache measurement (open tail block, sealing one block)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-records measurement (the same step over pages of 65536 keys)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the fixed-depth (136-bit, 68-bit) comparison scans")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--residency", choices=["staged", "direct"], default="direct",
                    help="host-resident records: read in place by the scan (default) or staged through HBM")
    ap.add_argument("--calibrate", action="store_true",
                    help="only run a 1 GiB device-to-device copy (the known-size kernel used to scale the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--copies", type=int, default=8,
                    help="HBM-resident workloads: distinct record copies cycled per step, so the "
                         "256 MB Infinity Cache cannot hold them")
    return ap.parse_args()


def algorithmic_bytes(union: np.ndarray, n: int) -> int:
    """Bytes the method must read per step: for every (KV head, channel) with a
    nonzero union depth t, its contiguous prefix run -- the block scales and t
    planes of its n keys (n/64 + t n/8 bytes for n a multiple of 1024)."""
    units = -(-((n + 127) // 128) // 8)
    t = union.astype(np.int64)
    return int(np.where(t > 0, 144 * units + (t - 1) * 128 * units, 0).sum())


def algorithmic_ops(depth: np.ndarray, union: np.ndarray, n: int) -> int:
    """VALU lane-operations of the reconstruction for all keys.  A lane holds 4
    keys' prefixes side by side in the bytes of one register, so per KV head,
    union channel and 4 keys: 2 ops per plane of the union depth (a rotate and
    an and-or), 5 per distinct depth read by some head (setting the midpoint
    bit, then 4 signed-byte conversions to float), and 4 FMAs per query head
    that reads the channel.  Counted over all KV-head keys."""
    hk, d = union.shape
    g = depth.shape[0] // hk
    dep = depth.reshape(hk, g, d).astype(np.int64)
    u = union.astype(np.int64)
    planes = u.sum()
    levels = sum(((dep == t).any(axis=1)).sum() for t in range(1, 5))
    fmas = (dep > 0).sum()
    return int((2 * planes + 5 * levels + 4 * fmas) * n // 4)


def kernel_code_digest(files=("scan.hip", "fathom_internal.h")) -> str:
    """sha256 of the kernel sources' code: comments dropped and whitespace
    collapsed, so that a comment edit does not disown counters taken from the
    same code."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        text = open(os.path.join(ROOT, "sparse_attention_top_query_amd", "csrc", f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: str, residency: str, kernel: str):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch from the committed
    rocprofv3 summary of this workload, or None when there is none or the scan
    code has changed since the counters were taken."""
    name = PROFILES.get((workload, residency))
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
        return None
    text = open(path).read()
    if "```figures" not in text:
        return None
    fig = {}
    for line in text.split("```figures", 1)[1].split("```", 1)[0].strip().splitlines():
        key, _, val = line.partition(":")
        fig[key.strip()] = val.strip()
    if fig.get("kernel_code_sha256") != kernel_code_digest() or "fetch_bytes_per_dispatch" not in fig:
        return None
    if not kernel.startswith(fig.get("kernel", "?").split("<")[0]):
        return None
    fetch, write = int(fig["fetch_bytes_per_dispatch"]), int(fig["write_bytes_per_dispatch"])
    return {"total": fetch + write, "fetch": fetch, "write": write, "source": f"profiles/{name}"}


def measure_h2d_peak(torch, dev, mib=512, reps=5) -> float:
    src = torch.empty(mib << 20, dtype=torch.uint8, pin_memory=True)
    src.fill_(1)
    dst = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev)
    best = 1e30
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        dst.copy_(src, non_blocking=True)
        b.record(s)
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    return (mib << 20) / (best * 1e-3) / 1e9


def build_records(torch, F, wl, dev, layer=0, caches=False, nibbles=False):
    """Generate K per KV head (numpy, threaded), pack on the GPU, return records
    resident where the workload puts them, plus q and sigma2 on the device.
    With `caches`, also the bf16 K and V cache rows [h_kv, n, d] (as int16 bit
    patterns) in the same residency, for the attention over the selection; with
    `nibbles`, also the token-major 4-bit copy (codes, scales) there."""
    from synthetic import kv_head, queries, to_bf16_bits, values
    hk = wl.sessions * wl.h_kv
    r = F.record_bytes(wl.n)
    host = wl.residency == "host"
    if host:
        records = torch.empty((hk, wl.d, r), dtype=torch.uint8, pin_memory=True)
    else:
        records = torch.empty((hk, wl.d, r), dtype=torch.uint8, device=dev)
    s2 = np.empty((hk, wl.d), np.float32)
    q = np.empty((hk * wl.g, wl.d), np.float32)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    stage = torch.empty((1, wl.d, r), dtype=torch.uint8, device=dev)
    kc = vc = None
    nib = None
    if nibbles:
        nb = -(-wl.n // 128)
        nib = (torch.empty((hk, wl.n, wl.d // 2), dtype=torch.uint8, pin_memory=host, device=None if host else dev),
               torch.empty((hk, nb, wl.d), dtype=torch.float16, pin_memory=host, device=None if host else dev))
    if caches:
        kc = torch.empty((hk, wl.n, wl.d), dtype=torch.int16, pin_memory=host, device=None if host else dev)
        vc = torch.empty((hk, wl.n, wl.d), dtype=torch.int16, pin_memory=host, device=None if host else dev)

    def gen(v):
        s, g = divmod(v, wl.h_kv)
        k, sig2 = kv_head(wl.key, layer, s, g, wl.n, wl.d, wl.outliers)
        kb = vb = None
        if caches:
            kb = torch.from_numpy(to_bf16_bits(k).view(np.int16))
            vb = torch.from_numpy(to_bf16_bits(values(wl.key, layer, s, g, wl.n, wl.d)).view(np.int16))
        return v, (k, sig2), kb, vb

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        for v, (k, sig2), kb, vb in ex.map(gen, range(hk)):
            s, g = divmod(v, wl.h_kv)
            if caches:
                kc[v].copy_(kb)
                vc[v].copy_(vb)
            s2[v] = sig2
            q[v * wl.g:(v + 1) * wl.g] = queries(wl.key, layer, s, g, wl.g, wl.d)
            kd = torch.from_numpy(k).to(dev)[None]
            F.pack(kd, records=stage if host else records[v:v + 1], status=status)
            if host:
                records[v:v + 1].copy_(stage)
            if nibbles:
                c4, sc = F.pack_nibbles(kd, status=status)
                nib[0][v:v + 1].copy_(c4)
                nib[1][v:v + 1].copy_(sc)
            del kd
    torch.cuda.synchronize(dev)
    assert int(status.item()) == 0, "pack reported non-finite keys or scale overflow"
    if nibbles:
        return records, torch.from_numpy(q).to(dev), torch.from_numpy(s2).to(dev), q, s2, kc, vc, nib
    return records, torch.from_numpy(q).to(dev), torch.from_numpy(s2).to(dev), q, s2, kc, vc


_CPU = {}


def _oracle_heads(seconds: float, first: int):
    """Worker: query-head scans of the oracle (allocation + fp64 scores + top-k)
    for about `seconds`, cycling over the group's heads from `first`."""
    from threadpoolctl import threadpool_limits

    from oracle import fathom_oracle as O
    c = _CPU
    heads = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while heads < 1 or time.perf_counter() - t0 < seconds:
            h = (first + heads) % c["q"].shape[0]
            t = O.waterfill_depths(O.importance(c["q"][h], c["s2"]), c["budget"])
            s, _ = O.scores(c["q"][h], c["kappa"], c["delta"], t)
            O.topk(s, c["k"])
            heads += 1
    return heads, time.perf_counter() - t0


def host_cpu_info() -> dict:
    """The host CPU as /proc/cpuinfo shows it: the model string, its
    family/model/stepping numbers, and how many logical CPUs and distinct
    physical cores (physical id, core id) this process may run on."""
    allowed = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else set(range(os.cpu_count() or 1))
    model, fms, cores, sockets = "unknown CPU", "?", set(), set()
    try:
        with open("/proc/cpuinfo") as f:
            text = f.read()
        for block in text.strip().split("\n\n"):
            kv = {}
            for line in block.splitlines():
                if ":" in line:
                    key, val = line.split(":", 1)
                    kv[key.strip()] = val.strip()
            if "processor" not in kv:
                continue
            model = kv.get("model name", model)
            fms = f"{kv.get('cpu family', '?')}/{kv.get('model', '?')}/{kv.get('stepping', '?')}"
            if int(kv["processor"]) in allowed:
                cores.add((kv.get("physical id", "0"), kv.get("core id", kv["processor"])))
                sockets.add(kv.get("physical id", "0"))
    except (OSError, ValueError):
        pass
    return {"model": model, "fms": fms, "logical": len(allowed), "physical": len(cores) or None,
            "sockets": len(sockets) or None}


def cpu_baseline(wl, budget, seconds=15.0, workers=12):
    """The oracle timed on this host, before anything touches the GPU: the query
    heads of KV head 0 over all n keys (codes precomputed, not timed), first on
    one core, then on a pool of `workers` forked processes, one head scan each at
    a time.  The pool's aggregate rate is the value."""
    import multiprocessing as mp

    from oracle import fathom_oracle as O
    from synthetic import kv_head, queries
    k, s2 = kv_head(wl.key, 0, 0, 0, wl.n, wl.d, wl.outliers)
    delta = O.block_scales(k)
    _CPU.update(kappa=O.quantize_codes(k, delta), delta=delta, s2=s2, budget=budget, k=wl.k,
                q=queries(wl.key, 0, 0, 0, wl.g, wl.d))
    del k
    one_heads, one_dt = _oracle_heads(seconds / 3, 0)
    workers = max(1, min(workers, os.cpu_count() or 1))
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.starmap(_oracle_heads, [(2 * seconds / 3, i) for i in range(workers)])
    _CPU.clear()
    rate = sum(h * wl.n / dt for h, dt in res)
    info = host_cpu_info()
    return {"value": round(rate, 1), "unit": "keys/s", "cores": workers, "kind": "oracle",
            "single_core_value": round(one_heads * wl.n / one_dt, 1),
            "cpu_model": info["model"], "cpu_family_model_stepping": info["fms"],
            "logical_cpus_visible": info["logical"], "physical_cores_visible": info["physical"],
            "sockets": info["sockets"], "numpy": np.__version__,
            "host": f"{info['model']} (family/model/stepping {info['fms']}), {info['logical']} logical CPUs "
                    f"on {info['physical']} physical cores visible, numpy {np.__version__}",
            "sample": f"query-head scans of the {wl.g} heads of KV head 0 x {wl.n} keys (allocation + fp64 "
                      f"scores + top-{wl.k}, codes precomputed), numpy single-threaded per process: "
                      f"{sum(h for h, _ in res)} scans on {workers} forked processes in "
                      f"{max(dt for _, dt in res):.1f} s; {one_heads} scans on one core in {one_dt:.1f} s"}


def run_layers(args, torch, F, wl, dev):
    """A whole decode step over every layer of a multi-layer workload: per layer,
    allocate_depths with that layer's budget, then scan_topk over the layer's
    records (all layers resident together).  Prints one JSON line."""
    h2d_peak = measure_h2d_peak(torch, dev)
    host = wl.residency == "host"
    residency = F.HOST_DIRECT if host else F.HBM
    t_setup = time.perf_counter()
    layers = []
    for layer in range(wl.layers):
        records, q, s2, q_np, s2_np, _, _ = build_records(torch, F, wl, dev, layer=layer)
        layers.append((records, q, s2))
        print(f"layer {layer} built", file=sys.stderr, flush=True)
    setup_s = time.perf_counter() - t_setup
    hk, hq, n, d, k = wl.sessions * wl.h_kv, wl.sessions * wl.h_q, wl.n, wl.d, wl.k
    depth = torch.empty((hq, d), dtype=torch.uint8, device=dev)
    uni = [torch.empty((hk, d), dtype=torch.uint8, device=dev) for _ in range(wl.layers)]
    ws = torch.empty(F.workspace_bytes(hq, hk, n, d, k, residency), dtype=torch.uint8, device=dev)
    idx = torch.empty((wl.layers, hq, k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        for layer, (records, q, s2) in enumerate(layers):
            F.allocate(q, s2, wl.budgets[layer], depth=depth, union_depth=uni[layer])
            F.scan_topk(records, q, depth, uni[layer], n, k, residency=residency, workspace=ws, idx=idx[layer])

    steps = max(1, min(args.steps, 10))
    for _ in range(max(1, min(args.warmup, 2))):
        step()
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    step_ms = e0.elapsed_time(e1) / steps
    # the scan stage alone over all layers, with the depths of the last step
    scores = torch.empty((hq, n), dtype=torch.float32, device=dev)
    alg = 0
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dep_l = []
    for layer, (records, q, s2) in enumerate(layers):
        dl = torch.empty((hq, d), dtype=torch.uint8, device=dev)
        F.allocate(q, s2, wl.budgets[layer], depth=dl, union_depth=uni[layer])
        dep_l.append(dl)
        alg += algorithmic_bytes(uni[layer].cpu().numpy(), n)
    torch.cuda.synchronize(dev)
    s0.record(stream)
    for layer, (records, q, s2) in enumerate(layers):
        F.scan_scores(records, q, dep_l[layer], uni[layer], n, residency=residency, out=scores, workspace=ws)
    s1.record(stream)
    torch.cuda.synchronize(dev)
    scan_ms = s0.elapsed_time(s1)
    achieved = alg / (scan_ms * 1e-3) / 1e9
    peak = PCIE5_X16_GBPS if host else HBM_PEAK_GBPS
    out = {
        "metric": "keys scanned/s per top-k step at 1M tokens (host-resident), % of link/HBM BW",
        "value": round(wl.layers * hq * n / (step_ms * 1e-3), 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(1, min(args.warmup, 2)),
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.layers, "h_kv": hk, "h_q": hq, "d": d, "n": n,
                   "budget_bits_per_layer": list(wl.budgets), "k": k,
                   "residency": "pinned host, direct over the host link" if host else "HBM"},
        "roofline": {"bound": "host_link" if host else "hbm", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "GB/s", "frac": round(achieved / peak, 4), "traffic": None,
                     "measured_h2d_peak": round(h2d_peak, 2) if host else None,
                     "frac_of_measured_h2d": round(achieved / h2d_peak, 4) if host else None,
                     "kernel": "scan_kernel<4, 64>" if host else "scan_kernel<4, 8>",
                     "scan_ms_all_layers": round(scan_ms, 3), "bytes_all_layers": alg},
        "cpu_baseline": None,
        "record_bytes_resident": wl.layers * hk * d * F.record_bytes(n),
        "decode_steps_per_s": round(1000.0 / step_ms, 2),
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the scan shards by KV head "
              "or token range with no exchange inside a step, so one GPU's share at the real shape is "
              "what is measured", file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_attention_top_query_amd as F
    from synthetic import workloads
    # the oracle's CPU timing runs first, while no GPU state exists to fork
    cpu = None
    if not args.no_cpu and not args.calibrate and workloads()[args.workload].layers == 1:
        wl0 = workloads()[args.workload]
        cpu = cpu_baseline(wl0, wl0.budgets[0])
    F.load()
    dev = torch.device("cuda:0")
    if args.calibrate:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"calibration": "device-to-device copy", "bytes_per_copy": 1 << 30, "copies": 3}))
        return
    wl = workloads()[args.workload]
    if wl.layers != 1:
        run_layers(args, torch, F, wl, dev)
        return
    budget = wl.budgets[0]
    mode = F.WATERFILL if wl.mode == "waterfill" else F.TOPQ
    h2d_peak = measure_h2d_peak(torch, dev)

    t_setup = time.perf_counter()
    free_path = not args.no_compare and wl.d % 32 == 0 and wl.d <= 128
    built = build_records(torch, F, wl, dev, caches=not args.no_attend, nibbles=free_path)
    records, q, s2, q_np, s2_np, kc, vc = built[:7]
    nib = built[7] if free_path else None
    setup_s = time.perf_counter() - t_setup
    hk, hq, n, d, k = wl.sessions * wl.h_kv, wl.sessions * wl.h_q, wl.n, wl.d, wl.k

    host = wl.residency == "host"
    residency = (F.HOST_STAGED if args.residency == "staged" else F.HOST_DIRECT) if host else F.HBM
    copies = [records]
    if not host:
        copies += [records.clone() for _ in range(max(0, args.copies - 1))]
    depth = torch.empty((hq, d), dtype=torch.uint8, device=dev)
    uni = torch.empty((hk, d), dtype=torch.uint8, device=dev)
    ws = torch.empty(F.workspace_bytes(hq, hk, n, d, k, residency), dtype=torch.uint8, device=dev)
    idx = torch.empty((hq, k), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    it = [0]

    def step():
        rec = copies[it[0] % len(copies)]
        it[0] += 1
        F.allocate(q, s2, budget, mode=mode, depth=depth, union_depth=uni)
        F.scan_topk(rec, q, depth, uni, n, k, residency=residency, workspace=ws, idx=idx)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    step_ms = ev0.elapsed_time(ev1) / args.steps

    # the scan stage alone (the same launches as inside scan_topk), timed with
    # events on the stream it is launched on
    scores = torch.empty((hq, n), dtype=torch.float32, device=dev)
    F.scan_scores(records, q, depth, uni, n, residency=residency, out=scores, workspace=ws)
    torch.cuda.synchronize(dev)
    ka, kb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ka.record(stream)
    for r in range(args.kernel_reps):
        F.scan_scores(copies[r % len(copies)], q, depth, uni, n, residency=residency, out=scores, workspace=ws)
    kb.record(stream)
    torch.cuda.synchronize(dev)
    scan_ms = ka.elapsed_time(kb) / args.kernel_reps
    del scores

    union_np = uni.cpu().numpy()
    alg_bytes = algorithmic_bytes(union_np, n)
    achieved = alg_bytes / (scan_ms * 1e-3) / 1e9
    keys_per_s = hq * n / (step_ms * 1e-3)
    g = hq // hk
    if host and residency == F.HOST_STAGED:
        kname = f"stage_scan_kernel<{g}, 8>"
    else:
        kname = f"scan_kernel<{g}, {64 if g <= 4 else 16}>" if host else f"scan_kernel<{g}, 8>"
    res_key = args.residency if host else "hbm"
    traffic = measured_traffic(args.workload, res_key, kname)
    common = {"traffic": traffic["total"] if traffic else None,
              "traffic_fetch": traffic["fetch"] if traffic else None,
              "traffic_write": traffic["write"] if traffic else None,
              "traffic_source": traffic["source"] if traffic else None,
              "kernel": kname, "kernel_ms": round(scan_ms, 4), "bytes_per_launch": alg_bytes}
    if host:
        roof = {"bound": "host_link", "achieved": round(achieved, 2), "peak": PCIE5_X16_GBPS, "unit": "GB/s",
                "frac": round(achieved / PCIE5_X16_GBPS, 4), **common,
                "measured_h2d_peak": round(h2d_peak, 2), "frac_of_measured_h2d": round(achieved / h2d_peak, 4),
                "residency": args.residency}
    else:
        # records in HBM: the reconstruction's VALU work bounds the scan, not HBM
        ops = algorithmic_ops(depth.cpu().numpy(), union_np, n)
        tops = ops / (scan_ms * 1e-3) / 1e12
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), **common,
                "limiter": "alu: the reconstruction's vector work, not HBM, sets the scan's time",
                "alu_achieved": round(tops, 3), "alu_peak": round(VALU_PEAK_TOPS, 2), "alu_unit": "T lane-op/s",
                "alu_frac": round(tops / VALU_PEAK_TOPS, 4), "ops_per_launch": ops,
                "ns_per_kv_head_key": round(scan_ms * 1e6 / (hk * n), 5),
                "record_copies_cycled": len(copies)}
    # The pages compare the method against fixed-depth scans: 136 bits (34
    # channels x 4 planes) and 68 bits (17 x 4), channels by largest |q_c|.
    # Same records, queries and stream, timed the same way.
    comparison = None
    if not args.no_compare:
        def timed(b, m, steps):
            def one():
                rec = copies[it[0] % len(copies)]   # HBM: cycled like the step's, so not cache-resident
                it[0] += 1
                F.allocate(q, s2, b, mode=m, depth=depth, union_depth=uni)
                F.scan_topk(rec, q, depth, uni, n, k, residency=residency, workspace=ws, idx=idx)
            for _ in range(2):
                one()
            torch.cuda.synchronize(dev)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(steps):
                one()
            e1.record(stream)
            torch.cuda.synchronize(dev)
            ms = e0.elapsed_time(e1) / steps
            picks[name_of[(b, m)]] = idx[:hq // hk].cpu().numpy()
            return {"ms_per_step": round(ms, 4),
                    "bytes_per_key": round(algorithmic_bytes(uni.cpu().numpy(), n) / (hk * n), 3)}
        csteps = max(3, min(args.steps, 20))
        comparison = {"method_B": budget, "method_ms_per_step": round(step_ms, 4)}
        modes = []
        for name, b, m in ((f"method_B{budget}", budget, F.WATERFILL), ("fixed_136", 136, F.TOPQ),
                           ("fixed_68", 68, F.TOPQ), ("static_136", 136, F.STATIC), ("static_68", 68, F.STATIC),
                           ("method_B68", 68, F.WATERFILL), ("method_B46", 46, F.WATERFILL),
                           (f"group_shared_B{budget}", budget, F.WATERFILL_GROUP)):
            if all((b, m) != (b2, m2) for _, b2, m2 in modes):
                modes.append((name, b, m))
        picks, name_of = {}, {(b, m): name for name, b, m in modes}
        for name, b, m in modes:
            comparison[name] = timed(b, m, csteps)
        # informational: recall@k against the exact fp32 top-k of q . K on the
        # unquantised keys, for the query heads of KV head 0
        from synthetic import kv_head
        k0, _ = kv_head(wl.key, 0, 0, 0, n, d, wl.outliers)
        exact = [set(np.argpartition(-(k0 @ q_np[h]), k - 1)[:k].tolist()) for h in range(hq // hk)]
        del k0
        comparison["recall_at_k_vs_exact_fp32"] = {
            name: round(float(np.mean([len(exact[h] & set(sel[h].tolist())) / k for h in range(len(exact))])), 4)
            for name, sel in picks.items()}
        comparison["recall_sample"] = f"the {hq // hk} query heads of KV head 0, top-{k} of {n} keys"
        comparison["speedup_vs_fixed_136"] = round(comparison["fixed_136"]["ms_per_step"] / step_ms, 3)
        if nib is not None:
            # the free path: the same depths over the token-major 4-bit copy,
            # which every scan reads whole (d/2 + d/64 bytes per key)
            F.allocate(q, s2, budget, mode=mode, depth=depth, union_depth=uni)
            for _ in range(2):
                F.scan_topk_nibbles(nib[0], nib[1], q, depth, uni, k, workspace=ws, idx=idx)
            torch.cuda.synchronize(dev)
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            f0.record(stream)
            for _ in range(csteps):
                F.allocate(q, s2, budget, mode=mode, depth=depth, union_depth=uni)
                F.scan_topk_nibbles(nib[0], nib[1], q, depth, uni, k, workspace=ws, idx=idx)
            f1.record(stream)
            torch.cuda.synchronize(dev)
            fms = f0.elapsed_time(f1) / csteps
            fbytes = hk * (n * (d // 2) + -(-n // 128) * d * 2)   # codes, then one fp16 scale per block and channel
            fgbps = fbytes / (fms * 1e-3) / 1e9
            comparison[f"free_path_B{budget}"] = {
                "ms_per_step": round(fms, 4), "bytes_per_key": round(d / 2 + d / 64, 3),
                "bytes_per_step": fbytes, "gbps_over_the_step": round(fgbps, 2),
                "frac_of_measured_h2d" if host else "frac_of_hbm_peak":
                    round(fgbps / (h2d_peak if host else HBM_PEAK_GBPS), 4),
                "what": "the same depths over the token-major 4-bit copy (scan_topk_nibbles)"}
            comparison["speedup_vs_free_path"] = round(fms / step_ms, 3)
        b68 = name_of[(68, F.WATERFILL)]
        comparison["bytes_method_B68_vs_fixed_68"] = round(
            comparison[b68]["bytes_per_key"] / comparison["fixed_68"]["bytes_per_key"], 3)
    # Attention over the selected keys (the step after the scan): the bf16 K and
    # V rows of every query head's top-k, gathered from the same residency.
    attention = None
    if not args.no_attend:
        step()   # idx of the method's own selection at this budget
        scale = float(1.0 / np.sqrt(d))
        aws = torch.empty(F.attend_workspace_bytes(hq, d, k), dtype=torch.uint8, device=dev)
        aout = torch.empty((hq, d), dtype=torch.float32, device=dev)
        alse = torch.empty(hq, dtype=torch.float32, device=dev)
        for _ in range(3):
            F.attend(kc, vc, q, idx, scale, out=aout, lse=alse, workspace=aws)
        torch.cuda.synchronize(dev)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(5, args.kernel_reps)
        a0.record(stream)
        for _ in range(reps):
            F.attend(kc, vc, q, idx, scale, out=aout, lse=alse, workspace=aws)
        a1.record(stream)
        torch.cuda.synchronize(dev)
        att_ms = a0.elapsed_time(a1) / reps
        att_bytes = hq * k * d * 2 * 2
        att_gbps = att_bytes / (att_ms * 1e-3) / 1e9
        # rows selected by several query heads of a KV head need crossing the
        # link (or leaving HBM) only once: the distinct rows per KV head
        sel = idx.cpu().numpy().reshape(hk, hq // hk, k)
        uniq = sum(int(np.unique(sel[v]).size) for v in range(hk))
        uniq_bytes = uniq * d * 2 * 2
        uniq_gbps = uniq_bytes / (att_ms * 1e-3) / 1e9
        peak = h2d_peak if host else HBM_PEAK_GBPS
        attention = {"ms": round(att_ms, 4), "bytes_per_call": att_bytes,
                     "achieved_gbps": round(att_gbps, 2),
                     "distinct_row_bytes": uniq_bytes, "distinct_row_gbps": round(uniq_gbps, 2),
                     "frac": round(uniq_gbps / peak, 4),
                     "of": "measured H2D peak, distinct rows" if host else "8 TB/s HBM, distinct rows",
                     "kernel": "attend_kernel<16> + attend_merge" if d == 128 else "attend_kernel + attend_merge",
                     "rows": f"{hq} query heads x {k} selected keys x (K + V) bf16 rows of {d}",
                     "step_plus_attention_ms": round(step_ms + att_ms, 4)}
    # A growing cache: the last block left open (127 exact fp32 keys scored by
    # the tail kernel, the rest scanned as sealed blocks), and the cost of
    # sealing one 128-key block of every KV head.
    append = None
    if not args.no_append and n >= 256:
        from synthetic import kv_head
        n_sealed = (n - 1) // 128 * 128
        n_tail = n - 1 - n_sealed
        # rows n_sealed - 128 .. n - 2 of every KV head: the block to seal, then the tail
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            rows = np.stack(list(ex.map(
                lambda v: kv_head(wl.key, 0, v // wl.h_kv, v % wl.h_kv, n, d, wl.outliers)[0][n_sealed - 128:n - 1],
                range(hk))))
        tail = torch.from_numpy(np.ascontiguousarray(rows[:, 128:])).to(dev)
        blk = torch.from_numpy(np.ascontiguousarray(rows[:, :128])).to(dev)
        aws2 = torch.empty(F.workspace_bytes(hq, hk, n_sealed + n_tail, d, k, F.HBM), dtype=torch.uint8, device=dev)

        def step_tail():
            F.allocate(q, s2, budget, mode=mode, depth=depth, union_depth=uni)
            F.scan_topk_append(records, n, n_sealed, tail, q, depth, uni, k,
                               residency=F.HOST_DIRECT if host else F.HBM, workspace=aws2, idx=idx)
        for _ in range(2):
            step_tail()
        torch.cuda.synchronize(dev)
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tsteps = max(3, min(args.steps, 20))
        b0.record(stream)
        for _ in range(tsteps):
            step_tail()
        b1.record(stream)
        torch.cuda.synchronize(dev)
        # sealing: one block of every KV head into device records of the same capacity
        seal_rec = torch.empty((hk, d, F.record_bytes(n)), dtype=torch.uint8, device=dev)
        for _ in range(3):
            F.pack_blocks(blk, seal_rec, n, n_sealed // 128 - 1)
        torch.cuda.synchronize(dev)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(20):
            F.pack_blocks(blk, seal_rec, n, n_sealed // 128 - 1)
        c1.record(stream)
        torch.cuda.synchronize(dev)
        append = {"open_tail_keys": n_tail, "sealed_keys": n_sealed,
                  "step_with_open_tail_ms": round(b0.elapsed_time(b1) / tsteps, 4),
                  "seal_one_block_all_kv_heads_us": round(c0.elapsed_time(c1) / 20 * 1e3, 2)}
        del seal_rec, blk, tail, aws2
    # Paged records: the same step over pages of 65536 keys, each page its own
    # allocation in the workload's residency, placed in shuffled order and
    # reached through a device page table.
    paged = None
    page_keys = 65536
    if not args.no_paged and n % page_keys == 0:
        from synthetic import kv_head
        npages = n // page_keys
        pr = F.record_bytes(page_keys)
        slots = np.random.default_rng(7).permutation(hk * npages)
        pool = [torch.empty((d, pr), dtype=torch.uint8, pin_memory=True) if host else
                torch.empty((d, pr), dtype=torch.uint8, device=dev) for _ in range(hk * npages)]
        stage = torch.empty((1, d, pr), dtype=torch.uint8, device=dev)
        pages = [[None] * npages for _ in range(hk)]
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            for v, kv in enumerate(ex.map(lambda v: kv_head(wl.key, 0, v // wl.h_kv, v % wl.h_kv, n, d,
                                                            wl.outliers)[0], range(hk))):
                kd = torch.from_numpy(kv).to(dev)[None]
                for p in range(npages):
                    view = pool[int(slots[v * npages + p])]
                    F.pack_blocks(kd[:, p * page_keys:(p + 1) * page_keys], stage if host else view[None],
                                  page_keys, 0)
                    if host:
                        view.copy_(stage[0])
                    pages[v][p] = view
                del kd
        table = F.page_table(pages, residency=F.HOST_DIRECT if host else F.HBM)
        pres = F.HOST_DIRECT if host else F.HBM
        pidx = torch.empty((hq, k), dtype=torch.int32, device=dev)

        def step_paged():
            F.allocate(q, s2, budget, mode=mode, depth=depth, union_depth=uni)
            F.scan_topk_paged(table, page_keys, n, None, q, depth, uni, k, residency=pres, workspace=ws, idx=pidx)
        for _ in range(2):
            step_paged()
        torch.cuda.synchronize(dev)
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        psteps = max(3, min(args.steps, 20))
        p0.record(stream)
        for _ in range(psteps):
            step_paged()
        p1.record(stream)
        torch.cuda.synchronize(dev)
        step()
        torch.cuda.synchronize(dev)
        paged = {"page_keys": page_keys, "pages_per_kv_head": npages,
                 "step_ms": round(p0.elapsed_time(p1) / psteps, 4),
                 "contiguous_step_ms": round(step_ms, 4),
                 "same_selection_as_contiguous": bool(torch.equal(pidx, idx))}
        del pool, pages, table, stage
    out = {
        "metric": "keys scanned/s per top-k step at 1M tokens (host-resident), % of link/HBM BW",
        "value": round(keys_per_s, 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "h_kv": hk, "h_q": hq, "d": d, "n": n, "budget_bits": budget,
                   "k": k, "residency": (f"pinned host, {args.residency} over the host link" if host else "HBM"),
                   "mode": wl.mode},
        "roofline": roof,
        "cpu_baseline": cpu,
        "pages_context": PAGES_CONTEXT,
        "comparison": comparison,
        "attention": attention,
        "append": append,
        "paged": paged,
        "bytes_per_key": round(alg_bytes / (hk * n), 3),
        "link_frac_of_measured_h2d_per_step": round(alg_bytes / (step_ms * 1e-3) / 1e9 / h2d_peak, 4)
        if host else None,
        "keys_per_s_kv_heads": round(hk * n / (step_ms * 1e-3), 1),
        "tokens_per_s": round(n / (step_ms * 1e-3), 1),
        "wall_s_timed": round(wall, 3),
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
