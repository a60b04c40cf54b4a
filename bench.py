"""Throughput of the block-quantized dequant-GEMV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--nb NB] [--warm]
                    [--no-extras] [--no-cpu]

A step is one pass of the hot path over one batch of synthetic input, with every input already
resident in HBM.  The default workload is the metric's gate: one Q4_0 GEMV at nb = 1 on the
lm_head-sized matrix W[65536 x 2048] (75.5 MB of weights, K = hidden 2048).  Weights are rotated
over copies totalling >= 1 GiB so that neither the L2 nor the 256 MB Infinity Cache can serve
them ("cold"); --warm reuses one copy (cache-assisted, labelled as such).

The K timed steps are captured once in a HIP graph and replayed under HIP events on the launch
stream (the launches run back to back, without per-launch host work); the same steps issued
eagerly from Python are reported as `ms_per_step_eager`.

Printed: ONE JSON line.  `value` is weight GB/s (weight bytes per step / time per step);
`roofline` is the dominant launch's algorithmic bytes over its average duration against the
8 TB/s HBM peak; `cpu_baseline` is the f64 oracle on this host's cores (all of them and one).
`extras` holds the other configurations of the metric measured the same way in the same run:
the nb = 16 row batch on the same matrix, the routed Q4_K experts (nb = 16), the Q8_0 QKV with
the norm prologue (nb = 16), the decode MLP step, lm_head + argmax, the warm (cache-assisted)
gate, and the attainable read rate of a plain 16-byte-load kernel on the same box.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weight GB/s and % of HBM peak for Q4 dequant-GEMV, nb=1 and nb=16"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
COLD_BYTES = 1 << 30
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_DIR = os.path.join(ROOT, "dequant_gemv_q4_amd", "csrc")
# The pages' end-to-end figure for the LFM2 WebGPU demo ("Crate inferencelayer", crate summary);
# the hardware is not given, so it is context, not a target.
PAGES_CONTEXT = {"value": 1400, "unit": "tok/s",
                 "what": "LFM2 WebGPU demo decode (Q4_0 dequant-in-GEMV), hardware not given; "
                         "context only, not comparable"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Bench:
    """One workload: rotated weight copies on the device and the launches of one step."""

    def __init__(self, name, weight_bytes, alg_bytes, dominant, step, dom, cpu, config,
                 flops=0):
        self.name, self.weight_bytes, self.alg_bytes = name, weight_bytes, alg_bytes
        self.dominant, self.step, self.dom, self.cpu, self.config = dominant, step, dom, cpu, config
        self.flops = flops


def _copies(total_bytes, warm):
    return 1 if warm else max(2, -(-COLD_BYTES // total_bytes))


def _rotated(t, R):
    return [t] + [t.clone() for _ in range(R - 1)]


def make_decode_mlp(warm):
    import torch
    import dequant_gemv_q4_amd as q
    from dequant_gemv_q4_amd import device as D
    import workloads as wl

    w = wl.decode_mlp()
    a = w.arrays
    H, I, eps = 2048, 8192, w.params["eps"]
    packed = [D.pack(q.Q4_0, a[k], *s) for k, s in (("Wg", (I, H)), ("Wu", (I, H)), ("Wd", (H, I)))]
    per_set = sum(p.numel() for p in packed)
    R = _copies(per_set, warm)
    sets = [packed] + [[p.clone() for p in packed] for _ in range(R - 1)]
    x, gamma = D.to_device(a["x"]), D.to_device(a["gamma"])
    h = torch.empty((1, I), dtype=torch.float32, device="cuda")
    y = torch.empty((1, H), dtype=torch.float32, device="cuda")
    wbytes = sum(a[k].nbytes for k in ("Wg", "Wu", "Wd"))

    def gus(i):
        Wg, Wu, _ = sets[i % R]
        q.qgemv_gus_nrm(q.Q4_0, Wg, Wu, I, H, x, gamma, eps, 1, h)

    def step(i):
        gus(i)
        q.qgemv_res(q.Q4_0, sets[i % R][2], H, I, h, x, 1, y)

    def cpu():
        import oracle
        hr = oracle.qgemv_gus_nrm(q.Q4_0, a["Wg"], a["Wu"], I, H, a["x"], a["gamma"], eps)[0]
        oracle.qgemv_res(q.Q4_0, a["Wd"], H, I, hr, a["x"])
        return wbytes

    # gate/up launch: both weight matrices, x and gamma read once, h written
    alg = a["Wg"].nbytes + a["Wu"].nbytes + 2 * H * 4 + I * 4
    cfg = {"workload": w.name, "nb": 1, "format": "q4_0", "hidden": H, "inter": I,
           "launches_per_step": 2, "weight_copies": R, "cold": not warm}
    return Bench(w.name, wbytes, alg, "qgemv_gus_nrm (q4_0, 2 x 8192x2048, nb=1)", step, gus,
                 cpu, cfg, flops=2 * 3 * H * I)


def make_lm_head(warm, nb):
    import torch
    import dequant_gemv_q4_amd as q
    from dequant_gemv_q4_amd import device as D
    import workloads as wl

    w = wl.lm_head(nb=nb)
    a = w.arrays
    Wp = D.pack(q.Q4_0, a["W"], w.N, w.K)
    R = _copies(Wp.numel(), warm)
    sets = _rotated(Wp, R)
    x = D.to_device(a["x"])
    logits = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")
    idx = torch.empty((nb,), dtype=torch.int32, device="cuda")
    ws = D.workspace(q.OP_ARGMAX, q.Q4_0, w.N, w.K, nb)

    def step(i):
        q.qgemv_argmax(q.Q4_0, sets[i % R], w.N, w.K, x, nb, logits, idx, ws)

    def cpu():
        import oracle
        oracle.qgemv_argmax(q.Q4_0, a["W"], w.N, w.K, a["x"])
        return a["W"].nbytes

    alg = a["W"].nbytes + nb * w.K * 4 + nb * w.N * 4 + nb * 4
    cfg = {"workload": w.name, "nb": nb, "format": "q4_0", "N": w.N, "K": w.K,
           "launches_per_step": 2, "weight_copies": R, "cold": not warm}
    return Bench(w.name, a["W"].nbytes, alg, f"qgemv_argmax (q4_0, {w.N}x{w.K}, nb={nb})", step,
                 step, cpu, cfg, flops=2 * nb * w.N * w.K)


def make_gemv(warm, nb, rows=65536, hidden=2048, fmt=None):
    """Plain GEMV, by default Q4_0 on the lm_head-sized matrix (65536 x 2048): the nb=1 gate
    shape; --rows / --hidden pick other sizes, fmt another block format (same seeded recipe:
    the lm_head workload's x, the format's own generator for W)."""
    import torch
    import dequant_gemv_q4_amd as q
    from dequant_gemv_q4_amd import device as D
    import workloads as wl

    fmt = q.Q4_0 if fmt is None else fmt
    w = wl.lm_head(nb=nb, vocab=rows, hidden=hidden)
    a = w.arrays
    if fmt != q.Q4_0:
        a = dict(a, W=wl.matrix(fmt, wl.rng(3, wl.T_W), w.N, w.K))
    cb = wl.iq4_codebook() if fmt in (q.IQ4_NL, q.IQ4_XS) else None
    Wp = D.pack(fmt, a["W"], w.N, w.K, codebook=cb)
    R = _copies(Wp.numel(), warm)
    sets = _rotated(Wp, R)
    x = D.to_device(a["x"])
    y = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")

    def step(i):
        q.qgemv(fmt, sets[i % R], w.N, w.K, x, nb, y)

    def cpu():
        import oracle
        if cb is not None:
            oracle.set_codebook(cb)
        oracle.qgemv(fmt, a["W"], w.N, w.K, a["x"])
        return a["W"].nbytes

    fname = wl.FMT_NAME[fmt]
    alg = a["W"].nbytes + nb * w.K * 4 + nb * w.N * 4
    name = f"{fname}_gemv_{w.N}x{w.K}_nb{nb}"
    cfg = {"workload": name, "nb": nb, "format": fname, "N": w.N, "K": w.K,
           "launches_per_step": 1, "weight_copies": R, "cold": not warm}
    return Bench(name, a["W"].nbytes, alg, f"qgemv ({fname}, {w.N}x{w.K}, nb={nb})", step, step,
                 cpu, cfg, flops=2 * nb * w.N * w.K)


def make_qkv(warm, nb):
    import torch
    import dequant_gemv_q4_amd as q
    from dequant_gemv_q4_amd import device as D
    import workloads as wl

    w = wl.qkv_q8(nb=nb)
    a = w.arrays
    Wp = D.pack(q.Q8_0, a["W"], w.N, w.K)
    R = _copies(Wp.numel(), warm)
    sets = _rotated(Wp, R)
    x, gamma = D.to_device(a["x"]), D.to_device(a["gamma"])
    y = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")

    def step(i):
        q.qgemv_nrm(q.Q8_0, sets[i % R], w.N, w.K, x, gamma, w.params["eps"], nb, y)

    def cpu():
        import oracle
        oracle.qgemv_nrm(q.Q8_0, a["W"], w.N, w.K, a["x"], a["gamma"], w.params["eps"])
        return a["W"].nbytes

    alg = a["W"].nbytes + nb * w.K * 4 + w.K * 4 + nb * w.N * 4
    cfg = {"workload": w.name, "nb": nb, "format": "q8_0", "N": w.N, "K": w.K,
           "launches_per_step": 1, "weight_copies": R, "cold": not warm}
    return Bench(w.name, a["W"].nbytes, alg, f"qgemv_nrm (q8_0, {w.N}x{w.K}, nb={nb})", step, step,
                 cpu, cfg, flops=2 * nb * w.N * w.K)


def make_qkv_attn(warm, nb, n_q_heads=12, n_kv_heads=2, head_dim=128, theta=1e6):
    """The attention-side chain of the QKV workload: norm + Q8_0 QKV GEMV + bias (one launch),
    then the per-head QK RMSNorm + RoPE in place (a second launch) at positions 1000 + r."""
    import torch
    import dequant_gemv_q4_amd as q
    from dequant_gemv_q4_amd import device as D
    import workloads as wl

    w = wl.qkv_q8(nb=nb)
    a = w.arrays
    g = wl.rng(2, 7)
    rh = head_dim // 2
    Wp = D.pack(q.Q8_0, a["W"], w.N, w.K)
    R = _copies(Wp.numel(), warm)
    sets = _rotated(Wp, R)
    x, gamma = D.to_device(a["x"]), D.to_device(a["gamma"])
    bias = D.to_device(wl.normal_f32(g, (w.N,)))
    qg, kg = D.to_device(wl.gamma_f32(g, head_dim)), D.to_device(wl.gamma_f32(g, head_dim))
    ang = (1000 + np.arange(nb))[:, None] / theta ** (2.0 * np.arange(rh)[None, :] / head_dim)
    cs, sn = D.to_device(np.cos(ang).astype(np.float32)), D.to_device(np.sin(ang).astype(np.float32))
    y = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")

    def gemv(i):
        q.qgemv_nrm_bias(q.Q8_0, sets[i % R], w.N, w.K, x, gamma, w.params["eps"], bias, nb, y)

    def step(i):
        gemv(i)
        q.qgemv_qk_norm_rope(y, nb, n_q_heads, n_kv_heads, head_dim, rh, qg, kg, 1e-6, cs, sn)

    alg = a["W"].nbytes + nb * w.K * 4 + w.K * 4 + w.N * 4 + nb * w.N * 4
    name = f"qkv_attn_q8_0_{w.N}x{w.K}_nb{nb}"
    cfg = {"workload": name, "nb": nb, "format": "q8_0", "N": w.N, "K": w.K, "bias": True,
           "qk_norm_rope": {"q_heads": n_q_heads, "kv_heads": n_kv_heads, "head_dim": head_dim},
           "launches_per_step": 2, "weight_copies": R, "cold": not warm}
    return Bench(name, a["W"].nbytes, alg, f"qgemv_nrm_bias (q8_0, {w.N}x{w.K}, nb={nb})", step,
                 gemv, lambda: 0, cfg, flops=2 * nb * w.N * w.K)


def make_moe(warm):
    import torch
    import dequant_gemv_q4_amd as q
    from dequant_gemv_q4_amd import device as D
    import workloads as wl

    w = wl.moe_q4k()
    a = w.arrays
    n_exp, topk, nb = w.params["n_exp"], w.params["topk"], w.nb
    Wp = D.pack(q.Q4_K, a["W"], n_exp * w.N, w.K)
    R = _copies(Wp.numel(), warm)
    sets = _rotated(Wp, R)
    x, ids, p = D.to_device(a["x"]), D.to_device(a["ids"]), D.to_device(a["p"])
    y = torch.empty((nb, w.N), dtype=torch.float32, device="cuda")
    ws = D.workspace(q.OP_MOE, q.Q4_K, w.N, w.K, nb, n_exp, topk)
    touched = len(np.unique(a["ids"]))
    per_exp = a["W"].nbytes // n_exp

    def step(i):
        q.qgemv_moe(q.Q4_K, sets[i % R], n_exp, w.N, w.K, x, nb, ids, p, topk, y, ws)

    def cpu():
        import oracle
        oracle.qgemv_moe(q.Q4_K, a["W"], n_exp, w.N, w.K, a["x"], a["ids"], a["p"])
        return touched * per_exp

    wbytes = touched * per_exp
    alg = wbytes + nb * w.K * 4 + nb * w.N * 4 + 2 * nb * topk * w.N * 4 + 2 * nb * topk * 4
    cfg = {"workload": w.name, "nb": nb, "format": "q4_k", "N": w.N, "K": w.K, "n_exp": n_exp,
           "topk": topk, "experts_touched": touched, "launches_per_step": 2,
           "weight_copies": R, "cold": not warm}
    return Bench(w.name, wbytes, alg, f"qgemv_moe (q4_k, {touched} of {n_exp} x {w.N}x{w.K}, nb={nb})",
                 step, step, cpu, cfg, flops=2 * nb * topk * w.N * w.K)


def make_gemm(warm, M=512, N=8192, K=2048, fmt=None):
    """Wide row batch (a prefill chunk of M rows): qgemm on an N x K matrix (default the decode
    MLP's Q4_0 gate matrix, 8192 x 2048, with a 512-row chunk).  Compute-bound at these M: the
    roofline is the f16 MFMA peak (2.5 PFLOP/s dense) over 2 M N K flops."""
    import torch
    import dequant_gemv_q4_amd as q
    from dequant_gemv_q4_amd import device as D
    import workloads as wl

    fmt = q.Q4_0 if fmt is None else fmt
    g = wl.rng(5, wl.T_W)
    W = wl.matrix(fmt, g, N, K)
    x = wl.normal_f32(wl.rng(5, wl.T_X), (M, K))
    Wp = D.pack(fmt, W, N, K)
    R = _copies(Wp.numel(), warm)
    sets = _rotated(Wp, R)
    xd = D.to_device(x)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(q.qgemm_workspace_bytes(fmt, N, K, M), dtype=torch.uint8, device="cuda")

    def step(i):
        q.qgemm(fmt, sets[i % R], N, K, xd, M, y, ws)

    def cpu():
        import oracle
        oracle.gemv(fmt, W, N, K, x)
        return W.nbytes

    fname = wl.FMT_NAME[fmt]
    name = f"{fname}_gemm_{N}x{K}_m{M}"
    alg = W.nbytes + M * K * 4 + M * N * 4
    cfg = {"workload": name, "M": M, "format": fname, "N": N, "K": K, "launches_per_step": 2,
           "weight_copies": R, "cold": not warm}
    return Bench(name, W.nbytes, alg, f"qgemm ({fname}, {N}x{K}, M={M})", step, step, cpu, cfg,
                 flops=2 * M * N * K)


def make_read(warm, nbytes=75497472, shape=(256, 1024), chunked=False):
    """The attainable read rate: the plain 16-byte-load read kernel (libqgbw.so) over the same
    number of bytes as the gate's weights, rotated over >= 1 GiB like the GEMV, at one launch
    shape, in grid-stride order or one contiguous chunk per workgroup."""
    import torch
    from dequant_gemv_q4_amd import bwref

    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(7)
    R = _copies(nbytes, warm)
    sets = _rotated(buf, R)
    grid, threads = shape
    out = torch.empty(grid * threads // 64, dtype=torch.int32, device="cuda")

    def step(i):
        bwref.read(sets[i % R], nbytes, out, grid, threads, chunked)

    order = "chunked" if chunked else "grid_stride"
    name = f"read_{nbytes}B_{grid}x{threads}_{order}"
    cfg = {"workload": name, "bytes": nbytes, "grid": grid, "threads": threads, "order": order,
           "launches_per_step": 1, "weight_copies": R, "cold": not warm}
    return Bench(name, nbytes, nbytes, f"plain 16-byte read ({grid} x {threads}, {order})", step,
                 step, lambda: 0, cfg)


def make_copy(warm):
    """A plain device-to-device copy of 256 MiB (torch's copy kernel): the known-size kernel that
    calibrates the HBM byte counters."""
    import torch

    n = 256 << 20
    srcs = [torch.empty(n, dtype=torch.uint8, device="cuda").fill_(i + 1) for i in range(4)]
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")

    def step(i):
        dst.copy_(srcs[i % len(srcs)])

    cfg = {"workload": "device_copy_256MiB", "bytes_read": n, "bytes_written": n,
           "launches_per_step": 1, "weight_copies": len(srcs), "cold": True}
    return Bench(cfg["workload"], n, 2 * n, "torch copy_ (256 MiB)", step, step, lambda: 0, cfg)


def time_loop(fn, start, count, torch):
    """Eager: `count` calls of fn issued from Python, HIP events around them (ms per call)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for i in range(count):
        fn(start + i)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / count   # ms per call


def time_graph(fn, start, count, torch):
    """The same `count` calls captured once in a HIP graph (the launches are recorded, not run),
    then one replay timed with HIP events on the replay stream (ms per call).  A first replay,
    untimed, warms the graph."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(count):
            fn(start + i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / count


def stored_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed PMC summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    if rec.get("kernel_sha256") != kernel_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


def kernel_sha256():
    """One hash over every kernel and library source: a counter reading is only valid for the
    code it was taken on."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_DIR)):
        if name.endswith((".hip", ".h", ".cpp")) and name != "bw_read.hip":
            h.update(name.encode())
            h.update(open(os.path.join(KERNEL_DIR, name), "rb").read())
    return h.hexdigest()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(b, reps=5):
    """The f64 oracle on the same workload: 1 warm-up, then the median of `reps` full steps, with
    all host threads and again with one."""
    import oracle
    oracle.build(force=False)
    out = {}
    all_threads = oracle.threads()
    for label, n in (("all", all_threads), ("one", 1)):
        used = oracle.set_threads(n)
        b.cpu()
        ts = []
        moved = 0
        for _ in range(reps):
            t0 = time.perf_counter()
            moved = b.cpu()
            ts.append(time.perf_counter() - t0)
        med = statistics.median(ts)
        out[label] = {"threads": used, "median_s": med, "gbps": moved / med / 1e9}
    oracle.set_threads(all_threads)
    return {"value": round(out["all"]["gbps"], 4), "unit": "GB/s", "cores": out["all"]["threads"],
            "kind": "oracle",
            "sample": f"full steps of {b.name} in the f64 oracle, median of {reps} after one "
                      f"warm-up (OpenMP over output rows)",
            "ms_median": round(out["all"]["median_s"] * 1e3, 3),
            "value_1thread": round(out["one"]["gbps"], 4),
            "ms_median_1thread": round(out["one"]["median_s"] * 1e3, 3),
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "label": "f64 oracle (correctness reference, not a tuned CPU GEMV)"}


def measure(b, steps, warmup, eager, torch):
    """(ms per step graph-replayed, ms per step eager, ms per dominant launch)."""
    for i in range(warmup):
        b.step(i)
    torch.cuda.synchronize()
    ms_eager = time_loop(b.step, warmup, steps, torch)
    ms_step = ms_eager if eager else time_graph(b.step, warmup, steps, torch)
    if b.dom is b.step:
        ms_dom = ms_step
    else:
        for i in range(warmup):
            b.dom(i)
        ms_dom = (time_loop if eager else time_graph)(b.dom, warmup, steps, torch)
    return ms_step, ms_eager, ms_dom


def summary(b, ms_step, ms_eager, ms_dom):
    value = b.weight_bytes / (ms_step * 1e-3) / 1e9
    achieved = b.alg_bytes / (ms_dom * 1e-3) / 1e9
    out = {"workload": b.name, "value": round(value, 2), "unit": "GB/s",
           "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
           "us_per_step": round(ms_step * 1e3, 3), "us_per_step_eager": round(ms_eager * 1e3, 3),
           "roofline": {"bound": "hbm", "kernel": b.dominant, "achieved": round(achieved, 2),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(achieved / HBM_PEAK_GBPS, 4),
                        "traffic": stored_traffic(b.name), "alg_bytes_per_launch": b.alg_bytes,
                        "us_per_launch": round(ms_dom * 1e3, 3)},
           "config": b.config}
    if b.flops:
        out["tflops"] = round(b.flops / (ms_step * 1e-3) / 1e12, 3)
        if "M" in b.config:    # wide row batch: bound by the matrix cores, not by HBM
            out["roofline"].update({
                "bound": "mfma", "achieved": round(b.flops / (ms_dom * 1e-3) / 1e12, 2),
                "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(b.flops / (ms_dom * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                "hbm_gbps": round(achieved, 2)})
    return out


def run_extra(name, factory, steps, warmup, torch):
    log(f"bench: extra {name}")
    b = factory()
    ms_step, ms_eager, ms_dom = measure(b, steps, warmup, False, torch)
    out = summary(b, ms_step, ms_eager, ms_dom)
    log(f"bench:   {out['us_per_step']:.2f} us/step, {out['value']:.0f} GB/s "
        f"({out['pct_of_hbm_peak']:.1f}% of 8 TB/s)")
    del b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gemv",
                    choices=["gemv", "decode_mlp", "lm_head", "qkv", "moe", "gemm", "read", "copy"])
    ap.add_argument("--nb", type=int, default=None)
    ap.add_argument("--rows", type=int, default=65536, help="gemv workload: output rows")
    ap.add_argument("--hidden", type=int, default=2048, help="gemv workload: reduction length")
    ap.add_argument("--format", default="q4_0",
                    choices=["q4_0", "q5_0", "q8_0", "q4_k", "q5_k", "q6_k", "iq4_nl", "iq4_xs",
                             "q1_0", "aq4"],
                    help="gemv / gemm workloads: block format of W (gemm: q4_0, q8_0, q1_0)")
    ap.add_argument("--warm", action="store_true", help="reuse one weight copy (cache-assisted)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--extra-steps", type=int, default=200)
    ap.add_argument("--eager", action="store_true",
                    help="time launches issued from Python instead of one HIP graph replay")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (every entry "
              "point would shard by output rows, one GPU's share being the single-GPU kernel "
              "at N / G rows)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dequant_gemv_q4_amd as q

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    q.lib()
    torch.cuda.set_device(0)

    wl_name = args.workload
    import workloads as wlm
    fmt = {v: k for k, v in wlm.FMT_NAME.items()}[args.format]
    if wl_name == "decode_mlp":
        b = make_decode_mlp(args.warm)
    elif wl_name == "lm_head":
        b = make_lm_head(args.warm, args.nb or 1)
    elif wl_name == "gemv":
        b = make_gemv(args.warm, args.nb or 1, args.rows, args.hidden, fmt=fmt)
    elif wl_name == "qkv":
        b = make_qkv(args.warm, args.nb or 16)
    elif wl_name == "gemm":
        b = make_gemm(args.warm, args.nb or 512, fmt=fmt)
    elif wl_name == "read":
        b = make_read(args.warm)
        args.no_cpu = True
    elif wl_name == "copy":
        b = make_copy(args.warm)
        args.no_cpu = True
    else:
        b = make_moe(args.warm)
    log(f"bench: {b.name}, copies={b.config['weight_copies']}, warmup={args.warmup}, steps={args.steps}")

    ms_step, ms_eager, ms_dom = measure(b, args.steps, args.warmup, args.eager, torch)
    log(f"bench: {ms_step * 1e3:.2f} us per step ({ms_eager * 1e3:.2f} us issued eagerly), "
        f"dominant launch {ms_dom * 1e3:.2f} us")
    s = summary(b, ms_step, ms_eager, ms_dom)
    out = {
        "metric": METRIC,
        "value": s["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "ms_per_step_eager": round(ms_eager, 6),
        "timing": "eager" if args.eager else "hip_graph",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32",
        "data": "synthetic",
        "pct_of_hbm_peak": s["pct_of_hbm_peak"],
        "config": b.config,
        "roofline": s["roofline"],
        "cpu_baseline": None,
        "pages_context": PAGES_CONTEXT,
        "host_loadavg": list(os.getloadavg()),
    }
    if "tflops" in s:
        out["tflops"] = s["tflops"]

    cpu_b = Bench(b.name, 0, 0, "", None, None, b.cpu, {})   # the oracle needs host arrays only
    if (not args.no_extras and wl_name == "gemv" and not args.warm and args.nb in (None, 1) and
            args.format == "q4_0"):
        del b
        torch.cuda.empty_cache()
        es, ew = args.extra_steps, min(args.warmup, 20)
        extras = {}
        extras["gemv_nb16"] = run_extra("gemv nb=16", lambda: make_gemv(False, 16), es, ew, torch)
        extras["moe_q4k_nb16"] = run_extra("moe", lambda: make_moe(False), es, ew, torch)
        extras["qkv_q8_nb16"] = run_extra("qkv nb=16", lambda: make_qkv(False, 16), es, ew, torch)
        extras["decode_mlp"] = run_extra("decode mlp", lambda: make_decode_mlp(False), es, ew, torch)
        extras["qkv_attn_nb1"] = run_extra("qkv + bias + qk norm + rope",
                                           lambda: make_qkv_attn(False, 1), es, ew, torch)
        extras["lm_head_nb1"] = run_extra("lm_head", lambda: make_lm_head(False, 1), es, ew, torch)
        extras["lm_head_nb4"] = run_extra("lm_head nb=4", lambda: make_lm_head(False, 4), es, ew,
                                          torch)
        # the gate's GEMV over shorter matrices (K = 2048): where the launch ramp takes over
        for n in (2048, 8192, 16384, 32768):
            extras[f"gemv_q4_0_n{n}"] = run_extra(f"gemv N={n}",
                                                  lambda n=n: make_gemv(False, 1, n, 2048),
                                                  es, ew, torch)
        import dequant_gemv_q4_amd as qq
        for f, nm in ((qq.Q8_0, "q8_0"), (qq.Q4_K, "q4_k"), (qq.Q5_0, "q5_0"), (qq.Q5_K, "q5_k"),
                      (qq.Q6_K, "q6_k"), (qq.IQ4_NL, "iq4_nl"), (qq.IQ4_XS, "iq4_xs"),
                      (qq.Q1_0, "q1_0"), (qq.AQ4, "aq4")):
            extras[f"{nm}_gemv_nb1"] = run_extra(f"{nm} gemv", lambda f=f: make_gemv(False, 1, fmt=f),
                                                 es, ew, torch)
        for M in (64, 512, 2048):
            extras[f"gemm_q4_0_m{M}"] = run_extra(f"gemm M={M}", lambda M=M: make_gemm(False, M),
                                                  min(es, 50), 5, torch)
        extras["gemm_q1_0_m2048"] = run_extra("gemm q1_0 M=2048",
                                              lambda: make_gemm(False, 2048, fmt=q.Q1_0),
                                              min(es, 50), 5, torch)
        w = run_extra("gemv warm", lambda: make_gemv(True, 1), es, ew, torch)
        w["label"] = "cache-assisted: one weight copy reused, served in part by the 256 MB MALL"
        extras["gemv_nb1_warm"] = w
        # attainable: the plain read kernel over the gate's bytes at a few launch shapes and
        # both orders (best kept)
        best = None
        for chunked in (False, True):
            for shape in ((256, 1024), (512, 1024), (1024, 512), (2048, 256)):
                r = run_extra(f"read {shape}{' chunked' if chunked else ''}",
                              lambda: make_read(False, shape=shape, chunked=chunked), es, ew, torch)
                if best is None or r["value"] > best["value"]:
                    best = r
        best["label"] = ("plain 16-byte non-temporal read of the same bytes, best launch shape "
                         "and order")
        extras["read_attainable"] = best
        out["attainable_read_gbps"] = best["value"]
        out["pct_of_attainable"] = round(100 * out["value"] / best["value"], 2)
        out["extras"] = extras
    if not args.no_cpu:
        log("bench: timing the f64 oracle on this host")
        out["cpu_baseline"] = cpu_baseline(cpu_b)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
