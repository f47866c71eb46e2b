#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 linear layer (fused low-rank branch) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--sweep] [--peaks]

One step = one forward pass of the layer over one batch: the fused
activation pass (smoothing + group quantization + rank-r down-projection)
followed by the 4-bit GEMM with the low-rank slab and bias epilogue, i.e. one
``svdq_linear`` call.  Offline weight preparation runs once, before timing.
Inputs and prepared weights are resident in HBM when timing starts; every
step works on the next of several copies of (X, blob, workspace, Y) whose
total exceeds the 256 MB Infinity Cache, so no step is served from a warm
last-level cache.

Protocol: every workload is first warmed up for at least a second of
launches (and at least --warmup steps), so that the clock has settled;
then exactly --steps fused steps are timed between two synchronizations
(the headline value and ms_per_step); then --steps rounds run the fused
layer, the unfused layer and the two kernels of the fused layer one after
the other, each call timed with HIP events on its stream, and the medians,
10th and 90th percentiles of those per-call times give the kernel times,
the rooflines and the fused-versus-unfused speedup (interleaving keeps the
variants on the same clock; every call, whatever its variant, takes the next
buffer set, so none rereads what the call before it left in the cache).

Printed: one JSON line with the effective TOPS of the layer (2 M K N per
layer time), the kernel roofline of the dominant kernel (the 4-bit GEMM),
the activation kernel's HBM roofline, the fused-versus-unfused speedup, the
low-rank slab's overhead t(r) / t(r = 0), further workloads, and the CPU
oracle's throughput on a bounded row sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks (dense)
PEAK_TFLOPS = {"int4": 5000.0, "fp4": 10100.0}   # 8-bit MFMA (INT4 runs on the E4M3 one) / FP4 MFMA
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
INFINITY_CACHE = 256 << 20
HEADLINE = "c3_fc1_4608x3072x12288_fp4"
EXTRAS = ("c3_fc1_4608x3072x12288_int4,c2_qkv_4608x3072x9216_int4,c4_fc2_4608x12288x3072_int4,"
          "c4_fc2_4608x12288x3072_fp4,c5_M16384_K3072_N12288_r64")
WARM_SECONDS = 1.0


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0, help="oracle row sample (0: automatic)")
    ap.add_argument("--sweep", action="store_true", help="also time the shape sweep (one line each, to stderr)")
    ap.add_argument("--profile-only", action="store_true",
                    help="short run for profilers: warmup + steps of the fused layer, no baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="with --profile-only: first run a plain device copy of known size, the "
                         "reference that scales the HBM byte counters")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/gemm_<workload>_hbm_counters.json from two rocprofv3 --pmc "
                         "runs (FETCH_SIZE, WRITE_SIZE) of --profile-only --calibrate-copy")
    ap.add_argument("--summarize-util", nargs="+", metavar="PMC_DIR",
                    help="write profiles/gemm_<workload>_mfma_counters.json from rocprofv3 --pmc runs of "
                         "--profile-only (SQ / GRBM / TCC counters; one directory per pass)")
    ap.add_argument("--no-w4a16", dest="w4a16", action="store_false",
                    help="skip timing the weight-only layer on the modulation projection's shape")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write profiles/<kind>_<workload>_kernel_trace.txt from a rocprofv3 --kernel-trace "
                         "--stats run of --profile-only (or of --w4a16-only with --workload w4a16)")
    ap.add_argument("--norm-only", action="store_true",
                    help="time only the LayerNorm-fused layer against the separate norm (one JSON line; for profilers)")
    ap.add_argument("--summarize-sweep", metavar="SWEEP_STDERR",
                    help="write profiles/sweep_c5_int4.txt from the stderr of a --sweep run")
    ap.add_argument("--trace-kind", default="layer", choices=("layer", "w4a16", "norm"),
                    help="with --summarize-trace: which run the trace is of")
    ap.add_argument("--w4a16-only", action="store_true",
                    help="time only the weight-only layer (one JSON line; for profilers)")
    ap.add_argument("--no-norm", dest="norm", action="store_false",
                    help="skip timing the LayerNorm-fused layer against a separate norm pass")
    ap.add_argument("--lora", type=int, default=16,
                    help="also time the main workload with an extra rank-LORA branch merged in (0: skip)")
    ap.add_argument("--extra", default=EXTRAS,
                    help="comma-separated further workloads reported in the same line ('' for none)")
    ap.add_argument("--rank0", default="c3_fc1_4608x3072x12288_fp4,c2_qkv_4608x3072x9216_int4",
                    help="workloads whose rank-0 layer is timed too (slab overhead t(r) / t(0))")
    ap.add_argument("--no-peaks", dest="peaks", action="store_false",
                    help="skip the MFMA and HBM peak microbenchmarks (libsvdq_peaks)")
    return ap.parse_args()


# the sources each profiled kernel is built from: a counter summary stays
# valid while these are unchanged
KERNEL_SOURCES = {
    "fp4": ("gemm_fp4.hip", "svdq_device.h", "svdq_kernels.h"),
    "int4": ("gemm.hip", "svdq_device.h", "svdq_kernels.h"),
    "act": ("quant.hip", "svdq_device.h", "svdq_kernels.h"),
}


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a4_quantized_gemm_amd", "csrc")
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def algorithmic(cfg):
    """Algorithmic work of one layer call (per-unit figures x units)."""
    M, K, N, r = cfg.M, cfg.K, cfg.N, cfg.rank
    g = 64 if cfg.fmt == "int4" else 32
    sbytes = 2 if cfg.fmt == "int4" else 1
    q_bytes = 2 * M * K + M * K // 2 + M * (K // g) * sbytes + 2 * M * r + 2 * K * r + 4 * K
    gemm_ops = 2 * M * K * N
    slab_flops = 2 * M * r * N
    gemm_bytes = (M * K // 2 + M * (K // g) * sbytes + N * K // 2 + (K // g) * N * sbytes
                  + 2 * M * r + 2 * N * r + 2 * M * N + (4 * N if cfg.has_bias else 0))
    return dict(q_bytes=q_bytes, gemm_ops=gemm_ops, slab_flops=slab_flops, gemm_bytes=gemm_bytes)


class Rig:
    """Device buffers for one workload, replicated to defeat the Infinity Cache."""

    def __init__(self, cfg, torch, S, WL, O_bits_to_tensor, lora: int = 0):
        self.cfg = cfg
        dev = "cuda:0"
        X_bits, W_bits, b_bits = WL.make_layer(cfg)
        self.X_bits, self.W_bits, self.b_bits = X_bits, W_bits, b_bits
        X = O_bits_to_tensor(X_bits, dev)
        W = O_bits_to_tensor(W_bits, dev)
        bias = None if b_bits is None else O_bits_to_tensor(b_bits, dev)
        a = torch.empty(cfg.K, dtype=torch.float32, device=dev)
        S.svdq_act_absmax(X, a)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        layer = S.SVDQLinear.prepare(W, a, cfg.rank, cfg.fmt, cfg.alpha, bias=bias)
        torch.cuda.synchronize()
        self.prep_s = time.perf_counter() - t0
        if lora:
            # an extra low-rank branch (a LoRA update dW = A B) merged into the
            # 16-bit branch: the residual codes are shared, the slab grows
            g = torch.Generator(device="cpu").manual_seed(cfg.seed + 1)
            A = (torch.randn(cfg.K, lora, generator=g) * 0.02).to(torch.bfloat16).to(dev)
            B = (torch.randn(lora, cfg.N, generator=g) * 0.02).to(torch.bfloat16).to(dev)
            layer = layer.merge_lowrank(A, B)
            torch.cuda.synchronize()
        self.layer = layer
        del W
        M, N = cfg.M, cfg.N
        per_set = (X.numel() * 2 + layer.blob.numel() + S.svdq_workspace_bytes(layer.desc, M) + M * N * 2)
        self.nsets = max(2, -(-2 * INFINITY_CACHE // per_set))
        self.sets = []
        c_b, s_b, t_b = S.svdq_act_sizes(layer.desc, M)
        for i in range(self.nsets):
            Xi = X if i == 0 else X.clone()
            bi = layer.blob if i == 0 else layer.blob.clone()
            ws = torch.zeros(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            codes = torch.empty(c_b, dtype=torch.uint8, device=dev)
            scales = torch.empty(s_b, dtype=torch.uint8, device=dev)
            T = torch.empty(max(t_b // 2, 1), dtype=torch.bfloat16, device=dev)
            self.sets.append(dict(X=Xi, blob=bi, ws=ws, Y=Y, codes=codes, scales=scales, T=T))
        self.working_set = per_set * self.nsets
        torch.cuda.synchronize()


def pct(xs):
    """Median, 10th and 90th percentile (linear interpolation) of a list."""
    xs = sorted(xs)
    n = len(xs)

    def q(p):
        i = (n - 1) * p
        lo = int(i)
        hi = min(lo + 1, n - 1)
        return xs[lo] + (xs[hi] - xs[lo]) * (i - lo)
    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9)}


def us(d):
    return {k: v * 1e3 for k, v in d.items()}


def warm(torch, fns, min_iters, min_seconds=WARM_SECONDS):
    """Round-robin over fns (each called with the round index) until each
    ran min_iters times and min_seconds of wall time passed."""
    t0 = time.perf_counter()
    k = 0
    while True:
        for f in fns:
            f(k)
        k += 1
        if k % 8 == 0:
            torch.cuda.synchronize()
        if k >= min_iters and time.perf_counter() - t0 >= min_seconds:
            break
    torch.cuda.synchronize()


def bracket(torch, fn, steps):
    """Exactly `steps` calls between two synchronizations: ms per call from
    events at both ends (the stream's own clock) and the wall time."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for k in range(steps):
        fn(k)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - t0


GATE_CYCLES = 200_000     # a short busy kernel ahead of every timed call (see interleaved)


def interleaved(torch, variants, rounds, gate=False):
    """`rounds` rounds, each calling every variant once in order, each call
    bracketed by events on the current stream; returns the per-call times
    (ms) of every variant.  Each call gets the running call count as its
    index, so consecutive calls work on different buffer sets: no variant
    finds the previous call's inputs in the Infinity Cache (with the round
    as the index, every variant after a round's first would reread the
    buffers that the first had just pulled in).  Where a round's GPU work is long the host runs
    ahead and the events time the launches on the GPU.  For calls of a few
    microseconds (gate=True) a fixed-length busy kernel (torch.cuda._sleep)
    runs ahead of each bracket, so the host has enqueued the call's launches
    before the stream reaches them: the events then time the launches back
    to back, not the host's launch overhead."""
    evs = {name: [] for name, _ in variants}
    sleep = getattr(torch.cuda, "_sleep", None) if gate else None
    nv = len(variants)
    for k in range(rounds):
        for v, (name, fn) in enumerate(variants):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if sleep is not None:
                sleep(GATE_CYCLES)
            e0.record()
            fn(k * nv + v)
            e1.record()
            evs[name].append((e0, e1))
    torch.cuda.synchronize()
    return {name: [a.elapsed_time(b) for a, b in lst] for name, lst in evs.items()}


def layer_fns(S, rig):
    """The timed calls on a rig (each takes a call index, which picks the
    buffer set): fused layer, unfused layer, and the fused layer's two
    launches on their own (activation pass, GEMM), which read and write the
    buffers of one svdq_linear call."""
    d = rig.layer.desc
    n = rig.nsets
    M = rig.cfg.M

    def fused(k):
        s = rig.sets[k % n]
        S.svdq_linear(d, s["blob"], s["X"], s["Y"], s["ws"], S.OUT_BF16)

    def unfused(k):
        s = rig.sets[k % n]
        S.svdq_linear_unfused(d, s["blob"], s["X"], s["Y"], s["ws"], S.OUT_BF16)

    def quant(k):
        s = rig.sets[k % n]
        S.svdq_quantize_act(d, s["blob"], s["X"], s["codes"], s["scales"], s["T"] if d.rank else None, s["ws"])

    def gemm(k):
        s = rig.sets[k % n]
        S.svdq_gemm(d, s["blob"], s["codes"], s["scales"], s["T"] if d.rank else None, M, s["Y"], S.OUT_BF16,
                    s["ws"])

    return fused, unfused, quant, gemm


def time_norm(torch, S, rig, steps, warmup, eps=1e-6):
    """The layer on a LayerNorm's input: the norm fused into the activation
    pass (svdq_linear_ln) against the norm as its own pass (torch's
    layer_norm writing the bf16 normalized activations) followed by
    svdq_linear, interleaved.  Returns (fused, separate) median ms."""
    d = rig.layer.desc
    n = rig.nsets
    g = torch.Generator(device="cpu").manual_seed(rig.cfg.seed + 2)
    gamma = (1.0 + 0.1 * torch.randn(d.K, generator=g)).to(torch.bfloat16).to("cuda:0")
    beta = (0.1 * torch.randn(d.K, generator=g)).to(torch.bfloat16).to("cuda:0")
    F = torch.nn.functional

    def fused(k):
        s = rig.sets[k % n]
        S.svdq_linear_ln(d, s["blob"], s["X"], gamma, beta, eps, s["Y"], s["ws"], S.OUT_BF16)

    def separate(k):
        s = rig.sets[k % n]
        xn = F.layer_norm(s["X"], (d.K,), gamma, beta, eps)
        S.svdq_linear(d, s["blob"], xn, s["Y"], s["ws"], S.OUT_BF16)

    warm(torch, [fused, separate], warmup, 0.3)
    t = interleaved(torch, [("fused", fused), ("separate", separate)], steps)
    return statistics.median(t["fused"]), statistics.median(t["separate"])


W4A16_SHAPE = (3072, 18432)        # AdaLN modulation projection: 3072 -> 6 x 3072
W4A16_ROWS = (1, 16)                # one sample / a batch of 16


def time_w4a16(torch, S, WL, to_tensor, steps, warmup, fmts=("int4", "fp4")):
    """The weight-only 4-bit layer on the modulation projection's shape,
    against torch's bf16 matmul of the same weights and the W4A4 layer
    (rank 0) at the same M, interleaved.  Enough blob copies rotate to
    defeat the Infinity Cache.  Returns one dict per (format, M)."""
    res = []
    K, N = W4A16_SHAPE
    dev = "cuda:0"
    for fmt in fmts:
        cfg = WL.C2.with_(name="w4a16", M=64, K=K, N=N, rank=0, fmt=fmt, w_std=1 / K ** 0.5, bias_std=0.02, seed=5)
        X_bits, W_bits, b_bits = WL.make_layer(cfg)
        Xf, W, b = to_tensor(X_bits, dev), to_tensor(W_bits, dev), to_tensor(b_bits, dev)
        a = torch.empty(K, dtype=torch.float32, device=dev)
        S.svdq_act_absmax(Xf, a)
        layer = S.SVDQLinear.prepare(W, a, 0, fmt, cfg.alpha, bias=b)
        ncopy = max(2, -(-2 * INFINITY_CACHE // layer.blob.numel()))
        blobs = [layer.blob] + [layer.blob.clone() for _ in range(ncopy - 1)]
        nw = max(2, -(-2 * INFINITY_CACHE // (W.numel() * 2)))
        Ws = [W] + [W.clone() for _ in range(nw - 1)]
        wbytes = K * N // 2 + (K // (64 if fmt == "int4" else 32)) * N * (2 if fmt == "int4" else 1)
        for M in W4A16_ROWS:
            X = Xf[:M].contiguous()
            ws = layer.workspace(M)
            ws4 = layer.workspace(M)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            fns = [("w4a16", lambda k: S.svdq_linear_w4a16(layer.desc, blobs[k % ncopy], X, Y, ws, S.OUT_BF16)),
                   ("w4a4", lambda k: S.svdq_linear(layer.desc, blobs[k % ncopy], X, Y, ws4, S.OUT_BF16)),
                   ("bf16", lambda k: torch.matmul(X, Ws[k % nw]))]
            warm(torch, [f for _, f in fns], warmup, 0.3)
            t = interleaved(torch, fns, steps, gate=True)
            med = {k: statistics.median(v) * 1e3 for k, v in t.items()}
            res.append({"M": M, "K": K, "N": N, "format": fmt, "us": med["w4a16"],
                        "weight_gbs": wbytes / (med["w4a16"] * 1e-6) / 1e9,
                        "frac_hbm": wbytes / (med["w4a16"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
                        "us_bf16_matmul": med["bf16"], "us_w4a4_rank0": med["w4a4"]})
        del blobs, Ws, layer, W, Xf
        torch.cuda.empty_cache()
    return res


def cpu_baseline(rig, rows_req):
    """The oracle as it stands, on a row sample of the same workload."""
    import numpy as np
    import oracle as O
    from threadpoolctl import threadpool_info
    cfg = rig.cfg
    sec = rig.layer.blob.cpu().numpy()
    import w4a4_quantized_gemm_amd as S
    L = S.svdq_blob_layout_of(rig.layer.desc)
    r, K, N = cfg.rank, cfg.K, cfg.N
    l1t, l2t = S.blob_factors(rig.layer.desc, sec)
    factors = (O.bf16_bits_to_f64(l1t).T.copy(), O.bf16_bits_to_f64(l2t).T.copy())
    t0 = time.perf_counter()
    prep = O.prepare(rig.W_bits, O.act_absmax(rig.X_bits), alpha=cfg.alpha, rank=r, fmt=cfg.fmt,
                     bias_bits=rig.b_bits, factors=factors)
    prep_s = time.perf_counter() - t0
    rows = rows_req
    if rows <= 0:
        # size the sample for roughly 10-20 s of oracle work: time a small probe first
        probe = 64
        t0 = time.perf_counter()
        O.linear(prep, rig.X_bits[:probe], "bf16")
        dt = time.perf_counter() - t0
        rows = int(min(cfg.M, max(probe, 12.0 / max(dt, 1e-3) * probe)))
    # repeat the sample until about 10 s of oracle work have been timed
    reps, dt = 0, 0.0
    while dt < 10.0 and reps < 50:
        t0 = time.perf_counter()
        O.linear(prep, rig.X_bits[:rows], "bf16")
        dt += time.perf_counter() - t0
        reps += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    tops = 2.0 * rows * K * N * reps / dt / 1e12
    return {"value": tops, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {cfg.M} token rows of the same layer, {reps} times (oracle.linear: act "
                      f"quantization, down-projection, fp64 dequantized product, low-rank, bias); weight "
                      f"prep ({prep_s:.1f} s) excluded",
            "seconds": dt, "cpu": _cpu_model()}


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load_traffic(workload, fmt):
    """HBM traffic per launch of the GEMM kernel and of the activation pass
    from the committed rocprofv3 counter summary, each only if it was taken
    on that kernel's current sources: (gemm_bytes, act_bytes), None where
    unknown."""
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None, None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None, None
    g = d.get("traffic_bytes_per_launch") if d.get("kernel_source_hash") == kernel_source_hash(fmt) else None
    a = d.get("act_traffic_bytes_per_launch") if d.get("act_source_hash") == kernel_source_hash("act") else None
    return g, a


COPY_BYTES = 1 << 30          # the calibration copy moves this many bytes each way


def calibration_copy(torch):
    """A plain device-to-device copy of COPY_BYTES (read COPY_BYTES, write
    COPY_BYTES): the reference the HBM byte counters are scaled by."""
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def summarize_counters(fetch_dir, write_dir, cfg):
    """Per-dispatch HBM traffic of the GEMM kernel from two rocprofv3 --pmc
    runs (FETCH_SIZE, WRITE_SIZE, KiB per dispatch), each scaled by the ratio
    of the calibration copy's known bytes to what the same counter read for
    it.  Writes profiles/gemm_<workload>_hbm_counters.json."""
    import csv
    import glob

    def read(d, counter):
        rows = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return rows

    def pick(rows, pred):
        vals = [v for k, vs in rows.items() if pred(k) for v in vs]
        return vals

    is_gemm = (lambda k: k.startswith("void svdq::gemm_fp4_kernel<")) if cfg.fmt == "fp4" else \
        (lambda k: k.startswith("void svdq::gemm_kernel<"))
    # torch's copy kernel of the calibration: the largest elementwise-copy dispatch
    is_copy = lambda k: "copy" in k.lower() and not k.startswith("void svdq::")
    out = {"workload": cfg.name, "kernel_source_hash": kernel_source_hash(cfg.fmt),
           "act_source_hash": kernel_source_hash("act"), "copy_bytes": COPY_BYTES,
           "commands": [f"rocprofv3 --pmc {c} --output-format csv -d gpurun_out/pmc_{c}_{cfg.name} -o run -- "
                        f"python3 bench.py --profile-only --calibrate-copy --steps 4 --warmup 1 --workload {cfg.name}"
                        for c in ("FETCH_SIZE", "WRITE_SIZE")] +
                       [f"python3 bench.py --summarize-counters gpurun_out/pmc_FETCH_SIZE_{cfg.name} "
                        f"gpurun_out/pmc_WRITE_SIZE_{cfg.name} --workload {cfg.name}"],
           "note": "FETCH_SIZE / WRITE_SIZE per dispatch of the GEMM kernel and of the activation pass "
                   "(act_kernel + t_reduce_kernel), each scaled by the ratio of the calibration copy's known "
                   "bytes (torch copy of copy_bytes, one read and one write) to what the same counter read "
                   "for that copy"}
    total = 0.0
    act_total = 0.0
    # the fused path's activation pass: act_kernel with quantization and
    # down-projection, then the partial-T reduction
    is_act = lambda k: k.startswith("void svdq::act_kernel<") and ", true, true," in k
    is_red = lambda k: k.startswith("svdq::t_reduce_kernel")
    for name, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = read(d, counter)
        g = pick(rows, is_gemm)
        c = pick(rows, is_copy)
        if not g or not c:
            raise SystemExit(f"no {counter} rows for the GEMM or the calibration copy in {d}")
        copy_kib = max(c)                                  # the 1 GiB copy is the largest copy dispatch
        factor = COPY_BYTES / (copy_kib * 1024.0)
        gemm_kib = statistics.mean(g)
        out[name] = {"counter": counter, "gemm_kib_per_dispatch": gemm_kib, "dispatches": len(g),
                     "copy_kib": copy_kib, "scale": factor, "gemm_bytes_per_launch": gemm_kib * 1024.0 * factor}
        total += gemm_kib * 1024.0 * factor
        a, r = pick(rows, is_act), pick(rows, is_red)
        if a:
            ab = statistics.mean(a) * 1024.0 * factor
            rb = statistics.mean(r) * 1024.0 * factor if r else 0.0
            out[name].update({"act_kib_per_dispatch": statistics.mean(a), "act_bytes_per_launch": ab,
                              "t_reduce_bytes_per_launch": rb})
            act_total += ab + rb
    out["traffic_bytes_per_launch"] = total
    out["act_traffic_bytes_per_launch"] = act_total
    path = os.path.join(ROOT, "profiles", f"gemm_{cfg.name}_hbm_counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def summarize_trace(trace_dir, name, kind):
    """Per-kernel call count and average / min / max duration from a
    rocprofv3 --kernel-trace --stats run (its kernel_stats CSV), written as
    text next to the command that produced it."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(files[0])))
    w4 = kind == "w4a16"
    run = {"w4a16": "python3 bench.py --w4a16-only --steps 50 --warmup 10",
           "norm": f"python3 bench.py --norm-only --steps 50 --warmup 10 --workload {name}",
           "layer": f"python3 bench.py --profile-only --steps 50 --warmup 10 --workload {name}"}[kind]
    tag = "w4a16" if w4 else name
    lines = [f"rocprofv3 kernel-trace summary, workload {name}", "",
             "command (from the repository root, on one MI355X):",
             f"  rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/kt_{kind}_{tag} -o run -- \\",
             f"      {run}",
             f"  python3 bench.py --summarize-trace gpurun_out/kt_{kind}_{tag} --trace-kind {kind} --workload {name}", ""]
    if kind == "norm":
        lines += ["The run prepares the layer and times the layer on a LayerNorm's input, interleaved:",
                  "svdq_linear_ln (norm_stats_kernel, then act_kernel with the norm folded in, then the GEMM)",
                  "against torch's layer_norm writing the normalized bf16 activations followed by",
                  "svdq_linear (act_kernel + GEMM); warm-up runs for at least 0.3 s.  Durations in",
                  "microseconds."]
    elif w4:
        lines += ["The run prepares a 3072 x 18432 rank-0 layer per format (INT4, FP4) and times the",
                  "weight-only layer at 1 and 16 rows against torch's bf16 matmul (the Cijk_* kernels) and",
                  "the W4A4 layer at the same rows (act_kernel + gemm kernels), interleaved; warm-up runs",
                  "for at least 0.3 s, so the call counts are large.  spin_kernel is the fixed busy kernel",
                  "ahead of each timed call.  Durations in microseconds."]
    else:
        lines += ["The run prepares the layer once (dgemm/residual/wquant/...: offline weight preparation),",
                  "then times fused layer calls (act_kernel with quantization and down-projection, then the",
                  "GEMM with the slab), unfused calls (quantize-only and down-only activation passes, the",
                  "GEMM without the slab, up_kernel) and split calls (quantize_act + gemm), interleaved, so",
                  "the fused path's kernels appear twice as often.  Durations in microseconds."]
    lines += ["Every timed call works on the next of several buffer copies (together over twice the",
              "256 MB Infinity Cache), so no call finds its inputs left in the cache by the call before."]
    lines += ["", f"{'kernel':92s} {'calls':>6} {'avg':>9} {'min':>9} {'max':>9}"]
    for r in rows:
        lines.append(f"{r['Name'][:92]:92s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.1f} "
                     f"{float(r['MinNs']) / 1e3:9.1f} {float(r['MaxNs']) / 1e3:9.1f}")
    path = os.path.join(ROOT, "profiles", f"{kind}_{tag}_kernel_trace.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


SWEEP_CMD = ('python3 bench.py --steps 50 --warmup 5 --sweep --no-w4a16 --no-norm --no-peaks --extra "" '
             '--lora 0 --no-cpu-baseline --rank0 "" > gpurun_out/bench_sweep.json 2> gpurun_out/bench_sweep.err')


def summarize_sweep(path):
    """The shape sweep's per-point records (one JSON line each on stderr) as
    a table."""
    rows = [json.loads(l) for l in open(path) if l.strip().startswith("{")]
    lines = ["INT4 shape sweep: M x K -> N at ranks 16/32/64 (c2 generators), fused layer against the",
             "unfused one, times in microseconds (median of per-call HIP events, interleaved rounds).", "",
             "command (from the repository root, on one MI355X):", f"  {SWEEP_CMD}",
             "  python3 bench.py --summarize-sweep gpurun_out/bench_sweep.err", "",
             f"{'workload':30s} {'fused':>8} {'unfused':>8} {'speedup':>8} {'eff TOPS':>9} {'G us':>8} "
             f"{'G frac':>7} {'Q us':>7}"]
    for d in rows:
        lines.append(f"{d['workload']:30s} {d['us_per_layer']['median']:8.1f} {d['us_per_layer_unfused']['median']:8.1f} "
                     f"{d['fused_vs_unfused_speedup']:8.3f} {d['effective_tops']:9.0f} {d['gemm_us']['median']:8.1f} "
                     f"{d['gemm_frac_peak']:7.3f} {d['quant_us']['median']:7.1f}")
    out = os.path.join(ROOT, "profiles", "sweep_c5_int4.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


UTIL_PASSES = (
    "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_INSTS_VALU "
    "SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT",
    "GRBM_GUI_ACTIVE SQ_ACTIVE_INST_MFMA SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VMEM "
    "SQ_INST_LEVEL_VMEM SQ_INSTS_VMEM_RD SQ_ACTIVE_INST_LDS SQ_WAIT_ANY",
    "TCC_HIT_sum TCC_MISS_sum TCP_PENDING_STALL_CYCLES_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum",
)
N_XCD, N_SIMD = 8, 1024      # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_util(dirs, cfg):
    """MFMA / VALU / wait counters of the GEMM kernel and the activation pass
    from rocprofv3 --pmc passes of --profile-only (per-dispatch means), with
    the derived figures: the shader clock (GRBM_GUI_ACTIVE is summed over the
    XCDs), the share of SIMD cycles the matrix core was busy, the MFMA
    throughput and the wave time spent waiting.  Writes
    profiles/gemm_<workload>_mfma_counters.json."""
    import csv
    import glob

    kernels = {"gemm": ("void svdq::gemm_fp4_kernel<" if cfg.fmt == "fp4" else "void svdq::gemm_kernel<"),
               "act": "void svdq::act_kernel<"}
    vals = {k: {} for k in kernels}
    durs = {k: [] for k in kernels}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            seen = set()
            for r in csv.DictReader(open(f)):
                for k, pre in kernels.items():
                    name = r["Kernel_Name"]
                    if not name.startswith(pre) or (k == "act" and ", true, true," not in name):
                        continue
                    vals[k].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    key = (f, r["Dispatch_Id"])
                    if key not in seen:
                        seen.add(key)
                        durs[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    out = {"workload": cfg.name, "kernel_source_hash": kernel_source_hash(cfg.fmt),
           "act_source_hash": kernel_source_hash("act"),
           "commands": [f"rocprofv3 --pmc {p} --output-format csv -d gpurun_out/pmc_{cfg.name}_{i + 1} -o run -- "
                        f"python3 bench.py --profile-only --steps 4 --warmup 1 --workload {cfg.name}"
                        for i, p in enumerate(UTIL_PASSES)] +
                       [f"python3 bench.py --workload {cfg.name} --summarize-util " +
                        " ".join(f"gpurun_out/pmc_{cfg.name}_{i + 1}" for i in range(len(UTIL_PASSES)))],
           "note": "per-dispatch means; cycles = GRBM_GUI_ACTIVE / 8 XCDs; mfma_busy = "
                   "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x cycles); wave_wait = SQ_WAIT_INST_ANY / "
                   "SQ_WAVE_CYCLES (share of wave lifetime stalled at s_waitcnt); l2_hit = TCC_HIT / "
                   "(TCC_HIT + TCC_MISS); durations are the profiled dispatches' (counters slow them down)"}
    for k in kernels:
        v = {c: statistics.mean(x) for c, x in vals[k].items()}
        if not v:
            continue
        rec = {"counters": v, "dispatch_us": statistics.mean(durs[k]) * 1e6 if durs[k] else None}
        if "GRBM_GUI_ACTIVE" in v:
            cyc = v["GRBM_GUI_ACTIVE"] / N_XCD
            rec["cycles"] = cyc
            if durs[k] and k == "gemm":      # long enough for the counter window to match the dispatch
                rec["clock_ghz"] = cyc / statistics.mean(durs[k]) / 1e9
            if "SQ_VALU_MFMA_BUSY_CYCLES" in v:
                rec["mfma_busy"] = v["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * cyc)
            if "SQ_INSTS_VALU" in v:
                rec["valu_insts_per_simd"] = (v["SQ_INSTS_VALU"] - v.get("SQ_INSTS_MFMA", 0.0)) / N_SIMD
        if "SQ_WAIT_INST_ANY" in v and v.get("SQ_WAVE_CYCLES"):
            rec["wave_wait"] = v["SQ_WAIT_INST_ANY"] / v["SQ_WAVE_CYCLES"]
        if "TCC_HIT_sum" in v and "TCC_MISS_sum" in v:
            rec["l2_hit"] = v["TCC_HIT_sum"] / max(1.0, v["TCC_HIT_sum"] + v["TCC_MISS_sum"])
        out[k] = rec
    path = os.path.join(ROOT, "profiles", f"gemm_{cfg.name}_mfma_counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps({k: {x: out[k][x] for x in ("clock_ghz", "mfma_busy", "wave_wait", "l2_hit") if x in out[k]}
                      for k in kernels if k in out}))


PEAK_KINDS = (("fp4", 0, PEAK_TFLOPS["fp4"]), ("fp6", 1, 10100.0), ("fp8", 2, 5000.0), ("int8", 3, 5000.0),
              ("bf16", 4, PEAK_BF16_TFLOPS), ("f16", 5, 2500.0))


def measure_peaks(torch):
    """The matrix-core and HBM ceilings measured on this device with
    libsvdq_peaks (simple unobstructed loops; include/svdq_peaks.h), next to
    the datasheet figures the rooflines use."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "w4a4_quantized_gemm_amd", "libsvdq_peaks.so"))
    lib.svdq_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.svdq_peak_hbm.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    st = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(256 * cus, dtype=torch.float32, device="cuda:0")
    tops, ms = ctypes.c_double(), ctypes.c_double()
    out = {"note": "one wave per SIMD, 8 independent MFMAs per wave (32x32 shapes); 'random' operands are "
                   "pseudo-random valid codes, 'const' one repeated code; HBM: 1 GiB buffers, read-only and copy",
           "mfma": {}}
    for name, kind, datasheet in PEAK_KINDS:
        rec = {"datasheet_tops": datasheet}
        for rnd in (0, 1):
            lib.svdq_peak_mfma(kind, 2000, 0, rnd, sink.data_ptr(), ctypes.byref(tops), ctypes.byref(ms), st)
            iters = max(2000, int(2000 * 40.0 / max(ms.value, 1e-3)))       # about 40 ms
            rc = lib.svdq_peak_mfma(kind, iters, 0, rnd, sink.data_ptr(), ctypes.byref(tops), ctypes.byref(ms), st)
            if rc:
                raise RuntimeError(f"svdq_peak_mfma({name}) failed: {rc}")
            rec["random_tops" if rnd else "const_tops"] = tops.value
        rec["random_frac_of_datasheet"] = rec["random_tops"] / datasheet
        out["mfma"][name] = rec
    nbytes = 1 << 30
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    gbs = ctypes.c_double()
    for mode, key in ((0, "hbm_read_gbs"), (1, "hbm_copy_gbs")):
        lib.svdq_peak_hbm(mode, a.data_ptr(), b.data_ptr(), nbytes, ctypes.byref(gbs), ctypes.byref(ms), st)
        best = 0.0
        for _ in range(3):
            if lib.svdq_peak_hbm(mode, a.data_ptr(), b.data_ptr(), nbytes, ctypes.byref(gbs), ctypes.byref(ms), st):
                raise RuntimeError("svdq_peak_hbm failed")
            best = max(best, gbs.value)
        out[key] = best
    out["hbm_datasheet_gbs"] = PEAK_HBM_GBS
    del a, b, sink
    torch.cuda.empty_cache()
    return out


def vendor_fp4_gemm_fn(torch, cfg):
    """The vendor library's FP4 GEMM on the layer's GEMM shape, for context:
    torch._scaled_mm on MX-FP4 operands (random E2M1 codes, E8M0 scales per
    32 K, bf16 out; two operand sets alternate).  It has neither the low-rank
    slab nor the bias.  None where this torch build does not offer it."""
    if not (hasattr(torch, "float4_e2m1fn_x2") and hasattr(torch, "float8_e8m0fnu") and hasattr(torch, "_scaled_mm")):
        return None
    M, K, N = cfg.M, cfg.K, cfg.N
    try:
        gen = torch.Generator(device="cuda")
        gen.manual_seed(5)
        sets = []
        for _ in range(2):
            a = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda", generator=gen)
            b = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=gen)
            sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda")
            sb = torch.full((N, K // 32), 127, dtype=torch.uint8, device="cuda")
            sets.append((a.view(torch.float4_e2m1fn_x2), b.view(torch.float4_e2m1fn_x2),
                         sa.view(torch.float8_e8m0fnu), sb.view(torch.float8_e8m0fnu)))

        def fn(k):
            a, b, sa, sb = sets[k % 2]
            return torch._scaled_mm(a, b.t(), sa, sb, out_dtype=torch.bfloat16)
        fn(0)
        torch.cuda.synchronize()
        return fn
    except Exception as ex:                      # not supported by this build or device
        print(f"vendor FP4 GEMM unavailable: {ex!r}"[:300], file=sys.stderr)
        return None


def measure(args, cfg, torch, S, WL, to_tensor, with_cpu=False, lora=0, norm=False, rank0=False, contract=False):
    """All timings of one workload (see the module docstring)."""
    rig = Rig(cfg, torch, S, WL, to_tensor, lora)
    fused, unfused, quant, gemm = layer_fns(S, rig)
    warm(torch, [fused, unfused, quant, gemm], args.warmup)
    out = dict(rig=rig, A=algorithmic(cfg))
    if contract:
        out["ms_bracket"], out["wall"] = bracket(torch, fused, args.steps)
    variants = [("fused", fused), ("unfused", unfused), ("quant", quant), ("gemm", gemm)]
    vendor = vendor_fp4_gemm_fn(torch, cfg) if cfg.fmt == "fp4" and lora == 0 else None
    if vendor is not None:
        warm(torch, [vendor], args.warmup, 0.3)
        variants.append(("vendor_fp4_gemm", vendor))
    rig0 = None
    if rank0 and cfg.rank > 0:
        rig0 = Rig(cfg.with_(rank=0), torch, S, WL, to_tensor)
        fused0 = layer_fns(S, rig0)[0]
        warm(torch, [fused0], args.warmup, 0.3)
        variants.append(("fused_rank0", fused0))
        # the slab overhead from back-to-back calls at both ranks (per-call
        # events carry a few microseconds of their own)
        out["ms_bracket_pair"] = (bracket(torch, fused, args.steps)[0], bracket(torch, fused0, args.steps)[0])
    t = interleaved(torch, variants, args.steps)
    out["t"] = {k: pct(v) for k, v in t.items()}
    if rig0 is not None:
        out["prep_s_rank0"] = rig0.prep_s
        del rig0
    out["ms_norm"] = time_norm(torch, S, rig, args.steps, args.warmup) if norm else None
    if with_cpu:
        out["cpu"] = cpu_baseline(rig, args.cpu_rows)
    return out


def summary(r, cfg):
    """The per-workload record (times in microseconds)."""
    A, t = r["A"], r["t"]
    f, u, q, g = t["fused"]["median"], t["unfused"]["median"], t["quant"]["median"], t["gemm"]["median"]
    gt = A["gemm_ops"] / (g / 1e3) / 1e12
    rec = {"us_per_layer": us(t["fused"]), "us_per_layer_unfused": us(t["unfused"]),
           "fused_vs_unfused_speedup": u / f, "effective_tops": A["gemm_ops"] / (f / 1e3) / 1e12,
           "gemm_us": us(t["gemm"]), "gemm_tops": gt, "gemm_frac_peak": gt / PEAK_TFLOPS[cfg.fmt],
           "peak_tops": PEAK_TFLOPS[cfg.fmt], "quant_us": us(t["quant"]),
           "quant_frac_hbm": A["q_bytes"] / (q / 1e3) / 1e9 / PEAK_HBM_GBS}
    if "vendor_fp4_gemm" in t:
        # torch._scaled_mm MX-FP4 on the same M, K, N (no slab, no bias)
        rec["vendor_fp4_gemm_us"] = us(t["vendor_fp4_gemm"])
        rec["gemm_speedup_vs_vendor"] = t["vendor_fp4_gemm"]["median"] / g
    if "fused_rank0" in t:
        rec["us_per_layer_rank0"] = us(t["fused_rank0"])
        rec["slab_overhead_per_call"] = f / t["fused_rank0"]["median"]
        b_r, b_0 = r["ms_bracket_pair"]
        rec["us_per_layer_back_to_back"] = {"rank": b_r * 1e3, "rank0": b_0 * 1e3}
        rec["slab_overhead"] = b_r / b_0
    if r.get("ms_norm"):
        rec["us_per_layer_norm_fused"] = r["ms_norm"][0] * 1e3
        rec["us_per_layer_norm_separate"] = r["ms_norm"][1] * 1e3
    return rec


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world > 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the layer's multi-GPU "
                                   "sharding is a design note, not built (use --gpus 1)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, args.trace_kind)
        return
    if args.summarize_sweep:
        summarize_sweep(args.summarize_sweep)
        return
    import torch
    import w4a4_quantized_gemm_amd as S
    import workloads as WL
    import numpy as np

    def to_tensor(bits, dev):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    S.load()
    cfgs = {c.name: c for c in list(WL.CONFIGS.values()) + WL.sweep_configs()}
    cfg = cfgs[args.workload]

    if args.summarize_util:
        summarize_util(args.summarize_util, cfg)
        return

    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], cfg)
        return

    if args.norm_only:
        rig = Rig(cfg, torch, S, WL, to_tensor)
        f_ms, s_ms = time_norm(torch, S, rig, args.steps, args.warmup)
        print(json.dumps({"workload": cfg.name, "us_norm_fused": f_ms * 1e3, "us_norm_separate": s_ms * 1e3}),
              flush=True)
        return

    if args.w4a16_only:
        print(json.dumps({"w4a16_modulation": time_w4a16(torch, S, WL, to_tensor, args.steps, args.warmup)}),
              flush=True)
        return

    if args.profile_only:
        if args.calibrate_copy:
            calibration_copy(torch)
        rig = Rig(cfg, torch, S, WL, to_tensor)
        fused, unfused, quant, gemm = layer_fns(S, rig)
        warm(torch, [fused, unfused, quant, gemm], args.warmup, 0.0)
        t = interleaved(torch, [("fused", fused), ("unfused", unfused), ("quant", quant), ("gemm", gemm)],
                        args.steps)
        print(json.dumps({"workload": cfg.name, **{k: statistics.median(v) for k, v in t.items()}}), flush=True)
        return

    rank0 = set(n for n in args.rank0.split(",") if n)
    r = measure(args, cfg, torch, S, WL, to_tensor, with_cpu=not args.no_cpu_baseline, norm=args.norm,
                rank0=cfg.name in rank0, contract=True)
    A, rig = r["A"], r["rig"]
    fmt = cfg.fmt
    rec = summary(r, cfg)
    t_layer_s = r["ms_bracket"] / 1e3
    tops = A["gemm_ops"] / t_layer_s / 1e12
    g_ms, q_ms = r["t"]["gemm"]["median"], r["t"]["quant"]["median"]
    gemm_tops = A["gemm_ops"] / (g_ms / 1e3) / 1e12
    q_gbs = A["q_bytes"] / (q_ms / 1e3) / 1e9
    src_hash = kernel_source_hash(fmt)
    traffic, act_traffic = load_traffic(cfg.name, fmt)
    line = {
        "metric": "W4A4+low-rank linear effective TOPS & % MFMA peak; fused vs unfused speedup",
        "value": tops,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_bracket"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4" if fmt == "int4" else "fp4-e2m1",
        "data": "synthetic (seeded generators with the workload's shapes and outlier structure; no checkpoint)",
        "config": {"workload": cfg.name, "M": cfg.M, "K": cfg.K, "N": cfg.N, "rank": cfg.rank,
                   "format": "int4_g64_fp16" if fmt == "int4" else "fp4_e2m1_g32_e8m0",
                   "bias": cfg.has_bias, "out": "bf16"},
        "roofline": {"bound": "mfma", "achieved": gemm_tops, "peak": PEAK_TFLOPS[fmt], "unit": "TFLOP/s",
                     "frac": gemm_tops / PEAK_TFLOPS[fmt], "traffic": traffic,
                     "kernel": ("gemm_fp4_kernel (FP4 block-scaled MFMA GEMM" if fmt == "fp4" else
                                "gemm_kernel (INT4 codes on the block-scaled MFMA") + f" + rank-{cfg.rank} bf16 slab + bias)",
                     "avg_us": g_ms * 1e3, "timing": "median of per-launch HIP events"},
        "roofline_quant": {"bound": "hbm", "achieved": q_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": q_gbs / PEAK_HBM_GBS, "traffic": act_traffic,
                           "kernel": "activation pass (smooth + quantize + down-projection)",
                           "avg_us": q_ms * 1e3, "bytes": A["q_bytes"]},
        **rec,
        "slab_share_of_ops": A["slab_flops"] / A["gemm_ops"],
        "prep_seconds": rig.prep_s,
        "working_set_mb": rig.working_set / 2 ** 20,
        "buffer_sets": rig.nsets,
        "kernel_source_hash": src_hash,
        "blob_bytes": int(rig.layer.blob.numel()),
        "blob_vs_bf16_weight": rig.layer.blob.numel() / (2 * cfg.K * cfg.N),
    }
    if "cpu" in r:
        line["cpu_baseline"] = r["cpu"]
    del r, rig
    torch.cuda.empty_cache()
    extra = {}
    for name in [n for n in args.extra.split(",") if n and n != cfg.name]:
        c = cfgs[name]
        rr = measure(args, c, torch, S, WL, to_tensor, norm=False, rank0=name in rank0)
        extra[name] = summary(rr, c)
        del rr
        torch.cuda.empty_cache()
    if args.lora:
        rr = measure(args, cfg, torch, S, WL, to_tensor, lora=args.lora)
        rec_l = summary(rr, cfg)
        rec_l["rank"] = cfg.rank + args.lora
        rec_l["overhead_vs_base"] = rec_l["us_per_layer"]["median"] / line["us_per_layer"]["median"] - 1.0
        extra[f"{cfg.name}+lora{args.lora}"] = rec_l
        del rr
        torch.cuda.empty_cache()
    if extra:
        line["extra_workloads"] = extra
    if args.w4a16:
        line["w4a16_modulation"] = time_w4a16(torch, S, WL, to_tensor, min(args.steps, 200), args.warmup)
    if args.peaks:
        line["measured_peaks"] = measure_peaks(torch)
    print(json.dumps(line), flush=True)

    if args.sweep:
        for c in WL.sweep_configs():
            rr = measure(args, c, torch, S, WL, to_tensor)
            rec = {"workload": c.name, **summary(rr, c)}
            print(json.dumps(rec), file=sys.stderr, flush=True)
            del rr
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
