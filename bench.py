#!/usr/bin/env python3
"""Benchmark of the SVDQuant W4A4 linear layer (fused low-rank branch) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--sweep]

One step = one forward pass of the layer over one batch: the fused
activation pass (smoothing + group quantization + rank-r down-projection)
followed by the 4-bit GEMM with the low-rank slab and bias epilogue, i.e. one
``svdq_linear`` call.  Offline weight preparation runs once, before timing.
Inputs and prepared weights are resident in HBM when timing starts; every
step works on the next of several copies of (X, blob, workspace, Y) whose
total exceeds the 256 MB Infinity Cache, so no step is served from a warm
last-level cache.

Printed: one JSON line with the effective TOPS of the layer (2 M K N per
layer time), the kernel roofline of the dominant kernel (the 4-bit GEMM,
timed with HIP events on the stream it is launched on), the activation
kernel's HBM roofline, the fused-versus-unfused speedup, and the CPU oracle's
throughput on a bounded row sample of the same workload.
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


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2_qkv_4608x3072x9216_int4")
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
    ap.add_argument("--no-norm", dest="norm", action="store_false",
                    help="skip timing the LayerNorm-fused layer against a separate norm pass")
    ap.add_argument("--lora", type=int, default=16,
                    help="also time the main workload with an extra rank-LORA branch merged in (0: skip)")
    ap.add_argument("--extra", default="c3_fc1_4608x3072x12288_fp4",
                    help="comma-separated further workloads reported in the same line ('' for none)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4a4_quantized_gemm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h", ".cpp")):
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
            ws = torch.empty(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            codes = torch.empty(c_b, dtype=torch.uint8, device=dev)
            scales = torch.empty(s_b, dtype=torch.uint8, device=dev)
            T = torch.empty(max(t_b // 2, 1), dtype=torch.bfloat16, device=dev)
            self.sets.append(dict(X=Xi, blob=bi, ws=ws, Y=Y, codes=codes, scales=scales, T=T))
        self.working_set = per_set * self.nsets
        torch.cuda.synchronize()


def time_fused(torch, S, rig, steps, warmup, unfused=False):
    d = rig.layer.desc
    fn = S.svdq_linear_unfused if unfused else S.svdq_linear
    n = rig.nsets
    for k in range(warmup):
        s = rig.sets[k % n]
        fn(d, s["blob"], s["X"], s["Y"], s["ws"], S.OUT_BF16)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for k in range(steps):
        s = rig.sets[k % n]
        fn(d, s["blob"], s["X"], s["Y"], s["ws"], S.OUT_BF16)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_norm(torch, S, rig, steps, warmup, eps=1e-6):
    """The layer on a LayerNorm's input: the norm fused into the activation
    pass (svdq_linear_ln) against the norm as its own pass (torch's
    layer_norm writing the bf16 normalized activations) followed by
    svdq_linear.  Returns (fused ms, separate ms) per step."""
    d = rig.layer.desc
    n = rig.nsets
    g = torch.Generator(device="cpu").manual_seed(rig.cfg.seed + 2)
    gamma = (1.0 + 0.1 * torch.randn(d.K, generator=g)).to(torch.bfloat16).to("cuda:0")
    beta = (0.1 * torch.randn(d.K, generator=g)).to(torch.bfloat16).to("cuda:0")
    F = torch.nn.functional

    def fused(s):
        S.svdq_linear_ln(d, s["blob"], s["X"], gamma, beta, eps, s["Y"], s["ws"], S.OUT_BF16)

    def separate(s):
        xn = F.layer_norm(s["X"], (d.K,), gamma, beta, eps)
        S.svdq_linear(d, s["blob"], xn, s["Y"], s["ws"], S.OUT_BF16)

    out = []
    for fn in (fused, separate):
        for k in range(warmup):
            fn(rig.sets[k % n])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in range(steps):
            fn(rig.sets[k % n])
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    return out[0], out[1]


W4A16_SHAPES = ((1, 3072, 18432), (16, 3072, 18432))   # AdaLN modulation projection: one sample / a batch of 16


def time_w4a16(torch, S, WL, to_tensor, steps, warmup, fmt="int4"):
    """The weight-only 4-bit layer on the modulation projection's shape
    (3072 -> 6 x 3072), against torch's bf16 matmul of the same weights and
    the W4A4 layer (rank 0) at the same M.  Enough blob copies rotate to
    defeat the Infinity Cache.  Returns one dict per M."""
    res = []
    for M, K, N in W4A16_SHAPES:
        cfg = WL.C2.with_(name="w4a16", M=64, K=K, N=N, rank=0, fmt=fmt, w_std=1 / K ** 0.5, bias_std=0.02, seed=5)
        X_bits, W_bits, b_bits = WL.make_layer(cfg)
        dev = "cuda:0"
        Xf, W, b = to_tensor(X_bits, dev), to_tensor(W_bits, dev), to_tensor(b_bits, dev)
        a = torch.empty(K, dtype=torch.float32, device=dev)
        S.svdq_act_absmax(Xf, a)
        layer = S.SVDQLinear.prepare(W, a, 0, fmt, cfg.alpha, bias=b)
        X = Xf[:M].contiguous()
        ncopy = max(2, -(-2 * INFINITY_CACHE // layer.blob.numel()))
        blobs = [layer.blob] + [layer.blob.clone() for _ in range(ncopy - 1)]
        nw = max(2, -(-2 * INFINITY_CACHE // (W.numel() * 2)))
        Ws = [W] + [W.clone() for _ in range(nw - 1)]
        ws = torch.empty(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def run(fn, n):
            for k in range(warmup):
                fn(k % n)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for k in range(steps):
                fn(k % n)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / steps * 1e3

        us = run(lambda i: S.svdq_linear_w4a16(layer.desc, blobs[i], X, Y, ws, S.OUT_BF16), len(blobs))
        ws4 = torch.empty(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev)
        us_w4a4 = run(lambda i: S.svdq_linear(layer.desc, blobs[i], X, Y, ws4, S.OUT_BF16), len(blobs))
        us_bf16 = run(lambda i: torch.matmul(X, Ws[i]), len(Ws))
        wbytes = K * N // 2 + (K // (64 if fmt == "int4" else 32)) * N * (2 if fmt == "int4" else 1)
        res.append({"M": M, "K": K, "N": N, "format": fmt, "us": us, "weight_gbs": wbytes / (us * 1e-6) / 1e9,
                    "frac_hbm": wbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, "us_bf16_matmul": us_bf16,
                    "us_w4a4_rank0": us_w4a4})
        del blobs, Ws, layer, W, Xf
        torch.cuda.empty_cache()
    return res


def time_kernels(torch, S, rig, steps, warmup):
    """Per-kernel durations with events on the launch stream: the activation
    pass (svdq_quantize_act) and the GEMM (svdq_gemm), which together are the
    same two launches as svdq_linear."""
    d = rig.layer.desc
    n = rig.nsets
    M = rig.cfg.M

    def one(s, evs=None):
        if evs:
            evs[0].record()
        S.svdq_quantize_act(d, s["blob"], s["X"], s["codes"], s["scales"], s["T"] if d.rank else None, s["ws"])
        if evs:
            evs[1].record()
        S.svdq_gemm(d, s["blob"], s["codes"], s["scales"], s["T"] if d.rank else None, M, s["Y"], S.OUT_BF16)
        if evs:
            evs[2].record()

    for k in range(warmup):
        one(rig.sets[k % n])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        one(rig.sets[k % n], evs[k])
    torch.cuda.synchronize()
    tq = [e[0].elapsed_time(e[1]) for e in evs]
    tg = [e[1].elapsed_time(e[2]) for e in evs]
    return tq, tg


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


def load_traffic(workload, src_hash):
    """HBM traffic per launch of the GEMM kernel and of the activation pass
    from the committed rocprofv3 counter summary, if it was taken on the
    current kernel sources: (gemm_bytes, act_bytes), None where unknown."""
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None, None
    try:
        d = json.load(open(path))
    except (OSError, ValueError):
        return None, None
    if d.get("kernel_source_hash") != src_hash:
        return None, None
    return d.get("traffic_bytes_per_launch"), d.get("act_traffic_bytes_per_launch")


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


def summarize_counters(fetch_dir, write_dir, cfg, src_hash):
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
    out = {"workload": cfg.name, "kernel_source_hash": src_hash, "copy_bytes": COPY_BYTES,
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


UTIL_PASSES = (
    "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_INSTS_VALU "
    "SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_LDS_BANK_CONFLICT",
    "GRBM_GUI_ACTIVE SQ_ACTIVE_INST_MFMA SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_VMEM "
    "SQ_INST_LEVEL_VMEM SQ_INSTS_VMEM_RD SQ_ACTIVE_INST_LDS SQ_WAIT_ANY",
    "TCC_HIT_sum TCC_MISS_sum TCP_PENDING_STALL_CYCLES_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum",
)
N_XCD, N_SIMD = 8, 1024      # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_util(dirs, cfg, src_hash):
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
    out = {"workload": cfg.name, "kernel_source_hash": src_hash,
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


def run_config(args, cfg, torch, S, WL, to_tensor, with_cpu, lora=0, norm=False):
    rig = Rig(cfg, torch, S, WL, to_tensor, lora)
    ms_fused, wall = time_fused(torch, S, rig, args.steps, args.warmup)
    tq, tg = time_kernels(torch, S, rig, args.steps, args.warmup)
    ms_unfused, _ = time_fused(torch, S, rig, args.steps, args.warmup, unfused=True)
    ms_norm = time_norm(torch, S, rig, args.steps, args.warmup) if norm else None
    A = algorithmic(cfg)
    tq_ms, tg_ms = statistics.mean(tq), statistics.mean(tg)
    out = dict(rig=rig, ms_fused=ms_fused, wall=wall, ms_unfused=ms_unfused, tq=tq, tg=tg, A=A,
               tq_ms=tq_ms, tg_ms=tg_ms, ms_norm=ms_norm)
    if with_cpu:
        out["cpu"] = cpu_baseline(rig, args.cpu_rows)
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world > 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the layer's multi-GPU "
                                   "sharding is a design note, not built (use --gpus 1)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
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
        summarize_util(args.summarize_util, cfg, kernel_source_hash())
        return

    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.summarize_counters[1], cfg, kernel_source_hash())
        return

    if args.profile_only:
        if args.calibrate_copy:
            calibration_copy(torch)
        rig = Rig(cfg, torch, S, WL, to_tensor)
        ms, _ = time_fused(torch, S, rig, args.steps, args.warmup)
        time_fused(torch, S, rig, args.steps, args.warmup, unfused=True)
        tq, tg = time_kernels(torch, S, rig, args.steps, args.warmup)
        print(json.dumps({"workload": cfg.name, "ms_per_step": ms, "quant_ms": statistics.mean(tq),
                          "gemm_ms": statistics.mean(tg)}), flush=True)
        return

    r = run_config(args, cfg, torch, S, WL, to_tensor, with_cpu=not args.no_cpu_baseline, norm=args.norm)
    A, rig = r["A"], r["rig"]
    fmt = cfg.fmt
    t_layer_s = r["ms_fused"] / 1e3
    tops = A["gemm_ops"] / t_layer_s / 1e12
    gemm_tops = A["gemm_ops"] / (r["tg_ms"] / 1e3) / 1e12
    q_gbs = A["q_bytes"] / (r["tq_ms"] / 1e3) / 1e9
    src_hash = kernel_source_hash()
    traffic, act_traffic = load_traffic(cfg.name, src_hash)
    line = {
        "metric": "W4A4+low-rank linear effective TOPS & % MFMA peak; fused vs unfused speedup",
        "value": tops,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_fused"],
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
                                "gemm_kernel (INT4 codes on the E4M3 block-scaled MFMA") + f" + rank-{cfg.rank} bf16 slab + bias)",
                     "avg_us": r["tg_ms"] * 1e3},
        "roofline_quant": {"bound": "hbm", "achieved": q_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": q_gbs / PEAK_HBM_GBS, "traffic": act_traffic,
                           "kernel": "act_kernel (smooth + quantize + down-proj) + t_reduce_kernel",
                           "avg_us": r["tq_ms"] * 1e3, "bytes": A["q_bytes"]},
        "us_per_layer": r["ms_fused"] * 1e3,
        "us_per_layer_unfused": r["ms_unfused"] * 1e3,
        "fused_vs_unfused_speedup": r["ms_unfused"] / r["ms_fused"],
        "gemm_effective_tops": gemm_tops,
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
    if r.get("ms_norm"):
        nf, ns = r["ms_norm"]
        line["layernorm_fused"] = {"us_per_layer_norm_fused": nf * 1e3, "us_per_layer_norm_separate": ns * 1e3,
                                   "speedup": ns / nf,
                                   "note": "svdq_linear_ln on the norm's input against torch layer_norm (bf16 "
                                           "out) followed by svdq_linear"}
    extra = {}
    for name in [n for n in args.extra.split(",") if n and n != cfg.name]:
        c = cfgs[name]
        rr = run_config(args, c, torch, S, WL, to_tensor, with_cpu=False, norm=args.norm)
        Ax = rr["A"]
        gt = Ax["gemm_ops"] / (rr["tg_ms"] / 1e3) / 1e12
        extra[name] = {"us_per_layer": rr["ms_fused"] * 1e3, "us_per_layer_unfused": rr["ms_unfused"] * 1e3,
                       "fused_vs_unfused_speedup": rr["ms_unfused"] / rr["ms_fused"],
                       "effective_tops": Ax["gemm_ops"] / (rr["ms_fused"] / 1e3) / 1e12,
                       "gemm_us": rr["tg_ms"] * 1e3, "gemm_tops": gt, "gemm_frac_peak": gt / PEAK_TFLOPS[c.fmt],
                       "peak_tops": PEAK_TFLOPS[c.fmt], "quant_us": rr["tq_ms"] * 1e3,
                       "quant_frac_hbm": Ax["q_bytes"] / (rr["tq_ms"] / 1e3) / 1e9 / PEAK_HBM_GBS}
        if rr.get("ms_norm"):
            extra[name]["us_per_layer_norm_fused"] = rr["ms_norm"][0] * 1e3
            extra[name]["us_per_layer_norm_separate"] = rr["ms_norm"][1] * 1e3
        del rr
        torch.cuda.empty_cache()
    if args.w4a16:
        line["w4a16_modulation"] = time_w4a16(torch, S, WL, to_tensor, min(args.steps, 200), args.warmup)
    if args.lora:
        rr = run_config(args, cfg, torch, S, WL, to_tensor, with_cpu=False, lora=args.lora)
        extra[f"{cfg.name}+lora{args.lora}"] = {
            "rank": cfg.rank + args.lora, "us_per_layer": rr["ms_fused"] * 1e3,
            "us_per_layer_unfused": rr["ms_unfused"] * 1e3,
            "fused_vs_unfused_speedup": rr["ms_unfused"] / rr["ms_fused"],
            "overhead_vs_base": rr["ms_fused"] / r["ms_fused"] - 1.0, "gemm_us": rr["tg_ms"] * 1e3,
            "quant_us": rr["tq_ms"] * 1e3}
        del rr
        torch.cuda.empty_cache()
    if extra:
        line["extra_workloads"] = extra
    print(json.dumps(line), flush=True)

    if args.sweep:
        for c in WL.sweep_configs():
            rr = run_config(args, c, torch, S, WL, to_tensor, with_cpu=False)
            A = rr["A"]
            rec = {"workload": c.name, "us_per_layer": rr["ms_fused"] * 1e3,
                   "us_unfused": rr["ms_unfused"] * 1e3, "speedup": rr["ms_unfused"] / rr["ms_fused"],
                   "effective_tops": A["gemm_ops"] / (rr["ms_fused"] / 1e3) / 1e12,
                   "gemm_frac_int8_peak": A["gemm_ops"] / (rr["tg_ms"] / 1e3) / 1e12 / PEAK_TFLOPS["int4"],
                   "quant_gbs": A["q_bytes"] / (rr["tq_ms"] / 1e3) / 1e9}
            print(json.dumps(rec), file=sys.stderr, flush=True)
            del rr
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
