"""GPU parity of libsvdq against the CPU oracle, through the C ABI.

Bar (per the layer's definition):
  * activation codes and scales: byte-equal to the oracle's;
  * weight codes and scales: byte-equal to the oracle's quantization of the
    residual taken against the blob's own lambda32, L1b, L2b (the SVD factors
    are not unique, so the split itself is checked by Eckart-Young instead);
  * lambda32: within one fp32 ulp of the oracle's (device pow vs host pow);
  * Tb: within one bf16 ulp element-wise (fp32 vs fp64 accumulation order);
  * Y: relative Frobenius error <= 1e-3 against the oracle's own quantized
    computation (fp64 accumulation), rounded to the same output type; the
    unfused path against the oracle's unfused rounding model.
Sizes: small cases span several 128-wide tiles with ragged tails; the
measured workloads run at full size and are checked on sampled rows and
columns, in the launch configuration the benchmark times.
"""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as WL
from svdq_testlib import (blob_sections, decode_act, np_bits_to_bf16_tensor, oracle_prep_from_blob, to_np, untile_bf16,
                          u16_tensor_to_np)

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a4_quantized_gemm_amd as S
    S.load()          # fails loudly if the library is missing
    return torch, "cuda:0"


def _fmt_name(fmt_id):
    import w4a4_quantized_gemm_amd as S
    return O.INT4 if fmt_id == S.INT4 else O.FP4


def _prepare(torch_dev, cfg, X_bits, W_bits, b_bits, **kw):
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    X = np_bits_to_bf16_tensor(X_bits, dev)
    W = np_bits_to_bf16_tensor(W_bits, dev)
    a = torch.empty(cfg.K, dtype=torch.float32, device=dev)
    S.svdq_act_absmax(X, a)
    bias = None if b_bits is None else np_bits_to_bf16_tensor(b_bits, dev)
    layer = S.SVDQLinear.prepare(W, a, cfg.rank, cfg.fmt, cfg.alpha, bias=bias, **kw)
    torch.cuda.synchronize()
    return layer, X, a


def _check_weights(layer, W_bits, fmt, b_bits=None, cols=None, X_bits=None, alpha=0.5, no_smoothing=False):
    """Weight codes, scales and bias of the blob against the oracle's
    quantization of the residual taken against the blob's L1b, L2b.  With the
    calibration activations (or no smoothing) the blob's lambda32 must equal
    the oracle's bit for bit, and the reference uses the oracle's own."""
    sec = blob_sections(layer)
    lam_ref = None
    if X_bits is not None or no_smoothing:
        lam_ref = _check_lambda(sec, X_bits, W_bits, alpha, no_smoothing)
    ref = oracle_prep_from_blob(sec, W_bits, fmt, b_bits, cols, lam32=lam_ref)
    codes, scales = sec["w_codes"], sec["w_scales"]
    if cols is not None:
        codes, scales = codes[:, cols], scales[:, cols]
    assert np.array_equal(codes, ref["w_codes"]), "weight codes differ"
    assert np.array_equal(scales, ref["w_scales"]), "weight scales differ"
    if b_bits is not None:
        bref = O.bf16_bits_to_f64(b_bits if cols is None else b_bits[cols])
        got = sec["bias"] if cols is None else sec["bias"][cols]
        assert np.array_equal(got, bref)
    # inv_lambda is fp32(1 / lambda32) exactly
    assert np.array_equal(sec["inv32"], O.to_fp32(1.0 / sec["lam32"]))
    return sec, ref


def _check_lambda(sec, X_bits, W_bits, alpha, no_smoothing=False):
    """lambda32 bit-equal to the oracle's (the real lambda rounded once to
    fp32, on both sides); returns the oracle's."""
    a = np.zeros(sec["lam32"].size, np.float32) if X_bits is None else O.act_absmax(X_bits)
    lam32, _ = O.smoothing_factors(a, O.bf16_bits_to_f64(W_bits), alpha, no_smoothing)
    assert np.array_equal(sec["lam32"], lam32), int(np.sum(sec["lam32"] != lam32))
    return lam32


def _run_act(torch_dev, layer, X, M, with_ws):
    """The activation pass alone; with the workspace it may split K."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    cb, sb, tb = S.svdq_act_sizes(layer.desc, M)
    codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    scales = torch.empty(sb, dtype=torch.uint8, device=dev)
    T = torch.empty(max(tb // 2, 1), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev) if with_ws else None
    S.svdq_quantize_act(layer.desc, layer.blob, X, codes, scales, T if layer.desc.rank else None, ws)
    torch.cuda.synchronize()
    return codes, scales, T


def _check_act(torch_dev, layer, X, X_bits, ref_prep, rows=None):
    for with_ws in (True, False):
        out = _check_act_once(torch_dev, layer, X, X_bits, ref_prep, rows, with_ws)
    return out


def _check_act_once(torch_dev, layer, X, X_bits, ref_prep, rows, with_ws):
    M, K = X_bits.shape
    codes, scales, T = _run_act(torch_dev, layer, X, M, with_ws)
    q, s, raw, sraw = decode_act(codes, scales, layer.desc.fmt, M, K)
    Xr = X_bits if rows is None else X_bits[rows]
    ref = O.quantize_act(Xr, ref_prep["inv32"], ref_prep["fmt"])
    sel = slice(None) if rows is None else rows
    assert np.array_equal(raw[sel], ref["packed"]), "activation codes differ"
    assert np.array_equal(sraw[sel], ref["scale_bytes"]), "activation scales differ"
    if layer.desc.rank:
        r = layer.desc.rank
        Tg = O.bf16_bits_to_f64(untile_bf16(u16_tensor_to_np(T), M, r))[sel]
        T64, Tref = O.down_proj(ref["xhat"], ref_prep["L1b"])
        # Tg is one bf16 rounding of an fp32 sum of K exact products (in an
        # order the kernel chooses): within half a bf16 ulp plus the fp32
        # summation bound K 2^-24 sum |products| of the fp64 sum
        sabs = np.abs(O.to_bf16(ref["xhat"])) @ np.abs(np.asarray(ref_prep["L1b"], dtype=np.float64))
        mag = np.maximum(np.maximum(np.abs(T64), np.abs(Tg)), 1e-30)
        half_ulp = np.exp2(np.floor(np.log2(mag)) - 8)
        err = np.abs(Tg - T64)
        bound = half_ulp + K * 2.0 ** -24 * sabs
        assert np.all(err <= bound * 1.0001), float(np.max(err / bound))
        mism = float(np.mean(Tg != Tref))
        assert mism < 0.01, mism
    return codes, scales, T


def _run_linear(torch_dev, layer, X, out, unfused):
    import w4a4_quantized_gemm_amd as S
    torch, _ = torch_dev
    Y = layer(X, out_dtype=out, unfused=unfused)
    torch.cuda.synchronize()
    return Y.float().cpu().numpy().astype(np.float64)


def _check_linear(torch_dev, layer, X, X_bits, ref_prep, rows=None, cols=None, modes=None):
    import w4a4_quantized_gemm_amd as S
    Xr = X_bits if rows is None else X_bits[rows]
    errs = {}
    for out, unfused in modes or [(S.OUT_BF16, False), (S.OUT_F32, False), (S.OUT_BF16, True), (S.OUT_F32, True)]:
        oname = "bf16" if out == S.OUT_BF16 else "f32"
        ref = (O.linear_unfused if unfused else O.linear)(ref_prep, Xr, oname)["Y"]
        Y = _run_linear(torch_dev, layer, X, out, unfused)
        if rows is not None:
            Y = Y[rows]
        if cols is not None:
            Y = Y[:, cols]
        assert np.all(np.isfinite(Y)), "non-finite output"
        e = O.rel_fro(Y, ref)
        errs[(oname, unfused)] = e
        assert e <= TOL, (oname, unfused, e)
    return errs


# ------------------------------------------------------------------ calibration
def test_act_absmax_exact(torch_dev):
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say("case: act_absmax c1")
    X_bits = WL.make_x(WL.C1)
    X = np_bits_to_bf16_tensor(X_bits, dev)
    a = torch.empty(WL.C1.K, dtype=torch.float32, device=dev)
    S.svdq_act_absmax(X, a)
    assert np.array_equal(to_np(a), O.act_absmax(X_bits))
    S.svdq_act_absmax(X[:100], a)
    S.svdq_act_absmax(X[100:], a, accumulate=True)
    assert np.array_equal(to_np(a), O.act_absmax(X_bits))


# ------------------------------------------------------------------ tiny workload
@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_tiny_config_end_to_end(torch_dev, fmt):
    cfg = WL.C1.with_(fmt=fmt)
    _say(f"case: tiny config {cfg.name} fmt={fmt}")
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    import w4a4_quantized_gemm_amd as S
    S.svdq_check_blob(layer.desc, layer.blob)
    sec, ref = _check_weights(layer, W_bits, fmt, X_bits=X_bits, alpha=cfg.alpha)
    # the GPU SVD reaches the Eckart-Young optimum (walkthrough: SVD gives the
    # minimal ||W_hat - L1 L2||_F over rank-r approximations)
    sig = np.linalg.svd(ref["W_hat"], compute_uv=False)
    opt = np.sqrt(np.sum(sig[cfg.rank:] ** 2))
    assert opt * (1 - 1e-12) <= np.linalg.norm(ref["R"]) <= opt * (1 + 1e-4)
    _check_act(torch_dev, layer, X, X_bits, ref)
    errs = _check_linear(torch_dev, layer, X, X_bits, ref)
    _say(f"  rel errors {errs}")


# ------------------------------------------------------------------ small shapes, edge cases
SMALL = [
    # M, K, N, rank, bias, fmt
    (300, 384, 320, 16, True, O.INT4),
    (300, 384, 320, 16, True, O.FP4),
    (1, 128, 64, 0, False, O.INT4),
    (17, 256, 192, 48, True, O.FP4),
    (129, 512, 448, 128, False, O.INT4),
    (64, 1024, 128, 32, True, O.INT4),
    (257, 640, 576, 64, False, O.FP4),
    (16400, 256, 64, 16, False, O.FP4),    # M above the K-split limit: one part per row block
    # 17 x 16 = 272 FP4 output tiles on 256 compute units: the last 16 tiles
    # run as 32 column-half items (straight-line and general schedules)
    (4352, 384, 4096, 16, True, O.FP4),
    (4352, 256, 4096, 16, False, O.FP4),
]


@pytest.mark.parametrize("M,K,N,rank,bias,fmt", SMALL)
def test_small_shapes(torch_dev, M, K, N, rank, bias, fmt):
    _say(f"case: small M={M} K={K} N={N} r={rank} bias={bias} fmt={fmt}")
    cfg = WL.C2.with_(name="small", M=M, K=K, N=N, rank=rank, fmt=fmt, w_std=1 / np.sqrt(K),
                      n_outlier_channels=min(8, K // 16), bias_std=0.02 if bias else 0.0, seed=M + K + N)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    sec, ref = _check_weights(layer, W_bits, fmt, b_bits, X_bits=X_bits, alpha=cfg.alpha)
    _check_act(torch_dev, layer, X, X_bits, ref)
    _check_linear(torch_dev, layer, X, X_bits, ref)


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
@pytest.mark.parametrize("M,K,N,rank", [(100, 2048, 384, 32), (300, 1536, 256, 16)])
def test_gemm_k_split(torch_dev, M, K, N, rank, fmt):
    """Layers with few output tiles split the GEMM's K over workgroups
    (fp32 partial results in the workspace's last section, added in part
    order with the bias by a second kernel; FP4 parts other than the first
    zero their low-rank operand).  With the full workspace the
    split runs; with a workspace that ends before that optional section the
    GEMM runs unsplit.  Both match the oracle within the layer's tolerance,
    in both output types and in the unfused path, and both are
    deterministic (a repeated call is bit-equal)."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say(f"case: GEMM K split fmt={fmt} M={M} K={K} N={N} r={rank}")
    cfg = WL.C2.with_(name="ksplit", M=M, K=K, N=N, rank=rank, fmt=fmt, w_std=1 / np.sqrt(K),
                      bias_std=0.02, seed=M + K)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    sec, ref = _check_weights(layer, W_bits, fmt, b_bits, X_bits=X_bits, alpha=cfg.alpha)
    full = S.svdq_workspace_bytes(layer.desc, M)
    split_bytes = 256 * 128 * 128 * 4
    ys = {}
    for ws_bytes in (full, full - split_bytes):
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
        for out in (S.OUT_BF16, S.OUT_F32):
            oname = "bf16" if out == S.OUT_BF16 else "f32"
            dt = torch.bfloat16 if out == S.OUT_BF16 else torch.float32
            for unfused in (False, True):
                fn = S.svdq_linear_unfused if unfused else S.svdq_linear
                Y = torch.empty((M, N), dtype=dt, device=dev)
                fn(layer.desc, layer.blob, X, Y, ws, out)
                Y2 = torch.full((M, N), float("nan"), dtype=dt, device=dev)
                fn(layer.desc, layer.blob, X, Y2, ws, out)
                torch.cuda.synchronize()
                assert torch.equal(Y, Y2), "repeated call differs"
                Yn = Y.float().cpu().numpy().astype(np.float64)
                refY = (O.linear_unfused if unfused else O.linear)(ref, X_bits, oname)["Y"]
                e = O.rel_fro(Yn, refY)
                _say(f"  ws={'full' if ws_bytes == full else 'no split section'} {oname} unfused={unfused}: rel err {e:.2e}")
                assert np.all(np.isfinite(Yn)) and e <= TOL, e
                ys[(ws_bytes == full, oname, unfused)] = Yn
    # split and unsplit differ only in the fp32 summation order of the K parts
    for oname in ("bf16", "f32"):
        for unfused in (False, True):
            assert O.rel_fro(ys[(True, oname, unfused)], ys[(False, oname, unfused)]) <= 1e-3
    # the GEMM stage on its own: with the workspace it splits as svdq_linear
    # does (bit-equal), without it it runs unsplit (bit-equal to the
    # truncated-workspace layer)
    ws = torch.zeros(full, dtype=torch.uint8, device=dev)
    cb, sb, tb = S.svdq_act_sizes(layer.desc, M)
    codes = torch.empty(cb, dtype=torch.uint8, device=dev)
    scales = torch.empty(sb, dtype=torch.uint8, device=dev)
    T = torch.empty(tb // 2, dtype=torch.bfloat16, device=dev)
    S.svdq_quantize_act(layer.desc, layer.blob, X, codes, scales, T, ws)
    for wsarg, key in ((ws, True), (None, False)):
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        S.svdq_gemm(layer.desc, layer.blob, codes, scales, T, M, Y, S.OUT_F32, wsarg)
        torch.cuda.synchronize()
        assert np.array_equal(Y.cpu().numpy().astype(np.float64), ys[(key, "f32", False)])


@pytest.mark.parametrize("alpha,fmt", [(0.25, O.INT4), (0.75, O.INT4), (0.25, O.FP4), (0.75, O.FP4)])
def test_smoothing_strengths(torch_dev, alpha, fmt):
    """Smoothing strengths other than 0.5 (the handbook's SmoothQuant
    section: alpha is a tuning knob, commonly 0.5): lambda32 bit-equal to
    the oracle's, then the usual weight, activation and layer parity."""
    _say(f"case: alpha={alpha} fmt={fmt}")
    cfg = WL.C2.with_(name="alpha", M=300, K=384, N=320, rank=16, fmt=fmt, alpha=alpha, w_std=1 / np.sqrt(384),
                      bias_std=0.02, seed=41)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    sec, ref = _check_weights(layer, W_bits, fmt, b_bits, X_bits=X_bits, alpha=alpha)
    assert np.ptp(np.log2(sec["lam32"])) > 1.0                 # smoothing is active
    _check_act(torch_dev, layer, X, X_bits, ref)
    _check_linear(torch_dev, layer, X, X_bits, ref)


def test_blob_round_trip(torch_dev, tmp_path):
    """A prepared blob is position independent: written to a file, read back
    into a new device buffer, it passes the header check and gives the same
    output bit for bit."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say("case: blob save / reload")
    cfg = WL.C1.with_(fmt=O.FP4, bias_std=0.02)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    path = tmp_path / "layer.npy"
    np.save(path, to_np(layer.blob))
    pad = torch.empty(4096, dtype=torch.uint8, device=dev)       # a different device address
    blob2 = torch.from_numpy(np.load(path)).to(dev)
    layer2 = S.SVDQLinear(layer.desc, blob2)
    S.svdq_check_blob(layer2.desc, layer2.blob)
    assert layer2.blob.data_ptr() != layer.blob.data_ptr()
    y1 = layer(X, out_dtype=S.OUT_F32)
    y2 = layer2(X, out_dtype=S.OUT_F32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    del pad


def test_factors_given_and_no_smoothing(torch_dev):
    """Caller-supplied factors are stored verbatim; with them the whole blob
    equals the oracle's preparation."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say("case: factors given + no smoothing")
    cfg = WL.C1.with_(M=200, K=512, N=384, rank=32, seed=3)
    X_bits, W_bits, _ = WL.make_layer(cfg)
    a = O.act_absmax(X_bits)
    ref = O.prepare(W_bits, a, alpha=0.5, rank=32, fmt=O.INT4)
    L1 = np_bits_to_bf16_tensor(O.bf16_bits_of(ref["L1b"].astype(np.float32)), dev)
    L2 = np_bits_to_bf16_tensor(O.bf16_bits_of(ref["L2b"].astype(np.float32)), dev)
    X = np_bits_to_bf16_tensor(X_bits, dev)
    W = np_bits_to_bf16_tensor(W_bits, dev)
    ad = torch.from_numpy(a).to(dev)
    layer = S.SVDQLinear.prepare(W, ad, 32, "int4", 0.5, L1=L1, L2=L2)
    sec = blob_sections(layer)
    assert np.array_equal(sec["L1b"], ref["L1b"]) and np.array_equal(sec["L2b"], ref["L2b"])
    sec, ref2 = _check_weights(layer, W_bits, O.INT4, X_bits=X_bits, alpha=0.5)
    _check_linear(torch_dev, layer, X, X_bits, ref2)
    # no smoothing: lambda = 1 exactly
    layer = S.SVDQLinear.prepare(W, None, 32, "fp4", 0.5, no_smoothing=True)
    sec = blob_sections(layer)
    assert np.all(sec["lam32"] == 1.0) and np.all(sec["inv32"] == 1.0)
    sec, ref3 = _check_weights(layer, W_bits, O.FP4, no_smoothing=True)
    _check_act(torch_dev, layer, X, X_bits, ref3)
    _check_linear(torch_dev, layer, X, X_bits, ref3)


@pytest.mark.parametrize("fmt,re", [(O.INT4, 16), (O.FP4, 32)])
def test_merge_lowrank(torch_dev, fmt, re):
    """An extra low-rank branch (a LoRA) merged into a prepared layer: lambda,
    the residual codes and scales and the bias are copied, the merged
    factors equal the oracle's merge bit for bit, the input blob is
    untouched, and the merged layer matches the oracle's merged layer."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say(f"case: merge low-rank fmt={fmt} r_extra={re}")
    M, K, N, r = 200, 384, 320, 16
    cfg = WL.C2.with_(name="merge", M=M, K=K, N=N, rank=r, fmt=fmt, w_std=1 / np.sqrt(K),
                      n_outlier_channels=8, bias_std=0.02, seed=77)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    sec, ref = _check_weights(layer, W_bits, fmt, b_bits, X_bits=X_bits, alpha=cfg.alpha)
    rng = np.random.default_rng(78)
    A_bits = O.bf16_bits_of(O.to_bf16(rng.standard_normal((K, re)) * 0.05).astype(np.float32))
    B_bits = O.bf16_bits_of(O.to_bf16(rng.standard_normal((re, N)) * 0.05).astype(np.float32))
    merged = layer.merge_lowrank(np_bits_to_bf16_tensor(A_bits, dev), np_bits_to_bf16_tensor(B_bits, dev))
    torch.cuda.synchronize()
    assert merged.desc.rank == r + re
    S.svdq_check_blob(merged.desc, merged.blob)
    msec = blob_sections(merged)
    for k in ("lam32", "inv32", "w_codes", "w_scales", "bias", "raw_wcodes", "raw_wscales"):
        assert np.array_equal(msec[k], sec[k]), k
    after = blob_sections(layer)
    assert all(np.array_equal(after[k], sec[k]) for k in ("L1b", "L2b", "raw_wcodes", "raw_wscales"))
    mref = O.merge_lowrank(ref, A_bits, B_bits)
    assert np.array_equal(msec["L1b"], mref["L1b"]) and np.array_equal(msec["L2b"], mref["L2b"])
    _check_act(torch_dev, merged, X, X_bits, mref)
    errs = _check_linear(torch_dev, merged, X, X_bits, mref)
    _say(f"  rel errors {errs}")


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
@pytest.mark.parametrize("M,K,N", [(1, 3072, 576), (3, 1024, 320), (5, 256, 64), (16, 4096, 192), (16, 1024, 9216),
                                   (9, 3072, 18432), (1, 16384, 64), (9, 16384, 128)])
def test_w4a16(torch_dev, fmt, M, K, N):
    """The weight-only 4-bit layer on a rank-0 blob against the oracle's
    weight-only layer (x_hat unquantized, fp64 product): the products are
    exact on both sides and only the fp32 accumulation differs, so the f32
    output agrees to 1e-5.  Shapes: one and two operand planes (M <= 8,
    M <= 16), 1-3 column blocks per workgroup, fewer 64-blocks than waves,
    and K = 16384, where the workgroup's scales (K bytes per column block)
    exceed the LDS staging area and every lane loads its own."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say(f"case: w4a16 fmt={fmt} M={M} K={K} N={N}")
    cfg = WL.C2.with_(name="w4a16", M=max(M, 64), K=K, N=N, rank=0, fmt=fmt, w_std=1 / np.sqrt(K),
                      n_outlier_channels=8, bias_std=0.02, seed=M + K)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, Xfull, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    sec, ref = _check_weights(layer, W_bits, fmt, b_bits, X_bits=X_bits, alpha=cfg.alpha)
    X = Xfull[:M].contiguous()
    ws = torch.zeros(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev)
    for out, oname in ((S.OUT_F32, "f32"), (S.OUT_BF16, "bf16")):
        Y = torch.empty((M, N), dtype=torch.float32 if out == S.OUT_F32 else torch.bfloat16, device=dev)
        S.svdq_linear_w4a16(layer.desc, layer.blob, X, Y, ws, out)
        torch.cuda.synchronize()
        r = O.linear_w4a16(ref, X_bits[:M], oname)
        e = O.rel_fro(Y.float().cpu().numpy().astype(np.float64), r["Y"])
        assert e <= (1e-5 if oname == "f32" else TOL), (oname, e)


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_prepare_gptq(torch_dev, fmt):
    """GPTQ on the residual.  Uncorrelated calibration channels (a diagonal
    H) reproduce the round-to-nearest blob byte for byte; correlated ones
    lower the calibration error well below rounding's, match the oracle's
    GPTQ on the blob's own residual (codes almost all equal; the error
    within 2%: GPTQ passes every rounding difference on), and the layer
    computed from the GPTQ blob matches the oracle given its codes."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say(f"case: gptq fmt={fmt}")
    M, K, N, r = 200, 384, 320, 16
    cfg = WL.C2.with_(name="gptq", M=M, K=K, N=N, rank=r, fmt=fmt, w_std=1 / np.sqrt(K),
                      n_outlier_channels=8, bias_std=0.02, seed=55)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, a = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    W = np_bits_to_bf16_tensor(W_bits, dev)
    bias = np_bits_to_bf16_tensor(b_bits, dev)
    rtn = blob_sections(layer)
    # (1) diagonal H: calibration rows e_k * c_k
    xd = np.zeros((K, K))
    xd[np.arange(K), np.arange(K)] = np.linspace(0.5, 2.0, K)
    Xd = np_bits_to_bf16_tensor(O.bf16_bits_of(O.to_bf16(xd).astype(np.float32)), dev)
    g1 = S.SVDQLinear.prepare(W, a, r, fmt, cfg.alpha, bias=bias, gptq=(Xd, 0.01))
    torch.cuda.synchronize()
    assert torch.equal(g1.blob, layer.blob), "diagonal H must give the round-to-nearest blob"
    # (2) correlated calibration activations
    rng = np.random.default_rng(56)
    xc = rng.standard_normal((512, 16)) @ rng.standard_normal((16, K)) + 0.3 * rng.standard_normal((512, K))
    Xc_bits = O.bf16_bits_of(O.to_bf16(xc).astype(np.float32))
    g2 = S.SVDQLinear.prepare(W, a, r, fmt, cfg.alpha, bias=bias, gptq=(np_bits_to_bf16_tensor(Xc_bits, dev), 0.01))
    torch.cuda.synchronize()
    sec = blob_sections(g2)
    for k in ("lam32", "inv32", "L1b", "L2b", "bias"):
        assert np.array_equal(sec[k], rtn[k]), k
    ref = oracle_prep_from_blob(sec, W_bits, fmt, b_bits)
    xh = O.smooth_act(Xc_bits, ref["inv32"])
    q_or, s_or = O.gptq_weights(ref["R"], xh, fmt, 0.01)
    agree = float(np.mean(sec["w_codes"] == q_or))
    assert agree > 0.98, agree

    def calib_err(codes, scales):
        return np.linalg.norm(xh @ (ref["R"] - O.dequant_groups(codes.T, scales.T, fmt).T))

    e_gpu, e_or, e_rtn = calib_err(sec["w_codes"], sec["w_scales"]), calib_err(q_or, s_or), calib_err(ref["w_codes"], ref["w_scales"])
    _say(f"  codes agreeing {agree:.4f}; calibration error gpu {e_gpu:.4g} oracle {e_or:.4g} rounding {e_rtn:.4g}")
    assert e_gpu < 0.8 * e_rtn and abs(e_gpu - e_or) <= 0.02 * e_or, (e_gpu, e_or, e_rtn)
    ref_g = dict(ref, w_codes=sec["w_codes"], w_scales=sec["w_scales"])
    _check_linear(torch_dev, g2, X, X_bits, ref_g, modes=[(S.OUT_BF16, False), (S.OUT_F32, False)])


E2M1_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
@pytest.mark.parametrize("M,K,N", [(300, 384, 320), (4608, 256, 128), (64, 3072, 128), (40, 12288, 64), (32, 16384, 64),
                                    (24, 20480, 64)])
def test_norm_fused_pass(torch_dev, fmt, M, K, N):
    """The LayerNorm-fused activation pass and layer against the oracle's
    norm path.  x_hat comes from fp32 row statistics, so it may differ from
    the oracle's by a few fp32 ulps: scales must be equal except in groups
    whose absmax sits within 1e-5 of a scale rounding boundary, and in every
    other group the codes must be equal except for elements within 1e-4 of a
    rounding tie (where either neighbour is right); T within 2 bf16 ulps plus
    the fp32 sum's error and the flips of x_hat's bf16 rounding next to a
    midpoint; Y to the usual tolerance.  At M = 4608 the pass runs 8-wave
    workgroups over whole row blocks (FP4: 32-row blocks of two halves); the
    K values take the row statistics' register-held forms (2, 6, 24 and 32
    vectors per lane) and the streamed one (K = 20480)."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say(f"case: norm-fused pass fmt={fmt} M={M} K={K} N={N}")
    r, eps = 16, 1e-5
    cfg = WL.C2.with_(name="norm", M=M, K=K, N=N, rank=r, fmt=fmt, w_std=1 / np.sqrt(K),
                      n_outlier_channels=8, bias_std=0.02, seed=91)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    rng = np.random.default_rng(92)
    # a per-row offset and scale, so that the norm has work to do
    xf = O.bf16_bits_to_f64(X_bits) * rng.uniform(0.5, 3.0, (M, 1)) + rng.standard_normal((M, 1))
    X_bits = O.bf16_bits_of(O.to_bf16(xf).astype(np.float32))
    g_bits = O.bf16_bits_of(O.to_bf16(rng.uniform(0.5, 1.5, K)).astype(np.float32))
    be_bits = O.bf16_bits_of(O.to_bf16(rng.standard_normal(K) * 0.1).astype(np.float32))
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    sec, ref = _check_weights(layer, W_bits, fmt, b_bits, X_bits=X_bits, alpha=cfg.alpha)
    gamma, beta = np_bits_to_bf16_tensor(g_bits, dev), np_bits_to_bf16_tensor(be_bits, dev)
    for beta_t, beta_b in ((beta, be_bits), (None, None)):
        norm = (g_bits, beta_b, eps)
        cb, sb, tb = S.svdq_act_sizes(layer.desc, M)
        codes = torch.empty(cb, dtype=torch.uint8, device=dev)
        scales = torch.empty(sb, dtype=torch.uint8, device=dev)
        T = torch.empty(tb // 2, dtype=torch.bfloat16, device=dev)
        ws = torch.zeros(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev)
        S.svdq_quantize_act_ln(layer.desc, layer.blob, X, gamma, beta_t, eps, codes, scales, T, ws)
        torch.cuda.synchronize()
        q, s, _, _ = decode_act(codes, scales, layer.desc.fmt, M, K)
        qa = O.quantize_act(X_bits, ref["inv32"], fmt, norm)
        g = 64 if fmt == O.INT4 else 32
        xh = qa["xhat"].reshape(M, K // g, g)
        if fmt == O.INT4:
            same = s == qa["scales"]
            a7 = np.abs(xh).max(axis=2) / 7.0
            # fp16 rounding boundaries near a7: midpoints between neighbouring fp16 values
            e = np.floor(np.log2(np.maximum(a7, 2.0 ** -24)))
            ulp = 2.0 ** (np.maximum(e, -14) - 10)
            near_b = np.abs(a7 / ulp - np.floor(a7 / ulp) - 0.5) < 1e-5 * a7 / ulp
            t = xh / np.where(qa["scales"] > 0, qa["scales"], 1.0)[..., None]
            near_tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-4
        else:
            same = s == qa["scales"]
            amax = np.abs(xh).max(axis=2)
            near_b = np.abs(amax / (6.0 * np.exp2(qa["scales"])) - 1.0) < 1e-5
            t = np.abs(xh) / np.exp2(qa["scales"])[..., None]
            near_tie = np.min(np.abs(t[..., None] - E2M1_MIDPOINTS), axis=-1) < 1e-4
        assert np.all(same | near_b), "scales differ away from a rounding boundary"
        qg = q.reshape(M, K // g, g).astype(np.int64)
        rg = qa["codes"].reshape(M, K // g, g).astype(np.int64)
        bad = (qg != rg) & same[..., None] & ~near_tie
        assert not np.any(bad), f"{int(bad.sum())} codes differ away from a rounding tie"
        mism = float(np.mean((qg != rg) & same[..., None]))
        assert mism < 1e-3, mism
        _say(f"  beta={'yes' if beta_b is not None else 'no'}: scales differing {int((~same).sum())}, codes at ties "
             f"differing {int(((qg != rg) & same[..., None]).sum())}")
        Tg = O.bf16_bits_to_f64(untile_bf16(u16_tensor_to_np(T), M, r))
        _, Tref = O.down_proj(qa["xhat"], ref["L1b"])
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(Tref), 1e-30))) - 7)
        # T's bound: 2 bf16 ulps (x_hat from fp32 row statistics), plus the
        # fp32 summation's K 2^-24 sum|products|, plus one bf16 ulp of x_hat
        # times |L1| for every x_hat within 2^-20 (relative) of a bf16
        # rounding midpoint, where the kernel's x_hat, a few fp32 ulps away,
        # may round the other way; the last two terms matter only where T
        # cancels
        xh64 = qa["xhat"]
        xb16 = O.to_bf16(xh64)
        u16 = np.exp2(np.floor(np.log2(np.maximum(np.abs(xh64), 1e-30))) - 7)
        near = np.abs(np.abs(xh64 - xb16) - u16 / 2) <= 2.0 ** -20 * np.abs(xh64)
        L1a = np.abs(ref["L1b"])
        bound = 2 * ulp + K * 2.0 ** -24 * (np.abs(xb16) @ L1a) + (near * u16) @ L1a
        excess = np.abs(Tg - Tref) / bound
        assert np.all(excess <= 1.0001), (float(excess.max()), int((excess > 1.0001).sum()))
        for out in (S.OUT_BF16, S.OUT_F32):
            oname = "bf16" if out == S.OUT_BF16 else "f32"
            Y = layer(X, out_dtype=out, norm=(gamma, beta_t, eps))
            torch.cuda.synchronize()
            e_rel = O.rel_fro(Y.float().cpu().numpy().astype(np.float64), O.linear(ref, X_bits, oname, norm)["Y"])
            assert e_rel <= TOL, (oname, e_rel)


def test_quantizer_edge_values(torch_dev):
    """Zero rows, exact ties of x/s, tiny values with subnormal fp16 scales,
    E2M1 midpoints, large magnitudes, E8M0 exponents near -127 and bf16
    subnormal inputs, in both formats."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say("case: quantizer edge values")
    K, N, M = 256, 64, 48
    rng = np.random.default_rng(5)
    x = rng.standard_normal((M, K))
    x[0] = 0.0                                            # all-zero row: s = 0, codes 0
    x[1, :64] = np.arange(64) % 15 - 7.0                  # max 7 -> s = 1: integer codes
    x[1, 64:128] = (np.arange(64) % 15 - 7.0) + 0.5       # ties at s = 7.5/7 -> fp16 rounding
    x[2] = rng.standard_normal(K) * 1e-6                  # subnormal fp16 scales
    x[3] = rng.standard_normal(K) * 2.0 ** -26            # scales that underflow to 0
    x[4] = rng.standard_normal(K) * 3e3                   # large values
    x[5, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4)   # E2M1 midpoints (A = 6: e = 0)
    x[6] = -x[5]
    x[7] = rng.standard_normal(K) * 2.0 ** -125           # E8M0 exponents near -127 (exact FP4 path)
    x[8] = rng.standard_normal(K) * 2.0 ** -118           # around the -120 switch of the FP4 conversion
    x[9] = (np.arange(K) % 7 - 3.0) * 2.0 ** -131         # bf16 subnormals
    x[10] = rng.standard_normal(K) * 1.0e6                # INT4 scales saturate at 65504 (A / 7 > 65520)
    x[11, :64] = 7.0 * 65504.0                             # exactly at the largest finite scale
    x[11, 64:128] = np.linspace(-1.0e7, 1.0e7, 64)
    X_bits = O.bf16_bits_of(O.to_bf16(x).astype(np.float32))
    W_bits = O.bf16_bits_of(O.to_bf16(rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    X = np_bits_to_bf16_tensor(X_bits, dev)
    W = np_bits_to_bf16_tensor(W_bits, dev)
    for fmt in ("int4", "fp4"):
        layer = S.SVDQLinear.prepare(W, None, 16, fmt, 0.5, no_smoothing=True)
        sec, ref = _check_weights(layer, W_bits, fmt, no_smoothing=True)
        _check_act(torch_dev, layer, X, X_bits, ref)
        _check_linear(torch_dev, layer, X, X_bits, ref, modes=[(S.OUT_F32, False), (S.OUT_F32, True)])


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_workspace_reuse_across_shapes(torch_dev, fmt):
    """One zero-filled workspace serves calls of different M (different K
    splits of the activation pass, whose arrival counters must be back at
    zero after every call): T, codes and scales equal those of a fresh
    workspace each time, and T equals the oracle's."""
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say(f"case: workspace reuse fmt={fmt}")
    cfg = WL.C2.with_(name="reuse", M=4608, K=1536, N=256, rank=32, fmt=fmt, w_std=1 / np.sqrt(1536),
                      bias_std=0.0, seed=71)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    sec, ref = _check_weights(layer, W_bits, fmt, b_bits, X_bits=X_bits, alpha=cfg.alpha)
    ws = torch.zeros(S.svdq_workspace_bytes(layer.desc, cfg.M), dtype=torch.uint8, device=dev)
    for M in (4608, 200, 4608, 1000, 33):
        cb, sb, tb = S.svdq_act_sizes(layer.desc, M)
        outs = []
        for w in (ws, torch.zeros(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev)):
            # zero-filled: rows past M in the padded 32-row blocks are never written
            codes = torch.zeros(cb, dtype=torch.uint8, device=dev)
            scales = torch.zeros(sb, dtype=torch.uint8, device=dev)
            T = torch.zeros(tb // 2, dtype=torch.bfloat16, device=dev)
            S.svdq_quantize_act(layer.desc, layer.blob, X[:M].contiguous(), codes, scales, T, w)
            outs.append((codes, scales, T))
        torch.cuda.synchronize()
        for a, b in zip(*outs):
            assert torch.equal(a, b), f"M={M}: reused workspace differs"
        Tg = O.bf16_bits_to_f64(untile_bf16(u16_tensor_to_np(outs[0][2]), M, cfg.rank))
        _, Tref = O.down_proj(O.quantize_act(X_bits[:M], ref["inv32"], fmt)["xhat"], ref["L1b"])
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(Tref), 1e-30))) - 7)
        assert np.all(np.abs(Tg - Tref) <= ulp * 1.0001), M


def test_determinism_and_bad_blob(torch_dev):
    import w4a4_quantized_gemm_amd as S
    torch, dev = torch_dev
    _say("case: determinism + bad blob")
    cfg = WL.C1
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    y1 = layer(X, out_dtype=S.OUT_F32).clone()
    y2 = layer(X, out_dtype=S.OUT_F32).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    blob2 = layer.blob.clone()
    blob2[0] ^= 0xFF
    with pytest.raises(S.SvdqError) as ei:
        S.svdq_check_blob(layer.desc, blob2)
    assert ei.value.status == 6
    with pytest.raises(S.SvdqError) as ei:
        ws = torch.empty(16, dtype=torch.uint8, device=dev)
        S.svdq_linear(layer.desc, layer.blob, X, torch.empty_like(y1), ws, S.OUT_F32)
    assert ei.value.status == 4


# ------------------------------------------------------------------ measured workloads, full size
FULL = [WL.C2, WL.C3, WL.C4_INT4, WL.C4_FP4]


@pytest.mark.parametrize("cfg", FULL, ids=[c.name for c in FULL])
def test_full_size_workloads(torch_dev, cfg):
    _say(f"case: full size {cfg.name}")
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(cfg.M, 192, replace=False), [0, cfg.M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(cfg.N, 384, replace=False), [0, cfg.N - 1]]))
    sec, ref = _check_weights(layer, W_bits, cfg.fmt, b_bits, cols=cols, X_bits=X_bits, alpha=cfg.alpha)
    if cfg is not WL.C4_FP4:            # the same weight (and split) as the INT4 variant
        # the GPU's randomized SVD reaches the Eckart-Young optimum at full
        # size too: ||R||_F within (1 + 1e-4) of sqrt(sum_{i > r} sigma_i^2)
        W_hat = sec["lam32"][:, None] * O.bf16_bits_to_f64(W_bits)
        R_norm = np.linalg.norm(O.residual(W_hat, sec["L1b"], sec["L2b"]))
        sig = np.linalg.svd(W_hat, compute_uv=False)
        opt = np.sqrt(np.sum(sig[cfg.rank:] ** 2))
        _say(f"  ||R||_F / optimum - 1 = {R_norm / opt - 1:.3e}")
        assert opt * (1 - 1e-12) <= R_norm <= opt * (1 + 1e-4)
        del W_hat
    _check_act(torch_dev, layer, X, X_bits, ref, rows=rows)
    errs = _check_linear(torch_dev, layer, X, X_bits, ref, rows=rows, cols=cols)
    _say(f"  rel errors {errs}")


# ---------------------------------------------- further large shapes, sampled
SAMPLED = [
    # the FP4 GEMM's general path (rank above 96, or fewer stages than the
    # straight-line schedule needs) with more tiles than compute units
    WL.C3.with_(name="c3_fc1_rank128_fp4", rank=128),
    WL.C3.with_(name="fp4_4608x256x4096_r16", K=256, N=4096, rank=16, w_std=1 / 16.0, seed=7),
    # two points of the shape sweep: few rows over a long K (the activation
    # pass splits K eight ways), and the largest M
    [c for c in WL.sweep_configs() if c.name == "c5_M256_K12288_N3072_r64"][0],
    [c for c in WL.sweep_configs() if c.name == "c5_M16384_K3072_N12288_r32"][0],
]


@pytest.mark.parametrize("cfg", SAMPLED, ids=[c.name for c in SAMPLED])
def test_sampled_shapes(torch_dev, cfg):
    _say(f"case: sampled {cfg.name} ({cfg.M}x{cfg.K}x{cfg.N}, r={cfg.rank}, {cfg.fmt})")
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    layer, X, _ = _prepare(torch_dev, cfg, X_bits, W_bits, b_bits)
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([rng.choice(cfg.M, min(cfg.M, 160), replace=False), [0, cfg.M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(cfg.N, 320, replace=False), [0, cfg.N - 1]]))
    sec, ref = _check_weights(layer, W_bits, cfg.fmt, b_bits, cols=cols, X_bits=X_bits, alpha=cfg.alpha)
    _check_act(torch_dev, layer, X, X_bits, ref, rows=rows)
    errs = _check_linear(torch_dev, layer, X, X_bits, ref, rows=rows, cols=cols)
    _say(f"  rel errors {errs}")
