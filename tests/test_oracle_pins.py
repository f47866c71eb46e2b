"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests re-types an oracle formula and compares it with itself:
each checks a printed value, a closed form, an invariant, a brute-force
evaluation with exact rational arithmetic, or an independent library
conversion.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from workloads import C1, make_layer

HERE = os.path.dirname(os.path.abspath(__file__))


# ------------------------------------------------------------------ rounding
def test_round_binary_matches_ieee_casts():
    rng = np.random.default_rng(1)
    y = np.concatenate([
        rng.standard_normal(200000) * np.exp2(rng.integers(-30, 30, 200000)),
        rng.standard_normal(20000) * 1e-6,      # fp16 subnormals
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e-8, 6e-8, 3e-8]),
    ])
    assert np.array_equal(O.to_fp32(y), y.astype(np.float32).astype(np.float64))
    assert np.array_equal(O.to_fp16(y), y.astype(np.float16).astype(np.float64))


def test_round_bf16_matches_torch_and_hand_cases():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    f = (rng.standard_normal(100000) * np.exp2(rng.integers(-60, 60, 100000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.to_bf16(f.astype(np.float64)), ref)
    one = 1.0
    # 1 + 2^-8 is the midpoint of 1 and 1 + 2^-7: ties to even (1.0)
    assert O.to_bf16(one + 2.0 ** -8) == 1.0
    assert O.to_bf16(one + 3 * 2.0 ** -8) == one + 2 * 2.0 ** -7
    # a hair above the midpoint rounds up even though the fp32 value would tie
    assert O.to_bf16(one + 2.0 ** -8 + 2.0 ** -40) == one + 2.0 ** -7


# ------------------------------------------------------------ eq. (1), INT4
def _int4_one_group(vals):
    v = np.zeros(64)
    v[: len(vals)] = vals
    q, s = O.quantize_int4_groups(v[None, :])
    return q[0, : len(vals)], s[0, 0]


def test_int4_hand_worked_unit_scale():
    # max |x| = 7 gives s = 7/7 = 1 exactly, so codes are round-half-even of x
    q, s = _int4_one_group([7.0, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5, -7.0, 6.49, -3.51])
    assert s == 1.0
    assert q.tolist() == [7, 2, -2, 4, 0, 0, 2, -7, 6, -4]
    # -0.5 rounds to zero and is encoded +0
    assert O.int4_nibble(q).tolist()[5] == 0


def test_int4_hand_worked_fp16_scale():
    # max |x| = 1.4: 1.4/7 = 0.2 -> fp16 0.199951171875 (= 3276 * 2^-14)
    q, s = _int4_one_group([1.4, 0.7, -0.1, 0.05])
    assert s == 0.199951171875
    # 0.7 / s = 3.50085... -> 4 ; 1.4 / s = 7.0017 -> 7 ; 0.1/s = 0.50012 -> 1
    assert q.tolist() == [7, 4, -1, 0]


def test_int4_zero_group_and_exact_ties():
    q, s = _int4_one_group([0.0, -0.0])
    assert s == 0.0 and q.tolist() == [0, 0]
    # s = fp16(5/7) = 0.71435546875; put values exactly on (k + 1/2) s and one
    # fp32 ulp either side of it
    s_expect = O.to_fp16(5.0 / 7.0)
    ties = [(k + 0.5) * s_expect for k in range(0, 6)]
    up = [np.nextafter(np.float32(t), np.float32(10)) for t in ties]
    dn = [np.nextafter(np.float32(t), np.float32(-10)) for t in ties]
    vals = [5.0] + ties + [float(u) for u in up] + [float(d) for d in dn]
    q, s = _int4_one_group(vals)
    assert s == s_expect
    k = np.arange(6)
    assert q[1:7].tolist() == [int(x) for x in np.where(k % 2 == 0, k, k + 1)]
    assert q[7:13].tolist() == (k + 1).tolist()
    assert q[13:19].tolist() == k.tolist()


def test_int4_matches_exact_rational_brute_force():
    """Scalar re-derivation with Fractions: A, s, and round-half-even of x/s."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((3, 192)) * np.exp2(rng.integers(-8, 8, (3, 1)))).astype(np.float32)
    x[0, :64] = np.round(x[0, :64] * 4) / 4            # many exact ties
    q, s = O.quantize_int4_groups(x.astype(np.float64))
    for i in range(3):
        for g in range(3):
            grp = [Fraction(float(v)) for v in x[i, 64 * g: 64 * g + 64]]
            A = max(abs(v) for v in grp)
            s_ref = Fraction(float(np.float16(float(A / 7))))   # fp16 of the exact quotient
            # np.float16(float(A/7)): A/7 rounded to fp64 first; fp64 has
            # enough precision for the fp16 rounding to be unaffected
            assert s[i, g] == float(s_ref)
            for j, v in enumerate(grp):
                ref = 0 if s_ref == 0 else max(-7, min(7, round(v / s_ref)))
                assert q[i, 64 * g + j] == ref


def test_fp16_scale_double_rounding_is_innocuous():
    """fp16(fp32(A/7)) == fp16(A/7) for fp32 A (the GPU divides in fp32)."""
    rng = np.random.default_rng(4)
    A = (rng.random(400000) * np.exp2(rng.integers(-30, 16, 400000))).astype(np.float32)
    # plus A = 7 m (and fp32 neighbours) for fp16 midpoints m
    h = (rng.random(50000) * 8 + 2.0 ** -10).astype(np.float16).astype(np.float64)
    m = h + np.exp2(np.floor(np.log2(h)) - 11)
    a0 = (7 * m).astype(np.float32)
    near = [a0]
    for _ in range(3):
        near.append(np.nextafter(near[-1], np.float32(np.inf)))
    lo = [a0]
    for _ in range(3):
        lo.append(np.nextafter(lo[-1], np.float32(0)))
    A = np.concatenate([A] + near + lo)
    via32 = (A / np.float32(7.0)).astype(np.float16).astype(np.float64)
    assert np.array_equal(via32, O.to_fp16(A.astype(np.float64) / 7.0))


# ------------------------------------------------------------- FP4 E2M1/E8M0
def test_e8m0_boundaries():
    A = np.array([6.0, 6.0 * (1 + 2.0 ** -23), 3.0, 3.0000001, 1.5, 0.0,
                  6.0 * 2.0 ** 100, 1e-45, 2.0 ** -130])
    e = O.e8m0_exponent(A)
    assert e.tolist() == [0, 1, -1, 0, -2, -127, 100, -127, -127]
    rng = np.random.default_rng(5)
    a = rng.random(100000) * np.exp2(rng.integers(-100, 100, 100000))
    e = O.e8m0_exponent(a).astype(np.float64)
    assert np.all(a <= 6 * np.exp2(e)) and np.all(a > 6 * np.exp2(e - 1))


def test_e2m1_midpoints_and_grid():
    y = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert O.e2m1_value(O.e2m1_code(y)).tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    eps = 1e-9
    assert O.e2m1_value(O.e2m1_code(y + eps)).tolist() == [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert O.e2m1_value(O.e2m1_code(y - eps)).tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    assert O.e2m1_code(grid).tolist() == list(range(8))
    assert O.e2m1_code(-grid).tolist() == [0] + [8 + i for i in range(1, 8)]
    assert O.e2m1_code(np.array([-0.2, -0.0])).tolist() == [0, 0]   # +0 encoding


def test_fp4_group_quant_brute_force():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((2, 64)) * 3).astype(np.float32).astype(np.float64)
    codes, e = O.quantize_fp4_groups(x)
    grid = [Fraction(v) for v in (0, .5, 1, 1.5, 2, 3, 4, 6)]
    for i in range(2):
        for g in range(2):
            vals = [Fraction(float(v)) for v in x[i, 32 * g: 32 * g + 32]]
            A = max(abs(v) for v in vals)
            ee = -200
            while A > 6 * Fraction(2) ** ee:
                ee += 1
            assert e[i, g] == ee
            for j, v in enumerate(vals):
                y = abs(v) / Fraction(2) ** ee
                d = [abs(y - gv) for gv in grid]
                best = min(d)
                cands = [k for k in range(8) if d[k] == best]
                k = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
                sgn = 8 if (v < 0 and k > 0) else 0
                assert codes[i, 32 * g + j] == (k | sgn)


def test_nibble_packing_layout():
    nib = np.array([[1, 2, 3, 4, 15, 8]], dtype=np.uint8)
    assert O.pack_nibbles(nib).tolist() == [[0x21, 0x43, 0x8F]]
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(nib)), nib)
    assert O.nibble_to_int4(O.int4_nibble(np.arange(-7, 8))).tolist() == list(range(-7, 8))


# ------------------------------------------------------- smoothing and split
def _c1_small():
    X, W, _ = make_layer(C1)
    return X, W


def test_smoothing_equivalence():
    X, Wb = _c1_small()
    Xf = O.bf16_bits_to_f64(X)
    W = O.bf16_bits_to_f64(Wb)
    a = O.act_absmax(X)
    assert np.array_equal(a, np.abs(Xf).max(axis=0))
    # exact lambda: X diag(lam)^-1 diag(lam) W = X W to fp64 rounding
    lam = a.astype(np.float64) ** 0.5 / np.abs(W).max(axis=1) ** 0.5
    Y = Xf @ W
    assert O.rel_fro((Xf / lam) @ (lam[:, None] * W), Y) < 1e-12
    # stored (lam32, inv32) pair with fp32 x_hat
    lam32, inv32 = O.smoothing_factors(a, W, 0.5)
    assert np.all(np.abs(lam32 * inv32 - 1) < 2 ** -23)
    xh = O.smooth_act(X, inv32)
    assert O.rel_fro(xh @ (lam32[:, None] * W), Y) < 1e-6
    # smoothing flattens the activation outliers (channels 0-3 were x50):
    # with alpha = 0.5 the outlier-to-typical ratio of channel maxima drops
    # roughly to its square root
    before = a[:4].max() / np.median(a)
    ah = np.abs(xh).max(axis=0)
    after = ah[:4].max() / np.median(ah)
    assert before > 40 and after < before / 4


def test_smoothing_degenerate_channels():
    a = np.array([0.0, 4.0, 4.0], np.float32)
    W = np.array([[1.0, -2.0], [0.0, 0.0], [0.5, 0.25]])
    lam32, inv32 = O.smoothing_factors(a, W, 0.5)
    assert lam32.tolist()[:2] == [1.0, 1.0]
    assert lam32[2] == O.to_fp32(np.sqrt(4.0) / np.sqrt(0.5))
    lam32, _ = O.smoothing_factors(a, W, 0.5, no_smoothing=True)
    assert lam32.tolist() == [1.0, 1.0, 1.0]


def test_eckart_young_on_known_spectrum():
    rng = np.random.default_rng(7)
    K, N, r = 96, 80, 8
    U, _ = np.linalg.qr(rng.standard_normal((K, K)))
    V, _ = np.linalg.qr(rng.standard_normal((N, N)))
    sig = np.sort(rng.random(N) * 10)[::-1]
    sig[:4] += 50
    W = (U[:, :N] * sig) @ V.T
    L1, L2 = O.lowrank_factors(W, r)
    best = (U[:, :r] * sig[:r]) @ V[:, :r].T
    assert O.rel_fro(L1 @ L2, best) < 1e-10
    assert abs(np.linalg.norm(W - L1 @ L2) - np.sqrt(np.sum(sig[r:] ** 2))) < 1e-9 * sig[0]
    # L2 rows are orthonormal, L1 columns carry the singular values
    assert np.allclose(L2 @ L2.T, np.eye(r), atol=1e-12)
    assert np.allclose(np.linalg.norm(L1, axis=0), sig[:r], rtol=1e-12)


def test_exact_split_and_residual_order():
    X, Wb = _c1_small()
    prep = O.prepare(Wb, O.act_absmax(X), alpha=0.5, rank=16, fmt=O.INT4)
    recon = prep["L1b"] @ prep["L2b"] + prep["R"]
    assert np.max(np.abs(recon - prep["W_hat"])) < 1e-13 * np.abs(prep["W_hat"]).max()
    # an exactly rank-r product of the stored factors leaves no residual
    L1b, L2b = prep["L1b"], prep["L2b"]
    P = L1b @ L2b
    assert np.max(np.abs(O.residual(P, L1b, L2b))) <= 1e-14 * np.abs(P).max()
    # the low-rank branch absorbs the outliers (walkthrough Fig. 4: the
    # residual's range is much narrower than W_hat's) ...
    assert np.abs(prep["R"]).max() < 0.5 * np.abs(prep["W_hat"]).max()
    # ... and rounding the factors to bf16 costs only second order in ||R||
    sig = np.linalg.svd(prep["W_hat"], compute_uv=False)
    opt = np.sqrt(np.sum(sig[16:] ** 2))
    assert opt <= np.linalg.norm(prep["R"]) <= opt * (1 + 1e-4)


# ------------------------------------------------------------ linear layer
def _brute_linear(prep, X_bits, act):
    """Triple loop from the group-wise definition (eq. (2) per group + low-rank + bias)."""
    fmt = prep["fmt"]
    g = O.GROUP[fmt]
    M, K = X_bits.shape
    N = prep["N"]
    Tb = O.down_proj(act["xhat"], prep["L1b"])[1]
    Y = np.zeros((M, N))
    for i in range(M):
        for n in range(N):
            acc = 0.0
            for gi in range(K // g):
                if fmt == O.INT4:
                    sx, sw = act["scales"][i, gi], prep["w_scales"][gi, n]
                    p = sum(int(act["codes"][i, k]) * int(prep["w_codes"][k, n])
                            for k in range(gi * g, gi * g + g))
                else:
                    sx = 2.0 ** act["scales"][i, gi]
                    sw = 2.0 ** prep["w_scales"][gi, n]
                    p = sum(O.e2m1_value(act["codes"][i, k]) * O.e2m1_value(prep["w_codes"][k, n])
                            for k in range(gi * g, gi * g + g))
                acc += sx * sw * p
            for t in range(prep["rank"]):
                acc += Tb[i, t] * prep["L2b"][t, n]
            if prep["bias"] is not None:
                acc += prep["bias"][n]
            Y[i, n] = acc
    return Y


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_linear_matches_brute_force(fmt):
    rng = np.random.default_rng(8)
    M, K, N, r = 5, 128, 6, 4
    X = O.bf16_bits_of(O.to_bf16(rng.standard_normal((M, K)) * 2).astype(np.float32))
    W = O.bf16_bits_of(O.to_bf16(rng.standard_normal((K, N)) * 0.1).astype(np.float32))
    b = O.bf16_bits_of(O.to_bf16(rng.standard_normal(N)).astype(np.float32))
    prep = O.prepare(W, O.act_absmax(X), alpha=0.5, rank=r, fmt=fmt, bias_bits=b)
    res = O.linear(prep, X, out="f32")
    ref = _brute_linear(prep, X, res["act"])
    assert np.max(np.abs(res["Y64"] - ref)) <= 1e-12 * np.abs(ref).max()


def test_lossless_special_case():
    """lambda = 1, r = 0, integer X and W in [-7, 7] with a 7 in every group:
    every scale is 1 and the layer is exactly X W."""
    rng = np.random.default_rng(9)
    M, K, N = 16, 256, 24
    X = rng.integers(-7, 8, (M, K)).astype(np.float64)
    W = rng.integers(-7, 8, (K, N)).astype(np.float64)
    X[:, ::64] = 7
    W[::64, :] = -7
    Xb = O.bf16_bits_of(X.astype(np.float32))
    Wb = O.bf16_bits_of(W.astype(np.float32))
    prep = O.prepare(Wb, O.act_absmax(Xb), alpha=0.5, rank=0, fmt=O.INT4, no_smoothing=True)
    res = O.linear(prep, Xb, out="f32")
    assert np.all(res["act"]["scales"] == 1.0) and np.all(prep["w_scales"] == 1.0)
    assert np.array_equal(res["Y64"], X @ W)


def test_eq6_residual_error_identity():
    """With an exact low-rank branch, the layer error equals E(X_hat, R)."""
    X, Wb = _c1_small()
    prep = O.prepare(Wb, O.act_absmax(X), alpha=0.5, rank=16, fmt=O.INT4, no_smoothing=True)
    res = O.linear(prep, X, out="f32")
    xh = res["act"]["xhat"]                       # lambda = 1: x_hat is X exactly (bf16)
    assert np.array_equal(O.to_bf16(xh), xh)
    Y_exactT = res["main"] + res["T"] @ prep["L2b"]
    lhs = np.linalg.norm(xh @ prep["W_hat"] - Y_exactT)
    Qx = O.dequant_groups(res["act"]["codes"], res["act"]["scales"], O.INT4)
    QR = O.dequant_groups(prep["w_codes"].T, prep["w_scales"].T, O.INT4).T
    rhs = O.quant_error(xh, prep["R"], Qx, QR)
    assert abs(lhs - rhs) <= 1e-9 * rhs


@pytest.mark.parametrize("seed", range(20))
def test_prop41_bound_random(seed):
    rng = np.random.default_rng(100 + seed)
    M, K, N = rng.integers(1, 40), 64 * rng.integers(1, 4), rng.integers(1, 40)
    X = rng.standard_normal((M, K)) * np.exp(rng.standard_normal(K))[None, :]
    W = rng.standard_normal((K, N))
    QX = O.dequant_groups(*O.quantize_int4_groups(X), O.INT4)
    QWt = O.dequant_groups(*O.quantize_int4_groups(W.T), O.INT4)
    assert O.quant_error(X, W, QX, QWt.T) <= O.prop41_bound(X, W, QX, QWt.T) * (1 + 1e-12)
    Xf = O.dequant_groups(*O.quantize_fp4_groups(X), O.FP4)
    Wf = O.dequant_groups(*O.quantize_fp4_groups(W.T), O.FP4).T
    assert O.quant_error(X, W, Xf, Wf) <= O.prop41_bound(X, W, Xf, Wf) * (1 + 1e-12)


def test_eq8_gaussian_residual_bound_monte_carlo():
    """eq. (8) with eq. (12)-(14)'s c: E||R - Q(R)|| <= c sqrt(n)/q_max E||R||."""
    rng = np.random.default_rng(11)
    n_side = 64
    errs, norms = [], []
    for _ in range(30):
        R = rng.standard_normal((n_side, n_side)) * 0.3
        errs.append(np.linalg.norm(R - O.q_eq1(R, 4)))
        norms.append(np.linalg.norm(R))
    size = n_side * n_side
    c = O.gaussian_c(size)
    assert np.mean(errs) <= c * np.sqrt(size) / 7 * np.mean(norms)
    # eq. (12): E max|R| <= sigma sqrt(2 log size); eq. (13): E||R|| >= sigma sqrt(2 size / pi)
    Rs = rng.standard_normal((200, size))
    assert np.abs(Rs).max(axis=1).mean() <= np.sqrt(2 * np.log(size))
    assert np.linalg.norm(Rs, axis=1).mean() >= np.sqrt(2 * size / np.pi)


def test_unfused_rounding_model_differs_only_by_double_rounding():
    X, Wb = _c1_small()
    prep = O.prepare(Wb, O.act_absmax(X), alpha=0.5, rank=16, fmt=O.INT4)
    fused = O.linear(prep, X, out="bf16")
    unf = O.linear_unfused(prep, X, out="bf16")
    assert O.rel_fro(unf["Y"], fused["Y64"]) < 1e-2
    assert O.rel_fro(fused["Y"], fused["Y64"]) < 5e-3


# ---------------------------------------------------- the handbook's tables
def _toy_inputs():
    """The toy tensors of the handbook's quantization chapter, regenerated:
    torch's generator seeded with 0, a 1024 x 512 standard normal activation
    and a 512 x 512 weight of standard deviation 0.02, drawn in that order
    (the chapter's shapes and seed; the printed tables depend on them)."""
    torch = pytest.importorskip("torch")
    torch.manual_seed(0)
    x = torch.randn(1024, 512).double().numpy()
    W = (torch.randn(512, 512) * 0.02).double().numpy()
    return x, W


def _with_outliers(x, factor):
    """Channels 0-3 scaled by ``factor`` (the chapter's outlier channels)."""
    y = x.copy()
    y[:, :4] *= factor
    return y


def test_handbook_printed_tables():
    """The oracle's eq. (1) quantizer, smoothing factors and eq. (5) split
    reproduce the three toy tables of the handbook's quantization chapter
    (outlier table; SmoothQuant table; SVDQuant rank table) to their four
    printed decimals."""
    gold = json.load(open(os.path.join(HERE, "golden", "handbook_toy_tables.json")))
    x0, W = _toy_inputs()
    tol = 6e-5   # printed to 4 decimals; the page computed in fp32
    for factor, row in gold["outlier_table"]["rows"].items():
        x = _with_outliers(x0, float(factor))
        normal = slice(4, None)            # the error is reported on the normal channels
        got = [O.rel_fro(O.q_eq1(x, bits, axis)[:, normal], x[:, normal])
               for bits, axis in ((8, None), (8, 0), (4, None), (4, 0))]
        assert np.allclose(got, row, atol=tol), (factor, got, row)
    x = _with_outliers(x0, 50.0)
    y = x @ W
    lam32, inv32 = O.smoothing_factors(np.abs(x).max(axis=0), W, 0.5)
    x_hat, W_hat = x * inv32[None, :], W * lam32[:, None]
    sq = gold["smoothquant_table"]
    for key, a, b, bits in (("w8a8_direct", x, W, 8), ("w8a8_smooth", x_hat, W_hat, 8),
                            ("w4a4_direct", x, W, 4), ("w4a4_smooth", x_hat, W_hat, 4)):
        got = O.rel_fro(O.q_eq1(a, bits) @ O.q_eq1(b, bits), y)
        assert abs(got - sq[key]) < tol, (key, got, sq[key])
    for r, want in gold["svdquant_table"]["rank"].items():
        got = O.rel_fro(O.eq5_toy(x_hat, W_hat, int(r), 4), y)
        assert abs(got - want) < tol, (r, got, want)
    floor = O.rel_fro(O.q_eq1(x0, 4) @ O.q_eq1(W, 4), x0 @ W)
    assert abs(floor - gold["svdquant_table"]["no_outlier_w4a4_floor"]) < tol


def test_error_ordering_on_tiny_config():
    """Naive W4A4 > smoothing only > SVDQuant, and error falls with rank."""
    X, Wb = _c1_small()
    Xf, W = O.bf16_bits_to_f64(X), O.bf16_bits_to_f64(Wb)
    y = Xf @ W
    a = O.act_absmax(X)
    naive = O.prepare(Wb, a, alpha=0.5, rank=0, fmt=O.INT4, no_smoothing=True)
    errs = [O.rel_fro(O.linear(naive, X, "f32")["Y64"], y)]
    for r in (0, 16, 32, 64):
        p = O.prepare(Wb, a, alpha=0.5, rank=r, fmt=O.INT4)
        errs.append(O.rel_fro(O.linear(p, X, "f32")["Y64"], y))
    assert all(errs[i] > errs[i + 1] for i in range(len(errs) - 1)), errs


def test_merge_lowrank_exact_case():
    """lambda = 1, no low-rank base, integer X and W whose 4-bit branch is
    exact, and a LoRA whose A has one +-1 per column: the merged layer is
    exactly X W + X A B (walkthrough, Fig. 9 / Fig. 16 section: the LoRA
    joins the low-rank branch, the residual is untouched)."""
    rng = np.random.default_rng(21)
    M, K, N, re = 8, 128, 16, 16
    X = rng.integers(-7, 8, (M, K)).astype(np.float64)
    W = rng.integers(-7, 8, (K, N)).astype(np.float64)
    X[:, ::64] = 7
    W[::64, :] = -7
    A = np.zeros((K, re))
    A[rng.permutation(K)[:re], np.arange(re)] = rng.choice([-1.0, 1.0], re)
    B = rng.integers(-3, 4, (re, N)).astype(np.float64)
    Xb, Wb = O.bf16_bits_of(X.astype(np.float32)), O.bf16_bits_of(W.astype(np.float32))
    Ab, Bb = O.bf16_bits_of(A.astype(np.float32)), O.bf16_bits_of(B.astype(np.float32))
    prep = O.prepare(Wb, O.act_absmax(Xb), alpha=0.5, rank=0, fmt=O.INT4, no_smoothing=True)
    merged = O.merge_lowrank(prep, Ab, Bb)
    assert merged["rank"] == re and merged["L1b"].shape == (K, re) and merged["L2b"].shape == (re, N)
    assert np.array_equal(merged["w_codes"], prep["w_codes"]) and np.array_equal(merged["w_scales"], prep["w_scales"])
    assert np.array_equal(O.linear(merged, Xb, out="f32")["Y64"], X @ W + X @ A @ B)


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_merge_lowrank_adds_the_update(fmt):
    """With smoothing and a real low-rank base, merging dW = A B changes the
    layer by X A B up to the bf16 roundings of the 16-bit branch (x_hat, the
    scaled A and T, each at most 2^-9 relative): |dY - X A B| <= 3.1 * 2^-9
    |X| |A| |B| elementwise.  Scaling A by 1/lambda instead of lambda, or a
    transposed B, breaks it."""
    rng = np.random.default_rng(22)
    M, K, N, r, re = 12, 256, 24, 8, 16
    X, W = _c1_small()
    X, W = X[:M, :K], W[:K, :N]
    A = O.to_bf16(rng.standard_normal((K, re)) * 0.05)
    B = O.to_bf16(rng.standard_normal((re, N)) * 0.05)
    prep = O.prepare(W, O.act_absmax(X), alpha=0.5, rank=r, fmt=fmt)
    assert np.ptp(prep["lam32"]) > 0.1                         # smoothing is active
    merged = O.merge_lowrank(prep, O.bf16_bits_of(A.astype(np.float32)), O.bf16_bits_of(B.astype(np.float32)))
    assert np.array_equal(merged["L1b"][:, :r], prep["L1b"]) and np.array_equal(merged["L2b"][:r], prep["L2b"])
    assert np.array_equal(merged["L1b"][:, r:], O.to_bf16(prep["lam32"][:, None] * A))
    dY = O.linear(merged, X, out="f32")["Y64"] - O.linear(prep, X, out="f32")["Y64"]
    x = O.bf16_bits_to_f64(X)
    bound = 3.1 * 2.0 ** -9 * (np.abs(x) @ np.abs(A) @ np.abs(B))
    assert np.all(np.abs(dY - x @ A @ B) <= bound)
    assert np.max(np.abs(x @ A @ B)) > 10 * np.max(bound)       # the update is well above the bound


def _bits(a):
    return O.bf16_bits_of(O.to_bf16(np.asarray(a, dtype=np.float64)).astype(np.float32))


def test_norm_act_two_valued_rows_closed_form():
    """Rows alternating a, b: mu = (a + b) / 2, var = ((a - b) / 2)^2, so with
    gamma = 1, beta = 0 and lambda = 1 every x_hat is +-d / sqrt(d^2 + eps),
    d = (a - b) / 2 (handbook SmoothQuant section: the norm that the
    smoothing folds into)."""
    K, eps = 256, 1e-6
    ab = [(3.0, -1.0), (0.5, 0.25), (-7.0, 9.0)]
    X = np.array([[a if k % 2 == 0 else b for k in range(K)] for a, b in ab])
    xh = O.norm_act(_bits(X), _bits(np.ones(K)), None, eps, np.ones(K))
    for i, (a, b) in enumerate(ab):
        d = (a - b) / 2
        v = d / np.sqrt(d * d + eps)
        assert np.array_equal(xh[i], O.to_fp32(np.where(np.arange(K) % 2 == 0, v, -v)))


def test_norm_act_invariances_and_fold():
    """LayerNorm is invariant to a per-row shift and positive scale (up to
    eps); its rows have zero mean and variance var / (var + eps); and the fold
    keeps the layer: x_hat (lambda W) = norm(x) W."""
    rng = np.random.default_rng(23)
    M, K, N, eps = 6, 128, 8, 1e-5
    x = rng.integers(-100, 101, (M, K)) / 8.0        # x, 4 x and 4 x + 3 are all exact in bf16
    one = np.ones(K)
    plain = O.norm_act(_bits(x), _bits(one), None, eps, one)
    assert np.all(np.abs(plain.mean(axis=1)) < 1e-6)
    var = x.var(axis=1)
    assert np.allclose((plain ** 2).mean(axis=1), var / (var + eps), rtol=1e-6)
    shifted = O.norm_act(_bits(x * 4 + 3), _bits(one), None, eps * 16, one)
    assert np.allclose(shifted, plain, rtol=0, atol=1e-6)
    g = O.to_bf16(rng.uniform(0.5, 1.5, K))
    b = O.to_bf16(rng.standard_normal(K) * 0.1)
    lam32 = O.to_fp32(rng.uniform(0.2, 5.0, K))
    inv32 = O.to_fp32(1.0 / lam32)
    W = rng.standard_normal((K, N))
    xh = O.norm_act(_bits(x), _bits(g), _bits(b), eps, inv32)
    y = (x - x.mean(axis=1, keepdims=True)) / np.sqrt(var[:, None] + eps) * g + b
    lhs, rhs = xh @ (lam32[:, None] * W), y @ W
    assert np.max(np.abs(lhs - rhs)) <= 1e-6 * np.max(np.abs(rhs))
    # smoothing applied the other way round (times lambda) would break the fold
    assert np.max(np.abs(O.norm_act(_bits(x), _bits(g), _bits(b), eps, lam32) @ (lam32[:, None] * W) - rhs)) > 0.1


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_w4a16_exact_when_weights_are_on_the_grid(fmt):
    """Weights already on the 4-bit grid with a full-range element in every
    group (so every scale is 1, or 2^e for FP4) and no smoothing: the
    weight-only layer is exactly X W for any bf16 X, which the W4A4 layer
    (activations rounded to 4 bits) is not."""
    rng = np.random.default_rng(24)
    M, K, N = 5, 128, 12
    if fmt == O.INT4:
        W = rng.integers(-7, 8, (K, N)).astype(np.float64)
        W[::64, :] = 7
    else:
        W = rng.choice(np.concatenate([O.E2M1_GRID, -O.E2M1_GRID]), (K, N)) * 4.0
        W[::32, :] = 24.0                          # 6 * 2^2: the group exponent is 2
    X = O.to_bf16(rng.standard_normal((M, K)))
    Wb = O.bf16_bits_of(W.astype(np.float32))
    Xb = O.bf16_bits_of(X.astype(np.float32))
    prep = O.prepare(Wb, O.act_absmax(Xb), alpha=0.5, rank=0, fmt=fmt, no_smoothing=True)
    y = O.linear_w4a16(prep, Xb, out="f32")["Y64"]
    assert np.allclose(y, X @ W, rtol=1e-13, atol=1e-12)
    assert not np.allclose(O.linear(prep, Xb, out="f32")["Y64"], X @ W, rtol=1e-6, atol=1e-6)


def _gptq_case(seed, K=256, N=24, M=512, correlated=True):
    rng = np.random.default_rng(seed)
    R = rng.standard_normal((K, N)) * 0.05
    if correlated:
        # calibration activations with strongly correlated channels
        B = rng.standard_normal((K, 16))
        x = rng.standard_normal((M, 16)) @ B.T + 0.3 * rng.standard_normal((M, K))
    else:
        x = rng.standard_normal((M, K))
    return R, x


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_gptq_reduces_to_rounding_for_a_diagonal_hessian(fmt):
    """With uncorrelated calibration channels (x_hat = diag(d), so H is
    diagonal) the Cholesky factor of H^-1 is diagonal, no error is passed on,
    and GPTQ gives exactly the round-to-nearest codes and scales."""
    R, _ = _gptq_case(25, correlated=False)
    K = R.shape[0]
    x = np.diag(np.linspace(0.5, 2.0, K))
    q, s = O.gptq_weights(R, x, fmt, damp=0.01)
    q0, s0 = O.quantize_weights(R, fmt)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_gptq_lowers_the_calibration_error(fmt):
    """GPTQ's purpose: ||x_hat (R - Q(R))||_F on the calibration data is
    clearly below round-to-nearest's (walkthrough, Table 3 row on GPTQ), while
    every code stays on the grid with its group's scale."""
    R, x = _gptq_case(26)
    q, s = O.gptq_weights(R, x, fmt, damp=0.01)
    q0, s0 = O.quantize_weights(R, fmt)
    dq = O.dequant_groups(q.T, s.T, fmt).T
    dq0 = O.dequant_groups(q0.T, s0.T, fmt).T
    e_gptq = np.linalg.norm(x @ (R - dq))
    e_rtn = np.linalg.norm(x @ (R - dq0))
    assert e_gptq < 0.8 * e_rtn, (e_gptq, e_rtn)
    if fmt == O.INT4:
        assert np.all(np.abs(q) <= 7)
    else:
        assert np.all(q < 16)


# ---------------------------------------------------------- exact hand cases
def test_smoothing_exponents_hand_cases():
    """lambda = a^alpha / w^(1 - alpha) (handbook SmoothQuant section) at
    alpha != 0.5, on values whose powers are exact: swapping the two
    exponents, or the roles of a and w, changes every one of these."""
    a = np.array([16.0, 1.0, 81.0, 16.0, 625.0], np.float32)
    W = np.array([[1.0], [16.0], [1.0], [81.0], [1.0]])
    lam32, inv32 = O.smoothing_factors(a, W, 0.25)
    # 16^.25 = 2; 1 / 16^.75 = 1/8; 81^.25 = 3; 16^.25 / 81^.75 = 2/27; 625^.25 = 5
    assert lam32.tolist() == [2.0, 0.125, 3.0, float(np.float32(2.0 / 27.0)), 5.0]
    assert inv32.tolist() == [0.5, 8.0, float(np.float32(1.0 / np.float32(3.0))), float(np.float32(27.0 / 2.0)), float(np.float32(1.0 / np.float32(5.0)))]
    lam32, _ = O.smoothing_factors(a, W, 0.75)
    # 16^.75 = 8; 1 / 16^.25 = 1/2; 81^.75 = 27; 16^.75 / 81^.25 = 8/3; 625^.75 = 125
    assert lam32.tolist() == [8.0, 0.5, 27.0, float(np.float32(8.0 / 3.0)), 125.0]


def test_smoothing_lambda_is_correctly_rounded():
    """At alpha = 0.5 and w a power of two, lambda = sqrt(a / w) with a / w
    exact in fp32, and IEEE's fp32 square root is correctly rounded: the
    stored lambda32 must be exactly that value (a value computed in fp64
    and then rounded to fp32 is not, for some inputs)."""
    rng = np.random.default_rng(31)
    a = (rng.random(4000) * np.exp2(rng.integers(-20, 20, 4000))).astype(np.float32)
    w = np.exp2(rng.integers(-10, 10, 4000)).astype(np.float64)
    lam32, _ = O.smoothing_factors(a, w[:, None], 0.5)
    ref = np.sqrt((a.astype(np.float64) / w).astype(np.float32)).astype(np.float64)
    assert np.array_equal(lam32, ref)


def _fp32_rounding_of_sqrt(r: Fraction) -> float:
    """The fp32 value nearest to sqrt(r) (ties to the even significand),
    decided with exact rationals: c is the answer when sqrt(r) lies between
    the midpoints to its neighbours, i.e. when their squares bracket r."""
    c = np.float32(np.sqrt(float(r)))
    for x in (np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))):
        lo = (Fraction(float(np.nextafter(x, np.float32(0)))) + Fraction(float(x))) / 2
        hi = (Fraction(float(x)) + Fraction(float(np.nextafter(x, np.float32(np.inf))))) / 2
        if lo * lo < r < hi * hi or ((lo * lo == r or hi * hi == r) and int(x.view(np.uint32)) % 2 == 0):
            return float(x)
    raise AssertionError("no candidate brackets sqrt(r)")


def test_smoothing_lambda_hard_rounding_case():
    """lambda = sqrt(a / w) at alpha = 0.5 (handbook, SmoothQuant section)
    for an fp32 activation maximum a and a bf16 weight maximum w chosen
    (by a search) so that sqrt(a / w) lies just past an fp32 rounding
    midpoint: the value computed in fp64 as a^0.5 / w^0.5 and then rounded
    to fp32 is one ulp low; the correctly rounded lambda32 is the exact
    rational decision."""
    a = np.float32(float.fromhex("0x1.19e7b4p+1"))
    w = float.fromhex("0x1.1ap+1")                         # a bf16 value
    want = _fp32_rounding_of_sqrt(Fraction(float(a)) / Fraction(w))
    assert want == float.fromhex("0x1.ffe9f2p-1")
    assert float(np.float32(float(a) ** 0.5 / w ** 0.5)) != want    # the fp64 route misses it
    lam32, inv32 = O.smoothing_factors(np.array([a]), np.array([[w]]), 0.5)
    assert lam32[0] == want
    assert inv32[0] == float(np.float32(1.0 / want))


def test_down_projection_rounds_xhat_to_bf16():
    """The down-projection's operand is x_hat rounded to bf16 (the bf16
    matrix-core input of the low-rank branch, walkthrough Fig. 6), not the
    fp32 x_hat: with x_hat = (1 + 2^-9, 1) and L1 = (1, -1)^T, bf16(1 + 2^-9)
    = 1 (2^-9 is below half a bf16 ulp at 1), so T = 0 exactly, while the
    fp32 operand would give T = 2^-9."""
    T, Tb = O.down_proj(np.array([[1.0 + 2.0 ** -9, 1.0]]), np.array([[1.0], [-1.0]]))
    assert T.tolist() == [[0.0]] and Tb.tolist() == [[0.0]]


def test_quantizer_decides_on_fp32_xhat():
    """The quantizer sees x_hat = fp32(x * inv_lambda), one rounding of the
    product (the smoothed activation is an fp32 tensor): x = 5.5 and inv =
    fp32(12/11), which is above 12/11 by 3.3e-8, give x * inv = 6 + 1.8e-7,
    within half an fp32 ulp of 6, so x_hat = 6 exactly; the FP4 group scale is
    then 2^0 (6 <= 6 * 2^0) and the code is 6, where the unrounded product
    would need 2^1 and code 3."""
    inv = np.ones(32)
    inv[0] = float(np.float32(12.0 / 11.0))
    assert Fraction(11, 2) * Fraction(inv[0]) > 6
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 5.5
    qa = O.quantize_act(O.bf16_bits_of(x), inv, O.FP4)
    assert qa["xhat"][0, 0] == 6.0
    assert qa["scales"].tolist() == [[0]] and qa["scale_bytes"].tolist() == [[127]]
    assert int(qa["codes"][0, 0]) == 7                     # E2M1 code of +6 (index 7)


def test_int4_scale_saturates_at_fp16_max():
    """A group absmax beyond 7 * 65504 keeps the largest finite fp16 scale
    (no infinity), and its codes clamp to +-7."""
    q, s = _int4_one_group([1.0e6, -3.0e5, 65504.0 * 7.0, 1.0, 0.0])
    assert s == 65504.0
    assert q.tolist() == [7, -5, 7, 0, 0]
    assert O.int4_scale(np.array([7 * 65504.0, 7 * 65519.0, 7 * 65520.0, 1e30])).tolist() == [65504.0] * 4


def test_unfused_rounding_hand_case():
    """The unfused model rounds twice (walkthrough, Nunchaku section: the
    separate branch writes the 4-bit product and adds the low-rank part in a
    second pass).  A hand-built layer with main + b exactly on a bf16 tie:
    main = 7 * 1 - 6 * 1 = 1, Tb = (7 - 6) 2^-12, low = Tb * (+-8) = +-2^-9.
      column 0: b = 2^-8    fused bf16(1 + 3 2^-9) = 1 + 2^-7;
                            unfused bf16(bf16(1 + 2^-8) + 2^-9) = bf16(1 + 2^-9) = 1
      column 1: b = 3 2^-9  fused bf16(1 + 2^-8) = 1 (tie to even);
                            unfused bf16(bf16(1 + 3 2^-9) - 2^-9) = bf16(1 + 3 2^-9) = 1 + 2^-7"""
    K, N = 64, 2
    x = np.zeros((1, K))
    x[0, 0], x[0, 1] = 7.0, -6.0
    w_codes = np.zeros((K, N), np.int8)
    w_codes[0], w_codes[1] = 1, 1
    L1b = np.zeros((K, 1))
    L1b[0, 0] = L1b[1, 0] = 2.0 ** -12
    prep = dict(fmt=O.INT4, K=K, N=N, rank=1, inv32=np.ones(K), L1b=L1b, L2b=np.array([[8.0, -8.0]]),
                w_codes=w_codes, w_scales=np.ones((1, N)), bias=np.array([2.0 ** -8, 3 * 2.0 ** -9]))
    X_bits = O.bf16_bits_of(x.astype(np.float32))
    fused = O.linear(prep, X_bits, "bf16")
    unfused = O.linear_unfused(prep, X_bits, "bf16")
    assert fused["act"]["scales"].tolist() == [[1.0]] and fused["Tb"].tolist() == [[2.0 ** -12]]
    assert fused["Y"].tolist() == [[1.0 + 2.0 ** -7, 1.0]]
    assert unfused["Y"].tolist() == [[1.0, 1.0 + 2.0 ** -7]]


def test_prop41_bound_is_attained():
    """Proposition 4.1 (walkthrough eq. (4) / (9)) is attained when every
    factor is rank one and aligned: X = 2 u a^T, W = 3 a c^T, Q(X) = 3 u a^T,
    Q(W) = 4 a c^T (unit u, a, c) give E = ||6 u c^T - 12 u c^T|| = 6 and the
    bound 2 * 1 + 1 * (3 + 1) = 6."""
    rng = np.random.default_rng(32)
    u, a, c = (v / np.linalg.norm(v) for v in (rng.standard_normal(5), rng.standard_normal(7), rng.standard_normal(3)))
    X, W = 2 * np.outer(u, a), 3 * np.outer(a, c)
    QX, QW = 3 * np.outer(u, a), 4 * np.outer(a, c)
    assert abs(O.quant_error(X, W, QX, QW) - 6.0) < 1e-12
    assert abs(O.prop41_bound(X, W, QX, QW) - 6.0) < 1e-12


def test_gaussian_c_against_monte_carlo():
    """eq. (10)-(14): for Gaussian R, E max|R| <= c E||R||_F with c the ratio
    of the eq. (12) upper bound to the eq. (13) lower bound; both bounds are
    within ~10-25% of the true expectations, so c sits between the measured
    ratio and 1.5 times it, at several sizes (a base-2 logarithm in place of
    the natural one gives about 1.6 times)."""
    rng = np.random.default_rng(33)
    for n in (256, 4096, 65536):
        R = rng.standard_normal((64, n))
        ratio = np.abs(R).max(axis=1).mean() / np.linalg.norm(R, axis=1).mean()
        c = O.gaussian_c(n)
        assert ratio <= c <= 1.5 * ratio, (n, ratio, c)
