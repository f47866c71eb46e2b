"""CPU oracle for the SVDQuant W4A4 linear layer with a 16-bit low-rank branch.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
shares no code, header, table or constant generator with it.

It is a plain, slow, obviously-correct restatement of what the layer computes,
in float64 except where a step is declared to round to fp32 / fp16 / bf16.
Sources (the pages are cited by title and section / equation):
  [walkthrough] "SVDQuant" paper walkthrough, devpress.csdn.net:
      eq. (1) quantizer, eq. (2) quantized linear, eq. (3) error,
      eq. (4)/(9) Proposition 4.1, eq. (5) low-rank split, eq. (6) residual
      error identity, eq. (7)/(8), (10)-(14) residual bound, Fig. 6 fusion,
      Table 4 latency.
  [handbook] ai-infra handbook, quantization chapter ("扩散模型和 LLM 不一样的
      地方"): printed toy tables (per-tensor / per-channel error, SmoothQuant
      and rank tables), SmoothQuant section (lambda_j = max|X_j|^a / max|W_j|^(1-a)), SVDQuant
      section (L1 = U_r S_r, L2 = V_r^T, R = W_hat - L1 L2; per-64-element
      group scales), timestep section (dynamic activation scales).

Readings where the pages leave a step open (each is also listed in the design
notes of the repository):
  * round() in eq. (1) is round-half-to-even of the EXACT real quotient x/s
    (the handbook uses torch.round, which is half-to-even).
  * INT4 groups: 64 consecutive elements along K (per token row for X, per
    output column for the residual R); scale s = fp16(max|v| / 7) (round to
    nearest even), saturating at 65504; s == 0 gives all-zero codes; codes
    clamp to [-7, 7].
  * FP4 groups: 32 along K; E2M1 codes (grid 0, .5, 1, 1.5, 2, 3, 4, 6) with
    round-to-nearest, ties to the even code; a power-of-two (E8M0) scale
    2^e with e the smallest integer such that max|v| <= 6 * 2^e, clamped to
    [-127, 127]; an all-zero group has e = -127.
  * Negative values that round to zero are encoded as +0 (code 0).
  * Smoothing factors are stored as fp32 lambda (the real lambda rounded once)
    and fp32 1/lambda; the runtime activation is x_hat = fp32(x * inv_lambda);
    W_hat = lambda32 * W (exact).
  * Low-rank factors are stored in bf16; the residual is computed from the
    stored bf16 factors: R = W_hat - sum_t L1b[:, t] L2b[t, :] (fp64, t
    increasing) so that W_hat = L1b L2b + R holds to fp64 rounding.
  * The down-projection input is bf16(x_hat) (the 16-bit branch), accumulated
    in fp64 and rounded once to bf16 (Tb); the up-projection Tb L2b, the 4-bit
    product and the bias are summed in fp64, then rounded once to the output
    type.  The unfused form rounds the partial output (4-bit product + bias)
    to the output type first, then adds Tb L2b and rounds again.
"""
from __future__ import annotations

from decimal import Decimal, localcontext

import numpy as np

INT4 = "int4"
FP4 = "fp4"
GROUP = {INT4: 64, FP4: 32}
QMAX = {INT4: 7, FP4: 6}

# ============================================================ rounding helpers


def round_binary(y, sig_bits: int, min_normal_exp: int, max_finite: float) -> np.ndarray:
    """Round fp64 values to a binary floating-point format, nearest-even.

    The format has ``sig_bits`` significand bits (implicit bit included),
    normal numbers down to 2**min_normal_exp, gradual underflow below it, and
    overflow to +-inf beyond ``max_finite`` (IEEE 754 round-to-nearest-even).
    Works by scaling each value by the power-of-two quantum of its binade,
    which is exact, and rounding that integer-valued quotient half-to-even.
    """
    y = np.asarray(y, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e = np.frexp(y)                      # |y| in [2^(e-1), 2^e)
        e = np.maximum(e, min_normal_exp + 1)   # subnormal binade shares the min quantum
        quantum = np.ldexp(1.0, e - sig_bits)
        r = np.rint(y / quantum) * quantum
        r = np.where(np.abs(r) > max_finite, np.copysign(np.inf, y), r)
        r = np.where(np.isfinite(y), r, y)
    return r


BF16_MAX = float.fromhex("0x1.fep127")
FP16_MAX = 65504.0
FP32_MAX = float.fromhex("0x1.fffffep127")


def to_bf16(y):
    return round_binary(y, 8, -126, BF16_MAX)


def to_fp16(y):
    return round_binary(y, 11, -14, FP16_MAX)


def to_fp32(y):
    return round_binary(y, 24, -126, FP32_MAX)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits_of(values) -> np.ndarray:
    """Bit pattern of values that are already exactly bf16."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def fp16_bits_of(values) -> np.ndarray:
    """Bit pattern of values that are already exactly fp16."""
    return np.ascontiguousarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)


def fp16_bits_to_f64(bits) -> np.ndarray:
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ============================================================ eq. (1) quantizer


def rne_quotient(num, den) -> np.ndarray:
    """Round-half-even of the exact real quotient num/den (den > 0).

    Valid when den has at most 24 significant bits and |num/den| < 2^20, so
    that the half-way points (q +- 0.5) * den are exact in fp64 and the
    comparisons below are exact (larger quotients only occur with a
    saturated scale, where the caller clamps the result to +-7 anyway).  The fp64 quotient picks a candidate q;
    the exact comparisons move q by one where the candidate is on the wrong
    side of (or exactly on) a half-way point.
    """
    num = np.asarray(num, dtype=np.float64)
    den = np.asarray(den, dtype=np.float64)
    q = np.rint(num / den)
    hi = (q + 0.5) * den
    lo = (q - 0.5) * den
    odd = np.mod(q, 2.0) != 0.0
    up = (num > hi) | ((num == hi) & odd)
    down = (num < lo) | ((num == lo) & odd)
    return q + up.astype(np.float64) - down.astype(np.float64)


def _groups(v: np.ndarray, group: int) -> np.ndarray:
    """View the last axis as (n_groups, group)."""
    K = v.shape[-1]
    assert K % group == 0, (K, group)
    return v.reshape(v.shape[:-1] + (K // group, group))


def int4_scale(A) -> np.ndarray:
    """INT4 group scale from the group absmax A: s = fp16(A / 7), saturating
    at the largest finite fp16 value (65504) instead of overflowing to
    infinity for A / 7 >= 65520; the codes then clamp to +-7."""
    return np.minimum(to_fp16(np.asarray(A, dtype=np.float64) / 7.0), FP16_MAX)


def quantize_int4_groups(v) -> tuple[np.ndarray, np.ndarray]:
    """Eq. (1) per group of 64 along the last axis, q_max = 7, fp16 scale.

    [walkthrough] eq. (1): Q = round(X / s), s = max|X| / q_max, q_max =
    2^(k-1) - 1 for signed k-bit integers; [handbook] SVDQuant section: one
    scale per 64 elements.  Returns (codes int8 with v's shape, scale values
    fp64 of shape (..., K/64), each exactly an fp16 number).
    """
    g = _groups(np.asarray(v, dtype=np.float64), 64)
    A = np.max(np.abs(g), axis=-1)
    s = int4_scale(A)
    safe = np.where(s > 0, s, 1.0)[..., None]
    q = np.clip(rne_quotient(g, safe), -7, 7)
    q = np.where((s > 0)[..., None], q, 0.0)
    return q.reshape(np.shape(v)).astype(np.int8), s


E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e8m0_exponent(A) -> np.ndarray:
    """Smallest integer e with A <= 6 * 2^e, clamped to [-127, 127]; A = 0 -> -127.

    The 4-bit float of eq. (1) has q_max = 6 ([walkthrough], text after
    eq. (1)); the scale is restricted to a power of two so that it is an
    E8M0 byte.  Start from the real logarithm and correct by exact
    comparisons (6 * 2^e is exact in fp64).
    """
    A = np.asarray(A, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(np.where(A > 0, A, 1.0) / 6.0))
    e = e + (A > 6.0 * np.exp2(e))              # too small: raise
    e = e - (A <= 6.0 * np.exp2(e - 1.0))       # not the smallest: lower
    e = np.where(A > 0, e, -127.0)
    return np.clip(e, -127, 127).astype(np.int32)


def e2m1_code(y) -> np.ndarray:
    """Nearest E2M1 value to y (|y| <= 6), ties to the even code; 4-bit code.

    Code = sign << 3 | index into (0, .5, 1, 1.5, 2, 3, 4, 6); index parity is
    the mantissa bit, so 'even code' is round-half-to-even on this grid.
    A value that rounds to zero gets code 0 (+0).
    """
    y = np.asarray(y, dtype=np.float64)
    m = np.abs(y)
    d = np.abs(m[..., None] - E2M1_GRID)        # distance to each grid point
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    sign = (y < 0) & (idx > 0)
    return (idx | (sign.astype(np.int64) << 3)).astype(np.uint8)


def e2m1_value(code) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_GRID[code & 7]
    return np.where(code & 8, -mag, mag)


def quantize_fp4_groups(v) -> tuple[np.ndarray, np.ndarray]:
    """4-bit float codes per group of 32 along the last axis, power-of-two scale.

    Returns (E2M1 codes uint8 with v's shape, exponents int32 (..., K/32)).
    v * 2^-e is exact (a power-of-two scaling) and lies in [-6, 6].
    """
    g = _groups(np.asarray(v, dtype=np.float64), 32)
    e = e8m0_exponent(np.max(np.abs(g), axis=-1))
    y = g * np.exp2(-e.astype(np.float64))[..., None]
    return e2m1_code(y).reshape(np.shape(v)), e


def int4_nibble(q) -> np.ndarray:
    """Two's-complement 4-bit pattern of an integer code in [-7, 7]."""
    return (np.asarray(q, dtype=np.int64) & 0xF).astype(np.uint8)


def nibble_to_int4(n) -> np.ndarray:
    n = np.asarray(n, dtype=np.int64) & 0xF
    return np.where(n >= 8, n - 16, n).astype(np.int8)


def pack_nibbles(nib) -> np.ndarray:
    """Pack 4-bit codes two per byte along the last axis, even index in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def dequant_groups(codes, scales, fmt: str) -> np.ndarray:
    """Exact real values s * q of group-quantized codes (last axis = K).

    INT4: codes are signed integers, scales the fp16 values.
    FP4: codes are E2M1 codes, scales the integer exponents e.
    """
    if fmt == INT4:
        q = np.asarray(codes, dtype=np.float64)
        s = np.asarray(scales, dtype=np.float64)
        g = GROUP[INT4]
    else:
        q = e2m1_value(codes)
        s = np.exp2(np.asarray(scales, dtype=np.float64))
        g = GROUP[FP4]
    qg = _groups(q, g)
    return (qg * s[..., None]).reshape(q.shape)


# ============================================================ offline preparation


def act_absmax(X_bits) -> np.ndarray:
    """a_j = max_i |X[i, j]| over calibration activations (exact, fp32 values)."""
    return np.max(np.abs(bf16_bits_to_f64(X_bits)), axis=0).astype(np.float32)


def real_to_fp32(v: Decimal) -> float:
    """The fp32 number nearest to the positive real v (a Decimal), ties to
    the even significand: the neighbours of a first guess are compared with
    v exactly (Decimal(float) is exact)."""
    f = np.float32(float(v))
    cands = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Decimal(float(c)) - v), int(np.float32(c).view(np.uint32)) & 1))
    return float(best)


def smoothing_factors(a, W, alpha: float, no_smoothing: bool = False):
    """[handbook] SmoothQuant section: lambda_j = max|X_j|^alpha / max|W_j|^(1-alpha),
    where W_j is row j of the K x N weight; [walkthrough] eq. (5): X W =
    (X diag(lambda)^-1)(diag(lambda) W).

    lambda32 is the real lambda_j rounded once to fp32 (evaluated as
    exp(alpha ln a - (1 - alpha) ln w) with 60 significant digits, far more
    than the rounding needs); inv32 = fp32(1 / lambda32).  A channel with a
    zero activation or weight maximum keeps lambda = 1.
    """
    a = np.asarray(a, dtype=np.float64)
    w = np.max(np.abs(np.asarray(W, dtype=np.float64)), axis=1)
    lam32 = np.ones_like(a)
    if not no_smoothing:
        with localcontext() as ctx:
            ctx.prec = 60
            al = Decimal(float(alpha))
            for j in range(a.size):
                if a[j] > 0 and w[j] > 0:
                    v = (al * Decimal(float(a[j])).ln() - (1 - al) * Decimal(float(w[j])).ln()).exp()
                    lam32[j] = real_to_fp32(v)
    inv32 = to_fp32(1.0 / lam32)
    return lam32, inv32


def lowrank_factors(W_hat, rank: int):
    """Top-r SVD factors of W_hat: L1 = U_r Sigma_r (K x r), L2 = V_r^T (r x N).

    [walkthrough] eq. (5) and the text after it; [handbook] SVDQuant section.
    The singular value decomposition is LAPACK's (a library primitive);
    Eckart-Young makes L1 L2 the best rank-r approximation in Frobenius norm.
    """
    if rank == 0:
        K, N = W_hat.shape
        return np.zeros((K, 0)), np.zeros((0, N))
    U, S, Vt = np.linalg.svd(W_hat, full_matrices=False)
    return U[:, :rank] * S[:rank], Vt[:rank]


def residual(W_hat, L1b, L2b) -> np.ndarray:
    """R = W_hat - sum_t L1b[:, t] L2b[t, :]  ([walkthrough] text after eq. (5)).

    Summed in fp64 with t increasing; every product of two bf16 numbers is
    exact in fp64, so this is a fixed, reproducible sequence of roundings.
    """
    S = np.zeros_like(np.asarray(W_hat, dtype=np.float64))
    for t in range(L1b.shape[1]):
        S += L1b[:, t, None] * L2b[None, t, :]
    return W_hat - S


def quantize_weights(R, fmt: str):
    """Group-quantize the residual along K for every output column.

    Returns (codes K x N, scales (K/g) x N): INT4 codes are signed integers
    with fp16 scale values; FP4 codes are E2M1 codes with integer exponents.
    """
    Rt = np.ascontiguousarray(np.asarray(R, dtype=np.float64).T)   # N x K: groups along K
    if fmt == INT4:
        q, s = quantize_int4_groups(Rt)
    else:
        q, s = quantize_fp4_groups(Rt)
    return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def gptq_weights(R, xhat_cal, fmt: str, damp: float = 0.01):
    """GPTQ on the residual instead of rounding each group on its own.

    [walkthrough] Table 3 row: quantizing the residual with GPTQ gives a
    further gain in most settings.  Steps (GPTQ, restated): H = x_hat^T x_hat
    of the calibration activations plus damp * mean(diag H) on the diagonal
    (a channel never active gets 1); U the upper Cholesky factor of H^-1
    (H^-1 = U^T U).  The residual's rows (input channels k) are quantized in
    increasing k; a group's scales (per output column) are taken from the
    current, already updated rows when k reaches the group's first row; the
    rounding error of row k, divided by U[k, k], is subtracted from the rows
    not yet quantized with weights U[k, k+1:].  Returns (codes K x N, scales
    (K/g) x N) like ``quantize_weights``.
    """
    R = np.array(R, dtype=np.float64)
    K, N = R.shape
    g = GROUP[fmt]
    x = np.asarray(xhat_cal, dtype=np.float64)
    H = x.T @ x
    d = np.diag(H).copy()
    dead = d == 0
    H[dead, dead] = 1.0
    H += damp * np.mean(np.diag(H)) * np.eye(K)
    Hinv = np.linalg.inv(H)
    U = np.linalg.cholesky(Hinv).T                              # upper, H^-1 = U^T U
    codes = np.zeros((K, N), dtype=np.int64)
    scales = np.zeros((K // g, N), dtype=np.float64 if fmt == INT4 else np.int64)
    for k in range(K):
        if k % g == 0:
            A = np.max(np.abs(R[k:k + g]), axis=0)
            scales[k // g] = int4_scale(A) if fmt == INT4 else e8m0_exponent(A)
        s = scales[k // g]
        if fmt == INT4:
            safe = np.where(s > 0, s, 1.0)
            q = np.where(s > 0, np.clip(rne_quotient(R[k], safe), -7, 7), 0.0)
            deq = q * s
        else:
            q = e2m1_code(R[k] * np.exp2(-s.astype(np.float64)))
            deq = e2m1_value(q) * np.exp2(s.astype(np.float64))
        codes[k] = q
        err = (R[k] - deq) / U[k, k]
        R[k + 1:] -= U[k, k + 1:, None] * err[None, :]
    if fmt == INT4:
        return codes.astype(np.int8), scales
    return codes.astype(np.uint8), scales.astype(np.int32)


def prepare(W_bits, a, *, alpha: float, rank: int, fmt: str, bias_bits=None,
            no_smoothing: bool = False, factors=None, gptq=None) -> dict:
    """Offline preparation of one layer.

    W_bits: bf16 bits, K x N.  a: fp32 per-channel activation maxima (K,).
    factors: optional (L1b, L2b) fp64 arrays of bf16 values that replace the
    SVD (a caller-supplied split, e.g. factors read back from another
    implementation); the residual is then taken against them.  gptq:
    optional (calibration X bf16 bits, damping) to quantize the residual with
    ``gptq_weights`` instead of rounding.
    """
    W = bf16_bits_to_f64(W_bits)
    lam32, inv32 = smoothing_factors(a, W, alpha, no_smoothing)
    W_hat = lam32[:, None] * W                              # exact: 24 x 8 bits
    if factors is None:
        L1, L2 = lowrank_factors(W_hat, rank)
        L1b, L2b = to_bf16(L1), to_bf16(L2)
    else:
        L1b, L2b = (np.asarray(f, dtype=np.float64) for f in factors)
    R = residual(W_hat, L1b, L2b)
    if gptq is None:
        w_codes, w_scales = quantize_weights(R, fmt)
    else:
        # gptq = (calibration X bf16 bits, damping): the quantizer sees x_hat
        w_codes, w_scales = gptq_weights(R, smooth_act(gptq[0], inv32), fmt, gptq[1])
    bias = None if bias_bits is None else bf16_bits_to_f64(bias_bits)
    return dict(fmt=fmt, K=W.shape[0], N=W.shape[1], rank=rank, lam32=lam32,
                inv32=inv32, W_hat=W_hat, L1b=L1b, L2b=L2b, R=R,
                w_codes=w_codes, w_scales=w_scales, bias=bias)


# ============================================================ runtime


def merge_lowrank(prep: dict, A_bits, B_bits) -> dict:
    """An extra low-rank branch dW = A B (A: K x r_e, B: r_e x N, bf16 bits)
    merged into the 16-bit branch of a prepared layer.

    [walkthrough] Fig. 9 / Fig. 16 section: a LoRA joins the existing
    low-rank branch, so the quantized residual is not redone.  The layer
    computes with X_hat = X diag(1/lambda), so X dW = X_hat diag(lambda) A B:
    L1 gains the columns bf16(lambda32 * A) (row j times lambda32_j, exact in
    fp64, rounded once) and L2 the rows B; R, its codes and scales, lambda and
    the bias stay as they are.
    """
    A = bf16_bits_to_f64(A_bits)
    B = bf16_bits_to_f64(B_bits)
    out = dict(prep)
    out["L1b"] = np.concatenate([prep["L1b"], to_bf16(prep["lam32"][:, None] * A)], axis=1)
    out["L2b"] = np.concatenate([prep["L2b"], B], axis=0)
    out["rank"] = out["L1b"].shape[1]
    return out


def smooth_act(X_bits, inv32) -> np.ndarray:
    """x_hat = fp32(x * inv_lambda) (the product of two fp32 numbers, rounded once)."""
    return to_fp32(bf16_bits_to_f64(X_bits) * np.asarray(inv32, dtype=np.float64)[None, :])


def norm_act(X_bits, gamma_bits, beta_bits, eps: float, inv32) -> np.ndarray:
    """x_hat of the norm-fused activation pass: LayerNorm over K of each row
    with its affine, the smoothing folded into the affine.

    [handbook] SmoothQuant section: the smoothing factor is merged into the
    preceding normalization's weights, so inference has no separate
    operator.  In fp64: mu = mean_k x, var = mean_k (x - mu)^2,
    y = (x - mu) / sqrt(var + eps) * gamma + beta, x_hat = y * inv_lambda32;
    returned rounded once to fp32, the precision in which the quantizer
    decides.  beta_bits None means beta = 0.
    """
    x = bf16_bits_to_f64(X_bits)
    g = bf16_bits_to_f64(gamma_bits)
    b = np.zeros_like(g) if beta_bits is None else bf16_bits_to_f64(beta_bits)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps) * g[None, :] + b[None, :]
    return to_fp32(y * np.asarray(inv32, dtype=np.float64)[None, :])


def quantize_act(X_bits, inv32, fmt: str, norm=None) -> dict:
    """Smoothing + dynamic per-token group quantization of the activations.

    [handbook] timestep section: dynamic scales computed from the current
    activation; groups along K per token row.  Returns the API byte formats
    (packed codes M x K/2, INT4 fp16 scale bits / FP4 E8M0 bytes M x K/g)
    together with the unpacked codes, scale values and x_hat.  With ``norm``
    = (gamma_bits, beta_bits, eps), X is the pre-norm input and x_hat comes
    from ``norm_act``.
    """
    xh = smooth_act(X_bits, inv32) if norm is None else norm_act(X_bits, norm[0], norm[1], norm[2], inv32)
    if fmt == INT4:
        q, s = quantize_int4_groups(xh)
        nib = int4_nibble(q)
        scale_bytes = fp16_bits_of(s)
    else:
        nib, s = quantize_fp4_groups(xh)
        q = nib
        scale_bytes = (s + 127).astype(np.uint8)
    return dict(xhat=xh, codes=q, scales=s, packed=pack_nibbles(nib),
                scale_bytes=scale_bytes)


def down_proj(xhat, L1b):
    """T = bf16(x_hat) L1b accumulated in fp64; Tb = bf16(T)  ([walkthrough]
    Fig. 6: the down-projection shares the quantizer's input)."""
    T = to_bf16(xhat) @ np.asarray(L1b, dtype=np.float64)
    return T, to_bf16(T)


def _round_out(Y, out: str):
    return to_bf16(Y) if out == "bf16" else to_fp32(Y)


def linear(prep: dict, X_bits, out: str = "bf16", norm=None) -> dict:
    """Fused layer: Y = Q(x_hat) Q(R) + Tb L2b + b, then one rounding.

    [walkthrough] eq. (5): X W ~ X_hat L1 L2 + Q(X_hat) Q(R); eq. (2): the
    4-bit product is s_x s_w Q_x Q_w per group.  Dequantization is exact in
    fp64, so the 4-bit product is one fp64 matrix product of the dequantized
    operands.  Returns Y64 (unrounded), Y (rounded to ``out``) and the
    activation-side intermediates.  ``norm`` as in ``quantize_act``.
    """
    fmt = prep["fmt"]
    qa = quantize_act(X_bits, prep["inv32"], fmt, norm)
    T, Tb = down_proj(qa["xhat"], prep["L1b"])
    Xdq = dequant_groups(qa["codes"], qa["scales"], fmt)
    Wdq = dequant_groups(prep["w_codes"].T, prep["w_scales"].T, fmt).T
    main = Xdq @ Wdq
    low = Tb @ prep["L2b"]
    bias = 0.0 if prep["bias"] is None else prep["bias"][None, :]
    Y64 = main + low + bias
    return dict(Y64=Y64, Y=_round_out(Y64, out), main=main, low=low, Tb=Tb, T=T, act=qa)


def linear_w4a16(prep: dict, X_bits, out: str = "bf16") -> dict:
    """Weight-only 4-bit layer (16-bit activations): Y = x_hat dequant(Q(R)) + b.

    [diffusers] page: next to the W4A4 operator for the attention and MLP
    layers, the engine runs a second one with 4-bit weights and 16-bit
    activations for the adaptive-norm and modulation projections.  Reading: the prepared layer with rank 0 (R = W_hat), the same
    smoothing x_hat = fp32(x * inv_lambda) and the same weight codes and
    scales; the activations are not quantized; the product in fp64.
    """
    assert prep["rank"] == 0
    xh = smooth_act(X_bits, prep["inv32"])
    Wdq = dequant_groups(prep["w_codes"].T, prep["w_scales"].T, prep["fmt"]).T
    bias = 0.0 if prep["bias"] is None else prep["bias"][None, :]
    Y64 = xh @ Wdq + bias
    return dict(Y64=Y64, Y=_round_out(Y64, out), xhat=xh)


def linear_unfused(prep: dict, X_bits, out: str = "bf16", norm=None) -> dict:
    """Unfused rounding model: Yp = round(main + b); Y = round(Yp + Tb L2b)."""
    r = linear(prep, X_bits, out, norm)
    bias = 0.0 if prep["bias"] is None else prep["bias"][None, :]
    Yp = _round_out(r["main"] + bias, out)
    r["Yp"] = Yp
    r["Y"] = _round_out(Yp + r["low"], out)
    return r


def linear_rows(prep: dict, X_bits_rows, out: str = "bf16") -> dict:
    """``linear`` on a subset of token rows (rows are independent)."""
    return linear(prep, X_bits_rows, out)


# ============================================================ error analysis


def q_eq1(x, bits: int, axis=None) -> np.ndarray:
    """Q(x) of [walkthrough] eq. (1) as real values, for the pages' toy
    tables: s * round(x / s) with s = max|x| / q_max and q_max = 2^(bits-1) - 1,
    one scale for the whole tensor (axis None) or one per slice along
    ``axis``; round is half-to-even of the fp64 quotient (the toy tables
    are printed to 4 decimals).  A slice with max|x| = 0 quantizes to 0 (the
    group reading of ``quantize_int4_groups``).  |x / s| <= q_max holds by
    the choice of s, so no clamp is needed."""
    x = np.asarray(x, dtype=np.float64)
    q_max = float(2 ** (bits - 1) - 1)
    s = np.broadcast_to(np.max(np.abs(x), axis=axis, keepdims=axis is not None) / q_max, x.shape)
    codes = np.rint(np.divide(x, s, out=np.zeros_like(x), where=s > 0))
    return codes * s


def eq5_toy(x_hat, W_hat, rank: int, bits: int) -> np.ndarray:
    """[walkthrough] eq. (5) with the toy tables' per-tensor quantizer:
    X_hat L1 L2 + Q(X_hat) Q(R), R = W_hat - L1 L2, L1 L2 the rank-r SVD
    factors (no bf16 rounding: the toy tables keep the branch in high
    precision)."""
    L1, L2 = lowrank_factors(W_hat, rank)
    R = residual(W_hat, L1, L2)
    return q_eq1(x_hat, bits) @ q_eq1(R, bits) + (x_hat @ L1) @ L2


def quant_error(X, W, QX, QW) -> float:
    """[walkthrough] eq. (3): E(X, W) = ||X W - Q(X) Q(W)||_F."""
    return float(np.linalg.norm(X @ W - QX @ QW))


def prop41_bound(X, W, QX, QW) -> float:
    """[walkthrough] eq. (4)/(9): ||X||_F ||W - Q(W)||_F
    + ||X - Q(X)||_F (||W||_F + ||W - Q(W)||_F)."""
    nf = np.linalg.norm
    return float(nf(X) * nf(W - QW) + nf(X - QX) * (nf(W) + nf(W - QW)))


def gaussian_c(size: int) -> float:
    """[walkthrough] eq. (12)-(14): c = sqrt(pi * log(size) / size) for Gaussian R."""
    return float(np.sqrt(np.pi * np.log(size) / size))


def rel_fro(a, b) -> float:
    """||a - b||_F / ||b||_F."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))
