"""Test helpers: read libsvdq's buffers back into the canonical arrays the
oracle produces.  The decoding follows the byte layouts documented in
include/svdq.h; it is test code, shared by neither the oracle nor the
library."""
from __future__ import annotations

import numpy as np

import oracle as O


def to_np(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def u16_tensor_to_np(t) -> np.ndarray:
    """bf16 / fp16 / int16 tensor -> raw uint16 bits."""
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def np_bits_to_bf16_tensor(bits: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def untile_codes(raw: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Code bytes stored in the MFMA operand-block order of include/svdq.h ->
    row-major [rows][K/2].  The byte of codes (k, k+1) of row i sits at
    ((i/32)*(K/64) + k/64)*1024 + (i%32 + 32*((k%64)/32))*16 + (k%32)/2."""
    raw = np.asarray(raw).reshape(-1)
    i = np.arange(rows, dtype=np.int64)[:, None]
    k = 2 * np.arange(K // 2, dtype=np.int64)[None, :]
    off = ((i // 32) * (K // 64) + k // 64) * 1024 + (i % 32 + 32 * ((k % 64) // 32)) * 16 + (k % 32) // 2
    assert off.max() < raw.size, "code buffer smaller than the block layout needs"
    return raw[off]


def int4_words_to_q(raw: np.ndarray) -> np.ndarray:
    """INT4 codes from code bytes in K order (rows x K/2, as untile_codes
    returns them) -> rows x K int8, per the word format of include/svdq.h:
    each little-endian 32-bit word holds codes k .. k+7; code j < 4 is byte
    j of (word & 0x87878787), code j >= 4 byte j-4 of (rotr(word, 4) &
    0x87878787); a byte is sign (bit 7) and magnitude (bits 0-2).  A
    negative zero (byte 0x80) is rejected: zero must be encoded +0."""
    raw = np.asarray(raw, dtype=np.uint8)
    rows, half = raw.shape
    b = raw.reshape(rows, half // 4, 4).astype(np.uint64)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    lo = w & 0x87878787
    hi = ((w >> 4) | (w << 28)) & 0xFFFFFFFF & 0x87878787
    c = np.empty((rows, half // 4, 8), dtype=np.int64)
    for j in range(4):
        c[..., j] = (lo >> (8 * j)) & 0xFF
        c[..., 4 + j] = (hi >> (8 * j)) & 0xFF
    assert not np.any(c == 0x80), "INT4 zero encoded with the sign bit set"
    q = (c & 7) * np.where(c & 0x80, -1, 1)
    return q.reshape(rows, 2 * half).astype(np.int8)


def q_to_int4_words(q: np.ndarray) -> np.ndarray:
    """Inverse of int4_words_to_q: rows x K integer codes in [-7, 7] -> rows x
    K/2 code bytes in K order."""
    q = np.asarray(q, dtype=np.int64)
    rows, K = q.shape
    assert np.all(np.abs(q) <= 7)
    c = (np.where(q < 0, 0x80, 0) | np.abs(q)).astype(np.uint64).reshape(rows, K // 8, 8)
    lo = c[..., 0] | (c[..., 1] << 8) | (c[..., 2] << 16) | (c[..., 3] << 24)
    hi = c[..., 4] | (c[..., 5] << 8) | (c[..., 6] << 16) | (c[..., 7] << 24)
    w = (lo | (((hi << 4) | (hi >> 28)) & 0xFFFFFFFF)).astype(np.uint32)
    return w.view(np.uint8).reshape(rows, K // 2)


def untile_bf16(raw_u16: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """bf16 matrix (as uint16) stored in the operand-block order of
    include/svdq.h -> row-major [rows][cols].  Element (i, t) sits at
    ((i/32)*(cols/16) + t/16)*512 + (i%32 + 32*((t%16)/8))*8 + t%8."""
    raw = np.asarray(raw_u16).reshape(-1)
    i = np.arange(rows, dtype=np.int64)[:, None]
    t = np.arange(cols, dtype=np.int64)[None, :]
    off = ((i // 32) * (cols // 16) + t // 16) * 512 + (i % 32 + 32 * ((t % 16) // 8)) * 8 + t % 8
    if off.size == 0:
        return np.zeros((rows, cols), dtype=raw.dtype)
    assert off.max() < raw.size, "bf16 buffer smaller than the block layout needs"
    return raw[off]


def untile_fp4_scales(raw: np.ndarray, rows: int, K: int) -> np.ndarray:
    """FP4 E8M0 scale bytes in operand-block order -> [rows][K/32].  The byte
    of (row i, group k/32) sits at
    ((i/32)*(K/128) + k/128)*128 + (i%32 + 32*((k/32)%2))*2 + (k/64)%2."""
    raw = np.asarray(raw).reshape(-1)
    i = np.arange(rows, dtype=np.int64)[:, None]
    k = 32 * np.arange(K // 32, dtype=np.int64)[None, :]
    off = ((i // 32) * (K // 128) + k // 128) * 128 + (i % 32 + 32 * ((k // 32) % 2)) * 2 + (k // 64) % 2
    assert off.max() < raw.size, "scale buffer smaller than the block layout needs"
    return raw[off]


def untile_l1(raw_u16: np.ndarray, r: int, K: int) -> np.ndarray:
    """r x K matrix from the L1 operand order (1 KB blocks per 128-wide K
    chunk, 16-row block and 8-wide step, in 16x16x32 MFMA lane order)."""
    out = np.empty((r, K), dtype=raw_u16.dtype)
    blocks = raw_u16.reshape(K // 128, r // 16, 4, 4, 16, 8)   # chunk, t block, step j, kq, t % 16, k % 8
    for c in range(K // 128):
        for nb in range(r // 16):
            for j in range(4):
                for kq in range(4):
                    k0 = c * 128 + kq * 32 + j * 8
                    out[nb * 16:nb * 16 + 16, k0:k0 + 8] = blocks[c, nb, j, kq]
    return out


def blob_sections(layer):
    """Canonical numpy views of a prepared blob.

    Returns dict(lam32, inv32, L1b (K x r), L2b (r x N), w_codes (K x N),
    w_scales (K/g x N values: fp16 values for INT4, exponents for FP4),
    bias (N or None), raw_wcodes, raw_wscales)."""
    import ctypes
    from w4a4_quantized_gemm_amd import svdq_blob_layout_of, INT4
    d = layer.desc
    L = svdq_blob_layout_of(d)
    blob = to_np(layer.blob)
    K, N, r = d.K, d.N, d.rank
    g = 64 if d.fmt == INT4 else 32

    def sec(off, nbytes):
        return blob[off:off + nbytes]

    lam32 = sec(L.lambda_, 4 * K).view(np.float32).astype(np.float64)
    inv32 = sec(L.inv_lambda, 4 * K).view(np.float32).astype(np.float64)
    l1t = untile_l1(sec(L.l1t, 2 * r * K).view(np.uint16), r, K)
    l2t = untile_bf16(sec(L.l2t, 2 * N * r).view(np.uint16), N, r)
    L1b = O.bf16_bits_to_f64(l1t).T.copy()
    L2b = O.bf16_bits_to_f64(l2t).T.copy()
    raw_codes = untile_codes(sec(L.wcodes, N * K // 2), N, K)
    if d.fmt == INT4:
        q = int4_words_to_q(raw_codes)                       # N x K
        codes = q.T.copy()
        raw_codes = O.pack_nibbles(O.int4_nibble(q))         # the oracle's byte format
        raw_scales = sec(L.wscales, 2 * (K // g) * N).view(np.uint16).reshape(N, K // g).T
        scales = O.fp16_bits_to_f64(raw_scales)
    else:
        codes = O.unpack_nibbles(raw_codes).T.copy()
        raw_scales = untile_fp4_scales(sec(L.wscales, (K // g) * N), N, K).T
        scales = raw_scales.astype(np.int32) - 127
    bias = None
    if d.flags & 4:
        bias = sec(L.bias, 4 * N).view(np.float32).astype(np.float64)
    return dict(lam32=lam32, inv32=inv32, L1b=L1b, L2b=L2b, w_codes=codes, w_scales=scales,
                bias=bias, raw_wcodes=raw_codes, raw_wscales=raw_scales, l1t=l1t, l2t=l2t)


def oracle_prep_from_blob(sections, W_bits, fmt: str, bias_bits=None, cols=None, lam32=None) -> dict:
    """The oracle's prepared layer built on the blob's stored L1b, L2b (the
    SVD factors are not unique, so parity is checked given them) and on
    ``lam32`` (the oracle's own smoothing factors; the blob's when None).
    ``cols`` restricts the residual to a subset of output columns."""
    W = O.bf16_bits_to_f64(W_bits)
    lam32 = sections["lam32"] if lam32 is None else np.asarray(lam32, dtype=np.float64)
    inv32 = O.to_fp32(1.0 / lam32)
    L2b = sections["L2b"]
    if cols is not None:
        W = W[:, cols]
        L2b = L2b[:, cols]
        if bias_bits is not None:
            bias_bits = bias_bits[cols]
    W_hat = lam32[:, None] * W
    R = O.residual(W_hat, sections["L1b"], L2b)
    w_codes, w_scales = O.quantize_weights(R, fmt)
    bias = None if bias_bits is None else O.bf16_bits_to_f64(bias_bits)
    return dict(fmt=fmt, K=W.shape[0], N=W.shape[1], rank=sections["L1b"].shape[1], lam32=lam32,
                inv32=inv32, W_hat=W_hat, L1b=sections["L1b"], L2b=L2b, R=R, w_codes=w_codes,
                w_scales=w_scales, bias=bias)


def untile_int4_act_scales(raw_u16: np.ndarray, M: int, K: int) -> np.ndarray:
    """M x K/64 fp16 bits from the INT4 activation scale blocks: per 32-row
    block and 128-wide stage, 32 words of the stage's two groups."""
    i = np.arange(M)[:, None]
    g = np.arange(K // 64)[None, :]
    off = ((i // 32) * (K // 128) + g // 2) * 64 + (i % 32) * 2 + g % 2
    assert off.max() < raw_u16.size, "scale buffer smaller than the block layout needs"
    return raw_u16[off]


def decode_act(codes_t, scales_t, fmt_id: int, M: int, K: int):
    """Packed activation codes / scales from the GPU -> (codes M x K, scale
    values, codes packed in the oracle's byte format, raw scale bits)."""
    from w4a4_quantized_gemm_amd import INT4
    raw = untile_codes(to_np(codes_t), M, K)
    if fmt_id == INT4:
        q = int4_words_to_q(raw)
        sc = untile_int4_act_scales(to_np(scales_t).view(np.uint16), M, K)
        return q, O.fp16_bits_to_f64(sc), O.pack_nibbles(O.int4_nibble(q)), sc
    sc = untile_fp4_scales(to_np(scales_t), M, K)
    return O.unpack_nibbles(raw), sc.astype(np.int32) - 127, raw, sc
