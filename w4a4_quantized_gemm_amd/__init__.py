"""Python binding of libsvdq (the SVDQuant W4A4 linear layer for MI355X).

Argument marshalling only: every function here forwards torch tensors'
device pointers and the current HIP stream to the C ABI declared in
``include/svdq.h`` and raises ``SvdqError`` on a non-zero status.  All
arithmetic runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")

INT4 = 0   # SVDQ_INT4_G64_FP16
FP4 = 1    # SVDQ_FP4_E2M1_G32_E8M0
OUT_BF16 = 0
OUT_F32 = 1
F_NO_SMOOTHING = 1
F_FACTORS_GIVEN = 2
F_HAS_BIAS = 4

FORMAT_NAMES = {"int4": INT4, "fp4": FP4}
GROUP = {INT4: 64, FP4: 32}

STATUS_NAMES = {
    0: "SVDQ_OK", 1: "SVDQ_ERR_INVALID_ARGUMENT", 2: "SVDQ_ERR_UNSUPPORTED_SHAPE",
    3: "SVDQ_ERR_UNSUPPORTED_DEVICE", 4: "SVDQ_ERR_BUFFER_TOO_SMALL", 5: "SVDQ_ERR_HIP",
    6: "SVDQ_ERR_BAD_BLOB", 7: "SVDQ_ERR_MISALIGNED",
}

# every symbol include/svdq.h declares
EXPORTED = (
    "svdq_status_string", "svdq_version", "svdq_prepared_bytes", "svdq_workspace_bytes",
    "svdq_act_sizes", "svdq_act_absmax", "svdq_prepare_weights", "svdq_prepare_weights_gptq", "svdq_merge_lowrank",
    "svdq_check_blob",
    "svdq_quantize_act", "svdq_quantize_act_ln", "svdq_gemm", "svdq_linear", "svdq_linear_ln", "svdq_linear_w4a16",
    "svdq_linear_unfused", "svdq_blob_layout_of", "svdq_linear_noalloc",
)

# bytes of the library's scratch array behind svdq_linear_noalloc (per device)
NOALLOC_SCRATCH_BYTES = 64 << 20


class SvdqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().svdq_status_string(status).decode() if _LIB is not None else STATUS_NAMES.get(status, "?")
        super().__init__(f"{where}: {msg} (status {status})")


class LayerDesc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("fmt", ctypes.c_int32), ("alpha", ctypes.c_float), ("flags", ctypes.c_uint32)]

    def __repr__(self):
        return (f"LayerDesc(K={self.K}, N={self.N}, rank={self.rank}, fmt={self.fmt}, "
                f"alpha={self.alpha}, flags={self.flags})")


class BlobLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in
                ("header", "lambda_", "inv_lambda", "l1t", "l2t", "wcodes", "wscales", "bias", "total")]


_LIB: Optional[ctypes.CDLL] = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m w4a4_quantized_gemm_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I, Z, S, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
        D = ctypes.POINTER(LayerDesc)
        sig = {
            "svdq_status_string": ([I], ctypes.c_char_p),
            "svdq_version": ([], I),
            "svdq_prepared_bytes": ([D], Z),
            "svdq_workspace_bytes": ([D, I, I], Z),
            "svdq_act_sizes": ([D, I, ctypes.POINTER(Z), ctypes.POINTER(Z), ctypes.POINTER(Z)], S),
            "svdq_act_absmax": ([P, I, I, P, I, P], S),
            "svdq_prepare_weights": ([D, P, P, P, P, P, P, Z, P], S),
            "svdq_prepare_weights_gptq": ([D, P, P, P, P, P, P, I, F, P, Z, P], S),
            "svdq_merge_lowrank": ([D, P, P, P, I, P, Z, P], S),
            "svdq_check_blob": ([D, P, P], S),
            "svdq_quantize_act": ([D, P, P, I, P, P, P, P, Z, P], S),
            "svdq_quantize_act_ln": ([D, P, P, P, P, F, I, P, P, P, P, Z, P], S),
            "svdq_gemm": ([D, P, P, P, P, I, P, I, P, Z, P], S),
            "svdq_linear_ln": ([D, P, P, P, P, F, I, P, I, P, Z, P], S),
            "svdq_linear_w4a16": ([D, P, P, I, P, I, P, Z, P], S),
            "svdq_linear": ([D, P, P, I, P, I, P, Z, P], S),
            "svdq_linear_unfused": ([D, P, P, I, P, I, P, Z, P], S),
            "svdq_linear_noalloc": ([D, P, P, I, P, I, P], S),
            "svdq_blob_layout_of": ([D, ctypes.POINTER(BlobLayout)], S),
        }
        for name, (args, res) in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = lib
    return _LIB


def load() -> ctypes.CDLL:
    """Load libsvdq.so (raises ImportError if it has not been built)."""
    return _lib()


def _check(status: int, where: str):
    if status != 0:
        raise SvdqError(status, where)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_desc(K: int, N: int, rank: int, fmt, alpha: float = 0.5, flags: int = 0) -> LayerDesc:
    if isinstance(fmt, str):
        fmt = FORMAT_NAMES[fmt]
    return LayerDesc(K, N, rank, fmt, alpha, flags)


# ----------------------------------------------------------------- size queries
def svdq_prepared_bytes(desc: LayerDesc) -> int:
    return _lib().svdq_prepared_bytes(ctypes.byref(desc))


def svdq_workspace_bytes(desc: LayerDesc, M: int, unfused: bool = False) -> int:
    return _lib().svdq_workspace_bytes(ctypes.byref(desc), M, int(unfused))


def svdq_act_sizes(desc: LayerDesc, M: int):
    c, s, t = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib().svdq_act_sizes(ctypes.byref(desc), M, ctypes.byref(c), ctypes.byref(s), ctypes.byref(t)),
           "svdq_act_sizes")
    return c.value, s.value, t.value


def svdq_blob_layout_of(desc: LayerDesc) -> BlobLayout:
    out = BlobLayout()
    _check(_lib().svdq_blob_layout_of(ctypes.byref(desc), ctypes.byref(out)), "svdq_blob_layout_of")
    return out


# ----------------------------------------------------------------- GPU calls
def svdq_act_absmax(X, out, accumulate: bool = False, stream=None):
    """out[j] = max_i |X[i, j]| (X: M x K bf16 tensor, out: K float32 tensor)."""
    M, K = X.shape
    _check(_lib().svdq_act_absmax(_ptr(X), M, K, _ptr(out), int(accumulate), _stream(stream)),
           "svdq_act_absmax")


def svdq_prepare_weights(desc: LayerDesc, W, act_absmax, prepared, bias=None, L1=None, L2=None,
                         stream=None):
    """Offline preparation into the uint8 device tensor ``prepared`` (synchronous)."""
    _check(_lib().svdq_prepare_weights(ctypes.byref(desc), _ptr(W), _ptr(act_absmax), _ptr(bias),
                                       _ptr(L1), _ptr(L2), _ptr(prepared), prepared.numel(),
                                       _stream(stream)), "svdq_prepare_weights")


def svdq_prepare_weights_gptq(desc: LayerDesc, W, act_absmax, prepared, Xcal, damp: float = 0.01, bias=None, L1=None,
                              L2=None, stream=None):
    """Offline preparation with the residual quantized by GPTQ on the
    calibration activations ``Xcal`` (bf16, M_cal x K); synchronous."""
    _check(_lib().svdq_prepare_weights_gptq(ctypes.byref(desc), _ptr(W), _ptr(act_absmax), _ptr(bias), _ptr(L1),
                                            _ptr(L2), _ptr(Xcal), Xcal.shape[0], float(damp), _ptr(prepared),
                                            prepared.numel(), _stream(stream)), "svdq_prepare_weights_gptq")


def svdq_merge_lowrank(desc: LayerDesc, prepared, A, B, out, stream=None):
    """Merge an extra low-rank branch dW = A B (A: K x r_extra, B: r_extra x N,
    bf16 tensors) into ``out``, the blob of ``desc`` with rank + r_extra
    (synchronous)."""
    r_extra = A.shape[1]
    _check(_lib().svdq_merge_lowrank(ctypes.byref(desc), _ptr(prepared), _ptr(A), _ptr(B), r_extra, _ptr(out),
                                     out.numel(), _stream(stream)), "svdq_merge_lowrank")


def svdq_check_blob(desc: LayerDesc, prepared, stream=None):
    _check(_lib().svdq_check_blob(ctypes.byref(desc), _ptr(prepared), _stream(stream)), "svdq_check_blob")


def svdq_quantize_act(desc: LayerDesc, prepared, X, codes, scales, T=None, workspace=None, stream=None):
    """The activation pass; `workspace` (optional, svdq_workspace_bytes(desc, M) bytes) lets it split K."""
    M = X.shape[0]
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib().svdq_quantize_act(ctypes.byref(desc), _ptr(prepared), _ptr(X), M, _ptr(codes),
                                    _ptr(scales), _ptr(T), _ptr(workspace), ws_bytes, _stream(stream)),
           "svdq_quantize_act")


def svdq_quantize_act_ln(desc: LayerDesc, prepared, X, gamma, beta, eps: float, codes, scales, T, workspace,
                         stream=None):
    """The norm-fused activation pass: X is the LayerNorm's input; gamma and
    beta (bf16 [K], beta may be None) its affine; the workspace is required."""
    M = X.shape[0]
    _check(_lib().svdq_quantize_act_ln(ctypes.byref(desc), _ptr(prepared), _ptr(X), _ptr(gamma), _ptr(beta),
                                       float(eps), M, _ptr(codes), _ptr(scales), _ptr(T), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)),
           "svdq_quantize_act_ln")


def svdq_linear_ln(desc: LayerDesc, prepared, X, gamma, beta, eps: float, Y, workspace, out_dtype: int = OUT_BF16,
                   stream=None):
    M = X.shape[0]
    _check(_lib().svdq_linear_ln(ctypes.byref(desc), _ptr(prepared), _ptr(X), _ptr(gamma), _ptr(beta), float(eps),
                                 M, _ptr(Y), out_dtype, _ptr(workspace), workspace.numel(), _stream(stream)),
           "svdq_linear_ln")


def svdq_linear_w4a16(desc: LayerDesc, prepared, X, Y, workspace, out_dtype: int = OUT_BF16, stream=None):
    """The weight-only 4-bit layer (rank-0 blob, M <= 16 rows, bf16 activations)."""
    M = X.shape[0]
    _check(_lib().svdq_linear_w4a16(ctypes.byref(desc), _ptr(prepared), _ptr(X), M, _ptr(Y), out_dtype,
                                    _ptr(workspace), workspace.numel(), _stream(stream)), "svdq_linear_w4a16")


def svdq_gemm(desc: LayerDesc, prepared, codes, scales, T, M: int, Y, out_dtype: int = OUT_BF16,
              workspace=None, stream=None):
    """The GEMM stage alone, on the outputs of svdq_quantize_act (workspace
    optional: with it a small INT4 GEMM may split K)."""
    _check(_lib().svdq_gemm(ctypes.byref(desc), _ptr(prepared), _ptr(codes), _ptr(scales), _ptr(T), M,
                            _ptr(Y), out_dtype, _ptr(workspace), 0 if workspace is None else workspace.numel(),
                            _stream(stream)), "svdq_gemm")


def svdq_linear(desc: LayerDesc, prepared, X, Y, workspace, out_dtype: int = OUT_BF16, stream=None):
    M = X.shape[0]
    _check(_lib().svdq_linear(ctypes.byref(desc), _ptr(prepared), _ptr(X), M, _ptr(Y), out_dtype,
                              _ptr(workspace), workspace.numel(), _stream(stream)), "svdq_linear")


def svdq_linear_unfused(desc: LayerDesc, prepared, X, Y, workspace, out_dtype: int = OUT_BF16, stream=None):
    M = X.shape[0]
    _check(_lib().svdq_linear_unfused(ctypes.byref(desc), _ptr(prepared), _ptr(X), M, _ptr(Y), out_dtype,
                                      _ptr(workspace), workspace.numel(), _stream(stream)),
           "svdq_linear_unfused")


def svdq_linear_noalloc(desc: LayerDesc, prepared, X, Y, out_dtype: int = OUT_BF16, stream=None):
    """svdq_linear with the library's own scratch array instead of a
    workspace (for callers that cannot allocate); calls that overlap on one
    device race on that array."""
    M = X.shape[0]
    _check(_lib().svdq_linear_noalloc(ctypes.byref(desc), _ptr(prepared), _ptr(X), M, _ptr(Y), out_dtype,
                                      _stream(stream)),
           "svdq_linear_noalloc")


# ----------------------------------------------------------------- convenience
def blob_factors(desc: LayerDesc, blob_bytes):
    """The stored bf16 factor bits of a prepared blob (a host uint8 array):
    L1 transposed (rank x K) and L2 transposed (N x rank), each as uint16,
    row-major, undoing the blob's operand orders (layouts documented in
    include/svdq.h)."""
    import numpy as np
    L = svdq_blob_layout_of(desc)
    K, N, r = desc.K, desc.N, desc.rank
    t = np.arange(r)[:, None]
    k = np.arange(K)[None, :]
    off1 = (((k // 128) * (r // 16) + t // 16) * 4 + (k % 32) // 8) * 512 + (t % 16 + 16 * ((k % 128) // 32)) * 8 + k % 8
    l1t = blob_bytes[L.l1t:L.l1t + 2 * r * K].view(np.uint16)[off1]
    n = np.arange(N)[:, None]
    t2 = np.arange(r)[None, :]
    off2 = ((n // 32) * (r // 16) + t2 // 16) * 512 + (n % 32 + 32 * ((t2 % 16) // 8)) * 8 + t2 % 8
    l2t = blob_bytes[L.l2t:L.l2t + 2 * N * r].view(np.uint16)[off2]
    return l1t, l2t


class SVDQLinear:
    """A prepared layer held on the GPU: the blob plus its descriptor.

    ``SVDQLinear.prepare(W, act_absmax, rank, fmt, ...)`` runs the offline
    preparation; ``layer(X)`` runs the fused forward pass.  Buffers are torch
    tensors (device memory); the arithmetic is the library's.
    """

    def __init__(self, desc: LayerDesc, blob):
        self.desc = desc
        self.blob = blob
        self._ws = None

    @classmethod
    def prepare(cls, W, act_absmax, rank: int, fmt="int4", alpha: float = 0.5, bias=None,
                L1=None, L2=None, no_smoothing: bool = False, stream=None, gptq=None) -> "SVDQLinear":
        """``gptq`` = (calibration X, damping) quantizes the residual with GPTQ."""
        import torch
        K, N = W.shape
        flags = (F_HAS_BIAS if bias is not None else 0) | (F_NO_SMOOTHING if no_smoothing else 0) | \
                (F_FACTORS_GIVEN if L1 is not None else 0)
        desc = make_desc(K, N, rank, fmt, alpha, flags)
        nbytes = svdq_prepared_bytes(desc)
        if nbytes == 0:
            raise SvdqError(2, "svdq_prepared_bytes")
        blob = torch.empty(nbytes, dtype=torch.uint8, device=W.device)
        if gptq is not None:
            svdq_prepare_weights_gptq(desc, W, act_absmax, blob, gptq[0], gptq[1], bias=bias, L1=L1, L2=L2,
                                      stream=stream)
        else:
            svdq_prepare_weights(desc, W, act_absmax, blob, bias=bias, L1=L1, L2=L2, stream=stream)
        return cls(desc, blob)

    def merge_lowrank(self, A, B, stream=None) -> "SVDQLinear":
        """A new layer with the extra low-rank branch dW = A B (e.g. a LoRA)
        merged into the 16-bit branch; the quantized residual is shared
        unchanged (copied)."""
        import torch
        d = self.desc
        desc = make_desc(d.K, d.N, d.rank + A.shape[1], d.fmt, d.alpha, d.flags)
        nbytes = svdq_prepared_bytes(desc)
        if nbytes == 0:
            raise SvdqError(2, "svdq_prepared_bytes")
        blob = torch.empty(nbytes, dtype=torch.uint8, device=self.blob.device)
        svdq_merge_lowrank(d, self.blob, A, B, blob, stream)
        return SVDQLinear(desc, blob)

    def workspace(self, M: int, unfused: bool = False):
        import torch
        need = svdq_workspace_bytes(self.desc, M, unfused)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.blob.device)
        return self._ws

    def __call__(self, X, out_dtype: int = OUT_BF16, unfused: bool = False, Y=None, stream=None, norm=None):
        """Y = layer(X); with ``norm`` = (gamma, beta, eps), X is the input of
        the preceding LayerNorm, which runs fused into the activation pass."""
        import torch
        M = X.shape[0]
        if Y is None:
            Y = torch.empty((M, self.desc.N), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32,
                            device=X.device)
        if norm is not None:
            if unfused:
                raise ValueError("the norm-fused pass exists for the fused layer only")
            svdq_linear_ln(self.desc, self.blob, X, norm[0], norm[1], norm[2], Y, self.workspace(M), out_dtype, stream)
            return Y
        fn = svdq_linear_unfused if unfused else svdq_linear
        fn(self.desc, self.blob, X, Y, self.workspace(M, unfused), out_dtype, stream)
        return Y

    def section(self, name: str):
        """A uint8 view of one blob section (lambda_, inv_lambda, l1t, l2t, wcodes, wscales, bias)."""
        L = svdq_blob_layout_of(self.desc)
        names = ["header", "lambda_", "inv_lambda", "l1t", "l2t", "wcodes", "wscales", "bias", "total"]
        offs = [getattr(L, n) for n in names]
        i = names.index(name)
        start = offs[i]
        nxt = [o for o in offs[i + 1:] if o > start]
        end = min(nxt) if nxt else L.total
        return self.blob[start:end]
