"""CPU tests of the C ABI boundary: the library loads, exports every symbol
the header declares, validates arguments before touching a device, and its
host-side helpers (blob layout, eigensolver) are right.  No compute call
reaches a GPU here."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

import w4a4_quantized_gemm_amd as S  # noqa: E402


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(svdq_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = S.load()
    declared = _declared_functions()
    assert set(declared) == set(S.EXPORTED), (declared, S.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", S.LIB_PATH], capture_output=True, text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in declared:
        assert name in syms, name


def test_peaks_library_exports_its_header():
    """The peak-measurement probes (libsvdq_peaks.so) export what
    include/svdq_peaks.h declares, and refuse invalid arguments before any
    device call."""
    hdr = os.path.join(ROOT, "include", "svdq_peaks.h")
    text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(svdq_[a-z_0-9]+)\s*\(", text)))
    path = os.path.join(ROOT, "w4a4_quantized_gemm_amd", "libsvdq_peaks.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True).stdout
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    assert declared == ["svdq_peak_hbm", "svdq_peak_mfma"]
    assert all(n in syms for n in declared)
    lib = ctypes.CDLL(path)
    d = ctypes.c_double()
    lib.svdq_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.svdq_peak_hbm.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    assert lib.svdq_peak_mfma(9, 10, 0, 0, 1 << 20, ctypes.byref(d), ctypes.byref(d), None) == 1
    assert lib.svdq_peak_mfma(0, 0, 0, 0, 1 << 20, ctypes.byref(d), ctypes.byref(d), None) == 1
    assert lib.svdq_peak_hbm(2, 1 << 20, 1 << 21, 1 << 20, ctypes.byref(d), ctypes.byref(d), None) == 1
    assert lib.svdq_peak_hbm(0, 1 << 20, 1 << 21, 17, ctypes.byref(d), ctypes.byref(d), None) == 1


def test_status_strings_and_version():
    lib = S.load()
    for code, name in S.STATUS_NAMES.items():
        assert lib.svdq_status_string(code).decode().startswith(name)
    assert lib.svdq_status_string(999).decode() == "unknown svdq_status"
    assert lib.svdq_version() >= 100


def _desc(K=3072, N=9216, r=32, fmt=S.INT4, alpha=0.5, flags=0):
    return S.make_desc(K, N, r, fmt, alpha, flags)


@pytest.mark.parametrize("kw", [
    dict(K=100), dict(K=64), dict(K=3072 + 64), dict(N=32), dict(N=100), dict(r=8), dict(r=144),
    dict(r=-16), dict(K=128, r=144),
])
def test_unsupported_shapes(kw):
    d = _desc(**kw)
    assert S.svdq_prepared_bytes(d) == 0
    assert S.svdq_workspace_bytes(d, 16) == 0
    lib = S.load()
    st = lib.svdq_prepare_weights(ctypes.byref(d), 16, 16, None, None, None, 16, 1 << 30, None)
    assert st == 2


@pytest.mark.parametrize("kw", [dict(fmt=7), dict(alpha=-0.1), dict(alpha=1.5), dict(alpha=float("nan")),
                                dict(flags=64)])
def test_invalid_arguments(kw):
    d = _desc(**kw)
    lib = S.load()
    assert S.svdq_prepared_bytes(d) == 0
    assert lib.svdq_linear(ctypes.byref(d), 256, 256, 16, 256, 0, 256, 1 << 40, None) == 1


def test_runtime_validation_before_device():
    lib = S.load()
    d = _desc()
    ws = S.svdq_workspace_bytes(d, 4608)
    good = 1 << 20   # any 16-byte aligned non-null value: never dereferenced when validation fails
    # NULL pointers
    assert lib.svdq_linear(ctypes.byref(d), None, good, 4608, good, 0, good, ws, None) == 1
    assert lib.svdq_linear(ctypes.byref(d), good, good, 4608, None, 0, good, ws, None) == 1
    assert lib.svdq_linear(None, good, good, 4608, good, 0, good, ws, None) == 1
    # bad M, bad output dtype
    assert lib.svdq_linear(ctypes.byref(d), good, good, 0, good, 0, good, ws, None) == 2
    assert lib.svdq_linear(ctypes.byref(d), good, good, -5, good, 0, good, ws, None) == 2
    assert lib.svdq_linear(ctypes.byref(d), good, good, 4608, good, 3, good, ws, None) == 1
    # misaligned
    assert lib.svdq_linear(ctypes.byref(d), good + 8, good, 4608, good, 0, good, ws, None) == 7
    assert lib.svdq_linear_unfused(ctypes.byref(d), good, good, 4608, good + 2, 0, good, ws, None) == 7
    # workspace too small
    assert lib.svdq_linear(ctypes.byref(d), good, good, 4608, good, 0, good, ws - 1, None) == 4
    # prepared buffer too small; missing act_absmax / bias / factors
    pb = S.svdq_prepared_bytes(d)
    assert lib.svdq_prepare_weights(ctypes.byref(d), good, good, None, None, None, good, pb - 1, None) == 4
    assert lib.svdq_prepare_weights(ctypes.byref(d), good, None, None, None, None, good, pb, None) == 1
    db = _desc(flags=S.F_HAS_BIAS)
    assert lib.svdq_prepare_weights(ctypes.byref(db), good, good, None, None, None, good, pb, None) == 1
    dg = _desc(flags=S.F_FACTORS_GIVEN)
    assert lib.svdq_prepare_weights(ctypes.byref(dg), good, good, None, None, None, good, pb, None) == 1
    # prepare_weights_gptq: calibration activations required, damp >= 0 and finite, M_cal >= 1
    pg = lib.svdq_prepare_weights_gptq
    assert pg(ctypes.byref(d), good, good, None, None, None, None, 512, 0.01, good, pb, None) == 1
    assert pg(ctypes.byref(d), good, good, None, None, None, good, 512, -1.0, good, pb, None) == 1
    assert pg(ctypes.byref(d), good, good, None, None, None, good, 512, float("nan"), good, pb, None) == 1
    assert pg(ctypes.byref(d), good, good, None, None, None, good, 0, 0.01, good, pb, None) == 2
    assert pg(ctypes.byref(d), good, good, None, None, None, good, 512, 0.01, good, pb - 1, None) == 4
    # merge_lowrank: r_extra a positive multiple of 16 with rank + r_extra <= 128;
    # pointers, alignment, the output size and no overlap with the input
    out = 1 << 30
    d48 = _desc(r=48)
    pb48 = S.svdq_prepared_bytes(d48)
    merge = lib.svdq_merge_lowrank
    assert merge(ctypes.byref(d), good, good, good, 0, out, pb48, None) == 2
    assert merge(ctypes.byref(d), good, good, good, 8, out, pb48, None) == 2
    assert merge(ctypes.byref(d), good, good, good, 112, out, 1 << 40, None) == 2
    assert merge(ctypes.byref(d), good, None, good, 16, out, pb48, None) == 1
    assert merge(ctypes.byref(d), good, good, good, 16, None, pb48, None) == 1
    assert merge(ctypes.byref(d), good, good, good, 16, out + 8, pb48, None) == 7
    assert merge(ctypes.byref(d), good, good, good, 16, out, pb48 - 1, None) == 4
    assert merge(ctypes.byref(d), good, good, good, 16, good + 4096, pb48, None) == 1
    # the weight-only layer: rank-0 blobs and at most 16 rows
    d0 = _desc(r=0)
    ws0 = S.svdq_workspace_bytes(d0, 16)
    w16 = lib.svdq_linear_w4a16
    assert w16(ctypes.byref(d), good, good, 4, good, 0, good, ws, None) == 2
    assert w16(ctypes.byref(d0), good, good, 17, good, 0, good, S.svdq_workspace_bytes(d0, 17), None) == 2
    assert w16(ctypes.byref(d0), good, good, 16, None, 0, good, ws0, None) == 1
    # (the last 16 MiB, the partial tiles of a K-split GEMM of this INT4 layer
    # with 72 output tiles at 16 rows, are optional)
    split = 256 * 128 * 128 * 4
    assert w16(ctypes.byref(d0), good, good, 16, good, 0, good, ws0 - split - 1, None) == 4
    assert w16(ctypes.byref(d0), good, good, 16, good, 0, good, ws0 - split, None) != 4
    # the norm-fused calls: gamma required, eps > 0 and finite, workspace required
    ln = lib.svdq_linear_ln
    assert ln(ctypes.byref(d), good, good, None, None, 1e-5, 4608, good, 0, good, ws, None) == 1
    assert ln(ctypes.byref(d), good, good, good, None, 0.0, 4608, good, 0, good, ws, None) == 1
    assert ln(ctypes.byref(d), good, good, good, None, float("inf"), 4608, good, 0, good, ws, None) == 1
    assert ln(ctypes.byref(d), good, good, good, None, 1e-5, 4608, good, 0, good, ws - 1, None) == 4
    qln = lib.svdq_quantize_act_ln
    assert qln(ctypes.byref(d), good, good, good, None, 1e-5, 16, good, good, good, None, ws, None) == 1
    assert qln(ctypes.byref(d), good, good, good, None, 1e-5, 16, good, good, None, good, ws, None) == 1
    # quantize_act: T required when rank > 0
    assert lib.svdq_quantize_act(ctypes.byref(d), good, good, 16, good, good, None, None, 0, None) == 1


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device path")
def test_device_check_without_gpu():
    lib = S.load()
    d = _desc()
    ws = S.svdq_workspace_bytes(d, 64)
    good = 1 << 20
    assert lib.svdq_linear(ctypes.byref(d), good, good, 64, good, 0, good, ws, None) == 3
    assert lib.svdq_act_absmax(good, 64, 3072, good, 0, None) == 3
    d48 = _desc(r=48)
    assert lib.svdq_merge_lowrank(ctypes.byref(d), good, good, good, 16, 1 << 30, S.svdq_prepared_bytes(d48),
                                  None) == 3


def test_blob_layout_and_sizes():
    for fmt, g, sb in ((S.INT4, 64, 2), (S.FP4, 32, 1)):
        for flags in (0, S.F_HAS_BIAS):
            d = _desc(K=3072, N=9216, r=32, fmt=fmt, flags=flags)
            L = S.svdq_blob_layout_of(d)
            offs = [L.header, L.lambda_, L.inv_lambda, L.l1t, L.l2t, L.wcodes, L.wscales]
            sizes = [256, 4 * 3072, 4 * 3072, 2 * 32 * 3072, 2 * 9216 * 32, 9216 * 1536, (3072 // g) * 9216 * sb]
            if flags:
                offs.append(L.bias)
                sizes.append(4 * 9216)
            assert all(o % 256 == 0 for o in offs)
            for (o, s), o_next in zip(zip(offs, sizes), offs[1:] + [L.total]):
                assert o + s <= o_next
            assert L.total == S.svdq_prepared_bytes(d)
            assert (flags == 0) == (L.bias == 0)
            c, s, t = S.svdq_act_sizes(d, 4608)
            assert (c, s, t) == (4608 * 1536, 4608 * (3072 // g) * sb, 4608 * 32 * 2)
            assert S.svdq_workspace_bytes(d, 4608) >= c + s + t
            # codes, scales and T of both formats are padded to whole 32-row blocks
            c, s, t = S.svdq_act_sizes(d, 100)
            assert (c, s, t) == (128 * 1536, 128 * (3072 // g) * sb, 128 * 32 * 2)
    # compression: the 4-bit blob is ~0.27-0.28x the bf16 weight
    d = _desc(K=3072, N=12288, r=32, fmt=S.FP4)
    ratio = S.svdq_prepared_bytes(d) / (3072 * 12288 * 2)
    assert 0.26 < ratio < 0.30


def test_int4_code_word_format():
    """The INT4 word layout of include/svdq.h on a worked example and a round
    trip: codes 1..7, -7 -> low bytes 01 02 03 04 and high bytes 05 06 07 87
    rotated left by 4 -> 0x74736259."""
    from svdq_testlib import int4_words_to_q, q_to_int4_words
    q = np.array([[1, 2, 3, 4, 5, 6, 7, -7]])
    raw = q_to_int4_words(q)
    assert raw.tolist() == [[0x59, 0x62, 0x73, 0x74]]
    assert int4_words_to_q(raw).tolist() == q.tolist()
    # the E4M3 operand bytes: word & 0x87878787 and rotr(word, 4) & 0x87878787
    w = 0x74736259
    assert w & 0x87878787 == 0x04030201
    assert (((w >> 4) | (w << 28)) & 0xFFFFFFFF) & 0x87878787 == 0x87070605
    rng = np.random.default_rng(3)
    q = rng.integers(-7, 8, size=(5, 128))
    assert np.array_equal(int4_words_to_q(q_to_int4_words(q)), q)
    # a negative zero is not a valid code
    with pytest.raises(AssertionError):
        int4_words_to_q(np.array([[0x80, 0, 0, 0]], dtype=np.uint8))


JACOBI_MAIN = r"""
#include <cstdio>
#include <vector>
namespace svdq { void jacobi_eigh(int, std::vector<double>&, std::vector<double>&, std::vector<double>&); }
int main() {
  int n; if (scanf("%d", &n) != 1) return 1;
  std::vector<double> A(n * n), V, w;
  for (auto& x : A) if (scanf("%lf", &x) != 1) return 1;
  svdq::jacobi_eigh(n, A, V, w);
  for (int i = 0; i < n; i++) printf("%.17g\n", w[i]);
  for (int i = 0; i < n * n; i++) printf("%.17g\n", V[i]);
  return 0;
}
"""


def test_host_jacobi_eigensolver(tmp_path):
    src = tmp_path / "main.cpp"
    src.write_text(JACOBI_MAIN)
    exe = tmp_path / "jac"
    lin = os.path.join(ROOT, "w4a4_quantized_gemm_amd", "csrc", "svdq_linalg.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", str(src), lin, "-o", str(exe), "-lquadmath"], check=True)
    rng = np.random.default_rng(0)
    for n, kind in ((1, "rand"), (7, "rand"), (48, "rand"), (96, "lowrank"), (64, "zero")):
        if kind == "zero":
            A = np.zeros((n, n))
        elif kind == "lowrank":
            B = rng.standard_normal((n, 5))
            A = B @ B.T
        else:
            B = rng.standard_normal((n, n))
            A = B + B.T
        inp = f"{n}\n" + "\n".join(repr(float(x)) for x in A.ravel())
        out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split()
        vals = np.array([float(x) for x in out])
        w, V = vals[:n], vals[n:].reshape(n, n)
        assert np.all(np.diff(w) <= 1e-12 * max(1.0, abs(w).max()))
        ref = np.sort(np.linalg.eigvalsh(A))[::-1]
        assert np.allclose(w, ref, atol=1e-10 * max(1.0, abs(ref).max()))
        assert np.allclose(V.T @ V, np.eye(n), atol=1e-10)
        assert np.allclose(A @ V, V * w, atol=1e-9 * max(1.0, abs(ref).max()))


CHOL_MAIN = r"""
#include <cstdio>
#include <vector>
namespace svdq { bool cholesky_upper_of_inverse(int n, std::vector<double> A, std::vector<double>& U); }
int main() {
  int n; if (scanf("%d", &n) != 1) return 1;
  std::vector<double> A(n * n), U;
  for (auto& x : A) if (scanf("%lf", &x) != 1) return 1;
  if (!svdq::cholesky_upper_of_inverse(n, A, U)) { printf("notpd\n"); return 0; }
  for (double u : U) printf("%.17g\n", u);
  return 0;
}
"""


def test_host_cholesky_of_inverse(tmp_path):
    """The host factorization GPTQ uses: U upper triangular with U^T U = A^-1
    (against numpy's inverse), and a rejection of a matrix that is not
    positive definite."""
    src = tmp_path / "main.cpp"
    src.write_text(CHOL_MAIN)
    exe = tmp_path / "chol"
    lin = os.path.join(ROOT, "w4a4_quantized_gemm_amd", "csrc", "svdq_linalg.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", str(src), lin, "-o", str(exe), "-lquadmath"], check=True)
    rng = np.random.default_rng(1)
    for n in (1, 5, 40):
        B = rng.standard_normal((n, n))
        A = B @ B.T + 0.5 * np.eye(n)
        inp = f"{n}\n" + "\n".join(repr(float(x)) for x in A.ravel())
        out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split()
        U = np.array([float(x) for x in out]).reshape(n, n)
        assert np.all(np.tril(U, -1) == 0.0)
        assert np.allclose(U.T @ U, np.linalg.inv(A), atol=1e-10 * np.abs(np.linalg.inv(A)).max())
    bad = "2\n1 2\n2 1"
    assert subprocess.run([str(exe)], input=bad, capture_output=True, text=True, check=True).stdout.strip() == "notpd"


LAMBDA_MAIN = r"""
#include <cstdio>
#include <vector>
namespace svdq { void smoothing_lambda(const float*, const float*, int, float, bool, float*, float*); }
int main() {
  int n; float alpha; int nosm;
  if (scanf("%d %f %d", &n, &alpha, &nosm) != 3) return 1;
  std::vector<float> a(n), w(n), l(n), i(n);
  for (int j = 0; j < n; j++) if (scanf("%a %a", &a[j], &w[j]) != 2) return 1;
  svdq::smoothing_lambda(a.data(), w.data(), n, alpha, nosm != 0, l.data(), i.data());
  for (int j = 0; j < n; j++) printf("%a %a\n", l[j], i[j]);
  return 0;
}
"""


def test_host_smoothing_factors_match_oracle(tmp_path):
    """The library computes lambda32 on the host (the real a^alpha /
    w^(1 - alpha) rounded once to fp32): bit-equal to the oracle's at several
    strengths, on random maxima over many binades, zero channels and the
    no-smoothing flag."""
    import oracle as O
    src = tmp_path / "main.cpp"
    src.write_text(LAMBDA_MAIN)
    exe = tmp_path / "lam"
    lin = os.path.join(ROOT, "w4a4_quantized_gemm_amd", "csrc", "svdq_linalg.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", str(src), lin, "-o", str(exe), "-lquadmath"], check=True)
    rng = np.random.default_rng(3)
    n = 3000
    a = (rng.random(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    w = (rng.random(n) * np.exp2(rng.integers(-40, 40, n))).astype(np.float32)
    a[:5] = 0.0
    w[5:10] = 0.0
    # sqrt(a / w) just past an fp32 rounding midpoint (a^0.5 / w^0.5 in fp64
    # rounds the wrong way here)
    a[10], w[10] = float.fromhex("0x1.19e7b4p+1"), float.fromhex("0x1.1ap+1")
    for alpha, nosm in ((0.5, 0), (0.25, 0), (0.75, 0), (0.3, 0), (0.5, 1)):
        inp = f"{n} {float(np.float32(alpha)).hex()} {nosm}\n" + "\n".join(
            f"{float(x).hex()} {float(y).hex()}" for x, y in zip(a, w))
        out = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, check=True).stdout.split()
        got = np.array([float.fromhex(x) for x in out]).reshape(n, 2)
        lam32, inv32 = O.smoothing_factors(a, w.astype(np.float64)[:, None], float(np.float32(alpha)), nosm == 1)
        assert np.array_equal(got[:, 0], lam32), (alpha, int(np.sum(got[:, 0] != lam32)))
        assert np.array_equal(got[:, 1], inv32)
