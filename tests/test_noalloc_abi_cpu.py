"""Host-side validation of svdq_linear_noalloc (no GPU needed: every case
is refused before the device is touched)."""
import ctypes

import w4a4_quantized_gemm_amd as S


def test_noalloc_validation_before_device():
    lib = S.load()
    d = S.make_desc(3072, 9216, 32, "int4")
    good = 1 << 20     # 16-byte aligned and non-null; never dereferenced when validation fails
    assert lib.svdq_linear_noalloc(ctypes.byref(d), None, good, 4608, good, 0, None) == 1
    assert lib.svdq_linear_noalloc(ctypes.byref(d), good, good, 0, good, 0, None) == 2
    assert lib.svdq_linear_noalloc(ctypes.byref(d), good + 4, good, 4608, good, 0, None) == 7
    # the scratch holds the fused layer's workspace up to its size
    M = 1
    while S.svdq_workspace_bytes(d, M * 2) <= S.NOALLOC_SCRATCH_BYTES:
        M *= 2
    big = M * 4
    assert S.svdq_workspace_bytes(d, big) > S.NOALLOC_SCRATCH_BYTES
    assert lib.svdq_linear_noalloc(ctypes.byref(d), good, good, big, good, 0, None) == 4
