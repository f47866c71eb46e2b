"""svdq_linear_noalloc (the entry point for callers that cannot allocate)
against svdq_linear, through the C ABI: two calls in a row on the library's
scratch array, the second with fewer rows, each bit-equal to svdq_linear
with a caller workspace and within the layer's tolerance of the oracle; a
size beyond the array is refused before any launch."""
import sys

import numpy as np
import pytest

import oracle as O
import workloads as WL
from svdq_testlib import np_bits_to_bf16_tensor, blob_sections, oracle_prep_from_blob

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("fmt", [O.INT4, O.FP4])
def test_noalloc_matches_linear(fmt):
    import torch
    import w4a4_quantized_gemm_amd as S
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    S.load()
    dev = "cuda:0"
    _say(f"case: noalloc fmt={fmt}")
    cfg = WL.C2.with_(name="noalloc", M=600, K=768, N=640, rank=32, fmt=fmt, w_std=1 / np.sqrt(768),
                      bias_std=0.02, seed=61)
    X_bits, W_bits, b_bits = WL.make_layer(cfg)
    X = np_bits_to_bf16_tensor(X_bits, dev)
    W = np_bits_to_bf16_tensor(W_bits, dev)
    a = torch.empty(cfg.K, dtype=torch.float32, device=dev)
    S.svdq_act_absmax(X, a)
    layer = S.SVDQLinear.prepare(W, a, cfg.rank, fmt, cfg.alpha, bias=np_bits_to_bf16_tensor(b_bits, dev))
    ref_prep = oracle_prep_from_blob(blob_sections(layer), W_bits, fmt, b_bits)
    for M, out in ((600, S.OUT_F32), (211, S.OUT_BF16)):
        Xm = X[:M].contiguous()
        dt = torch.float32 if out == S.OUT_F32 else torch.bfloat16
        Y0 = torch.empty((M, cfg.N), dtype=dt, device=dev)
        Y1 = torch.full((M, cfg.N), float("nan"), dtype=dt, device=dev)
        ws = torch.zeros(S.svdq_workspace_bytes(layer.desc, M), dtype=torch.uint8, device=dev)
        S.svdq_linear(layer.desc, layer.blob, Xm, Y0, ws, out)
        S.svdq_linear_noalloc(layer.desc, layer.blob, Xm, Y1, out)
        torch.cuda.synchronize()
        assert torch.equal(Y0, Y1), f"M={M}: noalloc output differs from svdq_linear"
        oname = "f32" if out == S.OUT_F32 else "bf16"
        e = O.rel_fro(Y1.float().cpu().numpy().astype(np.float64), O.linear(ref_prep, X_bits[:M], oname)["Y"])
        _say(f"  M={M} {oname}: bit-equal to svdq_linear, rel err vs oracle {e:.2e}")
        assert e <= 1e-3


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import torch
    import w4a4_quantized_gemm_amd as S
    S.load()
    _say("case: noalloc size limit")
    desc = S.make_desc(12288, 64, 16, "fp4")
    M = 16384                                   # codes alone: 96 MiB
    assert S.svdq_workspace_bytes(desc, M) > S.NOALLOC_SCRATCH_BYTES
    blob = torch.zeros(S.svdq_prepared_bytes(desc), dtype=torch.uint8, device="cuda:0")
    X = torch.zeros((M, 12288), dtype=torch.bfloat16, device="cuda:0")
    Y = torch.zeros((M, 64), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(S.SvdqError) as ei:
        S.svdq_linear_noalloc(desc, blob, X, Y, S.OUT_BF16)
    assert ei.value.status == 4
    torch.cuda.synchronize()
    assert int(Y.abs().sum().item()) == 0       # nothing was launched
