"""The fusion ablation: the same layer with the 16-bit branch unfused
(svdq_linear_forward_unfused: the quantiser without the down-projection,
D = X L1s as its own bf16 GEMM, the 4-bit GEMM without the up-projection
into an fp32 result, then a second bf16 GEMM adding D L2 with the
epilogue) against the oracle, element by element, and against the fused
forward.  Bars as for the forward: Y within 2e-3 * max|Y_ref| (fp32 out),
(2e-3 + 2^-8) for bf16; with GELU, 1.13 x that plus a bf16 step."""
import numpy as np
import pytest
import torch

import synth
from oracle import glue as OG
from oracle import svdquant as O
from tests.conftest import announce
from tests.gpu_util import bf16_to_device, layer_from_oracle, rel_max_err, to_f64

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-3
TOL_BF16 = 2e-3 + 2.0 ** -8


@pytest.fixture(scope="module")
def S():
    import w4a4_rank_corrected_smooth_amd as lib
    lib.device_check()
    return lib


@pytest.mark.parametrize("M,N,K,rank,out,gelu", [
    (256, 512, 512, 16, torch.float32, False),
    (100, 200, 192, 5, torch.float32, False),
    (1, 64, 64, 1, torch.float32, False),
    (129, 257, 320, 40, torch.bfloat16, False),
    (300, 96, 128, 0, torch.float32, False),
    (130, 260, 256, 8, torch.bfloat16, True),
    (64, 256, 256, 256, torch.float32, False),       # maximum rank
    (100, 200, 1024, 8, torch.float32, False),       # the 4-bit GEMM K-splits
])
def test_unfused_branch_matches_oracle_and_fused(S, M, N, K, rank, out, gelu):
    c = synth.linear_case(f"unf{M}x{N}x{K}", 600 + M + rank, M, N, K, rank,
                          x_outlier_n=max(1, K // 64), x_outlier_scale=40.0,
                          w_outlier_n=max(1, K // 100), w_outlier_scale=8.0)
    announce(f"unfused branch M={M} N={N} K={K} r={rank} out={out} gelu={gelu}")
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, rank)
    layer = layer_from_oracle(ref)
    X = bf16_to_device(c.X)
    Yu = to_f64(S.linear_forward_unfused(layer, X, out_dtype=out, gelu=gelu))
    Yf = to_f64(S.linear_forward(layer, X, out_dtype=out, gelu=gelu))
    torch.cuda.synchronize()
    f = O.forward(ref, c.X)
    scale = np.max(np.abs(f["Y"]))
    if gelu:
        tol = 1.13 * TOL_F32 + 2.0 ** -8
        assert np.max(np.abs(Yu - OG.gelu_tanh_bf16(f["Y"]))) / scale <= tol
    else:
        tol = TOL_F32 if out == torch.float32 else TOL_BF16
        assert rel_max_err(Yu, f["Y"]) <= tol
    # fused and unfused differ only in the order of fp32 additions (and one
    # bf16 rounding of the output)
    assert np.max(np.abs(Yu - Yf)) / scale <= (1e-5 if out == torch.float32 and not gelu else 2.0 ** -7)


@pytest.mark.parametrize("which", ["qkv", "lowres"])
def test_unfused_branch_full_size_sampled_rows(S, which):
    c = synth.qkv_case() if which == "qkv" else synth.lowres_case()
    r = 32 if which == "qkv" else 128
    announce(f"unfused branch full size {which}: oracle prepare")
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, r)
    layer = layer_from_oracle(ref)
    X = bf16_to_device(c.X)
    Y = S.linear_forward_unfused(layer, X, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, c.M, max(1, c.M // 40)), [c.M - 1]]))
    f = O.forward(ref, c.X, rows=rows)
    err = rel_max_err(to_f64(Y)[rows], f["Y"])
    announce(f"  max rel err {err:.3e}")
    assert err <= TOL_F32
