"""The allocation-free forward (svdq_linear_forward_static): the same two
kernels as svdq_linear_forward with the library's file-scope device scratch
array as workspace.  Checked through the C ABI against the workspace-taking
forward (bit for bit: same kernels, same inputs, same K-split choice) and
against the oracle (Y within 2e-3 * max|Y_ref|), on two calls in a row, the
second with fewer rows, so the second call runs on an array the first call
left full."""
import numpy as np
import pytest
import torch

import synth
from oracle import svdquant as O
from tests.conftest import announce
from tests.gpu_util import bf16_to_device, layer_from_oracle, rel_max_err, to_f64

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-3


@pytest.fixture(scope="module")
def S():
    import w4a4_rank_corrected_smooth_amd as lib
    lib.device_check()
    return lib


@pytest.mark.parametrize("M1,M2,N,K,rank,gelu", [(300, 77, 320, 512, 16, False),
                                               (1024, 1, 3072, 3072, 32, True),
                                               (513, 200, 1536, 1024, 0, False)])
def test_static_forward_matches_forward_twice(S, M1, M2, N, K, rank, gelu):
    c = synth.linear_case(f"static{M1}x{N}x{K}", 900 + M1, M1, N, K, rank,
                          x_outlier_n=max(1, K // 64), x_outlier_scale=40.0)
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, rank)
    layer = layer_from_oracle(ref)
    for M in (M1, M2):
        announce(f"static forward M={M} N={N} K={K} r={rank} gelu={gelu}")
        X = bf16_to_device(c.X[:M])
        # a workspace capped at the static array's size makes the same K-split
        # choice (the split runs only when its partials fit)
        ws = torch.empty(min(layer.workspace_bytes(M), S.STATIC_SCRATCH_BYTES), dtype=torch.uint8,
                         device="cuda")
        for dt in (torch.float32, torch.bfloat16):
            Ys = torch.empty((M, N), dtype=dt, device="cuda")
            S.linear_forward_static(layer, X, Ys, gelu=gelu)
            Yw = S.linear_forward(layer, X, out_dtype=dt, gelu=gelu, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(Ys, Yw), f"static and workspace forwards differ (M={M}, {dt})"
        if not gelu:
            f = O.forward(ref, c.X[:M])
            assert rel_max_err(to_f64(Ys.float()), f["Y"]) <= TOL_F32 + 2.0 ** -8


def test_static_forward_refuses_oversized_shapes(S):
    c = synth.linear_case("static-big", 991, 8, 256, 16384, 8)
    ref = O.prepare(c.W, None, c.bias, 8)
    layer = layer_from_oracle(ref)
    X = torch.zeros((6144, 16384), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((6144, 256), dtype=torch.bfloat16, device="cuda")
    announce("static forward refusal M=6144 K=16384 (validation only)")
    with pytest.raises(S.SvdqError) as e:
        S.linear_forward_static(layer, X, Y)
    assert e.value.status == 5
