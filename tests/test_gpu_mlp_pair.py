"""The fused MLP pair: fc1's GEMM applies bias + GELU, rounds to bf16 and
quantises fc2's input in its epilogue (codes, scales and the low-rank
down-projection as a fixed-point sum), so the intermediate never goes to
memory.  The quantiser runs on exactly the bf16 values the unfused path
stores, so fc2's codes and scales must match the unfused quantiser's
bit for bit; fc2's output is checked against the oracle run on those same
bf16 values (the reading used for the unfused pair), and the fixed-point D
against the oracle's D.  Bars as in test_gpu_parity."""
import math

import numpy as np
import pytest
import torch

import synth
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


def _pair(S, name, seed, M, K1, N1, N2, r1, r2, gelu=True):
    announce(f"mlp pair {name}: M={M} {K1}->{N1}->{N2} r={r1},{r2} gelu={gelu}")
    c1 = synth.linear_case(name + "-1", seed, M, N1, K1, r1, x_outlier_n=max(1, K1 // 64),
                           x_outlier_scale=40.0)
    c2 = synth.linear_case(name + "-2", seed + 1, M, N2, N1, r2)   # W2, b2 only
    ref1 = O.prepare(c1.W, c1.calib_absmax(), c1.bias, r1)
    l1 = layer_from_oracle(ref1)
    X = bf16_to_device(c1.X)
    Y1 = S.linear_forward(l1, X, out_dtype=torch.bfloat16, gelu=gelu)
    torch.cuda.synchronize()
    X2 = Y1.cpu().view(torch.int16).numpy().view(np.uint16)
    ax2 = O.calibration_absmax(O.bf16_values(X2[:64]))
    ref2 = O.prepare(c2.W, ax2, c2.bias, r2)
    l2 = layer_from_oracle(ref2)
    return l1, l2, X, Y1, X2, ref2


def _regions(M, K, rank):
    """Byte offsets of the workspace's codes, scales and D (the device layout)."""
    Mp = -(-M // 256) * 256
    G = K // 64
    up = lambda x: -(-x // 256) * 256
    qa_bytes = Mp * K * 3 // 4
    sa_off = up(qa_bytes)
    d_off = up(sa_off + G * Mp * 16)              # scales as 16-byte operands
    return Mp, G, sa_off, d_off


CASES = [("ragged", 130, 256, 320, 200, 8, 5), ("tiles", 256, 512, 576, 384, 16, 32),
         ("one-row", 1, 64, 64, 64, 1, 1), ("rank0-next", 300, 192, 384, 96, 12, 0),
         ("wide-rank", 200, 128, 256, 130, 40, 70),
         ("split-fc2", 200, 256, 1024, 256, 8, 8),        # fc2's GEMM is K-split (2 tiles, 16 groups)
         ("narrow-fc2", 1024, 256, 512, 2048, 16, 32),   # fc2's GEMM runs narrow tiles on fixed-point D
         ("narrow-fc2-3-groups", 1024, 256, 192, 2048, 16, 8)]   # ... with fewer groups than its stages


@pytest.mark.parametrize("name,M,K1,N1,N2,r1,r2", CASES)
def test_fused_pair_codes_scales_and_D(S, name, M, K1, N1, N2, r1, r2):
    l1, l2, X, Y1, X2, ref2 = _pair(S, name, 400 + M, M, K1, N1, N2, r1, r2)
    ws1, ws2 = l1.new_workspace(M), l2.new_workspace(M)
    S.mlp_quantize(l1, l2, X, ws1, ws2)
    S.mlp_gemm1(l1, l2, M, ws1, ws2, gelu=True)
    ws2u = l2.new_workspace(M)
    S.linear_quantize(l2, Y1, ws2u)
    torch.cuda.synchronize()
    a, b = ws2.cpu().numpy(), ws2u.cpu().numpy()
    Mp, G, sa_off, d_off = _regions(M, N1, r2)
    T, tM = Mp // 32, math.ceil(M / 32)
    for g in range(G):
        lo, hi = g * T * 1536, (g * T + tM) * 1536
        assert np.array_equal(a[lo:hi], b[lo:hi]), f"codes of group {g}"
    sa = a[sa_off: sa_off + G * Mp * 16].reshape(G, Mp, 16)[:, :M]
    sb = b[sa_off: sa_off + G * Mp * 16].reshape(G, Mp, 16)[:, :M]
    assert np.array_equal(sa, sb), "scales"
    if r2 > 0:
        rp = -(-r2 // 32) * 32
        d = a[d_off: d_off + Mp * rp * 8].view(np.int64).reshape(Mp, rp)[:M, :r2] / 2.0 ** 32
        Dref = O.forward(ref2, X2)["D"]
        assert rel_max_err(d, Dref) <= 1e-5, "fixed-point down-projection"


@pytest.mark.parametrize("name,M,K1,N1,N2,r1,r2", CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fused_pair_output(S, name, M, K1, N1, N2, r1, r2, out_dtype):
    l1, l2, X, Y1, X2, ref2 = _pair(S, name, 400 + M, M, K1, N1, N2, r1, r2)
    Y = to_f64(S.mlp_forward(l1, l2, X, out_dtype=out_dtype))
    Yref = O.forward(ref2, X2)["Y"]
    assert rel_max_err(Y, Yref) <= (TOL_F32 if out_dtype == torch.float32 else TOL_BF16)


def test_fused_pair_without_gelu_is_deterministic(S):
    l1, l2, X, Y1, X2, ref2 = _pair(S, "nogelu", 77, 200, 256, 320, 192, 8, 16, gelu=False)
    ws1, ws2 = l1.new_workspace(200), l2.new_workspace(200)
    Ya = S.mlp_forward(l1, l2, X, out_dtype=torch.float32, gelu=False, ws1=ws1, ws2=ws2).clone()
    Yb = S.mlp_forward(l1, l2, X, out_dtype=torch.float32, gelu=False, ws1=ws1, ws2=ws2)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yb), "two runs differ"
    Yref = O.forward(ref2, X2)["Y"]
    assert rel_max_err(to_f64(Ya), Yref) <= TOL_F32
    # the stage calls are exactly the one-call pair
    S.mlp_quantize(l1, l2, X, ws1, ws2)
    S.mlp_gemm1(l1, l2, 200, ws1, ws2, gelu=False)
    Yc = S.mlp_gemm2(l2, 200, torch.empty_like(Ya), ws2)
    torch.cuda.synchronize()
    assert torch.equal(Ya, Yc)
