"""GPU parity of layers carrying a user LoRA on their low-rank branch
(svdq_merge_lora / svdq_mx_merge_lora, then the ordinary forward) against
the oracle's merged layer (``oracle/lora.py``), through the C ABI: the
activation codes and scales bit-exact (the 4-bit path is the base layer's),
the merged down-projection within 1e-5, Y within 2e-3 * max|Y_ref|; ranks
that are not multiples of the tile, the largest rank, and the Flux MLP fc1
shape with a rank-32 LoRA on sampled rows."""
import numpy as np
import pytest
import torch

import synth
from oracle import lora as LO
from oracle import mxfp4 as MX
from oracle import svdquant as O
from tests.conftest import announce
from tests.gpu_util import bf16_to_device, host_from_oracle, mx_host_from_oracle, rel_max_err, to_f64

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-3
TOL_BF16 = 2e-3 + 2.0 ** -8


@pytest.fixture(scope="module")
def S():
    import w4a4_rank_corrected_smooth_amd as lib
    lib.device_check()
    return lib


def merged_int4(S, c, rank, A, B, alpha):
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, rank)
    hw = S.merge_lora(host_from_oracle(ref), A, B, alpha)
    return LO.merge(ref, A, B, alpha), S.Linear(hw)


def merged_mx(S, c, rank, A, B, alpha):
    ref = MX.prepare(c.W, c.calib_absmax(), c.bias, rank)
    hw = S.mx_merge_lora(mx_host_from_oracle(ref), A, B, alpha)
    return LO.merge(ref, A, B, alpha), S.MxLinear(hw)


@pytest.mark.parametrize("form", ["int4", "mx"])
@pytest.mark.parametrize("M,N,K,rank,r2,alpha", [(100, 200, 192, 5, 7, 0.75), (256, 512, 512, 16, 16, 1.0),
                                                 (33, 130, 320, 0, 3, -2.0), (300, 96, 128, 40, 9, 0.3),
                                                 (64, 512, 512, 32, 224, 0.5)])
def test_lora_small_shapes(S, form, M, N, K, rank, r2, alpha):
    c = synth.linear_case(f"lora{M}x{N}x{K}", 600 + M, M, N, K, rank,
                          x_outlier_n=max(1, K // 64), x_outlier_scale=40.0)
    A, B = synth.lora_factors(700 + M, N, K, r2, b_std=0.05)
    announce(f"lora {form} M={M} N={N} K={K} r={rank}+{r2} alpha={alpha}")
    if form == "int4":
        ref, layer = merged_int4(S, c, rank, A, B, alpha)
        fwd, quant, run = O.forward, S.quantize_activations, S.linear_forward
    else:
        ref, layer = merged_mx(S, c, rank, A, B, alpha)
        fwd, quant, run = MX.forward, S.mx_quantize_activations, S.mx_linear_forward
    X = bf16_to_device(c.X)
    ws = layer.new_workspace(M)
    Y = run(layer, X, out_dtype=torch.float32, workspace=ws)
    q, s, d = quant(layer, X, ws)
    torch.cuda.synchronize()
    f = fwd(ref, c.X)
    if form == "int4":
        assert np.array_equal(q.cpu().numpy(), O.pack_int4(f["qA"])), "activation codes"
        assert np.array_equal(s.cpu().numpy(), f["sA"]), "activation scales"
    else:
        assert np.array_equal(q.cpu().numpy(), MX.pack_fp4(f["qA"])), "activation codes"
        assert np.array_equal(s.cpu().numpy().astype(np.int32) - 127, f["eA"]), "activation scales"
    assert rel_max_err(to_f64(d), f["D"]) <= 1e-5, "merged low-rank down-projection"
    err = rel_max_err(to_f64(Y), f["Y"])
    announce(f"lora {form} max rel err {err:.3e}")
    assert err <= TOL_F32


def test_lora_changes_only_the_branch(S):
    """Adding a LoRA and its negative gives back the base layer's output to
    within the branch's own rounding (the bf16 split of D)."""
    c = synth.linear_case("lora_cancel", 650, 130, 256, 256, 16, x_outlier_n=4, x_outlier_scale=40.0)
    A, B = synth.lora_factors(651, c.N, c.K, 8)
    announce("lora cancel M=130 N=256 K=256 r=16+8+8")
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, 16)
    hw0 = host_from_oracle(ref)
    hw2 = S.merge_lora(S.merge_lora(hw0, A, B, 1.5), A, B, -1.5)
    X = bf16_to_device(c.X)
    Y0 = to_f64(S.linear_forward(S.Linear(hw0), X, out_dtype=torch.float32))
    Y2 = to_f64(S.linear_forward(S.Linear(hw2), X, out_dtype=torch.float32))
    assert rel_max_err(Y2, Y0) <= 1e-5


def test_lora_fc1_shape_sampled_rows(S):
    """The Flux MLP fc1 shape (4608 x 3072 -> 12288, r = 32) with a rank-32
    LoRA, bf16 output with the fused GELU as the MLP runs it, on sampled
    rows; codes and scales bit-exact over all rows."""
    from oracle import glue as OG
    fc1, _, _ = synth.mlp_cases()
    A, B = synth.lora_factors(660, fc1.N, fc1.K, 32)
    announce("lora fc1: oracle prepare 12288x3072 r32 + LoRA 32")
    ref, layer = merged_int4(S, fc1, 32, A, B, 1.0)
    X = bf16_to_device(fc1.X)
    ws = layer.new_workspace(fc1.M)
    announce("lora fc1: device forward M=4608 r=64 gelu bf16")
    Y = S.linear_forward(layer, X, out_dtype=torch.bfloat16, gelu=True, workspace=ws)
    q, s, d = S.quantize_activations(layer, X, ws)
    torch.cuda.synchronize()
    qA, sA = O.quantize_activations(O.bf16_values(fc1.X), ref["iota"])
    assert np.array_equal(q.cpu().numpy(), O.pack_int4(qA)) and np.array_equal(s.cpu().numpy(), sA)
    rng = np.random.default_rng(661)
    rows = np.unique(np.concatenate([[0, fc1.M - 1], rng.choice(fc1.M, 40, replace=False)]))
    f = O.forward(ref, fc1.X, rows=rows)
    assert rel_max_err(to_f64(d)[rows], f["D"]) <= 1e-5
    G = to_f64(Y)[rows]
    err = np.max(np.abs(G - OG.gelu_tanh_bf16(f["Y"]))) / np.max(np.abs(f["Y"]))
    announce(f"lora fc1 max err / max|Y| {err:.3e}")
    assert err <= 1.13 * TOL_F32 + 2.0 ** -8
