"""Pins of the LoRA merge oracle (``oracle/lora.py``) against what fixes it
without a second implementation of the merge: a rank-1 LoRA that copies one
input channel into one output channel (values readable by eye), torch's own
two-projection LoRA forward in float64, bf16 rounding by torch's cast, the
exact cancellation of a LoRA by its negative, a LoRA equal to the base
branch doubling that branch, r' = 0 as the identity, and the 4-bit path of
the base layer left bit for bit as it was (INT4 and MXFP4 forms)."""
import numpy as np
import pytest
import torch

import synth
from oracle import lora as L
from oracle import mxfp4 as MX
from oracle import svdquant as O


def base_case(form="int4", M=24, N=96, K=192, rank=8, seed=31):
    c = synth.linear_case(f"lora_{form}", seed, M, N, K, rank, x_outlier_n=3, x_outlier_scale=30.0)
    prep = (O.prepare if form == "int4" else MX.prepare)(c.W, c.calib_absmax(), c.bias, rank)
    fwd = O.forward if form == "int4" else MX.forward
    return c, prep, fwd


def unit_bits(shape, index):
    a = np.zeros(shape, np.float32)
    a[index] = 1.0
    return synth.f32_to_bf16_bits(a)


@pytest.mark.parametrize("form", ["int4", "mx"])
def test_rank1_lora_copies_one_channel(form):
    c, prep, fwd = base_case(form)
    j, n = 17, 40
    A = unit_bits((1, c.K), (0, j))
    B = unit_bits((c.N, 1), (n, 0))
    for alpha in (1.0, 2.5):
        merged = L.merge(prep, A, B, alpha)
        y0, y1 = fwd(prep, c.X)["Y"], fwd(merged, c.X)["Y"]
        want = np.zeros_like(y0)
        want[:, n] = alpha * O.bf16_values(c.X)[:, j]
        assert np.allclose(y1 - y0, want, rtol=0, atol=1e-12 * np.abs(y0).max())
        assert merged["rank"] == prep["rank"] + 1


@pytest.mark.parametrize("form", ["int4", "mx"])
def test_matches_torch_lora_forward(form):
    """alpha a power of two keeps alpha B exact in bf16, so the merged layer's
    change of Y is exactly torch's LoRA forward alpha * B(A(x))."""
    c, prep, fwd = base_case(form)
    A, B = synth.lora_factors(5, c.N, c.K, 6)
    alpha = 0.5
    merged = L.merge(prep, A, B, alpha)
    d = fwd(merged, c.X)["Y"] - fwd(prep, c.X)["Y"]
    x = torch.from_numpy(O.bf16_values(c.X))
    ta = torch.from_numpy(O.bf16_values(A))
    tb = torch.from_numpy(O.bf16_values(B))
    want = alpha * torch.nn.functional.linear(torch.nn.functional.linear(x, ta), tb)
    assert np.allclose(d, want.numpy(), rtol=0, atol=1e-12 * np.abs(want.numpy()).max())


def test_scaled_up_factor_is_torchs_fp32_product_cast_to_bf16():
    _, B = synth.lora_factors(6, 64, 128, 5, b_std=3.0)
    for alpha in (0.3, -1.7, 1e-3, 7.0):
        got = L.scaled_up_factor(B, alpha)
        tb = torch.from_numpy(synth.bf16_bits_to_f32(B))
        want = (tb * torch.tensor(alpha, dtype=torch.float32)).to(torch.bfloat16).double().numpy().T
        assert np.array_equal(got, want)


@pytest.mark.parametrize("form", ["int4", "mx"])
def test_negative_lora_cancels(form):
    c, prep, fwd = base_case(form)
    A, B = synth.lora_factors(7, c.N, c.K, 4)
    both = L.merge(L.merge(prep, A, B, 0.7), A, B, -0.7)
    y0, y2 = fwd(prep, c.X)["Y"], fwd(both, c.X)["Y"]
    assert both["rank"] == prep["rank"] + 8
    assert np.allclose(y2, y0, rtol=0, atol=1e-12 * np.abs(y0).max())


def test_lora_equal_to_the_branch_doubles_it():
    """The branch is itself a LoRA on the raw activations (down L1s^T, up
    L2^T); adding it once more adds D L2 once more."""
    c, prep, fwd = base_case("int4")
    A = O.bf16_bits_of(prep["L1s"].T)
    B = O.bf16_bits_of(prep["L2b"].T)
    merged = L.merge(prep, A, B, 1.0)
    f0 = fwd(prep, c.X)
    d = fwd(merged, c.X)["Y"] - f0["Y"]
    branch = f0["D"] @ prep["L2b"]
    assert np.allclose(d, branch, rtol=0, atol=1e-12 * np.abs(f0["Y"]).max())


@pytest.mark.parametrize("form", ["int4", "mx"])
def test_rank0_is_identity_and_4bit_path_untouched(form):
    c, prep, fwd = base_case(form)
    same = L.merge(prep, np.zeros((0, c.K), np.uint16), np.zeros((c.N, 0), np.uint16), 3.0)
    assert np.array_equal(same["L1s"], prep["L1s"]) and np.array_equal(same["L2b"], prep["L2b"])
    A, B = synth.lora_factors(8, c.N, c.K, 3)
    merged = L.merge(prep, A, B, 1.0)
    keys = ("qW", "sW") if form == "int4" else ("qW", "eW")
    for k in keys + ("iota", "bias"):
        assert np.array_equal(merged[k], prep[k])
    f0, f1 = fwd(prep, c.X), fwd(merged, c.X)
    for k in ("qA", "sA") if form == "int4" else ("qA", "eA"):
        assert np.array_equal(f0[k], f1[k])
    # the input layer is left as it was
    assert prep["L1s"].shape[1] == prep["rank"] == c.rank
