"""GPU parity of the FP4 (MXFP4) form of the W4A4 path against the oracle
(``oracle/mxfp4.py``), through the C ABI.  Activation codes and E8M0 scales
bit-exact; Y within 2e-3 * max|Y_ref| (fp32 output) or (2e-3 + 2^-8)
(bf16); the low-rank down-projection within 1e-5; an exact result where
every partial sum is exactly representable; the full MLP shapes on sampled
rows."""
import numpy as np
import pytest
import torch

import synth
from oracle import mxfp4 as MX
from oracle import svdquant as O
from oracle import glue as OG
from tests.conftest import announce
from tests.gpu_util import bf16_to_device, mx_layer_from_oracle, rel_max_err, to_f64

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-3
TOL_BF16 = 2e-3 + 2.0 ** -8


@pytest.fixture(scope="module")
def S():
    import w4a4_rank_corrected_smooth_amd as lib
    lib.device_check()
    return lib


def run(S, c, rank, smooth=True, out_dtype=torch.float32, gelu=False):
    ax = c.calib_absmax() if smooth else None
    announce(f"mx {c.name} M={c.M} N={c.N} K={c.K} r={rank} smooth={smooth} out={out_dtype} gelu={gelu}")
    ref = MX.prepare(c.W, ax, c.bias, rank)
    layer = mx_layer_from_oracle(ref)
    X = bf16_to_device(c.X)
    ws = layer.new_workspace(c.M)
    Y = S.mx_linear_forward(layer, X, out_dtype=out_dtype, gelu=gelu, workspace=ws)
    q, e, d = S.mx_quantize_activations(layer, X, ws)
    torch.cuda.synchronize()
    f = MX.forward(ref, c.X)
    return ref, f, layer, X, ws, to_f64(Y), q.cpu().numpy(), e.cpu().numpy(), to_f64(d)


@pytest.mark.parametrize("M,N,K,rank", [(256, 512, 512, 16), (100, 200, 192, 5), (1, 64, 64, 1),
                                        (33, 130, 320, 7), (300, 96, 128, 40), (129, 257, 256, 0)])
def test_mx_small_shapes(S, M, N, K, rank):
    c = synth.linear_case(f"mx{M}x{N}x{K}", 400 + M, M, N, K, rank,
                          x_outlier_n=max(1, K // 64), x_outlier_scale=40.0,
                          w_outlier_n=max(1, K // 100), w_outlier_scale=8.0)
    ref, f, layer, X, ws, Y, q, e, d = run(S, c, rank)
    assert np.array_equal(q, MX.pack_fp4(f["qA"])), "activation codes"
    assert np.array_equal(e.astype(np.int32) - 127, f["eA"]), "activation scales"
    if rank > 0:
        assert rel_max_err(d, f["D"]) <= 1e-5, "low-rank down-projection"
    err = rel_max_err(Y, f["Y"])
    announce(f"mx {c.name} max rel err {err:.3e}")
    assert err <= TOL_F32


def test_mx_tiny_both_output_types_and_gelu(S):
    c = synth.tiny_case()
    ref, f, layer, X, ws, Y, q, e, d = run(S, c, 16, out_dtype=torch.bfloat16)
    assert rel_max_err(Y, f["Y"]) <= TOL_BF16
    G = to_f64(S.mx_linear_forward(layer, X, out_dtype=torch.bfloat16, gelu=True, workspace=ws))
    assert np.max(np.abs(G - OG.gelu_tanh_bf16(f["Y"]))) / np.max(np.abs(f["Y"])) <= 1.13 * TOL_F32 + 2.0 ** -8


def grid_rows(rng, rows, K):
    """Rows of E2M1 values (scale 1) whose blocks each hold a 4 or a 6."""
    codes = rng.integers(0, 16, size=(rows, K)).astype(np.uint8)
    codes[codes == 8] = 0
    for r in range(rows):
        for b in range(K // 32):
            codes[r, 32 * b + rng.integers(0, 32)] = rng.choice([6, 7, 14, 15])
    return MX.e2m1_value(codes)


def test_mx_exact_on_grid(S):
    """r = 0, no smoothing, X and W on the MXFP4 grid with unit scales: every
    block sum and every running sum is an exact multiple of 1/4 far below
    2^24, so the fp32 result equals X W^T + b exactly."""
    rng = np.random.default_rng(9)
    M, N, K = 96, 160, 512
    X, W = grid_rows(rng, M, K), grid_rows(rng, N, K)
    b = rng.integers(-16, 16, size=N) / 4.0
    ref = MX.prepare(O.bf16_bits_of(W), None, O.bf16_bits_of(b), 0)
    layer = mx_layer_from_oracle(ref)
    Y = to_f64(S.mx_linear_forward(layer, bf16_to_device(O.bf16_bits_of(X)), out_dtype=torch.float32))
    assert np.array_equal(Y, X @ W.T + b[None, :])


def test_mx_split_calls_and_determinism(S):
    c = synth.linear_case("mxsplit", 410, 200, 384, 256, 8, x_outlier_n=3, x_outlier_scale=30.0)
    ref = MX.prepare(c.W, c.calib_absmax(), c.bias, 8)
    layer = mx_layer_from_oracle(ref)
    X = bf16_to_device(c.X)
    ws = layer.new_workspace(c.M)
    Y1 = S.mx_linear_forward(layer, X, out_dtype=torch.float32, workspace=ws)
    S.mx_linear_quantize(layer, X, ws)
    Y2 = torch.empty_like(Y1)
    S.mx_linear_gemm(layer, c.M, Y2, ws)
    Y3 = S.mx_linear_forward(layer, X, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(Y1, Y3)


def test_mx_mlp_shapes_sampled_rows(S):
    """The Flux MLP pair's shapes (fc1 4608 x 3072 -> 12288 with GELU, fc2
    12288 -> 3072 on the device's own intermediate), sampled rows against the
    oracle."""
    fc1, W2, b2 = synth.mlp_cases()
    announce("mx mlp: oracle prepare fc1")
    ref1 = MX.prepare(fc1.W, fc1.calib_absmax(), fc1.bias, 32)
    l1 = mx_layer_from_oracle(ref1)
    X = bf16_to_device(fc1.X)
    Y1 = S.mx_linear_forward(l1, X, out_dtype=torch.bfloat16, gelu=True)
    Y1f = to_f64(S.mx_linear_forward(l1, X, out_dtype=torch.float32))
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, fc1.M - 1], rng.choice(fc1.M, 30, replace=False)]))
    f1 = MX.forward(ref1, fc1.X, rows=rows)
    assert rel_max_err(Y1f[rows], f1["Y"]) <= TOL_F32
    X2 = Y1.cpu().view(torch.int16).numpy().view(np.uint16)
    announce("mx mlp: oracle prepare fc2")
    ref2 = MX.prepare(W2, O.calibration_absmax(O.bf16_values(X2[:64])), b2, 32)
    l2 = mx_layer_from_oracle(ref2)
    Y2 = to_f64(S.mx_linear_forward(l2, Y1, out_dtype=torch.bfloat16))
    f2 = MX.forward(ref2, X2, rows=rows)
    err = rel_max_err(Y2[rows], f2["Y"])
    announce(f"mx fc2 bf16 max rel err {err:.3e}")
    assert err <= TOL_BF16
