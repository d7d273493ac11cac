"""GPU parity at sizes the oracle finishes in seconds (several tiles and a
ragged tail), plus the edge cases of the method.  Everything goes through the
C ABI; expected values come only from the oracle on the same seeded inputs.

Bars: INT4 codes, fp32 scales and int32 group sums bit-exact; Y within
2e-3 * max|Y_ref| (fp32 output) and (2e-3 + 2^-8) * max|Y_ref| (bf16 output,
whose own rounding is up to 2^-8 relative); the low-rank down-projection D
within 1e-5 * max|D_ref|."""
import numpy as np
import pytest
import torch

import synth
from oracle import svdquant as O
from oracle import glue as OG
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


def run_case(S, c, smooth=True, rank=None, out_dtype=torch.float32, gelu=False, check_codes=True):
    rank = c.rank if rank is None else rank
    ax = c.calib_absmax() if smooth else None
    announce(f"{c.name} M={c.M} N={c.N} K={c.K} r={rank} smooth={smooth} out={out_dtype} gelu={gelu}")
    ref = O.prepare(c.W, ax, c.bias, rank)
    layer = layer_from_oracle(ref)
    X = bf16_to_device(c.X)
    ws = layer.new_workspace(c.M)
    Y = S.linear_forward(layer, X, out_dtype=out_dtype, gelu=gelu, workspace=ws)
    f = O.forward(ref, c.X)
    if check_codes:
        q, s, d = S.quantize_activations(layer, X, ws)
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), O.pack_int4(f["qA"])), "activation codes"
        assert np.array_equal(s.cpu().numpy(), f["sA"]), "activation scales"
        if rank > 0:
            assert rel_max_err(to_f64(d), f["D"]) <= 1e-5, "low-rank down-projection"
    torch.cuda.synchronize()
    return ref, f, layer, X, ws, to_f64(Y)


@pytest.mark.parametrize("M,N,K,rank", [(256, 512, 512, 16), (100, 200, 192, 5), (1, 64, 64, 1),
                                        (33, 130, 320, 7), (300, 96, 128, 40), (129, 257, 256, 32)])
def test_forward_small_shapes(S, M, N, K, rank):
    c = synth.linear_case(f"small{M}x{N}x{K}", 200 + M, M, N, K, rank,
                          x_outlier_n=max(1, K // 64), x_outlier_scale=40.0,
                          w_outlier_n=max(1, K // 100), w_outlier_scale=8.0)
    ref, f, layer, X, ws, Y = run_case(S, c)
    assert rel_max_err(Y, f["Y"]) <= TOL_F32


def test_tiny_config_both_output_types(S):
    c = synth.tiny_case()
    ref, f, layer, X, ws, Y = run_case(S, c)
    assert rel_max_err(Y, f["Y"]) <= TOL_F32
    Yb = to_f64(S.linear_forward(layer, X, out_dtype=torch.bfloat16, workspace=ws))
    assert rel_max_err(Yb, f["Y"]) <= TOL_BF16


def test_group_sums_bit_exact(S):
    c = synth.linear_case("sums", 301, 300, 400, 256, 8, x_outlier_n=4, x_outlier_scale=40.0)
    ref, f, layer, X, ws, Y = run_case(S, c)
    for (m0, mc, n0, nc) in [(0, 64, 0, 64), (250, 50, 350, 50), (77, 130, 13, 200), (299, 1, 399, 1)]:
        announce(f"group sums window m0={m0} mc={mc} n0={n0} nc={nc}")
        P = S.debug_group_sums(layer, c.M, m0, mc, n0, nc, ws).cpu().numpy()
        Pref = O.group_sums(f["qA"][m0:m0 + mc], ref["qW"][n0:n0 + nc])
        assert np.array_equal(P, Pref)


def _layer_with_codes(S, qW, rank=8, seed=0):
    """A layer whose residual weight codes are exactly qW [N, K] (the other
    arrays are arbitrary: the group sums do not read them)."""
    from oracle.svdquant import pack_int4
    N, K = qW.shape
    rng = np.random.default_rng(seed)
    bf = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    hw = S.PreparedHost(N, K, rank, np.ones(K, np.float32), bf(rng.standard_normal((K, rank)) * 0.02),
                        bf(rng.standard_normal((rank, N)) * 0.02), pack_int4(qW),
                        np.full((N, K // 64), 0.01, np.float32), np.zeros(N, np.float32))
    return S.Linear(hw, "cuda")


@pytest.mark.parametrize("pattern", ["uniform", "extremes", "minus8"])
def test_group_sums_of_given_codes(S, pattern):
    """Caller-supplied canonical activation codes through the GEMM's own
    sums path (svdq_debug_group_sums_codes), against the oracle's integer
    group sums: codes uniform in -7..7; codes of magnitude 7 only, with weight
    rows that repeat activation rows' signs, so P reaches +-3136 = 64 * 49,
    the largest group sum; and canonical nibbles 0x8 (-8, outside the code
    set), which enter as 0."""
    M, N, K = 300, 330, 320
    rng = np.random.default_rng({"uniform": 7, "extremes": 8, "minus8": 9}[pattern])
    if pattern == "extremes":
        qA = np.where(rng.random((M, K)) < 0.5, -7, 7).astype(np.int8)
        qW = np.where(rng.random((N, K)) < 0.5, -7, 7).astype(np.int8)
        qW[:40] = qA[:40]            # P = +3136 on the diagonal of the first 40 rows
        qW[40:80] = -qA[40:80]       # and -3136 on the next 40
    else:
        qA = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
        qW = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    packed = O.pack_int4(qA)
    qA_eff = qA
    if pattern == "minus8":
        hole = rng.random((M, K // 2)) < 0.1          # some low nibbles become 0x8
        packed = np.where(hole, (packed & 0xF0) | 0x08, packed).astype(np.uint8)
        qA_eff = qA.copy()
        qA_eff[:, 0::2][hole] = 0
    layer = _layer_with_codes(S, qW)
    qact = torch.from_numpy(packed).to("cuda")
    ws = layer.new_workspace(M)
    for (m0, mc, n0, nc) in [(0, 256, 0, 256), (44, 256, 74, 256), (299, 1, 329, 1), (0, 80, 0, 80)]:
        announce(f"given codes {pattern}: window m0={m0} mc={mc} n0={n0} nc={nc}")
        P = S.debug_group_sums_codes(layer, qact, m0, mc, n0, nc, workspace=ws).cpu().numpy()
        Pref = O.group_sums(qA_eff[m0:m0 + mc], qW[n0:n0 + nc])
        assert np.array_equal(P, Pref)
        if pattern == "extremes" and m0 == 0 and mc == 80:
            d = np.arange(40)
            assert np.all(P[d, d] == 3136) and np.all(P[40 + d, 40 + d] == -3136)


def test_rank0_without_smoothing(S):
    c = synth.linear_case("r0", 302, 160, 192, 256, 0, x_outlier_n=3, x_outlier_scale=30.0)
    ref, f, layer, X, ws, Y = run_case(S, c, smooth=False)
    assert np.all(ref["iota"] == 1.0)
    assert rel_max_err(Y, f["Y"]) <= TOL_F32


def test_max_rank(S):
    c = synth.linear_case("rmax", 303, 64, 256, 256, 256, x_outlier_n=4, x_outlier_scale=40.0)
    ref, f, layer, X, ws, Y = run_case(S, c)
    assert rel_max_err(Y, f["Y"]) <= TOL_F32


@pytest.mark.parametrize("seed", [310, 311])
def test_on_grid_inputs_are_exact(S, seed):
    """Inputs on the INT4 grid with unit scales, r = 0, no smoothing, no bias:
    every product and partial sum is an exact small integer, so the fp32
    output must equal X W^T bit for bit."""
    c = synth.on_grid_case(seed, 96, 160, 320, exp_lo=0, exp_hi=0)
    ref, f, layer, X, ws, Y = run_case(S, c, smooth=False)
    exact = O.bf16_values(c.X) @ O.bf16_values(c.W).T
    assert np.array_equal(f["Y"], exact)
    assert np.array_equal(Y, exact)


def test_zero_activations_give_the_bias(S):
    c = synth.linear_case("zero", 312, 40, 96, 128, 4)
    c.X[:] = 0
    ref = O.prepare(c.W, None, c.bias, 4)
    layer = layer_from_oracle(ref)
    Y = to_f64(S.linear_forward(layer, bf16_to_device(c.X), out_dtype=torch.float32))
    assert np.array_equal(Y, np.broadcast_to(ref["bias"], Y.shape))


def test_split_calls_equal_forward_and_are_deterministic(S):
    c = synth.linear_case("split", 313, 200, 300, 384, 24, x_outlier_n=5, x_outlier_scale=50.0)
    ref, f, layer, X, ws, Y = run_case(S, c, check_codes=False)
    ws2 = layer.new_workspace(c.M)
    S.linear_quantize(layer, X, ws2)
    Y2 = torch.empty((c.M, c.N), dtype=torch.float32, device="cuda")
    S.linear_gemm(layer, c.M, Y2, ws2)
    Y3 = S.linear_forward(layer, X, out_dtype=torch.float32, workspace=ws2)
    torch.cuda.synchronize()
    assert np.array_equal(to_f64(Y2), Y) and np.array_equal(to_f64(Y3), Y)


def test_workspace_for_larger_M_serves_smaller_M(S):
    c = synth.linear_case("wsre", 314, 64, 128, 192, 8, x_outlier_n=2, x_outlier_scale=30.0)
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, 8)
    layer = layer_from_oracle(ref)
    big = layer.new_workspace(1000)
    Y = to_f64(S.linear_forward(layer, bf16_to_device(c.X), out_dtype=torch.float32, workspace=big))
    assert rel_max_err(Y, O.forward(ref, c.X)["Y"]) <= TOL_F32


def test_fused_gelu_epilogue(S):
    c = synth.linear_case("gelu", 315, 130, 260, 256, 8, x_outlier_n=4, x_outlier_scale=40.0)
    ref, f, layer, X, ws, _ = run_case(S, c, check_codes=False)
    G = to_f64(S.linear_forward(layer, X, out_dtype=torch.bfloat16, gelu=True, workspace=ws))
    Gref = OG.gelu_tanh_bf16(f["Y"])
    # gelu is 1.13-Lipschitz: the 2e-3 bar on Y carries through, plus bf16 output rounding
    assert np.max(np.abs(G - Gref)) <= (1.13 * TOL_F32 + 2.0 ** -8) * np.max(np.abs(f["Y"]))


@pytest.mark.parametrize("n", [8, 1000, 4099, 1 << 16])
def test_gelu_kernel_within_one_bf16_ulp(S, n):
    rng = np.random.default_rng(n)
    x = synth.f32_to_bf16_bits((rng.standard_normal(n) * 3).astype(np.float32))
    x[:7] = synth.f32_to_bf16_bits(np.array([0.0, -0.0, 20.0, -20.0, -7.5, -9.75, -10.0], np.float32))
    announce(f"gelu n={n}")
    y = S.gelu_tanh_bf16(bf16_to_device(x))
    got = to_f64(y)
    ref = OG.gelu_tanh_bf16(O.bf16_values(x))
    # one bf16 ulp of the reference; results smaller than 2^-100 in magnitude
    # (inputs below about -9.8) may flush to zero in the fp32 exp/reciprocal
    ulp = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(ref), 1e-300))) - 7, -133))
    tiny = (np.abs(ref) < 2.0 ** -100) & (np.abs(got) < 2.0 ** -100)
    assert np.all((np.abs(got - ref) <= ulp) | tiny)
    assert np.mean(got == ref) > 0.99


# K-split of the GEMM: tile grids smaller than the chip's CU count run as
# ksplit K ranges whose fp32 partial tiles a second kernel sums in order
# (sizing rule: tiles T of 128 x 256 < 128 -> ksplit = min(8, 512 // T,
# groups // 8) when that is at least 2).
def ksplit_of(M, N, K):
    T = -(-M // 128) * -(-N // 256)
    if T >= 128:
        return 1
    s = min(8, 512 // T, K // 64 // 8)
    return s if s >= 2 else 1


@pytest.mark.parametrize("M,N,K,rank,out,gelu", [(100, 200, 1024, 8, torch.float32, False),
                                                 (300, 600, 2048, 16, torch.float32, False),
                                                 (129, 257, 4096, 32, torch.float32, False),
                                                 (64, 512, 1600, 5, torch.bfloat16, True),
                                                 (1, 3072, 12288, 32, torch.bfloat16, False),
                                                 # N not a multiple of 8: the partial sum's per-element tail
                                                 (70, 300, 1024, 8, torch.bfloat16, False),
                                                 (33, 130, 2048, 4, torch.float32, True)])
def test_k_split_gemm(S, M, N, K, rank, out, gelu):
    ks = ksplit_of(M, N, K)
    assert ks >= 2
    c = synth.linear_case(f"ks{M}x{N}x{K}", 500 + M, M, N, K, rank,
                          x_outlier_n=max(1, K // 64), x_outlier_scale=40.0)
    ref, f, layer, X, ws, Y = run_case(S, c, out_dtype=out, gelu=gelu, check_codes=False)
    Yref = OG.gelu_tanh_bf16(f["Y"]) if gelu else f["Y"]
    tol = TOL_BF16 if out == torch.bfloat16 else TOL_F32
    err = np.max(np.abs(Y - Yref)) / np.max(np.abs(f["Y"]))
    announce(f"k-split {ks} max err / max|Y| {err:.3e}")
    assert err <= (1.13 * TOL_F32 + 2.0 ** -8 if gelu else tol)
    # the same layer with a workspace one byte short of the partials' room
    # runs the unsplit GEMM; both agree with the oracle and with each other
    part = ks * (-(-M // 256) * 256) * (-(-N // 256) * 256) * 4
    small = torch.empty(ws.numel() - part, dtype=torch.uint8, device=ws.device)
    Y1 = to_f64(S.linear_forward(layer, X, out_dtype=out, gelu=gelu, workspace=small))
    torch.cuda.synchronize()
    err1 = np.max(np.abs(Y1 - Yref)) / np.max(np.abs(f["Y"]))
    assert err1 <= (1.13 * TOL_F32 + 2.0 ** -8 if gelu else tol)
    assert np.max(np.abs(Y1 - Y)) / np.max(np.abs(f["Y"])) <= 2 * tol


# Narrow tiles: a grid of fewer than 128 tiles of 128 x 256 whose 64 x 128
# grid holds at least 256 tiles runs the narrow-tile GEMM (no K-split).
def narrow_of(M, N):
    wide = -(-M // 128) * -(-N // 256)
    return wide < 128 and -(-M // 64) * -(-N // 128) >= 256


@pytest.mark.parametrize("M,N,K,rank,out,gelu", [(1000, 2000, 640, 16, torch.float32, False),
                                                 # N not a multiple of 8: the epilogue's scalar tail
                                                 (777, 4100, 1088, 32, torch.bfloat16, True),
                                                 (1024, 3072, 3072, 0, torch.float32, False),
                                                 (1100, 2100, 1024, 100, torch.bfloat16, False),
                                                 # fewer groups than the four stages in flight
                                                 (1024, 2048, 64, 0, torch.bfloat16, False),
                                                 (1024, 2048, 128, 8, torch.float32, False),
                                                 (1024, 3072, 192, 16, torch.float32, True)])
def test_narrow_tile_gemm(S, M, N, K, rank, out, gelu):
    """The narrow-tile GEMM (64 x 128 workgroup tiles, one row of matrix
    tiles per wavefront) against the oracle: ragged M and N, rank 0 and
    ranks of one to four 32-rank chunks, GELU, both output types."""
    assert narrow_of(M, N)
    c = synth.linear_case(f"nt{M}x{N}x{K}", 700 + M, M, N, K, rank,
                          x_outlier_n=max(1, K // 64), x_outlier_scale=40.0)
    ref, f, layer, X, ws, Y = run_case(S, c, out_dtype=out, gelu=gelu, check_codes=False)
    Yref = OG.gelu_tanh_bf16(f["Y"]) if gelu else f["Y"]
    tol = TOL_BF16 if out == torch.bfloat16 else TOL_F32
    err = np.max(np.abs(Y - Yref)) / np.max(np.abs(f["Y"]))
    announce(f"narrow tiles max err / max|Y| {err:.3e}")
    assert err <= (1.13 * TOL_F32 + 2.0 ** -8 if gelu else tol)


def test_matrix_probe_runs_and_is_deterministic(S):
    """The matrix-instruction probe behind the achievable-peak figures (not
    part of the layer): every kind runs, and two runs fold to the same words."""
    sink = torch.zeros(8, dtype=torch.int32, device="cuda")
    for kind in list(S.MFMA_KINDS) + list(S.MFMA_MIXES):
        S.measure_mfma(kind, 16, 8, sink)
        a = sink.clone()
        S.measure_mfma(kind, 16, 8, sink)
        torch.cuda.synchronize()
        assert torch.equal(a, sink), kind
