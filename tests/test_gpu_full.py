"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times: the Flux-like fused QKV projection, the MLP pair (fc1 with
the fused GELU epilogue feeding fc2), the low-resolution high-rank layer and
the AWQ W4A16 modulation projection.  Activation codes, scales and the
low-rank down-projection are compared in full; group sums on windows; the
outputs on sampled token rows (every output channel of each sampled row)
which the oracle evaluates directly."""
import numpy as np
import pytest
import torch

import synth
from oracle import svdquant as O
from oracle import awq as OA
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


def sample_rows(M, seed, n=40):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, n, replace=False)]))


def layer_run(S, name, ref, X_bits, M, out_dtype=torch.float32, gelu=False):
    announce(f"{name}: device forward M={M} N={ref['N']} K={ref['K']} r={ref['rank']} gelu={gelu}")
    layer = layer_from_oracle(ref)
    X = bf16_to_device(X_bits)
    ws = layer.new_workspace(M)
    Y = S.linear_forward(layer, X, out_dtype=out_dtype, gelu=gelu, workspace=ws)
    q, s, d = S.quantize_activations(layer, X, ws)
    torch.cuda.synchronize()
    return dict(layer=layer, X=X, ws=ws, Y=Y, q=q, s=s, d=d)


def check_codes(ref, X_bits, run):
    qA, sA = O.quantize_activations(O.bf16_values(X_bits), ref["iota"])
    assert np.array_equal(run["q"].cpu().numpy(), O.pack_int4(qA)), "activation codes"
    assert np.array_equal(run["s"].cpu().numpy(), sA), "activation scales"
    D = O.lowrank_down(O.bf16_values(X_bits), ref["L1s"])
    assert rel_max_err(to_f64(run["d"]), D) <= 1e-5, "low-rank down-projection"
    return qA


# ---------------------------------------------------------------- QKV
@pytest.fixture(scope="module")
def qkv(S):
    c = synth.qkv_case()
    announce("qkv: oracle prepare 9216x3072 r32")
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, c.rank)
    return c, ref, layer_run(S, "qkv", ref, c.X, c.M)


def test_qkv_codes_scales_and_down_projection(qkv):
    c, ref, run = qkv
    check_codes(ref, c.X, run)


def test_qkv_group_sums_windows(S, qkv):
    c, ref, run = qkv
    qA, _ = O.quantize_activations(O.bf16_values(c.X), ref["iota"])
    for (m0, mc, n0, nc) in [(0, 128, 0, 128), (4480, 128, 9088, 128), (2000, 70, 5000, 90)]:
        announce(f"qkv group sums m0={m0} n0={n0}")
        P = S.debug_group_sums(run["layer"], c.M, m0, mc, n0, nc, run["ws"]).cpu().numpy()
        assert np.array_equal(P, O.group_sums(qA[m0:m0 + mc], ref["qW"][n0:n0 + nc]))


def test_qkv_output_sampled_rows(qkv):
    c, ref, run = qkv
    rows = sample_rows(c.M, 1)
    f = O.forward(ref, c.X, rows=rows)
    Y = to_f64(run["Y"])[rows]
    err = rel_max_err(Y, f["Y"])
    announce(f"qkv max rel err {err:.3e}")
    assert err <= TOL_F32


# ---------------------------------------------------------------- MLP
@pytest.fixture(scope="module")
def mlp(S):
    fc1, W2, b2 = synth.mlp_cases()
    announce("mlp: oracle prepare fc1 12288x3072 r32")
    ref1 = O.prepare(fc1.W, fc1.calib_absmax(), fc1.bias, 32)
    announce("mlp: oracle fc1 forward (full) for fc2's input")
    Y1 = O.forward(ref1, fc1.X)["Y"]
    X2 = O.bf16_bits_of(OG.gelu_tanh_bf16(Y1))
    del Y1
    announce("mlp: oracle prepare fc2 3072x12288 r32")
    ax2 = O.calibration_absmax(O.bf16_values(X2[:64]))
    ref2 = O.prepare(W2, ax2, b2, 32)
    return fc1, ref1, X2, ref2


def test_mlp_fc1_fused_gelu_as_benchmarked(S, mlp):
    fc1, ref1, X2, ref2 = mlp
    run = layer_run(S, "fc1", ref1, fc1.X, fc1.M, out_dtype=torch.bfloat16, gelu=True)
    check_codes(ref1, fc1.X, run)
    rows = sample_rows(fc1.M, 2)
    Yref = O.forward(ref1, fc1.X, rows=rows)["Y"]
    G = to_f64(run["Y"])[rows]
    err = np.max(np.abs(G - OG.gelu_tanh_bf16(Yref))) / np.max(np.abs(Yref))
    announce(f"fc1+gelu max err / max|Y| {err:.3e}")
    assert err <= 1.13 * TOL_F32 + 2.0 ** -8
    Yf = to_f64(S.linear_forward(run["layer"], run["X"], out_dtype=torch.float32,
                                 workspace=run["ws"]))[rows]
    assert rel_max_err(Yf, Yref) <= TOL_F32


def test_mlp_fc2(S, mlp):
    fc1, ref1, X2, ref2 = mlp
    run = layer_run(S, "fc2", ref2, X2, fc1.M, out_dtype=torch.bfloat16)
    check_codes(ref2, X2, run)
    rows = sample_rows(fc1.M, 3)
    Yref = O.forward(ref2, X2, rows=rows)["Y"]
    err = rel_max_err(to_f64(run["Y"])[rows], Yref)
    announce(f"fc2 bf16 max rel err {err:.3e}")
    assert err <= TOL_BF16
    Yf = to_f64(S.linear_forward(run["layer"], run["X"], out_dtype=torch.float32,
                                 workspace=run["ws"]))[rows]
    assert rel_max_err(Yf, Yref) <= TOL_F32


def test_mlp_pair_fused_as_benchmarked(S, mlp):
    """The benchmarked step's MLP: fc1's GEMM quantises fc2's input in its
    epilogue.  fc2's codes and scales equal the unfused quantiser's on the
    same bf16 intermediate (the device's own GELU(fc1) output), bit for bit;
    fc2's output on sampled rows matches the oracle run on that intermediate;
    the fixed-point down-projection matches the oracle's."""
    fc1, ref1, _, ref2 = mlp
    M = fc1.M
    announce("mlp fused pair: device")
    l1, l2 = layer_from_oracle(ref1), layer_from_oracle(ref2)
    X = bf16_to_device(fc1.X)
    Y1 = S.linear_forward(l1, X, out_dtype=torch.bfloat16, gelu=True)
    ws1, ws2, ws2u = l1.new_workspace(M), l2.new_workspace(M), l2.new_workspace(M)
    Y2 = S.mlp_forward(l1, l2, X, out_dtype=torch.bfloat16, ws1=ws1, ws2=ws2)
    S.linear_quantize(l2, Y1, ws2u)
    torch.cuda.synchronize()
    K2, G2, Mp, rp = ref2["K"], ref2["K"] // 64, -(-M // 256) * 256, 32
    qa_bytes = Mp * K2 * 3 // 4
    sa_off = -(-qa_bytes // 256) * 256
    sa_bytes = G2 * Mp * 16                        # scales as 16-byte operands
    d_off = -(-(sa_off + sa_bytes) // 256) * 256
    assert torch.equal(ws2[:qa_bytes], ws2u[:qa_bytes]), "fc2 codes"
    assert torch.equal(ws2[sa_off:sa_off + sa_bytes], ws2u[sa_off:sa_off + sa_bytes]), "fc2 scales"
    X2 = Y1.cpu().view(torch.int16).numpy().view(np.uint16)
    rows = sample_rows(M, 5)
    f = O.forward(ref2, X2, rows=rows)
    err = rel_max_err(to_f64(Y2)[rows], f["Y"])
    announce(f"mlp fused pair bf16 max rel err {err:.3e}")
    assert err <= TOL_BF16
    d = ws2[d_off:d_off + Mp * rp * 8].cpu().numpy().view(np.int64).reshape(Mp, rp)[rows, :32] / 2.0 ** 32
    assert rel_max_err(d, f["D"]) <= 1e-5, "fixed-point down-projection"


# -------------------------------------------------------------- low-res
def test_lowres_high_rank_full(S):
    c = synth.lowres_case()
    announce("lowres: oracle prepare 3072x3072 r128")
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, c.rank)
    run = layer_run(S, "lowres", ref, c.X, c.M)
    check_codes(ref, c.X, run)
    f = O.forward(ref, c.X)
    err = rel_max_err(to_f64(run["Y"]), f["Y"])
    announce(f"lowres max rel err {err:.3e}")
    assert err <= TOL_F32


# ------------------------------------------------------------------ AWQ
@pytest.fixture(scope="module")
def awq(S):
    a = synth.awq_case()
    announce("awq: oracle quantize 18432x3072")
    q, s, z = OA.quantize(a.W)
    layer = S.AwqLinear(OA.pack(q), s, z, "cuda")
    return a, q, s, z, layer


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_awq_full(S, awq, M):
    a, q, s, z, layer = awq
    announce(f"awq M={M}")
    x = torch.from_numpy(np.ascontiguousarray(a.x[:M])).to("cuda")
    y = to_f64(S.awq_forward(layer, x))
    yref = OA.forward(a.x[:M], q, s, z)
    assert rel_max_err(y, yref) <= 2e-3 + 2.0 ** -11


@pytest.mark.parametrize("M,N,K", [(5, 100, 192), (16, 250, 1600), (4, 100, 1600), (9, 48, 768),
                                   (7, 17, 832), (1, 33, 64), (12, 4100, 3072), (10, 40, 64),
                                   (13, 272, 4160), (8, 64, 3200), (16, 96, 12288), (11, 16, 128),
                                   (14, 9, 640), (16, 33, 3072)])
def test_awq_ragged_with_bias(S, M, N, K):
    """Both shapes of the AWQ kernel (one tile and chunks of 12 groups up to
    8 rows; two tiles per workgroup and chunks of 4 groups from 9): ragged
    column tiles, an odd tile count (the last workgroup's second tile past
    the end), a single tile, spare wavefronts, odd group counts, one chunk,
    several chunks, a last chunk past a wavefront's groups, a wavefront with
    no groups of its own."""
    announce(f"awq ragged M={M} N={N} K={K}")
    a = synth.awq_case(m_max=M, N=N, K=K, seed=44 + M)
    q, s, z = OA.quantize(a.W)
    layer = S.AwqLinear(OA.pack(q), s, z, "cuda")
    bias = (np.random.default_rng(1).standard_normal(N) * 0.01).astype(np.float16)
    y = to_f64(S.awq_forward(layer, torch.from_numpy(a.x).to("cuda"),
                             bias=torch.from_numpy(bias).to("cuda")))
    yref = OA.forward(a.x, q, s, z, bias.astype(np.float64))
    assert rel_max_err(y, yref) <= 2e-3 + 2.0 ** -11


# ------------------------------------------------------- largest input
def test_largest_input_accepted(S):
    """M * K = 2^31, the largest input the C ABI accepts (131072 tokens x
    16384 channels, 4 GiB of bf16 activations; N = 256, r = 16): codes,
    scales, the down-projection and Y on sampled rows, the first and last
    rows among them; one row more is rejected before any launch."""
    M, N, K, r = 131072, 256, 16384, 16
    assert M * K == 2 ** 31
    dev = torch.device("cuda")
    announce(f"largest: drawing X {M}x{K} on the device")
    X, _ = synth.device_normal_bf16(M, K, 800, dev, outlier_n=64, outlier_scale=40.0)
    w = synth.linear_case("largest_w", 801, 8, N, K, r)
    ax = O.calibration_absmax(X[:64].float().cpu().numpy())
    announce("largest: oracle prepare 256x16384 r16")
    ref = O.prepare(w.W, ax, w.bias, r)
    layer = layer_from_oracle(ref)
    ws = layer.new_workspace(M)
    announce(f"largest: device forward, workspace {ws.numel() / 2**30:.2f} GiB")
    Y = S.linear_forward(layer, X, out_dtype=torch.bfloat16, workspace=ws)
    q, s, d = S.quantize_activations(layer, X, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(802)
    rows = np.unique(np.concatenate([[0, 1, M // 2, M - 2, M - 1], rng.choice(M, 40, replace=False)]))
    ridx = torch.from_numpy(rows).to(dev)
    Xr = X[ridx].cpu().view(torch.int16).numpy().view(np.uint16)
    f = O.forward(ref, Xr)
    assert np.array_equal(q[ridx].cpu().numpy(), O.pack_int4(f["qA"])), "activation codes"
    assert np.array_equal(s[ridx].cpu().numpy(), f["sA"]), "activation scales"
    assert rel_max_err(to_f64(d[ridx]), f["D"]) <= 1e-5, "low-rank down-projection"
    err = rel_max_err(to_f64(Y[ridx]), f["Y"])
    announce(f"largest max rel err {err:.3e}")
    assert err <= TOL_BF16
    import ctypes
    st = S._lib.svdq_linear_forward(ctypes.byref(layer._w), X.data_ptr(), M + 1, Y.data_ptr(), S.BF16, 0,
                                    ws.data_ptr(), ws.numel(), None)
    assert st == 2, "one row past M * K = 2^31 is an unsupported shape"
