"""GPU parity on the quantisers' edge cases, element by element against the
oracle, through the C ABI:

* INT4 quantiser (kernel 1): inputs that land exactly on k + 1/2 after the
  multiply by fl32(7/a) (round half to even decides them), groups whose
  max |x_hat| is below 2^-100 (scale 0, codes 0), exactly 2^-100 (the
  smallest live group), bf16 subnormals, -0, and smoothing factors that
  move values in and out of the fp32 subnormal range;
* the quantiser inside fc1's GEMM epilogue for a fused MLP pair, fed the
  same kinds of values through a crafted fc1 whose output is exact;
* the MXFP4 encoder (kernel 1, FP4 form): every multiple of 1/128 in
  [-8, 8] as a scaled value, FP4 midpoints, saturation past 6, -0, huge and
  tiny block maxima;
* the forward on weights prepared by the library's own svdq_prepare_weights
  (rank 32), checked against the oracle's forward on those same artifacts.

Bars: codes and scales bit-exact; Y within 2e-3 * max|Y_ref| (fp32 out),
D within 1e-5 * max|D_ref|."""
import numpy as np
import pytest
import torch

import synth
from oracle import glue as OG
from oracle import mxfp4 as MX
from oracle import svdquant as O
from tests.conftest import announce
from tests.gpu_util import (bf16_to_device, decode_fp6_codes, decode_scales, layer_from_oracle,
                            mx_layer_from_oracle, rel_max_err, to_f64, workspace_regions)

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-3
F32 = np.float32


@pytest.fixture(scope="module")
def S():
    import w4a4_rank_corrected_smooth_amd as lib
    lib.device_check()
    return lib


def bits(values) -> np.ndarray:
    """float values that are exactly bf16 -> bf16 bit patterns."""
    return O.bf16_bits_of(np.asarray(values, dtype=np.float64))


def tie_fraction(X_vals: np.ndarray, iota: np.ndarray) -> tuple:
    """(# elements whose fl32(x_hat * fl32(7/a)) is exactly k + 1/2, # groups
    with 0 < a < 2^-100) in the oracle's own arithmetic: the test checks
    that its inputs really exercise those branches."""
    xh = O.smooth_activations(X_vals, iota)
    M, K = xh.shape
    g = xh.reshape(M, K // 64, 64)
    a = np.abs(g).max(axis=-1)
    live = a >= F32(2.0 ** -100)
    inv = (F32(7.0) / np.where(live, a, F32(1.0))).astype(F32)
    t = (g * inv[..., None]).astype(F32)
    ties = (t - np.floor(t) == 0.5) & live[..., None]
    return int(ties.sum()), int(((a > 0) & ~live).sum())


def int4_edge_rows(rng, M, K):
    """bf16 activation rows, each group of a row built to hit one edge."""
    G = K // 64
    X = np.zeros((M, K))
    for m in range(M):
        for g in range(G):
            kind = (m + 3 * g) % 9
            v = np.zeros(64)
            if kind in (0, 1):      # a = 7: half-integers are ties after x 1
                v = rng.integers(-13, 14, 64) / 2.0
                v[rng.integers(64)] = 7.0 * (1 if kind == 0 else -1)
            elif kind == 2:         # a = 14: odd integers are ties after x 1/2
                v = rng.integers(-14, 15, 64).astype(float)
                v[rng.integers(64)] = -14.0
            elif kind == 3:         # a = 3.5: odd quarters are ties after x 2
                v = rng.integers(-14, 15, 64) / 4.0
                v[rng.integers(64)] = 3.5
            elif kind == 4:         # 0 < a < 2^-100: scale 0, codes 0
                v = rng.choice([-1, 1], 64) * 2.0 ** rng.integers(-126, -101, 64)
            elif kind == 5:         # a = 2^-100 exactly: smallest live group, ties at 3.5
                v = rng.choice([-1.0, 1.0], 64) * rng.choice([2.0 ** -101, 3 * 2.0 ** -102, 2.0 ** -103], 64)
                v[rng.integers(64)] = 2.0 ** -100
            elif kind == 6:         # bf16 subnormals only (fp32 subnormal after x 1)
                v = rng.choice([-1, 1], 64) * rng.integers(1, 128, 64) * 2.0 ** -133
            elif kind == 7:         # -0 everywhere, and -0 among normal values
                v = np.full(64, -0.0)
                if m % 2:
                    v[::3] = rng.integers(-7, 8, len(v[::3])) + 0.5
            else:                   # ordinary values with subnormals and -0 mixed in
                v = np.round(rng.standard_normal(64) * 64) / 32
                v[::5] = -0.0
                v[1::7] = rng.integers(1, 128, len(v[1::7])) * 2.0 ** -133
            X[m, 64 * g: 64 * g + 64] = v
    return bits(X)


def check_quantiser(S, layer, ref, Xb):
    X = bf16_to_device(Xb)
    ws = layer.new_workspace(Xb.shape[0])
    q, s, d = S.quantize_activations(layer, X, ws)
    Y = S.linear_forward(layer, X, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    f = O.forward(ref, Xb)
    assert np.array_equal(q.cpu().numpy(), O.pack_int4(f["qA"])), "activation codes"
    sd = s.cpu().numpy()
    assert np.array_equal(sd.view(np.uint32), f["sA"].view(np.uint32)), "activation scales (bits)"
    if ref["rank"] > 0 and np.max(np.abs(f["D"])) > 0:
        assert rel_max_err(to_f64(d), f["D"]) <= 1e-5
    assert rel_max_err(to_f64(Y), f["Y"]) <= TOL_F32
    return f


@pytest.mark.parametrize("M,K,rank", [(96, 576, 8), (45, 192, 0)])
def test_int4_quantiser_ties_tiny_subnormal_negzero(S, M, K, rank):
    rng = np.random.default_rng(7000 + M)
    Xb = int4_edge_rows(rng, M, K)
    c = synth.linear_case("edge-w", 7100 + M, 8, 136, K, rank)
    ref = O.prepare(c.W, None, c.bias, rank)               # no smoothing: iota = 1
    ties, tiny = tie_fraction(O.bf16_values(Xb), ref["iota"])
    announce(f"int4 edges M={M} K={K} r={rank}: {ties} exact ties, {tiny} tiny groups")
    assert ties > 200 and tiny > 5
    f = check_quantiser(S, layer_from_oracle(ref), ref, Xb)
    assert np.any(f["sA"] == 0) and np.any(f["sA"] == F32(2.0 ** -100) / F32(7))


def test_int4_quantiser_smoothing_through_subnormal_range(S):
    """Smoothing factors from 2^-24 to 2^24 (fp32 values, as the layer
    carries them) move x_hat across the fp32 subnormal range and back; one
    fl32 multiply per element, as the oracle does."""
    rng = np.random.default_rng(7200)
    M, K = 64, 384
    c = synth.linear_case("edge-s", 7201, 8, 96, K, 4)
    ref = dict(O.prepare(c.W, None, c.bias, 4))
    iota = (2.0 ** rng.integers(-24, 25, K) * (1 + rng.integers(0, 2 ** 23, K) / 2.0 ** 23)).astype(F32)
    ref["iota"] = iota
    X = np.zeros((M, K))
    for m in range(M):
        e = rng.integers(-133, -95)
        X[m] = rng.choice([-1, 1], K) * rng.integers(1, 256, K) * 2.0 ** e
        X[m, ::11] = -0.0
        if m % 4 == 0:
            X[m] = O.round_to_bf16(rng.standard_normal(K))
    Xb = bits(O.round_to_bf16(X))
    xh = O.smooth_activations(O.bf16_values(Xb), iota)
    sub = (xh != 0) & (np.abs(xh) < 2.0 ** -126)
    announce(f"int4 smoothing edges: {int(sub.sum())} subnormal x_hat")
    assert sub.sum() > 100
    check_quantiser(S, layer_from_oracle(ref), ref, Xb)


# ----------------------------------------------------- fused epilogue quantiser
def crafted_fc1(rng, M, G2, gelu):
    """fc1 whose output is exact and whose every 64-channel group (fc2's
    quantisation groups) is built to hit one edge.  Rank 0, no smoothing;
    each output channel n reads one input channel with weight +-1 (code
    +-7, scale fl32(1/7)), so Y1[m, n] = +-X[m, j(n)] + b[n] exactly for
    integer |X| <= 7 (7 fl32(1/7) = 1 + 3e-8 rounds away), X being integers
    in [-6, 6] except the anchor columns 0 and 64 (value 7, so every input
    group has scale 1 and codes equal to X)."""
    K1, N1 = 128, 64 * G2
    X = rng.integers(-6, 7, size=(M, K1)).astype(float)
    X[:, 0] = 7.0
    X[:, 64] = 7.0
    W = np.zeros((N1, K1))
    b = np.zeros(N1)
    for g in range(G2):
        kind = g % 8
        cols = slice(64 * g, 64 * g + 64)
        if kind in (0, 1):                      # ties: half-integers, group max exactly 7
            src = rng.integers(1, 64, 64) + 64 * rng.integers(0, 2, 64)
            src[src == 64] = 65
            W[np.arange(64 * g, 64 * g + 64), src] = rng.choice([-1.0, 1.0], 64)
            b[cols] = rng.choice([-0.5, 0.0, 0.5], 64)
            W[64 * g, :] = 0.0
            W[64 * g, 0] = 1.0                  # reads the anchor: 7
            b[64 * g] = 0.0
        elif kind == 2:                         # all zero (or all -0 after GELU's tail)
            b[cols] = -20.0 if gelu else 0.0
        elif kind == 3:                         # 0 < a < 2^-100
            b[cols] = rng.choice([-1, 1], 64) * 2.0 ** -110
        elif kind == 4:                         # a = 2^-100: ties at 3.5
            b[cols] = rng.choice([-1, 1], 64) * rng.choice([2.0 ** -101, 3 * 2.0 ** -102], 64)
            b[64 * g + 5] = 2.0 ** -100
        elif kind == 5:                         # just below the live threshold
            b[cols] = rng.choice([-1, 1], 64) * 2.0 ** -100 * (255 / 256)
        elif kind == 6:                         # bf16 subnormal biases
            b[cols] = rng.choice([-1, 1], 64) * rng.integers(1, 128, 64) * 2.0 ** -133
        else:                                   # ordinary values, some -0 after GELU
            src = rng.integers(0, 128, 64)
            W[np.arange(64 * g, 64 * g + 64), src] = 1.0
            b[cols] = rng.choice([0.25, -0.75, -20.0], 64)
    return bits(X), bits(W), bits(b)


@pytest.mark.parametrize("gelu,r2", [(False, 0), (False, 8), (True, 8)])
def test_fused_epilogue_quantiser_edges(S, gelu, r2):
    rng = np.random.default_rng(7300 + r2 + gelu)
    M, G2, N2 = 96, 8, 72
    Xb, W1b, b1b = crafted_fc1(rng, M, G2, gelu)
    ref1 = O.prepare(W1b, None, b1b, 0)
    l1 = layer_from_oracle(ref1)
    c2 = synth.linear_case("edge-fc2", 7310, 8, N2, 64 * G2, r2)
    ref2 = O.prepare(c2.W, None, c2.bias, r2)                # fc2 unsmoothed: iota = 1
    l2 = layer_from_oracle(ref2)
    X = bf16_to_device(Xb)
    announce(f"fused epilogue edges gelu={gelu} r2={r2}")
    # fc1's output as the unfused path stores it (the values the fused
    # epilogue quantises, by the reading that fc2's input is the device's own
    # fc1 output)
    Y1 = S.linear_forward(l1, X, out_dtype=torch.bfloat16, gelu=gelu)
    ws1, ws2 = l1.new_workspace(M), l2.new_workspace(M)
    S.mlp_quantize(l1, l2, X, ws1, ws2)
    S.mlp_gemm1(l1, l2, M, ws1, ws2, gelu=gelu)
    Y = S.mlp_gemm2(l2, M, torch.empty((M, N2), dtype=torch.float32, device="cuda"), ws2)
    torch.cuda.synchronize()
    X2 = Y1.cpu().view(torch.int16).numpy().view(np.uint16)
    y1_ref = O.forward(ref1, Xb)["Y"]
    if not gelu:
        # the crafted fc1 is exact: the device output is the oracle's, to the bit
        assert np.array_equal(O.bf16_values(X2), O.round_to_bf16(y1_ref))
    else:
        ref_g = OG.gelu_tanh_bf16(y1_ref)
        got = O.bf16_values(X2)
        tail = (np.abs(ref_g) < 2.0 ** -100) & (np.abs(got) < 2.0 ** -100)
        assert np.all((np.abs(got - ref_g) <= np.abs(ref_g) * 2.0 ** -8) | tail)
        assert np.any((got == 0) & np.signbit(got)), "GELU's tail gives -0"
    qA, sA = O.quantize_activations(O.bf16_values(X2), ref2["iota"])
    ties, tiny = tie_fraction(O.bf16_values(X2), ref2["iota"])
    announce(f"  fc2 input: {ties} exact ties, {tiny} tiny groups")
    assert tiny > 0 and (gelu or ties > 100)
    w = ws2.cpu().numpy()
    assert np.array_equal(decode_fp6_codes(w, M, 64 * G2), qA), "fused epilogue codes"
    sd = decode_scales(w, M, 64 * G2)
    assert np.array_equal(sd.view(np.uint32), sA.view(np.uint32)), "fused epilogue scales (bits)"
    f2 = O.forward(ref2, X2)
    if r2 > 0:
        _, _, _, d_off = workspace_regions(M, 64 * G2)
        Mp = -(-M // 256) * 256
        d = w[d_off: d_off + Mp * 32 * 8].view(np.int64).reshape(Mp, 32)[:M, :r2] / 2.0 ** 32
        assert rel_max_err(d, f2["D"]) <= 1e-5
    assert rel_max_err(to_f64(Y), f2["Y"]) <= TOL_F32


# ------------------------------------------------------------ MXFP4 encoder
def test_mx_encoder_sweep_every_128th(S):
    """Scaled values x_hat / 2^e on every multiple of 1/128 in [-8, 8]: each
    row is x = +-1, +-1/2, 2^100, 2^-120, -0 or alternating signs against
    per-channel smoothing factors that carry the sweep, each 32-channel
    block anchored by a factor of 7.9921875 so its scale is 2^0 (times the
    row's power of two).  The oracle's E2M1 rounding (nearest, ties to the
    even mantissa bit, saturation at 6, zero as +0) decides every element."""
    sweep = np.arange(-1024, 1025) / 128.0
    sweep = sweep[sweep != 0]                       # positive factors only: sign comes from x
    mags = np.unique(np.abs(sweep))                 # 1/128 .. 8
    per = 31
    nblk = -(-len(mags) // per)
    nblk += nblk % 2                                # whole groups of 64
    iota = np.full(nblk * 32, 1.0 / 128)
    for bk in range(nblk):
        chunk = mags[bk * per: (bk + 1) * per]
        iota[32 * bk: 32 * bk + len(chunk)] = chunk
        iota[32 * bk + 31] = 7.9921875
    iota = iota.astype(F32)
    K = len(iota)
    rows = [1.0, -1.0, 0.5, -0.5, 2.0 ** 100, -(2.0 ** -120), -0.0, 3.0]
    X = np.array([np.full(K, r) for r in rows])
    alt = np.where(np.arange(K) % 2, 1.0, -1.0)
    X = np.vstack([X, alt[None, :], -alt[None, :]])
    Xb = bits(X)
    M = Xb.shape[0]
    c = synth.linear_case("mx-sweep", 7400, 8, 64, K, 4)
    ref = dict(MX.prepare(c.W, None, c.bias, 4))
    ref["iota"] = iota
    announce(f"mx encoder sweep K={K} rows={M}")
    layer = mx_layer_from_oracle(ref)
    Xd = bf16_to_device(Xb)
    ws = layer.new_workspace(M)
    q, e, d = S.mx_quantize_activations(layer, Xd, ws)
    Y = S.mx_linear_forward(layer, Xd, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    f = MX.forward(ref, Xb)
    assert np.array_equal(e.cpu().numpy().astype(np.int64) - 127, f["eA"]), "E8M0 scales"
    assert np.array_equal(q.cpu().numpy(), MX.pack_fp4(f["qA"])), "E2M1 codes"
    # the sweep covers ties, saturation and signed zeros
    xh = O.smooth_activations(O.bf16_values(Xb), iota)
    r = xh / np.exp2(np.repeat(f["eA"], 32, axis=1))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert np.isin(np.abs(r), mids).sum() >= 7 * 8
    assert (np.abs(r) > 6).sum() > 0 and np.any((xh == 0) & np.signbit(xh))
    assert not np.any(f["qA"] == 8)                 # no -0 code
    assert rel_max_err(to_f64(Y), f["Y"]) <= TOL_F32


# ----------------------------------------------- library-prepared weights
def oracle_ref_from_library(hw) -> dict:
    """The library's prepared artifacts as the oracle's layer dict (shared
    artifacts: the SVD's signs and rotations are free, so the forward is
    checked on the library's own factors, codes and scales)."""
    return dict(N=hw.N, K=hw.K, rank=hw.rank, iota=hw.inv_lambda.astype(F32),
                L1s=O.bf16_values(hw.l1s), L2b=O.bf16_values(hw.l2),
                qW=O.unpack_int4(hw.qweight), sW=hw.wscales.astype(F32),
                bias=hw.bias.astype(np.float64))


@pytest.mark.parametrize("which", ["tiny", "flux_width"])
def test_library_prepared_weights_forward(S, which):
    if which == "tiny":
        c = synth.tiny_case()
        rows = None
    else:
        # Flux-width projection (3072 -> 3072) on the QKV activation
        # distribution (0.5% of channels x50, weight channels x8), all 4608 tokens
        c = synth.linear_case("flux-width", 7501, 4608, 3072, 3072, 32, x_outlier_frac=0.005,
                              x_outlier_scale=50.0, w_outlier_frac=0.01, w_outlier_scale=8.0)
        rows = np.unique(np.concatenate([np.arange(0, 4608, 97), [4607]]))
    announce(f"library-prepared {which}: M={c.M} N={c.N} K={c.K} r=32")
    hw = S.prepare_weights(c.W, c.calib_absmax(), c.bias, 32)
    ref = oracle_ref_from_library(hw)
    layer = S.Linear(hw)
    X = bf16_to_device(c.X)
    ws = layer.new_workspace(c.M)
    q, s, d = S.quantize_activations(layer, X, ws)
    Y = S.linear_forward(layer, X, out_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    qA, sA = O.quantize_activations(O.bf16_values(c.X), ref["iota"])
    assert np.array_equal(q.cpu().numpy(), O.pack_int4(qA)), "activation codes"
    assert np.array_equal(s.cpu().numpy(), sA), "activation scales"
    f = O.forward(ref, c.X, rows=rows)
    Yd = to_f64(Y) if rows is None else to_f64(Y[torch.from_numpy(rows).cuda()])
    Dd = to_f64(d) if rows is None else to_f64(d[torch.from_numpy(rows).cuda()])
    assert rel_max_err(Dd, f["D"]) <= 1e-5
    err = rel_max_err(Yd, f["Y"])
    announce(f"  max rel err {err:.3e}")
    assert err <= TOL_F32
    # quality sanity (not parity): the library's artifacts approximate the
    # layer about as well as the oracle's own prepare
    Xv = O.bf16_values(c.X if rows is None else c.X[rows])
    exact = Xv @ O.bf16_values(c.W).T + O.bf16_values(c.bias)[None, :]
    own = O.forward(O.prepare(c.W, c.calib_absmax(), c.bias, 32), c.X, rows=rows)["Y"]
    assert np.linalg.norm(Yd - exact) <= 1.1 * np.linalg.norm(own - exact)
