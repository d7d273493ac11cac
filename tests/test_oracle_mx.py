"""Pins of the MXFP4 oracle (``oracle/mxfp4.py``) against what fixes it
without a second implementation: the FP4 E2M1 encoding's closed form (sign,
two exponent bits with bias 1, one mantissa bit, subnormals at exponent 0),
nearest-value rounding checked by brute force over the whole code table,
the tie and saturation cases written out by hand, the block-scale rule on
blocks whose answer is known, exact round trips of values already on the
grid, an exact forward on on-grid inputs, and an independent scalar
implementation on small inputs."""
import itertools

import numpy as np
import pytest

import synth
from oracle import mxfp4 as MX
from oracle import svdquant as O


def e2m1_closed_form(code: int) -> float:
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def test_e2m1_table_from_bit_fields():
    got = MX.e2m1_value(np.arange(16))
    want = np.array([e2m1_closed_form(c) for c in range(16)])
    assert np.array_equal(got, want)
    assert list(np.unique(np.abs(want))) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def brute_force_code(r: float) -> int:
    """Nearest of the 15 distinct values; ties to the code with mantissa bit
    0; beyond 6 in magnitude the largest; zero as +0."""
    best = None
    for c in range(16):
        if c == 8:
            continue                                     # -0: zero is stored as +0
        v = e2m1_closed_form(c)
        d = abs(r - v)
        key = (d, c & 1)                                 # prefer the even mantissa on ties
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_rounding_is_nearest_by_brute_force():
    rng = np.random.default_rng(5)
    r = np.concatenate([rng.uniform(-7.9, 7.9, 4000), rng.uniform(-1, 1, 1000),
                        np.arange(-31, 32) / 4.0])       # every multiple of 1/4: all the ties
    got = MX.e2m1_round(r)
    want = np.array([brute_force_code(float(x)) for x in r], np.uint8)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("r,v", [(0.25, 0.0), (0.2500001, 0.5), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0),
                                 (2.5, 2.0), (3.5, 4.0), (5.0, 4.0), (5.0001, 6.0), (6.5, 6.0),
                                 (7.99, 6.0), (-2.5, -2.0), (-5.0, -4.0), (-0.1, 0.0), (1e-30, 0.0)])
def test_ties_saturation_and_signed_zero(r, v):
    c = int(MX.e2m1_round(np.array([r]))[0])
    assert MX.e2m1_value(np.array([c]))[0] == v
    if v == 0.0:
        assert c == 0                                    # zeros are +0


def test_block_scale_rule():
    rows = []
    for k in (-3, 0, 5):
        b = np.zeros(32)
        b[7] = 6 * 2.0 ** k;  rows.append((b.copy(), k, 7))       # max maps to 6
        b[7] = -4 * 2.0 ** k; rows.append((b.copy(), k, 8 | 6))   # to -4
        b[7] = 7.9 * 2.0 ** k; rows.append((b.copy(), k, 7))      # above 6: saturates
        b[7] = 2.0 ** k;      rows.append((b.copy(), k - 2, 6))   # a power of two maps to 4
    V = np.stack([r[0] for r in rows]).astype(np.float32)
    q, e = MX.quantize_rows(V)
    for i, (_, ek, ck) in enumerate(rows):
        assert e[i, 0] == ek and q[i, 7] == ck
    # an all-zero block, and blocks far below the normal range
    Z = np.zeros((1, 32), np.float32)
    qz, ez = MX.quantize_rows(Z)
    assert ez[0, 0] == -127 and not qz.any()
    T = np.zeros((1, 32), np.float32)
    T[0, 3] = np.float32(2.0 ** -140)
    qt, et = MX.quantize_rows(T)
    assert et[0, 0] == -127                              # clamped at the E8M0 minimum
    assert MX.dequantize(qt, et)[0, 3] in (0.0, 2.0 ** -127 * 0.5)


def on_grid_rows(rng, rows, K, e_lo=-4, e_hi=4):
    """Rows whose blocks are 2**e times E2M1 values, each block holding a 4
    or a 6 in magnitude so that its exponent is e exactly."""
    codes = rng.integers(0, 16, size=(rows, K)).astype(np.uint8)
    codes[codes == 8] = 0
    nb = K // 32
    pos = rng.integers(0, 32, size=(rows, nb))
    big = rng.choice([6, 7, 14, 15], size=(rows, nb))  # +-4, +-6
    for r in range(rows):
        for b in range(nb):
            codes[r, 32 * b + pos[r, b]] = big[r, b]
    e = rng.integers(e_lo, e_hi + 1, size=(rows, nb)).astype(np.int32)
    return codes, e, MX.dequantize(codes, e)


def test_on_grid_round_trip_is_exact():
    rng = np.random.default_rng(11)
    codes, e, v = on_grid_rows(rng, 20, 256)
    q2, e2 = MX.quantize_rows(v.astype(np.float32))
    assert np.array_equal(q2, codes) and np.array_equal(e2, e)


def test_forward_exact_on_grid_without_smoothing_or_branch():
    """r = 0 and lambda = 1: the residual is W itself; with X and W on the
    MXFP4 grid (and exactly bf16), Y = X W^T + b exactly."""
    rng = np.random.default_rng(12)
    M, N, K = 24, 40, 128
    _, _, X = on_grid_rows(rng, M, K, -3, 2)
    _, _, W = on_grid_rows(rng, N, K, -6, -3)
    b = rng.integers(-8, 8, size=N) / 16.0
    Xb, Wb, bb = O.bf16_bits_of(X), O.bf16_bits_of(W), O.bf16_bits_of(b)
    prep = MX.prepare(Wb, None, bb, 0)
    f = MX.forward(prep, Xb)
    assert np.array_equal(f["Y"], X @ W.T + b[None, :])


def scalar_quantize_row(v):
    K = len(v)
    codes, exps = [], []
    for b in range(K // 32):
        blk = [float(np.float32(x)) for x in v[32 * b: 32 * b + 32]]
        a = max(abs(x) for x in blk)
        if a == 0:
            e = -127
        else:
            e = -200
            while 2.0 ** (e + 1) <= a:                   # e = floor(log2 a) by search
                e += 1
            e = min(max(e - 2, -127), 127)
        exps.append(e)
        codes.extend(brute_force_code(x / 2.0 ** e) for x in blk)
    return codes, exps


def test_scalar_implementation_agrees_on_small_layers():
    """An independent scalar implementation of the activation encoding and of
    Y = sum over blocks 2**(eA + eW) * sum(values) + D L2 + b."""
    c = synth.linear_case("mx_small", 77, 6, 10, 128, 3, x_outlier_n=2, x_outlier_scale=30.0)
    prep = MX.prepare(c.W, c.calib_absmax(), c.bias, 3)
    f = MX.forward(prep, c.X)
    Xh = O.smooth_activations(O.bf16_values(c.X), prep["iota"])
    D = O.bf16_values(c.X) @ prep["L1s"]
    for m in range(c.M):
        codes, exps = scalar_quantize_row(Xh[m])
        assert list(f["qA"][m]) == codes and list(f["eA"][m]) == exps
        for n in range(c.N):
            y = 0.0
            for b in range(c.K // 32):
                s = sum(e2m1_closed_form(codes[32 * b + i]) * e2m1_closed_form(int(prep["qW"][n, 32 * b + i]))
                        for i in range(32))
                y += 2.0 ** (exps[b] + int(prep["eW"][n, b])) * s
            y += float(D[m] @ prep["L2b"][:, n]) + prep["bias"][n]
            assert abs(y - f["Y"][m, n]) <= 1e-12 * max(1.0, abs(y))


def test_block_sums_are_exact_multiples_of_a_quarter():
    rng = np.random.default_rng(3)
    qa = rng.integers(0, 16, size=(5, 96)).astype(np.uint8)
    qw = rng.integers(0, 16, size=(7, 96)).astype(np.uint8)
    S = MX.block_sums(qa, qw)
    assert np.array_equal(S * 4, np.rint(S * 4)) and np.abs(S).max() <= 32 * 36
    for m, n, b in itertools.product(range(5), range(7), range(3)):
        want = sum(e2m1_closed_form(int(qa[m, 32 * b + i])) * e2m1_closed_form(int(qw[n, 32 * b + i]))
                   for i in range(32))
        assert S[m, n, b] == want


def test_quality_sanity_outliers_and_rank():
    """Not parity: on an outlier layer the MXFP4 layer tracks X W^T + b, and
    the low-rank branch lowers its error."""
    c = synth.linear_case("mx_q", 78, 64, 96, 256, 16, x_outlier_n=4, x_outlier_scale=40.0,
                          w_outlier_n=3, w_outlier_scale=8.0)
    X, W = O.bf16_values(c.X), O.bf16_values(c.W)
    exact = X @ W.T + O.bf16_values(c.bias)[None, :]
    errs = []
    for r in (0, 16):
        prep = MX.prepare(c.W, c.calib_absmax(), c.bias, r)
        errs.append(np.linalg.norm(MX.forward(prep, c.X)["Y"] - exact) / np.linalg.norm(exact))
    assert errs[1] < errs[0] < 0.25
