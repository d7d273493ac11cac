"""Pins for the CPU oracle: closed forms, hand-derived fixtures, library
routines, brute force on tiny inputs and exact special cases.  None of these
re-types the oracle's own formula and compares it with itself; each check is
chosen so that a plausible slip (dropped term, wrong sign or index,
transposed operand, wrong rounding) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle import svdquant as O
from oracle import awq as OA
from oracle import glue as OG
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def f32(x):
    return np.float32(x)


def nearest_f32_exact(fr: Fraction) -> np.float32:
    """Correctly rounded float32 of an exact rational, found by checking the
    float32 neighbours of a double approximation (independent of numpy's
    float32 arithmetic)."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        if best is None or d < best[0] or (d == best[0] and (cand.view(np.uint32) & 1) == 0):
            best = (d, cand)
    return np.float32(best[1])


# ======================================================== group quantiser (O5)
def test_quantizer_golden():
    for case in gold("quantize_group.json")["cases"]:
        v = np.array(case["v"], np.float32)
        q, s = O.quantize_groups(v[None, :])
        assert np.array_equal(q[0], np.array(case["q"], np.int8)), case["derivation"]
        assert s[0] == np.float32(case["s"]), case["derivation"]


def _bruteforce_codes(v: np.ndarray):
    """Scalar reference for one group: exact rational checks of s and 7/a,
    the product v*inv computed exactly in float64 then rounded once to float32,
    and the code chosen by exhaustive search over all 15 candidates
    (nearest, ties to the even candidate)."""
    a = max(abs(float(x)) for x in v)
    if a < 2.0 ** -100:
        return [0] * len(v), np.float32(0.0)
    s = nearest_f32_exact(Fraction(a) / 7)
    inv = nearest_f32_exact(Fraction(7) / Fraction(a))
    codes = []
    for x in v:
        t = np.float32(float(x) * float(inv))     # exact double product, one rounding
        best = None
        for c in range(-7, 8):
            d = abs(Fraction(float(t)) - c)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        codes.append(best[1])
    return codes, s


@pytest.mark.parametrize("seed", range(6))
def test_quantizer_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    groups = []
    for kind in range(8):
        v = rng.standard_normal(64).astype(np.float32) * np.float32(10.0 ** rng.uniform(-6, 4))
        if kind == 1:   # force ties: a = 7 makes inv = 1, so half-integers tie
            v = (rng.integers(-14, 15, 64) / 2.0).astype(np.float32)
            v[0] = 7.0
        if kind == 2:
            v[rng.integers(0, 64)] *= 50.0        # outlier inside the group
        groups.append(v)
    V = np.stack(groups)
    q, s = O.quantize_groups(V)
    for i, v in enumerate(groups):
        codes, sref = _bruteforce_codes(v)
        assert s[i] == sref
        assert list(q[i].astype(int)) == codes


def test_quantizer_absmax_maps_to_seven():
    rng = np.random.default_rng(7)
    a = np.float32(10.0) ** rng.uniform(-20, 20, 200000).astype(np.float32)
    inv = (np.float32(7.0) / a.astype(np.float32)).astype(np.float32)
    t = (a.astype(np.float32) * inv).astype(np.float32)
    assert np.all(np.rint(t) == 7.0)
    V = np.zeros((1000, 64), np.float32)
    V[:, 0] = a[:1000]
    V[:, 1] = -a[1000:2000] * np.float32(0.999)
    q, s = O.quantize_groups(V)
    assert np.all(np.abs(q).max(axis=1) == 7)


def test_quantizer_error_bound_and_range():
    rng = np.random.default_rng(11)
    V = (rng.standard_normal((5000, 64)) * 10.0 ** rng.uniform(-3, 3, (5000, 1))).astype(np.float32)
    q, s = O.quantize_groups(V)
    assert q.min() >= -7 and q.max() <= 7
    err = np.abs(V.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] * 0.5 * (1 + 2.0 ** -20))


def test_quantizer_on_grid_reproduces_codes_and_scale():
    rng = np.random.default_rng(12)
    for e in range(-30, 30, 3):
        c = rng.integers(-7, 8, 64)
        c[rng.integers(0, 64)] = 7 * (1 if rng.integers(0, 2) else -1)
        v = (c * 2.0 ** e).astype(np.float32)
        q, s = O.quantize_groups(v[None])
        assert np.array_equal(q[0], c.astype(np.int8))
        assert s[0] == np.float32(2.0 ** e)


def test_pack_canonical_nibble_order():
    # codes 1, -1, 7, -7: low nibble holds the even position, two's complement
    q = np.array([[1, -1, 7, -7]], np.int8)
    assert list(O.pack_int4(q)[0]) == [0xF1, 0x97]
    rng = np.random.default_rng(3)
    q = rng.integers(-8, 8, (5, 128)).astype(np.int8)
    assert np.array_equal(O.unpack_int4(O.pack_int4(q)), q)


# ============================================================ smoothing (O1)
def test_smoothing_golden():
    g = gold("smoothing.json")
    ax = np.array(g["ax"], np.float32)
    aw = np.array(g["aw"], np.float32)
    W = np.zeros((3, len(aw)))
    W[1] = aw
    W[2] = -aw * 0.5
    lam, iota = O.smoothing_factors(ax, W)
    for j in range(len(ax)):
        if g["lam"][j] is not None:
            assert lam[j] == np.float32(g["lam"][j])
        if g["iota"][j] is not None:
            assert iota[j] == np.float32(g["iota"][j])
        # every entry: exact-rational check of the float32 chain
        a = max(float(ax[j]), float(np.float32(1e-5)))
        w = max(float(aw[j]), float(np.float32(1e-5)))
        ratio = nearest_f32_exact(Fraction(a) / Fraction(w))
        # correctly rounded float32 sqrt: double sqrt of a float32 then one
        # rounding to float32 is correctly rounded (53 >= 2*24 + 2)
        lref = np.float32(math.sqrt(float(ratio)))
        assert lam[j] == lref
        assert iota[j] == nearest_f32_exact(Fraction(1) / Fraction(float(lref)))


def test_smoothing_random_against_exact_rationals():
    rng = np.random.default_rng(5)
    K = 256
    ax = (np.abs(rng.standard_normal(K)) * 10.0 ** rng.uniform(-7, 3, K)).astype(np.float32)
    W = (rng.standard_normal((32, K)) * 0.02).astype(np.float32).astype(np.float64)
    lam, iota = O.smoothing_factors(ax, W)
    aw = np.abs(W).max(axis=0)
    for j in range(K):
        a = max(float(ax[j]), float(np.float32(1e-5)))
        w = max(float(np.float32(aw[j])), float(np.float32(1e-5)))
        ratio = nearest_f32_exact(Fraction(a) / Fraction(w))
        assert lam[j] == np.float32(math.sqrt(float(ratio)))
        assert iota[j] == nearest_f32_exact(Fraction(1) / Fraction(float(lam[j])))


def test_smoothing_none_is_identity():
    lam, iota = O.smoothing_factors(None, np.ones((4, 128)))
    assert np.all(lam == 1) and np.all(iota == 1)


def test_smoothing_preserves_the_product():
    c = synth.tiny_case()
    X = O.bf16_values(c.X)
    W = O.bf16_values(c.W)
    lam, iota = O.smoothing_factors(c.calib_absmax(), W)
    Xh = X * iota.astype(np.float64)
    Wh = O.smooth_weight(W, lam)
    ref = X @ W.T
    got = Xh @ Wh.T
    # iota*lam = 1 up to one float32 rounding of 1/lambda
    assert np.max(np.abs(got - ref)) <= 2.0 ** -22 * np.max(np.abs(X) @ np.abs(W).T)
    # the outlier channels are the ones pulled down most
    assert np.median(iota[c.x_outliers]) < np.median(np.delete(iota, c.x_outliers))


# ====================================================== bf16 rounding (O3)
def test_round_to_bf16_golden():
    g = gold("bf16_rounding.json")
    got = O.round_to_bf16(np.array(g["x"]))
    assert np.array_equal(got, np.array(g["y"])), g["derivation"]


def test_round_to_bf16_matches_bit_rounding_on_float32_inputs():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(200000) * 10.0 ** rng.uniform(-30, 30, 200000)).astype(np.float32)
    ref = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(O.round_to_bf16(x.astype(np.float64)), ref)


# ===================================================== low-rank split (O3/O4)
def _small_weight(seed=0, N=96, K=128):
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K)) * 0.02
    W[:, rng.choice(K, 4, replace=False)] *= 8.0
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(W.astype(np.float32))).astype(np.float64)


def test_singular_values_match_a_second_lapack_driver():
    W = _small_weight(1)
    lam = np.float32(1.0) + np.abs(np.random.default_rng(2).standard_normal(128)).astype(np.float32)
    Wh = O.smooth_weight(W, lam)
    _, _, s = O.lowrank_split(Wh, 8, np.ones(128, np.float32))
    ref = scipy.linalg.svd(Wh, compute_uv=False, lapack_driver="gesvd")
    assert np.allclose(s, ref, rtol=1e-10, atol=0)


@pytest.mark.parametrize("rank", [1, 5, 17])
def test_eckart_young_and_factor_structure(rank):
    W = _small_weight(3)
    lam = (np.float32(0.5) + np.random.default_rng(4).random(128).astype(np.float32))
    iota = (np.float32(1.0) / lam).astype(np.float32)
    Wh = O.smooth_weight(W, lam)
    L1s, L2, s = O.lowrank_split(Wh, rank, iota, round_factors=False)
    L1 = L1s * lam.astype(np.float64)[:, None] / (iota.astype(np.float64) * lam)[:, None]
    # L1 = V S^1/2 and L2 = S^1/2 U^T: Gram matrices are diag(S_r)
    assert np.allclose(L1.T @ L1, np.diag(s[:rank]), atol=1e-12 * s[0])
    assert np.allclose(L2 @ L2.T, np.diag(s[:rank]), atol=1e-12 * s[0])
    approx = (L1 @ L2).T
    resid = np.sum((Wh - approx) ** 2)
    assert abs(resid - np.sum(s[rank:] ** 2)) <= 1e-9 * np.sum(s ** 2)
    # the branch takes the top singular directions: residual norm equals
    # the (r+1)-th singular value
    assert np.isclose(np.linalg.norm(Wh - approx, 2), s[rank], rtol=1e-9)


def test_full_rank_leaves_zero_residual():
    W = _small_weight(5, N=64, K=128)
    lam = (np.float32(0.5) + np.random.default_rng(6).random(128).astype(np.float32))
    iota = (np.float32(1.0) / lam).astype(np.float32)
    Wh = O.smooth_weight(W, lam)
    # exact (float64) factors at r = min(N, K): nothing left for the 4-bit path
    L1s, L2, _ = O.lowrank_split(Wh, 64, iota, round_factors=False)
    lam_eff = 1.0 / iota.astype(np.float64)     # undo the fold exactly
    R = Wh - ((L1s * lam_eff[:, None]) @ L2).T
    assert np.max(np.abs(R)) <= 1e-12 * np.max(np.abs(Wh))
    # with the bf16 factors the residual is what the rounding left behind:
    # no larger than the factor rounding, and it reconstructs W_hat
    L1s, L2b, _ = O.lowrank_split(Wh, 64, iota)
    R32 = O.residual(Wh, lam, L1s, L2b)
    branch = ((L1s * lam.astype(np.float64)[:, None]) @ L2b).T
    assert np.max(np.abs(R32 + branch - Wh)) <= 2.0 ** -24 * np.max(np.abs(R32)) * 1.01
    assert np.max(np.abs(R32)) <= 2.0 ** -6 * np.max(np.abs(Wh))


def test_residual_shrinks_with_rank():
    c = synth.tiny_case()
    norms = []
    for r in (0, 4, 16, 64):
        p = O.prepare(c.W, c.calib_absmax(), c.bias, r)
        norms.append(np.linalg.norm(p["R32"].astype(np.float64)))
    assert all(a > b for a, b in zip(norms, norms[1:]))


# ================================================ activations, D, P (O7-O9)
def test_activation_smoothing_multiply_is_one_rounding():
    rng = np.random.default_rng(8)
    X = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(rng.standard_normal((16, 128)).astype(np.float32)))
    iota = (np.float32(1.0) / (np.float32(0.3) + rng.random(128).astype(np.float32))).astype(np.float32)
    xh = O.smooth_activations(X, iota)
    exact = X.astype(np.float64) * iota.astype(np.float64)   # 8x24 bits: exact in float64
    assert np.array_equal(xh, exact.astype(np.float32))


def test_lowrank_down_and_group_sums_bruteforce():
    rng = np.random.default_rng(10)
    M, N, K, r = 3, 4, 128, 3
    X = rng.standard_normal((M, K))
    L1s = rng.standard_normal((K, r))
    D = O.lowrank_down(X, L1s)
    for m in range(M):
        for t in range(r):
            assert math.isclose(D[m, t], math.fsum(X[m, k] * L1s[k, t] for k in range(K)), rel_tol=1e-13, abs_tol=1e-13)
    qA = rng.integers(-7, 8, (M, K)).astype(np.int8)
    qW = rng.integers(-7, 8, (N, K)).astype(np.int8)
    P = O.group_sums(qA, qW)
    for m in range(M):
        for n in range(N):
            for g in range(K // 64):
                assert P[m, n, g] == sum(int(qA[m, k]) * int(qW[n, k]) for k in range(64 * g, 64 * g + 64))
    # extreme group sum
    assert O.group_sums(np.full((1, 64), 7, np.int8), np.full((1, 64), -7, np.int8))[0, 0, 0] == -3136


# ============================================================ output (O10)
def test_output_two_routes_agree():
    c = synth.linear_case("t", 21, 24, 40, 256, 6, x_outlier_n=3, x_outlier_scale=30.0)
    p = O.prepare(c.W, c.calib_absmax(), c.bias, c.rank)
    f = O.forward(p, c.X)
    P = O.group_sums(f["qA"], p["qW"])
    Y2 = O.linear_output_from_sums(P, f["sA"], p["sW"], f["D"], p["L2b"], p["bias"])
    assert np.allclose(f["Y"], Y2, rtol=0, atol=1e-12 * np.max(np.abs(Y2)))


def test_output_bruteforce_scalar_loops():
    """Tiny layer evaluated from the definitions with Python scalars only."""
    c = synth.linear_case("b", 22, 3, 5, 128, 2, x_outlier_n=2, x_outlier_scale=20.0)
    p = O.prepare(c.W, c.calib_absmax(), c.bias, c.rank)
    f = O.forward(p, c.X)
    X = synth.bf16_bits_to_f32(c.X)
    for m in range(c.M):
        # activation codes by the scalar brute-force quantiser
        xh = [np.float32(float(X[m, k]) * float(p["iota"][k])) for k in range(c.K)]
        for g in range(c.K // 64):
            codes, s = _bruteforce_codes(np.array(xh[64 * g: 64 * g + 64], np.float32))
            assert list(f["qA"][m, 64 * g: 64 * g + 64].astype(int)) == codes
            assert f["sA"][m, g] == s
        for n in range(c.N):
            acc = Fraction(0)
            for g in range(c.K // 64):
                Pg = sum(int(f["qA"][m, k]) * int(p["qW"][n, k]) for k in range(64 * g, 64 * g + 64))
                acc += Fraction(float(f["sA"][m, g])) * Fraction(float(p["sW"][n, g])) * Pg
            for t in range(c.rank):
                d = math.fsum(float(X[m, k]) * p["L1s"][k, t] for k in range(c.K))
                acc += Fraction(d) * Fraction(p["L2b"][t, n])
            acc += Fraction(p["bias"][n])
            assert math.isclose(f["Y"][m, n], float(acc), rel_tol=1e-12, abs_tol=1e-12)


@pytest.mark.parametrize("seed", [31, 32, 33])
def test_on_grid_inputs_give_the_exact_matmul(seed):
    """r = 0, no smoothing, inputs already on the INT4 grid: the 4-bit path
    is lossless, so Y must equal X W^T exactly."""
    c = synth.on_grid_case(seed, 16, 24, 256, exp_lo=-3, exp_hi=3)
    p = O.prepare(c.W, None, c.bias, 0)
    f = O.forward(p, c.X)
    X = synth.bf16_bits_to_f32(c.X).astype(np.float64)
    W = synth.bf16_bits_to_f32(c.W).astype(np.float64)
    assert np.array_equal(f["Y"], X @ W.T)


def test_rank0_no_smoothing_is_per_group_fake_quant():
    """With r = 0 and lambda = 1 the layer reduces to textbook per-group W4A4
    fake quantisation; compare with torch's per-channel fake-quantiser applied
    to each group with the oracle's scales (torch divides by the scale instead
    of multiplying by 7/a, so a tiny fraction of codes may differ by one)."""
    import torch
    c = synth.linear_case("fq", 23, 64, 48, 256, 0, x_outlier_n=4, x_outlier_scale=25.0)
    p = O.prepare(c.W, None, c.bias, 0)
    f = O.forward(p, c.X)

    def fake(vals, scales):
        rows, K = vals.shape
        t = torch.from_numpy(vals.reshape(-1, 64).astype(np.float32))
        sc = torch.from_numpy(scales.reshape(-1).astype(np.float32))
        sc = torch.where(sc > 0, sc, torch.ones_like(sc))
        out = torch.fake_quantize_per_channel_affine(t, sc, torch.zeros_like(sc, dtype=torch.int32), 0, -7, 7)
        return out.double().numpy().reshape(rows, K)

    X = synth.bf16_bits_to_f32(c.X)
    W = synth.bf16_bits_to_f32(c.W)
    Xq = fake(X, f["sA"])
    Wq = fake(W, p["sW"])
    # torch returns code*scale rounded to float32
    f32d = lambda q, s: O.dequantize(q, s).astype(np.float32).astype(np.float64)
    assert np.mean(Xq != f32d(f["qA"], f["sA"])) < 1e-3
    assert np.mean(Wq != f32d(p["qW"], p["sW"])) < 1e-3
    Yfq = Xq @ Wq.T + p["bias"][None, :]
    assert np.max(np.abs(Yfq - f["Y"])) <= 0.02 * np.max(np.abs(f["Y"]))


def test_low_rank_branch_beats_plain_w4a4_on_outliers():
    """Quality sanity (not parity): the smoothed + low-rank layer is closer
    to the exact product than plain W4A4, and error falls with rank."""
    c = synth.tiny_case()
    X = synth.bf16_bits_to_f32(c.X).astype(np.float64)
    W = synth.bf16_bits_to_f32(c.W).astype(np.float64)
    exact = X @ W.T + O.bf16_values(c.bias)[None, :]
    plain = O.forward(O.prepare(c.W, None, c.bias, 0), c.X)["Y"]
    errs = [np.linalg.norm(O.forward(O.prepare(c.W, c.calib_absmax(), c.bias, r), c.X)["Y"] - exact)
            for r in (0, 16, 64)]
    assert errs[0] < np.linalg.norm(plain - exact)
    assert errs[0] > errs[1] > errs[2]


# ================================================================ AWQ (O11)
def test_awq_golden():
    g = gold("awq_group.json")
    w = np.array(g["w"], np.float16)[None, :]
    q, s, z = OA.quantize(w)
    assert list(q[0].astype(int)) == g["q"], g["derivation"]
    assert float(s[0, 0]) == g["s"] and float(z[0, 0]) == g["z"]


def test_awq_on_grid_is_lossless():
    rng = np.random.default_rng(40)
    N, K = 8, 256
    s = np.exp2(rng.integers(-8, -3, (N, K // 64))).astype(np.float64)
    z = rng.integers(1, 15, (N, K // 64)).astype(np.float64)
    c = rng.integers(0, 16, (N, K // 64, 64)).astype(np.float64)
    c[:, :, 0] = 0
    c[:, :, 1] = 15
    W = ((c - z[:, :, None]) * s[:, :, None]).reshape(N, K)
    q, s16, z16 = OA.quantize(W.astype(np.float16))
    assert np.array_equal(OA.dequantize(q, s16, z16), W)


def test_awq_error_bound_and_m1_is_dgemv():
    a = synth.awq_case(m_max=4, N=64, K=512, seed=41)
    q, s, z = OA.quantize(a.W)
    Wd = OA.dequantize(q, s, z)
    W = a.W.astype(np.float64)
    sg = np.repeat(s.astype(np.float64), 64, axis=1)
    assert np.all(np.abs(W - Wd) <= sg * 0.5 * (1 + 1e-3) + 1e-12)
    x = a.x[:1].astype(np.float64)
    y = OA.forward(a.x[:1], q, s, z)
    assert np.allclose(y, x @ Wd.T, rtol=0, atol=1e-12 * np.max(np.abs(y)))


def test_awq_bruteforce_tiny():
    a = synth.awq_case(m_max=2, N=3, K=128, seed=42)
    q, s, z = OA.quantize(a.W)
    bias = np.array([0.5, -0.25, 0.0])
    y = OA.forward(a.x, q, s, z, bias)
    for m in range(2):
        for n in range(3):
            acc = Fraction(0)
            for k in range(128):
                g = k // 64
                acc += Fraction(float(a.x[m, k])) * (int(q[n, k]) - Fraction(float(z[n, g]))) * Fraction(float(s[n, g]))
            acc += Fraction(bias[n])
            assert math.isclose(y[m, n], float(acc), rel_tol=1e-12, abs_tol=1e-14)
    assert np.array_equal(OA.unpack(OA.pack(q)), q)
    assert list(OA.pack(np.array([[1, 15, 0, 9]], np.uint8))[0]) == [0xF1, 0x90]


# ================================================================ GELU (a7)
def test_gelu_identities_and_library():
    import torch
    y = np.concatenate([np.linspace(-12, 12, 20001), [0.0]])
    g = OG.gelu_tanh(y)
    # odd-part identity of the tanh form: gelu(y) - gelu(-y) = y
    assert np.allclose(g - OG.gelu_tanh(-y), y, rtol=0, atol=1e-14)
    assert OG.gelu_tanh(np.array([0.0]))[0] == 0.0
    ref = torch.nn.functional.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    assert np.allclose(g, ref, rtol=1e-14, atol=1e-15)
    # far negative tail: the printed form cancels, the logistic form keeps
    # relative accuracy; check against a 50-digit evaluation
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    for yv in (-6.0, -8.5, -10.0):
        yd = Decimal(yv)
        u = Decimal(2).sqrt() / Decimal(math.pi).sqrt() * (yd + Decimal("0.044715") * yd ** 3)
        exact = float(yd / (1 + (-2 * u).exp()))
        assert math.isclose(OG.gelu_tanh(np.array([yv]))[0], exact, rel_tol=1e-12)
    erf_form = 0.5 * y * (1.0 + scipy.special.erf(y / math.sqrt(2.0)))
    assert np.max(np.abs(g - erf_form)) < 1e-3
    gb = OG.gelu_tanh_bf16(y)
    assert np.array_equal(gb, O.round_to_bf16(g))
    assert np.all(np.abs(gb - g) <= np.abs(g) * 2.0 ** -8 + 1e-40)
