"""CPU tests of libsvdq's host half: the library loads without a GPU and
exports every symbol the header declares; offline preparation agrees with
the oracle bit for bit where the method fixes every rounding (smoothing
factors, residual codes and scales at rank 0, AWQ codes), and satisfies the
SVD invariants where several results are correct (rank > 0); the device
packer places codes where the documented layout says; every status code
that can be forced from the host is returned.  No compute reaches a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest
import scipy.linalg

import synth
from oracle import svdquant as O
from oracle import awq as OA

import w4a4_rank_corrected_smooth_amd as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ------------------------------------------------------------------ exports
def _header_functions():
    text = open(os.path.join(ROOT, "include", "svdq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:svdq|awq)_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert len(names) >= 18
    lib = ctypes.CDLL(S.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(S.EXPORTS) == names
    assert S.abi_version() == 1


def test_status_strings():
    lib = S._lib
    for code in range(8):
        assert lib.svdq_status_string(code)
    assert b"unknown" in lib.svdq_status_string(99)


# ----------------------------------------------------- prepare vs the oracle
def test_smoothing_and_rank0_codes_bit_exact():
    c = synth.tiny_case()
    ax = c.calib_absmax()
    hw = S.prepare_weights(c.W, ax, c.bias, 0)
    ref = O.prepare(c.W, ax, c.bias, 0)
    assert np.array_equal(hw.inv_lambda, ref["iota"])
    assert np.array_equal(hw.qweight, O.pack_int4(ref["qW"]))
    assert np.array_equal(hw.wscales, ref["sW"])
    assert np.array_equal(hw.bias, ref["bias"].astype(np.float32))


def test_calibration_absmax_matches():
    c = synth.tiny_case()
    assert np.array_equal(S.calibration_absmax(c.X[:64]), O.calibration_absmax(O.bf16_values(c.X[:64])))


@pytest.mark.parametrize("seed,N,K", [(50, 192, 256), (51, 320, 128), (52, 128, 512)])
def test_rank0_no_smoothing_bit_exact(seed, N, K):
    c = synth.linear_case("r0", seed, 8, N, K, 0, w_outlier_n=5, w_outlier_scale=8.0)
    hw = S.prepare_weights(c.W, None, None, 0)
    ref = O.prepare(c.W, None, None, 0)
    assert np.array_equal(hw.qweight, O.pack_int4(ref["qW"]))
    assert np.array_equal(hw.wscales, ref["sW"])
    assert np.all(hw.inv_lambda == 1.0) and np.all(hw.bias == 0.0)


def _cpp_branch(hw, lam):
    L1s = O.bf16_values(hw.l1s)
    L2 = O.bf16_values(hw.l2)
    return ((L1s * lam.astype(np.float64)[:, None]) @ L2).T


@pytest.mark.parametrize("rank", [1, 8, 16, 40])
def test_lowrank_split_invariants(rank):
    c = synth.linear_case("svd", 60 + rank, 64, 160, 256, rank, x_outlier_n=6, x_outlier_scale=40.0,
                          w_outlier_n=4, w_outlier_scale=8.0)
    ax = c.calib_absmax()
    hw = S.prepare_weights(c.W, ax, c.bias, rank)
    ref = O.prepare(c.W, ax, c.bias, rank)
    lam, _ = O.smoothing_factors(ax, O.bf16_values(c.W))
    W_hat = O.smooth_weight(O.bf16_values(c.W), lam)
    sig = scipy.linalg.svd(W_hat, compute_uv=False)
    A = _cpp_branch(hw, lam)
    # (1) the branch is the top-r part: residual energy matches Eckart-Young
    #     up to the bf16 rounding of the factors
    e_cpp = np.sum((W_hat - A) ** 2)
    e_opt = np.sum(sig[rank:] ** 2)
    assert e_opt <= e_cpp <= e_opt + 4 * 2.0 ** -8 * np.sqrt(e_opt) * sig[:rank].sum() + 1e-12
    # (2) same branch as the oracle's (its own SVD, own signs) up to bf16 rounding
    Aref = ((ref["L1s"] * lam.astype(np.float64)[:, None]) @ ref["L2b"]).T
    assert np.linalg.norm(A - Aref) <= 2.0 ** -6 * np.linalg.norm(Aref)
    # (3) factor structure: columns of L1 (iota folded back out) and rows of
    #     L2 carry sigma_t: ||L1_t|| * ||L2_t|| ~ sigma_t
    L1 = O.bf16_values(hw.l1s) * lam.astype(np.float64)[:, None]
    L2 = O.bf16_values(hw.l2)
    prod = np.linalg.norm(L1, axis=0) * np.linalg.norm(L2, axis=1)
    assert np.allclose(prod, sig[:rank], rtol=2.0 ** -6)
    # (4) residual codes reconstruct W_hat within half a quantisation step
    deq = O.dequantize(O.unpack_int4(hw.qweight), hw.wscales)
    step = np.repeat(hw.wscales.astype(np.float64), 64, axis=1)
    err = np.abs(W_hat - A - deq)
    assert np.all(err <= 0.5 * step * (1 + 2.0 ** -20) + 2.0 ** -24 * np.abs(W_hat - A) + 1e-30)


def test_full_rank_leaves_only_factor_rounding():
    c = synth.linear_case("fr", 70, 8, 64, 128, 64)
    hw = S.prepare_weights(c.W, None, None, 64)
    W = O.bf16_values(c.W)
    A = _cpp_branch(hw, np.ones(128, np.float32))
    # an exact SVD at r = min(N, K) leaves nothing but the factors' bf16 rounding
    assert np.max(np.abs(W - A)) <= 2.0 ** -6 * np.max(np.abs(W))
    assert np.max(hw.wscales) <= 2.0 ** -6 * np.max(np.abs(W)) / 7 * 8


def test_prepare_is_deterministic():
    c = synth.linear_case("det", 71, 8, 256, 192, 12, x_outlier_n=3, x_outlier_scale=30.0)
    ax = c.calib_absmax()
    a = S.prepare_weights(c.W, ax, c.bias, 12)
    b = S.prepare_weights(c.W, ax, c.bias, 12)
    for f in ("inv_lambda", "l1s", "l2", "qweight", "wscales", "bias"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


def test_singular_values_of_a_tall_and_a_wide_matrix():
    """Both Gram sides (N > K and N < K) give the top singular directions."""
    for N, K in ((320, 128), (96, 384)):
        c = synth.linear_case("tw", 72 + N, 8, N, K, 10, w_outlier_n=3, w_outlier_scale=8.0)
        hw = S.prepare_weights(c.W, None, None, 10)
        W = O.bf16_values(c.W)
        sig = scipy.linalg.svd(W, compute_uv=False)
        A = _cpp_branch(hw, np.ones(K, np.float32))
        assert abs(np.linalg.norm(W - A) ** 2 - np.sum(sig[10:] ** 2)) <= \
            4 * 2.0 ** -8 * np.linalg.norm(W) * sig[:10].sum()


# ------------------------------------------------------------- device packer
E2M3_INT = {0: 0, 8: 1, 16: 2, 20: 3, 24: 4, 26: 5, 28: 6, 30: 7}


def _e2m3_to_int(v):
    return -E2M3_INT[v & 31] if v & 32 else E2M3_INT[v & 31]


def test_device_blob_layout():
    """Weight codes sit where the documented tiling says, as FP6 E2M3 fields:
    block (g, tile) of 1536 bytes; lane = row % 32 + 32 * half; code c at
    bits 6c of the lane's 192-bit string, stored as three 8-byte pairs at
    512 j + 8 lane."""
    c = synth.linear_case("pk", 80, 8, 100, 192, 5, x_outlier_n=2, x_outlier_scale=20.0)
    hw = S.prepare_weights(c.W, c.calib_absmax(), c.bias, 5)
    blob = S.pack_device_weights(hw)
    N, K, G = 100, 192, 3
    Np = 256
    T = Np // 32
    codes = O.unpack_int4(hw.qweight)
    qbytes = Np * K * 3 // 4
    qdev = blob[:qbytes]
    for n in range(0, N, 7):
        for k in range(K):
            g, kk = divmod(k, 64)
            h = (kk % 16) // 8
            cidx = 8 * (kk // 16) + kk % 8
            lane = n % 32 + 32 * h
            base = (g * T + n // 32) * 1536 + lane * 8
            words = b"".join(bytes(qdev[base + 512 * j: base + 512 * j + 8]) for j in range(3))
            bits = int.from_bytes(words, "little")
            assert _e2m3_to_int((bits >> (6 * cidx)) & 63) == codes[n, k]
    # padded rows hold zero codes
    assert not np.any(qdev.reshape(G, T, 1536)[:, 4:, :])
    # scales as the GEMM's column operands: bf16 slots b1 b2 b3 b1 b2 b3 b1 b2
    # with s = b1 + b2 + b3 exactly, b1 and b2 the top bits of s and of the
    # remainder, [G][Np] x 16 bytes
    s_off = (qbytes + 255) // 256 * 256
    ops = blob[s_off: s_off + G * Np * 16].view(np.uint16).reshape(G, Np, 8)
    assert np.array_equal(ops[:, :, 3:6], ops[:, :, 0:3]) and np.array_equal(ops[:, :, 6:8], ops[:, :, 0:2])
    piece = (ops[:, :, :3].astype(np.uint32) << 16).view(np.float32)
    s = (piece[:, :, 0] + piece[:, :, 1]) + piece[:, :, 2]
    assert np.array_equal(s[:, :N].T, hw.wscales) and not np.any(ops[:, N:])
    hi = hw.wscales.T.view(np.uint32) >> 16
    assert np.array_equal(ops[:, :N, 0], hi.astype(np.uint16))


def test_fp6_block_decoder_reads_the_packed_weights():
    """The tests' reader of the fp6 code blocks (used on device workspaces)
    recovers the canonical codes from the library's weight blob, which uses
    the same block layout: pins the reader independently of any kernel."""
    from tests.gpu_util import decode_fp6_codes
    c = synth.linear_case("dec", 95, 8, 300, 320, 0, w_outlier_n=3, w_outlier_scale=8.0)
    hw = S.prepare_weights(c.W, None, c.bias, 0)
    blob = S.pack_device_weights(hw)
    assert np.array_equal(decode_fp6_codes(blob, c.N, c.K), O.unpack_int4(hw.qweight))


def test_awq_quantizer_bit_exact_and_packer():
    a = synth.awq_case(m_max=1, N=96, K=256, seed=81)
    q, s, z = S.awq_quantize_weights(a.W)
    rq, rs, rz = OA.quantize(a.W)
    assert np.array_equal(q, OA.pack(rq))
    assert np.array_equal(s.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(z.view(np.uint16), rz.view(np.uint16))


def test_awq_blob_layout():
    """AWQ codes and scale words sit where the documented layout says: tiles
    of 16 output channels; per (tile, pair of groups) a 1024-byte block where
    lane = column + 16 * quarter holds 16 bytes (first group of the pair, then
    the second); in each 32-bit word the even channels fill the low half,
    nibble j = channel 2 j, the odd ones the high half.  Scale words
    (s | z << 16) follow as [Np][G rounded up to 4].  Padding is zero."""
    rng = np.random.default_rng(7)
    N, K = 40, 320                       # 3 tiles (last one ragged), G = 5: odd
    G, T, P, G4 = 5, 3, 3, 8
    q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.integers(0x3000, 0x4000, size=(N, G), dtype=np.uint16)
    # zero points are integers 0..15 held in fp16 (the packer refuses others)
    z = rng.integers(0, 16, size=(N, G)).astype(np.float16).view(np.uint16)
    n_bytes = S._lib.awq_device_weights_bytes(N, K)
    qbytes = T * P * 1024
    s_off = (qbytes + 255) // 256 * 256
    assert n_bytes == (s_off + T * 16 * G4 * 4 + 255) // 256 * 256
    blob = np.empty(n_bytes, np.uint8)
    assert S._lib.awq_pack_device_weights(q.ctypes.data, s.ctypes.data, z.ctypes.data, N, K,
                                          blob.ctypes.data, n_bytes) == 0
    codes = np.empty((N, K), np.int64)
    codes[:, 0::2] = q & 15
    codes[:, 1::2] = q >> 4
    qdev = blob[:qbytes]
    seen = np.zeros(qbytes, bool)
    for n in range(N):
        for k in range(K):
            g, kk = divmod(k, 64)
            lane = n % 16 + 16 * (kk // 16)
            word_at = ((n // 16) * P + g // 2) * 1024 + lane * 16 + 8 * (g % 2) + 4 * ((kk % 16) // 8)
            word = int.from_bytes(bytes(qdev[word_at: word_at + 4]), "little")
            c = kk % 8
            shift = 4 * (c // 2) + (16 if c % 2 else 0)
            assert (word >> shift) & 15 == codes[n, k], (n, k)
            seen[word_at: word_at + 4] = True
    assert not np.any(qdev[~seen])       # padded columns, the missing sixth group
    sz = blob[s_off: s_off + T * 16 * G4 * 4].view(np.uint32).reshape(T * 16, G4)
    assert np.array_equal(sz[:N, :G], s.astype(np.uint32) | (z.astype(np.uint32) << 16))
    assert not np.any(sz[N:]) and not np.any(sz[:, G:])


def test_awq_packer_refuses_bad_zero_points_and_scales():
    """The kernel forms q - z exactly as (1024 + q) - (1024 + z) in fp16,
    which holds for integer zero points 0..15 only: the packer refuses any
    other zero point, and non-finite scales, before writing anything."""
    N, K = 16, 128
    q = np.zeros((N, K // 2), np.uint8)
    s = np.full((N, K // 64), 0.01, np.float16).view(np.uint16)
    n_bytes = S._lib.awq_device_weights_bytes(N, K)
    blob = np.full(n_bytes, 0xAB, np.uint8)

    def pack(zv, sv=None):
        z = np.full((N, K // 64), 3.0, np.float16)
        z[5, 1] = zv
        ss = s.copy()
        if sv is not None:
            ss.view(np.float16)[2, 0] = sv
        return S._lib.awq_pack_device_weights(q.ctypes.data, ss.ctypes.data,
                                              z.view(np.uint16).ctypes.data, N, K,
                                              blob.ctypes.data, n_bytes)
    for bad in (2.5, -1.0, 16.0, np.inf, np.nan, 15.5):
        assert pack(bad) == INV, bad
        assert "zero point" in S._lib.svdq_last_error().decode()
    assert pack(3.0, np.inf) == 6 and pack(3.0, np.nan) == 6
    assert np.all(blob == 0xAB)                  # nothing written on refusal
    assert pack(0.0) == 0 and pack(15.0) == 0


def test_static_forward_validation():
    """svdq_linear_forward_static validates like the forward and refuses
    shapes whose workspace exceeds the static scratch array, all before any
    HIP call."""
    lib = S._lib
    w = _dw()
    call = lambda **kw: lib.svdq_linear_forward_static(
        ctypes.byref(kw.get("w", w)), kw.get("X", FAKE), kw.get("M", 64), kw.get("Y", FAKE),
        kw.get("dt", S.BF16), kw.get("epi", 0), None)
    assert call(X=None) == INV
    assert call(X=FAKE + 4) == INV
    assert call(Y=None) == INV
    assert call(M=0) == SHAPE
    assert call(dt=S.FP16) == INV
    assert call(epi=3) == INV
    assert call(w=_dw(K=100)) == SHAPE
    big = _dw(N=256, K=16384, rank=32)
    # M = 6144, K = 16384: the fp6 codes alone are 72 MiB
    assert call(w=big, M=6144) == WS
    assert "limit" in lib.svdq_last_error().decode()


def test_wrappers_check_outputs_and_bias():
    """The Python wrappers refuse caller outputs of the wrong shape, dtype or
    layout (the kernels write exactly M x N elements of the output type) and
    AWQ biases that are not fp16 of N elements, before calling the library."""
    import torch
    dev = torch.device("cpu")
    good = torch.empty((4, 8), dtype=torch.bfloat16)
    S._check_out(good, 4, 8, dev)
    S._check_out(torch.empty((4, 8), dtype=torch.float32), 4, 8, dev)
    with pytest.raises(ValueError):
        S._check_out(torch.empty((4, 7), dtype=torch.bfloat16), 4, 8, dev)
    with pytest.raises(ValueError):
        S._check_out(torch.empty((4, 8), dtype=torch.float16), 4, 8, dev)
    with pytest.raises(ValueError):
        S._check_out(torch.empty((8, 4), dtype=torch.bfloat16).t(), 4, 8, dev)
    with pytest.raises(ValueError):
        S._check_out(torch.empty((4, 8), dtype=torch.float32), 4, 8, dev, dtypes=(torch.float16,))
    S._check_bias(torch.zeros(8, dtype=torch.float16), 8, dev)
    with pytest.raises(ValueError):
        S._check_bias(torch.zeros(8, dtype=torch.float32), 8, dev)
    with pytest.raises(ValueError):
        S._check_bias(torch.zeros(7, dtype=torch.float16), 8, dev)


# ----------------------------------------------------------- MXFP4 form
from oracle import mxfp4 as MXO  # noqa: E402


@pytest.mark.parametrize("smooth", [False, True])
def test_mx_rank0_codes_and_scales_bit_exact(smooth):
    c = synth.linear_case("mxr0", 90, 64, 96, 320, 0, x_outlier_n=3, x_outlier_scale=40.0,
                          w_outlier_n=4, w_outlier_scale=8.0)
    ax = c.calib_absmax() if smooth else None
    hw = S.mx_prepare_weights(c.W, ax, c.bias, 0)
    ref = MXO.prepare(c.W, ax, c.bias, 0)
    assert np.array_equal(hw.inv_lambda, ref["iota"])
    assert np.array_equal(hw.qweight, MXO.pack_fp4(ref["qW"]))
    assert np.array_equal(hw.wscales.astype(np.int32) - 127, ref["eW"])
    assert np.array_equal(hw.bias, ref["bias"].astype(np.float32))


def test_mx_quantiser_edge_values_bit_exact():
    """Rows built to hit every rounding boundary (ties on both sides, values
    just off them), saturation above 6, all-zero and subnormal blocks, mixed
    signs and negative zero: with rank 0 and no smoothing the residual is W
    itself, so the host encoder must match the oracle's bit for bit."""
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.5, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0])
    rows = []
    for k in (-20, -3, 0, 4):
        b = np.concatenate([ties, -ties]) * 2.0 ** k
        b[0] = 4.0 * 2.0 ** k                           # keeps the block exponent at k
        rows.append(b)
        rows.append(b * (1 + 2.0 ** -7))                # just above every boundary
        rows.append(b * (1 - 2.0 ** -7))                # just below
    rows.append(np.zeros(32))
    rows.append(np.concatenate([[2.0 ** -130, -2.0 ** -131], np.zeros(30)]))
    z = np.zeros(32)
    z[3] = -0.0
    z[5] = 3.0
    rows.append(z)
    W = np.stack([np.concatenate([r, r[::-1]]) for r in rows])   # K = 64
    Wb = O.bf16_bits_of(O.round_to_bf16(W))
    hw = S.mx_prepare_weights(Wb, None, None, 0)
    ref = MXO.prepare(Wb, None, None, 0)
    assert np.array_equal(hw.qweight, MXO.pack_fp4(ref["qW"]))
    assert np.array_equal(hw.wscales.astype(np.int32) - 127, ref["eW"])


def test_mx_residual_within_half_a_step():
    c = synth.linear_case("mxres", 91, 64, 128, 256, 12, x_outlier_n=4, x_outlier_scale=40.0)
    ax = c.calib_absmax()
    hw = S.mx_prepare_weights(c.W, ax, c.bias, 12)
    lam, _ = O.smoothing_factors(ax, O.bf16_values(c.W))
    W_hat = O.smooth_weight(O.bf16_values(c.W), lam)
    R = W_hat - _cpp_branch(hw, lam)
    e = hw.wscales.astype(np.int32) - 127
    deq = MXO.dequantize(MXO.unpack_fp4(hw.qweight), e)
    scale = np.repeat(np.exp2(e.astype(np.float64)), 32, axis=1)
    # the grid step is at most 2 x scale (between 4 and 6); saturation only
    # clips values in (6, 8) x scale, and the block max is below 8 x scale
    assert np.all(np.abs(R - deq) <= 2.0 * scale * (1 + 2.0 ** -20) + 2.0 ** -24 * np.abs(R))


def test_mx_blob_layout():
    """Codes and scales sit where the documented MXFP4 tiling says: for
    K-step s and tile t, lane l = row % 32 + 32 h holds the row's canonical
    bytes 32 s + 16 h + [0, 16) at ((s T + t) 64 + l) 16, and the E8M0 scale
    of MX block 2 s + h at (s T + 4 (t // 4)) 64 + 4 l + t % 4 of the scale
    array (byte t % 4 of the lane's word for its group of four tiles)."""
    c = synth.linear_case("mxpk", 92, 8, 100, 192, 5, x_outlier_n=2, x_outlier_scale=20.0)
    hw = S.mx_prepare_weights(c.W, c.calib_absmax(), c.bias, 5)
    blob = S.mx_pack_device_weights(hw)
    N, K, G, Np = 100, 192, 3, 256
    T = Np // 32
    qbytes = Np * K // 2
    q = blob[:qbytes]
    s_off = (qbytes + 255) // 256 * 256
    sc = blob[s_off: s_off + Np * (K // 32)]
    for n in range(N):
        for s_ in range(G):
            for h in range(2):
                lane = n % 32 + 32 * h
                base = ((s_ * T + n // 32) * 64 + lane) * 16
                assert np.array_equal(q[base: base + 16], hw.qweight[n, 32 * s_ + 16 * h: 32 * s_ + 16 * h + 16])
                t = n // 32
                assert sc[(s_ * T + 4 * (t // 4)) * 64 + 4 * lane + t % 4] == hw.wscales[n, 2 * s_ + h]
    # padded rows: +0 codes and the smallest scale byte (0)
    assert not np.any(q.reshape(G, T, 64, 16)[:, 3, 4:32]) and not np.any(q.reshape(G, T, 64, 16)[:, 4:])
    sc4 = sc.reshape(G, T // 4, 64, 4)
    assert not np.any(sc4[:, 1:]) and not np.any(sc4[:, 0, 4:32, 3]) and not np.any(sc4[:, 0, 36:, 3])


# ---------------------------------------------------------------- errors
INV, SHAPE, NODEV, WS, NUM = 1, 2, 3, 5, 6
FAKE = 1 << 20          # aligned, never dereferenced: validation fails first


def _dw(N=128, K=128, rank=4, blob=FAKE):
    return S.DeviceWeights(blob, N, K, rank)


def test_prepare_errors():
    lib = S._lib
    W = np.zeros((16, 64), np.uint16)
    hw = S.PreparedHost(16, 64, 0, np.zeros(64, np.float32), np.zeros((64, 0), np.uint16),
                        np.zeros((0, 16), np.uint16), np.zeros((16, 32), np.uint8),
                        np.zeros((16, 1), np.float32), np.zeros(16, np.float32)).as_struct()
    assert lib.svdq_prepare_weights(None, 16, 64, None, None, 0, 64, ctypes.byref(hw)) == INV
    assert lib.svdq_prepare_weights(W.ctypes.data, 16, 64, None, None, 0, 32, ctypes.byref(hw)) == SHAPE
    assert lib.svdq_prepare_weights(W.ctypes.data, 16, 60, None, None, 0, 64, ctypes.byref(hw)) == SHAPE
    assert lib.svdq_prepare_weights(W.ctypes.data, 16, 64, None, None, 17, 64, ctypes.byref(hw)) == SHAPE
    assert lib.svdq_prepare_weights(W.ctypes.data, 16, 64, None, None, -1, 64, ctypes.byref(hw)) == SHAPE
    assert lib.svdq_prepare_weights(W.ctypes.data, 0, 64, None, None, 0, 64, ctypes.byref(hw)) == SHAPE
    Wn = W.copy()
    Wn[3, 5] = 0x7FC0                      # bf16 NaN
    assert lib.svdq_prepare_weights(Wn.ctypes.data, 16, 64, None, None, 0, 64, ctypes.byref(hw)) == NUM
    ax = np.ones(64, np.float32)
    ax[2] = np.inf
    assert lib.svdq_prepare_weights(W.ctypes.data, 16, 64, ax.ctypes.data, None, 0, 64, ctypes.byref(hw)) == NUM
    assert b"act_absmax" in lib.svdq_last_error()
    with pytest.raises(S.SvdqError):
        S.prepare_weights(np.zeros((8, 100), np.uint16), None, None, 0)


def test_forward_validation_errors():
    lib = S._lib
    w = _dw()
    ws = S.workspace_bytes(64, 128, 128, 4)
    call = lambda **kw: lib.svdq_linear_forward(
        ctypes.byref(kw.get("w", w)), kw.get("X", FAKE), kw.get("M", 64), kw.get("Y", FAKE),
        kw.get("dt", S.BF16), kw.get("epi", 0), kw.get("ws", FAKE), kw.get("wsb", ws), None)
    assert call(X=None) == INV
    assert call(X=FAKE + 4) == INV                 # misaligned
    assert call(M=0) == SHAPE
    assert call(M=(1 << 31) // 128 + 1, wsb=1 << 40) == SHAPE      # M * K past 2^31
    assert call(dt=S.FP16) == INV
    assert call(epi=7) == INV
    assert call(wsb=ws - 1) == WS
    assert call(w=_dw(K=100)) == SHAPE
    assert call(w=_dw(rank=200)) == SHAPE
    assert call(w=_dw(blob=0)) == INV
    assert lib.awq_w4a16_forward(FAKE, 64, 128, FAKE, 17, None, FAKE, None) == SHAPE
    assert lib.awq_w4a16_forward(FAKE, 64, 100, FAKE, 1, None, FAKE, None) == SHAPE
    assert lib.awq_w4a16_forward(None, 64, 128, FAKE, 1, None, FAKE, None) == INV
    assert lib.svdq_debug_group_sums(ctypes.byref(w), 64, 0, 300, 0, 8, FAKE, FAKE, ws, None) == SHAPE
    assert lib.svdq_debug_group_sums(ctypes.byref(w), 64, 60, 8, 0, 8, FAKE, FAKE, ws, None) == SHAPE
    assert lib.svdq_debug_group_sums_codes(ctypes.byref(w), FAKE, 64, 0, 300, 0, 8, FAKE, FAKE, ws,
                                           None) == SHAPE
    assert lib.svdq_debug_group_sums_codes(ctypes.byref(w), None, 64, 0, 8, 0, 8, FAKE, FAKE, ws,
                                           None) == INV
    assert lib.svdq_gelu_tanh_bf16(FAKE + 2, FAKE, 16, None) == INV
    # measurement probes: argument checks come before any device work
    assert lib.svdq_measure_mfma(8, 10, 8, FAKE, None) == INV
    assert lib.svdq_measure_mfma(-1, 10, 8, FAKE, None) == INV
    assert lib.svdq_measure_mfma(0, 10, 8, None, None) == INV
    assert lib.svdq_measure_mfma(0, 0, 8, FAKE, None) == SHAPE
    assert lib.svdq_measure_mfma(0, 10, 0, FAKE, None) == SHAPE
    assert lib.svdq_measure_stream(FAKE, None, 4096, 8, 0, None, None) == INV     # a read needs a sink
    assert lib.svdq_measure_stream(FAKE, FAKE, 4100, 8, 1, None, None) == INV     # 16-byte multiples
    assert lib.svdq_measure_stream(FAKE, FAKE, 4096, 0, 1, None, None) == SHAPE
    assert S._lib.svdq_workspace_bytes(0, 128, 128, 4) == 0
    assert S._lib.svdq_device_weights_bytes(128, 100, 4) == 0


def test_mlp_pair_argument_errors():
    """The fused MLP pair's entry points reject shapes that do not chain, a
    shared workspace and undersized workspaces before any HIP call."""
    lib = S._lib
    w1, w2 = _dw(N=256, K=128), _dw(N=128, K=256)
    ws1 = S.workspace_bytes(64, 256, 128, 4)
    ws2 = S.workspace_bytes(64, 128, 256, 4)
    bad = _dw(N=128, K=192)
    B1, B2 = FAKE, FAKE + (1 << 24)
    assert lib.svdq_mlp_forward(ctypes.byref(w1), ctypes.byref(bad), FAKE, 64, FAKE, S.BF16, 1,
                                B1, ws1, B2, S.workspace_bytes(64, 128, 192, 4), None) == SHAPE
    assert lib.svdq_mlp_gemm1(ctypes.byref(w1), ctypes.byref(w2), 64, 1, B1, ws1, B1, ws2, None) == INV
    assert lib.svdq_mlp_gemm1(ctypes.byref(w1), ctypes.byref(w2), 64, 1, B1, ws1, B2, ws2 - 256, None) == WS
    assert lib.svdq_mlp_gemm1(ctypes.byref(w1), ctypes.byref(w2), 64, 7, B1, ws1, B2, ws2, None) in (INV, NODEV)
    assert lib.svdq_mlp_quantize(ctypes.byref(w1), ctypes.byref(w2), None, 64, B1, ws1, B2, ws2, None) in (INV, NODEV)
    assert lib.svdq_mlp_gemm2(ctypes.byref(w2), 64, None, S.BF16, B2, ws2, None) == INV


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-device path")
def test_no_device_is_reported():
    assert S._lib.svdq_device_check() == NODEV
    w = _dw()
    ws = S.workspace_bytes(64, 128, 128, 4)
    assert S._lib.svdq_linear_forward(ctypes.byref(w), FAKE, 64, FAKE, S.BF16, 0, FAKE, ws, None) == NODEV
    assert S._lib.svdq_gelu_tanh_bf16(FAKE, FAKE, 16, None) == NODEV
    w1, w2 = _dw(N=256, K=128), _dw(N=128, K=256)
    assert S._lib.svdq_mlp_forward(ctypes.byref(w1), ctypes.byref(w2), FAKE, 64, FAKE, S.BF16, 1,
                                   FAKE, S.workspace_bytes(64, 256, 128, 4), FAKE + (1 << 24),
                                   S.workspace_bytes(64, 128, 256, 4), None) == NODEV


def test_host_weights_accept_fortran_ordered_arrays():
    """Arrays handed to the C side are made row-major first (an oracle SVD
    factor is a transposed view, i.e. Fortran-ordered)."""
    c = synth.linear_case("fo", 90, 8, 96, 128, 6, x_outlier_n=2, x_outlier_scale=20.0)
    ref = O.prepare(c.W, c.calib_absmax(), c.bias, 6)
    assert not ref["L1s"].flags.c_contiguous
    from tests.gpu_util import host_from_oracle
    hw = host_from_oracle(ref)
    assert hw.l1s.flags.c_contiguous and hw.l2.flags.c_contiguous
    blob = S.pack_device_weights(hw)
    L = S.device_weights_bytes(96, 128, 6)
    Np, rp, K = 256, 32, 128
    off_l2t = Np * K * 3 // 4 + 2 * Np * 16      # codes, then 2 groups of 16-byte scale operands
    off_l1t = off_l2t + Np * rp * 2
    # L1s in the quantiser's fragment order: [group][32-rank block][16-channel
    # step j][lane][8 channels]; lane l is rank l % 32 of the block, channels
    # 16 j + 8 (l // 32) + [0, 8) of the group
    frag = blob[off_l1t: off_l1t + rp * K * 2].view(np.uint16).reshape(K // 64, rp // 32, 4, 64, 8)
    l1 = np.zeros((K, rp), np.uint16)
    for g in range(K // 64):
        for b in range(rp // 32):
            for j in range(4):
                for lane in range(64):
                    k0 = 64 * g + 16 * j + 8 * (lane // 32)
                    l1[k0:k0 + 8, 32 * b + lane % 32] = frag[g, b, j, lane]
    assert np.array_equal(l1[:, :6], O.bf16_bits_of(ref["L1s"]))
    assert not l1[:, 6:].any()
    l2t = blob[off_l2t: off_l2t + Np * rp * 2].view(np.uint16).reshape(Np, rp)
    assert np.array_equal(l2t[:96, :6].T, O.bf16_bits_of(ref["L2b"]))
    assert L == len(blob)


# ------------------------------------------------------- user LoRA merge
from oracle import lora as LO  # noqa: E402


@pytest.mark.parametrize("form", ["int4", "mx"])
@pytest.mark.parametrize("rank,r2,alpha", [(8, 5, 0.3), (0, 16, -1.25), (16, 0, 2.0)])
def test_merge_lora_bit_exact(form, rank, r2, alpha):
    c = synth.linear_case("lmerge", 92, 8, 96, 192, rank, x_outlier_n=2, x_outlier_scale=20.0)
    A, B = synth.lora_factors(93, c.N, c.K, r2, b_std=0.7)
    if form == "int4":
        hw = S.prepare_weights(c.W, c.calib_absmax(), c.bias, rank)
        ref = LO.merge(O.prepare(c.W, c.calib_absmax(), c.bias, rank), A, B, alpha)
        got = S.merge_lora(hw, A, B, alpha)
    else:
        hw = S.mx_prepare_weights(c.W, c.calib_absmax(), c.bias, rank)
        ref = LO.merge(MXO.prepare(c.W, c.calib_absmax(), c.bias, rank), A, B, alpha)
        got = S.mx_merge_lora(hw, A, B, alpha)
    assert got.rank == rank + r2 == ref["rank"]
    # the appended LoRA factors bit for bit (the base factors' singular
    # vectors may differ from the oracle's in sign, so those are compared
    # with the host's own base layer below)
    assert np.array_equal(got.l1s[:, rank:], O.bf16_bits_of(ref["L1s"][:, rank:]))
    assert np.array_equal(got.l2[rank:], O.bf16_bits_of(ref["L2b"][rank:]))
    # the 4-bit arrays are the base layer's own buffers, untouched
    assert got.qweight is hw.qweight and got.wscales is hw.wscales
    assert np.array_equal(got.l1s[:, :rank], hw.l1s) and np.array_equal(got.l2[:rank], hw.l2)


def test_merge_lora_copies_into_separate_buffers_and_errors():
    lib = S._lib
    c = synth.linear_case("lmerr", 94, 8, 64, 128, 4, x_outlier_n=2, x_outlier_scale=20.0)
    hw = S.prepare_weights(c.W, c.calib_absmax(), c.bias, 4)
    A, B = synth.lora_factors(95, c.N, c.K, 3)
    src = hw.as_struct()
    out = S.PreparedHost(c.N, c.K, 7, np.zeros(c.K, np.float32), np.zeros((c.K, 7), np.uint16),
                         np.zeros((7, c.N), np.uint16), np.zeros_like(hw.qweight),
                         np.zeros_like(hw.wscales), np.zeros_like(hw.bias))
    dst = out.as_struct()
    assert lib.svdq_merge_lora(ctypes.byref(src), A.ctypes.data, B.ctypes.data, 3, 1.0,
                               ctypes.byref(dst)) == 0
    for k in ("inv_lambda", "qweight", "wscales", "bias"):
        assert np.array_equal(getattr(out, k), getattr(hw, k))
    assert (dst.N, dst.K, dst.rank, dst.group_size) == (c.N, c.K, 7, 64)
    # errors: merged rank too large, non-finite alpha / factors / product,
    # negative rank, missing factors, output factors aliasing the input's
    big = np.zeros((c.N - 2, c.K), np.uint16), np.zeros((c.N, c.N - 2), np.uint16)
    assert lib.svdq_merge_lora(ctypes.byref(src), big[0].ctypes.data, big[1].ctypes.data, c.N - 2,
                               1.0, ctypes.byref(dst)) == SHAPE
    assert lib.svdq_merge_lora(ctypes.byref(src), A.ctypes.data, B.ctypes.data, 3, float("nan"),
                               ctypes.byref(dst)) == NUM
    An = A.copy()
    An[1, 7] = 0x7F80                      # bf16 +inf
    assert lib.svdq_merge_lora(ctypes.byref(src), An.ctypes.data, B.ctypes.data, 3, 1.0,
                               ctypes.byref(dst)) == NUM
    Bh = B.copy()
    Bh[5, 1] = 0x7F00                      # 2^127: times 4 overflows float32
    before = out.l2.copy()
    assert lib.svdq_merge_lora(ctypes.byref(src), A.ctypes.data, Bh.ctypes.data, 3, 4.0,
                               ctypes.byref(dst)) == NUM
    assert np.array_equal(out.l2, before)  # nothing written on failure
    assert lib.svdq_merge_lora(ctypes.byref(src), A.ctypes.data, B.ctypes.data, -1, 1.0,
                               ctypes.byref(dst)) == SHAPE
    assert lib.svdq_merge_lora(ctypes.byref(src), None, B.ctypes.data, 3, 1.0,
                               ctypes.byref(dst)) == INV
    alias = S.HostWeights(c.N, c.K, 7, 64, dst.inv_lambda, src.l1s, dst.l2, dst.qweight,
                          dst.wscales, dst.bias)
    assert lib.svdq_merge_lora(ctypes.byref(src), A.ctypes.data, B.ctypes.data, 3, 1.0,
                               ctypes.byref(alias)) == INV
    with pytest.raises(ValueError):
        S.merge_lora(hw, A, B[:, :2])


def test_workspace_includes_k_split_partials():
    """svdq_workspace_bytes adds ksplit * Mp * Np * 4 bytes of fp32 partial
    tiles exactly when the GEMM's 128 x 256 tile grid has fewer than 128
    tiles (ksplit = min(8, 512 // tiles, groups // 8) >= 2) and not from
    128 tiles on."""
    lib = S._lib
    up = lambda x: -(-x // 256) * 256
    def base(M, K, r):
        Mp, G, rp = up(M), K // 64, -(-r // 32) * 32 if r else 0
        T = Mp // 32
        gmin = 12 if r > 0 and G >= 12 else 4   # quantiser splits: with a branch, >= 12 groups each
        Ssp = 1
        for s_ in range(1, G + 1):
            if G % s_:
                continue
            if s_ == 1 or G // s_ >= gmin:
                Ssp = s_
            if G // s_ >= gmin and T * s_ >= 384:
                break
        # fp6 codes, 16-byte scale operands, fp32 partials of D
        return up(Mp * K * 3 // 4) + up(G * Mp * 16) + up(max(Ssp, 2) * Mp * rp * 4)
    for M, N, K, r, ks in [(4608, 12288, 3072, 32, 1), (1024, 3072, 3072, 128, 5), (100, 200, 1024, 8, 2),
                           (1, 3072, 12288, 32, 8), (64, 512, 448, 4, 1), (4608, 3072, 12288, 32, 1),
                           (512, 9216, 3072, 32, 1), (512, 3072, 3072, 32, 6), (1024, 3072, 3072, 0, 5)]:
        want = base(M, K, r) + (ks * up(M) * up(N) * 4 if ks > 1 else 0)
        assert lib.svdq_workspace_bytes(M, N, K, r) == want, (M, N, K, r)


def test_package_refuses_to_load_without_the_library(tmp_path):
    """The product path has no fallback: a copy of the package without
    libsvdq.so fails at import with an error that names the missing file."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "w4a4_rank_corrected_smooth_amd")
    dst = tmp_path / "w4a4_rank_corrected_smooth_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "*.so.*", "__pycache__", "csrc"))
    r = subprocess.run([sys.executable, "-c", "import w4a4_rank_corrected_smooth_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libsvdq.so" in r.stderr and "missing" in r.stderr
