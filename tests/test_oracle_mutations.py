"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch each one.  A pin suite that passes a broken oracle proves nothing."""
import numpy as np
import pytest

from oracle import svdquant as O
from oracle import awq as OA
import tests.test_oracle_pins as pins


def _half_up_groups(v):
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).max(axis=-1)
    live = a >= O.TINY
    a_safe = np.where(live, a, np.float32(1.0)).astype(np.float32)
    s = np.where(live, a_safe / np.float32(7), np.float32(0)).astype(np.float32)
    inv = (np.float32(7) / a_safe).astype(np.float32)
    t = (v * inv[..., None]).astype(np.float32)
    q = np.clip(np.floor(t + np.float32(0.5)), -7, 7)          # mistake: ties up
    return np.where(live[..., None], q, 0).astype(np.int8), s


def _scale_over_8(v):
    q, s = ORIG["quantize_groups"](v)
    return q, (s * np.float32(7.0 / 8.0)).astype(np.float32)   # mistake: s = a/8


def _swapped_pack(q):
    q = np.asarray(q, dtype=np.int8).astype(np.uint8) & 0x0F
    return (q[..., 1::2] | (q[..., 0::2] << 4)).astype(np.uint8)  # mistake: nibble order


def _residual_plus(W_hat, lam, L1s, L2b):
    branch = (L1s @ L2b) * lam.astype(np.float64)[:, None]
    return (W_hat + branch.T).astype(np.float32)               # mistake: sign


def _residual_no_lambda(W_hat, lam, L1s, L2b):
    return (W_hat - (L1s @ L2b).T).astype(np.float32)          # mistake: dropped diag(lambda)


def _output_no_bias(qA, sA, qW, sW, D, L2b, bias):
    return O.dequantize(qA, sA) @ O.dequantize(qW, sW).T + D @ L2b  # mistake: dropped bias


def _output_no_branch(qA, sA, qW, sW, D, L2b, bias):
    return O.dequantize(qA, sA) @ O.dequantize(qW, sW).T + bias[None, :]


def _smoothing_inverted(act_absmax, W):
    lam, iota = ORIG["smoothing_factors"](act_absmax, W)
    return iota, lam                                          # mistake: lambda <-> 1/lambda


def _smooth_acts_with_lambda(X, iota):
    return (np.asarray(X, np.float32) / iota.astype(np.float32)[None, :]).astype(np.float32)


def _lowrank_u_v_swapped(W_hat, rank, iota, round_factors=True):
    N, K = W_hat.shape
    U, s, Vt = np.linalg.svd(W_hat, full_matrices=False)
    if rank == 0:
        return np.zeros((K, 0)), np.zeros((0, N)), s
    root = np.sqrt(s[:rank])
    L1 = Vt[:rank].T * root[None, :]
    L2 = (root[:, None] * U[:, :rank].T)[:, ::-1]              # mistake: column order of U
    L1s = iota.astype(np.float64)[:, None] * L1
    if round_factors:
        return O.round_to_bf16(L1s), O.round_to_bf16(L2), s
    return L1s, L2, s


def _awq_zero_sign(W_fp16):
    q, s, z = ORIG_AWQ(W_fp16)
    W = np.asarray(W_fp16, np.float16).astype(np.float32)
    N, K = W.shape
    Wg = W.reshape(N, K // 64, 64)
    sf = s.astype(np.float32)
    z2 = np.clip(np.rint((Wg.min(axis=2) / sf).astype(np.float32)), 0, 15).astype(np.float32)  # mistake: sign
    q2 = np.clip(np.rint((Wg / sf[:, :, None]).astype(np.float32)) + z2[:, :, None], 0, 15)
    return q2.reshape(N, K).astype(np.uint8), s, z2.astype(np.float16)


ORIG = {"quantize_groups": O.quantize_groups, "smoothing_factors": O.smoothing_factors}
ORIG_AWQ = OA.quantize

MUTANTS = [
    ("quantize_groups", O, _half_up_groups, ["test_quantizer_golden", "test_quantizer_bruteforce"]),
    ("quantize_groups", O, _scale_over_8, ["test_quantizer_golden", "test_quantizer_on_grid_reproduces_codes_and_scale"]),
    ("pack_int4", O, _swapped_pack, ["test_pack_canonical_nibble_order"]),
    ("residual", O, _residual_plus, ["test_full_rank_leaves_zero_residual", "test_residual_shrinks_with_rank"]),
    ("residual", O, _residual_no_lambda, ["test_full_rank_leaves_zero_residual"]),
    ("linear_output", O, _output_no_bias, ["test_output_two_routes_agree", "test_output_bruteforce_scalar_loops"]),
    ("linear_output", O, _output_no_branch, ["test_output_two_routes_agree", "test_output_bruteforce_scalar_loops"]),
    ("smoothing_factors", O, _smoothing_inverted, ["test_smoothing_golden", "test_smoothing_preserves_the_product"]),
    ("smooth_activations", O, _smooth_acts_with_lambda, ["test_activation_smoothing_multiply_is_one_rounding", "test_output_bruteforce_scalar_loops"]),
    ("lowrank_split", O, _lowrank_u_v_swapped, ["test_low_rank_branch_beats_plain_w4a4_on_outliers", "test_residual_shrinks_with_rank"]),
    ("quantize", OA, _awq_zero_sign, ["test_awq_golden", "test_awq_on_grid_is_lossless"]),
]


def _run(name):
    fn = getattr(pins, name)
    if name == "test_quantizer_bruteforce":
        for seed in range(6):
            fn(seed)
    elif name == "test_on_grid_inputs_give_the_exact_matmul":
        fn(31)
    elif name == "test_eckart_young_and_factor_structure":
        fn(5)
    else:
        fn()


@pytest.mark.parametrize("attr,mod,mutant,catchers", MUTANTS,
                         ids=[f"{m[0]}:{m[2].__name__}" for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, attr, mod, mutant, catchers):
    monkeypatch.setattr(mod, attr, mutant)
    caught = 0
    for name in catchers:
        try:
            _run(name)
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1, f"no pin caught mutant {mutant.__name__}"
