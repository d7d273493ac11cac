"""CPU oracle: the SVDQuant linear layer, written out step by step.

TEST INFRASTRUCTURE.  This module is the slow, obviously-correct statement of
what the device path computes.  Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product
library never does, and shares no code with it.

Sources.  "Bringing Nunchaku 4-bit diffusion inference to Diffusers"
(Vietnamese edition, section "Bối cảnh: SVDQuant và Nunchaku"; Korean edition,
section "SVDQuant 및 Nunchaku 엔진") describe the method: activation outliers
are migrated into the weights by a per-channel smoothing, the hardest part of
each smoothed weight matrix is kept as a small 16-bit low-rank branch, and
the remaining residual is quantised to 4 bits, with 4-bit activations on the
main path (W4A4).  The Hacker News thread "SVDQuant: 4-Bit Quantization Powers
12B Flux on a 16GB 4090 GPU with 3x Speedup" adds that the low-rank branch
behaves like a LoRA that reconstructs what quantisation would lose.  The
pages give no formulas; the readings used here (smoothing with migration
strength 1/2, balanced sqrt(Sigma) split, symmetric INT4 in [-7, 7] per group
of 64 consecutive input channels with fp32 scales) are listed, with reasons,
in the design notes of this repository.

Notation follows ``nn.Linear``: W is [N (out), K (in)], X is [M, K],
Y = X W^T + b.  Arrays of bf16 or fp32 *values* are held in float64 or
float32 numpy arrays; every float32 operation below is a single IEEE
round-to-nearest-even numpy operation (numpy never fuses multiply-add).

Parity status: every function here is pinned by the CPU tests
(``tests/test_oracle_pins.py``) against closed forms, library routines,
brute force, or exact special cases.
"""
from __future__ import annotations

import numpy as np

GROUP = 64                      # input channels per quantisation group
QMAX = 7                        # symmetric INT4 codes live in [-7, 7]
TINY = np.float32(2.0 ** -100)  # groups whose max |v| is below this quantise to 0
EPS_ABSMAX = np.float32(1e-5)   # floor on the per-channel maxima in the smoothing ratio
F32 = np.float32


# ------------------------------------------------------------------ rounding
def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values straight to the nearest bfloat16 value (8
    significant bits, ties to even), returned as float64.  One rounding, no
    detour through float32.  Subnormal bf16 quantum is 2**-133."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    q = np.exp2(np.maximum(e - 8, -133).astype(np.float64))
    return np.rint(x / q) * q                # x / q is exact (power of two)


def bf16_bits_of(values: np.ndarray) -> np.ndarray:
    """float64 values that are exactly bf16 -> uint16 bit patterns."""
    f = np.asarray(values, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ------------------------------------------------------------- O1 smoothing
def calibration_absmax(x_cal: np.ndarray) -> np.ndarray:
    """Per input channel max |x| over the calibration rows (float32, exact)."""
    return np.abs(np.asarray(x_cal, dtype=np.float32)).max(axis=0)


def smoothing_factors(act_absmax, W: np.ndarray):
    """Per-input-channel smoothing factors.

    The activation outliers are moved into the weights (Vietnamese edition,
    "Bối cảnh: SVDQuant và Nunchaku").  Reading used: migration strength 1/2,
        lambda_j = sqrt( max(ax_j, 1e-5) / max(aw_j, 1e-5) )
    with ax_j = max |X_cal[:, j]| and aw_j = max_n |W[n, j]|, every operation
    in float32; the runtime multiplies activations by iota_j = fl32(1 / lambda_j).
    ``act_absmax=None`` means no smoothing: lambda = iota = 1.
    Returns (lam, iota), float32 [K]."""
    W = np.asarray(W)
    K = W.shape[1]
    if act_absmax is None:
        return np.ones(K, F32), np.ones(K, F32)
    ax = np.asarray(act_absmax, dtype=F32)
    aw = np.abs(W.astype(F32)).max(axis=0)
    ratio = np.maximum(ax, EPS_ABSMAX) / np.maximum(aw, EPS_ABSMAX)   # fp32 divide
    lam = np.sqrt(ratio.astype(F32)).astype(F32)                      # fp32 sqrt
    iota = (F32(1.0) / lam).astype(F32)                               # fp32 divide
    return lam, iota


# -------------------------------------------------------- O2 smoothed weight
def smooth_weight(W: np.ndarray, lam: np.ndarray) -> np.ndarray:
    """W_hat = W diag(lambda) in float64 (exact: 8-bit x 24-bit mantissas)."""
    return np.asarray(W, dtype=np.float64) * lam.astype(np.float64)[None, :]


# ----------------------------------------------------- O3 low-rank branch
def lowrank_split(W_hat: np.ndarray, rank: int, iota: np.ndarray,
                  round_factors: bool = True):
    """Top-r singular triplets of W_hat carried as a 16-bit branch.

    The hardest part of each smoothed weight is represented by a small
    low-rank branch (Vietnamese edition, "Bối cảnh: SVDQuant và Nunchaku";
    Korean edition, "SVDQuant 및 Nunchaku 엔진").  With W_hat = U S V^T
    (singular values descending):
        L1 = V_r S_r^(1/2)          [K, r]
        L2 = S_r^(1/2) U_r^T        [r, N]
    so that W_hat ~ (L1 L2)^T.  The runtime feeds the *unsmoothed* X to the
    branch, so 1/lambda is folded into L1:  L1s = bf16(diag(iota) L1),
    L2b = bf16(L2).  ``round_factors=False`` keeps float64 factors (used only
    to pin the exact-SVD special case).
    Returns (L1s [K, r], L2b [r, N], sigma [min(N, K)]) as float64."""
    N, K = W_hat.shape
    if rank == 0:
        s = np.linalg.svd(W_hat, compute_uv=False)
        return np.zeros((K, 0)), np.zeros((0, N)), s
    U, s, Vt = np.linalg.svd(W_hat, full_matrices=False)
    root = np.sqrt(s[:rank])
    L1 = Vt[:rank].T * root[None, :]
    L2 = root[:, None] * U[:, :rank].T
    L1s = iota.astype(np.float64)[:, None] * L1
    if round_factors:
        return round_to_bf16(L1s), round_to_bf16(L2), s
    return L1s, L2, s


# ------------------------------------------------------------ O4 residual
def residual(W_hat: np.ndarray, lam: np.ndarray, L1s: np.ndarray,
             L2b: np.ndarray) -> np.ndarray:
    """What the 4-bit path must carry: R = W_hat - (diag(lambda) L1s L2b)^T,
    in float64 against the *rounded* factors (so the branch's own rounding is
    absorbed by the residual), then rounded once to float32."""
    branch = (L1s @ L2b) * lam.astype(np.float64)[:, None]     # [K, N]
    return (W_hat - branch.T).astype(F32)


# ------------------------------------------------------- O5 group quantiser
def quantize_groups(v: np.ndarray):
    """Symmetric INT4 quantisation of each trailing group of 64 float32 values.

        a   = max |v_i|                      (exact)
        a < 2**-100:  s = 0, all codes 0
        else:         s   = fl32(a / 7)
                      inv = fl32(7 / a)
                      q_i = clamp(rint(fl32(v_i * inv)), -7, 7)   (ties to even)

    Returns (q int8 [..., 64], s float32 [...]).  The element of largest
    magnitude always lands on +-7."""
    v = np.asarray(v, dtype=F32)
    assert v.shape[-1] == GROUP
    a = np.abs(v).max(axis=-1)
    live = a >= TINY
    a_safe = np.where(live, a, F32(1.0)).astype(F32)
    s = np.where(live, a_safe / F32(QMAX), F32(0.0)).astype(F32)
    inv = (F32(QMAX) / a_safe).astype(F32)
    t = (v * inv[..., None]).astype(F32)
    q = np.clip(np.rint(t), -QMAX, QMAX)
    q = np.where(live[..., None], q, 0.0).astype(np.int8)
    return q, s


def quantize_rows(R32: np.ndarray):
    """Apply the group quantiser along each row: [rows, K] float32 ->
    codes int8 [rows, K], scales float32 [rows, K/64]."""
    rows, K = R32.shape
    q, s = quantize_groups(R32.reshape(rows, K // GROUP, GROUP))
    return q.reshape(rows, K), s


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Canonical packing: byte j of a row holds code 2j in its low nibble and
    code 2j+1 in its high nibble, two's complement."""
    q = np.asarray(q, dtype=np.int8).astype(np.uint8) & 0x0F
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ------------------------------------------------------------- prepare
def prepare(W_bits: np.ndarray, act_absmax, bias_bits, rank: int,
            round_factors: bool = True) -> dict:
    """Offline preparation of one linear layer (O1-O6): smoothing factors,
    low-rank branch, residual, per-group INT4 residual codes and scales.

    W_bits: bf16 patterns [N, K]; act_absmax: float32 [K] or None;
    bias_bits: bf16 patterns [N] or None."""
    W = bf16_values(W_bits)
    N, K = W.shape
    assert K % GROUP == 0 and 0 <= rank <= min(N, K)
    lam, iota = smoothing_factors(act_absmax, W)
    W_hat = smooth_weight(W, lam)
    L1s, L2b, sigma = lowrank_split(W_hat, rank, iota, round_factors)
    R32 = residual(W_hat, lam, L1s, L2b)
    qW, sW = quantize_rows(R32)
    bias = (bf16_values(bias_bits) if bias_bits is not None else np.zeros(N))
    return dict(N=N, K=K, rank=rank, lam=lam, iota=iota, L1s=L1s, L2b=L2b,
                sigma=sigma, R32=R32, qW=qW, sW=sW, bias=bias.astype(np.float64))


# ------------------------------------------------- O7 activation quantiser
def smooth_activations(X: np.ndarray, iota: np.ndarray) -> np.ndarray:
    """x_hat = fl32(x * iota_k), one float32 multiply per element."""
    return (np.asarray(X, dtype=F32) * iota.astype(F32)[None, :]).astype(F32)


def quantize_activations(X: np.ndarray, iota: np.ndarray):
    """Runtime 4-bit activations (the A of W4A4): smooth, then the same group
    quantiser along each token row.  Returns (qA int8 [M, K], sA f32 [M, K/64])."""
    return quantize_rows(smooth_activations(X, iota))


# ------------------------------------------------------ O8 low-rank down
def lowrank_down(X: np.ndarray, L1s: np.ndarray) -> np.ndarray:
    """D = X L1s in float64 on the raw (unsmoothed) activations; equal to
    X diag(iota) L1 because iota is folded into L1s."""
    return np.asarray(X, dtype=np.float64) @ L1s


# ------------------------------------------------------- O9 group sums
def group_sums(qA: np.ndarray, qW: np.ndarray) -> np.ndarray:
    """P[m, n, g] = sum_{k in group g} qA[m, k] qW[n, k], exact int64."""
    M, K = qA.shape
    N = qW.shape[0]
    G = K // GROUP
    a = qA.astype(np.int64).reshape(M, G, GROUP)
    w = qW.astype(np.int64).reshape(N, G, GROUP)
    return np.einsum("mgk,ngk->mng", a, w)


# ----------------------------------------------------------- O10 output
def linear_output_from_sums(P, sA, sW, D, L2b, bias) -> np.ndarray:
    """Y[m, n] = sum_g sA[m,g] sW[n,g] P[m,n,g] + sum_t D[m,t] L2b[t,n] + b[n]
    in float64, straight from the definition (small shapes)."""
    scaled = P.astype(np.float64) * sA.astype(np.float64)[:, None, :] \
        * sW.astype(np.float64)[None, :, :]
    return scaled.sum(axis=2) + D @ L2b + bias[None, :]


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """codes * group scale, float64 (exact: 3-bit x 24-bit)."""
    rows, K = q.shape
    return (q.astype(np.float64).reshape(rows, K // GROUP, GROUP)
            * s.astype(np.float64)[:, :, None]).reshape(rows, K)


def linear_output(qA, sA, qW, sW, D, L2b, bias) -> np.ndarray:
    """Same quantity as ``linear_output_from_sums`` evaluated as one float64
    GEMM of the dequantised operands (equal up to float64 summation order),
    for large shapes."""
    return dequantize(qA, sA) @ dequantize(qW, sW).T + D @ L2b + bias[None, :]


def forward(prep: dict, X_bits: np.ndarray, rows=None) -> dict:
    """Runtime forward of one prepared layer on bf16 activations.
    ``rows`` optionally restricts the computation to a subset of token rows."""
    X = bf16_values(X_bits)
    if rows is not None:
        X = X[rows]
    qA, sA = quantize_activations(X, prep["iota"])
    D = lowrank_down(X, prep["L1s"])
    Y = linear_output(qA, sA, prep["qW"], prep["sW"], D, prep["L2b"], prep["bias"])
    return dict(qA=qA, sA=sA, D=D, Y=Y)
