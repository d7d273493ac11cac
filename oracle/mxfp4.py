"""CPU oracle: the FP4 variant of the SVDQuant linear layer, in the OCP
Microscaling format MXFP4, written out step by step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product library never
does and shares no code with it.  Parity status: every function here is
pinned by ``tests/test_oracle_mx.py`` (the OCP element table, rounding ties,
saturation, the scale rule, on-grid exactness, an independent scalar
implementation on small inputs).

Sources.  "Bringing Nunchaku 4-bit diffusion inference to Diffusers"
(Vietnamese edition, section "Giới thiệu Nunchaku Lite"; Korean edition,
section "Diffusers 내 Nunchaku Lite 통합") name an FP4 form of the 4-bit path
(NVFP4, for Blackwell GPUs) beside the INT4 one, without defining its
numerics.  The reading here keeps everything of the INT4 method (smoothing,
low-rank split, residual, 16-bit branch) and changes only the 4-bit
encoding of the residual weights and of the smoothed activations, to the
block-scaled FP4 format that gfx950's matrix instructions take natively:

* OCP Microscaling Formats (MX) v1.0: a block of 32 consecutive values along
  the reduction axis K shares one 8-bit power-of-two scale X = 2**e (E8M0,
  e in [-127, 127], stored biased by 127); each value is an FP4 E2M1
  element: sign, 2 exponent bits (bias 1), 1 mantissa bit, magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* Scale: e = floor(log2(max |v|)) - 2, 2 being the largest exponent of
  E2M1, clamped to [-127, 127]; an all-zero block takes e = -127.
* Elements: v / X rounded to the nearest E2M1 value, ties to the value with
  an even mantissa bit, magnitudes above 6 saturating to 6.  A value that
  rounds to zero is stored as +0 (code 0), whatever its sign.

The product of two E2M1 elements is exact, and so is a block's sum of 32 of
them (multiples of 1/4 below 2**11), so each block contributes
2**(eA + eW) * sum exactly; the oracle evaluates Y in float64.
"""
from __future__ import annotations

import numpy as np

from . import svdquant as O

BLOCK = 32
EMAX_E2M1 = 2
E8M0_MIN, E8M0_MAX = -127, 127
# code (0..15) -> value: bit 3 sign, bits 2..0 index into the magnitudes
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
F32 = np.float32


def e2m1_value(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 codes -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def e2m1_round(r: np.ndarray) -> np.ndarray:
    """float64 values (already divided by the block scale) -> E2M1 codes:
    nearest magnitude, ties to the even mantissa bit (even code index),
    saturation at 6; zero magnitudes get code 0."""
    r = np.asarray(r, dtype=np.float64)
    mag = np.abs(r)
    lo_i = np.clip(np.searchsorted(E2M1_MAGNITUDES, mag, side="right") - 1, 0, 7)
    hi_i = np.minimum(lo_i + 1, 7)
    lo, hi = E2M1_MAGNITUDES[lo_i], E2M1_MAGNITUDES[hi_i]
    d_lo, d_hi = mag - lo, hi - mag
    take_hi = (lo_i < 7) & ((d_hi < d_lo) | ((d_hi == d_lo) & (hi_i % 2 == 0)))
    idx = np.where(take_hi, hi_i, lo_i)
    sign = np.where((r < 0) & (idx > 0), 8, 0)
    return (sign | idx).astype(np.uint8)


def block_exponents(v: np.ndarray) -> np.ndarray:
    """Shared scale exponent of each block of 32 along the last axis of a
    float32 array [rows, K]: floor(log2(max |v|)) - 2, clamped; -127 for an
    all-zero block.  Returns int32 [rows, K/32]."""
    rows, K = v.shape
    a = np.abs(v.astype(np.float64)).reshape(rows, K // BLOCK, BLOCK).max(axis=2)
    _, f = np.frexp(a)                       # a = m * 2**f, 0.5 <= m < 1: floor(log2 a) = f - 1
    e = np.where(a > 0, f - 1 - EMAX_E2M1, E8M0_MIN)
    return np.clip(e, E8M0_MIN, E8M0_MAX).astype(np.int32)


def quantize_rows(v: np.ndarray):
    """MXFP4 encoding of each row of a float32 array [rows, K] in blocks of
    32 consecutive values: (codes uint8 [rows, K], exponents int32
    [rows, K/32])."""
    v = np.asarray(v, dtype=F32)
    rows, K = v.shape
    assert K % BLOCK == 0
    e = block_exponents(v)
    scale = np.exp2(e.astype(np.float64))
    r = v.astype(np.float64).reshape(rows, K // BLOCK, BLOCK) / scale[:, :, None]
    return e2m1_round(r).reshape(rows, K), e


def dequantize(codes: np.ndarray, e: np.ndarray) -> np.ndarray:
    """codes * 2**e per block, float64 (exact)."""
    rows, K = codes.shape
    return (e2m1_value(codes).reshape(rows, K // BLOCK, BLOCK)
            * np.exp2(e.astype(np.float64))[:, :, None]).reshape(rows, K)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """Canonical packing: byte (r, j) = code[r, 2j] | code[r, 2j+1] << 4."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_fp4(p: np.ndarray) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# ------------------------------------------------------------- prepare
def prepare(W_bits: np.ndarray, act_absmax, bias_bits, rank: int) -> dict:
    """Offline preparation: smoothing, low-rank split and residual exactly as
    in the INT4 method (``svdquant``), then the residual rows in MXFP4."""
    base = O.prepare(W_bits, act_absmax, bias_bits, rank)
    qW, eW = quantize_rows(base["R32"])
    out = {k: base[k] for k in ("N", "K", "rank", "lam", "iota", "L1s", "L2b", "sigma",
                                "R32", "bias")}
    out.update(qW=qW, eW=eW)
    return out


def quantize_activations(X: np.ndarray, iota: np.ndarray):
    """x_hat = fl32(x * iota) (the INT4 path's smoothing), then MXFP4 rows."""
    return quantize_rows(O.smooth_activations(X, iota))


def block_sums(qA: np.ndarray, qW: np.ndarray) -> np.ndarray:
    """S[m, n, b] = sum over block b of value(qA[m, k]) value(qW[n, k]),
    exact (multiples of 1/4), float64 [M, N, K/32]."""
    M, K = qA.shape
    N = qW.shape[0]
    a = e2m1_value(qA).reshape(M, K // BLOCK, BLOCK)
    w = e2m1_value(qW).reshape(N, K // BLOCK, BLOCK)
    return np.einsum("mbk,nbk->mnb", a, w)


def linear_output(qA, eA, qW, eW, D, L2b, bias) -> np.ndarray:
    """Y = dequant(A) dequant(W)^T + D L2b + b in float64."""
    return dequantize(qA, eA) @ dequantize(qW, eW).T + D @ L2b + bias[None, :]


def forward(prep: dict, X_bits: np.ndarray, rows=None) -> dict:
    X = O.bf16_values(X_bits)
    if rows is not None:
        X = X[rows]
    qA, eA = quantize_activations(X, prep["iota"])
    D = O.lowrank_down(X, prep["L1s"])
    Y = linear_output(qA, eA, prep["qW"], prep["eW"], D, prep["L2b"], prep["bias"])
    return dict(qA=qA, eA=eA, D=D, Y=Y)
