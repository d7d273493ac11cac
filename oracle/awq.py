"""CPU oracle: AWQ-style W4A16 linear (4-bit weights, 16-bit activations).

TEST INFRASTRUCTURE (same import rule as ``oracle.svdquant``).

Source.  "Bringing Nunchaku 4-bit diffusion inference to Diffusers" (Russian
edition, section "Технические детали и поддержка железа"; Korean edition,
section "Diffusers 내 Nunchaku Lite 통합") name a second kernel family,
awq_w4a16: 4-bit weights with 16-bit activations, used for memory-bound,
precision-sensitive layers such as the adaptive-normalisation / modulation
projections.  The pages do not describe AWQ's activation-aware scale search;
the reading used is plain round-to-nearest asymmetric quantisation per group
of 64 input channels with fp16 scales and fp16 (integer-valued) zero points:

    s  = fp16( fl32( max(wmax - wmin, 1e-5) / 15 ) )
    z  = clamp( rint( fl32(-wmin / s) ), 0, 15 )
    q  = clamp( rint( fl32(w / s) ) + z, 0, 15 )
    w~ = (q - z) * s
    y[m, n] = sum_g s[n,g] * sum_{k in g} x[m,k] (q[n,k] - z[n,g])  (+ b[n])

Parity status: pinned by the CPU tests (``tests/test_oracle_pins.py``).
"""
from __future__ import annotations

import numpy as np

GROUP = 64
F32 = np.float32


def quantize(W_fp16: np.ndarray):
    """RTN asymmetric INT4 per group of 64 along each row.
    W_fp16: float16 [N, K].  Returns (q uint8 [N, K] in 0..15,
    s float16 [N, K/64], z float16 [N, K/64])."""
    W = np.asarray(W_fp16, dtype=np.float16).astype(F32)
    N, K = W.shape
    G = K // GROUP
    Wg = W.reshape(N, G, GROUP)
    wmax = Wg.max(axis=2)
    wmin = Wg.min(axis=2)
    rng = np.maximum((wmax - wmin).astype(F32), F32(1e-5))
    s32 = (rng / F32(15.0)).astype(F32)
    s16 = s32.astype(np.float16)
    s = s16.astype(F32)
    z = np.clip(np.rint((-wmin / s).astype(F32)), 0, 15).astype(F32)
    q = np.clip(np.rint((Wg / s[:, :, None]).astype(F32)) + z[:, :, None], 0, 15)
    return q.reshape(N, K).astype(np.uint8), s16, z.astype(np.float16)


def pack(q: np.ndarray) -> np.ndarray:
    """Canonical packing: unsigned nibbles, low nibble = even k."""
    q = np.asarray(q, dtype=np.uint8) & 0x0F
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def unpack(p: np.ndarray) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def dequantize(q: np.ndarray, s: np.ndarray, z: np.ndarray) -> np.ndarray:
    """w~ = (q - z) * s in float64 (exact)."""
    N, K = q.shape
    qg = q.astype(np.float64).reshape(N, K // GROUP, GROUP)
    return ((qg - z.astype(np.float64)[:, :, None]) * s.astype(np.float64)[:, :, None]).reshape(N, K)


def forward(x: np.ndarray, q: np.ndarray, s: np.ndarray, z: np.ndarray, bias=None) -> np.ndarray:
    """y = sum_g s * sum_{k in g} x (q - z) (+ b), float64, group-factored."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    N = q.shape[0]
    G = K // GROUP
    xg = x.reshape(M, G, GROUP)
    qg = q.astype(np.float64).reshape(N, G, GROUP) - z.astype(np.float64)[:, :, None]
    inner = np.einsum("mgk,ngk->mng", xg, qg)
    y = (inner * s.astype(np.float64)[None, :, :]).sum(axis=2)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return y
