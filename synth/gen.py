"""Seeded generators for the linear-layer workloads.

Every workload is drawn from ``numpy.random.default_rng(seed)`` (PCG64) in a
fixed order: activations X, the activation outlier channels, weights W, the
weight outlier channels, the bias, then (for the MLP pair) the second layer's
weight and bias.  Draws are float32; outlier channels multiply whole columns
(input channels) of X or W in float32; the result is rounded to the storage
type with round-to-nearest-even.

Shapes and distributions follow the diffusion-transformer projections the
pages discuss: a fused QKV projection and an MLP pair of a 3072-wide Flux-like
block at 1024x1024 (4096 image + 512 text tokens), a low-resolution high-rank
stress case, and the AWQ W4A16 modulation (adaptive-norm) projection.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


# ---------------------------------------------------------------- storage types
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16.  Inputs are finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _n_outliers(fraction: float, k: int) -> int:
    return int(round(fraction * k))


# ---------------------------------------------------------------- case records
@dataclass
class LinearCase:
    """One SVDQuant linear workload.  ``X``, ``W``, ``bias`` are bf16 bit
    patterns (uint16); ``x_outliers`` / ``w_outliers`` list the scaled
    channels; ``calib_rows`` is the calibration slice length (rows 0..63 of X
    supply the activation channel maxima)."""
    name: str
    seed: int
    M: int
    N: int
    K: int
    rank: int
    X: np.ndarray
    W: np.ndarray
    bias: np.ndarray
    x_outliers: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    w_outliers: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    calib_rows: int = 64
    group: int = 64

    def calib_absmax(self) -> np.ndarray:
        """Per-input-channel max |X| over the calibration rows, float32.
        (A max of absolute values: storage bookkeeping, exact in float32.)"""
        xc = bf16_bits_to_f32(self.X[: self.calib_rows])
        return np.abs(xc).max(axis=0).astype(np.float32)


@dataclass
class AwqCase:
    """AWQ W4A16 modulation workload: ``x`` fp16 [Mmax, K], ``W`` fp16 [N, K]."""
    name: str
    seed: int
    N: int
    K: int
    x: np.ndarray
    W: np.ndarray
    bias: Optional[np.ndarray] = None
    group: int = 64


# ---------------------------------------------------------------- generators
def linear_case(name: str, seed: int, M: int, N: int, K: int, rank: int,
                x_outlier_frac: float = 0.0, x_outlier_n: Optional[int] = None,
                x_outlier_scale: float = 1.0,
                w_outlier_frac: float = 0.0, w_outlier_n: Optional[int] = None,
                w_outlier_scale: float = 1.0,
                w_std: float = 0.02, b_std: float = 0.01) -> LinearCase:
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K), dtype=np.float32)
    nx = x_outlier_n if x_outlier_n is not None else _n_outliers(x_outlier_frac, K)
    xi = np.sort(rng.choice(K, nx, replace=False)) if nx > 0 else np.zeros(0, np.int64)
    if nx > 0:
        X[:, xi] *= np.float32(x_outlier_scale)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)
    nw = w_outlier_n if w_outlier_n is not None else _n_outliers(w_outlier_frac, K)
    wi = np.sort(rng.choice(K, nw, replace=False)) if nw > 0 else np.zeros(0, np.int64)
    if nw > 0:
        W[:, wi] *= np.float32(w_outlier_scale)
    b = rng.standard_normal(N, dtype=np.float32) * np.float32(b_std)
    return LinearCase(name=name, seed=seed, M=M, N=N, K=K, rank=rank,
                      X=f32_to_bf16_bits(X), W=f32_to_bf16_bits(W),
                      bias=f32_to_bf16_bits(b), x_outliers=xi, w_outliers=wi)


def tiny_case() -> LinearCase:
    """256x512 -> 512, rank 16, 8 activation channels x40 (seed 0)."""
    return linear_case("tiny", 0, 256, 512, 512, 16,
                       x_outlier_n=8, x_outlier_scale=40.0)


def qkv_case() -> LinearCase:
    """Fused QKV projection: 4608 tokens, 3072 -> 9216, rank 32; 0.5% of the
    activation channels x50, 1% of the weight input channels x8 (seed 1)."""
    return linear_case("qkv", 1, 4608, 9216, 3072, 32,
                       x_outlier_frac=0.005, x_outlier_scale=50.0,
                       w_outlier_frac=0.01, w_outlier_scale=8.0)


def mlp_cases():
    """MLP pair (seed 2): fc1 4608 x 3072 -> 12288 and fc2 12288 -> 3072, both
    rank 32, activation distribution of the tiny case (8 channels x40), plain
    weights.  Returns (fc1 LinearCase, W2 bits, b2 bits); fc2's activations
    are GELU(fc1 output) and are produced by whoever runs fc1."""
    M, K1, N1 = 4608, 3072, 12288
    rng = np.random.default_rng(2)
    X = rng.standard_normal((M, K1), dtype=np.float32)
    xi = np.sort(rng.choice(K1, 8, replace=False))
    X[:, xi] *= np.float32(40.0)
    W1 = rng.standard_normal((N1, K1), dtype=np.float32) * np.float32(0.02)
    b1 = rng.standard_normal(N1, dtype=np.float32) * np.float32(0.01)
    W2 = rng.standard_normal((K1, N1), dtype=np.float32) * np.float32(0.02)
    b2 = rng.standard_normal(K1, dtype=np.float32) * np.float32(0.01)
    fc1 = LinearCase(name="mlp_fc1", seed=2, M=M, N=N1, K=K1, rank=32,
                     X=f32_to_bf16_bits(X), W=f32_to_bf16_bits(W1),
                     bias=f32_to_bf16_bits(b1), x_outliers=xi)
    return fc1, f32_to_bf16_bits(W2), f32_to_bf16_bits(b2)


def lowres_case() -> LinearCase:
    """512x512 image (1024 tokens), 3072 -> 3072, rank 128, 2% of the
    activation channels x100 (seed 3)."""
    return linear_case("lowres", 3, 1024, 3072, 3072, 128,
                       x_outlier_frac=0.02, x_outlier_scale=100.0)


def awq_case(m_max: int = 16, N: int = 18432, K: int = 3072, seed: int = 4) -> AwqCase:
    """AWQ W4A16 modulation projection (6 x 3072 outputs), activations
    N(0,1) fp16, weights N(0, 0.02) rounded to fp16 (seed 4)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m_max, K), dtype=np.float32).astype(np.float16)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)).astype(np.float16)
    return AwqCase(name="awq", seed=seed, N=N, K=K, x=x, W=W)


def lora_factors(seed: int, N: int, K: int, rank: int, a_std: float = 0.02,
                 b_std: float = 0.02):
    """A user LoRA for a [N, K] linear layer: down factor A [rank, K] and up
    factor B [N, rank], both N(0, std) rounded to bf16 (A drawn first).
    Returns the two arrays of bf16 patterns."""
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((rank, K), dtype=np.float32) * np.float32(a_std)
    B = rng.standard_normal((N, rank), dtype=np.float32) * np.float32(b_std)
    return f32_to_bf16_bits(A), f32_to_bf16_bits(B)


def device_normal_bf16(M: int, K: int, seed: int, device, outlier_n: int = 0,
                       outlier_scale: float = 1.0):
    """Activations too large to draw on the host: N(0, 1) float32 from
    torch's generator on `device` (seeded), `outlier_n` channels (drawn with
    numpy's PCG64 from the same seed) scaled in float32, then rounded to
    bf16 (torch's cast: nearest, ties to even).  Returns (X bf16 tensor
    [M, K] on the device, outlier channel indices)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    X = torch.randn(M, K, generator=g, device=device, dtype=torch.float32)
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(K, outlier_n, replace=False)) if outlier_n > 0 else np.zeros(0, np.int64)
    if outlier_n > 0:
        X[:, torch.from_numpy(idx).to(device)] *= outlier_scale
    Xb = X.to(torch.bfloat16)
    del X
    return Xb, idx


def on_grid_case(seed: int, M: int, N: int, K: int, exp_lo: int = 0, exp_hi: int = 0,
                 group: int = 64) -> LinearCase:
    """Activations and weights that already lie on the signed INT4 grid: every
    group of 64 consecutive input channels of every row is ``2**e * c`` with
    integer codes c in [-7, 7], at least one code of magnitude 7, and a
    power-of-two ``2**e`` (e drawn in [exp_lo, exp_hi]).  Bias is zero.
    Rank 0; intended for use without smoothing."""
    rng = np.random.default_rng(seed)

    def grid(rows):
        g = K // group
        c = rng.integers(-7, 8, size=(rows, g, group)).astype(np.float32)
        pos = rng.integers(0, group, size=(rows, g))
        sign = np.where(rng.integers(0, 2, size=(rows, g)) == 0, -1.0, 1.0).astype(np.float32)
        np.put_along_axis(c, pos[..., None], (7.0 * sign)[..., None], axis=2)
        e = rng.integers(exp_lo, exp_hi + 1, size=(rows, g, 1)).astype(np.float32)
        v = c * np.exp2(e)
        return f32_to_bf16_bits(v.reshape(rows, K).astype(np.float32))

    X = grid(M)
    W = grid(N)
    return LinearCase(name=f"ongrid_{seed}", seed=seed, M=M, N=N, K=K, rank=0,
                      X=X, W=W, bias=np.zeros(N, np.uint16))


WORKLOADS = {
    "tiny": "tiny SVDQuant linear 256x512->512 r16",
    "qkv": "Flux-like fused QKV 4608x3072->9216 r32",
    "mlp": "Flux-like MLP fc1 4608x3072->12288, GELU, fc2 4608x12288->3072, r32",
    "lowres": "low-res high-rank 1024x3072->3072 r128",
    "awq": "AWQ W4A16 modulation M<=16 x3072->18432",
}
