"""CPU oracle: the activation between the two projections of the MLP pair.

TEST INFRASTRUCTURE (same import rule as ``oracle.svdquant``).

Source.  "Bringing Nunchaku 4-bit diffusion inference to Diffusers"
(Vietnamese edition, section "Giới thiệu Nunchaku Lite") credits part of the
original engine's speed to fused GELU/MLP kernels.  The pages do not say which
GELU; the reading used is the tanh form

    gelu(y) = 0.5 y (1 + tanh( sqrt(2/pi) (y + 0.044715 y^3) ))

evaluated in float64 and rounded once to bfloat16 (the MLP's activations are
bf16).  Parity status: pinned by the CPU tests (identities, a library
routine, and the erf form).
"""
from __future__ import annotations

import numpy as np

from .svdquant import round_to_bf16

SQRT_2_OVER_PI = np.sqrt(2.0 / np.pi)
GELU_CUBIC = 0.044715


def gelu_tanh(y: np.ndarray) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(SQRT_2_OVER_PI * (y + GELU_CUBIC * y ** 3)))


def gelu_tanh_bf16(y: np.ndarray) -> np.ndarray:
    """gelu_tanh rounded to bfloat16 values (float64 container)."""
    return round_to_bf16(gelu_tanh(y))
