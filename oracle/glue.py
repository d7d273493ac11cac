"""CPU oracle: the activation between the two projections of the MLP pair.

TEST INFRASTRUCTURE (same import rule as ``oracle.svdquant``).

Source.  "Bringing Nunchaku 4-bit diffusion inference to Diffusers"
(Vietnamese edition, section "Giới thiệu Nunchaku Lite") credits part of the
original engine's speed to fused GELU/MLP kernels.  The pages do not say which
GELU; the reading used is the tanh form

    gelu(y) = 0.5 y (1 + tanh( sqrt(2/pi) (y + 0.044715 y^3) ))

evaluated in float64 and rounded once to bfloat16 (the MLP's activations are
bf16).  It is computed in the algebraically identical logistic form
y * sigma(2u) = y / (1 + exp(-2u)): the printed form's 1 + tanh(u) cancels
for large negative y and loses all relative accuracy there.  Parity status:
pinned by the CPU tests (identities, a library routine, and the erf form).
"""
from __future__ import annotations

import numpy as np

from .svdquant import round_to_bf16

SQRT_2_OVER_PI = np.sqrt(2.0 / np.pi)
GELU_CUBIC = 0.044715


def gelu_tanh(y: np.ndarray) -> np.ndarray:
    y = np.asarray(y, dtype=np.float64)
    u = SQRT_2_OVER_PI * (y + GELU_CUBIC * y ** 3)
    with np.errstate(over="ignore"):
        return y / (1.0 + np.exp(-2.0 * u))      # = 0.5 y (1 + tanh u)


def gelu_tanh_bf16(y: np.ndarray) -> np.ndarray:
    """gelu_tanh rounded to bfloat16 values (float64 container)."""
    return round_to_bf16(gelu_tanh(y))
