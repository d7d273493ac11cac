"""CPU oracle: a user LoRA merged into the SVDQuant layer's low-rank branch.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the product library never
does and shares no code with it.  Parity status: pinned by
``tests/test_oracle_lora.py`` (a rank-1 LoRA that copies one input channel
into one output, the merged layer against torch's two-linear LoRA forward in
float64, cancellation of a LoRA by its negative, a LoRA equal to the base
branch doubling that branch, r' = 0 as the identity, and the base layer's
quantised path left untouched).

Sources.  "Bringing Nunchaku 4-bit diffusion inference to Diffusers"
(Vietnamese edition, section "Tải nguyên bản trong Diffusers"; Russian
edition, closing paragraph) keep LoRA loading working on a quantised model,
and the Hacker News thread "SVDQuant: 4-Bit Quantization Powers 12B Flux on a
16GB 4090 GPU with 3x Speedup" describes the 16-bit branch as a LoRA in all
but name.  The pages do not say how a user LoRA meets the branch.  The
reading here: a LoRA with down factor A [r', K], up factor B [N, r'] and
scale alpha adds alpha (X A^T) B^T to Y; it rides on the branch by
concatenation,

    L1s' = [L1s | A^T]                 [K, r + r']
    L2'  = [L2 ; bf16(fl32(alpha B^T))] [r + r', N]

with the scaled up factor formed in float32 and stored as bf16 like the
branch itself.  A acts on the raw activations (the smoothing already sits
inside L1s; a LoRA knows nothing of it).  Everything else of the layer
(smoothing factors, residual codes and scales, bias) is unchanged, so the
4-bit path is bit-for-bit the base layer's.
"""
from __future__ import annotations

import numpy as np

from . import svdquant as O

F32 = np.float32


def scaled_up_factor(B_bits: np.ndarray, alpha: float) -> np.ndarray:
    """bf16(fl32(alpha * B))^T as float64 values [r', N]: one float32
    product per element, then one round to bf16."""
    B = O.bf16_values(B_bits).astype(F32)              # exact: bf16 values are float32 values
    prod = (F32(alpha) * B).astype(F32)                # IEEE float32 product
    return O.round_to_bf16(prod.astype(np.float64)).T


def merge(prep: dict, A_bits: np.ndarray, B_bits: np.ndarray, alpha: float) -> dict:
    """A prepared layer (``svdquant.prepare`` or ``mxfp4.prepare``) with the
    LoRA (A [r', K] bf16 patterns, B [N, r'] bf16 patterns, scale alpha)
    concatenated onto its low-rank branch.  The input dict is not modified."""
    A = O.bf16_values(A_bits)
    r2, K = A.shape
    N = prep["N"]
    assert K == prep["K"] and B_bits.shape == (N, r2)
    out = dict(prep)
    out["L1s"] = np.concatenate([prep["L1s"], A.T], axis=1)
    out["L2b"] = np.concatenate([prep["L2b"], scaled_up_factor(B_bits, alpha)], axis=0)
    out["rank"] = prep["rank"] + r2
    return out
