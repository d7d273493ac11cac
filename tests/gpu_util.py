"""Helpers for the GPU parity tests: move oracle-prepared layers and seeded
inputs onto the device through the library's own packer.  The device path
never sees anything the oracle did not produce from the seeded inputs."""
import numpy as np
import torch

from oracle import svdquant as O


def host_from_oracle(ref: dict):
    import w4a4_rank_corrected_smooth_amd as S
    return S.PreparedHost(ref["N"], ref["K"], ref["rank"], ref["iota"].astype(np.float32),
                          O.bf16_bits_of(ref["L1s"]), O.bf16_bits_of(ref["L2b"]),
                          O.pack_int4(ref["qW"]), ref["sW"].astype(np.float32),
                          ref["bias"].astype(np.float32))


def layer_from_oracle(ref: dict, device="cuda"):
    import w4a4_rank_corrected_smooth_amd as S
    return S.Linear(host_from_oracle(ref), device)


def bf16_to_device(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def mx_host_from_oracle(ref: dict):
    """An MXFP4 layer's host arrays from the oracle's prepared dict."""
    import w4a4_rank_corrected_smooth_amd as S
    from oracle import mxfp4 as MX
    return S.PreparedHostMx(ref["N"], ref["K"], ref["rank"], ref["iota"].astype(np.float32),
                            O.bf16_bits_of(ref["L1s"]), O.bf16_bits_of(ref["L2b"]),
                            MX.pack_fp4(ref["qW"]), (ref["eW"] + 127).astype(np.uint8),
                            ref["bias"].astype(np.float32))


def mx_layer_from_oracle(ref: dict, device="cuda"):
    import w4a4_rank_corrected_smooth_amd as S
    return S.MxLinear(mx_host_from_oracle(ref), device)


def _up256(x: int) -> int:
    return -(-x // 256) * 256


SCALE_OP_BYTES = 16


def workspace_regions(M: int, K: int):
    """Byte offsets of the INT4 workspace's code and scale regions (the
    device layout: fp6 code blocks [G][Mp/32] x 1536, then the scales as
    16-byte matrix operands [G][Mp], each region 256-byte aligned)."""
    Mp, G = _up256(M), K // 64
    sa_off = _up256(Mp * K * 3 // 4)
    d_off = _up256(sa_off + G * Mp * SCALE_OP_BYTES)
    return Mp, G, sa_off, d_off


def scale_from_operand(words: np.ndarray) -> np.ndarray:
    """fp32 scales from their 16-byte operand form (bf16 slots a1 a1 a1 a2 a2
    a2 a3 a3): s = a1 + a2 + a3, exact in float32 (test-side reader of the
    documented layout)."""
    w = np.asarray(words, dtype=np.uint8).reshape(-1, 8).view(np.uint16).reshape(-1, 8)
    a = (w.astype(np.uint32) << 16).view(np.float32)
    return ((a[:, 0] + a[:, 3]) + a[:, 6]).astype(np.float32)


def decode_fp6_codes(ws: np.ndarray, M: int, K: int) -> np.ndarray:
    """INT4 activation codes [M, K] (int) from a workspace's fp6 blocks.

    Test-side reader of the documented layout: for every (group g, tile t
    of 32 rows) a 1536-byte block; lane l covers row 32 t + l % 32 and half
    h = l / 32 of the group; its 8-byte word pair j (j = 0..2) sits at byte
    512 j + 8 l; its code c occupies bits 6c..6c+5 of the 24 bytes and is
    input channel 64 g + 16 (c / 8) + 8 h + c % 8, an OCP FP6 E2M3 value
    (sign bit 5, exponent bits 4..3 with bias 1, mantissa bits 2..0)."""
    Mp, G, _, _ = workspace_regions(M, K)
    T = Mp // 32
    raw = np.asarray(ws[: G * T * 1536], dtype=np.uint8).reshape(G, T, 3, 64, 8)
    lane_bytes = raw.transpose(0, 1, 3, 2, 4).reshape(G, T, 64, 24)
    bits = np.unpackbits(lane_bytes, axis=-1, bitorder="little").reshape(G, T, 64, 32, 6)
    v = (bits.astype(np.int64) << np.arange(6)).sum(axis=-1)          # fp6 code
    e, m = (v >> 3) & 3, v & 7
    mag = np.where(e == 0, m / 8.0, (1.0 + m / 8.0) * np.exp2(e - 1.0))
    val = np.where(v & 0x20, -mag, mag)
    out = np.zeros((Mp, K), np.float64)
    lane = np.arange(64)
    c = np.arange(32)
    rows = (np.arange(T)[:, None, None] * 32 + (lane % 32)[None, :, None])      # [T, 64, 1]
    for g in range(G):
        ks = 64 * g + 16 * (c[None, :] // 8) + 8 * (lane[:, None] // 32) + c[None, :] % 8   # [64, 32]
        out[np.broadcast_to(rows, (T, 64, 32)), np.broadcast_to(ks[None], (T, 64, 32))] = val[g]
    out = out[:M]                       # padding rows are not written by every kernel
    assert np.all(out == np.rint(out)), "a code is not an integer"
    return out.astype(np.int64)


def decode_scales(ws: np.ndarray, M: int, K: int) -> np.ndarray:
    """fp32 activation scales [M, K/64] from a workspace's [G][Mp] operand region."""
    Mp, G, sa_off, _ = workspace_regions(M, K)
    raw = np.asarray(ws[sa_off: sa_off + G * Mp * SCALE_OP_BYTES], dtype=np.uint8).reshape(G, Mp, 16)
    return scale_from_operand(raw[:, :M].reshape(-1)).reshape(G, M).T.copy()
