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
