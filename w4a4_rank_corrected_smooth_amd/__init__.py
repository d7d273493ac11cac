"""Python binding of libsvdq: the SVDQuant W4A4 + low-rank linear layer and
the AWQ W4A16 linear on MI355X (gfx950).

This module only marshals arguments into the C ABI declared in
``include/svdq.h``: every step of the method runs in the library (host
preparation in C++, the forward in HIP kernels).  PyTorch supplies device
memory and streams.  Importing fails loudly when the library is missing;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch  # loaded first so the library binds to the HIP runtime torch uses

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvdq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python w4a4_rank_corrected_smooth_amd/build.py` (hipcc, gfx950)")
_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

OK = 0
STATUS = {0: "SVDQ_OK", 1: "SVDQ_ERR_INVALID_ARGUMENT", 2: "SVDQ_ERR_UNSUPPORTED_SHAPE",
          3: "SVDQ_ERR_NO_DEVICE", 4: "SVDQ_ERR_UNSUPPORTED_DEVICE",
          5: "SVDQ_ERR_WORKSPACE_TOO_SMALL", 6: "SVDQ_ERR_NUMERICAL", 7: "SVDQ_ERR_HIP"}
BF16, FP16, FP32 = 0, 1, 2
EPILOGUE_NONE, EPILOGUE_GELU_TANH = 0, 1

EXPORTS = [
    "svdq_abi_version", "svdq_status_string", "svdq_last_error", "svdq_device_check",
    "svdq_host_weights_sizes", "svdq_calibration_absmax", "svdq_prepare_weights",
    "svdq_device_weights_bytes", "svdq_pack_device_weights", "svdq_workspace_bytes",
    "svdq_linear_forward", "svdq_linear_forward_static", "svdq_linear_quantize",
    "svdq_unfused_workspace_bytes", "svdq_linear_forward_unfused", "svdq_linear_gemm", "svdq_mlp_forward",
    "svdq_mlp_quantize", "svdq_mlp_gemm1", "svdq_mlp_gemm2", "svdq_gelu_tanh_bf16",
    "svdq_quantize_activations",
    "svdq_debug_group_sums", "svdq_debug_group_sums_codes", "awq_quantize_weights", "awq_device_weights_bytes",
    "awq_pack_device_weights", "awq_w4a16_forward",
    "svdq_mx_host_weights_sizes", "svdq_mx_prepare_weights", "svdq_mx_device_weights_bytes",
    "svdq_mx_pack_device_weights", "svdq_mx_workspace_bytes", "svdq_mx_linear_forward",
    "svdq_mx_linear_quantize", "svdq_mx_linear_gemm", "svdq_mx_quantize_activations",
    "svdq_merge_lora", "svdq_mx_merge_lora", "svdq_measure_stream", "svdq_measure_mfma",
]


class HostWeights(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("inv_lambda", _vp), ("l1s", _vp), ("l2", _vp),
                ("qweight", _vp), ("wscales", _vp), ("bias", _vp)]


class MxHostWeights(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int32), ("K", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("inv_lambda", _vp), ("l1s", _vp), ("l2", _vp), ("qweight", _vp),
                ("wscales", _vp), ("bias", _vp)]


class DeviceWeights(ctypes.Structure):
    _fields_ = [("blob", _vp), ("N", ctypes.c_int32), ("K", ctypes.c_int32),
                ("rank", ctypes.c_int32)]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = args


_sig("svdq_abi_version", _i, [])
_sig("svdq_status_string", ctypes.c_char_p, [_i])
_sig("svdq_last_error", ctypes.c_char_p, [])
_sig("svdq_device_check", _i, [])
_sig("svdq_host_weights_sizes", _i, [_i, _i, _i, ctypes.POINTER(_sz)])
_sig("svdq_calibration_absmax", _i, [_vp, _i, _i, _vp])
_sig("svdq_prepare_weights", _i, [_vp, _i, _i, _vp, _vp, _i, _i, ctypes.POINTER(HostWeights)])
_sig("svdq_device_weights_bytes", _sz, [_i, _i, _i])
_sig("svdq_pack_device_weights", _i, [ctypes.POINTER(HostWeights), _vp, _sz])
_sig("svdq_workspace_bytes", _sz, [_i, _i, _i, _i])
_sig("svdq_linear_forward", _i, [ctypes.POINTER(DeviceWeights), _vp, _i, _vp, _i, _i, _vp, _sz, _vp])
_sig("svdq_linear_forward_static", _i, [ctypes.POINTER(DeviceWeights), _vp, _i, _vp, _i, _i, _vp])
_sig("svdq_unfused_workspace_bytes", _sz, [_i, _i, _i, _i])
_sig("svdq_linear_forward_unfused", _i, [ctypes.POINTER(DeviceWeights), _vp, _i, _vp, _i, _i, _vp, _sz, _vp])
_sig("svdq_linear_quantize", _i, [ctypes.POINTER(DeviceWeights), _vp, _i, _vp, _sz, _vp])
_sig("svdq_linear_gemm", _i, [ctypes.POINTER(DeviceWeights), _i, _vp, _i, _i, _vp, _sz, _vp])
_sig("svdq_gelu_tanh_bf16", _i, [_vp, _vp, _sz, _vp])
_W = ctypes.POINTER(DeviceWeights)
_sig("svdq_mlp_forward", _i, [_W, _W, _vp, _i, _vp, _i, _i, _vp, _sz, _vp, _sz, _vp])
_sig("svdq_mlp_quantize", _i, [_W, _W, _vp, _i, _vp, _sz, _vp, _sz, _vp])
_sig("svdq_mlp_gemm1", _i, [_W, _W, _i, _i, _vp, _sz, _vp, _sz, _vp])
_sig("svdq_mlp_gemm2", _i, [_W, _i, _vp, _i, _vp, _sz, _vp])
_sig("svdq_quantize_activations", _i, [ctypes.POINTER(DeviceWeights), _vp, _i, _vp, _vp, _vp,
                                       _vp, _sz, _vp])
_sig("svdq_debug_group_sums", _i, [ctypes.POINTER(DeviceWeights), _i, _i, _i, _i, _i, _vp, _vp,
                                   _sz, _vp])
_sig("svdq_debug_group_sums_codes", _i, [ctypes.POINTER(DeviceWeights), _vp, _i, _i, _i, _i, _i,
                                         _vp, _vp, _sz, _vp])
_sig("awq_quantize_weights", _i, [_vp, _i, _i, _i, _vp, _vp, _vp])
_sig("awq_device_weights_bytes", _sz, [_i, _i])
_sig("awq_pack_device_weights", _i, [_vp, _vp, _vp, _i, _i, _vp, _sz])
_sig("awq_w4a16_forward", _i, [_vp, _i, _i, _vp, _i, _vp, _vp, _vp])
_sig("svdq_mx_host_weights_sizes", _i, [_i, _i, _i, ctypes.POINTER(_sz)])
_sig("svdq_mx_prepare_weights", _i, [_vp, _i, _i, _vp, _vp, _i, ctypes.POINTER(MxHostWeights)])
_sig("svdq_mx_device_weights_bytes", _sz, [_i, _i, _i])
_sig("svdq_mx_pack_device_weights", _i, [ctypes.POINTER(MxHostWeights), _vp, _sz])
_sig("svdq_mx_workspace_bytes", _sz, [_i, _i, _i, _i])
_sig("svdq_mx_linear_forward", _i, [_W, _vp, _i, _vp, _i, _i, _vp, _sz, _vp])
_sig("svdq_mx_linear_quantize", _i, [_W, _vp, _i, _vp, _sz, _vp])
_sig("svdq_mx_linear_gemm", _i, [_W, _i, _vp, _i, _i, _vp, _sz, _vp])
_sig("svdq_mx_quantize_activations", _i, [_W, _vp, _i, _vp, _vp, _vp, _vp, _sz, _vp])
_sig("svdq_measure_stream", _i, [_vp, _vp, _sz, _i, _i, _vp, _vp])
_sig("svdq_measure_mfma", _i, [_i, _i, _i, _vp, _vp])
_sig("svdq_merge_lora", _i, [ctypes.POINTER(HostWeights), _vp, _vp, _i, ctypes.c_float,
                             ctypes.POINTER(HostWeights)])
_sig("svdq_mx_merge_lora", _i, [ctypes.POINTER(MxHostWeights), _vp, _vp, _i, ctypes.c_float,
                                ctypes.POINTER(MxHostWeights)])


class SvdqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.svdq_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS.get(status, status)}: {msg}")


def _check(status: int, where: str) -> None:
    if status != OK:
        raise SvdqError(status, where)


def _check_out(out: torch.Tensor, M: int, N: int, device, dtypes=(torch.bfloat16, torch.float32)) -> None:
    """A caller-supplied output must be a contiguous [M, N] tensor of an
    accepted dtype on the inputs' device: the kernels write exactly M * N
    elements of that type."""
    if not isinstance(out, torch.Tensor):
        raise TypeError("out must be a torch.Tensor")
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {(M, N)}")
    if out.dtype not in dtypes:
        raise ValueError(f"out has dtype {out.dtype}, expected one of {dtypes}")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if out.device != torch.device(device):
        raise ValueError(f"out is on {out.device}, expected {device}")


def _check_bias(bias: torch.Tensor, N: int, device) -> None:
    if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float16 or bias.numel() != N \
            or not bias.is_contiguous() or bias.device != torch.device(device):
        raise ValueError(f"bias must be a contiguous float16 tensor of {N} elements on {device}")


def _ptr(a) -> Optional[int]:
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        return a.data_ptr()
    return a.ctypes.data


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def abi_version() -> int:
    return _lib.svdq_abi_version()


def device_check() -> None:
    _check(_lib.svdq_device_check(), "svdq_device_check")


# ------------------------------------------------------------ offline, host
@dataclass
class PreparedHost:
    """Output of svdq_prepare_weights (host numpy arrays, canonical layouts)."""
    N: int
    K: int
    rank: int
    inv_lambda: np.ndarray   # float32 [K]
    l1s: np.ndarray          # uint16 (bf16) [K, rank]
    l2: np.ndarray           # uint16 (bf16) [rank, N]
    qweight: np.ndarray      # uint8 [N, K/2]
    wscales: np.ndarray      # float32 [N, K/64]
    bias: np.ndarray         # float32 [N]

    def __post_init__(self):
        # the C side reads row-major buffers of exactly these types
        self.inv_lambda = np.ascontiguousarray(self.inv_lambda, dtype=np.float32)
        self.l1s = np.ascontiguousarray(self.l1s, dtype=np.uint16)
        self.l2 = np.ascontiguousarray(self.l2, dtype=np.uint16)
        self.qweight = np.ascontiguousarray(self.qweight, dtype=np.uint8)
        self.wscales = np.ascontiguousarray(self.wscales, dtype=np.float32)
        self.bias = np.ascontiguousarray(self.bias, dtype=np.float32)

    def as_struct(self) -> HostWeights:
        return HostWeights(self.N, self.K, self.rank, 64, _ptr(self.inv_lambda),
                           _ptr(self.l1s) if self.rank else None,
                           _ptr(self.l2) if self.rank else None, _ptr(self.qweight),
                           _ptr(self.wscales), _ptr(self.bias))


def calibration_absmax(X_bits: np.ndarray) -> np.ndarray:
    X_bits = np.ascontiguousarray(X_bits, dtype=np.uint16)
    rows, K = X_bits.shape
    out = np.empty(K, np.float32)
    _check(_lib.svdq_calibration_absmax(_ptr(X_bits), rows, K, _ptr(out)), "svdq_calibration_absmax")
    return out


def prepare_weights(W_bits: np.ndarray, act_absmax: Optional[np.ndarray],
                    bias_bits: Optional[np.ndarray], rank: int) -> PreparedHost:
    """Host preparation (smoothing, top-r SVD split, residual INT4 quantisation)."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    ax = None if act_absmax is None else np.ascontiguousarray(act_absmax, dtype=np.float32)
    b = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
    G = max(K // 64, 1)
    out = PreparedHost(N, K, rank, np.empty(K, np.float32), np.empty((K, rank), np.uint16),
                       np.empty((rank, N), np.uint16), np.empty((N, max(K // 2, 1)), np.uint8),
                       np.empty((N, G), np.float32), np.empty(N, np.float32))
    hw = out.as_struct()
    _check(_lib.svdq_prepare_weights(_ptr(W_bits), N, K, _ptr(ax), _ptr(b), rank, 64,
                                     ctypes.byref(hw)), "svdq_prepare_weights")
    return out


def device_weights_bytes(N: int, K: int, rank: int) -> int:
    return _lib.svdq_device_weights_bytes(N, K, rank)


def pack_device_weights(hw: PreparedHost) -> np.ndarray:
    n = device_weights_bytes(hw.N, hw.K, hw.rank)
    if n == 0:
        raise SvdqError(2, "svdq_device_weights_bytes")
    blob = np.empty(n, np.uint8)
    s = hw.as_struct()
    _check(_lib.svdq_pack_device_weights(ctypes.byref(s), _ptr(blob), n), "svdq_pack_device_weights")
    return blob


def _lora_args(hw, A_bits, B_bits):
    A = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B = np.ascontiguousarray(B_bits, dtype=np.uint16)
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != hw.K or B.shape != (hw.N, A.shape[0]):
        raise ValueError(f"LoRA factors must be A [r', K={hw.K}] and B [N={hw.N}, r'], "
                         f"got {A.shape} and {B.shape}")
    return A, B, A.shape[0]


def merge_lora(hw: PreparedHost, A_bits: np.ndarray, B_bits: np.ndarray,
               alpha: float = 1.0) -> PreparedHost:
    """A user LoRA (down A [r', K], up B [N, r'], bf16 patterns) concatenated
    onto the low-rank branch of `hw` (svdq_merge_lora).  The 4-bit arrays are
    shared with `hw`, not copied; `hw` is unchanged."""
    A, B, r2 = _lora_args(hw, A_bits, B_bits)
    rt = hw.rank + r2
    out = PreparedHost(hw.N, hw.K, rt, hw.inv_lambda, np.empty((hw.K, rt), np.uint16),
                       np.empty((rt, hw.N), np.uint16), hw.qweight, hw.wscales, hw.bias)
    src, dst = hw.as_struct(), out.as_struct()
    _check(_lib.svdq_merge_lora(ctypes.byref(src), _ptr(A), _ptr(B), r2, float(alpha),
                                ctypes.byref(dst)), "svdq_merge_lora")
    return out


class Linear:
    """A prepared SVDQuant layer resident on one device."""

    def __init__(self, hw: PreparedHost, device="cuda"):
        self.N, self.K, self.rank = hw.N, hw.K, hw.rank
        self.blob = torch.from_numpy(pack_device_weights(hw)).to(device)
        self.device = self.blob.device
        self._w = DeviceWeights(self.blob.data_ptr(), self.N, self.K, self.rank)

    def workspace_bytes(self, M: int) -> int:
        return workspace_bytes(M, self.N, self.K, self.rank)

    def new_workspace(self, M: int) -> torch.Tensor:
        return torch.empty(self.workspace_bytes(M), dtype=torch.uint8, device=self.device)


def workspace_bytes(M: int, N: int, K: int, rank: int) -> int:
    n = _lib.svdq_workspace_bytes(M, N, K, rank)
    if n == 0:
        raise SvdqError(2, "svdq_workspace_bytes")
    return n


# ------------------------------------------------------------- device calls
def linear_forward(layer: Linear, X: torch.Tensor, out: Optional[torch.Tensor] = None,
                   out_dtype=torch.bfloat16, gelu: bool = False,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X W^T + b through the SVDQuant path (optionally gelu_tanh(Y))."""
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and X.shape[1] == layer.K
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, layer.N), dtype=out_dtype, device=X.device)
    _check_out(out, M, layer.N, X.device)
    if workspace is None:
        workspace = layer.new_workspace(M)
    dt = FP32 if out.dtype == torch.float32 else BF16
    _check(_lib.svdq_linear_forward(ctypes.byref(layer._w), X.data_ptr(), M, out.data_ptr(), dt,
                                    EPILOGUE_GELU_TANH if gelu else EPILOGUE_NONE,
                                    workspace.data_ptr(), workspace.numel(), _stream(X.device)),
           "svdq_linear_forward")
    return out


def unfused_workspace_bytes(M: int, N: int, K: int, rank: int) -> int:
    n = _lib.svdq_unfused_workspace_bytes(M, N, K, rank)
    if n == 0:
        raise SvdqError(2, "svdq_unfused_workspace_bytes")
    return n


def linear_forward_unfused(layer: Linear, X: torch.Tensor, out: Optional[torch.Tensor] = None,
                           out_dtype=torch.bfloat16, gelu: bool = False,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """svdq_linear_forward_unfused: the forward with the low-rank branch as
    two separate bf16 GEMMs (the fusion ablation)."""
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and X.shape[1] == layer.K
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, layer.N), dtype=out_dtype, device=X.device)
    _check_out(out, M, layer.N, X.device)
    if workspace is None:
        workspace = torch.empty(unfused_workspace_bytes(M, layer.N, layer.K, layer.rank),
                                dtype=torch.uint8, device=X.device)
    dt = FP32 if out.dtype == torch.float32 else BF16
    _check(_lib.svdq_linear_forward_unfused(ctypes.byref(layer._w), X.data_ptr(), M, out.data_ptr(), dt,
                                            EPILOGUE_GELU_TANH if gelu else EPILOGUE_NONE,
                                            workspace.data_ptr(), workspace.numel(), _stream(X.device)),
           "svdq_linear_forward_unfused")
    return out


STATIC_SCRATCH_BYTES = 64 << 20     # SVDQ_STATIC_SCRATCH_BYTES


def linear_forward_static(layer: Linear, X: torch.Tensor, out: torch.Tensor,
                          gelu: bool = False) -> torch.Tensor:
    """svdq_linear_forward_static: the forward with the library's own device
    scratch array as workspace (no allocation in the call); `out` is the
    caller's [M, N] bf16 or fp32 tensor."""
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and X.shape[1] == layer.K
    _check_out(out, X.shape[0], layer.N, X.device)
    dt = FP32 if out.dtype == torch.float32 else BF16
    _check(_lib.svdq_linear_forward_static(ctypes.byref(layer._w), X.data_ptr(), X.shape[0],
                                           out.data_ptr(), dt,
                                           EPILOGUE_GELU_TANH if gelu else EPILOGUE_NONE,
                                           _stream(X.device)), "svdq_linear_forward_static")
    return out


def linear_quantize(layer: Linear, X: torch.Tensor, workspace: torch.Tensor) -> None:
    """Kernel (1) of the forward alone: fills `workspace` from X."""
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and X.shape[1] == layer.K
    _check(_lib.svdq_linear_quantize(ctypes.byref(layer._w), X.data_ptr(), X.shape[0],
                                     workspace.data_ptr(), workspace.numel(), _stream(X.device)),
           "svdq_linear_quantize")


def linear_gemm(layer: Linear, M: int, out: torch.Tensor, workspace: torch.Tensor,
                gelu: bool = False) -> torch.Tensor:
    """Kernel (2) of the forward alone, from a workspace filled by linear_quantize."""
    _check_out(out, M, layer.N, workspace.device)
    dt = FP32 if out.dtype == torch.float32 else BF16
    _check(_lib.svdq_linear_gemm(ctypes.byref(layer._w), M, out.data_ptr(), dt,
                                 EPILOGUE_GELU_TANH if gelu else EPILOGUE_NONE,
                                 workspace.data_ptr(), workspace.numel(), _stream(out.device)),
           "svdq_linear_gemm")
    return out


def mlp_forward(l1: Linear, l2: Linear, X: torch.Tensor, out: Optional[torch.Tensor] = None,
                out_dtype=torch.bfloat16, gelu: bool = True,
                ws1: Optional[torch.Tensor] = None, ws2: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = l2(bf16(gelu_tanh(l1(X)))) with l1's GEMM quantising l2's input in
    its epilogue (the intermediate never goes to memory)."""
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and X.shape[1] == l1.K
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, l2.N), dtype=out_dtype, device=X.device)
    _check_out(out, M, l2.N, X.device)
    ws1 = l1.new_workspace(M) if ws1 is None else ws1
    ws2 = l2.new_workspace(M) if ws2 is None else ws2
    dt = FP32 if out.dtype == torch.float32 else BF16
    _check(_lib.svdq_mlp_forward(ctypes.byref(l1._w), ctypes.byref(l2._w), X.data_ptr(), M,
                                 out.data_ptr(), dt, EPILOGUE_GELU_TANH if gelu else EPILOGUE_NONE,
                                 ws1.data_ptr(), ws1.numel(), ws2.data_ptr(), ws2.numel(),
                                 _stream(X.device)), "svdq_mlp_forward")
    return out


def mlp_quantize(l1: Linear, l2: Linear, X: torch.Tensor, ws1: torch.Tensor,
                 ws2: torch.Tensor) -> None:
    """First kernel of mlp_forward: l1's quantiser (and clearing l2's D)."""
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and X.shape[1] == l1.K
    _check(_lib.svdq_mlp_quantize(ctypes.byref(l1._w), ctypes.byref(l2._w), X.data_ptr(), X.shape[0],
                                  ws1.data_ptr(), ws1.numel(), ws2.data_ptr(), ws2.numel(),
                                  _stream(X.device)), "svdq_mlp_quantize")


def mlp_gemm1(l1: Linear, l2: Linear, M: int, ws1: torch.Tensor, ws2: torch.Tensor,
              gelu: bool = True) -> None:
    """Second kernel of mlp_forward: l1's GEMM, writing l2's codes, scales and D."""
    _check(_lib.svdq_mlp_gemm1(ctypes.byref(l1._w), ctypes.byref(l2._w), M,
                               EPILOGUE_GELU_TANH if gelu else EPILOGUE_NONE,
                               ws1.data_ptr(), ws1.numel(), ws2.data_ptr(), ws2.numel(),
                               _stream(ws1.device)), "svdq_mlp_gemm1")


def mlp_gemm2(l2: Linear, M: int, out: torch.Tensor, ws2: torch.Tensor) -> torch.Tensor:
    """Third kernel of mlp_forward: l2's GEMM from the workspace mlp_gemm1 filled."""
    _check_out(out, M, l2.N, ws2.device)
    dt = FP32 if out.dtype == torch.float32 else BF16
    _check(_lib.svdq_mlp_gemm2(ctypes.byref(l2._w), M, out.data_ptr(), dt, ws2.data_ptr(),
                               ws2.numel(), _stream(out.device)), "svdq_mlp_gemm2")
    return out


def gelu_tanh_bf16(x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    assert x.dtype == torch.bfloat16 and x.is_contiguous()
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != torch.bfloat16 or not out.is_contiguous() \
            or out.device != x.device:
        raise ValueError("out must be a contiguous bf16 tensor shaped like the input")
    _check(_lib.svdq_gelu_tanh_bf16(x.data_ptr(), out.data_ptr(), x.numel(), _stream(x.device)),
           "svdq_gelu_tanh_bf16")
    return out


def quantize_activations(layer: Linear, X: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Canonical-layout export of the quantiser kernel: (codes uint8 [M, K/2],
    scales float32 [M, K/64], low-rank down float32 [M, rank])."""
    M = X.shape[0]
    dev = X.device
    q = torch.empty((M, layer.K // 2), dtype=torch.uint8, device=dev)
    s = torch.empty((M, layer.K // 64), dtype=torch.float32, device=dev)
    d = torch.empty((M, max(layer.rank, 1)), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = layer.new_workspace(M)
    _check(_lib.svdq_quantize_activations(ctypes.byref(layer._w), X.data_ptr(), M, q.data_ptr(),
                                          s.data_ptr(), d.data_ptr(), workspace.data_ptr(),
                                          workspace.numel(), _stream(dev)),
           "svdq_quantize_activations")
    return q, s, d[:, :layer.rank]


def debug_group_sums(layer: Linear, M: int, m0: int, mcount: int, n0: int, ncount: int,
                     workspace: torch.Tensor) -> torch.Tensor:
    P = torch.empty((mcount, ncount, layer.K // 64), dtype=torch.int32, device=workspace.device)
    _check(_lib.svdq_debug_group_sums(ctypes.byref(layer._w), M, m0, mcount, n0, ncount,
                                      P.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                      _stream(workspace.device)), "svdq_debug_group_sums")
    return P


def debug_group_sums_codes(layer: Linear, qact: torch.Tensor, m0: int, mcount: int, n0: int,
                           ncount: int, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact group sums of caller-supplied canonical activation codes qact
    (uint8 [M, K/2] on the device) against the layer's weight codes."""
    assert qact.dtype == torch.uint8 and qact.is_contiguous() and qact.dim() == 2
    assert qact.shape[1] == layer.K // 2 and qact.device.type == "cuda"
    M = qact.shape[0]
    if workspace is None:
        workspace = layer.new_workspace(M)
    P = torch.empty((mcount, ncount, layer.K // 64), dtype=torch.int32, device=qact.device)
    _check(_lib.svdq_debug_group_sums_codes(ctypes.byref(layer._w), qact.data_ptr(), M, m0, mcount,
                                            n0, ncount, P.data_ptr(), workspace.data_ptr(),
                                            workspace.numel(), _stream(qact.device)),
           "svdq_debug_group_sums_codes")
    return P


# ------------------------------------------------------------ MXFP4 variant
@dataclass
class PreparedHostMx:
    """Output of svdq_mx_prepare_weights (host numpy arrays, canonical layouts)."""
    N: int
    K: int
    rank: int
    inv_lambda: np.ndarray   # float32 [K]
    l1s: np.ndarray          # uint16 (bf16) [K, rank]
    l2: np.ndarray           # uint16 (bf16) [rank, N]
    qweight: np.ndarray      # uint8 [N, K/2] E2M1 codes
    wscales: np.ndarray      # uint8 [N, K/32] E8M0
    bias: np.ndarray         # float32 [N]

    def __post_init__(self):
        # the C side reads row-major buffers of exactly these types
        self.inv_lambda = np.ascontiguousarray(self.inv_lambda, dtype=np.float32)
        self.l1s = np.ascontiguousarray(self.l1s, dtype=np.uint16)
        self.l2 = np.ascontiguousarray(self.l2, dtype=np.uint16)
        self.qweight = np.ascontiguousarray(self.qweight, dtype=np.uint8)
        self.wscales = np.ascontiguousarray(self.wscales, dtype=np.uint8)
        self.bias = np.ascontiguousarray(self.bias, dtype=np.float32)

    def as_struct(self) -> MxHostWeights:
        return MxHostWeights(self.N, self.K, self.rank, _ptr(self.inv_lambda),
                             _ptr(self.l1s) if self.rank else None,
                             _ptr(self.l2) if self.rank else None, _ptr(self.qweight),
                             _ptr(self.wscales), _ptr(self.bias))


def mx_prepare_weights(W_bits: np.ndarray, act_absmax: Optional[np.ndarray],
                       bias_bits: Optional[np.ndarray], rank: int) -> PreparedHostMx:
    """Host preparation of the MXFP4 form (smoothing, SVD split, residual in MXFP4)."""
    W_bits = np.ascontiguousarray(W_bits, dtype=np.uint16)
    N, K = W_bits.shape
    ax = None if act_absmax is None else np.ascontiguousarray(act_absmax, dtype=np.float32)
    b = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
    out = PreparedHostMx(N, K, rank, np.empty(K, np.float32), np.empty((K, rank), np.uint16),
                         np.empty((rank, N), np.uint16), np.empty((N, max(K // 2, 1)), np.uint8),
                         np.empty((N, max(K // 32, 1)), np.uint8), np.empty(N, np.float32))
    hw = out.as_struct()
    _check(_lib.svdq_mx_prepare_weights(_ptr(W_bits), N, K, _ptr(ax), _ptr(b), rank,
                                        ctypes.byref(hw)), "svdq_mx_prepare_weights")
    return out


def mx_pack_device_weights(hw: PreparedHostMx) -> np.ndarray:
    n = _lib.svdq_mx_device_weights_bytes(hw.N, hw.K, hw.rank)
    if n == 0:
        raise SvdqError(2, "svdq_mx_device_weights_bytes")
    blob = np.empty(n, np.uint8)
    s = hw.as_struct()
    _check(_lib.svdq_mx_pack_device_weights(ctypes.byref(s), _ptr(blob), n),
           "svdq_mx_pack_device_weights")
    return blob


def mx_merge_lora(hw: PreparedHostMx, A_bits: np.ndarray, B_bits: np.ndarray,
                  alpha: float = 1.0) -> PreparedHostMx:
    """merge_lora for an MXFP4 layer (svdq_mx_merge_lora)."""
    A, B, r2 = _lora_args(hw, A_bits, B_bits)
    rt = hw.rank + r2
    out = PreparedHostMx(hw.N, hw.K, rt, hw.inv_lambda, np.empty((hw.K, rt), np.uint16),
                         np.empty((rt, hw.N), np.uint16), hw.qweight, hw.wscales, hw.bias)
    src, dst = hw.as_struct(), out.as_struct()
    _check(_lib.svdq_mx_merge_lora(ctypes.byref(src), _ptr(A), _ptr(B), r2, float(alpha),
                                   ctypes.byref(dst)), "svdq_mx_merge_lora")
    return out


class MxLinear:
    """A prepared MXFP4 SVDQuant layer resident on one device."""

    def __init__(self, hw: PreparedHostMx, device="cuda"):
        self.N, self.K, self.rank = hw.N, hw.K, hw.rank
        self.blob = torch.from_numpy(mx_pack_device_weights(hw)).to(device)
        self.device = self.blob.device
        self._w = DeviceWeights(self.blob.data_ptr(), self.N, self.K, self.rank)

    def workspace_bytes(self, M: int) -> int:
        n = _lib.svdq_mx_workspace_bytes(M, self.N, self.K, self.rank)
        if n == 0:
            raise SvdqError(2, "svdq_mx_workspace_bytes")
        return n

    def new_workspace(self, M: int) -> torch.Tensor:
        return torch.empty(self.workspace_bytes(M), dtype=torch.uint8, device=self.device)


def mx_linear_forward(layer: MxLinear, X: torch.Tensor, out: Optional[torch.Tensor] = None,
                      out_dtype=torch.bfloat16, gelu: bool = False,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X W^T + b through the MXFP4 path (optionally gelu_tanh(Y))."""
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and X.shape[1] == layer.K
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, layer.N), dtype=out_dtype, device=X.device)
    _check_out(out, M, layer.N, X.device)
    if workspace is None:
        workspace = layer.new_workspace(M)
    dt = FP32 if out.dtype == torch.float32 else BF16
    _check(_lib.svdq_mx_linear_forward(ctypes.byref(layer._w), X.data_ptr(), M, out.data_ptr(), dt,
                                       EPILOGUE_GELU_TANH if gelu else EPILOGUE_NONE,
                                       workspace.data_ptr(), workspace.numel(), _stream(X.device)),
           "svdq_mx_linear_forward")
    return out


def mx_linear_quantize(layer: MxLinear, X: torch.Tensor, workspace: torch.Tensor) -> None:
    assert X.dtype == torch.bfloat16 and X.is_contiguous() and X.shape[1] == layer.K
    _check(_lib.svdq_mx_linear_quantize(ctypes.byref(layer._w), X.data_ptr(), X.shape[0],
                                        workspace.data_ptr(), workspace.numel(), _stream(X.device)),
           "svdq_mx_linear_quantize")


def mx_linear_gemm(layer: MxLinear, M: int, out: torch.Tensor, workspace: torch.Tensor,
                   gelu: bool = False) -> torch.Tensor:
    _check_out(out, M, layer.N, workspace.device)
    dt = FP32 if out.dtype == torch.float32 else BF16
    _check(_lib.svdq_mx_linear_gemm(ctypes.byref(layer._w), M, out.data_ptr(), dt,
                                    EPILOGUE_GELU_TANH if gelu else EPILOGUE_NONE,
                                    workspace.data_ptr(), workspace.numel(), _stream(out.device)),
           "svdq_mx_linear_gemm")
    return out


def mx_quantize_activations(layer: MxLinear, X: torch.Tensor, workspace: Optional[torch.Tensor] = None):
    """Canonical export of the MXFP4 quantiser: (codes uint8 [M, K/2], E8M0
    scales uint8 [M, K/32], low-rank down float32 [M, rank])."""
    M = X.shape[0]
    dev = X.device
    q = torch.empty((M, layer.K // 2), dtype=torch.uint8, device=dev)
    e = torch.empty((M, layer.K // 32), dtype=torch.uint8, device=dev)
    d = torch.empty((M, max(layer.rank, 1)), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = layer.new_workspace(M)
    _check(_lib.svdq_mx_quantize_activations(ctypes.byref(layer._w), X.data_ptr(), M, q.data_ptr(),
                                             e.data_ptr(), d.data_ptr(), workspace.data_ptr(),
                                             workspace.numel(), _stream(dev)),
           "svdq_mx_quantize_activations")
    return q, e, d[:, :layer.rank]


# ------------------------------------------------------------------- AWQ
def awq_quantize_weights(W_fp16: np.ndarray):
    W = np.ascontiguousarray(W_fp16, dtype=np.float16)
    N, K = W.shape
    q = np.empty((N, K // 2), np.uint8)
    s = np.empty((N, K // 64), np.uint16)
    z = np.empty((N, K // 64), np.uint16)
    _check(_lib.awq_quantize_weights(_ptr(W.view(np.uint16)), N, K, 64, _ptr(q), _ptr(s), _ptr(z)),
           "awq_quantize_weights")
    return q, s.view(np.float16), z.view(np.float16)


class AwqLinear:
    def __init__(self, q: np.ndarray, s: np.ndarray, z: np.ndarray, device="cuda"):
        self.N, self.K = q.shape[0], q.shape[1] * 2
        n = _lib.awq_device_weights_bytes(self.N, self.K)
        if n == 0:
            raise SvdqError(2, "awq_device_weights_bytes")
        blob = np.empty(n, np.uint8)
        q = np.ascontiguousarray(q, np.uint8)
        s = np.ascontiguousarray(s, np.float16).view(np.uint16)
        z = np.ascontiguousarray(z, np.float16).view(np.uint16)
        _check(_lib.awq_pack_device_weights(_ptr(q), _ptr(s), _ptr(z), self.N, self.K, _ptr(blob), n),
               "awq_pack_device_weights")
        self.blob = torch.from_numpy(blob).to(device)


def awq_forward(layer: AwqLinear, x: torch.Tensor, bias: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    assert x.dtype == torch.float16 and x.is_contiguous() and x.shape[1] == layer.K
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, layer.N), dtype=torch.float16, device=x.device)
    _check_out(out, M, layer.N, x.device, dtypes=(torch.float16,))
    if bias is not None:
        _check_bias(bias, layer.N, x.device)
    _check(_lib.awq_w4a16_forward(layer.blob.data_ptr(), layer.N, layer.K, x.data_ptr(), M,
                                  None if bias is None else bias.data_ptr(), out.data_ptr(),
                                  _stream(x.device)), "awq_w4a16_forward")
    return out


# ------------------------------------------------------------ measurement
MFMA_KINDS = {0: ("fp6 32x32x64", 2 * 32 * 32 * 64), 1: ("fp4 32x32x64", 2 * 32 * 32 * 64),
              2: ("bf16 32x32x16", 2 * 32 * 32 * 16), 3: ("bf16 32x32x8", 2 * 32 * 32 * 8),
              4: ("int8 32x32x32", 2 * 32 * 32 * 32)}
# instruction mixes (time per slot, no operation count): kind -> label
MFMA_MIXES = {5: "fp6 32x32x64 + 16 fp32 FMA", 6: "16 fp32 FMA", 7: "GEMM step: bf16 32x32x8 + fp6 32x32x64 + 16 FMA"}


def measure_mfma(kind: int, iters: int, grid: int, sink: torch.Tensor) -> None:
    """svdq_measure_mfma: `grid` workgroups, each wavefront four chains of
    `iters` matrix instructions of `kind` (MFMA_KINDS) or instruction-mix
    slots (MFMA_MIXES); the caller times it."""
    if sink.dtype != torch.int32 or sink.numel() < grid or sink.device.type != "cuda":
        raise ValueError("sink must be an int32 device tensor of at least `grid` elements")
    _check(_lib.svdq_measure_mfma(kind, iters, grid, sink.data_ptr(), _stream(sink.device)),
           "svdq_measure_mfma")


def measure_stream(src: torch.Tensor, grid: int, dst: Optional[torch.Tensor] = None,
                   sink: Optional[torch.Tensor] = None) -> None:
    """svdq_measure_stream: a plain streaming read of `src` (dst None) or
    copy into `dst`, with `grid` workgroups: the practical HBM floor."""
    nbytes = src.numel() * src.element_size()
    if dst is None:
        if sink is None or sink.numel() < grid or sink.dtype != torch.int32:
            raise ValueError("a read needs an int32 sink of at least `grid` elements")
        _check(_lib.svdq_measure_stream(src.data_ptr(), None, nbytes, grid, 0, sink.data_ptr(),
                                        _stream(src.device)), "svdq_measure_stream")
    else:
        if dst.numel() * dst.element_size() < nbytes:
            raise ValueError("dst is smaller than src")
        _check(_lib.svdq_measure_stream(src.data_ptr(), dst.data_ptr(), nbytes, grid, 1, None,
                                        _stream(src.device)), "svdq_measure_stream")
