"""Python binding of libmoe.so, the gfx950 routed-MoE layer (see include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so. Tensors are PyTorch-ROCm device tensors (device memory and streams
are all torch provides); pointers, sizes and the current HIP stream are passed
through ctypes under the same function names as the C ABI. There is no
fallback: if the library is missing, importing this package raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch  # loads the HIP runtime that libmoe.so then shares

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_F32, MOE_BF16, MOE_FP8_E4M3, MOE_FP4_E2M1 = 0, 1, 2, 3
MOE_QMODE_W, MOE_QMODE_F8 = 0, 1
DTYPE_NAMES = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3, "fp4": MOE_FP4_E2M1}
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARGUMENT", 2: "MOE_ERR_UNSUPPORTED",
          3: "MOE_ERR_WORKSPACE_TOO_SMALL", 4: "MOE_ERR_LAUNCH"}

ENTRY_POINTS = ("moe_status_string", "moe_route_workspace_size", "moe_route",
                "moe_permute_workspace_size", "moe_permute", "moe_experts_workspace_size",
                "moe_experts", "moe_experts_rows16", "moe_finalize", "moe_finalize_rows16",
                "moe_finalize_norm", "moe_finalize_norm_rows16", "moe_forward_workspace_size",
                "moe_forward", "moe_forward_norm", "moe_forward_noalloc",
                "moe_hbm_read")


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


class CExpertWeights(ctypes.Structure):
    """struct moe_expert_weights"""
    _fields_ = [("dtype", ctypes.c_int32), ("qmode", ctypes.c_int32),
                ("gate_up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("gate_up_scale", ctypes.c_void_p), ("down_scale", ctypes.c_void_p),
                ("gate_up_gscale", ctypes.c_void_p), ("down_gscale", ctypes.c_void_p)]


_lib = None
_vp, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t


def load_library(path: str = LIB_PATH):
    """Load libmoe.so (built by sparse_moe_layer_gemm_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python sparse_moe_layer_gemm_amd/build.py`")
    lib = ctypes.CDLL(path)
    sig = {
        "moe_status_string": (ctypes.c_char_p, [_i32]),
        "moe_route_workspace_size": (_sz, [_i64, _i32, _i32]),
        "moe_route": (_i32, [_vp, _i32, _i64, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                             _vp, _sz, _vp]),
        "moe_permute_workspace_size": (_sz, [_i64, _i32, _i32]),
        "moe_permute": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "moe_experts_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32, ctypes.POINTER(CExpertWeights)]),
        "moe_experts": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                               ctypes.POINTER(CExpertWeights), _vp, _vp, _sz, _vp]),
        "moe_finalize": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
        "moe_experts_rows16": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                                      ctypes.POINTER(CExpertWeights), _vp, _vp, _vp, _sz, _vp]),
        "moe_finalize_rows16": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
        "moe_finalize_norm": (_i32, [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, ctypes.c_float,
                                     _vp, _vp, _vp]),
        "moe_finalize_norm_rows16": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp,
                                            ctypes.c_float, _vp, _vp, _vp]),
        "moe_forward_norm": (_i32, [_vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                                    ctypes.POINTER(CExpertWeights), _vp, _vp, _vp, ctypes.c_float,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "moe_forward_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32, ctypes.POINTER(CExpertWeights)]),
        "moe_forward": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                               ctypes.POINTER(CExpertWeights), _i32, _vp, _vp, _i32, _vp, _vp, _vp,
                               _vp, _sz, _vp]),
        "moe_forward_noalloc": (_i32, [_vp, _i32, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                                       ctypes.POINTER(CExpertWeights), _i32, _vp, _vp, _i32, _vp,
                                       _vp, _vp, _vp]),
        "moe_hbm_read": (_i32, [_vp, _sz, _vp, _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


load_library()


# ---------------------------------------------------------------- marshalling helpers
def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _check(fn: str, status: int):
    if status != 0:
        raise MoEError(fn, status)


@dataclasses.dataclass
class ExpertWeights:
    """Device expert weights of one layer (layouts in include/moe.h)."""
    dtype: int
    gate_up: torch.Tensor
    down: torch.Tensor
    gate_up_scale: Optional[torch.Tensor] = None
    down_scale: Optional[torch.Tensor] = None
    gate_up_gscale: Optional[torch.Tensor] = None
    down_gscale: Optional[torch.Tensor] = None
    qmode: int = MOE_QMODE_W

    def c_struct(self) -> CExpertWeights:
        return CExpertWeights(self.dtype, self.qmode, _ptr(self.gate_up), _ptr(self.down),
                              _ptr(self.gate_up_scale), _ptr(self.down_scale),
                              _ptr(self.gate_up_gscale), _ptr(self.down_gscale))


# ---------------------------------------------------------------- the C ABI, same names
def moe_route_workspace_size(T: int, H: int, E: int) -> int:
    return _lib.moe_route_workspace_size(T, H, E)


def moe_route(x, w_router, bias, k: int, logits_dtype: int, logits, logits_f32, topk_ids, topk_w,
              workspace, stream=None):
    T, H = x.shape
    E = w_router.shape[1]
    _check("moe_route", _lib.moe_route(
        _ptr(x), _dt(x), T, H, _ptr(w_router), _ptr(bias), E, k, logits_dtype, _ptr(logits),
        _ptr(logits_f32), _ptr(topk_ids), _ptr(topk_w), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_permute_workspace_size(T: int, k: int, E: int) -> int:
    return _lib.moe_permute_workspace_size(T, k, E)


def moe_permute(topk_ids, E: int, counts, offsets, sorted_pair, pair_pos, workspace=None,
                stream=None):
    T, k = topk_ids.shape
    if workspace is None:
        need = moe_permute_workspace_size(T, k, E)
        workspace = globals()["workspace"](need, topk_ids.device) if need else None
    _check("moe_permute", _lib.moe_permute(
        _ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_experts_workspace_size(T: int, H: int, I: int, E: int, k: int, w: ExpertWeights) -> int:
    s = w.c_struct()
    return _lib.moe_experts_workspace_size(T, H, I, E, k, ctypes.byref(s))


def moe_experts(x, I: int, E: int, k: int, offsets, sorted_pair, w: ExpertWeights, y_sorted,
                workspace, stream=None):
    T, H = x.shape
    s = w.c_struct()
    _check("moe_experts", _lib.moe_experts(
        _ptr(x), _dt(x), T, H, I, E, k, _ptr(offsets), _ptr(sorted_pair), ctypes.byref(s),
        _ptr(y_sorted), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_experts_rows16(x, I: int, E: int, k: int, offsets, sorted_pair, w: ExpertWeights, y16,
                       y16_scale, workspace, stream=None):
    """y16 [T*k, H] int16/uint16 (fp16 bits), y16_scale [T*k, H/64] uint8."""
    T, H = x.shape
    s = w.c_struct()
    _check("moe_experts_rows16", _lib.moe_experts_rows16(
        _ptr(x), _dt(x), T, H, I, E, k, _ptr(offsets), _ptr(sorted_pair), ctypes.byref(s),
        _ptr(y16), _ptr(y16_scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def moe_finalize_rows16(y16, y16_scale, pair_pos, topk_w, out, out_f32=None, stream=None):
    T, k = topk_w.shape
    H = y16.shape[1]
    _check("moe_finalize_rows16", _lib.moe_finalize_rows16(
        _ptr(y16), _ptr(y16_scale), _ptr(pair_pos), _ptr(topk_w), T, k, H, _dt(out), _ptr(out),
        _ptr(out_f32), _stream(stream)))


def moe_finalize(y_sorted, pair_pos, topk_w, out, out_f32=None, stream=None):
    T, k = topk_w.shape
    H = y_sorted.shape[1]
    _check("moe_finalize", _lib.moe_finalize(
        _ptr(y_sorted), _ptr(pair_pos), _ptr(topk_w), T, k, H, _dt(out), _ptr(out), _ptr(out_f32),
        _stream(stream)))


def moe_finalize_norm(y_sorted, pair_pos, topk_w, residual, gamma_post, gamma_next, eps: float,
                      residual_out, normed, stream=None):
    """residual, residual_out, normed: [T, H] bf16 (residual_out may be residual);
    gamma_post, gamma_next: [H] bf16."""
    T, k = topk_w.shape
    H = y_sorted.shape[1]
    for t in (residual, gamma_post, gamma_next, residual_out, normed):
        if t.dtype != torch.bfloat16:
            raise ValueError("moe_finalize_norm takes bf16 residual, norm weights and outputs")
    _check("moe_finalize_norm", _lib.moe_finalize_norm(
        _ptr(y_sorted), _ptr(pair_pos), _ptr(topk_w), T, k, H, _ptr(residual), _ptr(gamma_post),
        _ptr(gamma_next), float(eps), _ptr(residual_out), _ptr(normed), _stream(stream)))


def moe_finalize_norm_rows16(y16, y16_scale, pair_pos, topk_w, residual, gamma_post, gamma_next,
                             eps: float, residual_out, normed, stream=None):
    """moe_finalize_norm over compact rows (y16 [T*k, H] fp16 bits, y16_scale [T*k, H/64])."""
    T, k = topk_w.shape
    H = y16.shape[1]
    for t in (residual, gamma_post, gamma_next, residual_out, normed):
        if t.dtype != torch.bfloat16:
            raise ValueError("moe_finalize_norm_rows16 takes bf16 residual, norm weights and outputs")
    _check("moe_finalize_norm_rows16", _lib.moe_finalize_norm_rows16(
        _ptr(y16), _ptr(y16_scale), _ptr(pair_pos), _ptr(topk_w), T, k, H, _ptr(residual),
        _ptr(gamma_post), _ptr(gamma_next), float(eps), _ptr(residual_out), _ptr(normed),
        _stream(stream)))


def moe_forward_workspace_size(T: int, H: int, I: int, E: int, k: int, w: ExpertWeights) -> int:
    s = w.c_struct()
    return _lib.moe_forward_workspace_size(T, H, I, E, k, ctypes.byref(s))


def moe_forward(x, w_router, bias, w: ExpertWeights, I: int, k: int, out, workspace,
                out_f32=None, logits_dtype: Optional[int] = None, logits=None, topk_ids=None,
                topk_w=None, stream=None):
    T, H = x.shape
    E = w_router.shape[1]
    if logits_dtype is None:
        logits_dtype = _dt(x)
    s = w.c_struct()
    _check("moe_forward", _lib.moe_forward(
        _ptr(x), _dt(x), T, H, I, E, k, _ptr(w_router), _ptr(bias), ctypes.byref(s), _dt(out),
        _ptr(out), _ptr(out_f32), logits_dtype, _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_forward_norm(x, w_router, bias, w: ExpertWeights, I: int, k: int, residual, gamma_post,
                     gamma_next, eps: float, residual_out, normed, workspace, logits=None,
                     topk_ids=None, topk_w=None, stream=None):
    """The layer ending in the fused finalize + sandwich norms (bf16 x, residual and outputs)."""
    T, H = x.shape
    E = w_router.shape[1]
    for t in (x, residual, gamma_post, gamma_next, residual_out, normed):
        if t.dtype != torch.bfloat16:
            raise ValueError("moe_forward_norm takes bf16 x, residual, norm weights and outputs")
    s = w.c_struct()
    _check("moe_forward_norm", _lib.moe_forward_norm(
        _ptr(x), T, H, I, E, k, _ptr(w_router), _ptr(bias), ctypes.byref(s), _ptr(residual),
        _ptr(gamma_post), _ptr(gamma_next), float(eps), _ptr(residual_out), _ptr(normed),
        _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def moe_forward_noalloc(x, w_router, bias, w: ExpertWeights, I: int, k: int, out, out_f32=None,
                        logits_dtype: Optional[int] = None, logits=None, topk_ids=None, topk_w=None,
                        stream=None):
    """moe_forward on the library's own scratch area (no workspace argument, no allocation)."""
    T, H = x.shape
    E = w_router.shape[1]
    if logits_dtype is None:
        logits_dtype = _dt(x)
    s = w.c_struct()
    _check("moe_forward_noalloc", _lib.moe_forward_noalloc(
        _ptr(x), _dt(x), T, H, I, E, k, _ptr(w_router), _ptr(bias), ctypes.byref(s), _dt(out),
        _ptr(out), _ptr(out_f32), logits_dtype, _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
        _stream(stream)))


# ---------------------------------------------------------------- device plumbing
def moe_hbm_read(buf, sink, stream=None):
    """Streaming read of every byte of buf (device, 16-byte aligned, size a
    multiple of 16); sink: a one-word device tensor the kernel may write."""
    _check("moe_hbm_read", _lib.moe_hbm_read(_ptr(buf), buf.numel() * buf.element_size(),
                                             _ptr(sink), _stream(stream)))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A device byte buffer (256-byte aligned by the caching allocator)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def to_device_bf16(bits, device="cuda") -> torch.Tensor:
    """bf16 values given as their uint16 bit patterns (numpy) -> bf16 device tensor."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def experts_to_device(host: dict, device="cuda", qmode: int = MOE_QMODE_W) -> ExpertWeights:
    """Expert weights as stored on the host (numpy) -> ExpertWeights on the device."""
    import numpy as np
    dt = DTYPE_NAMES[host["dtype"]]

    def dev(key):
        a = host.get(key)
        if a is None:
            return None
        if a.dtype == np.uint16:
            return to_device_bf16(a, device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    return ExpertWeights(dt, dev("gate_up"), dev("down"), dev("gate_up_scale"), dev("down_scale"),
                         dev("gate_up_gscale"), dev("down_gscale"), qmode)
