"""Thin Python binding of libfp4.so (include/fp4.h), same names as the C calls.

Argument marshalling only: every step of the path runs in the HIP kernels behind
the C ABI. torch supplies device memory (outputs are allocated with
``torch.empty`` on the input's device) and the current stream. There is no
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "FP4_MXFP4",
    "FP4_NVFP4",
    "Fp4Error",
    "library_path",
    "load_library",
    "fp4_rotate_quantize",
    "fp4_quantize_weights",
    "fp4_linear",
    "fp4_rotate_quantize_linear",
    "fp4_rotate_quantize_linear_noalloc",
    "linear_workspace_bytes",
    "fp4_abi_version",
    "group_size",
]

FP4_MXFP4 = 0
FP4_NVFP4 = 1
_FMT = {"mxfp4": FP4_MXFP4, "nvfp4": FP4_NVFP4, FP4_MXFP4: FP4_MXFP4, FP4_NVFP4: FP4_NVFP4}
_STATUS = {0: "OK", -1: "NULLPTR", -2: "SHAPE", -3: "BLOCK", -4: "FORMAT", -5: "ALIGN", -6: "HIP"}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class Fp4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{_STATUS.get(status, status)}] {message}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, "libfp4.so")


def load_library() -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; build it with `python -m microscaling_fp4_quantized_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    q_args = [vp, i64, i64, i64, i32, i32, vp, vp, vp, vp]
    for name in ("fp4_rotate_quantize", "fp4_quantize_weights"):
        f = getattr(lib, name)
        f.argtypes = q_args
        f.restype = i32
    qx_args = [vp, i64, i64, i64, i32, i32, i32, vp, vp, vp, vp, vp]
    for name in ("fp4_rotate_quantize_ex", "fp4_quantize_weights_ex"):
        f = getattr(lib, name)
        f.argtypes = qx_args
        f.restype = i32
    lib.fp4_rotate_quantize_linear.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, vp, i32, vp, ctypes.c_size_t, vp]
    lib.fp4_rotate_quantize_linear.restype = i32
    lib.fp4_rotate_quantize_linear_noalloc.argtypes = [vp, i64, i64, i64, i32, vp, vp, i64, vp, i32, vp]
    lib.fp4_rotate_quantize_linear_noalloc.restype = i32
    lib.fp4_linear.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, i32, vp]
    lib.fp4_linear.restype = i32
    lib.fp4_last_error.argtypes = []
    lib.fp4_last_error.restype = ctypes.c_char_p
    lib.fp4_abi_version.argtypes = []
    lib.fp4_abi_version.restype = i32
    _LIB = lib
    return lib


def group_size(fmt) -> int:
    return 32 if _FMT[fmt] == FP4_MXFP4 else 16


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _launch(dev, fn, *args):
    """Call an entry point with the operands' device current (the library launches on the current
    device) and that device's current stream as the last argument."""
    for t in args:
        if isinstance(t, torch.Tensor):
            raise TypeError("pass data pointers, not tensors")
    if dev.index is not None and torch.cuda.current_device() != dev.index:
        with torch.cuda.device(dev):
            return fn(*args, _stream(dev))
    return fn(*args, _stream(dev))


def _same_device(name, dev, *tensors):
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.device != dev:
            raise ValueError(f"{name}: every operand must be on {dev}, got one on {t.device}")


def _check(status: int):
    if status != 0:
        raise Fp4Error(status, load_library().fp4_last_error().decode())


SCALE_RULES = {"standard": 0, "ocp_floor": 1, "oas": 2, "fit": 3}
TENSOR_SCALE_IN = 0x10


def _expect(t, shape, dtype, name, what):
    """Refuse anything but a contiguous CUDA tensor of this shape and dtype: the kernels take plain
    pointers and trust the sizes they imply, so a short buffer would be read or written out of bounds."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype or \
            tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        got = repr(t) if not isinstance(t, torch.Tensor) else f"{tuple(t.shape)} {t.dtype} on {t.device}"
        raise ValueError(f"{name}: {what} must be a contiguous {dtype} CUDA tensor of shape {tuple(shape)}, got {got}")


def _quantize(name: str, x: torch.Tensor, block: int, fmt, out=None, rule=None, signs=None, tensor_scale=None):
    lib = load_library()
    f = _FMT[fmt]
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError(f"{name}: expects a 2-D bf16 CUDA tensor with unit column stride")
    M, K = x.shape
    g = group_size(f)
    if out is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((M, K // g), dtype=torch.uint8, device=x.device)
        ts = torch.empty((1,), dtype=torch.float32, device=x.device) if f == FP4_NVFP4 else None
    else:
        codes, scales, ts = out
        _expect(codes, (M, K // 2), torch.uint8, name, "codes")
        _expect(scales, (M, K // g), torch.uint8, name, "scales")
        if f == FP4_NVFP4:
            if tensor_scale is None:
                _expect(ts, (1,), torch.float32, name, "tensor scale")
        elif ts is not None:
            raise ValueError(f"{name}: MXFP4 has no tensor scale")
    if tensor_scale is not None:
        # a given s_t: a device float32 [1] that the call reads and leaves unchanged
        if tensor_scale.dtype != torch.float32 or not tensor_scale.is_cuda or tensor_scale.numel() != 1:
            raise ValueError(f"{name}: tensor_scale must be a float32 CUDA tensor of one element")
        ts = tensor_scale
    _same_device(name, x.device, codes, scales, ts, signs, tensor_scale)
    if rule is None and signs is None and tensor_scale is None:
        _check(_launch(x.device, getattr(lib, name), _ptr(x), M, K, x.stride(0), int(block), f, _ptr(codes),
                       _ptr(scales), _ptr(ts)))
    else:
        if signs is not None and (signs.dtype != torch.int8 or not signs.is_cuda or signs.numel() != K
                                  or not signs.is_contiguous()):
            raise ValueError(f"{name}: signs must be a contiguous int8 CUDA tensor of K entries")
        r = SCALE_RULES[rule or "standard"] | (TENSOR_SCALE_IN if tensor_scale is not None else 0)
        _check(_launch(x.device, getattr(lib, name + "_ex"), _ptr(x), M, K, x.stride(0), int(block), f, r,
                       _ptr(signs), _ptr(codes), _ptr(scales), _ptr(ts)))
    return codes, scales, ts


def fp4_rotate_quantize(x: torch.Tensor, block: int, fmt="mxfp4", out=None, rule=None, signs=None,
                        tensor_scale=None):
    """Online block-Hadamard rotation + FP4 quantization of bf16 activations.

    Returns (codes [M, K/2] uint8, scales [M, K/g] uint8, tensor_scale [1] float32 or None).
    ``out`` may pass preallocated (codes, scales, tensor_scale). ``rule`` ("standard",
    "ocp_floor", "oas", "fit"), ``signs`` (int8 [K] of +-1) and ``tensor_scale`` (NVFP4: a
    given s_t, float32 [1] on the device) select fp4_rotate_quantize_ex.
    """
    return _quantize("fp4_rotate_quantize", x, block, fmt, out, rule, signs, tensor_scale)


def fp4_quantize_weights(w: torch.Tensor, block: int, fmt="mxfp4", out=None, rule=None, signs=None,
                         tensor_scale=None):
    """Offline rotation + quantization of a weight matrix [N, K] (same contract)."""
    return _quantize("fp4_quantize_weights", w, block, fmt, out, rule, signs, tensor_scale)


def fp4_linear(xq, xs, wq, ws, fmt="mxfp4", x_ts=None, w_ts=None, out_dtype=torch.float32, out=None):
    """Y = dq(Xq) dq(Wq)^T, [M, N] in float32 or bf16."""
    lib = load_library()
    f = _FMT[fmt]
    for t in (xq, wq):
        if not isinstance(t, torch.Tensor) or t.dim() != 2:
            raise ValueError("fp4_linear: Xq and Wq must be 2-D tensors of packed codes")
    M, N, K = xq.shape[0], wq.shape[0], 2 * xq.shape[1]
    if wq.shape[1] * 2 != K:
        raise ValueError("fp4_linear: X and W disagree on K")
    g = group_size(f)
    _expect(xq, (M, K // 2), torch.uint8, "fp4_linear", "Xq")
    _expect(wq, (N, K // 2), torch.uint8, "fp4_linear", "Wq")
    _expect(xs, (M, K // g), torch.uint8, "fp4_linear", "Xs")
    _expect(ws, (N, K // g), torch.uint8, "fp4_linear", "Ws")
    if f == FP4_NVFP4:
        _expect(x_ts, (1,), torch.float32, "fp4_linear", "x_ts")
        _expect(w_ts, (1,), torch.float32, "fp4_linear", "w_ts")
    elif x_ts is not None or w_ts is not None:
        raise ValueError("fp4_linear: MXFP4 has no tensor scales")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("fp4_linear: out_dtype must be torch.float32 or torch.bfloat16")
    ydt = {torch.float32: 0, torch.bfloat16: 1}[out_dtype]
    if out is None:
        y = torch.empty((M, N), dtype=out_dtype, device=xq.device)
    else:
        _expect(out, (M, N), out_dtype, "fp4_linear", "out")
        y = out
    _same_device("fp4_linear", xq.device, xs, wq, ws, x_ts, w_ts, y)
    _check(_launch(xq.device, lib.fp4_linear, _ptr(xq), _ptr(xs), _ptr(x_ts), _ptr(wq), _ptr(ws), _ptr(w_ts), M, N,
                   K, f, _ptr(y), ydt))
    return y


def linear_workspace_bytes(M: int, K: int) -> int:
    """FP4_LINEAR_WORKSPACE_BYTES(M, K) of include/fp4.h: X's codes, then its scales at the next
    256-byte boundary."""
    return ((M * K // 2 + 255) // 256) * 256 + M * K // 32


def fp4_rotate_quantize_linear(x: torch.Tensor, wq, ws, block: int, out_dtype=torch.float32, out=None,
                               workspace="auto"):
    """Decode step (MXFP4, 1 <= M <= 16): Y = fp4_linear(fp4_rotate_quantize(x), wq, ws).

    workspace: "auto" allocates one of linear_workspace_bytes(M, K) bytes, which lets the library
    take two launches where that is faster; None forces the one-launch kernel; or a contiguous
    uint8 CUDA tensor of at least that size."""
    lib = load_library()
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("fp4_rotate_quantize_linear: expects a 2-D bf16 CUDA tensor with unit column stride")
    for t in (wq, ws):
        if not t.is_cuda or t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("fp4_rotate_quantize_linear: weight codes and scales must be contiguous uint8 CUDA tensors")
    M, K = x.shape
    if wq.dim() != 2 or wq.shape[1] * 2 != K:
        raise ValueError("fp4_rotate_quantize_linear: X and W disagree on K")
    N = wq.shape[0]
    _expect(ws, (N, K // 32), torch.uint8, "fp4_rotate_quantize_linear", "Ws")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("fp4_rotate_quantize_linear: out_dtype must be torch.float32 or torch.bfloat16")
    ydt = {torch.float32: 0, torch.bfloat16: 1}[out_dtype]
    if out is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _expect(out, (M, N), out_dtype, "fp4_rotate_quantize_linear", "out")
        y = out
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('fp4_rotate_quantize_linear: workspace must be "auto", None or a uint8 tensor')
        workspace = torch.empty(linear_workspace_bytes(M, K), dtype=torch.uint8, device=x.device)
    if workspace is None:
        wsp, wsb = None, 0
        _same_device("fp4_rotate_quantize_linear", x.device, wq, ws, y)
    else:
        if not workspace.is_cuda or workspace.dtype != torch.uint8 or not workspace.is_contiguous():
            raise ValueError("fp4_rotate_quantize_linear: workspace must be a contiguous uint8 CUDA tensor")
        if workspace.numel() < linear_workspace_bytes(M, K):
            raise ValueError("fp4_rotate_quantize_linear: workspace too small")
        wsp, wsb = _ptr(workspace), workspace.numel()
        _same_device("fp4_rotate_quantize_linear", x.device, wq, ws, y, workspace)
    _check(_launch(x.device, lib.fp4_rotate_quantize_linear, _ptr(x), M, K, x.stride(0), int(block), _ptr(wq),
                   _ptr(ws), N, _ptr(y), ydt, wsp, wsb))
    return y


def fp4_rotate_quantize_linear_noalloc(x: torch.Tensor, wq, ws, block: int, out_dtype=torch.float32, out=None):
    """The decode step through the allocation-free entry point: where two launches pay off, the
    library uses its own per-GPU array instead of a workspace. Calls that overlap on one GPU race
    on that array. With `out` given, nothing is allocated here either."""
    lib = load_library()
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_cuda or x.stride(1) != 1:
        raise ValueError("fp4_rotate_quantize_linear_noalloc: expects a 2-D bf16 CUDA tensor with unit column stride")
    for t in (wq, ws):
        if not t.is_cuda or t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError("fp4_rotate_quantize_linear_noalloc: weight codes and scales must be contiguous uint8 "
                             "CUDA tensors")
    M, K = x.shape
    if wq.dim() != 2 or wq.shape[1] * 2 != K:
        raise ValueError("fp4_rotate_quantize_linear_noalloc: X and W disagree on K")
    N = wq.shape[0]
    _expect(ws, (N, K // 32), torch.uint8, "fp4_rotate_quantize_linear_noalloc", "Ws")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("fp4_rotate_quantize_linear_noalloc: out_dtype must be torch.float32 or torch.bfloat16")
    ydt = {torch.float32: 0, torch.bfloat16: 1}[out_dtype]
    if out is None:
        y = torch.empty((M, N), dtype=out_dtype, device=x.device)
    else:
        _expect(out, (M, N), out_dtype, "fp4_rotate_quantize_linear_noalloc", "out")
        y = out
    _same_device("fp4_rotate_quantize_linear_noalloc", x.device, wq, ws, y)
    _check(_launch(x.device, lib.fp4_rotate_quantize_linear_noalloc, _ptr(x), M, K, x.stride(0), int(block),
                   _ptr(wq), _ptr(ws), N, _ptr(y), ydt))
    return y


def fp4_abi_version() -> int:
    return load_library().fp4_abi_version()
