"""Thin Python binding of libttt.so (C ABI in include/ttt.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors must live on the current GPU; calls are asynchronous on
``torch.cuda.current_stream()``.  Errors raise ``TTTError`` with the library's
message.  There is no CPU fallback: if the library is missing, the first call
raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libttt.so")

TTT_F32, TTT_BF16 = 0, 1
OPT_FORCE_GENERAL, OPT_SPLITS, OPT_NS_UNFUSED = 0, 1, 2
KERNEL_KINDS = ("conv", "cast", "grad", "reduce", "ns", "apply", "gate")
NORM_PRESERVE = 1
EXPORTS = ("ttt_last_error", "ttt_update_workspace_bytes", "ttt_apply_workspace_bytes", "ttt_update",
           "ttt_update_ex", "ttt_update_host_workspace_bytes", "ttt_update_host", "ttt_apply", "ttt_output_gate", "ttt_shortconv2d", "ttt_stream_workspace_bytes",
           "ttt_stream", "ttt_stream_ex", "ttt_set_option", "ttt_profile_enable", "ttt_profile_reset",
           "ttt_profile_read", "ttt_update_noalloc", "ttt_noalloc_scratch_bytes", "ttt_mfma_rate_probe")

_lib = None


class TTTError(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libttt.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise TTTError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    vp, szp, u32 = ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t), ctypes.c_uint32
    sig = {
        "ttt_last_error": (ctypes.c_char_p, []),
        "ttt_update_workspace_bytes": (ctypes.c_int, [i32, i32, i32, i64, i32, szp]),
        "ttt_apply_workspace_bytes": (ctypes.c_int, [i32, i32, i32, i64, i32, szp]),
        "ttt_stream_workspace_bytes": (ctypes.c_int, [i32, i32, i32, i64, i32, szp]),
        "ttt_update": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64, i64, f32, i32,
                                      i32, vp, vp, vp, sz, vp]),
        "ttt_update_ex": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64, i64, f32,
                                         i32, i32, u32, vp, vp, vp, sz, vp]),
        "ttt_update_noalloc": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64, i64, f32,
                                              i32, i32, u32, vp, vp, vp]),
        "ttt_noalloc_scratch_bytes": (ctypes.c_int, [szp]),
        "ttt_update_host_workspace_bytes": (ctypes.c_int, [i32, i32, i32, i64, i64, i32, szp]),
        "ttt_update_host": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, i64, i64, i64,
                                           f32, i32, i32, u32, vp, vp, vp, sz, vp]),
        "ttt_output_gate": (ctypes.c_int, [i32, vp, i64, vp, vp, f32, vp, i64, i64, i32, vp]),
        "ttt_stream_ex": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, i64, vp, i64, vp, i64, vp, i64, i64,
                                         i64, f32, i32, i32, u32, vp, sz, vp]),
        "ttt_apply": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, i64, vp, i64, i64, i32, vp, sz, vp]),
        "ttt_shortconv2d": (ctypes.c_int, [vp, vp, i64, vp, i32, i32, i32, i32, i32, i32, i32, vp]),
        "ttt_stream": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, i64, vp, i64, vp, i64, vp, i64, i64, i64,
                                      f32, i32, i32, vp, sz, vp]),
        "ttt_set_option": (ctypes.c_int, [i32, i64]),
        "ttt_profile_enable": (ctypes.c_int, [i32]),
        "ttt_profile_reset": (ctypes.c_int, []),
        "ttt_profile_read": (ctypes.c_int, [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
        "ttt_mfma_rate_probe": (ctypes.c_int, [i32, vp, ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        msg = load().ttt_last_error().decode(errors="replace")
        raise TTTError(f"libttt status {status}: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TTT_BF16
    if t.dtype == torch.float32:
        return TTT_F32
    raise TypeError(f"token tensors must be bfloat16 or float32, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _rows(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    return t.stride(0)


def _weights(w: Sequence[torch.Tensor]) -> Tuple[int, int, int]:
    w1, w3, w2 = w
    for x in w:
        if x.dtype != torch.float32 or not x.is_cuda or not x.is_contiguous():
            raise ValueError("fast weights must be contiguous float32 GPU tensors")
    H, m, d = w1.shape
    if w3.shape != (H, m, d) or w2.shape != (H, d, m):
        raise ValueError(f"weight shapes {tuple(w1.shape)}, {tuple(w3.shape)}, {tuple(w2.shape)} do not match")
    return H, d, m


def _eta_stride(eta: torch.Tensor, H: int, n: int, device, on_gpu: bool = True) -> int:
    """Head stride of the rates: [H, >=n] with unit token stride, or [>=n] shared by every head."""
    if eta.dtype != torch.float32:
        raise ValueError("eta must be float32")
    if on_gpu:
        if not eta.is_cuda or (device is not None and eta.device != torch.device(device)):
            raise ValueError("eta must be on the same GPU as the tokens")
    elif eta.is_cuda:
        raise ValueError("eta must be in host memory")
    if eta.dim() == 2:
        if eta.shape[0] != H or eta.shape[1] < n or (n > 1 and eta.stride(1) != 1) or eta.stride(0) < 0:
            raise ValueError(f"eta must be [H={H}, >={n}] with unit token stride")
        return eta.stride(0)
    if eta.dim() == 1:
        if eta.shape[0] < n or (n > 1 and eta.stride(0) != 1):
            raise ValueError(f"eta must be [>={n}] with unit stride")
        return 0
    raise ValueError("eta must be [H, N] or [N]")


def _same_rows(t: torch.Tensor, like: torch.Tensor, rows: int, width: int, name: str) -> int:
    """`t` is a [rows, >=width] tensor of like's dtype and device with unit column stride;
    returns its row stride."""
    if t.dtype != like.dtype:
        raise ValueError(f"{name} must have dtype {like.dtype}, got {t.dtype}")
    if t.device != like.device:
        raise ValueError(f"{name} must be on {like.device}")
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] < width or t.stride(1) != 1:
        raise ValueError(f"{name} must be [{rows}, >={width}] with unit column stride, got {tuple(t.shape)}")
    return t.stride(0)


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def set_option(option: int, value: int) -> None:
    _check(load().ttt_set_option(option, value))


def update_workspace_bytes(heads: int, d: int, m: int, n: int, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t()
    code = TTT_BF16 if dtype == torch.bfloat16 else TTT_F32
    _check(load().ttt_update_workspace_bytes(heads, d, m, n, code, ctypes.byref(out)))
    return out.value


def apply_workspace_bytes(heads: int, d: int, m: int, nq: int, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t()
    code = TTT_BF16 if dtype == torch.bfloat16 else TTT_F32
    _check(load().ttt_apply_workspace_bytes(heads, d, m, nq, code, ctypes.byref(out)))
    return out.value


def update(w: Sequence[torch.Tensor], k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor, lr: float,
           steps: int = 1, out: Optional[Sequence[torch.Tensor]] = None, grad_out: Optional[torch.Tensor] = None,
           ns_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           norm_preserve: bool = False):
    """Fast-weight update; returns (W1^, W3^, W2^).  ``out`` may be ``w`` (in place).

    ``norm_preserve`` selects the norm-preserving step (flag TTT_NORM_PRESERVE).
    """
    H, d, m = _weights(w)
    if out is None:
        out = tuple(torch.empty_like(x) for x in w)
    _weights(out)
    n = k.shape[0]
    code = _dtype_code(k)
    if v.dtype != k.dtype or v.shape != k.shape or v.stride() != k.stride():
        raise ValueError("k and v must share dtype, shape and strides")
    ld = _rows(k, "k")
    if k.shape[1] < H * d:
        raise ValueError(f"k rows must hold H*d = {H * d} columns")
    ehs = _eta_stride(eta, H, n, k.device)
    for t, name in ((grad_out, "grad_out"), (ns_out, "ns_out")):
        if t is not None and (t.dtype != torch.float32 or t.numel() != 3 * H * d * m or not t.is_contiguous()
                              or t.device != k.device):
            raise ValueError(f"{name} must be a contiguous float32 tensor of 3*H*m*d elements on k's GPU")
    need = update_workspace_bytes(H, d, m, n, k.dtype)
    if workspace is None:
        workspace = _workspace(need, k.device)
    flags = NORM_PRESERVE if norm_preserve else 0
    _check(load().ttt_update_ex(H, d, m, *map(_ptr, w), *map(_ptr, out), k.data_ptr(), v.data_ptr(), ld,
                                eta.data_ptr(), ehs, n, float(lr), int(steps), code, flags, _ptr(grad_out),
                                _ptr(ns_out), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                _stream()))
    return tuple(out)


def update_noalloc(w: Sequence[torch.Tensor], k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor, lr: float,
                   steps: int = 1, out: Optional[Sequence[torch.Tensor]] = None,
                   grad_out: Optional[torch.Tensor] = None, ns_out: Optional[torch.Tensor] = None,
                   norm_preserve: bool = False):
    """``update`` through the allocation-free entry point (library-owned scratch, no
    workspace).  ``out`` must be given by callers that may not allocate."""
    H, d, m = _weights(w)
    if out is None:
        out = tuple(torch.empty_like(x) for x in w)
    _weights(out)
    n = k.shape[0]
    code = _dtype_code(k)
    if v.dtype != k.dtype or v.shape != k.shape or v.stride() != k.stride():
        raise ValueError("k and v must share dtype, shape and strides")
    ld = _rows(k, "k")
    if k.shape[1] < H * d:
        raise ValueError(f"k rows must hold H*d = {H * d} columns")
    ehs = _eta_stride(eta, H, n, k.device)
    for t, name in ((grad_out, "grad_out"), (ns_out, "ns_out")):
        if t is not None and (t.dtype != torch.float32 or t.numel() != 3 * H * d * m or not t.is_contiguous()
                              or t.device != k.device):
            raise ValueError(f"{name} must be a contiguous float32 tensor of 3*H*m*d elements on k's GPU")
    flags = NORM_PRESERVE if norm_preserve else 0
    _check(load().ttt_update_noalloc(H, d, m, *map(_ptr, w), *map(_ptr, out), k.data_ptr(), v.data_ptr(), ld,
                                     eta.data_ptr(), ehs, n, float(lr), int(steps), code, flags, _ptr(grad_out),
                                     _ptr(ns_out), _stream()))
    return tuple(out)


def noalloc_scratch_bytes() -> int:
    out = ctypes.c_size_t()
    _check(load().ttt_noalloc_scratch_bytes(ctypes.byref(out)))
    return out.value


def update_host_workspace_bytes(heads: int, d: int, m: int, batch: int, ld: int, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t()
    code = TTT_BF16 if dtype == torch.bfloat16 else TTT_F32
    _check(load().ttt_update_host_workspace_bytes(heads, d, m, batch, ld, code, ctypes.byref(out)))
    return out.value


def update_host(w: Sequence[torch.Tensor], k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor, lr: float,
                steps: int = 1, batch: int = 65536, out: Optional[Sequence[torch.Tensor]] = None,
                grad_out: Optional[torch.Tensor] = None, ns_out: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None, norm_preserve: bool = False):
    """Fast-weight update with K, V, eta in host memory (pinned for overlap), streamed in batches."""
    H, d, m = _weights(w)
    if out is None:
        out = tuple(torch.empty_like(x) for x in w)
    _weights(out)
    n = k.shape[0]
    code = _dtype_code(k)
    if k.is_cuda or v.is_cuda or eta.is_cuda:
        raise ValueError("update_host takes k, v and eta in host memory")
    if v.dtype != k.dtype or v.shape != k.shape or v.stride() != k.stride() or k.dim() != 2 or k.stride(1) != 1:
        raise ValueError("k and v must be 2-D host tensors sharing dtype, shape and strides")
    if k.shape[1] < H * d:
        raise ValueError(f"k rows must hold H*d = {H * d} columns")
    ehs = _eta_stride(eta, H, n, None, on_gpu=False)
    for t, name in ((grad_out, "grad_out"), (ns_out, "ns_out")):
        if t is not None and (t.dtype != torch.float32 or t.numel() != 3 * H * d * m or not t.is_contiguous()
                              or t.device != w[0].device):
            raise ValueError(f"{name} must be a contiguous float32 tensor of 3*H*m*d elements on the weights' GPU")
    ld = k.stride(0)
    need = update_host_workspace_bytes(H, d, m, batch, ld, k.dtype)
    if workspace is None:
        workspace = _workspace(need, w[0].device)
    flags = NORM_PRESERVE if norm_preserve else 0
    _check(load().ttt_update_host(H, d, m, *map(_ptr, w), *map(_ptr, out), k.data_ptr(), v.data_ptr(), ld,
                                  eta.data_ptr(), ehs, n, batch, float(lr), int(steps), code, flags, _ptr(grad_out),
                                  _ptr(ns_out), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                  _stream()))
    return tuple(out)


def apply(w: Sequence[torch.Tensor], q: torch.Tensor, out: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """o_i = f_W(q_i) for every row of q."""
    H, d, m = _weights(w)
    code = _dtype_code(q)
    ldq = _rows(q, "q")
    if q.shape[1] < H * d:
        raise ValueError(f"q rows must hold H*d = {H * d} columns")
    if out is None:
        out = torch.empty((q.shape[0], H * d), dtype=q.dtype, device=q.device)
    ldo = _same_rows(out, q, q.shape[0], H * d, "out")
    need = apply_workspace_bytes(H, d, m, q.shape[0], q.dtype)
    if workspace is None:
        workspace = _workspace(need, q.device)
    _check(load().ttt_apply(H, d, m, *map(_ptr, w), q.data_ptr(), ldq, out.data_ptr(), ldo, q.shape[0], code,
                            _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream()))
    return out


def shortconv2d(v: torch.Tensor, wconv: torch.Tensor, frames: int, tokens_per_frame: int, n_special: int,
                grid_h: int, grid_w: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """V' = ShortConv2D(V) over each frame's patch grid (depthwise 3x3, zero padding)."""
    code = _dtype_code(v)
    ld = _rows(v, "v")
    C = v.shape[1]
    if wconv.dtype != torch.float32 or tuple(wconv.shape) != (C, 3, 3) or not wconv.is_contiguous():
        raise ValueError("wconv must be contiguous float32 [C, 3, 3]")
    if out is None:
        out = torch.empty_like(v)
    if out.stride() != v.stride():
        raise ValueError("out must have the same strides as v")
    _check(load().ttt_shortconv2d(v.data_ptr(), out.data_ptr(), ld, wconv.data_ptr(), frames, tokens_per_frame,
                                  n_special, grid_h, grid_w, C, code, _stream()))
    return out


def stream_workspace_bytes(heads: int, d: int, m: int, chunk: int, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t()
    code = TTT_BF16 if dtype == torch.bfloat16 else TTT_F32
    _check(load().ttt_stream_workspace_bytes(heads, d, m, chunk, code, ctypes.byref(out)))
    return out.value


def stream(w: Sequence[torch.Tensor], k: torch.Tensor, v: torch.Tensor, eta: torch.Tensor, q: torch.Tensor,
           lr: float, steps: int, chunk: int, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, norm_preserve: bool = False) -> torch.Tensor:
    """Chunked causal pass: per chunk apply then update; ``w`` is updated in place."""
    H, d, m = _weights(w)
    code = _dtype_code(k)
    n = k.shape[0]
    ld = _rows(k, "k")
    if k.shape[1] < H * d:
        raise ValueError(f"k rows must hold H*d = {H * d} columns")
    if v.stride() != k.stride():
        raise ValueError("k and v must share strides")
    _same_rows(v, k, n, H * d, "v")
    ldq = _same_rows(q, k, n, H * d, "q")
    if out is None:
        out = torch.empty((n, H * d), dtype=q.dtype, device=q.device)
    ldo = _same_rows(out, k, n, H * d, "out")
    ehs = _eta_stride(eta, H, n, k.device)
    need = stream_workspace_bytes(H, d, m, chunk, k.dtype)
    if workspace is None:
        workspace = _workspace(need, k.device)
    flags = NORM_PRESERVE if norm_preserve else 0
    _check(load().ttt_stream_ex(H, d, m, *map(_ptr, w), k.data_ptr(), v.data_ptr(), ld, eta.data_ptr(), ehs,
                                q.data_ptr(), ldq, out.data_ptr(), ldo, n, chunk, float(lr), int(steps), code, flags,
                                _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream()))
    return out


def output_gate(o: torch.Tensor, wg: torch.Tensor, gamma: torch.Tensor, eps: float,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """o_i = RMSNorm(o'_i) * SiLU(W_g o'_i) over rows of C = wg.shape[0] channels."""
    code = _dtype_code(o)
    C = wg.shape[0]
    if wg.dtype != o.dtype or tuple(wg.shape) != (C, C) or not wg.is_contiguous() or not wg.is_cuda:
        raise ValueError("wg must be a contiguous [C, C] GPU tensor of o's dtype")
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (C,) or not gamma.is_contiguous() or not gamma.is_cuda:
        raise ValueError("gamma must be a contiguous float32 [C] GPU tensor")
    ldi = _rows(o, "o")
    if o.shape[1] < C:
        raise ValueError(f"o rows must hold C = {C} columns")
    if wg.device != o.device or gamma.device != o.device:
        raise ValueError("wg and gamma must be on o's GPU")
    if out is None:
        out = torch.empty((o.shape[0], C), dtype=o.dtype, device=o.device)
    ldo = _same_rows(out, o, o.shape[0], C, "out")
    _check(load().ttt_output_gate(C, o.data_ptr(), ldi, wg.data_ptr(), gamma.data_ptr(), float(eps), out.data_ptr(),
                                  ldo, o.shape[0], code, _stream()))
    return out


# ------------------------------------------------------------------ timing
def profile_enable(on: bool = True) -> None:
    _check(load().ttt_profile_enable(1 if on else 0))


def profile_reset() -> None:
    _check(load().ttt_profile_reset())


def profile_read() -> dict:
    """{kind: (total_ms, launches)} since the last reset (synchronises the timing events)."""
    res = {}
    for i, name in enumerate(KERNEL_KINDS):
        ms, cnt = ctypes.c_double(), ctypes.c_int64()
        _check(load().ttt_profile_read(i, ctypes.byref(ms), ctypes.byref(cnt)))
        res[name] = (ms.value, cnt.value)
    return res


def mfma_rate_probe(iters: int = 16384) -> float:
    """Launch the dense bf16 MFMA rate probe on the current stream; returns its FLOP count.

    Time the launch with events on the current stream to get the sustained rate."""
    flop = ctypes.c_double()
    _check(load().ttt_mfma_rate_probe(int(iters), _stream(), ctypes.byref(flop)))
    return flop.value
