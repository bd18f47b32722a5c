"""Batched speculative-verify causal conv1d update for MI355X (gfx950).

Thin Python binding of the C ABI in include/conv_verify.h (libconvverify.so).  It
only marshals torch tensors into the ABI's shape struct and device pointers and
passes torch's current HIP stream; every step of the computation runs in the HIP
kernels.  PyTorch is used for device memory and streams only.

    conv_verify_update_dense(x, weight, bias, conv_state, out, snapshots, ...)
    conv_verify_update_dedup(x, weight, bias, conv_state, out, window_rows, ...)

Tensors (all on one GPU; bf16 or fp32 as the ABI allows):
    x, out       [n_seq, T, d_inner]     innermost stride 1, other strides free
    weight       [d_inner, d_conv]       contiguous
    bias         [d_inner] or None
    conv_state   [n_slots, d_inner, state_len]   contiguous below the slot dimension
    snapshots    [n_slots, T, d_inner, d_conv-1] contiguous below the slot dimension
    window_rows  [n_slots, d_inner, T+d_conv-2]  contiguous below the slot dimension
    slot_idx, num_accept_tokens: int32 [n_seq] or None
"""

from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib

__all__ = ["conv_verify_update_dense", "conv_verify_update_dedup", "conv_verify_describe",
           "conv_verify_abi_version", "prepare", "CvError", "library_path"]

library_path = _lib.LIB_PATH


class CvError(RuntimeError):
    """A non-zero return code of the C ABI."""

    def __init__(self, code: int, message: str):
        super().__init__(message)
        self.code = code


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return _lib.CV_F32
    if t.dtype == torch.bfloat16:
        return _lib.CV_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _contiguous_below_first(t) -> bool:
    expect = 1
    for size, stride in zip(reversed(t.shape[1:]), reversed(t.stride()[1:])):
        if size != 1 and stride != expect:
            return False
        expect *= size
    return True


def _marshal(dedup: bool, x, weight, bias, conv_state, out, windows, qk_channels, head_dim,
             l2_eps, slot_idx, num_accept_tokens):
    import torch

    tensors = [x, weight, conv_state, out, windows] + [
        t for t in (bias, slot_idx, num_accept_tokens) if t is not None]
    dev = x.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must live on the same GPU (no CPU path exists)")
    if x.dim() != 3 or out.shape != x.shape:
        raise ValueError(f"x and out must both be [n_seq, T, d_inner] (x {tuple(x.shape)}, "
                         f"out {tuple(out.shape)})")
    n_seq, T, d_inner = x.shape
    if x.stride(2) != 1 or out.stride(2) != 1:
        raise ValueError("x and out need a contiguous channel dimension")
    if weight.dim() != 2 or weight.shape[0] != d_inner or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [d_inner, d_conv] tensor")
    d_conv = weight.shape[1]
    if bias is not None and (tuple(bias.shape) != (d_inner,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [d_inner] tensor")
    for t in (weight, bias, out):
        if t is not None and t.dtype != x.dtype:
            raise TypeError("x, weight, bias and out must share one dtype")
    if conv_state.dim() != 3 or conv_state.shape[1] != d_inner or \
            not _contiguous_below_first(conv_state):
        raise ValueError("conv_state must be [n_slots, d_inner, state_len], contiguous "
                         "below the slot dimension")
    n_slots, _, state_len = conv_state.shape
    want = (n_slots, d_inner, T + d_conv - 2) if dedup else (n_slots, T, d_inner, d_conv - 1)
    if tuple(windows.shape) != want or not _contiguous_below_first(windows):
        raise ValueError(f"window buffer must be {want}, contiguous below the slot dimension "
                         f"(got {tuple(windows.shape)})")
    if windows.dtype != conv_state.dtype:
        raise TypeError("conv_state and the window buffer must share one dtype")
    for name, t in (("slot_idx", slot_idx), ("num_accept_tokens", num_accept_tokens)):
        if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (n_seq,) or
                              not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous int32 [n_seq] tensor")
    shape = _lib.CvShape(
        n_seq=n_seq, T=T, d_inner=d_inner, d_conv=d_conv, qk_channels=qk_channels,
        head_dim=head_dim, l2_eps=l2_eps, x_dtype=_dtype_code(x),
        state_dtype=_dtype_code(conv_state), n_slots=n_slots, state_len=state_len,
        x_seq_stride=x.stride(0), x_tok_stride=x.stride(1),
        out_seq_stride=out.stride(0), out_tok_stride=out.stride(1),
        state_slot_stride=conv_state.stride(0), win_slot_stride=windows.stride(0))
    return shape, dev


def _call(dedup: bool, x, weight, bias, conv_state, out, windows, qk_channels, head_dim,
          l2_eps, slot_idx, num_accept_tokens, stream):
    import torch

    lib = _lib.load()
    shape, dev = _marshal(dedup, x, weight, bias, conv_state, out, windows, qk_channels,
                          head_dim, l2_eps, slot_idx, num_accept_tokens)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    fn = lib.conv_verify_update_dedup if dedup else lib.conv_verify_update_dense
    with torch.cuda.device(dev):
        rc = fn(ctypes.byref(shape), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state),
                _ptr(slot_idx), _ptr(num_accept_tokens), _ptr(out), _ptr(windows),
                ctypes.c_void_p(handle))
    if rc != _lib.CV_OK:
        raise CvError(rc, _lib.error_message(lib, rc))


def prepare(dedup: bool, x, weight, bias, conv_state, out, windows, *, qk_channels: int,
            head_dim: int, l2_eps: float = 1e-6, slot_idx=None, num_accept_tokens=None,
            stream=None):
    """Marshal once; return a zero-argument callable that re-issues the same launch.

    For tight launch loops (benchmarks, serving steps): each call is one ctypes call
    into the C ABI with the arguments built here, on the stream resolved here.  The
    tensors must stay alive and keep their storage while the callable is in use.
    """
    import torch

    lib = _lib.load()
    shape, dev = _marshal(dedup, x, weight, bias, conv_state, out, windows, qk_channels,
                          head_dim, l2_eps, slot_idx, num_accept_tokens)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    fn = lib.conv_verify_update_dedup if dedup else lib.conv_verify_update_dense
    args = (ctypes.byref(shape), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state),
            _ptr(slot_idx), _ptr(num_accept_tokens), _ptr(out), _ptr(windows),
            ctypes.c_void_p(handle))
    keep = (shape, x, weight, bias, conv_state, out, windows, slot_idx, num_accept_tokens)

    def launch():
        rc = fn(*args)
        if rc != _lib.CV_OK:
            raise CvError(rc, _lib.error_message(lib, rc))

    launch.keepalive = keep
    return launch


def conv_verify_update_dense(x, weight, bias, conv_state, out, snapshots, *, qk_channels: int,
                             head_dim: int, l2_eps: float = 1e-6, slot_idx=None,
                             num_accept_tokens=None, stream=None) -> None:
    """Enqueue one launch writing out, dense snapshots and the committed conv_state."""
    _call(False, x, weight, bias, conv_state, out, snapshots, qk_channels, head_dim, l2_eps,
          slot_idx, num_accept_tokens, stream)


def conv_verify_update_dedup(x, weight, bias, conv_state, out, window_rows, *,
                             qk_channels: int, head_dim: int, l2_eps: float = 1e-6,
                             slot_idx=None, num_accept_tokens=None, stream=None) -> None:
    """Enqueue one launch writing out, deduplicated window rows and the committed state."""
    _call(True, x, weight, bias, conv_state, out, window_rows, qk_channels, head_dim, l2_eps,
          slot_idx, num_accept_tokens, stream)


def conv_verify_describe(dedup: bool, shape: "_lib.CvShape") -> "_lib.CvLaunchInfo":
    """Launch geometry for a shape (host only; raises CvError when the shape is refused)."""
    lib = _lib.load()
    info = _lib.CvLaunchInfo()
    rc = lib.conv_verify_describe(int(dedup), ctypes.byref(shape), ctypes.byref(info))
    if rc != _lib.CV_OK:
        raise CvError(rc, _lib.error_message(lib, rc))
    return info


def conv_verify_abi_version() -> int:
    return _lib.load().conv_verify_abi_version()
