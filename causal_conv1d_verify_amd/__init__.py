"""Batched speculative-verify causal conv1d update for MI355X (gfx950).

Thin Python binding of the C ABI in include/conv_verify.h (libconvverify.so).  It
only marshals torch tensors into the ABI's shape struct and device pointers and
passes torch's current HIP stream; every step of the computation runs in the HIP
kernels.  PyTorch is used for device memory and streams only.

    conv_verify_update(x, weight, bias, conv_state, out, windows, layout=..., ...)
    conv_verify_update_dense(...)  /  conv_verify_update_dedup(...)   (the chain verify)
    conv_verify_update_tree(x, weight, bias, conv_state, out, windows, parent, ...)
    conv_verify_restore(conv_state, windows, window_index, layout=..., ...)
    conv_prefill(x, weight, bias, conv_state, out, cu_seqlens, max_len=..., ...)
    conv_qk_l2norm(x, qk_channels=..., head_dim=..., ...)

Tensors (all on one GPU; bf16 or fp32 as the ABI allows):
    x, out       [n_seq, T, d_inner], or packed [total, d_inner] with cu_seqlens;
                 innermost stride 1, other strides free
    weight       [d_inner, d_conv]       contiguous
    bias         [d_inner] or None
    conv_state   [n_slots, d_inner, state_len], either contiguous below the slot
                 dimension (channel-major) or the transposed view of a time-major
                 [n_slots, state_len, >= d_inner] buffer (stride 1 along channels,
                 state_col_stride = the column stride)
    windows      by layout, contiguous below the slot dimension:
                   "dense"   [n_slots, T, d_inner, d_conv-1]
                   "dedup"   [n_slots, d_inner, T+d_conv-2]   (rows, channel-major)
                   "dedup_t" [n_slots, T+d_conv-2, d_inner]   (rows, time-major)
    slot_idx, num_accept_tokens, window_index, has_initial_state: int32 [n_seq] or None
    cu_seqlens   int32 [n_seq+1];  parent  int32 [n_seq, T]
"""

from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib

__all__ = ["conv_verify_update", "conv_verify_update_dense", "conv_verify_update_dedup",
           "conv_verify_update_tree", "conv_verify_restore", "conv_prefill", "conv_qk_l2norm",
           "conv_verify_describe", "conv_verify_abi_version", "conv_verify_debug_count",
           "write_count_library", "prepare", "CvError", "library_path", "LAYOUTS"]

library_path = _lib.LIB_PATH
LAYOUTS = {"dense": _lib.CV_WIN_DENSE, "dedup": _lib.CV_WIN_ROWS, "dedup_t": _lib.CV_WIN_ROWS_T}


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


def _same_gpu(*tensors):
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    if dev.type != "cuda" or any(t.device != dev for t in ts):
        raise ValueError("all tensors must live on the same GPU (no CPU path exists)")
    return dev


def _int32_vec(name, t, n):
    import torch

    if t is not None and (t.dtype != torch.int32 or tuple(t.shape) != (n,) or
                          not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous int32 [{n}] tensor")


def _stream_handle(stream, dev) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _window_T(layout: str, windows, d_inner: int, d_conv: int) -> int:
    """Draft positions of a window buffer, from its shape (checked against the layout)."""
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    w1 = d_conv - 1
    if layout == "dense":
        ok = windows.dim() == 4 and windows.shape[2] == d_inner and windows.shape[3] == w1
        T = windows.shape[1] if ok else 0
    elif layout == "dedup":
        ok = windows.dim() == 3 and windows.shape[1] == d_inner
        T = windows.shape[2] - w1 + 1 if ok else 0
    else:
        ok = windows.dim() == 3 and windows.shape[2] == d_inner
        T = windows.shape[1] - w1 + 1 if ok else 0
    if not ok or T < 1 or not _contiguous_below_first(windows):
        raise ValueError(f"window buffer {tuple(windows.shape)} does not fit layout {layout!r} "
                         f"for d_inner {d_inner}, d_conv {d_conv} (contiguous below the slot "
                         "dimension)")
    return T


def _check_state(conv_state, d_inner) -> int:
    """Validates conv_state's view; returns the ABI's state_col_stride (0: channel-major)."""
    if conv_state.dim() == 3 and conv_state.shape[1] == d_inner:
        if _contiguous_below_first(conv_state):
            return 0
        # time-major storage [n_slots, state_len, >= d_inner] seen as [n_slots, d, state_len]
        if conv_state.stride(1) == 1 and conv_state.stride(2) >= d_inner:
            return conv_state.stride(2)
    raise ValueError("conv_state must be [n_slots, d_inner, state_len], contiguous below the "
                     "slot dimension, or the [n_slots, d_inner, state_len] view of a time-major "
                     "[n_slots, state_len, >= d_inner] buffer")


def _check_window_slots(conv_state, windows) -> int:
    """The window buffer is indexed by slot like conv_state (the kernels bound a slot by
    n_slots, then address windows + slot * win_slot_stride), so it must hold at least as
    many slots as the pool.  Returns n_slots."""
    n_slots = conv_state.shape[0]
    if windows.shape[0] < n_slots:
        raise ValueError(f"the window buffer holds {windows.shape[0]} slots but conv_state has "
                         f"{n_slots}: windows are indexed by slot, so they need at least as many")
    return n_slots


def _verify_args(layout, tree, x, weight, bias, conv_state, out, windows, qk_channels,
                 head_dim, l2_eps, slot_idx, num_accept_tokens, cu_seqlens, parent, stream):
    import torch

    lib = _lib.load()
    dev = _same_gpu(x, weight, conv_state, out, windows, bias, slot_idx, num_accept_tokens,
                    cu_seqlens, parent)
    if out.shape != x.shape or x.stride(-1) != 1 or out.stride(-1) != 1:
        raise ValueError(f"x and out must have one shape and a contiguous channel dimension "
                         f"(x {tuple(x.shape)}, out {tuple(out.shape)})")
    if weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [d_inner, d_conv] tensor")
    d_inner, d_conv = weight.shape
    if x.shape[-1] != d_inner:
        raise ValueError("x's channel count differs from weight's")
    if bias is not None and (tuple(bias.shape) != (d_inner,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [d_inner] tensor")
    for t in (weight, bias, out):
        if t is not None and t.dtype != x.dtype:
            raise TypeError("x, weight, bias and out must share one dtype")
    state_col = _check_state(conv_state, d_inner)
    if windows.dtype != conv_state.dtype:
        raise TypeError("conv_state and the window buffer must share one dtype")
    T = _window_T(layout, windows, d_inner, d_conv)
    if cu_seqlens is not None:
        if x.dim() != 2:
            raise ValueError("packed rows: x and out must be [total, d_inner]")
        n_seq = cu_seqlens.shape[0] - 1
        _int32_vec("cu_seqlens", cu_seqlens, n_seq + 1)
        x_seq = out_seq = 0
        x_tok, out_tok = x.stride(0), out.stride(0)
    else:
        if x.dim() != 3 or x.shape[1] != T:
            raise ValueError(f"x and out must be [n_seq, {T}, d_inner] for this window buffer")
        n_seq = x.shape[0]
        x_seq, x_tok, out_seq, out_tok = x.stride(0), x.stride(1), out.stride(0), out.stride(1)
    _int32_vec("slot_idx", slot_idx, n_seq)
    _int32_vec("num_accept_tokens", num_accept_tokens, n_seq)
    if tree:
        if parent is None or parent.dtype != torch.int32 or tuple(parent.shape) != (n_seq, T) \
                or not parent.is_contiguous():
            raise ValueError(f"parent must be a contiguous int32 [{n_seq}, {T}] tensor")
    n_slots = _check_window_slots(conv_state, windows)
    state_len = conv_state.shape[2]
    shape = _lib.CvShape(
        n_seq=n_seq, T=T, d_inner=d_inner, d_conv=d_conv, qk_channels=qk_channels,
        head_dim=head_dim, l2_eps=l2_eps, x_dtype=_dtype_code(x),
        state_dtype=_dtype_code(conv_state), n_slots=n_slots, state_len=state_len,
        x_seq_stride=x_seq, x_tok_stride=x_tok, out_seq_stride=out_seq, out_tok_stride=out_tok,
        state_slot_stride=conv_state.stride(0), win_slot_stride=windows.stride(0),
        state_col_stride=state_col)
    h = ctypes.c_void_p(_stream_handle(stream, dev))
    if tree:
        fn = lib.conv_verify_update_tree
        args = (ctypes.byref(shape), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state),
                _ptr(slot_idx), _ptr(num_accept_tokens), _ptr(cu_seqlens), _ptr(parent),
                _ptr(out), _ptr(windows), h)
    else:
        fn = lib.conv_verify_update
        args = (ctypes.byref(shape), LAYOUTS[layout], _ptr(x), _ptr(weight), _ptr(bias),
                _ptr(conv_state), _ptr(slot_idx), _ptr(num_accept_tokens), _ptr(cu_seqlens),
                _ptr(out), _ptr(windows), h)
    keep = (shape, x, weight, bias, conv_state, out, windows, slot_idx, num_accept_tokens,
            cu_seqlens, parent)
    return lib, dev, fn, args, keep


def _restore_args(conv_state, windows, window_index, layout, d_conv, slot_idx, stream):
    lib = _lib.load()
    dev = _same_gpu(conv_state, windows, window_index, slot_idx)
    d_inner = conv_state.shape[1] if conv_state.dim() == 3 else -1
    state_col = _check_state(conv_state, d_inner)
    if windows.dtype != conv_state.dtype:
        raise TypeError("conv_state and the window buffer must share one dtype")
    T = _window_T(layout, windows, d_inner, d_conv)
    n_seq = window_index.shape[0]
    _int32_vec("window_index", window_index, n_seq)
    _int32_vec("slot_idx", slot_idx, n_seq)
    n_slots = _check_window_slots(conv_state, windows)
    state_len = conv_state.shape[2]
    dt = _dtype_code(conv_state)
    # the restore moves state-typed bits only; x_dtype just has to form a valid pair
    shape = _lib.CvShape(n_seq=n_seq, T=T, d_inner=d_inner, d_conv=d_conv, x_dtype=dt,
                         state_dtype=dt, n_slots=n_slots, state_len=state_len,
                         state_slot_stride=conv_state.stride(0),
                         win_slot_stride=windows.stride(0), state_col_stride=state_col)
    args = (ctypes.byref(shape), LAYOUTS[layout], _ptr(conv_state), _ptr(windows),
            _ptr(slot_idx), _ptr(window_index), ctypes.c_void_p(_stream_handle(stream, dev)))
    return lib, dev, lib.conv_verify_restore, args, (shape, conv_state, windows, window_index,
                                                     slot_idx)


def _prefill_args(x, weight, bias, conv_state, out, cu_seqlens, max_len, slot_idx,
                  has_initial_state, stream):
    lib = _lib.load()
    dev = _same_gpu(x, weight, conv_state, out, cu_seqlens, bias, slot_idx, has_initial_state)
    if x.dim() != 2 or out.shape != x.shape or x.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("x and out must be packed [total, d_inner] with unit channel stride")
    if weight.dim() != 2 or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [d_inner, d_conv] tensor")
    d_inner, d_conv = weight.shape
    if bias is not None and (tuple(bias.shape) != (d_inner,) or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [d_inner] tensor")
    for t in (weight, bias, out):
        if t is not None and t.dtype != x.dtype:
            raise TypeError("x, weight, bias and out must share one dtype")
    state_col = _check_state(conv_state, d_inner)
    n_seq = cu_seqlens.shape[0] - 1
    _int32_vec("cu_seqlens", cu_seqlens, n_seq + 1)
    _int32_vec("slot_idx", slot_idx, n_seq)
    _int32_vec("has_initial_state", has_initial_state, n_seq)
    n_slots, _, state_len = conv_state.shape
    shape = _lib.CvShape(n_seq=n_seq, T=max(1, int(max_len)), d_inner=d_inner, d_conv=d_conv,
                         x_dtype=_dtype_code(x), state_dtype=_dtype_code(conv_state),
                         n_slots=n_slots, state_len=state_len, x_tok_stride=x.stride(0),
                         out_tok_stride=out.stride(0), state_slot_stride=conv_state.stride(0),
                         state_col_stride=state_col)
    args = (ctypes.byref(shape), _ptr(x), _ptr(weight), _ptr(bias), _ptr(conv_state),
            _ptr(slot_idx), _ptr(cu_seqlens), _ptr(has_initial_state), _ptr(out),
            ctypes.c_void_p(_stream_handle(stream, dev)))
    keep = (shape, x, weight, bias, conv_state, out, cu_seqlens, slot_idx, has_initial_state)
    return lib, dev, lib.conv_prefill, args, keep


def _l2_args(x, qk_channels, head_dim, l2_eps, stream):
    lib = _lib.load()
    dev = _same_gpu(x)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be [rows, channels] with unit channel stride")
    shape = _lib.CvShape(d_inner=x.shape[1], qk_channels=qk_channels, head_dim=head_dim,
                         l2_eps=l2_eps, x_dtype=_dtype_code(x))
    args = (ctypes.byref(shape), x.shape[0], x.stride(0), _ptr(x),
            ctypes.c_void_p(_stream_handle(stream, dev)))
    return lib, dev, lib.conv_qk_l2norm, args, (shape, x)


def _issue(lib, dev, fn, args):
    import torch

    with torch.cuda.device(dev):
        rc = fn(*args)
    if rc != _lib.CV_OK:
        raise CvError(rc, _lib.error_message(lib, rc))


def conv_verify_update(x, weight, bias, conv_state, out, windows, *, layout: str,
                       qk_channels: int, head_dim: int, l2_eps: float = 1e-6, slot_idx=None,
                       num_accept_tokens=None, cu_seqlens=None, stream=None) -> None:
    """Enqueue one chain-verify launch in any window layout, optionally over packed rows."""
    if cu_seqlens is not None and x.shape[0] == 0:
        return   # no tokens at all: every packed row is empty, nothing to write
    _issue(*_verify_args(layout, False, x, weight, bias, conv_state, out, windows,
                         qk_channels, head_dim, l2_eps, slot_idx, num_accept_tokens,
                         cu_seqlens, None, stream)[:4])


def conv_verify_update_dense(x, weight, bias, conv_state, out, snapshots, *, qk_channels: int,
                             head_dim: int, l2_eps: float = 1e-6, slot_idx=None,
                             num_accept_tokens=None, stream=None) -> None:
    """Enqueue one launch writing out, dense snapshots and the committed conv_state."""
    conv_verify_update(x, weight, bias, conv_state, out, snapshots, layout="dense",
                       qk_channels=qk_channels, head_dim=head_dim, l2_eps=l2_eps,
                       slot_idx=slot_idx, num_accept_tokens=num_accept_tokens, stream=stream)


def conv_verify_update_dedup(x, weight, bias, conv_state, out, window_rows, *,
                             qk_channels: int, head_dim: int, l2_eps: float = 1e-6,
                             slot_idx=None, num_accept_tokens=None, stream=None) -> None:
    """Enqueue one launch writing out, deduplicated window rows and the committed state."""
    conv_verify_update(x, weight, bias, conv_state, out, window_rows, layout="dedup",
                       qk_channels=qk_channels, head_dim=head_dim, l2_eps=l2_eps,
                       slot_idx=slot_idx, num_accept_tokens=num_accept_tokens, stream=stream)


def conv_verify_update_tree(x, weight, bias, conv_state, out, windows, parent, *,
                            qk_channels: int, head_dim: int, l2_eps: float = 1e-6,
                            slot_idx=None, num_accept_tokens=None, cu_seqlens=None,
                            stream=None) -> None:
    """Enqueue one tree-verify launch (dense windows; conv_state is only read)."""
    _issue(*_verify_args("dense", True, x, weight, bias, conv_state, out, windows,
                         qk_channels, head_dim, l2_eps, slot_idx, num_accept_tokens,
                         cu_seqlens, parent, stream)[:4])


def conv_verify_restore(conv_state, windows, window_index, *, layout: str, d_conv: int,
                        slot_idx=None, stream=None) -> None:
    """Enqueue the accepted-prefix restore: window window_index[i] of row i's slot becomes
    conv_state columns 0..d_conv-2 (index -1 or slot -1: nothing for that row)."""
    _issue(*_restore_args(conv_state, windows, window_index, layout, d_conv, slot_idx,
                          stream)[:4])


def conv_prefill(x, weight, bias, conv_state, out, cu_seqlens, *, max_len: int, slot_idx=None,
                 has_initial_state=None, stream=None) -> None:
    """Enqueue the prefill conv (conv + SiLU, no L2) over packed prompts; each row's last
    window is committed to its state.  max_len >= the longest prompt."""
    _issue(*_prefill_args(x, weight, bias, conv_state, out, cu_seqlens, max_len, slot_idx,
                          has_initial_state, stream)[:4])


def conv_qk_l2norm(x, *, qk_channels: int, head_dim: int, l2_eps: float = 1e-6,
                   stream=None) -> None:
    """Enqueue the separate per-head L2 over the first qk_channels channels of each row of
    x ([rows, channels]), in place."""
    _issue(*_l2_args(x, qk_channels, head_dim, l2_eps, stream)[:4])


def prepare(kind, *args, **kwargs):
    """Marshal once; return a zero-argument callable that re-issues the same launch.

    kind: "update" (the conv_verify_update arguments), "tree"
    (conv_verify_update_tree's), "restore", "prefill" or "l2"; or True / False for the
    dedup / dense chain verify.  For tight launch loops (benchmarks, serving steps):
    each call is one ctypes call into the C ABI with the arguments built here, on the
    stream resolved here.  The tensors must stay alive while the callable is in use.
    """
    if kind is True or kind is False:
        x, weight, bias, conv_state, out, windows = args
        built = _verify_args("dedup" if kind else "dense", False, x, weight, bias, conv_state,
                             out, windows, kwargs["qk_channels"], kwargs["head_dim"],
                             kwargs.get("l2_eps", 1e-6), kwargs.get("slot_idx"),
                             kwargs.get("num_accept_tokens"), None, None, kwargs.get("stream"))
    elif kind in ("update", "tree"):
        x, weight, bias, conv_state, out, windows = args[:6]
        parent = args[6] if kind == "tree" else None
        built = _verify_args(kwargs.get("layout", "dense"), kind == "tree", x, weight, bias,
                             conv_state, out, windows, kwargs["qk_channels"],
                             kwargs["head_dim"], kwargs.get("l2_eps", 1e-6),
                             kwargs.get("slot_idx"), kwargs.get("num_accept_tokens"),
                             kwargs.get("cu_seqlens"), parent, kwargs.get("stream"))
    elif kind == "restore":
        conv_state, windows, window_index = args
        built = _restore_args(conv_state, windows, window_index, kwargs["layout"],
                              kwargs["d_conv"], kwargs.get("slot_idx"), kwargs.get("stream"))
    elif kind == "prefill":
        x, weight, bias, conv_state, out, cu_seqlens = args
        built = _prefill_args(x, weight, bias, conv_state, out, cu_seqlens, kwargs["max_len"],
                              kwargs.get("slot_idx"), kwargs.get("has_initial_state"),
                              kwargs.get("stream"))
    elif kind == "l2":
        (x,) = args
        built = _l2_args(x, kwargs["qk_channels"], kwargs["head_dim"],
                         kwargs.get("l2_eps", 1e-6), kwargs.get("stream"))
    else:
        raise ValueError(f"unknown launch kind {kind!r}")
    lib, _dev, fn, cargs, keep = built

    def launch():
        rc = fn(*cargs)
        if rc != _lib.CV_OK:
            raise CvError(rc, _lib.error_message(lib, rc))

    launch.keepalive = keep
    return launch


def conv_verify_describe(variant, shape: "_lib.CvShape") -> "_lib.CvLaunchInfo":
    """Launch geometry for a shape (host only; raises CvError when the shape is refused).
    variant: a layout name, True / False (dedup / dense), or "tree"."""
    lib = _lib.load()
    if variant is True or variant is False:
        code = int(variant)
    elif variant == "tree":
        code = _lib.CV_VARIANT_TREE
    else:
        code = LAYOUTS[variant]
    info = _lib.CvLaunchInfo()
    rc = lib.conv_verify_describe(code, ctypes.byref(shape), ctypes.byref(info))
    if rc != _lib.CV_OK:
        raise CvError(rc, _lib.error_message(lib, rc))
    return info


def conv_verify_abi_version() -> int:
    return _lib.load().conv_verify_abi_version()


# The write-count build of the library, for tests: within `with write_count_library():`
# every call above goes to libconvverify_wc.so.
write_count_library = _lib.write_count_library


def conv_verify_debug_count(ranges=()):
    """Write-count build only: count the global stores of later launches into each
    (buffer, counters) pair of `ranges` (at most 4): counters is an int32 tensor with one
    element per 2 bytes of buffer, on the same GPU, zeroed by the caller; both must stay
    alive until the next call (an empty `ranges` clears them)."""
    lib = _lib.load()
    if len(ranges) > 4:
        raise ValueError("at most 4 count ranges")
    lo = (ctypes.c_void_p * 4)()
    nbytes = (ctypes.c_uint64 * 4)()
    cnt = (ctypes.c_void_p * 4)()
    for k, (buf, counts) in enumerate(ranges):
        b = buf.numel() * buf.element_size()
        if not (buf.is_contiguous() and counts.is_contiguous()) or str(counts.dtype) != "torch.int32":
            raise ValueError("count ranges: contiguous buffers and int32 counters")
        if counts.numel() * 2 != b:
            raise ValueError(f"count range {k}: {counts.numel()} counters for {b} bytes")
        _same_gpu(buf, counts)
        lo[k], nbytes[k], cnt[k] = buf.data_ptr(), b, counts.data_ptr()
    rc = lib.conv_verify_debug_count(len(ranges), lo, nbytes, cnt)
    if rc != _lib.CV_OK:
        raise CvError(rc, _lib.error_message(lib, rc))
