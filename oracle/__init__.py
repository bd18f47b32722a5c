"""CPU oracle for the batched speculative-verify causal conv1d update (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: the plain per-token reference the HIP library is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU baseline leg of
``bench.py`` may import it; the product package never does, and this package imports
nothing from the product.  The arithmetic lives in ``conv_verify_oracle.c``; this
module only marshals numpy arrays.

bf16 arrays are numpy ``uint16`` bit patterns, fp32 arrays ``float32``.

Parity pins (see tests/test_oracle_*.py): fp64 brute force over the whole sequence
(bit-exact on dyadic inputs), torch's depthwise conv1d + SiLU for qk_channels = 0,
one-hot taps, L2 and window invariants, offset equivalence, batched == per-row
calls, a golden fixture of the window indexing, and planted-mistake mutants.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import numpy as np

from . import build as _build


class OrcProblem(ctypes.Structure):
    _fields_ = [
        ("n_seq", ctypes.c_int32), ("n_tok", ctypes.c_int32),
        ("d_inner", ctypes.c_int32), ("d_conv", ctypes.c_int32),
        ("qk_channels", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("l2_eps", ctypes.c_float),
        ("x_bf16", ctypes.c_int32), ("state_bf16", ctypes.c_int32),
        ("n_slots", ctypes.c_int32), ("state_len", ctypes.c_int32),
        ("x_seq_stride", ctypes.c_int64), ("x_tok_stride", ctypes.c_int64),
        ("out_seq_stride", ctypes.c_int64), ("out_tok_stride", ctypes.c_int64),
        ("state_slot_stride", ctypes.c_int64),
        ("dedup", ctypes.c_int32),
        ("win_slot_stride", ctypes.c_int64),
    ]


class OrcExt(ctypes.Structure):
    _fields_ = [
        ("layout", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("parent", ctypes.c_void_p),
        ("parent_stride", ctypes.c_int64),
        ("has_init", ctypes.c_void_p),
        ("do_l2", ctypes.c_int32),
        ("commit", ctypes.c_int32),
    ]


LAYOUTS = {"dense": 0, "dedup": 1, "dedup_t": 2}

_LIBS: dict = {}


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the oracle library (building it first if needed), or a given build of it."""
    if path is None:
        path = _build.ensure_built()
    if path not in _LIBS:
        lib = ctypes.CDLL(path)
        lib.orc_conv_verify.restype = ctypes.c_int
        lib.orc_conv_verify.argtypes = [ctypes.POINTER(OrcProblem)] + [ctypes.c_void_p] * 10
        lib.orc_verify_general.restype = ctypes.c_int
        lib.orc_verify_general.argtypes = [ctypes.POINTER(OrcProblem), ctypes.POINTER(OrcExt)] + \
            [ctypes.c_void_p] * 10
        lib.orc_restore.restype = ctypes.c_int
        lib.orc_restore.argtypes = [ctypes.POINTER(OrcProblem), ctypes.c_int] + [ctypes.c_void_p] * 4
        lib.orc_l2norm.restype = ctypes.c_int
        lib.orc_l2norm.argtypes = [ctypes.POINTER(OrcProblem), ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_void_p]
        lib.orc_round_bf16.restype = ctypes.c_uint16
        lib.orc_round_bf16.argtypes = [ctypes.c_double]
        lib.orc_round_f32.restype = ctypes.c_float
        lib.orc_round_f32.argtypes = [ctypes.c_double]
        _LIBS[path] = lib
    return _LIBS[path]


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _elem_strides(a: np.ndarray):
    return [s // a.itemsize for s in a.strides]


def _np_for(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


def conv_verify(x: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray],
                conv_state: np.ndarray, out: np.ndarray, windows: np.ndarray, *,
                d_inner: int, qk_channels: int, head_dim: int, l2_eps: float,
                x_dtype: str, state_dtype: str, layout: str,
                slot_idx: Optional[np.ndarray] = None,
                num_accept_tokens: Optional[np.ndarray] = None,
                debug: bool = False, lib: Optional[ctypes.CDLL] = None):
    """Run the oracle.  conv_state, out and windows are updated in place.

    x: [n_seq, T, >=d_inner] (channel stride 1), weight: [d_inner, d_conv],
    bias: [d_inner] or None, conv_state: [n_slots, d_inner, state_len],
    out: [n_seq, T, >=d_inner], windows: dense [n_slots, T, d_inner, d_conv-1] or
    dedup [n_slots, d_inner, T+d_conv-2].  Returns (pre, y) debug arrays if debug.
    """
    lib = lib or load()
    n_seq, T, _ = x.shape
    d_conv = weight.shape[1]
    n_slots, _, state_len = conv_state.shape
    xd, sd = _np_for(x_dtype), _np_for(state_dtype)
    for name, arr, dt in (("x", x, xd), ("weight", weight, xd), ("bias", bias, xd),
                          ("out", out, xd), ("conv_state", conv_state, sd),
                          ("windows", windows, sd)):
        if arr is not None and arr.dtype != dt:
            raise TypeError(f"{name} must be {np.dtype(dt)}, got {arr.dtype}")
    xs, os_, ss, ws = (_elem_strides(a) for a in (x, out, conv_state, windows))
    if xs[2] != 1 or os_[2] != 1 or ss[2] != 1 or ss[1] != state_len:
        raise ValueError("channel-contiguous x/out and [n_slots, d_inner, state_len] state required")
    if not (weight.flags.c_contiguous and (bias is None or bias.flags.c_contiguous)):
        raise ValueError("weight and bias must be contiguous")
    if list(windows.strides[1:]) != list(np.empty(windows.shape[1:], windows.dtype).strides):
        raise ValueError("windows must be contiguous below the slot dimension")
    p = OrcProblem(
        n_seq=n_seq, n_tok=T, d_inner=d_inner, d_conv=d_conv,
        qk_channels=qk_channels, head_dim=head_dim, l2_eps=l2_eps,
        x_bf16=int(x_dtype == "bf16"), state_bf16=int(state_dtype == "bf16"),
        n_slots=n_slots, state_len=state_len,
        x_seq_stride=xs[0], x_tok_stride=xs[1],
        out_seq_stride=os_[0], out_tok_stride=os_[1],
        state_slot_stride=ss[0], dedup=int(layout == "dedup"), win_slot_stride=ws[0],
    )
    slot = None if slot_idx is None else np.ascontiguousarray(slot_idx, dtype=np.int32)
    nat = None if num_accept_tokens is None else np.ascontiguousarray(num_accept_tokens,
                                                                       dtype=np.int32)
    pre = np.zeros((n_seq, T, d_inner), np.float32) if debug else None
    y = np.zeros((n_seq, T, d_inner), np.float64) if debug else None
    rc = lib.orc_conv_verify(ctypes.byref(p), _ptr(x), _ptr(weight), _ptr(bias),
                             _ptr(conv_state), _ptr(slot), _ptr(nat), _ptr(out),
                             _ptr(windows), _ptr(pre), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return (pre, y) if debug else None


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def verify_general(x: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray],
                   conv_state: np.ndarray, out: np.ndarray, windows: Optional[np.ndarray], *,
                   T: int, d_inner: int, qk_channels: int, head_dim: int, l2_eps: float,
                   x_dtype: str, state_dtype: str, layout: str = "dense",
                   slot_idx=None, num_accept_tokens=None, cu_seqlens=None, parent=None,
                   has_init=None, do_l2: bool = True, commit: bool = True,
                   debug: bool = False, lib: Optional[ctypes.CDLL] = None):
    """The general per-token loop (packed rows, tree parents, all window layouts).

    x/out: [n_seq, T, >=d_inner], or packed [total, >=d_inner] when cu_seqlens is given.
    windows: the layout's [n_slots, ...] buffer with T draft positions, or None.
    parent: [n_seq, T] int32 (-1 = the row's starting window), dense windows only.
    Returns (pre, y) debug arrays ([n_seq, T, d_inner]) if debug.
    """
    lib = lib or load()
    n_seq = (len(cu_seqlens) - 1) if cu_seqlens is not None else x.shape[0]
    d_conv = weight.shape[1]
    n_slots, _, state_len = conv_state.shape
    xd, sd = _np_for(x_dtype), _np_for(state_dtype)
    for name, arr, dt in (("x", x, xd), ("weight", weight, xd), ("bias", bias, xd),
                          ("out", out, xd), ("conv_state", conv_state, sd),
                          ("windows", windows, sd)):
        if arr is not None and arr.dtype != dt:
            raise TypeError(f"{name} must be {np.dtype(dt)}, got {arr.dtype}")
    xs, os_, ss = (_elem_strides(a) for a in (x, out, conv_state))
    if xs[-1] != 1 or os_[-1] != 1 or ss[2] != 1 or ss[1] != state_len:
        raise ValueError("channel-contiguous x/out and [n_slots, d_inner, state_len] state required")
    if windows is not None and list(windows.strides[1:]) != list(
            np.empty(windows.shape[1:], windows.dtype).strides):
        raise ValueError("windows must be contiguous below the slot dimension")
    packed = cu_seqlens is not None
    p = OrcProblem(
        n_seq=n_seq, n_tok=T, d_inner=d_inner, d_conv=d_conv,
        qk_channels=qk_channels, head_dim=head_dim, l2_eps=l2_eps,
        x_bf16=int(x_dtype == "bf16"), state_bf16=int(state_dtype == "bf16"),
        n_slots=n_slots, state_len=state_len,
        x_seq_stride=0 if packed else xs[0], x_tok_stride=xs[0] if packed else xs[1],
        out_seq_stride=0 if packed else os_[0], out_tok_stride=os_[0] if packed else os_[1],
        state_slot_stride=ss[0], dedup=int(layout == "dedup"),
        win_slot_stride=0 if windows is None else _elem_strides(windows)[0],
    )
    cu, par, hi = _i32(cu_seqlens), _i32(parent), _i32(has_init)
    e = OrcExt(layout=LAYOUTS[layout], cu_seqlens=_ptr(cu), parent=_ptr(par),
               parent_stride=0 if par is None else par.shape[1], has_init=_ptr(hi),
               do_l2=int(do_l2), commit=int(commit))
    slot, nat = _i32(slot_idx), _i32(num_accept_tokens)
    pre = np.zeros((n_seq, T, d_inner), np.float32) if debug else None
    y = np.zeros((n_seq, T, d_inner), np.float64) if debug else None
    rc = lib.orc_verify_general(ctypes.byref(p), ctypes.byref(e), _ptr(x), _ptr(weight),
                                _ptr(bias), _ptr(conv_state), _ptr(slot), _ptr(nat),
                                _ptr(out), _ptr(windows), _ptr(pre), _ptr(y))
    if rc != 0:
        raise ValueError(f"oracle rejected the problem (code {rc})")
    return (pre, y) if debug else None


def restore(conv_state: np.ndarray, windows: np.ndarray, win_k, *, T: int, d_conv: int,
            state_dtype: str, layout: str, slot_idx=None, lib: Optional[ctypes.CDLL] = None):
    """Accepted-prefix restore, in place on conv_state: window win_k[i] of row i's slot
    becomes columns 0..d_conv-2 of its state (win_k = -1 or slot -1: nothing)."""
    lib = lib or load()
    n_slots, d_inner, state_len = conv_state.shape
    ss = _elem_strides(conv_state)
    k = _i32(win_k)
    p = OrcProblem(n_seq=len(k), n_tok=T, d_inner=d_inner, d_conv=d_conv,
                   x_bf16=1 if state_dtype == "bf16" else 0,
                   state_bf16=int(state_dtype == "bf16"), n_slots=n_slots,
                   state_len=state_len, state_slot_stride=ss[0],
                   dedup=int(layout == "dedup"), win_slot_stride=_elem_strides(windows)[0])
    rc = lib.orc_restore(ctypes.byref(p), LAYOUTS[layout], _ptr(conv_state), _ptr(windows),
                         _ptr(_i32(slot_idx)), _ptr(k))
    if rc != 0:
        raise ValueError(f"oracle rejected the restore (code {rc})")


def l2norm(x: np.ndarray, *, d_inner: int, qk_channels: int, head_dim: int, l2_eps: float,
           x_dtype: str, lib: Optional[ctypes.CDLL] = None):
    """Separate per-head L2 over the q|k channels of each row of x ([rows, >=d_inner]),
    in place."""
    lib = lib or load()
    xs = _elem_strides(x)
    if xs[-1] != 1 or x.ndim != 2:
        raise ValueError("x must be [rows, >=d_inner] with unit channel stride")
    p = OrcProblem(n_seq=0, n_tok=1, d_inner=d_inner, d_conv=2, qk_channels=qk_channels,
                   head_dim=head_dim, l2_eps=l2_eps, x_bf16=int(x_dtype == "bf16"))
    rc = lib.orc_l2norm(ctypes.byref(p), x.shape[0], xs[0], _ptr(x))
    if rc != 0:
        raise ValueError(f"oracle rejected the L2 problem (code {rc})")


def prefill(x: np.ndarray, weight: np.ndarray, bias: Optional[np.ndarray],
            conv_state: np.ndarray, out: np.ndarray, cu_seqlens, *, d_inner: int,
            x_dtype: str, state_dtype: str, slot_idx=None, has_init=None,
            lib: Optional[ctypes.CDLL] = None):
    """Prefill conv over packed prompts: conv + SiLU only (no L2, no rollback windows),
    each row starting from its state window (or zeros where has_init is 0) and leaving
    its last window in conv_state.  x/out: [total, >=d_inner]."""
    cu = _i32(cu_seqlens)
    t_max = max(1, int(np.max(np.diff(cu))) if len(cu) > 1 else 1)
    verify_general(x, weight, bias, conv_state, out, None, T=t_max, d_inner=d_inner,
                   qk_channels=0, head_dim=1, l2_eps=0.0, x_dtype=x_dtype,
                   state_dtype=state_dtype, slot_idx=slot_idx, cu_seqlens=cu,
                   has_init=has_init, do_l2=False, commit=True, lib=lib)


def round_bf16(v: float) -> int:
    return int(load().orc_round_bf16(float(v)))


def run_inputs(inp, debug: bool = False, lib: Optional[ctypes.CDLL] = None):
    """Run the oracle on a ``workloads.Inputs`` problem with poison-filled outputs.

    Returns a dict with ``out``, ``windows``, ``conv_state`` (the updated copy) and,
    with debug, ``pre`` and ``y``.  The inputs themselves are not modified.
    """
    import workloads  # the shared seeded-input module (no method arithmetic)

    wl = inp.wl
    state = inp.conv_state.copy()
    out = workloads.poison(inp.x.shape, wl.x_dtype)
    windows = workloads.poison_like_windows(wl)
    r = conv_verify(inp.x, inp.weight, inp.bias, state, out, windows,
                    d_inner=wl.d_inner, qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                    l2_eps=wl.l2_eps, x_dtype=wl.x_dtype, state_dtype=wl.state_dtype,
                    layout=wl.layout, slot_idx=inp.slot_idx,
                    num_accept_tokens=inp.num_accept_tokens, debug=debug, lib=lib)
    res = {"out": out, "windows": windows, "conv_state": state}
    if debug:
        res["pre"], res["y"] = r
    return res
