"""ctypes view of libconvverify.so (the C ABI declared in include/conv_verify.h)."""

from __future__ import annotations

import contextlib
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libconvverify.so")
# The write-count build (tests only; see conv_verify_debug_count in the header).
LIB_WC_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libconvverify_wc.so")

CV_F32 = 0
CV_BF16 = 1
CV_OK = 0
CV_EINVAL = -22
CV_ENOTSUP = -95
CV_EHIP_BASE = -1000
CV_WIN_DENSE = 0
CV_WIN_ROWS = 1
CV_WIN_ROWS_T = 2
CV_VARIANT_TREE = 3
CV_LAUNCH_STATE_TIME_MAJOR = 1
CV_LAUNCH_SLOT_FIRST = 2
CV_LAUNCH_XCD_ORDER = 4
CV_LAUNCH_LINE_ALIGNED = 8
CV_LAUNCH_HEAD_BLOCKS = 16

EXPORTS = (
    "conv_verify_update_dense",
    "conv_verify_update_dedup",
    "conv_verify_update",
    "conv_verify_update_tree",
    "conv_verify_restore",
    "conv_prefill",
    "conv_qk_l2norm",
    "conv_verify_describe",
    "conv_verify_strerror",
    "conv_verify_last_error",
    "conv_verify_abi_version",
    "conv_verify_debug_count",
)


class CvShape(ctypes.Structure):
    _fields_ = [
        ("n_seq", ctypes.c_int32), ("T", ctypes.c_int32),
        ("d_inner", ctypes.c_int32), ("d_conv", ctypes.c_int32),
        ("qk_channels", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("l2_eps", ctypes.c_float),
        ("x_dtype", ctypes.c_int32), ("state_dtype", ctypes.c_int32),
        ("n_slots", ctypes.c_int32), ("state_len", ctypes.c_int32),
        ("x_seq_stride", ctypes.c_int64), ("x_tok_stride", ctypes.c_int64),
        ("out_seq_stride", ctypes.c_int64), ("out_tok_stride", ctypes.c_int64),
        ("state_slot_stride", ctypes.c_int64),
        ("win_slot_stride", ctypes.c_int64),
        ("state_col_stride", ctypes.c_int64),
    ]


class CvLaunchInfo(ctypes.Structure):
    _fields_ = [
        ("workgroups", ctypes.c_int64), ("threads", ctypes.c_int32),
        ("channel_blocks", ctypes.c_int32), ("channels_per_wave", ctypes.c_int32),
        ("channels_per_lane", ctypes.c_int32), ("token_bucket", ctypes.c_int32),
        ("lds_bytes", ctypes.c_int32), ("head_lanes", ctypes.c_int32),
        ("token_chunks", ctypes.c_int32), ("flags", ctypes.c_int32),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = _open(LIB_PATH)
    return _lib


@contextlib.contextmanager
def write_count_library():
    """Within the block, the binding calls the write-count build of the library (tests).
    The GPU is initialised first: the library's device variables are looked up by symbol,
    which fails for a code object registered before the HIP runtime found its devices."""
    import torch

    global _lib
    torch.cuda.init()
    prev = _lib
    _lib = _open(LIB_WC_PATH)
    try:
        yield _lib
    finally:
        _lib = prev


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m causal_conv1d_verify_amd.build` "
            "(or __graft_entry__.build()); the verify conv has no non-HIP implementation")
    lib = ctypes.CDLL(path)
    upd = [ctypes.POINTER(CvShape)] + [ctypes.c_void_p] * 9
    for name in ("conv_verify_update_dense", "conv_verify_update_dedup"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = upd
    P, V, I32 = ctypes.POINTER(CvShape), ctypes.c_void_p, ctypes.c_int32
    lib.conv_verify_update.restype = ctypes.c_int
    lib.conv_verify_update.argtypes = [P, I32] + [V] * 10
    lib.conv_verify_update_tree.restype = ctypes.c_int
    lib.conv_verify_update_tree.argtypes = [P] + [V] * 11
    lib.conv_verify_restore.restype = ctypes.c_int
    lib.conv_verify_restore.argtypes = [P, I32] + [V] * 5
    lib.conv_prefill.restype = ctypes.c_int
    lib.conv_prefill.argtypes = [P] + [V] * 9
    lib.conv_qk_l2norm.restype = ctypes.c_int
    lib.conv_qk_l2norm.argtypes = [P, ctypes.c_int64, ctypes.c_int64, V, V]
    lib.conv_verify_describe.restype = ctypes.c_int
    lib.conv_verify_describe.argtypes = [ctypes.c_int, ctypes.POINTER(CvShape),
                                         ctypes.POINTER(CvLaunchInfo)]
    lib.conv_verify_strerror.restype = ctypes.c_char_p
    lib.conv_verify_strerror.argtypes = [ctypes.c_int]
    lib.conv_verify_last_error.restype = ctypes.c_char_p
    lib.conv_verify_last_error.argtypes = []
    lib.conv_verify_abi_version.restype = ctypes.c_int
    lib.conv_verify_abi_version.argtypes = []
    lib.conv_verify_debug_count.restype = ctypes.c_int
    lib.conv_verify_debug_count.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                                            ctypes.POINTER(ctypes.c_uint64),
                                            ctypes.POINTER(ctypes.c_void_p)]
    return lib


def error_message(lib, code: int) -> str:
    detail = lib.conv_verify_last_error().decode()
    return f"{lib.conv_verify_strerror(code).decode()} ({code}): {detail}"
