"""Host-side tests of the C ABI: exports, validation, launch geometry.  No GPU needed.

Nothing here launches a kernel.  Shape validation goes through conv_verify_describe
(no pointers at all); the pointer checks of the update entry points run in a child
process that sees no GPU, so even a validation bug could not turn a fake pointer into
a launch.
"""

import ctypes
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv_verify.h")

lib_mod = pytest.importorskip("causal_conv1d_verify_amd._lib")


def _lib():
    if not os.path.exists(lib_mod.LIB_PATH):
        pytest.skip("libconvverify.so not built (run __graft_entry__.build())")
    return lib_mod.load()


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*CV_API\s+(?:const\s+)?\w+\s*\*?\s*(conv_\w+)\s*\(",
                                 text, re.M)))


def test_header_and_binding_agree():
    assert _header_functions() == sorted(lib_mod.EXPORTS)
    assert len(lib_mod.EXPORTS) == 12


def test_library_exports_nothing_else():
    _lib()
    res = subprocess.run(["nm", "-D", "--defined-only", lib_mod.LIB_PATH], capture_output=True,
                         text=True, check=True)
    exported = set(re.findall(r"\bT (\w+)$", res.stdout, re.M))
    assert exported == set(lib_mod.EXPORTS), sorted(exported ^ set(lib_mod.EXPORTS))


def test_write_count_library_exports_the_same_symbols():
    _lib()
    if not os.path.exists(lib_mod.LIB_WC_PATH):
        pytest.skip("libconvverify_wc.so not built")
    res = subprocess.run(["nm", "-D", "--defined-only", lib_mod.LIB_WC_PATH], capture_output=True,
                         text=True, check=True)
    exported = set(re.findall(r"\bT (\w+)$", res.stdout, re.M))
    assert exported == set(lib_mod.EXPORTS), sorted(exported ^ set(lib_mod.EXPORTS))


def test_regular_library_does_not_count_writes():
    """Only the write-count build counts: the regular library refuses, touching no GPU."""
    lib = _lib()
    rc = lib.conv_verify_debug_count(0, None, None, None)
    assert rc == lib_mod.CV_ENOTSUP
    assert b"write-count build" in lib.conv_verify_last_error()


def test_library_exports_every_declared_symbol():
    _lib()
    res = subprocess.run(["nm", "-D", "--defined-only", lib_mod.LIB_PATH], capture_output=True,
                         text=True, check=True)
    exported = set(re.findall(r"\bT (\w+)$", res.stdout, re.M))
    for name in _header_functions():
        assert name in exported, f"{name} declared in conv_verify.h but not exported"
    assert not any(n.startswith("orc_") for n in exported), "oracle code linked into the library"


def test_abi_version_matches_header():
    lib = _lib()
    want = int(re.search(r"#define CONV_VERIFY_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.conv_verify_abi_version() == want


def test_shape_struct_layout():
    # offsets of the int64 strides must match the C struct (4-byte fields then 8-aligned)
    assert lib_mod.CvShape.x_seq_stride.offset == 48
    assert ctypes.sizeof(lib_mod.CvShape) == 104
    assert lib_mod.CvShape.state_col_stride.offset == 96
    assert ctypes.sizeof(lib_mod.CvLaunchInfo) == 48
    assert lib_mod.CvLaunchInfo.flags.offset == 40


def shape(**kw):
    d = dict(n_seq=4, T=8, d_inner=1024, d_conv=4, qk_channels=512, head_dim=128, l2_eps=1e-6,
             x_dtype=lib_mod.CV_BF16, state_dtype=lib_mod.CV_BF16, n_slots=4, state_len=3,
             x_seq_stride=8 * 1024, x_tok_stride=1024, out_seq_stride=8 * 1024,
             out_tok_stride=1024, state_slot_stride=1024 * 3, win_slot_stride=8 * 1024 * 3)
    d.update(kw)
    return lib_mod.CvShape(**d)


def describe(dedup, s):
    lib = _lib()
    info = lib_mod.CvLaunchInfo()
    rc = lib.conv_verify_describe(dedup, ctypes.byref(s), ctypes.byref(info))
    return rc, info, lib.conv_verify_last_error().decode()


EINVAL, ENOTSUP = lib_mod.CV_EINVAL, lib_mod.CV_ENOTSUP
BAD_SHAPES = [
    ("n_seq<0", dict(n_seq=-1), EINVAL),
    ("T=0", dict(T=0), EINVAL),
    ("T=33", dict(T=33), ENOTSUP),
    ("d_inner<0", dict(d_inner=-8), EINVAL),
    ("d_conv=0", dict(d_conv=0), EINVAL),
    ("d_conv=1", dict(d_conv=1), ENOTSUP),
    ("d_conv=5", dict(d_conv=5), ENOTSUP),
    ("dtype=7", dict(x_dtype=7), EINVAL),
    ("f32x_bf16state", dict(x_dtype=lib_mod.CV_F32), ENOTSUP),
    ("d_inner%8", dict(d_inner=1020, qk_channels=0), ENOTSUP),
    ("qk>d", dict(qk_channels=2048), EINVAL),
    ("qk<0", dict(qk_channels=-128), EINVAL),
    ("qk%head", dict(qk_channels=520, head_dim=128), EINVAL),
    ("head<=0", dict(head_dim=0), EINVAL),
    ("head%4", dict(qk_channels=6 * 20, head_dim=6), ENOTSUP),
    # a head that does not divide 256 channels: blocks of k whole heads, k * head_dim a
    # multiple of 8 (bf16) and at most 256 - none for 132 channels (33 lanes) - and q|k's
    # end (where the 256-channel blocks start) a multiple of 8 too
    ("head_block_none", dict(qk_channels=132 * 3, head_dim=132), ENOTSUP),
    ("head_blocks_qk%8", dict(qk_channels=12 * 3, head_dim=12), ENOTSUP),
    ("head_lanes>64", dict(qk_channels=1024, head_dim=512), ENOTSUP),
    ("head_dim>256", dict(qk_channels=520, head_dim=260), ENOTSUP),
    ("eps<0", dict(l2_eps=-1.0), EINVAL),
    ("eps_nan", dict(l2_eps=float("nan")), EINVAL),
    ("eps_inf", dict(l2_eps=float("inf")), EINVAL),
    ("n_slots<0", dict(n_slots=-1), EINVAL),
    ("state_len<D-1", dict(state_len=2), EINVAL),
    ("neg_stride", dict(x_tok_stride=-1024), EINVAL),
    ("out_tok_overlap", dict(out_tok_stride=512), EINVAL),
    ("out_seq_overlap", dict(out_seq_stride=4 * 1024), EINVAL),
    ("state_slot_overlap", dict(state_slot_stride=1024), EINVAL),
    ("x_stride%8", dict(x_tok_stride=1028, x_seq_stride=8 * 1028), ENOTSUP),
    ("state_slot_unaligned", dict(state_slot_stride=3 * 1024 + 4), ENOTSUP),
    # time-major conv_state: columns of >= d_inner elements, 16-byte multiples, and a
    # slot stride covering (state_len-1) columns plus d_inner
    ("state_col<0", dict(state_col_stride=-1024), EINVAL),
    ("state_col<d", dict(state_col_stride=1016), EINVAL),
    ("state_col_unaligned", dict(state_col_stride=1028, state_slot_stride=4096), ENOTSUP),
    ("state_col_slot_overlap", dict(state_col_stride=1032, state_slot_stride=3 * 1024 + 8),
     EINVAL),
]


@pytest.mark.parametrize("name,kw,code", BAD_SHAPES, ids=[b[0] for b in BAD_SHAPES])
def test_describe_rejects(name, kw, code):
    rc, _, detail = describe(0, shape(**kw))
    assert rc == code, (rc, detail)
    assert detail, "error detail missing"


def test_window_stride_checked_per_layout():
    # dense per slot = T*d*(D-1) = 24576; both row layouts per slot = d*(T+D-2) = 10240
    assert describe(0, shape(win_slot_stride=10240))[0] == EINVAL
    assert describe(1, shape(win_slot_stride=10240))[0] == 0
    assert describe(2, shape(win_slot_stride=10240))[0] == 0
    assert describe(2, shape(win_slot_stride=10232))[0] == EINVAL
    assert describe(3, shape(win_slot_stride=10240))[0] == EINVAL   # tree: dense windows
    assert describe(3, shape())[0] == 0


def test_describe_rejects_unknown_variants():
    for v in (-1, 4, 7):
        rc, _, detail = describe(v, shape())
        assert rc == EINVAL and detail


def test_tree_lds_holds_the_tile_and_the_slabs():
    # tree: (D-1 + bucket) tile rows of 256 channels (+16 bytes pitch) and two dense slabs
    for T, tb in ((8, 8), (17, 24), (32, 32)):
        rc, info, detail = describe(3, shape(T=T, win_slot_stride=T * 1024 * 3,
                                             x_seq_stride=T * 1024, out_seq_stride=T * 1024))
        assert rc == 0, detail
        assert info.token_bucket == tb
        assert info.lds_bytes == max(2048, (3 + tb) * (256 * 2 + 16) + 2 * 256 * 3 * 2)


def test_lds_limit():
    # a 256-channel wavefront stages its [256, state_len] state rows in LDS (the weights
    # pass through the same bytes first): fp32 rows of 160 columns fill the 160 KiB
    # exactly, 161 columns do not fit
    rc, _, detail = describe(1, shape(state_dtype=lib_mod.CV_F32, state_len=161,
                                      state_slot_stride=1024 * 161, win_slot_stride=1024 * 10))
    assert rc == ENOTSUP and "LDS" in detail
    rc, info, detail = describe(1, shape(state_dtype=lib_mod.CV_F32, state_len=160,
                                         state_slot_stride=1024 * 160, win_slot_stride=1024 * 10))
    assert rc == 0, detail
    assert info.lds_bytes == 163840


def test_time_major_state_needs_no_lds_region():
    # a channel-major state row wider than the LDS limit is refused; the same state
    # stored time-major is not staged, so the LDS is that of the windows alone
    big = dict(state_dtype=lib_mod.CV_F32, state_len=161, win_slot_stride=1024 * 10)
    rc, _, detail = describe(1, shape(state_slot_stride=1024 * 161, **big))
    assert rc == ENOTSUP and "LDS" in detail
    rc, info, detail = describe(1, shape(state_slot_stride=1024 * 161, state_col_stride=1024, **big))
    assert rc == 0, detail
    assert info.lds_bytes == 256 * 10 * 4 // 2   # the fp32 row block [256, 10], in halves
    # the stress shape: 18 bf16 columns per channel, 16 tokens
    st = dict(T=16, state_len=18, x_seq_stride=16 * 1024, out_seq_stride=16 * 1024,
              win_slot_stride=1024 * 18)
    rc, cm, _ = describe(1, shape(state_slot_stride=1024 * 18, **st))
    rc2, tm, _ = describe(1, shape(state_slot_stride=1024 * 18, state_col_stride=1024, **st))
    assert rc == rc2 == 0
    assert cm.lds_bytes == 256 * 18 * 2 and tm.lds_bytes == 256 * 18 * 2 // 2
    # a padded column stride, restore and prefill take the same shape
    assert describe(0, shape(state_col_stride=1032, state_slot_stride=3 * 1032))[0] == 0


@pytest.mark.parametrize("key", [0, 1, 2, 3, 4, "4b", "4s"])
def test_launch_geometry_of_workloads(key):
    import workloads

    wl = workloads.WORKLOADS[key]
    xb = 4 if wl.x_dtype == "f32" else 2
    sb = 4 if wl.state_dtype == "f32" else 2
    xs = wl.x_tok_stride or wl.d_inner
    win = wl.row_cols * wl.d_inner if wl.layout == "dedup" else wl.T * wl.d_inner * wl.win_cols
    s = shape(n_seq=wl.n_seq, T=wl.T, d_inner=wl.d_inner, d_conv=wl.d_conv,
              qk_channels=wl.qk_channels, head_dim=wl.head_dim,
              x_dtype=lib_mod.CV_F32 if xb == 4 else lib_mod.CV_BF16,
              state_dtype=lib_mod.CV_F32 if sb == 4 else lib_mod.CV_BF16, n_slots=wl.n_slots,
              state_len=wl.state_len, x_seq_stride=wl.T * xs, x_tok_stride=xs,
              out_seq_stride=wl.T * xs, out_tok_stride=xs,
              state_slot_stride=wl.d_inner * wl.state_len, win_slot_stride=win)
    rc, info, detail = describe(int(wl.layout == "dedup"), s)
    assert rc == 0, detail
    cpl = 4
    if info.flags & lib_mod.CV_LAUNCH_LINE_ALIGNED:
        # the line-aligned build (16-token dedup rows, some store range off 128-byte
        # lines): 4 wavefronts per workgroup over 1024 channels; LDS for the larger of the
        # staged state region (after one line) followed by the exchange buffers, and the
        # row block (after one line)
        assert wl.T == 16 and wl.layout == "dedup"
        assert (xs * xb) % 128 or (wl.d_inner * wl.state_len * sb) % 128 \
            or (wl.d_inner * wl.row_cols * sb) % 128
        assert info.threads == 256 and info.channels_per_wave == 256
        assert info.channel_blocks == -(-wl.d_inner // 1024) and info.token_chunks == 1
        assert info.workgroups == wl.n_seq * info.channel_blocks
        region = -(-(128 + 1024 * wl.state_len * sb) // 16) * 16
        assert info.lds_bytes == max(region + 2 * 4 * 1024 * xb, 128 + 1024 * wl.row_cols * sb)
        assert info.lds_bytes * 3 <= 163840
        return
    assert info.channels_per_lane == cpl and info.threads == 64
    assert info.channels_per_wave == 64 * cpl
    assert info.channel_blocks == -(-wl.d_inner // (64 * cpl))
    # the grid covers every (row, channel block, token chunk) exactly once
    assert info.workgroups == wl.n_seq * info.channel_blocks * info.token_chunks
    assert info.channel_blocks * info.channels_per_wave >= wl.d_inner
    assert (info.channel_blocks - 1) * info.channels_per_wave < wl.d_inner
    assert info.token_bucket * info.token_chunks >= wl.T
    assert info.token_bucket * (info.token_chunks - 1) < wl.T
    plain = wl.n_seq * info.channel_blocks
    chunks = -(-wl.T // 4)
    # token split: dense chains when the split grid has at most 5120 wavefronts; row
    # layouts (buckets 8 and 16) at most 2560
    split = wl.layout == "dense" and wl.T >= 8 and plain * chunks <= 5120
    rows_split = wl.layout != "dense" and 4 < wl.T <= 16 and plain * chunks <= 2560
    assert (info.token_chunks > 1) == (split or rows_split), (plain, wl.T)
    if split:
        assert info.token_bucket == 4
    else:
        assert info.token_bucket >= wl.T and info.token_bucket < 2 * wl.T + 1
    assert info.head_lanes * cpl == wl.head_dim
    # while loading: the weights (in whole 1 KiB load widths), then the state region
    # over the same bytes
    first = max(64 * cpl * wl.state_len * sb, -(-(64 * cpl * wl.d_conv * xb) // 1024) * 1024)
    if wl.layout == "dedup":
        # T is a bucket here: the row block [256, T+D-2] is staged lane by lane, in two
        # halves when it is over 8 KiB
        block = 64 * cpl * wl.row_cols * sb
        later = block // 2 if block > 8192 else block
    else:
        later = 64 * cpl * wl.win_cols * sb * (2 if wl.T > 1 else 1)
    if split:   # chunk 0's state region, the weights, two snapshot slabs
        first = 64 * cpl * wl.state_len * sb + -(-(64 * cpl * wl.d_conv * xb) // 1024) * 1024
        later = 2 * 64 * cpl * wl.win_cols * sb
        assert info.lds_bytes == first + later
    else:
        assert info.lds_bytes == max(first, later) <= 65536


_CHILD = r"""
import ctypes, json, sys
sys.path.insert(0, sys.argv[1])
from causal_conv1d_verify_amd import _lib as L
lib = L.load()
def shape(**kw):
    d = dict(n_seq=4, T=8, d_inner=1024, d_conv=4, qk_channels=512, head_dim=128, l2_eps=1e-6,
             x_dtype=L.CV_BF16, state_dtype=L.CV_BF16, n_slots=4, state_len=3,
             x_seq_stride=8192, x_tok_stride=1024, out_seq_stride=8192, out_tok_stride=1024,
             state_slot_stride=3072, win_slot_stride=24576)
    d.update(kw)
    return L.CvShape(**d)
A = 0x10000   # a 16-byte aligned stand-in address; never dereferenced on the host
res = {}
def call(name, dedup, s, ptrs):
    fn = lib.conv_verify_update_dedup if dedup else lib.conv_verify_update_dense
    rc = fn(ctypes.byref(s), *ptrs, None)
    res[name] = [rc, lib.conv_verify_last_error().decode()]
good = [A, A, None, A, None, None, A, A]
res["null_shape"] = [lib.conv_verify_update_dense(None, *good, None), ""]
call("null_x", 0, shape(), [None] + good[1:])
call("null_weight", 0, shape(), [A, None] + good[2:])
call("null_state", 1, shape(win_slot_stride=10240), [A, A, None, None, None, None, A, A])
call("null_out", 0, shape(), [A, A, None, A, None, None, None, A])
call("null_win", 1, shape(win_slot_stride=10240), [A, A, None, A, None, None, A, None])
call("misaligned_x", 0, shape(), [A + 2] + good[1:])
call("misaligned_bias", 0, shape(), [A, A, A + 8, A, None, None, A, A])
call("misaligned_win", 0, shape(), good[:7] + [A + 4])
call("identity_slots_short", 0, shape(n_slots=3), good)
call("empty_batch_no_pointers", 0, shape(n_seq=0), [None] * 8)
call("empty_channels_no_pointers", 1, shape(d_inner=0, qk_channels=0, win_slot_stride=0,
                                            state_slot_stride=0), [None] * 8)
def rc_of(name, rc):
    res[name] = [rc, lib.conv_verify_last_error().decode()]
s = shape()
rc_of("general_bad_layout", lib.conv_verify_update(ctypes.byref(s), 3, A, A, None, A, None,
                                                    None, None, A, A, None))
rc_of("general_rows_t_ok_empty", lib.conv_verify_update(ctypes.byref(shape(n_seq=0)), 2, *([None] * 10)))
rc_of("tree_null_parent", lib.conv_verify_update_tree(ctypes.byref(s), A, A, None, A, None, None,
                                                       None, None, A, A, None))
rc_of("restore_null_index", lib.conv_verify_restore(ctypes.byref(s), 0, A, A, None, None, None))
rc_of("restore_bad_layout", lib.conv_verify_restore(ctypes.byref(s), 5, A, A, None, A, None))
rc_of("restore_misaligned", lib.conv_verify_restore(ctypes.byref(s), 0, A + 2, A, None, A, None))
rc_of("restore_T33", lib.conv_verify_restore(ctypes.byref(shape(T=33)), 0, A, A, None, A, None))
ps = shape(T=100, x_tok_stride=1024, out_tok_stride=1024)
rc_of("prefill_null_cu", lib.conv_prefill(ctypes.byref(ps), A, A, None, A, None, None, None, A, None))
rc_of("prefill_tok_overlap", lib.conv_prefill(ctypes.byref(shape(T=100, x_tok_stride=512)),
                                              A, A, None, A, None, A, None, A, None))
rc_of("prefill_empty_ok", lib.conv_prefill(ctypes.byref(shape(n_seq=0, T=100)), *([None] * 9)))
rc_of("l2_null_x", lib.conv_qk_l2norm(ctypes.byref(s), 4, 1024, None, None))
rc_of("l2_bad_head", lib.conv_qk_l2norm(ctypes.byref(shape(head_dim=132, qk_channels=396)), 4, 1024, A, None))
rc_of("l2_short_stride", lib.conv_qk_l2norm(ctypes.byref(s), 4, 256, A, None))
rc_of("l2_no_rows_ok", lib.conv_qk_l2norm(ctypes.byref(s), 0, 1024, None, None))
print(json.dumps(res))
"""


def test_update_entry_points_validate_before_launch():
    _lib()
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    out = subprocess.run([sys.executable, "-c", _CHILD, ROOT], capture_output=True, text=True,
                         env=env, timeout=120)
    assert out.returncode == 0, out.stderr
    res = json.loads(out.stdout.strip().splitlines()[-1])
    expect = {
        "null_shape": EINVAL, "null_x": EINVAL, "null_weight": EINVAL, "null_state": EINVAL,
        "null_out": EINVAL, "null_win": EINVAL, "misaligned_x": ENOTSUP,
        "misaligned_bias": ENOTSUP, "misaligned_win": ENOTSUP,
        "identity_slots_short": EINVAL, "empty_batch_no_pointers": 0,
        "empty_channels_no_pointers": 0,
        "general_bad_layout": EINVAL, "general_rows_t_ok_empty": 0, "tree_null_parent": EINVAL,
        "restore_null_index": EINVAL, "restore_bad_layout": EINVAL,
        "restore_misaligned": ENOTSUP, "restore_T33": ENOTSUP, "prefill_null_cu": EINVAL,
        "prefill_tok_overlap": EINVAL, "prefill_empty_ok": 0, "l2_null_x": EINVAL,
        "l2_bad_head": ENOTSUP, "l2_short_stride": EINVAL, "l2_no_rows_ok": 0,
    }
    for k, code in expect.items():
        assert res[k][0] == code, (k, res[k])


def test_strerror_covers_codes():
    lib = _lib()
    for code in (0, EINVAL, ENOTSUP, lib_mod.CV_EHIP_BASE - 1, 12345):
        assert lib.conv_verify_strerror(code)


def test_product_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "causal_conv1d_verify_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "conv_verify_oracle" not in text and "liboracle" not in text, f


def test_abi_from_plain_c(tmp_path):
    """The header and the library used from C: gcc compiles tests/c/abi_from_c.c against
    include/conv_verify.h, links libconvverify.so and runs it (no GPU: every call is
    host-side validation or geometry)."""
    _lib()
    exe = tmp_path / "abi_from_c"
    libdir = os.path.dirname(lib_mod.LIB_PATH)
    cc = subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror",
                         f"-I{os.path.join(ROOT, 'include')}",
                         os.path.join(ROOT, "tests", "c", "abi_from_c.c"),
                         f"-L{libdir}", "-lconvverify", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "MISMATCH" not in run.stdout


def test_binding_state_views():
    """The binding reads the conv_state order from the tensor's view: a contiguous
    [n_slots, d, state_len] is channel-major (state_col_stride 0); the transposed view
    of a [n_slots, state_len, >= d] buffer is time-major with its column stride; any
    other view is refused."""
    import torch

    import causal_conv1d_verify_amd as cv

    n, d, sl = 3, 1032, 10
    assert cv._check_state(torch.zeros(n, d, sl), d) == 0
    tm = torch.zeros(n, sl, d)
    assert cv._check_state(tm.transpose(1, 2), d) == d
    padded = torch.zeros(n, sl, d + 8)[:, :, :d]
    assert cv._check_state(padded.transpose(1, 2), d) == d + 8
    # a state width of one column is the same memory in both orders
    assert cv._check_state(torch.zeros(n, 1, d).transpose(1, 2), d) == 0
    with pytest.raises(ValueError):
        cv._check_state(torch.zeros(n, sl, d), d)                      # wrong shape
    with pytest.raises(ValueError):
        cv._check_state(torch.zeros(n, d, 2 * sl)[:, :, ::2], d)       # strided columns
    # (a view whose slots overlap each other's columns passes here and is refused by the
    # library's slot-stride check: test_describe_rejects[state_col_slot_overlap])


def _flags(layout, **kw):
    rc, info, detail = describe(layout, shape(**kw))
    assert rc == 0, detail
    return info.workgroups, info.token_chunks, info.flags


def test_launch_flags_edges():
    """The data-movement choices reported by conv_verify_describe, on both sides of
    each rule: slot-first past one resident generation (5,120 wavefronts), the XCD
    order for a partial channel block, the time-major state build."""
    L = lib_mod
    rows = lambda n, T, d=10240: dict(n_seq=n, n_slots=n, T=T, d_inner=d, x_seq_stride=T * d,   # noqa: E731
                                      x_tok_stride=d, out_seq_stride=T * d, out_tok_stride=d,
                                      state_slot_stride=3 * d, win_slot_stride=d * (T + 2),
                                      qk_channels=4096)
    # the headline shape: 128 rows x 40 blocks = 5,120 wavefronts, exactly one generation
    wg, ch, f = _flags(1, **rows(128, 8))
    assert (wg, ch, f) == (5120, 1, 0)
    wg, ch, f = _flags(1, **rows(129, 8))
    assert wg == 5160 and f == L.CV_LAUNCH_SLOT_FIRST
    # a token-split grid counts its split wavefronts
    wg, ch, f = _flags(1, **rows(8, 16))
    assert ch == 4 and f == 0
    # a partial last channel block: the XCD order
    assert _flags(1, **rows(128, 8, d=10200))[2] == L.CV_LAUNCH_XCD_ORDER
    assert _flags(1, **rows(128, 8, d=10496))[2] & L.CV_LAUNCH_XCD_ORDER == 0
    # the time-major conv_state build
    f = _flags(1, **dict(rows(128, 8), state_col_stride=10240))[2]
    assert f == L.CV_LAUNCH_STATE_TIME_MAJOR
    # the line-aligned build: bf16, time-major state, dedup rows, T 16; 4-wavefront
    # workgroups over 1024 channels
    tm16 = lambda n, d, **kw: dict(rows(n, 16, d), state_col_stride=10240,   # noqa: E731
                                   state_slot_stride=10240 * 3, **kw)
    wg, ch, f = _flags(1, **tm16(512, 10200))
    assert wg == 512 * 10 and ch == 1
    assert f == L.CV_LAUNCH_STATE_TIME_MAJOR | L.CV_LAUNCH_SLOT_FIRST | L.CV_LAUNCH_LINE_ALIGNED
    # one generation is 5,120 wavefronts = 1,280 such workgroups
    assert _flags(1, **tm16(128, 10200))[2] & L.CV_LAUNCH_SLOT_FIRST == 0
    assert _flags(1, **tm16(129, 10200))[2] & L.CV_LAUNCH_SLOT_FIRST
    assert _flags(1, **tm16(512, 10240))[2] & L.CV_LAUNCH_LINE_ALIGNED
    # a channel-major state: only where a store range (rows of out, state regions, row
    # blocks) starts off lines, and its region (1024 channels x state_len) and the exchange
    # buffers fit 3 workgroups per compute unit
    f = _flags(1, **rows(512, 16, 10200))[2]
    assert f == L.CV_LAUNCH_LINE_ALIGNED | L.CV_LAUNCH_XCD_ORDER | L.CV_LAUNCH_SLOT_FIRST
    assert _flags(1, **rows(512, 16, 10240))[2] & L.CV_LAUNCH_LINE_ALIGNED == 0
    out_on_lines = dict(rows(512, 16, 10200), x_tok_stride=10240, out_tok_stride=10240,
                        x_seq_stride=16 * 10240, out_seq_stride=16 * 10240)
    assert _flags(1, **out_on_lines)[2] & L.CV_LAUNCH_LINE_ALIGNED
    all_on_lines = dict(out_on_lines, state_slot_stride=10240 * 3, win_slot_stride=10240 * 18)
    assert _flags(1, **all_on_lines)[2] == L.CV_LAUNCH_XCD_ORDER | L.CV_LAUNCH_SLOT_FIRST
    edge = dict(rows(512, 16, 10200), state_len=18, state_slot_stride=10200 * 18)
    assert _flags(1, **edge)[2] & L.CV_LAUNCH_LINE_ALIGNED
    wide = dict(rows(512, 16, 10200), state_len=19, state_slot_stride=10200 * 19)
    assert _flags(1, **wide)[2] & L.CV_LAUNCH_LINE_ALIGNED == 0
    # not for 15 tokens, dense windows or fp32
    assert _flags(1, **dict(rows(512, 15, 10200), state_col_stride=10240,
                            state_slot_stride=10240 * 3))[2] & L.CV_LAUNCH_LINE_ALIGNED == 0
    dense = dict(tm16(512, 10200), win_slot_stride=16 * 10200 * 3)
    assert _flags(0, **dense)[2] & L.CV_LAUNCH_LINE_ALIGNED == 0
    f32 = dict(tm16(512, 10200), x_dtype=L.CV_F32, state_dtype=L.CV_F32)
    assert _flags(1, **f32)[2] & L.CV_LAUNCH_LINE_ALIGNED == 0
    # a small grid takes the token split instead
    wg, ch, f = _flags(1, **tm16(8, 10200))
    assert ch == 4 and f & L.CV_LAUNCH_LINE_ALIGNED == 0


def _head_block(head_dim, align):
    """Channels per q|k block for a head that does not divide 256: the most whole heads
    within 256 channels whose channel count is a multiple of align."""
    k = 256 // head_dim
    while k and (k * head_dim) % align:
        k -= 1
    return k * head_dim


@pytest.mark.parametrize("head_dim", [12, 20, 24, 48, 80, 96, 112, 160, 192, 240, 252])
@pytest.mark.parametrize("dtypes", ["bf16", "f32", "bf16_f32"])
def test_head_blocks_geometry(head_dim, dtypes):
    """Heads that do not divide 256 channels: the q|k channels go in blocks of whole heads
    (then 256-channel blocks from qk on), the grid covers every block once, and no such
    launch takes the line-aligned build (whose workgroups span 1024 channels)."""
    L = lib_mod
    xd, sd = {"bf16": (L.CV_BF16, L.CV_BF16), "f32": (L.CV_F32, L.CV_F32),
              "bf16_f32": (L.CV_BF16, L.CV_F32)}[dtypes]
    align = 16 // min(2 if xd == L.CV_BF16 else 4, 2 if sd == L.CV_BF16 else 4)
    heads = 8 if head_dim % 8 == 0 or align == 4 else 6
    qk = heads * head_dim
    d = qk + 1000 + (align - (qk + 1000) % align) % align
    for layout, T, tm in ((1, 16, 0), (1, 16, d), (0, 8, 0), (2, 3, d), (1, 1, 0)):
        win = d * (T + 2) if layout else T * d * 3
        s = shape(n_seq=37, n_slots=37, T=T, d_inner=d, qk_channels=qk, head_dim=head_dim,
                  x_dtype=xd, state_dtype=sd, x_seq_stride=T * d, x_tok_stride=d,
                  out_seq_stride=T * d, out_tok_stride=d, state_len=3, state_slot_stride=3 * d,
                  state_col_stride=tm, win_slot_stride=win)
        rc, info, detail = describe(layout, s)
        ch = _head_block(head_dim, align)
        if ch == 0:
            assert rc == ENOTSUP, (rc, detail)
            return
        assert rc == 0, detail
        assert info.flags & L.CV_LAUNCH_HEAD_BLOCKS
        assert info.flags & L.CV_LAUNCH_LINE_ALIGNED == 0 and info.threads == 64
        assert info.head_lanes * 4 == head_dim
        assert info.channel_blocks == -(-qk // ch) + -(-(d - qk) // 256)
        assert info.workgroups == 37 * info.channel_blocks * info.token_chunks
    # the separate L2 takes the same blocks of whole heads (x's element size only)
    lib = _lib()
    rc = lib.conv_qk_l2norm(ctypes.byref(shape(d_inner=d, qk_channels=qk, head_dim=head_dim, x_dtype=xd,
                                               state_dtype=xd)), 0, d, None, None)
    assert rc == 0, lib.conv_verify_last_error().decode()


def test_power_of_two_heads_keep_uniform_blocks():
    for hd in (4, 8, 16, 32, 64, 128, 256):
        rc, info, detail = describe(1, shape(qk_channels=hd * 2, head_dim=hd))
        assert rc == 0, detail
        assert info.flags & lib_mod.CV_LAUNCH_HEAD_BLOCKS == 0
        assert info.channel_blocks == 4 and info.head_lanes * 4 == hd


def test_line_aligned_geometry():
    """The line-aligned build's grid covers every (row, 1024-channel range) once, with
    4 wavefronts per workgroup and LDS for the workgroup's row block after up to 112
    bytes of its first line (or two 4-token buffers of out, if larger)."""
    for d, d_conv in ((10200, 4), (1032, 3), (2600, 2), (136, 4), (10240, 4)):
        cols = 16 + d_conv - 2
        s = shape(n_seq=700, n_slots=700, T=16, d_inner=d, d_conv=d_conv, qk_channels=0,
                  x_seq_stride=16 * d, x_tok_stride=d, out_seq_stride=16 * d, out_tok_stride=d,
                  state_len=d_conv - 1, state_col_stride=d + 8,
                  state_slot_stride=(d + 8) * (d_conv - 1), win_slot_stride=d * cols)
        rc, info, detail = describe(1, s)
        assert rc == 0, detail
        assert info.flags & lib_mod.CV_LAUNCH_LINE_ALIGNED, d
        assert info.threads == 256 and info.channels_per_wave == 256
        assert info.channel_blocks == -(-d // 1024)
        assert info.workgroups == 700 * info.channel_blocks
        assert info.lds_bytes == max(2 * 4 * 1024 * 2, 128 + 1024 * cols * 2)


def test_binding_refuses_window_buffers_with_fewer_slots():
    """Windows are indexed by slot: a buffer with fewer slots than conv_state would let
    a valid slot address past its end, so the binding refuses it before any launch."""
    torch = pytest.importorskip("torch")
    import causal_conv1d_verify_amd as cv

    n, d, sl, T = 6, 256, 3, 4
    state = torch.zeros(n, d, sl)
    assert cv._check_window_slots(state, torch.zeros(n, T, d, 3)) == n
    assert cv._check_window_slots(state, torch.zeros(n + 2, d, T + 2)) == n
    with pytest.raises(ValueError, match="indexed by slot"):
        cv._check_window_slots(state, torch.zeros(n - 1, d, T + 2))
