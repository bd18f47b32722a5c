"""Single-writer check of every output buffer, on the GPU.

The write-count build of the library (libconvverify_wc.so: the same sources compiled with
CV_WRITE_COUNT; its verify kernels cover bf16 x and state, plus every restore, prefill and
L2 kernel) also adds 1, per 2-byte unit, to a counter for every global store a launch
makes into a registered range.  Registered here: out, the rollback windows and the whole
conv_state allocation.  For each launch:

* no unit is written more than once (one writer per element: no double or racing store);
* every unit whose bits changed was written by a counted store (the instrumentation sees
  every store that lands);
* the instrumented kernels still match the oracle (the counting does not change results).

The problems are small versions of the bench shapes, covering every launch kind: chain
verify in the three window layouts with both conv_state orders (and padded rows, offsets,
a partial channel block), packed rows, the token splits, the 5-wavefront 16-token build,
the line-aligned build, heads that do not divide 256 channels (blocks of whole heads),
tree verify, the restore from each layout, the prefill and the separate L2.
"""

import numpy as np
import pytest

import gpu_harness as gh
import workloads

pytestmark = pytest.mark.gpu

c = workloads.custom


def _units(t):
    import torch

    return t.contiguous().view(torch.int16).flatten().cpu().numpy()


def _counted(p, step):
    """Runs step() with out, the windows and conv_state registered; checks the counters."""
    import torch

    import causal_conv1d_verify_amd as cv

    state = p.state_raw if p.state_raw is not None else p.conv_state
    bufs = [p.out_full, state] + ([p.windows] if p.windows is not None else [])
    for b in bufs:
        assert b.is_contiguous()
    counts = [torch.zeros(b.numel() * b.element_size() // 2, dtype=torch.int32, device=b.device)
              for b in bufs]
    before = [_units(b) for b in bufs]
    cv.conv_verify_debug_count(list(zip(bufs, counts)))
    try:
        step()
        torch.cuda.synchronize()
    finally:
        cv.conv_verify_debug_count([])
    written = 0
    for name, b, n, b0 in zip(("out", "conv_state", "windows"), bufs, counts, before):
        n = n.cpu().numpy()
        assert n.min(initial=0) >= 0
        twice = np.flatnonzero(n > 1)
        assert twice.size == 0, f"{name}: {twice.size} 2-byte units written more than once, first at {twice[0]}"
        changed = np.flatnonzero(_units(b) != b0)
        missed = changed[n[changed] != 1]
        assert missed.size == 0, f"{name}: {missed.size} units changed without a counted store"
        written += int(n.sum())
    assert written > 0
    return written


VERIFY = []
for layout in ("dense", "dedup", "dedup_t"):
    for tm in (False, True):
        VERIFY.append(c(f"sw_{layout}{'_tm' if tm else ''}", n_seq=6, d_inner=1032,
                        qk_channels=512, head_dim=128, T=8, layout=layout, accept_offsets=True,
                        permute_slots=True, pad_frac=0.25, extra_slots=2, state_tm=tm,
                        state_len=12 if not tm else 10, state_col_pad=8 if tm else 0))
VERIFY += [
    # 16 tokens on grids too large for the token splits: the pipelined time-major builds
    # and the 5-wavefront channel-major build
    c("sw_dedup_T16_tm", n_seq=130, d_inner=1032, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2, state_tm=True,
      state_len=18),
    c("sw_dedup_T16_lean", n_seq=170, d_inner=1024, qk_channels=512, head_dim=128, T=16,
      layout="dedup", permute_slots=True),
    c("sw_dense_T16_tm", n_seq=48, d_inner=7168, qk_channels=2048, head_dim=128, T=16,
      layout="dense", state_tm=True, state_len=3),
    # the line-aligned build (4-wavefront workgroups; sw_dedup_T16_tm takes it too), with
    # 8-byte row pieces (D 3) and a last workgroup of 3 wavefronts
    c("sw_line_aligned_D3", n_seq=60, d_inner=2600, qk_channels=1280, head_dim=64, d_conv=3,
      T=16, layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.1,
      state_tm=True, state_len=17),
    c("sw_line_aligned_cm", n_seq=130, d_inner=1032, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2, state_len=18),
    # heads of 96 channels: q|k in blocks of two whole heads, then 256-channel blocks
    c("sw_heads96_dedup", n_seq=6, d_inner=1032, qk_channels=480, head_dim=96, T=8,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2, state_len=12),
    c("sw_heads192_dense_K17_split", n_seq=2, d_inner=1032, qk_channels=768, head_dim=192, T=17,
      layout="dense", accept_offsets=True, state_len=20),
    # token splits: the dense chain split kernel (small grid, K 17) and the rows split
    c("sw_dense_K17_split", n_seq=2, d_inner=1024, qk_channels=512, head_dim=128, T=17,
      layout="dense", accept_offsets=True, state_len=20),
    c("sw_dedup_T16_split", n_seq=2, d_inner=1024, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, state_len=18),
    # packed rows (some empty) in each layout
    c("sw_packed_dedup", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128, T=8,
      layout="dedup", varlen=True, min_len=0, permute_slots=True),
    c("sw_packed_dense_tm", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128, T=8,
      layout="dense", varlen=True, min_len=0, state_tm=True, state_len=3),
    c("sw_packed_dedup_t", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128, T=8,
      layout="dedup_t", varlen=True, min_len=0),
    # tree verify, split over token chunks on a small grid and not
    c("sw_tree_K17", n_seq=3, d_inner=1024, qk_channels=512, head_dim=128, T=17, tree=True),
    c("sw_tree_T8", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128, T=8, tree=True,
      permute_slots=True, pad_frac=0.2),
]


@pytest.mark.parametrize("wl", VERIFY, ids=[w.name for w in VERIFY])
def test_verify_writes_each_element_once(wl):
    import causal_conv1d_verify_amd as cv

    inp = workloads.make_inputs(wl)
    print(f"[single writer] {wl.name}", flush=True)
    with cv.write_count_library():
        p = gh.GeneralProblem(inp)
        _counted(p, p.verify)
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


RESTORE = [c(f"sw_restore_{layout}{'_tm' if tm else ''}", n_seq=6, d_inner=1032, qk_channels=512,
             head_dim=128, T=8, layout=layout, restore=True, accept_offsets=True,
             permute_slots=True, pad_frac=0.2, extra_slots=1, state_tm=tm,
             state_len=10, state_col_pad=8 if tm else 0)
           for layout in ("dense", "dedup", "dedup_t") for tm in (False, True)]


@pytest.mark.parametrize("wl", RESTORE, ids=[w.name for w in RESTORE])
def test_restore_writes_each_element_once(wl):
    import causal_conv1d_verify_amd as cv

    inp = workloads.make_inputs(wl)
    print(f"[single writer] {wl.name}", flush=True)
    with cv.write_count_library():
        p = gh.GeneralProblem(inp)
        p.verify()
        _counted(p, p.restore)
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=True), inp)


PREFILL = [c(f"sw_prefill{'_tm' if tm else ''}", n_seq=5, d_inner=1032, qk_channels=0, T=70,
             varlen=True, prefill=True, init_frac=0.5, permute_slots=True, state_len=6,
             state_tm=tm, state_col_pad=8 if tm else 0)
           for tm in (False, True)]


@pytest.mark.parametrize("wl", PREFILL, ids=[w.name for w in PREFILL])
def test_prefill_writes_each_element_once(wl):
    import causal_conv1d_verify_amd as cv

    inp = workloads.make_inputs(wl)
    print(f"[single writer] {wl.name}", flush=True)
    with cv.write_count_library():
        p = gh.GeneralProblem(inp)
        _counted(p, p.prefill)
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


def test_separate_l2_writes_each_qk_element_once():
    import torch

    import causal_conv1d_verify_amd as cv

    rng = np.random.default_rng(workloads.BASE_SEED + 4400)
    rows, d, qk = 37, 1024, 512
    x = torch.from_numpy(rng.standard_normal((rows, d), dtype=np.float32)).to("cuda", torch.bfloat16)
    before = _units(x)
    counts = torch.zeros(x.numel(), dtype=torch.int32, device="cuda")
    print("[single writer] separate L2", flush=True)
    with cv.write_count_library():
        cv.conv_verify_debug_count([(x, counts)])
        try:
            cv.conv_qk_l2norm(x, qk_channels=qk, head_dim=128)
            torch.cuda.synchronize()
        finally:
            cv.conv_verify_debug_count([])
    n = counts.cpu().numpy().reshape(rows, d)
    assert (n[:, :qk] == 1).all(), "q|k channels: each written exactly once"
    assert (n[:, qk:] == 0).all(), "V channels: never written"
    changed = (_units(x) != before).reshape(rows, d)
    assert not changed[:, qk:].any()
