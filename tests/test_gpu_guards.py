"""Guard bands around every buffer a call touches (the memory-checker analogue).

Each buffer (x, weight, bias, out, the windows, conv_state) is re-homed into a larger
poison-filled allocation with GUARD elements before and after it; after the call the
results must equal the oracle's as usual and every guard element must still hold its
poison bits, so no access of any kernel lands outside its buffer.  Cases cover every
step kind (verify in the three layouts, tree, packed rows, restore, prefill), both
conv_state orders, the token-split small grids, partial channel blocks and a grid past
one resident generation.
"""

import numpy as np
import pytest

import gpu_harness as gh
import workloads

pytestmark = pytest.mark.gpu

GUARD = 4096   # elements on each side (8-16 KB: more than one wavefront's block)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class _Guarded:
    """Copies of a problem's buffers inside poison-filled guard bands."""

    def __init__(self):
        self.bands = []   # (flat tensor, numel, dtype name)

    def wrap(self, t, dtype):
        flat = gh.to_torch(workloads.poison((t.numel() + 2 * GUARD,), dtype), dtype)
        view = flat[GUARD:GUARD + t.numel()].view(t.shape)
        view.copy_(t)
        self.bands.append((flat, t.numel(), dtype))
        return view

    def check(self):
        for flat, n, dtype in self.bands:
            bits = gh._bits(gh.to_numpy(flat, dtype))
            pz = gh._bits(workloads.poison((GUARD,), dtype))
            assert np.array_equal(bits[:GUARD], pz), "write before a buffer"
            assert np.array_equal(bits[GUARD + n:], pz), "write after a buffer"


def _guard_problem(p):
    wl = p.wl
    g = _Guarded()
    d = wl.d_inner
    p.x = g.wrap(p.x, wl.x_dtype)
    p.weight = g.wrap(p.weight, wl.x_dtype)
    if p.bias is not None:
        p.bias = g.wrap(p.bias, wl.x_dtype)
    p.out_full = g.wrap(p.out_full, wl.x_dtype)
    p.out = p.out_full[..., :d]
    if p.windows is not None:
        p.windows = g.wrap(p.windows, wl.state_dtype)
    if p.state_raw is not None:
        p.state_raw = g.wrap(p.state_raw, wl.state_dtype)
        p.conv_state = p.state_raw[:, :, :d].transpose(1, 2)
    else:
        p.conv_state = g.wrap(p.conv_state, wl.state_dtype)
    return g


c = workloads.custom
CASES = []
for layout in ("dense", "dedup", "dedup_t"):
    for tm in (False, True):
        CASES.append(c(f"guard_{layout}{'_tm' if tm else ''}", n_seq=4, d_inner=1032,
                       qk_channels=512, head_dim=128, T=9, layout=layout, accept_offsets=True,
                       permute_slots=True, pad_frac=0.25, extra_slots=1, state_tm=tm,
                       state_col_pad=8 if tm else 0))
CASES += [
    c("guard_split_T17", n_seq=2, d_inner=1024, qk_channels=512, head_dim=128, T=17,
      accept_offsets=True, state_tm=True),
    c("guard_rows_split_T16", n_seq=2, d_inner=1000, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True),
    c("guard_tree", n_seq=3, d_inner=1032, qk_channels=512, head_dim=128, T=12, tree=True,
      accept_offsets=True, permute_slots=True),
    c("guard_packed", n_seq=5, d_inner=1032, qk_channels=512, head_dim=128, T=8, layout="dedup",
      varlen=True, accept_offsets=True, permute_slots=True, pad_frac=0.2),
    c("guard_restore_rows", n_seq=4, d_inner=1032, qk_channels=512, head_dim=128, T=8,
      layout="dedup", restore=True, accept_offsets=True, permute_slots=True),
    c("guard_restore_tm", n_seq=4, d_inner=1032, qk_channels=512, head_dim=128, T=8,
      layout="dense", restore=True, accept_offsets=True, state_tm=True, state_col_pad=8),
    c("guard_prefill", n_seq=4, d_inner=1032, qk_channels=0, T=40, varlen=True, prefill=True,
      init_frac=0.5, state_len=6),
    c("guard_prefill_tm", n_seq=4, d_inner=1032, qk_channels=0, T=40, varlen=True, prefill=True,
      init_frac=0.5, state_tm=True),
    # past one resident generation (slot first), partial blocks (XCD order)
    c("guard_large", n_seq=1300, d_inner=1000, qk_channels=512, head_dim=128, T=4,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2, state_tm=True),
    c("guard_large_dense_t1", n_seq=1300, d_inner=1024, qk_channels=512, head_dim=128, T=1,
      state_dtype="f32"),
    # the line-aligned build (4-wavefront workgroups; the last one with 3 idle wavefronts),
    # time-major and channel-major state
    c("guard_line_aligned_tm", n_seq=130, d_inner=1032, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2, state_len=18,
      state_tm=True, state_col_pad=8),
    c("guard_line_aligned_cm", n_seq=130, d_inner=1032, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2, state_len=18),
]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_guard_bands(wl):
    print("[case]", wl, flush=True)
    inp = workloads.make_inputs(wl)
    p = gh.GeneralProblem(inp)
    g = _guard_problem(p)
    if wl.prefill:
        p.prefill()
        ref = gh.oracle_general(inp)
    else:
        p.verify()
        if wl.restore:
            p.restore()
        ref = gh.oracle_general(inp, restore=wl.restore)
    gh.compare_general(p.results(), ref, inp)
    g.check()
