"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph): every replay,
with eager work and synchronizations between replays, must give the bit patterns of
the eager launch on the same inputs.  The kernels record no memset node; each replay
here restarts from freshly copied inputs."""

import numpy as np
import pytest

import gpu_harness as gh
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_conv1d_verify_amd._lib as L

    L.load()


def _say(*a):
    print("[case]", *a, flush=True)


def _fresh(p, inp):
    """Reset a problem's mutable buffers from host copies (eager copies, outside graphs)."""
    wl = inp.wl
    p.conv_state.copy_(gh.to_torch(inp.conv_state, wl.state_dtype))
    p.out_full.copy_(gh.to_torch(workloads.poison(inp.x.shape, wl.x_dtype), wl.x_dtype))
    if p.windows is not None:
        p.windows.copy_(gh.to_torch(workloads.poison(tuple(p.windows.shape), wl.state_dtype),
                                    wl.state_dtype))


CASES = [
    workloads.custom("g_dedup", n_seq=6, d_inner=2048, qk_channels=1024, head_dim=128, T=8,
                     layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2),
    workloads.custom("g_dense_split", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128,
                     T=17, layout="dense", accept_offsets=True, permute_slots=True, pad_frac=0.2),
    workloads.custom("g_packed_tree", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128,
                     T=9, tree=True, varlen=True, permute_slots=True),
    workloads.custom("g_restore", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128, T=8,
                     layout="dedup_t", restore=True, permute_slots=True),
    workloads.custom("g_prefill", n_seq=4, d_inner=1032, qk_channels=512, head_dim=128, T=40,
                     varlen=True, prefill=True, init_frac=0.5),
    # the same step kinds with conv_state stored time-major
    workloads.custom("g_dedup_tmstate", n_seq=6, d_inner=2048, qk_channels=1024, head_dim=128,
                     T=16, layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2,
                     state_tm=True),
    workloads.custom("g_restore_tmstate", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128,
                     T=8, layout="dense", restore=True, accept_offsets=True, permute_slots=True,
                     state_tm=True, state_col_pad=8),
    workloads.custom("g_prefill_tmstate", n_seq=4, d_inner=1032, qk_channels=0, T=40,
                     varlen=True, prefill=True, init_frac=0.5, state_tm=True),
    # the line-aligned build (4-wavefront workgroups, LDS exchanges behind barriers)
    workloads.custom("g_line_aligned_tm", n_seq=130, d_inner=1032, qk_channels=512,
                     head_dim=128, T=16, layout="dedup", accept_offsets=True, permute_slots=True,
                     pad_frac=0.2, state_len=18, state_tm=True),
    workloads.custom("g_line_aligned_cm", n_seq=130, d_inner=1032, qk_channels=512,
                     head_dim=128, T=16, layout="dedup", accept_offsets=True, permute_slots=True,
                     pad_frac=0.2, state_len=18),
    # heads of 96 channels (q|k in blocks of whole heads, segmented head sums)
    workloads.custom("g_heads96", n_seq=6, d_inner=1032, qk_channels=480, head_dim=96, T=8,
                     layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2),
]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_graph_replays_match_eager(wl):
    import torch

    import causal_conv1d_verify_amd as cv

    inp = workloads.make_inputs(wl)
    _say(wl.name)
    p = gh.GeneralProblem(inp)

    def step():
        if wl.prefill:
            p.prefill()
            cv.conv_qk_l2norm(p.out, qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                              l2_eps=wl.l2_eps)
        else:
            p.verify()
            if wl.restore:
                p.restore()

    _fresh(p, inp)
    step()
    eager = p.results()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    _fresh(p, inp)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=side):
        step()
    torch.cuda.synchronize()
    scratch = torch.zeros(1 << 20, device="cuda")
    for r in range(4):
        _fresh(p, inp)
        scratch.add_(1.0)                  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = p.results()
        for k in eager:
            assert np.array_equal(gh._bits(got[k]), gh._bits(eager[k])), (r, k)
