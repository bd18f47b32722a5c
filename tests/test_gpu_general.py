"""GPU parity of the general entry points against the oracle's general loop.

Packed rows, the time-major row layout, tree verify, the accepted-prefix restore, the
prefill conv and the separate L2 - through the C ABI (Python binding), against
oracle.verify_general / restore / prefill / l2norm on the same seeded inputs.  Bars:
windows and conv_state bit-exact over the whole buffers, out within 1e-5 + 1e-5|r|
(fp32) or 1 bf16 ulp, and every element a call must not write keeps its poison.
"""

import dataclasses

import numpy as np
import pytest

import gpu_harness as gh
import oracle
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


def _verify_case(wl, layout=None):
    inp = workloads.make_inputs(wl)
    _say(wl.name, layout or wl.layout, wl)
    p = gh.GeneralProblem(inp, layout)
    p.verify()
    return gh.compare_general(p.results(), gh.oracle_general(inp, layout), inp)


c = workloads.custom
LAYOUT_CASES = []
for layout in ("dense", "dedup", "dedup_t"):
    for T in (1, 3, 8, 9, 16, 17, 32):
        LAYOUT_CASES.append(c(f"{layout}_T{T}", n_seq=3, d_inner=1032, qk_channels=512,
                              head_dim=128, T=T, layout=layout, accept_offsets=T > 1,
                              permute_slots=True, pad_frac=0.25, extra_slots=2))
    for xd, sd in (("f32", "f32"), ("bf16", "f32")):
        LAYOUT_CASES.append(c(f"{layout}_{xd}_{sd}", n_seq=3, d_inner=520, qk_channels=256,
                              head_dim=64, T=5, layout=layout, x_dtype=xd, state_dtype=sd,
                              accept_offsets=True, permute_slots=True, pad_frac=0.3))
    for D in (2, 3):
        LAYOUT_CASES.append(c(f"{layout}_D{D}", n_seq=4, d_inner=520, qk_channels=256,
                              head_dim=64, d_conv=D, T=6, layout=layout, accept_offsets=True))


# the rows layout's compile-time-length path: a 16-token block of bf16 rows staged in
# two halves with the 5-wavefront build (state_len 3), the same with the regular build
# (state_len 18), and 8 tokens of fp32 rows (a 10 KiB block, in halves)
LAYOUT_CASES += [
    c("dedup_T16_lean", n_seq=3, d_inner=1032, qk_channels=512, head_dim=128, T=16,
      layout="dedup", permute_slots=True, pad_frac=0.25, extra_slots=2),
    c("dedup_T16_wide_state", n_seq=3, d_inner=1032, qk_channels=512, head_dim=128, T=16,
      layout="dedup", state_len=18, permute_slots=True),
    c("dedup_T8_f32_rows", n_seq=3, d_inner=1032, qk_channels=512, head_dim=128, T=8,
      layout="dedup", state_dtype="f32", accept_offsets=True, permute_slots=True),
]


@pytest.mark.parametrize("wl", LAYOUT_CASES, ids=[w.name for w in LAYOUT_CASES])
def test_layouts(wl):
    _verify_case(wl)


PACKED = []
for layout in ("dense", "dedup", "dedup_t"):
    for T in (2, 8, 16, 17, 32):
        PACKED.append(c(f"packed_{layout}_T{T}", n_seq=6, d_inner=1032, qk_channels=512,
                        head_dim=128, T=T, layout=layout, varlen=True, accept_offsets=True,
                        permute_slots=True, pad_frac=0.2, extra_slots=1))
    PACKED.append(c(f"packed_{layout}_f32", n_seq=5, d_inner=520, qk_channels=256, head_dim=64,
                    T=9, layout=layout, x_dtype="f32", state_dtype="f32", varlen=True))
    PACKED.append(c(f"packed_{layout}_strided", n_seq=5, d_inner=1000, qk_channels=512,
                    head_dim=128, T=8, layout=layout, varlen=True, x_tok_stride=1024,
                    accept_offsets=True))


@pytest.mark.parametrize("wl", PACKED, ids=[w.name for w in PACKED])
def test_packed_rows(wl):
    _verify_case(wl)


TREES = []
for T in (1, 4, 8, 17, 32):
    TREES.append(c(f"tree_T{T}", n_seq=4, d_inner=1032, qk_channels=512, head_dim=128, T=T,
                   tree=True, accept_offsets=T > 1, permute_slots=True, pad_frac=0.25))
for D in (2, 3):
    TREES.append(c(f"tree_D{D}", n_seq=4, d_inner=520, qk_channels=256, head_dim=64, d_conv=D,
                   T=7, tree=True))
for xd, sd in (("f32", "f32"), ("bf16", "f32")):
    TREES.append(c(f"tree_{xd}_{sd}", n_seq=3, d_inner=520, qk_channels=256, head_dim=64, T=9,
                   x_dtype=xd, state_dtype=sd, tree=True, accept_offsets=True))
TREES.append(c("tree_packed", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128, T=12,
               tree=True, varlen=True, accept_offsets=True, permute_slots=True, pad_frac=0.2))
# small grids spread a tree row's 4-token chunks over wavefronts; 256 rows x 4 channel
# blocks is the first grid that keeps one wavefront per row
for n in (255, 256):
    TREES.append(c(f"tree_T17_n{n}", n_seq=n, d_inner=1024, qk_channels=512, head_dim=128,
                   T=17, tree=True, accept_offsets=True, permute_slots=True, pad_frac=0.1))


@pytest.mark.parametrize("wl", TREES, ids=[w.name for w in TREES])
def test_tree(wl):
    _verify_case(wl)


def test_tree_with_chain_parents_equals_chain():
    wl = c("chain_tree", n_seq=4, d_inner=1032, qk_channels=512, head_dim=128, T=9,
           accept_offsets=True, permute_slots=True)
    inp = workloads.make_inputs(wl)
    _say("tree with chain parents vs chain")
    chain = gh.GeneralProblem(inp)
    chain.verify()
    rc = chain.results()
    inp_t = dataclasses.replace(inp, wl=dataclasses.replace(wl, tree=True),
                                parent=np.tile(np.arange(-1, wl.T - 1, dtype=np.int32),
                                               (wl.n_seq, 1)))
    tree = gh.GeneralProblem(inp_t)
    tree.verify()
    rt = tree.results()
    assert np.array_equal(rc["out"], rt["out"])
    assert np.array_equal(rc["windows"], rt["windows"])
    assert np.array_equal(rt["conv_state"], inp.conv_state), "tree verify wrote conv_state"


RESTORES = []
for layout in ("dense", "dedup", "dedup_t"):
    for off in (False, True):
        RESTORES.append(c(f"restore_{layout}_{'off' if off else 'plain'}", n_seq=6,
                          d_inner=1032, qk_channels=512, head_dim=128, T=8, layout=layout,
                          restore=True, accept_offsets=off, permute_slots=True, pad_frac=0.2,
                          extra_slots=1))
    RESTORES.append(c(f"restore_{layout}_f32_D3", n_seq=4, d_inner=520, qk_channels=256,
                      head_dim=64, d_conv=3, T=5, layout=layout, x_dtype="f32",
                      state_dtype="f32", restore=True))
RESTORES.append(c("restore_tree", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128, T=10,
                  tree=True, restore=True, accept_offsets=True, permute_slots=True,
                  pad_frac=0.2))
RESTORES.append(c("restore_packed_rows", n_seq=6, d_inner=1032, qk_channels=512,
                  head_dim=128, T=8, layout="dedup", varlen=True, restore=True))


@pytest.mark.parametrize("wl", RESTORES, ids=[w.name for w in RESTORES])
def test_restore_after_verify(wl):
    inp = workloads.make_inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    p.restore()
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=True), inp)


PREFILLS = []
for D in (2, 3, 4):
    for xd, sd in (("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")):
        PREFILLS.append(c(f"prefill_D{D}_{xd}_{sd}", n_seq=5, d_inner=520, qk_channels=0,
                          d_conv=D, T=100, x_dtype=xd, state_dtype=sd, varlen=True,
                          prefill=True, init_frac=0.5, permute_slots=True,
                          seed=workloads.BASE_SEED + 3000 + D))
PREFILLS.append(c("prefill_short_rows", n_seq=8, d_inner=1032, qk_channels=0, T=3,
                  varlen=True, prefill=True, init_frac=0.5, bias=False))
PREFILLS.append(c("prefill_wide_state", n_seq=4, d_inner=1032, qk_channels=0, T=40,
                  state_len=8, varlen=True, prefill=True, init_frac=0.5, pad_frac=0.25,
                  extra_slots=1))
PREFILLS.append(c("prefill_strided", n_seq=3, d_inner=1000, qk_channels=0, T=64,
                  x_tok_stride=1024, varlen=True, prefill=True))


@pytest.mark.parametrize("wl", PREFILLS, ids=[w.name for w in PREFILLS])
def test_prefill(wl):
    inp = workloads.make_inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.prefill()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


# Dense-window chain verify (T >= 8) spreads each row's tokens over wavefronts of 4 tokens
# when that grid has at most 5120 wavefronts; one row more and the same shape takes the
# one-wavefront-per-row kernel.  Both sides of that edge, with offsets and padded rows.
SPLIT_EDGE = [c(f"split_edge_n{n}_T{T}", n_seq=n, d_inner=1024, qk_channels=512, head_dim=128,
                T=T, accept_offsets=True, permute_slots=True, pad_frac=0.1, extra_slots=1)
              for T, edge in ((8, 640), (13, 320)) for n in (edge, edge + 1)]


@pytest.mark.parametrize("wl", SPLIT_EDGE, ids=[w.name for w in SPLIT_EDGE])
def test_split_edge(wl):
    import causal_conv1d_verify_amd as cv
    import causal_conv1d_verify_amd._lib as L

    inp = workloads.make_inputs(wl)
    p = gh.GeneralProblem(inp)
    d, T = wl.d_inner, wl.T
    shape = L.CvShape(n_seq=wl.n_seq, T=T, d_inner=d, d_conv=wl.d_conv, qk_channels=wl.qk_channels,
                      head_dim=wl.head_dim, l2_eps=wl.l2_eps, x_dtype=L.CV_BF16,
                      state_dtype=L.CV_BF16, n_slots=wl.n_slots, state_len=wl.state_len,
                      x_seq_stride=p.x.stride(0), x_tok_stride=p.x.stride(1),
                      out_seq_stride=p.out.stride(0), out_tok_stride=p.out.stride(1),
                      state_slot_stride=p.conv_state.stride(0),
                      win_slot_stride=p.windows.stride(0))
    info = cv.conv_verify_describe("dense", shape)
    assert (info.token_chunks > 1) == (wl.n_seq * 4 * -(-T // 4) <= 5120)
    _say(wl.name, "token_chunks", info.token_chunks)
    p.verify()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


# Row layouts split a row's 4-token chunks when the split grid has at most 2560
# wavefronts (buckets 8 and 16; chunk 0 keeps the state commit and the row block); one
# row more and the same shape takes the one-wavefront-per-row kernel.
ROWS_EDGE = [c(f"rows_edge_{layout}_n{n}_T{T}", n_seq=n, d_inner=1024, qk_channels=512,
               head_dim=128, T=T, layout=layout, accept_offsets=True, permute_slots=True,
               pad_frac=0.1, extra_slots=1)
             for layout in ("dedup", "dedup_t") for T, edge in ((8, 320), (13, 160))
             for n in (edge, edge + 1)]


@pytest.mark.parametrize("wl", ROWS_EDGE, ids=[w.name for w in ROWS_EDGE])
def test_rows_split_edge(wl):
    _verify_case(wl)


# LDS past 64 KiB (a gfx950 workgroup may take up to 160 KiB): fp32 state rows of 120
# columns make a 120 KiB state region, so the weights' direct global->LDS loads, the
# packed-row image and the restore's state region all land beyond the first 64 KiB.
BIG_LDS = [c(f"big_lds_{layout}{'_packed' if packed else ''}", n_seq=3, d_inner=520,
             qk_channels=256, head_dim=64, T=8, layout=layout, state_dtype="f32",
             state_len=120, accept_offsets=True, permute_slots=True, varlen=packed)
           for layout in ("dense", "dedup", "dedup_t") for packed in (False, True)]


@pytest.mark.parametrize("wl", BIG_LDS, ids=[w.name for w in BIG_LDS])
def test_big_lds_verify(wl):
    _verify_case(wl)


def test_big_lds_restore_and_prefill():
    wl = c("big_lds_restore", n_seq=4, d_inner=520, qk_channels=256, head_dim=64, T=8,
           layout="dedup", state_dtype="f32", state_len=120, accept_offsets=True,
           permute_slots=True, restore=True)
    inp = workloads.make_inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    p.restore()
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=True), inp)
    wl = c("big_lds_prefill", n_seq=3, d_inner=520, qk_channels=0, T=40, state_dtype="f32",
           state_len=120, varlen=True, prefill=True, init_frac=0.5)
    inp = workloads.make_inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.prefill()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


@pytest.mark.parametrize("xd", ["bf16", "f32"])
@pytest.mark.parametrize("hd", [4, 8, 32, 128, 256])
def test_separate_l2(xd, hd):
    import causal_conv1d_verify_amd as cv

    rng = np.random.default_rng(workloads.BASE_SEED + 3100 + hd)
    rows, d, qk = 7, 1280, 768 if hd != 256 else 512
    x0 = workloads.to_storage(rng.standard_normal((rows, d + 16)).astype(np.float32), xd)
    ref = x0.copy()
    oracle.l2norm(ref, d_inner=d, qk_channels=qk, head_dim=hd, l2_eps=1e-6, x_dtype=xd)
    _say("l2", xd, hd)
    xt = gh.to_torch(x0, xd)
    cv.conv_qk_l2norm(xt[:, :d], qk_channels=qk, head_dim=hd, l2_eps=1e-6)
    got = gh.to_numpy(xt, xd)
    assert np.array_equal(gh._bits(got[:, qk:]), gh._bits(x0[:, qk:])), "L2 wrote past q|k"
    gh.compare_out_elements(got[:, :qk], ref[:, :qk], xd, "l2")


def test_prefill_then_l2_matches_oracle():
    """The prefill pipeline stage by stage: the conv against the oracle's prefill, then
    the L2 against the oracle's L2 of the GPU's own conv output (one rounding per
    stage, so each is held to one ulp on the same input)."""
    import causal_conv1d_verify_amd as cv

    wl = c("prefill_l2", n_seq=4, d_inner=1032, qk_channels=512, head_dim=128, T=50,
           varlen=True, prefill=True, init_frac=0.5)
    inp = workloads.make_inputs(wl)
    _say("prefill + l2")
    p = gh.GeneralProblem(inp)
    p.prefill()
    conv = p.results()
    gh.compare_general(conv, gh.oracle_general(inp), inp)
    cv.conv_qk_l2norm(p.out, qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                      l2_eps=wl.l2_eps)
    got = p.results()
    gh.compare_general({"out": got["out"]}, {"out": _l2_of(conv["out"], wl)}, inp)


def _l2_of(out, wl):
    out = out.copy()
    rows = out.reshape(-1, out.shape[-1])
    oracle.l2norm(rows, d_inner=wl.d_inner, qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                  l2_eps=wl.l2_eps, x_dtype=wl.x_dtype)
    return out


@pytest.mark.parametrize("key", ["2t", "2v", "1t"])
def test_full_size_verify(key):
    wl = workloads.WORKLOADS[key]
    _verify_case(wl)


@pytest.mark.parametrize("key", ["2r", "4r"])
def test_full_size_restore(key):
    wl = workloads.WORKLOADS[key]
    inp = workloads.make_inputs(wl)
    _say(wl.name)
    p = gh.GeneralProblem(inp)
    p.verify()
    p.restore()
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=True), inp)


def test_full_size_prefill():
    wl = workloads.WORKLOADS["p"]
    inp = workloads.make_inputs(wl)
    _say(wl.name)
    p = gh.GeneralProblem(inp)
    p.prefill()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


@pytest.mark.parametrize("layout", ["dense", "dedup", "dedup_t"])
def test_padded_slot_strides(layout):
    """State and window buffers whose slots are views into a larger allocation (slot
    strides with padding after each slot): results equal the oracle's, and the padding
    keeps its poison through a verify and a restore."""
    import torch

    import causal_conv1d_verify_amd as cv

    wl = c(f"pad_{layout}", n_seq=5, d_inner=1032, qk_channels=512, head_dim=128, T=6,
           layout=layout, accept_offsets=True, permute_slots=True, pad_frac=0.2, restore=True,
           extra_slots=1)
    inp = workloads.make_inputs(wl)
    _say("padded slots", layout)
    ref = gh.oracle_general(inp, restore=True)
    p = gh.GeneralProblem(inp)
    # re-home conv_state and the windows into padded slots (16 extra elements per slot)
    pad = 16
    st_full = torch.empty((wl.n_slots, wl.d_inner * wl.state_len + pad), device="cuda",
                          dtype=p.conv_state.dtype)
    st_full.copy_(gh.to_torch(workloads.poison(tuple(st_full.shape), wl.state_dtype),
                              wl.state_dtype))
    st = st_full[:, :wl.d_inner * wl.state_len].view(wl.n_slots, wl.d_inner, wl.state_len)
    st.copy_(p.conv_state)
    wshape = tuple(p.windows.shape)
    per = int(np.prod(wshape[1:]))
    w_full = gh.to_torch(workloads.poison((wl.n_slots, per + pad), wl.state_dtype), wl.state_dtype)
    win = w_full[:, :per].view(wshape)
    cv.conv_verify_update(p.x, p.weight, p.bias, st, p.out, win, layout=layout,
                          qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
                          slot_idx=p.slot_idx, num_accept_tokens=p.nat)
    cv.conv_verify_restore(st, win, p.restore_k, layout=layout, d_conv=wl.d_conv,
                           slot_idx=p.slot_idx)
    torch.cuda.synchronize()
    got = {"out": gh.to_numpy(p.out_full, wl.x_dtype),
           "conv_state": gh.to_numpy(st.contiguous(), wl.state_dtype),
           "windows": gh.to_numpy(win.contiguous(), wl.state_dtype)}
    gh.compare_general(got, ref, inp)
    pz = gh._bits(workloads.poison((wl.n_slots, pad), wl.state_dtype))
    assert np.array_equal(gh._bits(gh.to_numpy(st_full[:, -pad:].contiguous(), wl.state_dtype)), pz)
    assert np.array_equal(gh._bits(gh.to_numpy(w_full[:, -pad:].contiguous(), wl.state_dtype)), pz)


# Time-major conv_state: the pool stored [n_slots, state_len, d (+ pad)], the library
# handed its [n_slots, d, state_len] view (state_col_stride = the column stride).  Every
# step kind that reads or writes the state, both sides of the token-split thresholds,
# the three dtype pairs, D 2..4; padded column strides must keep their poison.
TM_STATE = []
for layout in ("dense", "dedup", "dedup_t"):
    for T, pad in ((1, 0), (3, 16), (8, 0), (16, 8), (17, 0)):
        TM_STATE.append(c(f"tm_{layout}_T{T}_pad{pad}", n_seq=3, d_inner=1032, qk_channels=512,
                          head_dim=128, T=T, layout=layout, accept_offsets=T > 1,
                          permute_slots=True, pad_frac=0.25, extra_slots=2, state_tm=True,
                          state_col_pad=pad))
    for xd, sd in (("f32", "f32"), ("bf16", "f32")):
        TM_STATE.append(c(f"tm_{layout}_{xd}_{sd}", n_seq=3, d_inner=520, qk_channels=256,
                          head_dim=64, T=9, layout=layout, x_dtype=xd, state_dtype=sd,
                          accept_offsets=True, permute_slots=True, pad_frac=0.3, state_tm=True,
                          state_col_pad=4 if sd == "f32" else 8))
    for D in (2, 3):
        TM_STATE.append(c(f"tm_{layout}_D{D}", n_seq=4, d_inner=520, qk_channels=256,
                          head_dim=64, d_conv=D, T=6, layout=layout, accept_offsets=True,
                          state_tm=True))
    TM_STATE.append(c(f"tm_packed_{layout}", n_seq=6, d_inner=1032, qk_channels=512,
                      head_dim=128, T=16, layout=layout, varlen=True, accept_offsets=True,
                      permute_slots=True, pad_frac=0.2, extra_slots=1, state_tm=True))
# one-wavefront-per-row grids (past the split thresholds) and the tree
TM_STATE += [
    c("tm_dense_nosplit", n_seq=641, d_inner=1024, qk_channels=512, head_dim=128, T=8,
      accept_offsets=True, permute_slots=True, pad_frac=0.1, state_tm=True),
    c("tm_dedup_nosplit", n_seq=321, d_inner=1024, qk_channels=512, head_dim=128, T=8,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.1, state_tm=True),
    c("tm_tree", n_seq=4, d_inner=1032, qk_channels=512, head_dim=128, T=17, tree=True,
      accept_offsets=True, permute_slots=True, pad_frac=0.25, state_tm=True, state_col_pad=8),
]


@pytest.mark.parametrize("wl", TM_STATE, ids=[w.name for w in TM_STATE])
def test_time_major_state_verify(wl):
    _verify_case(wl)


TM_RESTORE = [c(f"tm_restore_{layout}", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128,
                T=8, layout=layout, restore=True, accept_offsets=True, permute_slots=True,
                pad_frac=0.2, extra_slots=1, state_tm=True, state_col_pad=8)
              for layout in ("dense", "dedup", "dedup_t")]
TM_RESTORE.append(c("tm_restore_f32_D3", n_seq=4, d_inner=520, qk_channels=256, head_dim=64,
                    d_conv=3, T=5, layout="dedup", x_dtype="f32", state_dtype="f32",
                    restore=True, state_tm=True))
# dense windows and time-major rows into a time-major state at d 2600 (11 channel blocks,
# the last partial), D 2 and 3, bf16 and fp32 state
TM_RESTORE += [c(f"tm_restore_{layout}_D{D}_{sd}_d2600", n_seq=5, d_inner=2600, qk_channels=1024,
                 head_dim=128, d_conv=D, T=6, layout=layout, state_dtype=sd, restore=True,
                 accept_offsets=True, permute_slots=True, pad_frac=0.2, state_tm=True,
                 state_col_pad=8)
               for layout in ("dense", "dedup_t") for D, sd in ((2, "bf16"), (3, "f32"))]


@pytest.mark.parametrize("wl", TM_RESTORE, ids=[w.name for w in TM_RESTORE])
def test_time_major_state_restore(wl):
    inp = workloads.make_inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    p.restore()
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=True), inp)


TM_PREFILL = [c(f"tm_prefill_D{D}_{xd}_{sd}", n_seq=5, d_inner=520, qk_channels=0, d_conv=D,
                T=70, x_dtype=xd, state_dtype=sd, varlen=True, prefill=True, init_frac=0.5,
                permute_slots=True, state_len=D + 3, state_tm=True, state_col_pad=8,
                seed=workloads.BASE_SEED + 3200 + D)
              for D in (2, 3, 4) for xd, sd in (("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32"))]


@pytest.mark.parametrize("wl", TM_PREFILL, ids=[w.name for w in TM_PREFILL])
def test_time_major_state_prefill(wl):
    inp = workloads.make_inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.prefill()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


@pytest.mark.parametrize("key", ["4t", "4bt"])
def test_full_size_time_major_state(key):
    _verify_case(workloads.WORKLOADS[key])


@pytest.mark.parametrize("key", ["4rt", "4rtt"])
def test_full_size_time_major_state_restore(key):
    wl = workloads.WORKLOADS[key]
    inp = workloads.make_inputs(wl)
    _say(wl.name)
    p = gh.GeneralProblem(inp)
    p.verify()
    p.restore()
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=True), inp)


def test_time_major_state_equals_channel_major():
    """The same problem with the state pool in either storage order: identical bits."""
    wl = c("tm_vs_cm", n_seq=6, d_inner=1032, qk_channels=512, head_dim=128, T=8,
           layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2)
    inp = workloads.make_inputs(wl)
    _say("time-major vs channel-major state")
    a = gh.GeneralProblem(inp)
    a.verify()
    inp_t = dataclasses.replace(inp, wl=dataclasses.replace(wl, state_tm=True, state_col_pad=8))
    b = gh.GeneralProblem(inp_t)
    b.verify()
    ra, rb = a.results(), b.results()
    for k in ("out", "windows", "conv_state"):
        assert np.array_equal(gh._bits(ra[k]), gh._bits(rb[k])), k


# The line-aligned build: 4-wavefront workgroups over 1024 channels whose store ranges
# (tokens of out, state columns, row blocks) leave through LDS cut at 128-byte lines -
# bf16, time-major state, dedup rows, T 16.  Grids past the token-split threshold; last
# workgroups of 1 to 4 wavefronts with a partial one; D 2..4; padded and permuted slots,
# accept offsets, padded state columns, x and out with a wider token stride, q|k ending
# inside a workgroup, rows off lines only through the state's column stride, and rows on
# lines.  Each case checks that the build is the one launched.
LINE_ALIGNED = [
    c("la_d1032_D4", n_seq=130, d_inner=1032, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2, extra_slots=2,
      state_tm=True, state_len=18, state_col_pad=8),
    c("la_d2600_D3", n_seq=60, d_inner=2600, qk_channels=1280, head_dim=64, d_conv=3, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.1, state_tm=True,
      state_len=17),
    c("la_d136_D2", n_seq=650, d_inner=136, qk_channels=128, head_dim=128, d_conv=2, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.1, state_tm=True,
      state_len=16),
    c("la_d3080_qk1152", n_seq=60, d_inner=3080, qk_channels=1152, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, pad_frac=0.3, state_tm=True, state_len=18,
      x_tok_stride=3096),
    c("la_d1024_colpad", n_seq=170, d_inner=1024, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, state_tm=True, state_len=18,
      state_col_pad=8),
    c("la_d2048_aligned", n_seq=90, d_inner=2048, qk_channels=1024, head_dim=256, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.15, extra_slots=1,
      state_tm=True, state_len=18),
    # channel-major state (taken where the rows of out start off lines): the workgroup's
    # staged region leaves cut at lines too
    c("la_cm_d1032_D4", n_seq=130, d_inner=1032, qk_channels=512, head_dim=128, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.2, extra_slots=2,
      state_len=18),
    c("la_cm_d2600_D3", n_seq=60, d_inner=2600, qk_channels=1280, head_dim=64, d_conv=3, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.1, state_len=17),
    c("la_cm_d136_D2", n_seq=650, d_inner=136, qk_channels=128, head_dim=128, d_conv=2, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.1, state_len=16),
    c("la_cm_d3080_window_state", n_seq=60, d_inner=3080, qk_channels=1152, head_dim=128, T=16,
      layout="dedup", pad_frac=0.3, permute_slots=True, x_tok_stride=3096),
    c("la_cm_d2048_sl18", n_seq=90, d_inner=2048, qk_channels=1024, head_dim=256, T=16,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.15, state_len=18,
      x_tok_stride=2056),
]


@pytest.mark.parametrize("wl", LINE_ALIGNED, ids=[w.name for w in LINE_ALIGNED])
def test_line_aligned_build(wl):
    import causal_conv1d_verify_amd as cv
    import causal_conv1d_verify_amd._lib as L

    inp = workloads.make_inputs(wl)
    p = gh.GeneralProblem(inp)
    launch = cv.prepare("update", p.x, p.weight, p.bias, p.conv_state, p.out, p.windows,
                        layout=p.layout, qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                        l2_eps=wl.l2_eps, slot_idx=p.slot_idx, num_accept_tokens=p.nat)
    info = cv.conv_verify_describe(p.layout, launch.keepalive[0])
    assert info.flags & L.CV_LAUNCH_LINE_ALIGNED and info.threads == 256, (info.flags, info.threads)
    assert info.workgroups == wl.n_seq * -(-wl.d_inner // 1024)
    _say(wl.name, "workgroups", info.workgroups, "lds", info.lds_bytes)
    launch()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


# Grids past one resident generation (5,120 wavefronts) with a slot table read the
# slot before loading x, so padded rows load nothing; both sides of that edge.
SLOT_FIRST = [c(f"slot_first_{layout}_n{n}{'_tm' if tm else ''}", n_seq=n, d_inner=1024,
                qk_channels=512, head_dim=128, T=4, layout=layout, accept_offsets=True,
                permute_slots=True, pad_frac=0.3, extra_slots=2, state_tm=tm)
              for layout, tm in (("dedup", False), ("dense", True)) for n in (1280, 1281)]


@pytest.mark.parametrize("wl", SLOT_FIRST, ids=[w.name for w in SLOT_FIRST])
def test_slot_first_edge(wl):
    _verify_case(wl)


# bf16 x with a time-major fp32 state: the commit widens x into 16-byte fp32 columns and
# stores them back to back.  A 16-byte store whose scalar offset was an SGPR, followed at
# once by the widening of the next column into the same registers, wrote that next column
# into the fourth dword of some lanes now and then (the compiler adds no wait state for that
# form); every 16-byte store now takes its offset in the lane offset.  Several hundred rows
# per launch, in each layout, with packed rows and with full ones.
STORE_WIDE = [c(f"tm_f32_commit_{layout}{'_packed' if packed else ''}", n_seq=300, d_inner=2104,
                qk_channels=1536, head_dim=256, T=9, state_dtype="f32", layout=layout,
                accept_offsets=True, varlen=packed, min_len=0, extra_slots=1, state_tm=True,
                state_len=12, seed=workloads.BASE_SEED + 7700 + 2 * i + packed)
              for i, layout in enumerate(("dense", "dedup", "dedup_t")) for packed in (False, True)]


@pytest.mark.parametrize("wl", STORE_WIDE, ids=[w.name for w in STORE_WIDE])
def test_time_major_fp32_commit_stores(wl):
    _verify_case(wl)


# q|k ending inside a wavefront: lanes of one wavefront split between L2 heads and V
# channels, for several head sizes, both state orders and layouts.
QK_EDGE = [c(f"qk{qk}_h{hd}_{layout}{'_tm' if tm else ''}", n_seq=3, d_inner=1032, qk_channels=qk,
             head_dim=hd, T=T, layout=layout, accept_offsets=True, permute_slots=True,
             pad_frac=0.25, state_tm=tm)
           for qk, hd, layout, T, tm in ((384, 128, "dedup", 8, False), (96, 32, "dense", 5, True),
                                         (776, 8, "dedup_t", 9, False), (1032, 4, "dense", 17, False),
                                         (640, 64, "dedup", 16, True))]
QK_EDGE.append(c("one_head_fp32", n_seq=2, d_inner=264, qk_channels=256, head_dim=256, T=3,
                 x_dtype="f32", state_dtype="f32", accept_offsets=True))


@pytest.mark.parametrize("wl", QK_EDGE, ids=[w.name for w in QK_EDGE])
def test_qk_edges(wl):
    _verify_case(wl)


@pytest.mark.parametrize("tm", [True, False], ids=["tm", "cm"])
def test_line_aligned_out_stride_differs_from_x(tm):
    """The line-aligned build with out in a wider buffer than x (token stride 1048 against
    x's 1024, so only out's rows start off 128-byte lines): out lands at its own strides,
    the padding after each of its rows keeps its poison."""
    import causal_conv1d_verify_amd as cv
    import causal_conv1d_verify_amd._lib as L

    wl = c(f"la_out_stride_{'tm' if tm else 'cm'}", n_seq=170, d_inner=1024, qk_channels=512,
           head_dim=128, T=16, layout="dedup", accept_offsets=True, permute_slots=True,
           pad_frac=0.2, state_len=18, state_tm=tm)
    inp = workloads.make_inputs(wl)
    p = gh.GeneralProblem(inp)
    d, pad = wl.d_inner, 24
    wide0 = workloads.poison((wl.n_seq, wl.T, d + pad), wl.x_dtype)
    wide = gh.to_torch(wide0, wl.x_dtype)
    p.out = wide[..., :d]
    launch = cv.prepare("update", p.x, p.weight, p.bias, p.conv_state, p.out, p.windows,
                        layout=p.layout, qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                        l2_eps=wl.l2_eps, slot_idx=p.slot_idx, num_accept_tokens=p.nat)
    info = cv.conv_verify_describe(p.layout, launch.keepalive[0])
    assert info.flags & L.CV_LAUNCH_LINE_ALIGNED and info.threads == 256
    _say(wl.name, "workgroups", info.workgroups)
    launch()
    got = p.results()                      # windows and conv_state (out_full is untouched)
    ref = gh.oracle_general(inp)
    for k in ("windows", "conv_state"):
        assert np.array_equal(gh._bits(got[k]), gh._bits(ref[k])), k
    out = gh.to_numpy(wide, wl.x_dtype)
    assert np.array_equal(gh._bits(out[..., d:]), gh._bits(wide0[..., d:])), "padding written"
    mask = np.zeros(out[..., :d].shape, bool)
    for idx in gh.computed_tokens(inp):
        mask[idx + (slice(0, d),)] = True
    go, ro = out[..., :d], ref["out"][..., :d]
    assert np.array_equal(gh._bits(go)[~mask], gh._bits(ro)[~mask]), "out written outside the computed tokens"
    gh.compare_out_elements(go[mask], ro[mask], wl.x_dtype)
