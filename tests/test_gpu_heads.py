"""GPU parity for L2 heads whose size does not divide 256 channels (head_dim 12 ... 252).

Such heads would straddle the 256-channel wavefronts, so the q|k channels go in blocks of
whole heads and each head is summed by a segmented scan across its lanes (the launch
reports CV_LAUNCH_HEAD_BLOCKS).  Every kernel that normalises q|k is covered: the chain
verify in the three window layouts (token buckets 1 to 32, the 16-token lean build, the
row-layout token split, both conv_state orders, the three dtype pairs, D 2 to 4), packed
rows, the tree (split and not), the token-split dense verify, the separate L2, and
extreme magnitudes that take the rescaled second sum.  Bars as everywhere: windows and
conv_state bit-exact, out within 1e-5 + 1e-5|r| (fp32) or 1 bf16 ulp of the oracle.
"""

import numpy as np
import pytest

import gpu_harness as gh
import oracle
import workloads
from test_gpu_extremes import _inputs as _extreme_inputs

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


def _check_head_blocks(wl):
    """The host plans the blocks of whole heads for this head size, q|k width and dtype
    pair (its own report, on the same shape with plain strides)."""
    import causal_conv1d_verify_amd as cv
    import causal_conv1d_verify_amd._lib as L

    T, d, w1 = wl.T, wl.d_inner, wl.d_conv - 1
    dt = {"f32": L.CV_F32, "bf16": L.CV_BF16}
    s = L.CvShape(n_seq=wl.n_seq, T=T, d_inner=d, d_conv=wl.d_conv, qk_channels=wl.qk_channels,
                  head_dim=wl.head_dim, l2_eps=1e-6, x_dtype=dt[wl.x_dtype],
                  state_dtype=dt[wl.state_dtype], n_slots=wl.n_seq, state_len=w1,
                  x_seq_stride=T * d, x_tok_stride=d, out_seq_stride=T * d, out_tok_stride=d,
                  state_slot_stride=d * w1, win_slot_stride=T * d * w1)
    info = cv.conv_verify_describe("dense", s)
    assert info.flags & L.CV_LAUNCH_HEAD_BLOCKS, "expected the q|k blocks of whole heads"


def _verify_case(wl):
    inp = workloads.make_inputs(wl)
    _say(wl.name, wl)
    _check_head_blocks(wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


c = workloads.custom
# (head_dim, heads): q|k = heads * head_dim, a multiple of 8 channels
CASES = [
    c("h96_dedup_T8", n_seq=3, d_inner=1032, qk_channels=480, head_dim=96, T=8, layout="dedup",
      accept_offsets=True, permute_slots=True, pad_frac=0.25, extra_slots=2),
    c("h96_dense_T1_f32state", n_seq=5, d_inner=1032, qk_channels=480, head_dim=96, T=1,
      layout="dense", state_dtype="f32"),
    c("h192_dense_T17_tm", n_seq=3, d_inner=1032, qk_channels=768, head_dim=192, T=17,
      layout="dense", accept_offsets=True, state_tm=True, state_len=20),
    c("h192_dedup_t_T32", n_seq=3, d_inner=1032, qk_channels=576, head_dim=192, T=32,
      layout="dedup_t", accept_offsets=True, permute_slots=True),
    c("h12_dedup_t_T9", n_seq=3, d_inner=520, qk_channels=240, head_dim=12, T=9,
      layout="dedup_t", accept_offsets=True, permute_slots=True, pad_frac=0.25),
    c("h12_f32_dense_T3", n_seq=3, d_inner=520, qk_channels=252, head_dim=12, T=3,
      layout="dense", x_dtype="f32", state_dtype="f32", accept_offsets=True),
    c("h20_D2_dedup_T5", n_seq=4, d_inner=520, qk_channels=240, head_dim=20, d_conv=2, T=5,
      layout="dedup", accept_offsets=True),
    c("h20_D3_dense_T6", n_seq=4, d_inner=520, qk_channels=240, head_dim=20, d_conv=3, T=6,
      layout="dense", accept_offsets=True, state_tm=True),
    c("h48_dedup_T16_lean", n_seq=3, d_inner=1032, qk_channels=480, head_dim=48, T=16,
      layout="dedup", permute_slots=True, pad_frac=0.25),
    c("h80_dedup_T16_wide_state", n_seq=3, d_inner=1032, qk_channels=480, head_dim=80, T=16,
      layout="dedup", state_len=18, permute_slots=True),
    c("h80_dedup_T16_tm", n_seq=3, d_inner=1032, qk_channels=480, head_dim=80, T=16,
      layout="dedup", accept_offsets=True, state_tm=True, state_len=18, state_col_pad=8),
    c("h112_bf16_f32_dedup_T24", n_seq=3, d_inner=1032, qk_channels=448, head_dim=112, T=24,
      layout="dedup", state_dtype="f32", accept_offsets=True),
    c("h160_f32_dedup_t_T5", n_seq=3, d_inner=520, qk_channels=320, head_dim=160, T=5,
      layout="dedup_t", x_dtype="f32", state_dtype="f32", accept_offsets=True),
    c("h240_dense_T4", n_seq=3, d_inner=1032, qk_channels=720, head_dim=240, T=4,
      layout="dense", accept_offsets=True, permute_slots=True),
    c("h252_f32_dedup_T2", n_seq=3, d_inner=520, qk_channels=504, head_dim=252, T=2,
      layout="dedup", x_dtype="f32", state_dtype="f32"),
    # a small dense grid with T >= 8: the token-split kernel; small row-layout grids: the
    # rows token split (buckets 8 and 16)
    c("h96_split_dense_T12", n_seq=2, d_inner=1032, qk_channels=480, head_dim=96, T=12,
      layout="dense", accept_offsets=True),
    c("h96_rows_split_T16", n_seq=2, d_inner=1032, qk_channels=480, head_dim=96, T=16,
      layout="dedup", accept_offsets=True, state_len=18),
    # every q|k channel (no V blocks), and one head per block
    c("h96_all_qk", n_seq=3, d_inner=960, qk_channels=960, head_dim=96, T=8, layout="dedup"),
    c("h192_one_head", n_seq=3, d_inner=456, qk_channels=192, head_dim=192, T=8, layout="dense"),
    # packed rows and trees
    c("h96_packed_dedup_T8", n_seq=6, d_inner=1032, qk_channels=480, head_dim=96, T=8,
      layout="dedup", varlen=True, accept_offsets=True, permute_slots=True, pad_frac=0.2),
    c("h24_packed_dense_T17", n_seq=6, d_inner=1032, qk_channels=480, head_dim=24, T=17,
      layout="dense", varlen=True, min_len=0),
    c("h96_tree_T8", n_seq=4, d_inner=1032, qk_channels=480, head_dim=96, T=8, tree=True,
      accept_offsets=True, permute_slots=True, pad_frac=0.25),
    c("h192_tree_T17_split", n_seq=3, d_inner=1032, qk_channels=768, head_dim=192, T=17,
      tree=True, accept_offsets=True),
    # a grid of several generations (slot-first) at the pages' row width
    c("h96_dedup_bs64_d10240", n_seq=64, d_inner=10240, qk_channels=96 * 42, head_dim=96, T=8,
      layout="dedup", accept_offsets=True, permute_slots=True, pad_frac=0.1),
]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_head_blocks_verify(wl):
    _verify_case(wl)


EXTREME = [c(f"h96_ext_{tag}_{xd}_{layout}_T{T}", n_seq=3, d_inner=1032, qk_channels=480,
             head_dim=96, T=T, x_dtype=xd, state_dtype=xd, layout=layout, accept_offsets=True,
             permute_slots=True, l2_eps=eps)
           for tag, eps in (("eps1e-6", 1e-6), ("eps0", 0.0))
           for xd, layout, T in (("bf16", "dedup", 8), ("f32", "dense", 3), ("bf16", "dense", 12))]


@pytest.mark.parametrize("wl", EXTREME, ids=[w.name for w in EXTREME])
def test_head_blocks_extremes(wl):
    """Heads of 96 channels at the ends of fp32's range (the overflowing and underflowing
    sums of squares take the rescaled second sum over the same segmented scan)."""
    inp = _extreme_inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


@pytest.mark.parametrize("xd", ["bf16", "f32"])
@pytest.mark.parametrize("hd,qk", [(12, 480), (96, 768), (192, 768), (252, 504)])
def test_head_blocks_separate_l2(xd, hd, qk):
    import causal_conv1d_verify_amd as cv

    rng = np.random.default_rng(workloads.BASE_SEED + 3500 + hd)
    rows, d = 7, 1280
    x0 = workloads.to_storage(rng.standard_normal((rows, d + 16)).astype(np.float32), xd)
    if xd == "bf16" and hd == 252:
        # no block of whole 252-channel heads is a multiple of 8 bf16 channels: refused on
        # the host, nothing written
        with pytest.raises(cv.CvError):
            cv.conv_qk_l2norm(gh.to_torch(x0, xd)[:, :d], qk_channels=qk, head_dim=hd, l2_eps=1e-6)
        return
    ref = x0.copy()
    oracle.l2norm(ref, d_inner=d, qk_channels=qk, head_dim=hd, l2_eps=1e-6, x_dtype=xd)
    _say("l2", xd, hd, qk)
    xt = gh.to_torch(x0, xd)
    cv.conv_qk_l2norm(xt[:, :d], qk_channels=qk, head_dim=hd, l2_eps=1e-6)
    got = gh.to_numpy(xt, xd)
    assert np.array_equal(gh._bits(got[:, qk:]), gh._bits(x0[:, qk:])), "L2 wrote past q|k"
    gh.compare_out_elements(got[:, :qk], ref[:, :qk], xd, "l2")


NON_POW2 = (12, 20, 24, 36, 40, 48, 56, 72, 80, 96, 112, 144, 160, 192, 208, 240)


def _block(hd, align):
    k = 256 // hd
    while k and (k * hd) % align:
        k -= 1
    return k * hd


def _draw(k: int, rng: np.random.Generator):
    """A random verify with heads that do not divide 256 channels: any layout, tree,
    packed rows, dtype pair, width, token count, either conv_state order, offsets, padded
    rows, strided x; q|k a whole number of heads on the 16-byte channel multiple."""
    xd, sd = [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")][int(rng.integers(0, 3))]
    align = 4 if (xd, sd) == ("f32", "f32") else 8
    while True:
        hd = int(rng.choice(NON_POW2))
        heads = int(rng.integers(1, 12))
        if _block(hd, align) and (hd * heads) % align == 0:
            break
    qk = hd * heads
    d = qk + 8 * int(rng.integers(0, 80))
    T = int(rng.integers(1, 33))
    tree = bool(rng.random() < 0.2)
    layout = "dense" if tree else str(rng.choice(["dense", "dedup", "dedup_t"]))
    tm = bool(rng.random() < 0.5)
    varlen = bool(rng.random() < 0.3)
    stride = d + 8 * int(rng.integers(1, 5)) if not varlen and rng.random() < 0.3 else None
    return workloads.custom(
        f"rand_heads{k:02d}", n_seq=int(rng.integers(1, 7)), d_inner=d, qk_channels=qk,
        head_dim=hd, d_conv=int(rng.integers(2, 5)), T=T, x_dtype=xd, state_dtype=sd,
        layout=layout, bias=bool(rng.random() < 0.7), accept_offsets=bool(rng.random() < 0.6),
        pad_frac=float(rng.choice([0.0, 0.2, 0.5])), permute_slots=bool(rng.random() < 0.6),
        extra_slots=int(rng.integers(0, 3)), x_tok_stride=stride, varlen=varlen, tree=tree,
        state_tm=tm, state_col_pad=(8 * int(rng.integers(0, 3))) if tm else 0,
        seed=workloads.BASE_SEED + 5800 + k)


_rng = np.random.default_rng(workloads.BASE_SEED + 5799)
RANDOM = [_draw(k, _rng) for k in range(24)]


@pytest.mark.parametrize("wl", RANDOM, ids=[w.name for w in RANDOM])
def test_head_blocks_random(wl):
    _verify_case(wl)
