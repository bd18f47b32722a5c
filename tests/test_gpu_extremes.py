"""GPU parity at extreme magnitudes: SiLU deep in both tails and L2 heads whose fp32 sum
of squares overflows or underflows.

The bias of each channel is set so that the pre-activation lands where it is wanted
(the conv adds only ~N(0, 0.6) to it):

* V channels sweep bias through [-120, -80] and [80, 120], densest over [-97, -85]
  (where SiLU is a subnormal bf16 and exp(-p) is past fp32's range);
* q|k head 0 sweeps [-120, -80] with eps = 1e-6 (tiny and subnormal values, which eps
  swamps), and [-84, -60] with eps = 0 (values of 1e-35 to 1e-25: their fp32 sum of
  squares underflows, and the head is summed again rescaled).  With eps = 0 the L2
  multiplies y by 1/|y| ~ 1e33 here, so the head stays inside fp32's normal range: y
  is an fp32 value on the GPU (the oracle keeps it in fp64), and values below 2^-149,
  zero in fp32, would come out of the L2 as normal numbers on the oracle's side only;
* head 1 sweeps [80, 120] (plain large values);
* head 2 alternates +-1e20 (y = 1e20 or -0: the fp32 sum of squares overflows);
* head 3 has eight channels at 3e38 (near fp32's maximum) among ordinary ones.

Every kernel that evaluates SiLU or the L2 is covered: the chain verify in the three
window layouts and both token buckets' chunk shapes, both conv_state orders, the tree,
packed rows, the token-split dense verify, the prefill conv and the separate L2.  Bars
as everywhere: windows and conv_state bit-exact, out within 1e-5 + 1e-5|r| (fp32) or
1 bf16 ulp of the oracle.
"""

import numpy as np
import pytest

import gpu_harness as gh
import oracle
import workloads

pytestmark = pytest.mark.gpu

D_INNER, QK, HD = 1032, 512, 128


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_conv1d_verify_amd._lib as L

    L.load()


def _say(*a):
    print("[case]", *a, flush=True)


def extreme_bias(wl, bias_f32: np.ndarray) -> np.ndarray:
    """Per-channel bias driving the pre-activations into the ranges above."""
    b = bias_f32.astype(np.float32).copy()
    d, qk, hd = wl.d_inner, wl.qk_channels, wl.head_dim
    if qk >= 4 * hd:
        b[0:hd] = np.linspace(-84, -60, hd) if wl.l2_eps == 0.0 else np.linspace(-120, -80, hd)
        b[hd:2 * hd] = np.linspace(80, 120, hd)
        b[2 * hd:3 * hd] = np.where(np.arange(hd) % 2 == 0, 1e20, -1e20)
        b[3 * hd:3 * hd + 8] = 3e38
    nv = d - qk
    dense = nv // 2
    v = np.concatenate([np.linspace(-97, -85, dense),
                        np.linspace(-120, -80, (nv - dense) // 2),
                        np.linspace(80, 120, nv - dense - (nv - dense) // 2)])
    b[qk:] = v.astype(np.float32)
    return b


def _inputs(wl):
    inp = workloads.make_inputs(wl)
    b = workloads.bf16_bits_to_f32(inp.bias) if wl.x_dtype == "bf16" else inp.bias
    inp.bias = workloads.to_storage(extreme_bias(wl, b), wl.x_dtype)
    return inp


c = workloads.custom
CASES = []
for eps in (1e-6, 0.0):
    tag = "eps0" if eps == 0.0 else "eps1e-6"
    for xd, sd in (("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")):
        for layout in ("dense", "dedup", "dedup_t"):
            for T in (3, 16):
                CASES.append(c(f"ext_{tag}_{xd}_{sd}_{layout}_T{T}", n_seq=3, d_inner=D_INNER,
                               qk_channels=QK, head_dim=HD, T=T, x_dtype=xd, state_dtype=sd,
                               layout=layout, accept_offsets=True, permute_slots=True,
                               pad_frac=0.25, extra_slots=1, l2_eps=eps))
    CASES.append(c(f"ext_{tag}_tmstate_T16", n_seq=3, d_inner=D_INNER, qk_channels=QK,
                   head_dim=HD, T=16, layout="dedup", accept_offsets=True, permute_slots=True,
                   state_tm=True, state_col_pad=8, l2_eps=eps))
    CASES.append(c(f"ext_{tag}_tmstate_T8", n_seq=3, d_inner=D_INNER, qk_channels=QK,
                   head_dim=HD, T=8, layout="dense", accept_offsets=True, state_tm=True,
                   l2_eps=eps))
    CASES.append(c(f"ext_{tag}_tree_T9", n_seq=3, d_inner=D_INNER, qk_channels=QK, head_dim=HD,
                   T=9, tree=True, accept_offsets=True, permute_slots=True, l2_eps=eps))
    CASES.append(c(f"ext_{tag}_packed_T8", n_seq=5, d_inner=D_INNER, qk_channels=QK,
                   head_dim=HD, T=8, layout="dedup", varlen=True, accept_offsets=True,
                   permute_slots=True, l2_eps=eps))
    # a small dense grid with T >= 8 takes the token-split kernel (4-token wavefronts)
    CASES.append(c(f"ext_{tag}_split_T12", n_seq=2, d_inner=D_INNER, qk_channels=QK,
                   head_dim=HD, T=12, layout="dense", accept_offsets=True, l2_eps=eps))
    CASES.append(c(f"ext_{tag}_split_f32_T9", n_seq=2, d_inner=D_INNER, qk_channels=QK,
                   head_dim=HD, T=9, layout="dense", x_dtype="f32", state_dtype="f32",
                   l2_eps=eps))


def _strict_fp32_silu(got, ref, inp):
    """fp32 out of the V channels (SiLU alone, no L2) held to a relative bar, which the
    common fp32 tolerance (1e-5 absolute) would not be for values near zero:
    |g - r| <= 1e-5 |r| + 2^-147 (four steps of fp32's subnormal spacing)."""
    wl = inp.wl
    if wl.x_dtype != "f32":
        return
    for idx in gh.computed_tokens(inp):
        g = got["out"][idx][wl.qk_channels:wl.d_inner].astype(np.float64)
        r = ref["out"][idx][wl.qk_channels:wl.d_inner].astype(np.float64)
        bad = np.abs(g - r) > 1e-5 * np.abs(r) + 2.0 ** -147
        assert not bad.any(), f"fp32 SiLU at {idx}: gpu {g[bad][:4]} oracle {r[bad][:4]}"


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_extreme_verify(wl):
    inp = _inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    got, ref = p.results(), gh.oracle_general(inp)
    gh.compare_general(got, ref, inp)
    _strict_fp32_silu(got, ref, inp)


PREFILLS = [c(f"ext_prefill_{xd}_{sd}{'_tm' if tm else ''}", n_seq=4, d_inner=D_INNER,
              qk_channels=0, T=40, x_dtype=xd, state_dtype=sd, varlen=True, prefill=True,
              init_frac=0.5, state_tm=tm)
            for xd, sd in (("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")) for tm in (False, True)]


@pytest.mark.parametrize("wl", PREFILLS, ids=[w.name for w in PREFILLS])
def test_extreme_prefill(wl):
    inp = _inputs(wl)
    _say(wl.name, wl)
    p = gh.GeneralProblem(inp)
    p.prefill()
    got, ref = p.results(), gh.oracle_general(inp)
    gh.compare_general(got, ref, inp)
    _strict_fp32_silu(got, ref, inp)


def _l2_rows(xd, rows, d, qk, hd, rng):
    """Token rows whose heads span fp32's range: huge, near-maximal, tiny (scale 1e-36,
    so the heads' tails are subnormal) and ordinary values, mixed within and across
    heads."""
    x = rng.standard_normal((rows, d)).astype(np.float32)
    scales = [1e20, 3e37, 1e-30, 1e-36, 1.0, 1e10, 1e-20]
    for r in range(rows):
        for h in range(qk // hd):
            x[r, h * hd:(h + 1) * hd] *= np.float32(scales[(r + h) % len(scales)])
        x[r, :8] = np.float32(3e38) if r % 2 else np.float32(-3e38)
    return workloads.to_storage(x, xd)


@pytest.mark.parametrize("xd", ["bf16", "f32"])
@pytest.mark.parametrize("eps", [1e-6, 0.0])
@pytest.mark.parametrize("hd", [8, 128, 256])
def test_extreme_separate_l2(xd, eps, hd):
    import causal_conv1d_verify_amd as cv

    rng = np.random.default_rng(workloads.BASE_SEED + 3300 + hd)
    rows, d, qk = 7, 1280, 768 if hd != 256 else 512
    x0 = _l2_rows(xd, rows, d, qk, hd, rng)
    # the one case the kernels leave out (eps = 0 with a head's sum of squares below
    # 2^-256) must not occur in these inputs
    xv = (workloads.bf16_bits_to_f32(x0) if xd == "bf16" else x0)[:, :qk].astype(np.float64)
    assert (np.square(xv).reshape(rows, -1, hd).sum(-1) >= 2.0 ** -256).all()
    ref = x0.copy()
    oracle.l2norm(ref, d_inner=d, qk_channels=qk, head_dim=hd, l2_eps=eps, x_dtype=xd)
    _say("extreme l2", xd, eps, hd)
    xt = gh.to_torch(x0, xd)
    cv.conv_qk_l2norm(xt, qk_channels=qk, head_dim=hd, l2_eps=eps)
    got = gh.to_numpy(xt, xd)
    assert np.array_equal(gh._bits(got[:, qk:]), gh._bits(x0[:, qk:])), "L2 wrote past q|k"
    gh.compare_out_elements(got[:, :qk], ref[:, :qk], xd, "l2")


def test_extreme_full_size_headline():
    """The headline shape (128 x 10240, T 8, dedup rows) with the extreme bias, at the
    launch configuration the benchmark times."""
    wl = workloads.WORKLOADS[2]
    inp = _inputs(wl)
    _say("extreme headline", wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)
