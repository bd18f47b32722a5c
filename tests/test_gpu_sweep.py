"""GPU parity on a broad seeded sweep: 400 random verify problems over the whole argument
space the library accepts - heads that divide 256 channels and heads that do not, the three
window layouts, tree parents, packed rows (empty ones included), accept offsets, padded rows,
extra and permuted slots, strided x, both conv_state orders (time-major with padded
columns), widths 2-4, 1-32 tokens, the three dtype pairs, 1 to 300 rows, and the
accepted-prefix restore after a third of them.  Each is compared with the oracle's general
loop at the usual bar (windows and state bit-exact over the whole buffers, out within
tolerance, poison kept elsewhere).  The draws are fixed, so a failure names a reproducible
case.  (This sweep is what exposed the 16-byte store hazard described in cv_device.h.)
Then 60 random prefill launches, each followed by the separate L2 with a random head size.
"""

import numpy as np
import pytest

import gpu_harness as gh
import workloads

pytestmark = pytest.mark.gpu

NON_POW2 = (12, 20, 24, 36, 40, 48, 56, 72, 80, 96, 112, 144, 160, 192, 208, 240)
POW2 = (4, 8, 16, 32, 64, 128, 256)


def _block(hd, align):
    k = 256 // hd
    while k and (k * hd) % align:
        k -= 1
    return k * hd


def _draw(k: int, rng: np.random.Generator):
    xd, sd = [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")][int(rng.integers(0, 3))]
    align = 4 if (xd, sd) == ("f32", "f32") else 8
    pool = NON_POW2 if rng.random() < 0.5 else POW2
    while True:
        hd = int(rng.choice(pool))
        heads = int(rng.integers(0, 14))
        if hd in POW2 or (_block(hd, align) and (hd * heads) % align == 0):
            break
    qk = hd * heads
    d = max(8, qk + 8 * int(rng.integers(0 if qk else 1, 140)))
    d += (-d) % 8
    T = int(rng.integers(1, 33))
    tree = bool(rng.random() < 0.15)
    layout = "dense" if tree else str(rng.choice(["dense", "dedup", "dedup_t"]))
    tm = bool(rng.random() < 0.5)
    varlen = bool(rng.random() < 0.25)
    stride = d + 8 * int(rng.integers(1, 5)) if not varlen and rng.random() < 0.3 else None
    n = int(rng.choice([1, 2, 3, 5, 7, 16, 40, 130, 300]))
    D = int(rng.integers(2, 5))
    offsets = bool(rng.random() < 0.6)
    state_len = (T + D - 2 + int(rng.integers(0, 3))) if offsets else D - 1 + int(rng.integers(0, 3))
    return workloads.custom(
        f"sweep{k:03d}", n_seq=n, d_inner=d, qk_channels=qk, head_dim=hd, d_conv=D, T=T,
        x_dtype=xd, state_dtype=sd, layout=layout, bias=bool(rng.random() < 0.7),
        accept_offsets=offsets, state_len=state_len, pad_frac=float(rng.choice([0.0, 0.2, 0.5])),
        permute_slots=bool(rng.random() < 0.6), extra_slots=int(rng.integers(0, 3)),
        x_tok_stride=stride, varlen=varlen, tree=tree, state_tm=tm,
        state_col_pad=(8 * int(rng.integers(0, 3))) if tm else 0,
        restore=bool(rng.random() < 0.3) and not tree, seed=workloads.BASE_SEED + 90000 + k)


_rng = np.random.default_rng(workloads.BASE_SEED + 89999)
CASES = [_draw(k, _rng) for k in range(400)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_sweep(wl):
    print("[case]", wl, flush=True)
    inp = workloads.make_inputs(wl)
    if inp.x.shape[0] == 0:
        return   # an empty packed batch: nothing to launch or compare
    p = gh.GeneralProblem(inp)
    p.verify()
    if wl.restore:
        p.restore()
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=wl.restore), inp)


def _draw_prefill(k: int, rng: np.random.Generator):
    xd, sd = [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")][int(rng.integers(0, 3))]
    tm = bool(rng.random() < 0.5)
    return workloads.custom(
        f"sweep_prefill{k:02d}", n_seq=int(rng.integers(1, 9)), d_inner=8 * int(rng.integers(1, 400)),
        qk_channels=0, d_conv=int(rng.integers(2, 5)), T=int(rng.integers(1, 300)), x_dtype=xd,
        state_dtype=sd, varlen=True, prefill=True, init_frac=float(rng.choice([0.0, 0.5, 1.0])),
        permute_slots=bool(rng.random() < 0.5), state_len=int(rng.integers(3, 12)), state_tm=tm,
        state_col_pad=8 * int(rng.integers(0, 3)) if tm else 0, bias=bool(rng.random() < 0.6),
        seed=workloads.BASE_SEED + 95000 + k)


_rng_prefill = np.random.default_rng(workloads.BASE_SEED + 94999)
PREFILL = []
for _k in range(60):
    _wl = _draw_prefill(_k, _rng_prefill)
    # a separate L2 over the prefill's rows, with a head size that fits the row
    _hd = int(_rng_prefill.choice([4, 8, 16, 32, 64, 128, 12, 24, 48, 96]))
    _al = 16 // (4 if _wl.x_dtype == "f32" else 2)
    _nh = _wl.d_inner // _hd
    _qk = _hd * int(_rng_prefill.integers(0, _nh + 1)) if _nh else 0
    if _qk % _al or (_hd not in POW2 and not _block(_hd, _al)):
        _qk = 0
    PREFILL.append((_wl, _hd, _qk))


@pytest.mark.parametrize("case", PREFILL, ids=[c[0].name for c in PREFILL])
def test_sweep_prefill_then_l2(case):
    """Random prefill launches (packed prompts up to 300 tokens, empty ones included, either
    state order and dtype pair), then the separate L2 over the rows with a random head size
    (power of two or not) - each stage against the oracle on the same input."""
    import causal_conv1d_verify_amd as cv
    import oracle

    wl, hd, qk = case
    print("[case]", wl, "L2 heads", hd, "q|k", qk, flush=True)
    inp = workloads.make_inputs(wl)
    if inp.x.shape[0] == 0:
        return
    p = gh.GeneralProblem(inp)
    p.prefill()
    got = p.results()
    gh.compare_general(got, gh.oracle_general(inp), inp)
    out = got["out"][:, :wl.d_inner].copy()
    ref = out.copy()
    oracle.l2norm(ref, d_inner=wl.d_inner, qk_channels=qk, head_dim=hd, l2_eps=1e-6,
                  x_dtype=wl.x_dtype)
    xt = gh.to_torch(out, wl.x_dtype)
    cv.conv_qk_l2norm(xt, qk_channels=qk, head_dim=hd, l2_eps=1e-6)
    gh.compare_out_elements(gh.to_numpy(xt, wl.x_dtype), ref, wl.x_dtype, "l2")
