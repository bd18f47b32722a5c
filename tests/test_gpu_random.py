"""GPU parity on seeded random configurations.

120 problems drawn from one fixed seed over the whole argument space the verify
accepts: widths 2-4, 1-32 tokens, the three dtype pairs, the three window layouts, tree
parents, packed rows, accept offsets, padded rows, extra slots, strided x, both
conv_state orders (time-major with padded columns), q|k of any head count, channel
counts with partial blocks; about a third are followed by the accepted-prefix restore.
Six more on grids past one resident generation, and eight on the line-aligned build's
shapes (16-token bf16 dedup rows past the token-split threshold).
Each is compared with the oracle's general loop at the
usual bar (windows and state bit-exact over the whole buffers, out within tolerance,
poison kept elsewhere).  The draws are fixed, so a failure names a reproducible case.
"""

import numpy as np
import pytest

import gpu_harness as gh
import workloads

pytestmark = pytest.mark.gpu

HEADS = (4, 8, 16, 32, 64, 128, 256)


def _draw(k: int, rng: np.random.Generator):
    d = 8 * int(rng.integers(1, 300))
    hd = int(rng.choice(HEADS))
    qk = hd * int(rng.integers(0, d // hd + 1)) if d >= hd else 0
    T = int(rng.integers(1, 33))
    tree = bool(rng.random() < 0.2)
    layout = "dense" if tree else str(rng.choice(["dense", "dedup", "dedup_t"]))
    xd, sd = [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")][int(rng.integers(0, 3))]
    tm = bool(rng.random() < 0.5)
    varlen = bool(rng.random() < 0.3)
    stride = None
    if not varlen and rng.random() < 0.3:
        stride = d + 8 * int(rng.integers(1, 5))
    return workloads.custom(
        f"rand{k:02d}", n_seq=int(rng.integers(1, 7)), d_inner=d, qk_channels=qk, head_dim=hd,
        d_conv=int(rng.integers(2, 5)), T=T, x_dtype=xd, state_dtype=sd, layout=layout,
        bias=bool(rng.random() < 0.7), accept_offsets=bool(rng.random() < 0.6),
        pad_frac=float(rng.choice([0.0, 0.2, 0.5])), permute_slots=bool(rng.random() < 0.6),
        extra_slots=int(rng.integers(0, 3)), x_tok_stride=stride, varlen=varlen, tree=tree,
        state_tm=tm, state_col_pad=(8 * int(rng.integers(0, 3))) if tm else 0,
        restore=bool(rng.random() < 0.35), seed=workloads.BASE_SEED + 5000 + k)


_rng = np.random.default_rng(workloads.BASE_SEED + 4999)
CASES = [_draw(k, _rng) for k in range(120)]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_random_config(wl):
    print("[case]", wl, flush=True)
    inp = workloads.make_inputs(wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    if wl.restore:
        p.restore()
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=wl.restore), inp)


def _draw_large(k: int, rng: np.random.Generator):
    """A grid of at least one resident generation (>= 5,120 wavefronts), where the launch
    reads slots first and (partial blocks) follows the XCD order."""
    d = 8 * int(rng.integers(650, 1281))
    blocks = -(-d // 256)
    n = int(rng.integers(-(-5120 // blocks), 700))
    hd = int(rng.choice((64, 128, 256)))
    layout = str(rng.choice(["dense", "dedup", "dedup_t"]))
    tm = bool(rng.random() < 0.5)
    return workloads.custom(
        f"rand_large{k}", n_seq=n, d_inner=d, qk_channels=hd * int(rng.integers(0, d // hd + 1)),
        head_dim=hd, T=int(rng.integers(1, 17)), layout=layout,
        state_dtype=str(rng.choice(["bf16", "f32"])), bias=bool(rng.random() < 0.5),
        accept_offsets=True, pad_frac=0.15, permute_slots=True, extra_slots=1, state_tm=tm,
        state_col_pad=8 if tm else 0, seed=workloads.BASE_SEED + 5500 + k)


_rng_large = np.random.default_rng(workloads.BASE_SEED + 5499)
LARGE = [_draw_large(k, _rng_large) for k in range(6)]


@pytest.mark.parametrize("wl", LARGE, ids=[w.name for w in LARGE])
def test_random_large_grid(wl):
    print("[case]", wl, flush=True)
    inp = workloads.make_inputs(wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)


def _draw_line_aligned(k: int, rng: np.random.Generator):
    """16-token dedup rows in bf16 on grids past the token-split threshold: the
    line-aligned build (4-wavefront workgroups), with either conv_state order, random
    widths, heads, strides and offsets; most draws put some store range off 128-byte
    lines, where a channel-major state takes the build too."""
    d = 8 * int(rng.integers(8, 513))
    blocks = -(-d // 256)
    n = int(rng.integers(2560 // (4 * blocks) + 1, 2560 // (4 * blocks) + 40))
    hd = int(rng.choice((32, 64, 128, 256)))
    D = int(rng.integers(2, 5))
    offsets = bool(rng.random() < 0.7)
    tm = bool(rng.random() < 0.5)
    stride = d + 8 * int(rng.integers(1, 9)) if rng.random() < 0.4 else None
    return workloads.custom(
        f"rand_la{k}", n_seq=n, d_inner=d, qk_channels=hd * int(rng.integers(0, d // hd + 1)),
        head_dim=hd, d_conv=D, T=16, layout="dedup", bias=bool(rng.random() < 0.5),
        accept_offsets=offsets, state_len=(15 + D - 1) if offsets else int(rng.integers(D - 1, 19)),
        pad_frac=float(rng.choice([0.0, 0.15, 0.4])), permute_slots=bool(rng.random() < 0.7),
        extra_slots=int(rng.integers(0, 3)), x_tok_stride=stride, state_tm=tm,
        state_col_pad=8 * int(rng.integers(0, 3)) if tm else 0,
        restore=bool(rng.random() < 0.3), seed=workloads.BASE_SEED + 5600 + k)


_rng_la = np.random.default_rng(workloads.BASE_SEED + 5599)
LINE_ALIGNED = [_draw_line_aligned(k, _rng_la) for k in range(8)]


@pytest.mark.parametrize("wl", LINE_ALIGNED, ids=[w.name for w in LINE_ALIGNED])
def test_random_line_aligned(wl):
    print("[case]", wl, flush=True)
    inp = workloads.make_inputs(wl)
    p = gh.GeneralProblem(inp)
    p.verify()
    if wl.restore:
        p.restore()
    gh.compare_general(p.results(), gh.oracle_general(inp, restore=wl.restore), inp)
