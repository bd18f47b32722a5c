"""GPU parity at the size limits of the boundary.

* Rows that span almost the 2 GiB a buffer resource can address: x and out with a token
  stride that puts a row's last token 2^31 - 16 bytes after its first byte (the host's
  limit), so every per-token offset the kernels form sits just below 2^31, next to the
  out-of-range lane offset 2^31.
* Slot strides beyond 2 GiB (conv_state and the rollback windows, both state orders):
  slot bases are 64-bit, the offsets within a slot stay 32-bit.
* A grid of 131,072 wavefronts (4,096 rows x 8,192 channels, T 1, fp32 state).

The problems are small in values and large in address space: their buffers are
poison-filled device allocations of several GiB with the problem's elements placed through
strided views, and the oracle runs on the compact problem.  Bars as everywhere (windows and
state bit-exact, out within 1e-5 + 1e-5|r| or 1 bf16 ulp), plus sampled poison checks of the
bytes between the elements that must not be written.
"""

import numpy as np
import pytest

import gpu_harness as gh
import workloads

pytestmark = pytest.mark.gpu

SPAN = (1 << 31) - 16   # bytes a row (or a slot's state) may span


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import causal_conv1d_verify_amd._lib as L

    L.load()


def _say(*a):
    print("[case]", *a, flush=True)


def _tdtype(dt):
    import torch

    return torch.bfloat16 if dt == "bf16" else torch.float32


def _poison_bits(dt):
    return 0x7FBF if dt == "bf16" else 0x7FC00123


def _big(total, dt):
    """A poison-filled device buffer of `total` elements."""
    import torch

    t = torch.empty(total, dtype=_tdtype(dt), device="cuda")
    iv = t.view(torch.int16 if dt == "bf16" else torch.int32)
    iv.fill_(_poison_bits(dt))
    return t


def _place(buf, shape, strides, arr, dt):
    """The strided view of buf with the compact array's elements copied in."""
    v = buf.as_strided(shape, strides)
    v.copy_(gh.to_torch(arr, dt))
    return v


def _sample_poison(buf, dt, touched, n=4096, seed=0):
    """n random element positions outside `touched` (a sorted array of flat indices written
    or read by the problem) still hold the poison bits."""
    import torch

    rng = np.random.default_rng(seed)
    total = buf.numel()
    pos = rng.integers(0, total, size=n * 2)
    pos = pos[~np.isin(pos, touched)][:n]
    iv = buf.view(torch.int16 if dt == "bf16" else torch.int32)
    got = iv[torch.from_numpy(pos).to("cuda")].cpu().numpy().astype(np.int64) & (0xFFFF if dt == "bf16" else 0xFFFFFFFF)
    assert (got == _poison_bits(dt)).all(), "an element that no call may write was written"


def _flat_indices(shape, strides):
    idx = np.zeros(shape, dtype=np.int64)
    for ax, (n, s) in enumerate(zip(shape, strides)):
        sh = [1] * len(shape)
        sh[ax] = n
        idx = idx + (np.arange(n, dtype=np.int64) * s).reshape(sh)
    return np.sort(idx.ravel())


def test_row_span_at_the_limit():
    """x and out rows whose tokens lie 2^31 - 16 bytes apart (end to end)."""
    import causal_conv1d_verify_amd as cv

    wl = workloads.custom("span_limit", n_seq=2, d_inner=256, qk_channels=128, head_dim=64,
                          T=2, layout="dense", accept_offsets=True, state_len=4)
    inp = workloads.make_inputs(wl)
    d, T, n = wl.d_inner, wl.T, wl.n_seq
    tok = SPAN // 2 - d                 # ((T-1) * tok + d) * 2 bytes == SPAN
    seq = (T - 1) * tok + d
    total = (n - 1) * seq + (T - 1) * tok + d
    _say(wl.name, "token stride", tok, "elements, buffers of", total * 2 / 2**30, "GiB")
    xb, ob = _big(total, "bf16"), _big(total, "bf16")
    x = _place(xb, (n, T, d), (seq, tok, 1), inp.x, "bf16")
    out = ob.as_strided((n, T, d), (seq, tok, 1))
    p = gh.GeneralProblem(inp)
    cv.conv_verify_update(x, p.weight, p.bias, p.conv_state, out, p.windows, layout="dense",
                          qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
                          num_accept_tokens=p.nat)
    got = p.results()
    got["out"] = gh.to_numpy(out.contiguous(), "bf16")
    gh.compare_general(got, gh.oracle_general(inp), inp)
    _sample_poison(ob, "bf16", _flat_indices((n, T, d), (seq, tok, 1)))


@pytest.mark.parametrize("layout", ["dense", "dedup", "dedup_t"])
@pytest.mark.parametrize("tm", [False, True], ids=["cm", "tm"])
def test_slot_strides_beyond_2gib(layout, tm):
    """conv_state and windows whose slots lie more than 2 GiB apart; permuted slots and
    accept offsets, 16 tokens (the rows token split on this small grid, dense chains the
    token-split kernel)."""
    import causal_conv1d_verify_amd as cv

    wl = workloads.custom(f"slot_stride_{layout}_{'tm' if tm else 'cm'}", n_seq=3, d_inner=512,
                          qk_channels=256, head_dim=128, T=16, layout=layout, accept_offsets=True,
                          permute_slots=True, state_len=18)
    inp = workloads.make_inputs(wl)
    d, SL, ns = wl.d_inner, wl.state_len, wl.n_slots
    big = (1 << 30) + 64               # elements: 2 GiB + 128 bytes per slot (bf16)
    _say(wl.name, "slot stride", big, "elements")
    p = gh.GeneralProblem(inp)
    if tm:
        st_shape, st_strides = (ns, d, SL), (big, 1, d)       # time-major columns of d
        st_arr = inp.conv_state
    else:
        st_shape, st_strides = (ns, d, SL), (big, SL, 1)
        st_arr = inp.conv_state
    sb = _big((ns - 1) * big + d * SL, "bf16")
    state = _place(sb, st_shape, st_strides, st_arr, "bf16")
    wshape = tuple(p.windows.shape)
    wstrides = (big,) + tuple(p.windows.stride()[1:])
    wb = _big((ns - 1) * big + int(np.prod(wshape[1:])), "bf16")
    windows = _place(wb, wshape, wstrides, gh.to_numpy(p.windows, "bf16"), "bf16")
    cv.conv_verify_update(p.x, p.weight, p.bias, state, p.out, windows, layout=layout,
                          qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
                          slot_idx=p.slot_idx, num_accept_tokens=p.nat)
    got = p.results()
    got["conv_state"] = gh.to_numpy(state.contiguous(), "bf16")
    got["windows"] = gh.to_numpy(windows.contiguous(), "bf16")
    gh.compare_general(got, gh.oracle_general(inp), inp)
    _sample_poison(sb, "bf16", _flat_indices(st_shape, st_strides), seed=1)
    _sample_poison(wb, "bf16", _flat_indices(wshape, wstrides), seed=2)


def test_131072_wavefronts():
    """4,096 rows x 8,192 channels, T 1, dense windows, fp32 state: 131,072 wavefronts in
    25 resident generations (slot-first), every row checked against the oracle."""
    wl = workloads.custom("grid_4096x8192", n_seq=4096, d_inner=8192, qk_channels=4096,
                          head_dim=128, T=1, layout="dense", state_dtype="f32",
                          permute_slots=True, pad_frac=0.05, extra_slots=3)
    inp = workloads.make_inputs(wl)
    _say(wl.name)
    p = gh.GeneralProblem(inp)
    p.verify()
    gh.compare_general(p.results(), gh.oracle_general(inp), inp)
