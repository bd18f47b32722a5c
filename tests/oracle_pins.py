"""Pins of the CPU oracle against facts fixed outside it.

Each ``pin_*`` function runs the oracle (a given build of it: ``lib``) on small seeded
problems and raises AssertionError when the oracle disagrees with something that
does not come from the oracle itself: the fp64 brute force of ``brute.py`` (exact on
dyadic inputs), torch's depthwise conv1d, closed forms, invariants of the windows,
the golden window-indexing fixture, or the rounding rule.  ``test_oracle_pins.py``
runs them on the real oracle; ``test_oracle_mutations.py`` runs them on builds with
a planted mistake and requires that at least one fails.
"""

from __future__ import annotations

import dataclasses
import os

import numpy as np

import brute
import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _run(inp, lib, debug=True):
    return oracle.run_inputs(inp, debug=debug, lib=lib)


def _windows_bits(a, dtype):
    return brute.bits(a, dtype).astype(np.uint64)


def _check_against_brute(inp, lib, exact: bool):
    wl = inp.wl
    r = _run(inp, lib)
    b = brute.brute(inp.x, inp.weight, inp.bias, inp.conv_state, d_inner=wl.d_inner,
                    qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
                    x_dtype=wl.x_dtype, state_dtype=wl.state_dtype, layout=wl.layout,
                    slot_idx=inp.slot_idx, num_accept_tokens=inp.num_accept_tokens)
    rows = [i for i, _ in b["active"]]
    assert rows or wl.n_seq == 0 or inp.slot_idx is not None
    # rollback windows and the committed state: bit patterns
    wb = _windows_bits(r["windows"], wl.state_dtype)
    untouched = b["windows"] == 0xFFFFFFFF
    poison_bits = _windows_bits(workloads.poison_like_windows(wl), wl.state_dtype)
    assert np.array_equal(wb[~untouched], b["windows"][~untouched]), "rollback windows differ"
    assert np.array_equal(wb[untouched], poison_bits[untouched]), "untouched windows written"
    assert np.array_equal(brute.bits(r["conv_state"], wl.state_dtype),
                          b["conv_state"]), "committed conv_state differs"
    # conv (fp32, fused multiply-add per tap) and SiLU/L2 (fp64)
    pre_o = r["pre"][rows, :, :].astype(np.float64)
    pre_b = b["pre"][rows]
    if exact:
        assert np.array_equal(pre_o, pre_b), "conv pre-activation not exact on dyadic inputs"
        assert np.allclose(r["y"][rows], b["y"][rows], rtol=1e-12, atol=1e-300), "y differs"
    else:
        terms = np.abs(pre_b) + 8.0           # |bias| + sum |W v| is well below this here
        assert np.all(np.abs(pre_o - pre_b) <= wl.d_conv * 2.0 ** -24 * terms), "conv error"
        assert np.allclose(r["y"][rows], b["y"][rows], rtol=1e-5, atol=1e-6), "y differs"
    # outputs: rounded once from y; padded rows untouched
    out_o = r["out"][:, :, :wl.d_inner]
    if wl.x_dtype == "bf16":
        ob = out_o[rows]
        bb = b["out"][rows]
        if exact:
            assert np.array_equal(ob, bb), "bf16 outputs differ from exact rounding"
        else:
            diff = np.abs(ob.astype(np.int64) - bb.astype(np.int64))
            assert diff.max(initial=0) <= 1, "bf16 outputs differ by more than one ulp"
    else:
        if exact:
            assert np.array_equal(out_o[rows], b["out"][rows]), "fp32 outputs differ"
        else:
            assert np.allclose(out_o[rows], b["out"][rows], rtol=1e-6, atol=1e-7)
    pad_rows = [i for i in range(wl.n_seq) if i not in rows]
    if pad_rows:
        pz = workloads.poison(inp.x.shape, wl.x_dtype)
        assert np.array_equal(brute.bits(r["out"][pad_rows], wl.x_dtype),
                              brute.bits(pz[pad_rows], wl.x_dtype)), "padded row out written"
    if inp.x.shape[2] > wl.d_inner:
        pz = workloads.poison(inp.x.shape, wl.x_dtype)
        assert np.array_equal(brute.bits(r["out"][:, :, wl.d_inner:], wl.x_dtype),
                              brute.bits(pz[:, :, wl.d_inner:], wl.x_dtype)), "stride gap written"
    return r, b


# ---- cases ------------------------------------------------------------------------

def _cases():
    """Small problems covering the branches of the method (and a ragged everything)."""
    c = workloads.custom
    yield c("dense_bf16", T=3, layout="dense")
    yield c("dedup_bf16", T=5, layout="dedup")
    yield c("dense_f32", T=2, x_dtype="f32", state_dtype="f32")
    yield c("dedup_mixed", T=4, x_dtype="bf16", state_dtype="f32", layout="dedup")
    yield c("dense_mixed_t1", T=1, x_dtype="bf16", state_dtype="f32", bias=False)
    yield c("d2", d_conv=2, T=3, layout="dedup")
    yield c("d3", d_conv=3, T=2, layout="dense")
    yield c("qk0", qk_channels=0, T=3)
    yield c("qk_all", qk_channels=256, head_dim=32, T=2, layout="dedup")
    yield c("offsets_pads", n_seq=6, T=4, layout="dedup", accept_offsets=True,
            pad_frac=0.3, permute_slots=True, extra_slots=2)
    yield c("offsets_dense", n_seq=4, T=3, layout="dense", accept_offsets=True,
            permute_slots=True)
    yield c("strided_x", n_seq=3, T=3, d_inner=120, qk_channels=64, head_dim=16,
            x_tok_stride=136, layout="dedup")
    yield c("t17", n_seq=2, T=17, d_inner=64, qk_channels=32, head_dim=16)
    # heads of 12 and 24 channels (not dividing a power-of-two channel block)
    yield c("heads12", n_seq=2, T=3, d_inner=72, qk_channels=48, head_dim=12, layout="dedup")
    yield c("heads24_f32", n_seq=2, T=2, d_inner=80, qk_channels=72, head_dim=24,
            x_dtype="f32", state_dtype="f32")


def pin_brute_dyadic(lib):
    """Oracle == fp64 brute force, bit for bit, on dyadic inputs (every fp32 sum exact)."""
    for wl in _cases():
        wl = workloads.Workload(**{**wl.__dict__, "dist": "dyadic"})
        _check_against_brute(workloads.make_inputs(wl), lib, exact=True)


def pin_brute_normal(lib):
    """Oracle within fp32 rounding of the fp64 brute force on N(0,1) inputs."""
    for wl in _cases():
        _check_against_brute(workloads.make_inputs(wl), lib, exact=False)


def pin_torch_conv1d(lib):
    """qk_channels = 0 reduces to torch's depthwise causal conv1d (groups=d_inner) + SiLU."""
    import torch
    import torch.nn.functional as F

    for layout, T, D in (("dense", 4, 4), ("dedup", 6, 3), ("dense", 1, 2)):
        wl = workloads.custom("torch", n_seq=3, d_inner=96, qk_channels=0, head_dim=32,
                              d_conv=D, T=T, layout=layout, dist="dyadic",
                              accept_offsets=True)
        inp = workloads.make_inputs(wl)
        r = _run(inp, lib)
        xv = brute.values(inp.x, wl.x_dtype)
        sv = brute.values(inp.conv_state, wl.state_dtype)
        for i in range(wl.n_seq):
            a = int(inp.num_accept_tokens[i])
            seq = np.concatenate([sv[i, :, a:a + D - 1], xv[i].T], axis=1)     # [C, T+D-1]
            o = F.conv1d(torch.from_numpy(seq)[None], torch.from_numpy(
                brute.values(inp.weight, wl.x_dtype))[:, None, :],
                torch.from_numpy(brute.values(inp.bias, wl.x_dtype)), groups=wl.d_inner)
            y = F.silu(o)[0].numpy().T                                          # [T, C]
            assert np.allclose(r["y"][i], y, rtol=1e-13, atol=1e-300), "conv1d+silu differs"
            assert np.array_equal(r["pre"][i].astype(np.float64), o[0].numpy().T)


def pin_one_hot_taps(lib):
    """A one-hot tap on the newest input gives silu(x_t + b); on the oldest, a pure delay."""
    for tap in ("newest", "oldest"):
        wl = workloads.custom("onehot", n_seq=2, d_inner=64, qk_channels=0, d_conv=4, T=5,
                              x_dtype="f32", state_dtype="f32", bias=True)
        inp = workloads.make_inputs(wl)
        w = np.zeros_like(inp.weight)
        w[:, -1 if tap == "newest" else 0] = 1.0
        inp.weight = w
        r = _run(inp, lib)
        x = inp.x.astype(np.float64)
        b = inp.bias.astype(np.float64)
        if tap == "newest":
            want = x + b[None, None, :]
        else:
            st = inp.conv_state.astype(np.float64)
            seq = np.concatenate([np.transpose(st[:, :, 0:3], (0, 2, 1)), x], axis=1)
            want = seq[:, 0:wl.T, :] + b[None, None, :]
        assert np.array_equal(r["pre"].astype(np.float64),
                              want.astype(np.float32).astype(np.float64)), f"{tap} tap"


def pin_l2_closed_form(lib):
    """After L2 each q|k head has sum y^2 = S/(S+eps); V channels keep silu(pre).  Heads
    of 32 channels (4 heads) and of 24 (5 heads)."""
    for eps, hd, nh in ((1e-6, 32, 4), (0.5, 32, 4), (40.0, 32, 4), (1e-6, 24, 5), (40.0, 24, 5)):
        qk = hd * nh
        wl = workloads.custom("l2", n_seq=2, d_inner=192, qk_channels=qk, head_dim=hd,
                              T=3, l2_eps=eps)
        inp = workloads.make_inputs(wl)
        r = _run(inp, lib)
        pre = r["pre"].astype(np.float64)
        s = brute.silu(pre)
        y = r["y"]
        assert np.allclose(y[:, :, qk:], s[:, :, qk:], rtol=1e-13, atol=1e-300), "V touched"
        h = s[:, :, :qk].reshape(2, 3, nh, hd)
        S = (h * h).sum(-1)
        yh = y[:, :, :qk].reshape(2, 3, nh, hd)
        got = (yh * yh).sum(-1)
        assert np.allclose(got, S / (S + np.float64(np.float32(eps))), rtol=1e-12), "L2 form"
        # direction is unchanged by the normalisation
        assert np.all(np.sign(yh) == np.sign(h)), "L2 sign"


def pin_window_invariants(lib):
    """snap[t][j+1] == snap[t+1][j]; snap[T-1] == committed state; dedup row == dense."""
    for T in (1, 2, 5):
        base = dict(n_seq=3, d_inner=64, qk_channels=32, head_dim=16, T=T, accept_offsets=True,
                    permute_slots=True)
        wd = workloads.custom("inv_dense", layout="dense", **base)
        ww = workloads.custom("inv_dedup", layout="dedup", **base)
        rd = _run(workloads.make_inputs(wd), lib)
        rw = _run(workloads.make_inputs(ww), lib)
        snap = rd["windows"]                        # [n_slots, T, C, 3]
        row = rw["windows"]                         # [n_slots, C, T+2]
        for t in range(T - 1):
            assert np.array_equal(snap[:, t, :, 1:], snap[:, t + 1, :, :-1])
        assert np.array_equal(snap[:, T - 1], rd["conv_state"][:, :, 0:3])
        for t in range(T):
            assert np.array_equal(row[:, :, t:t + 3], snap[:, t]), "dedup view != dense window"
        assert np.array_equal(rd["out"], rw["out"]), "layout changed the outputs"
        assert np.array_equal(rd["conv_state"], rw["conv_state"])


def pin_batched_equals_rows(lib):
    """A batched call equals one call per row (each window is independent)."""
    wl = workloads.custom("batch", n_seq=5, d_inner=64, qk_channels=32, head_dim=16, T=4,
                          layout="dedup", accept_offsets=True, pad_frac=0.2,
                          permute_slots=True, extra_slots=1)
    inp = workloads.make_inputs(wl)
    r = _run(inp, lib)
    state = inp.conv_state.copy()
    windows = workloads.poison_like_windows(wl)
    out = workloads.poison(inp.x.shape, wl.x_dtype)
    for i in range(wl.n_seq):
        oracle.conv_verify(inp.x[i:i + 1], inp.weight, inp.bias, state, out[i:i + 1], windows,
                           d_inner=wl.d_inner, qk_channels=wl.qk_channels,
                           head_dim=wl.head_dim, l2_eps=wl.l2_eps, x_dtype=wl.x_dtype,
                           state_dtype=wl.state_dtype, layout=wl.layout,
                           slot_idx=inp.slot_idx[i:i + 1],
                           num_accept_tokens=inp.num_accept_tokens[i:i + 1], lib=lib)
    assert np.array_equal(out, r["out"]) and np.array_equal(windows, r["windows"])
    assert np.array_equal(state, r["conv_state"])


def pin_offset_equivalence(lib):
    """Offset a on state S == offset 0 on S' = S[:, :, a:a+D-1] (windows and outputs)."""
    wl = workloads.custom("off", n_seq=4, d_inner=64, qk_channels=32, head_dim=16, T=4,
                          layout="dense", accept_offsets=True)
    inp = workloads.make_inputs(wl)
    r = _run(inp, lib)
    for i in range(wl.n_seq):
        a = int(inp.num_accept_tokens[i])
        sub = np.ascontiguousarray(inp.conv_state[i:i + 1, :, a:a + 3])
        win = workloads.poison((1, wl.T, wl.d_inner, 3), wl.state_dtype)
        out = workloads.poison((1, wl.T, wl.d_inner), wl.x_dtype)
        oracle.conv_verify(inp.x[i:i + 1], inp.weight, inp.bias, sub, out, win,
                           d_inner=wl.d_inner, qk_channels=wl.qk_channels,
                           head_dim=wl.head_dim, l2_eps=wl.l2_eps, x_dtype=wl.x_dtype,
                           state_dtype=wl.state_dtype, layout="dense", lib=lib)
        assert np.array_equal(out[0], r["out"][i]), "offset changes outputs"
        assert np.array_equal(win[0], r["windows"][i]), "offset changes windows"
        assert np.array_equal(sub[0], r["conv_state"][i, :, 0:3])
        assert np.array_equal(r["conv_state"][i, :, 3:], inp.conv_state[i, :, 3:]), \
            "columns past the window were written"


def pin_golden_window_indexing(lib):
    """The hand-written fixture of tests/golden/window_indexing.txt."""
    g = load_golden(os.path.join(HERE, "golden", "window_indexing.txt"))
    state = np.array(g["state"], np.float32).reshape(1, 1, -1)
    x = np.array(g["x"], np.float32).reshape(1, -1, 1)
    T = x.shape[1]
    w = np.array(g["weight"], np.float32).reshape(1, -1)
    a = int(g["num_accept_tokens"][0])
    outs = {}
    for layout in ("dense", "dedup"):
        st = state.copy()
        win = np.zeros((1, T, 1, 3) if layout == "dense" else (1, 1, T + 2), np.float32)
        out = np.zeros((1, T, 1), np.float32)
        oracle.conv_verify(x, w, None, st, out, win, d_inner=1, qk_channels=0, head_dim=1,
                           l2_eps=1e-6, x_dtype="f32", state_dtype="f32", layout=layout,
                           num_accept_tokens=np.array([a], np.int32), lib=lib)
        outs[layout] = (st, win, out)
    st, win, _ = outs["dedup"]
    assert win.ravel().tolist() == g["dedup_row"], "dedup row"
    st_d, win_d, out_d = outs["dense"]
    for t in range(T):
        assert win_d[0, t, 0].tolist() == g[f"window_{t}"], f"window {t}"
    assert st_d.ravel().tolist() == g["state_after"], "committed state"
    # outputs: the conv over the page's windows [v_t, window_t] with v = [state, x]
    v = np.concatenate([np.array(g["state"]), np.array(g["x"])])
    pre = np.array([np.dot(g["weight"], v[t:t + 4]) for t in range(T)])
    assert np.array_equal(out_d.ravel(), brute.silu(pre).astype(np.float32)), "outputs"


def pin_rounding(lib):
    """fp64 -> bf16 round-to-nearest-even against an independent rounding and torch."""
    import torch

    rng = np.random.default_rng(7)
    ys = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 39, 20000),
        rng.standard_normal(2000) * 1e-39,                      # bf16 subnormals
        [0.0, -0.0, 3.3895313892515355e38, 3.3961775292304e38, 3.4e38, 1e39, -1e39,
         np.inf, -np.inf, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126],
    ])
    # exact midpoints between neighbouring bf16 values (ties) and one step off them
    mids = []
    for b in rng.integers(0x0001, 0x7F7F, 3000):
        lo = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        hi = float(np.array([(b + 1) << 16], np.uint32).view(np.float32)[0])
        m = (lo + hi) / 2
        mids += [m, -m, np.nextafter(m, 0), np.nextafter(m, np.inf)]
    ys = np.concatenate([ys, mids])
    got = np.array([lib.orc_round_bf16(float(v)) for v in ys], np.uint16)
    want = brute.round_bf16_exact(ys)
    assert np.array_equal(got, want), "bf16 rounding"
    f = rng.standard_normal(5000).astype(np.float32)
    tb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([lib.orc_round_bf16(float(v)) for v in f], np.uint16)
    assert np.array_equal(got, tb), "bf16 rounding vs torch"


def pin_bit_copies(lib):
    """Windows and state carry bit patterns: -0.0, subnormals and NaN payloads survive."""
    for xd, sd in (("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")):
        wl = workloads.custom("bits", n_seq=2, d_inner=32, qk_channels=0, T=3, x_dtype=xd,
                              state_dtype=sd, layout="dedup")
        inp = workloads.make_inputs(wl)
        specials_bf16 = np.array([0x8000, 0x0001, 0x807F, 0x7FA1, 0xFFC3, 0x7F80], np.uint16)
        specials_f32 = np.array([0x80000000, 0x00000001, 0x807FFFFF, 0x7FA00001, 0xFFC00003,
                                 0x7F800000], np.uint32).view(np.float32)
        xs = specials_bf16 if xd == "bf16" else specials_f32
        ss = specials_bf16 if sd == "bf16" else specials_f32
        inp.x[0, :, :6] = xs
        inp.conv_state[1, :6, 1] = ss
        r = _run(inp, lib)
        b = brute.brute(inp.x, inp.weight, inp.bias, inp.conv_state, d_inner=32,
                        qk_channels=0, head_dim=1, l2_eps=1e-6, x_dtype=xd, state_dtype=sd,
                        layout="dedup")
        assert np.array_equal(_windows_bits(r["windows"], sd), b["windows"])
        assert np.array_equal(brute.bits(r["conv_state"], sd), b["conv_state"])


def _round_f32_exact(q):
    """A rational rounded to the nearest fp32 (ties to even), computed exactly."""
    from fractions import Fraction

    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    e = max(e, -126)                       # subnormal quantum below 2^-126
    scaled = q / Fraction(2) ** (e - 23)   # significand with 23 fraction bits
    n, rem = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * rem
    if twice > scaled.denominator or (twice == scaled.denominator and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n) * Fraction(2) ** (e - 23))


def pin_fma_chain_exact(lib):
    """The conv is one correctly rounded fp32 fused multiply-add per tap, in tap order.

    Checked against an exact rational evaluation of acc <- round32(W[c,w]*v + acc),
    acc starting at the bias: each step has one rounding, with operands whose fp32
    products are not exact (fp32 activations, fp32 state).
    """
    from fractions import Fraction

    for xd, sd in (("f32", "f32"), ("bf16", "f32")):
        wl = workloads.custom("fma", n_seq=2, d_inner=48, qk_channels=0, d_conv=4, T=3,
                              x_dtype=xd, state_dtype=sd, bias=True)
        inp = workloads.make_inputs(wl)
        r = _run(inp, lib)
        xv = brute.values(inp.x, xd)
        sv = brute.values(inp.conv_state, sd)
        wv = brute.values(inp.weight, xd)
        bv = brute.values(inp.bias, xd)
        for i in range(wl.n_seq):
            seq = np.concatenate([sv[i, :, 0:3], xv[i].T], axis=1)
            for t in range(wl.T):
                for c in range(wl.d_inner):
                    acc = Fraction(float(bv[c]))
                    for w in range(4):
                        acc = Fraction(_round_f32_exact(
                            Fraction(float(wv[c, w])) * Fraction(float(seq[c, t + w])) + acc))
                    assert float(r["pre"][i, t, c]) == float(acc), "fma chain"


# ---- the general loop: packed rows, trees, all window layouts, restore, prefill ----------

def _general_oracle(inp, lib, *, layout=None, do_l2=True, commit=None):
    wl = inp.wl
    state = inp.conv_state.copy()
    out = workloads.poison(inp.x.shape, wl.x_dtype)
    windows = None if wl.prefill else workloads.poison(
        workloads.window_shape(dataclasses.replace(wl, layout=layout or wl.layout)),
        wl.state_dtype)
    commit = (not wl.tree) if commit is None else commit
    pre, y = oracle.verify_general(
        inp.x, inp.weight, inp.bias, state, out, windows, T=wl.T, d_inner=wl.d_inner,
        qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
        x_dtype=wl.x_dtype, state_dtype=wl.state_dtype, layout=layout or wl.layout,
        slot_idx=inp.slot_idx, num_accept_tokens=inp.num_accept_tokens,
        cu_seqlens=inp.cu_seqlens, parent=inp.parent, has_init=inp.has_init,
        do_l2=do_l2, commit=commit, debug=True, lib=lib)
    return {"out": out, "windows": windows, "conv_state": state, "pre": pre, "y": y}


def _brute_general(inp, *, layout=None, do_l2=True, commit=None):
    wl = inp.wl
    return brute.brute_general(
        inp.x, inp.weight, inp.bias, inp.conv_state, T=wl.T, d_inner=wl.d_inner,
        qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
        x_dtype=wl.x_dtype, state_dtype=wl.state_dtype, layout=layout or wl.layout,
        slot_idx=inp.slot_idx, num_accept_tokens=inp.num_accept_tokens,
        cu_seqlens=inp.cu_seqlens, parent=inp.parent, has_init=inp.has_init,
        do_l2=do_l2, commit=(not wl.tree) if commit is None else commit)


def _token_rows(inp, active):
    """(row, token, index into out's leading dims) of every token the call computes."""
    lens = inp.lengths
    for i, _ in active:
        for t in range(int(lens[i])):
            yield i, t, ((int(inp.cu_seqlens[i]) + t,) if inp.cu_seqlens is not None else (i, t))


def _check_general(inp, lib, *, layout=None, exact=True, do_l2=True):
    wl = inp.wl
    r = _general_oracle(inp, lib, layout=layout, do_l2=do_l2)
    b = _brute_general(inp, layout=layout, do_l2=do_l2)
    if r["windows"] is not None:
        wb = _windows_bits(r["windows"], wl.state_dtype)
        untouched = b["windows"] == 0xFFFFFFFF
        poison_bits = _windows_bits(workloads.poison(r["windows"].shape, wl.state_dtype),
                                    wl.state_dtype)
        assert np.array_equal(wb[~untouched], b["windows"][~untouched]), "rollback windows differ"
        assert np.array_equal(wb[untouched], poison_bits[untouched]), "untouched windows written"
    assert np.array_equal(brute.bits(r["conv_state"], wl.state_dtype),
                          b["conv_state"]), "conv_state differs"
    written = np.zeros(inp.x.shape[:-1], bool)
    for i, t, idx in _token_rows(inp, b["active"]):
        written[idx] = True
        po, pb = np.float64(r["pre"][i, t]), b["pre"][i, t]
        ob = brute.bits(r["out"][idx][:wl.d_inner], wl.x_dtype).astype(np.int64)
        bb = brute.bits(b["out"][i, t], wl.x_dtype).astype(np.int64)
        if exact:
            assert np.array_equal(po, pb), f"conv pre-activation differs (row {i}, token {t})"
            assert np.array_equal(ob, bb), f"outputs differ (row {i}, token {t})"
        else:
            assert np.allclose(r["y"][i, t], b["y"][i, t], rtol=1e-5, atol=1e-6)
    pz = brute.bits(workloads.poison(inp.x.shape, wl.x_dtype), wl.x_dtype)
    assert np.array_equal(brute.bits(r["out"], wl.x_dtype)[~written], pz[~written]), \
        "out written for a token the call does not compute"


def pin_window_layouts(lib):
    """Chain verify in all three window layouts (time-major rows included) against the
    path brute force, exactly, with offsets, permuted slots, padded rows, spare slots."""
    for layout in ("dense", "dedup", "dedup_t"):
        for D, T in ((4, 5), (3, 2), (2, 4)):
            wl = workloads.custom(f"lay_{layout}_{D}_{T}", n_seq=5, d_inner=24, qk_channels=16,
                                  head_dim=8, d_conv=D, T=T, layout=layout, dist="dyadic",
                                  accept_offsets=True, permute_slots=True, pad_frac=0.3,
                                  extra_slots=2, seed=workloads.BASE_SEED + 2100 + D * 10 + T)
            _check_general(workloads.make_inputs(wl), lib)


def pin_packed_rows(lib):
    """Packed variable-length rows (zero-length rows included) against the brute force
    run row by row on each row's own tokens, in every layout."""
    for k, layout in enumerate(("dense", "dedup", "dedup_t")):
        for xd, sd in (("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")):
            wl = workloads.custom(f"var_{layout}_{xd}_{sd}", n_seq=6, d_inner=16,
                                  qk_channels=8, head_dim=4, T=6, layout=layout, x_dtype=xd,
                                  state_dtype=sd, dist="dyadic", varlen=True,
                                  accept_offsets=True, permute_slots=True, pad_frac=0.2,
                                  seed=workloads.BASE_SEED + 2200 + k * 7 + len(xd + sd))
            _check_general(workloads.make_inputs(wl), lib)


def pin_tree_paths(lib):
    """Tree verify: each token's conv over its root window and the x of its ancestor
    path, windows dense, nothing committed - against the path brute force, exactly;
    also with packed rows and a zero-start row."""
    for k, (D, T, var) in enumerate(((4, 7, False), (3, 5, False), (4, 6, True))):
        wl = workloads.custom(f"tree_{D}_{T}_{var}", n_seq=5, d_inner=16, qk_channels=8,
                              head_dim=8, d_conv=D, T=T, dist="dyadic", tree=True,
                              varlen=var, accept_offsets=True, permute_slots=True,
                              pad_frac=0.2, init_frac=0.7,
                              seed=workloads.BASE_SEED + 2300 + k)
        _check_general(workloads.make_inputs(wl), lib)


def pin_tree_with_chain_parents(lib):
    """A tree whose parents form a chain (parent = t-1) gives the chain's outputs and
    windows; it leaves conv_state alone where the chain commits."""
    wl = workloads.custom("chain_tree", n_seq=4, d_inner=32, qk_channels=16, head_dim=8, T=6,
                          accept_offsets=True, permute_slots=True, pad_frac=0.25)
    inp = workloads.make_inputs(wl)
    chain = _general_oracle(inp, lib)
    inp.parent = np.tile(np.arange(-1, wl.T - 1, dtype=np.int32), (wl.n_seq, 1))
    tree = _general_oracle(inp, lib, commit=False)
    assert np.array_equal(brute.bits(chain["out"], wl.x_dtype), brute.bits(tree["out"], wl.x_dtype))
    assert np.array_equal(brute.bits(chain["windows"], wl.state_dtype),
                          brute.bits(tree["windows"], wl.state_dtype))
    assert np.array_equal(brute.bits(tree["conv_state"], wl.state_dtype),
                          brute.bits(inp.conv_state, wl.state_dtype)), "tree verify committed"


def pin_restore(lib):
    """Accepted-prefix restore: window k of the slot (chain or tree, every layout) lands in
    state columns 0..D-2 - compared with the brute force's window k, i.e. the committed
    state of a verify of the first k+1 tokens; later columns, slot -1 and k = -1 rows
    untouched."""
    cases = [("dense", False), ("dedup", False), ("dedup_t", False), ("dense", True)]
    for n, (layout, tree) in enumerate(cases):
        wl = workloads.custom(f"restore_{layout}_{tree}", n_seq=6, d_inner=16, qk_channels=8,
                              head_dim=8, T=5, layout=layout, tree=tree, restore=True,
                              accept_offsets=True, permute_slots=True, pad_frac=0.2,
                              extra_slots=1, seed=workloads.BASE_SEED + 2400 + n)
        inp = workloads.make_inputs(wl)
        r = _general_oracle(inp, lib)
        b = _brute_general(inp)
        state = r["conv_state"].copy()
        oracle.restore(state, r["windows"], inp.restore_k, T=wl.T, d_conv=wl.d_conv,
                       state_dtype=wl.state_dtype, layout=layout, slot_idx=inp.slot_idx,
                       lib=lib)
        want = brute.bits(r["conv_state"], wl.state_dtype).copy()
        W1 = wl.win_cols
        for i, s in b["active"]:
            k = int(inp.restore_k[i])
            if k < 0:
                continue
            if layout == "dense":
                w = b["windows"][s, k]
            elif layout == "dedup":
                w = b["windows"][s, :, k:k + W1]
            else:
                w = b["windows"][s, k:k + W1, :].T
            want[s, :, :W1] = w
        assert np.array_equal(brute.bits(state, wl.state_dtype), want), f"restore ({layout})"


def pin_prefill_torch(lib):
    """Prefill conv (conv + SiLU, no L2, no windows) over packed prompts against torch's
    depthwise conv1d: rows without an initial state are the textbook causal conv
    (zero left padding), rows with one prepend their state window; the last window
    is committed."""
    import torch
    import torch.nn.functional as F

    wl = workloads.custom("prefill", n_seq=5, d_inner=16, qk_channels=8, head_dim=8, T=40,
                          dist="dyadic", varlen=True, prefill=True, init_frac=0.5,
                          permute_slots=True, seed=workloads.BASE_SEED + 2500)
    inp = workloads.make_inputs(wl)
    state = inp.conv_state.copy()
    out = workloads.poison(inp.x.shape, wl.x_dtype)
    oracle.prefill(inp.x, inp.weight, inp.bias, state, out, inp.cu_seqlens, d_inner=wl.d_inner,
                   x_dtype=wl.x_dtype, state_dtype=wl.state_dtype, slot_idx=inp.slot_idx,
                   has_init=inp.has_init, lib=lib)
    W1, D, C = wl.win_cols, wl.d_conv, wl.d_inner
    w = torch.from_numpy(brute.values(inp.weight, wl.x_dtype)).reshape(C, 1, D)
    bvec = torch.from_numpy(brute.values(inp.bias, wl.x_dtype))
    for i in range(wl.n_seq):
        s = int(inp.slot_idx[i])
        t0, Ti = int(inp.cu_seqlens[i]), int(inp.cu_seqlens[i + 1] - inp.cu_seqlens[i])
        xr = torch.from_numpy(brute.values(inp.x[t0:t0 + Ti, :C], wl.x_dtype)).T   # [C, Ti]
        if inp.has_init[i]:
            left = torch.from_numpy(brute.values(inp.conv_state[s, :, :W1], wl.state_dtype))
        else:
            left = torch.zeros(C, W1, dtype=torch.float64)
        seq = torch.cat([left, xr], dim=1)
        pre = F.conv1d(seq[None], w, bvec, groups=C)[0]                       # [C, Ti]
        y = F.silu(pre).T.numpy()
        got = brute.bits(out[t0:t0 + Ti, :C], wl.x_dtype)
        assert np.array_equal(got, brute.round_bf16_exact(y).astype(np.uint32)), f"prefill row {i}"
        if Ti > 0:
            tail = np.concatenate([brute.bits(inp.conv_state[s, :, :W1], wl.state_dtype)
                                   if inp.has_init[i] else np.zeros((C, W1), np.uint32),
                                   brute.x_bits_as_state(inp.x[t0:t0 + Ti, :C], wl.x_dtype,
                                                         wl.state_dtype).T], axis=1)[:, -W1:]
            assert np.array_equal(brute.bits(state[s, :, :W1], wl.state_dtype), tail), \
                f"prefill row {i} committed window"
        assert np.array_equal(state[s, :, W1:], inp.conv_state[s, :, W1:])


def pin_separate_l2(lib):
    """The separate L2 pass: every q|k head ends with sum y^2 = S/(S+eps) (S the head's
    sum of squares before), V channels keep their bits, for fp32 and bf16 rows, a large eps
    that makes the eps term visible, and heads of 8, 12 and 24 channels."""
    rng = np.random.default_rng(workloads.BASE_SEED + 2600)
    for xd, eps, tol, hd in (("f32", 1e-6, 1e-6, 8), ("f32", 10.0, 1e-6, 8), ("bf16", 10.0, 2e-2, 8),
                             ("f32", 10.0, 1e-6, 12), ("bf16", 10.0, 2e-2, 24)):
        C, rows = 56, 5
        qk = 48 if hd != 8 else 32
        x0 = workloads.to_storage(rng.standard_normal((rows, C + 8)).astype(np.float32), xd)
        x = x0.copy()
        oracle.l2norm(x, d_inner=C, qk_channels=qk, head_dim=hd, l2_eps=eps, x_dtype=xd, lib=lib)
        v0 = brute.values(x0, xd)
        v1 = brute.values(x, xd)
        for h in range(qk // hd):
            sl = slice(h * hd, (h + 1) * hd)
            S = (v0[:, sl] ** 2).sum(axis=1)
            got = (v1[:, sl] ** 2).sum(axis=1)
            assert np.allclose(got, S / (S + eps), rtol=tol, atol=0), f"L2 head {h} ({xd}, eps {eps})"
        assert np.array_equal(brute.bits(x[:, qk:], xd), brute.bits(x0[:, qk:], xd)), "V written"


def load_golden(path):
    """Parse a ``key: v1 v2 ...`` fixture (lines starting with # are comments)."""
    g = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            g[k.strip()] = [float(t) for t in v.split()]
    return g


PINS = [pin_brute_dyadic, pin_brute_normal, pin_fma_chain_exact, pin_torch_conv1d,
        pin_one_hot_taps,
        pin_l2_closed_form, pin_window_invariants, pin_batched_equals_rows,
        pin_offset_equivalence, pin_golden_window_indexing, pin_rounding, pin_bit_copies,
        pin_window_layouts, pin_packed_rows, pin_tree_paths, pin_tree_with_chain_parents,
        pin_restore, pin_prefill_torch, pin_separate_l2]
