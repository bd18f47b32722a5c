"""Runs a seeded problem through the HIP library and compares it with the oracle.

Used by the GPU parity tests, smoke() and bench.py.  The GPU side goes through the
Python binding of the C ABI only; the oracle side through oracle.run_inputs.
"""

from __future__ import annotations

import numpy as np

import workloads


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    elif dtype == "i32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
    else:
        raise ValueError(dtype)
    return t.to(device)


def to_numpy(t, dtype: str) -> np.ndarray:
    import torch

    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceProblem:
    """Device copies of a problem's inputs plus poison-filled outputs."""

    def __init__(self, inp: workloads.Inputs, device="cuda"):
        wl = inp.wl
        self.inp, self.wl = inp, wl
        self.x = to_torch(inp.x, wl.x_dtype, device)[:, :, :wl.d_inner]
        self.weight = to_torch(inp.weight, wl.x_dtype, device)
        self.bias = None if inp.bias is None else to_torch(inp.bias, wl.x_dtype, device)
        self.conv_state = to_torch(inp.conv_state, wl.state_dtype, device)
        self.slot_idx = None if inp.slot_idx is None else to_torch(inp.slot_idx, "i32", device)
        self.nat = None if inp.num_accept_tokens is None else to_torch(
            inp.num_accept_tokens, "i32", device)
        self.out_full = to_torch(workloads.poison(inp.x.shape, wl.x_dtype), wl.x_dtype, device)
        self.out = self.out_full[:, :, :wl.d_inner]
        self.windows = to_torch(workloads.poison_like_windows(wl), wl.state_dtype, device)

    def run(self, stream=None):
        import causal_conv1d_verify_amd as cv

        fn = cv.conv_verify_update_dedup if self.wl.layout == "dedup" \
            else cv.conv_verify_update_dense
        fn(self.x, self.weight, self.bias, self.conv_state, self.out, self.windows,
           qk_channels=self.wl.qk_channels, head_dim=self.wl.head_dim, l2_eps=self.wl.l2_eps,
           slot_idx=self.slot_idx, num_accept_tokens=self.nat, stream=stream)

    def results(self):
        import torch

        torch.cuda.synchronize()
        wl = self.wl
        return {"out": to_numpy(self.out_full, wl.x_dtype),
                "windows": to_numpy(self.windows, wl.state_dtype),
                "conv_state": to_numpy(self.conv_state, wl.state_dtype)}


def run_gpu(inp: workloads.Inputs, stream=None):
    p = DeviceProblem(inp)
    p.run(stream)
    return p.results()


def _bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def bf16_ordered(b: np.ndarray) -> np.ndarray:
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


F32_ATOL = 1e-5
F32_RTOL = 1e-5
BF16_ULPS = 1


def compare(gpu: dict, ref: dict, wl: workloads.Workload, active_rows) -> dict:
    """Asserts parity; returns a small report.

    * rollback windows and conv_state: bit-exact over the whole buffers, so untouched
      slots and padded rows' slots are checked too;
    * out: fp32 |g-r| <= 1e-5 + 1e-5|r|; bf16 within 1 ulp of the oracle's
      correctly rounded value (NaN matches NaN); padded rows' out rows and the
      columns past d_inner (strided out) keep their poison bits.
    """
    rep = {}
    gw, rw = _bits(gpu["windows"]), _bits(ref["windows"])
    bad = np.flatnonzero(gw.ravel() != rw.ravel())
    assert bad.size == 0, f"{bad.size} window elements differ, first at {np.unravel_index(bad[0], gw.shape)}: gpu {gw.ravel()[bad[0]]:#x} oracle {rw.ravel()[bad[0]]:#x}"
    gs, rs = _bits(gpu["conv_state"]), _bits(ref["conv_state"])
    bad = np.flatnonzero(gs.ravel() != rs.ravel())
    assert bad.size == 0, f"{bad.size} conv_state elements differ, first at {np.unravel_index(bad[0], gs.shape)}"
    go, ro = gpu["out"], ref["out"]
    mask = np.zeros(go.shape, bool)
    if len(active_rows):
        mask[np.asarray(active_rows), :, :wl.d_inner] = True
    # everything outside the active rows' [T, d_inner] block keeps its poison bits
    assert np.array_equal(_bits(go)[~mask], _bits(ro)[~mask]), "out written outside active rows"
    g, r = go[mask], ro[mask]
    if wl.x_dtype == "f32":
        same = (np.isnan(g) & np.isnan(r)) | (g == r)      # equal infinities included
        with np.errstate(invalid="ignore"):
            err = np.where(same, 0.0, np.abs(g.astype(np.float64) - r.astype(np.float64)))
        lim = F32_ATOL + F32_RTOL * np.abs(r.astype(np.float64))
        with np.errstate(invalid="ignore"):
            ratio = np.where(err == 0, 0.0, err / lim)
        bad = np.flatnonzero(~(ratio <= 1.0))
        if bad.size:
            idx = np.argwhere(mask)[bad[:5]]
            raise AssertionError(
                f"fp32 out tolerance exceeded at {bad.size} elements; first (row, t, c) "
                f"{idx.tolist()}: gpu {g[bad[:5]].tolist()} oracle {r[bad[:5]].tolist()}")
        worst = float(np.max(ratio, initial=0.0))
        rep["out_max_err_over_tol"] = worst
    else:
        gn = (g & 0x7FFF) > 0x7F80
        rn = (r & 0x7FFF) > 0x7F80
        assert np.array_equal(gn, rn), "NaN positions differ"
        d = np.abs(bf16_ordered(g[~gn]) - bf16_ordered(r[~rn]))
        rep["out_max_ulp"] = int(d.max(initial=0))
        rep["out_ulp_hist"] = np.bincount(d.clip(0, 3), minlength=4).tolist()
        assert rep["out_max_ulp"] <= BF16_ULPS, f"bf16 out off by {rep['out_max_ulp']} ulp"
    return rep


def active_rows(inp: workloads.Inputs):
    if inp.slot_idx is None:
        return list(range(inp.wl.n_seq))
    return [i for i in range(inp.wl.n_seq) if inp.slot_idx[i] >= 0]


def check_against_oracle(inp: workloads.Inputs, stream=None) -> dict:
    import oracle

    ref = oracle.run_inputs(inp)
    gpu = run_gpu(inp, stream)
    return compare(gpu, ref, inp.wl, active_rows(inp))


# ---- the general entry points: packed rows, trees, all layouts, restore, prefill, L2 ------

def _tok_index(inp, i, t):
    return (int(inp.cu_seqlens[i]) + t,) if inp.cu_seqlens is not None else (i, t)


def computed_tokens(inp):
    """Out positions the call computes: active rows (slot >= 0), tokens below T_i."""
    lens = inp.lengths
    for i in range(inp.wl.n_seq):
        s = i if inp.slot_idx is None else int(inp.slot_idx[i])
        if s < 0:
            continue
        for t in range(int(lens[i])):
            yield _tok_index(inp, i, t)


class GeneralProblem:
    """Device copies of a general problem (any layout, packed rows, tree, restore
    indices, prefill flags) plus poison-filled outputs."""

    def __init__(self, inp: workloads.Inputs, layout=None, device="cuda"):
        import dataclasses

        wl = inp.wl
        self.inp, self.wl = inp, wl
        self.layout = layout or wl.layout
        d = wl.d_inner
        self.x = to_torch(inp.x, wl.x_dtype, device)[..., :d]
        self.weight = to_torch(inp.weight, wl.x_dtype, device)
        self.bias = None if inp.bias is None else to_torch(inp.bias, wl.x_dtype, device)
        self.state_raw = self.state_raw0 = None
        if wl.state_tm:
            # time-major storage [n_slots, state_len, d + pad]; the library gets the
            # [n_slots, d, state_len] view of it (channel stride 1)
            n, _, sl = inp.conv_state.shape
            raw = workloads.poison((n, sl, d + wl.state_col_pad), wl.state_dtype)
            raw[:, :, :d] = inp.conv_state.transpose(0, 2, 1)
            self.state_raw0 = raw
            self.state_raw = to_torch(raw, wl.state_dtype, device)
            self.conv_state = self.state_raw[:, :, :d].transpose(1, 2)
        else:
            self.conv_state = to_torch(inp.conv_state, wl.state_dtype, device)
        i32 = lambda a: None if a is None else to_torch(a, "i32", device)   # noqa: E731
        self.slot_idx, self.nat = i32(inp.slot_idx), i32(inp.num_accept_tokens)
        self.cu, self.parent = i32(inp.cu_seqlens), i32(inp.parent)
        self.restore_k, self.has_init = i32(inp.restore_k), i32(inp.has_init)
        self.out_full = to_torch(workloads.poison(inp.x.shape, wl.x_dtype), wl.x_dtype, device)
        self.out = self.out_full[..., :d]
        self.windows = None
        if not wl.prefill:
            shape = workloads.window_shape(dataclasses.replace(wl, layout=self.layout))
            self.windows = to_torch(workloads.poison(shape, wl.state_dtype), wl.state_dtype, device)

    def verify(self, stream=None):
        import causal_conv1d_verify_amd as cv

        wl = self.wl
        if self.cu is not None and self.x.shape[0] == 0:
            return   # every packed row is empty: nothing to compute or write
        kw = dict(qk_channels=wl.qk_channels, head_dim=wl.head_dim, l2_eps=wl.l2_eps,
                  slot_idx=self.slot_idx, num_accept_tokens=self.nat, cu_seqlens=self.cu,
                  stream=stream)
        if wl.tree:
            cv.conv_verify_update_tree(self.x, self.weight, self.bias, self.conv_state, self.out,
                                       self.windows, self.parent, **kw)
        else:
            cv.conv_verify_update(self.x, self.weight, self.bias, self.conv_state, self.out,
                                  self.windows, layout=self.layout, **kw)

    def restore(self, stream=None):
        import causal_conv1d_verify_amd as cv

        cv.conv_verify_restore(self.conv_state, self.windows, self.restore_k,
                               layout=self.layout, d_conv=self.wl.d_conv,
                               slot_idx=self.slot_idx, stream=stream)

    def prefill(self, stream=None):
        import causal_conv1d_verify_amd as cv

        cv.conv_prefill(self.x, self.weight, self.bias, self.conv_state, self.out, self.cu,
                        max_len=self.wl.T, slot_idx=self.slot_idx,
                        has_initial_state=self.has_init, stream=stream)

    def results(self):
        import torch

        torch.cuda.synchronize()
        wl = self.wl
        res = {"out": to_numpy(self.out_full, wl.x_dtype),
               "conv_state": to_numpy(self.conv_state, wl.state_dtype)}
        if self.state_raw is not None and wl.state_col_pad:
            pad = _bits(to_numpy(self.state_raw, wl.state_dtype))[:, :, wl.d_inner:]
            assert np.array_equal(pad, _bits(self.state_raw0)[:, :, wl.d_inner:]), \
                "time-major conv_state: padding after a column was written"
        if self.windows is not None:
            res["windows"] = to_numpy(self.windows, wl.state_dtype)
        return res


def oracle_general(inp: workloads.Inputs, layout=None, restore=False):
    """The oracle's general loop on inp (prefill or verify; then the restore if asked)."""
    import dataclasses

    import oracle

    wl = inp.wl
    layout = layout or wl.layout
    state = inp.conv_state.copy()
    out = workloads.poison(inp.x.shape, wl.x_dtype)
    if wl.prefill:
        oracle.prefill(inp.x, inp.weight, inp.bias, state, out, inp.cu_seqlens,
                       d_inner=wl.d_inner, x_dtype=wl.x_dtype, state_dtype=wl.state_dtype,
                       slot_idx=inp.slot_idx, has_init=inp.has_init)
        return {"out": out, "conv_state": state}
    windows = workloads.poison(workloads.window_shape(dataclasses.replace(wl, layout=layout)),
                               wl.state_dtype)
    oracle.verify_general(inp.x, inp.weight, inp.bias, state, out, windows, T=wl.T,
                          d_inner=wl.d_inner, qk_channels=wl.qk_channels,
                          head_dim=wl.head_dim, l2_eps=wl.l2_eps, x_dtype=wl.x_dtype,
                          state_dtype=wl.state_dtype, layout=layout, slot_idx=inp.slot_idx,
                          num_accept_tokens=inp.num_accept_tokens, cu_seqlens=inp.cu_seqlens,
                          parent=inp.parent, commit=not wl.tree)
    if restore:
        oracle.restore(state, windows, inp.restore_k, T=wl.T, d_conv=wl.d_conv,
                       state_dtype=wl.state_dtype, layout=layout, slot_idx=inp.slot_idx)
    return {"out": out, "windows": windows, "conv_state": state}


def compare_out_elements(g: np.ndarray, r: np.ndarray, x_dtype: str, where: str = "out") -> dict:
    """fp32 within 1e-5 + 1e-5|r| (NaN matches NaN), bf16 within one ulp."""
    rep = {}
    if x_dtype == "f32":
        same = (np.isnan(g) & np.isnan(r)) | (g == r)
        with np.errstate(invalid="ignore"):
            err = np.where(same, 0.0, np.abs(g.astype(np.float64) - r.astype(np.float64)))
            lim = F32_ATOL + F32_RTOL * np.abs(r.astype(np.float64))
            ratio = np.where(err == 0, 0.0, err / lim)
        bad = np.flatnonzero(~(ratio <= 1.0))
        assert bad.size == 0, (f"fp32 {where} tolerance exceeded at {bad.size} elements: gpu "
                               f"{g[bad[:5]].tolist()} oracle {r[bad[:5]].tolist()}")
        rep["max_err_over_tol"] = float(np.max(ratio, initial=0.0))
    else:
        gn = (g & 0x7FFF) > 0x7F80
        rn = (r & 0x7FFF) > 0x7F80
        assert np.array_equal(gn, rn), f"{where}: NaN positions differ"
        dd = np.abs(bf16_ordered(g[~gn]) - bf16_ordered(r[~rn]))
        rep["max_ulp"] = int(dd.max(initial=0))
        assert rep["max_ulp"] <= BF16_ULPS, f"bf16 {where} off by {rep['max_ulp']} ulp"
    return rep


def compare_general(gpu: dict, ref: dict, inp: workloads.Inputs) -> dict:
    """Windows and conv_state bit-exact over the whole buffers; out within tolerance on
    the computed tokens' channels and poison everywhere else."""
    for k in ("windows", "conv_state"):
        if k in ref:
            g, r = _bits(gpu[k]), _bits(ref[k])
            bad = np.flatnonzero(g.ravel() != r.ravel())
            assert bad.size == 0, (f"{bad.size} {k} elements differ, first at "
                                   f"{np.unravel_index(bad[0], g.shape)}: gpu {g.ravel()[bad[0]]:#x} "
                                   f"oracle {r.ravel()[bad[0]]:#x}")
    go, ro = gpu["out"], ref["out"]
    mask = np.zeros(go.shape, bool)
    for idx in computed_tokens(inp):
        mask[idx + (slice(0, inp.wl.d_inner),)] = True
    assert np.array_equal(_bits(go)[~mask], _bits(ro)[~mask]), "out written outside the computed tokens"
    return compare_out_elements(go[mask], ro[mask], inp.wl.x_dtype)
