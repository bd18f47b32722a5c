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
