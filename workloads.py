"""Seeded synthetic inputs for the batched speculative-verify causal conv1d update.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It holds shapes, seeds and random draws only: none of the method's
arithmetic lives here (no convolution, activation, normalisation or window
logic), so the oracle and the HIP path stay independent of each other.

Workloads (sizes and value distributions follow the pages' workloads):

* ``tiny_fp32_dense``      - n_seq 1, d_inner 512 (q|k 256 in two heads of 128), T 2,
                             fp32 everywhere, dense windows, bias on.
* ``gdn_k17_dense``        - n_seq 8, d_inner 8192 (q|k 4096), T 17 draft tokens
                             (the K=17 verify of the Atlas fused batched verify doc),
                             bf16, dense windows, no bias.
* ``dedup_bs128_t8``       - n_seq 128, d_inner 10240 (q|k 4096), T 8, bf16, dedup rows,
                             bias on (the GB300 workload of sglang PR 46184, "Motivation"
                             and "Benchmarking and Profiling").
* ``kda_t1_f32state``      - n_seq 256, d_inner 12288 (q|k|v = 3 x 32 heads x 128), T 1,
                             bf16 activations with an fp32 conv_state (Atlas KDA block,
                             ``KdaSeqState``), dense windows, no bias.
* ``stress_dedup_t16``     - n_seq 512, d_inner 10240, T 16, bf16, dedup rows, bias on,
                             per-row num_accept_tokens ~ U{0..T-1}, ~10% padded rows,
                             state_len = T + 2.  Pass ``b`` trims d_inner to 10200.

Beyond the fixed-T chain verify, a workload may ask for packed rows (``varlen``: row
i holds T_i ~ U{0..T} tokens, packed back to back, ``cu_seqlens`` their offsets), a
tree (``tree``: parent[i, 0] = -1, parent[i, t] ~ U{-1..t-1}), accepted-prefix
restore indices (``restore``: k_i ~ U{-1..T_i-1}), rows that start from zeros
(``init_frac``: Bernoulli probability that a row has an initial state), or a
prefill (``prefill``: long packed prompts, conv + SiLU with no rollback windows and
the per-head L2 as a separate pass).  These extra draws come after all the draws
above, so they never change the data of a workload that does not use them.

Distributions: state ~ N(0,1), x ~ N(0,1), weight ~ U(-0.5,0.5), bias ~ U(-0.5,0.5),
drawn as float32 from ``numpy.random.Generator(PCG64(seed))`` in exactly that order,
then rounded to the storage dtype (round-to-nearest-even for bf16).  bf16 arrays are
carried as ``numpy.uint16`` bit patterns, fp32 arrays as ``numpy.float32``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BASE_SEED = 20261202
L2_EPS = 1e-6


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_seq: int
    d_inner: int
    qk_channels: int
    head_dim: int
    d_conv: int
    T: int
    x_dtype: str          # "f32" | "bf16" : x, weight, bias, out
    state_dtype: str      # "f32" | "bf16" : conv_state and rollback windows
    layout: str           # "dense" | "dedup" (rows [d, T+D-2]) | "dedup_t" (rows [T+D-2, d])
    bias: bool
    state_len: int        # columns per state channel (>= d_conv - 1)
    seed: int
    accept_offsets: bool = False   # num_accept_tokens ~ U{0..T-1}
    pad_frac: float = 0.0          # Bernoulli probability that a row is padded (slot -1)
    permute_slots: bool = False    # non-padded row i -> slot perm[i]
    x_tok_stride: Optional[int] = None   # elements; None = d_inner (contiguous)
    l2_eps: float = L2_EPS
    dist: str = "normal"          # "normal": the distributions above; "dyadic": see below
    extra_slots: int = 0          # pool slots no row references (must stay untouched)
    varlen: bool = False          # packed rows of T_i ~ U{0..T} tokens
    min_len: int = 0              # lower bound of T_i when varlen
    tree: bool = False            # per-token parents (dense windows, no commit)
    restore: bool = False         # draw accepted-prefix restore indices
    init_frac: float = 1.0        # probability that a row starts from its state
    prefill: bool = False         # conv + SiLU only, no windows; L2 as a separate pass
    state_tm: bool = False        # conv_state stored time-major [n_slots, state_len, d + pad]
    state_col_pad: int = 0        # elements after each time-major state column (untouched)

    @property
    def win_cols(self) -> int:
        return self.d_conv - 1

    @property
    def row_cols(self) -> int:
        return self.T + self.d_conv - 2

    @property
    def n_slots(self) -> int:
        return self.n_seq + self.extra_slots


WORKLOADS = {
    0: Workload("tiny_fp32_dense", 1, 512, 256, 128, 4, 2, "f32", "f32", "dense",
                True, 3, BASE_SEED + 0),
    1: Workload("gdn_k17_dense", 8, 8192, 4096, 128, 4, 17, "bf16", "bf16", "dense",
                False, 3, BASE_SEED + 1),
    2: Workload("dedup_bs128_t8", 128, 10240, 4096, 128, 4, 8, "bf16", "bf16", "dedup",
                True, 3, BASE_SEED + 2),
    3: Workload("kda_t1_f32state", 256, 12288, 8192, 128, 4, 1, "bf16", "f32", "dense",
                False, 3, BASE_SEED + 3),
    4: Workload("stress_dedup_t16", 512, 10240, 4096, 128, 4, 16, "bf16", "bf16", "dedup",
                True, 18, BASE_SEED + 4, accept_offsets=True, pad_frac=0.1,
                permute_slots=True),
    "4b": Workload("stress_dedup_t16_d10200", 512, 10200, 4096, 128, 4, 16, "bf16", "bf16",
                   "dedup", True, 18, BASE_SEED + 104, accept_offsets=True, pad_frac=0.1,
                   permute_slots=True),
    "4s": Workload("stress_dedup_t16_d10200_xstride10240", 512, 10200, 4096, 128, 4, 16,
                   "bf16", "bf16", "dedup", True, 18, BASE_SEED + 104, accept_offsets=True,
                   pad_frac=0.1, permute_slots=True, x_tok_stride=10240),
    # the other rows of the benchmark table of sglang PR 46184 ("Benchmarking and Profiling")
    "b1": Workload("dedup_bs1_t8", 1, 10240, 4096, 128, 4, 8, "bf16", "bf16", "dedup", True, 3,
                   BASE_SEED + 52),
    "b64": Workload("dedup_bs64_t8", 64, 10240, 4096, 128, 4, 8, "bf16", "bf16", "dedup", True,
                    3, BASE_SEED + 62),
    "t16": Workload("dedup_bs128_t16", 128, 10240, 4096, 128, 4, 16, "bf16", "bf16", "dedup",
                    True, 3, BASE_SEED + 72),
    # the headline shape in the other row layout, with packed rows, and its restore
    "2t": Workload("dedup_t_bs128_t8", 128, 10240, 4096, 128, 4, 8, "bf16", "bf16", "dedup_t",
                   True, 3, BASE_SEED + 12),
    "2v": Workload("packed_dedup_bs128_t8", 128, 10240, 4096, 128, 4, 8, "bf16", "bf16",
                   "dedup", True, 3, BASE_SEED + 22, varlen=True, min_len=1),
    "2r": Workload("restore_dedup_bs128_t8", 128, 10240, 4096, 128, 4, 8, "bf16", "bf16",
                   "dedup", True, 3, BASE_SEED + 32, restore=True),
    "4r": Workload("restore_stress_dedup_t16", 512, 10240, 4096, 128, 4, 16, "bf16", "bf16",
                   "dedup", True, 18, BASE_SEED + 34, accept_offsets=True, pad_frac=0.1,
                   permute_slots=True, restore=True),
    # the stress problems with conv_state stored time-major ([n_slots, state_len, d]):
    # the same draws (same seeds), another storage order of the state pool
    "4t": Workload("stress_dedup_t16_tmstate", 512, 10240, 4096, 128, 4, 16, "bf16", "bf16",
                   "dedup", True, 18, BASE_SEED + 4, accept_offsets=True, pad_frac=0.1,
                   permute_slots=True, state_tm=True),
    "4bt": Workload("stress_dedup_t16_d10200_tmstate", 512, 10200, 4096, 128, 4, 16, "bf16",
                    "bf16", "dedup", True, 18, BASE_SEED + 104, accept_offsets=True,
                    pad_frac=0.1, permute_slots=True, state_tm=True),
    "4rt": Workload("restore_stress_dedup_t16_tmstate", 512, 10240, 4096, 128, 4, 16, "bf16",
                    "bf16", "dedup", True, 18, BASE_SEED + 34, accept_offsets=True,
                    pad_frac=0.1, permute_slots=True, restore=True, state_tm=True),
    # ... and from time-major rows, where a window's columns are contiguous: the restore
    # moves exactly its algorithmic bytes
    "4rtt": Workload("restore_stress_dedup_t_t16_tmstate", 512, 10240, 4096, 128, 4, 16, "bf16",
                     "bf16", "dedup_t", True, 18, BASE_SEED + 34, accept_offsets=True,
                     pad_frac=0.1, permute_slots=True, restore=True, state_tm=True),
    # tree verify at the K=17 GDN shape (dense windows, nothing committed)
    "1t": Workload("tree_k17_dense", 8, 8192, 4096, 128, 4, 17, "bf16", "bf16", "dense",
                   False, 3, BASE_SEED + 11, tree=True),
    # a batch of packed prompts through the prefill conv, then the separate q|k L2
    "p": Workload("prefill_8x2048", 8, 10240, 4096, 128, 4, 2048, "bf16", "bf16", "dense",
                  False, 3, BASE_SEED + 40, varlen=True, min_len=1024, prefill=True,
                  init_frac=0.5),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bit patterns.

    NaNs become the quiet NaN 0x7FC0 with their sign kept.  Input preparation only.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = ((u[nan] >> 16) & 0x8000).astype(np.uint16) | 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


def storage_np_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


@dataclasses.dataclass
class Inputs:
    """One seeded problem.  Arrays are host numpy arrays in storage dtype."""
    wl: Workload
    x: np.ndarray            # [n_seq, T, x_tok_stride] (first d_inner columns used)
    weight: np.ndarray       # [d_inner, d_conv]
    bias: Optional[np.ndarray]     # [d_inner] or None
    conv_state: np.ndarray   # [n_slots, d_inner, state_len]
    slot_idx: Optional[np.ndarray]   # int32 [n_seq] or None (identity)
    num_accept_tokens: Optional[np.ndarray]  # int32 [n_seq] or None
    cu_seqlens: Optional[np.ndarray] = None  # int32 [n_seq+1] (varlen): x is [total, xs]
    parent: Optional[np.ndarray] = None      # int32 [n_seq, T] (tree)
    restore_k: Optional[np.ndarray] = None   # int32 [n_seq] (restore)
    has_init: Optional[np.ndarray] = None    # int32 [n_seq] (init_frac < 1)

    @property
    def lengths(self) -> np.ndarray:
        """Tokens per row."""
        if self.cu_seqlens is not None:
            return np.diff(self.cu_seqlens).astype(np.int64)
        return np.full(self.wl.n_seq, self.wl.T, np.int64)


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw one problem in the fixed order state, x, weight, bias, offsets, pads, slots."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    n, T, d, D = wl.n_seq, wl.T, wl.d_inner, wl.d_conv
    xs = wl.x_tok_stride or d
    if wl.dist == "normal":
        state = rng.standard_normal((wl.n_slots, d, wl.state_len), dtype=np.float32)
        x = rng.standard_normal((n, T, d), dtype=np.float32)
        weight = rng.uniform(-0.5, 0.5, size=(d, D)).astype(np.float32)
        bias = rng.uniform(-0.5, 0.5, size=(d,)).astype(np.float32) if wl.bias else None
    elif wl.dist == "dyadic":
        # activations in {k/8 : |k| <= 16}, weights and bias in {j/16 : |j| <= 8}: every
        # product and every 4-term sum is exactly representable in fp32.
        state = (rng.integers(-16, 17, size=(wl.n_slots, d, wl.state_len)) / 8).astype(np.float32)
        x = (rng.integers(-16, 17, size=(n, T, d)) / 8).astype(np.float32)
        weight = (rng.integers(-8, 9, size=(d, D)) / 16).astype(np.float32)
        bias = (rng.integers(-8, 9, size=(d,)) / 16).astype(np.float32) if wl.bias else None
    else:
        raise ValueError(wl.dist)
    nat = None
    if wl.accept_offsets:
        nat = rng.integers(0, T, size=n, dtype=np.int64).astype(np.int32)
    slot = None
    if wl.pad_frac > 0 or wl.permute_slots:
        pad = rng.random(n) < wl.pad_frac if wl.pad_frac > 0 else np.zeros(n, dtype=bool)
        perm = rng.permutation(wl.n_slots).astype(np.int32) if wl.permute_slots \
            else np.arange(n, dtype=np.int32)
        slot = np.where(pad, np.int32(-1), perm[:n]).astype(np.int32)
    cu = parent = rk = has_init = None
    lengths = np.full(n, T, np.int64)
    if wl.varlen:
        lengths = rng.integers(wl.min_len, T + 1, size=n)
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    if wl.tree:
        parent = np.full((n, T), -1, np.int32)
        for t in range(1, T):
            parent[:, t] = rng.integers(-1, t, size=n)
    if wl.restore:
        rk = np.array([rng.integers(-1, max(int(L), 0)) if L > 0 else -1 for L in lengths],
                      dtype=np.int32)
    if wl.init_frac < 1.0:
        has_init = (rng.random(n) < wl.init_frac).astype(np.int32)
    x_st = to_storage(x, wl.x_dtype)
    if cu is not None:
        # packed rows: row i's first T_i draws, back to back
        x_st = np.concatenate([x_st[i, :lengths[i]] for i in range(n)] +
                              [np.zeros((0, d), x_st.dtype)], axis=0)
    if xs != d:
        pad_val = 0x7FBF if wl.x_dtype == "bf16" else np.float32(np.nan)
        xfull = np.full(x_st.shape[:-1] + (xs,), pad_val, dtype=storage_np_dtype(wl.x_dtype))
        xfull[..., :d] = x_st
        x_st = xfull
    return Inputs(
        wl=wl,
        x=x_st,
        weight=to_storage(weight, wl.x_dtype),
        bias=None if bias is None else to_storage(bias, wl.x_dtype),
        conv_state=to_storage(state, wl.state_dtype),
        slot_idx=slot,
        num_accept_tokens=nat,
        cu_seqlens=cu,
        parent=parent,
        restore_k=rk,
        has_init=has_init,
    )


def custom(name="custom", *, n_seq=2, d_inner=256, qk_channels=128, head_dim=64, d_conv=4,
           T=3, x_dtype="bf16", state_dtype="bf16", layout="dense", bias=True,
           state_len=None, seed=BASE_SEED + 1000, **kw) -> Workload:
    """A small problem of any shape, drawn by the same seeded generator."""
    if state_len is None:
        state_len = d_conv - 1 + ((T - 1) if kw.get("accept_offsets") else 0)
    return Workload(name, n_seq, d_inner, qk_channels, head_dim, d_conv, T, x_dtype,
                    state_dtype, layout, bias, state_len, seed, **kw)


def poison_like_windows(wl: Workload) -> np.ndarray:
    """A poison-filled rollback-window buffer (dense or dedup layout) for wl.

    Poison is a NaN bit pattern that no input draw produces, so any element the call
    fails to write (or writes when it must not) is visible bit-for-bit.
    """
    return poison(window_shape(wl), wl.state_dtype)


def window_shape(wl: Workload):
    """Shape of the rollback-window buffer of wl's layout."""
    if wl.layout == "dense":
        return (wl.n_slots, wl.T, wl.d_inner, wl.win_cols)
    if wl.layout == "dedup":
        return (wl.n_slots, wl.d_inner, wl.row_cols)
    if wl.layout == "dedup_t":
        return (wl.n_slots, wl.row_cols, wl.d_inner)
    raise ValueError(wl.layout)


def poison(shape, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full(shape, 0x7FBF, dtype=np.uint16)
    return np.full(shape, 0x7FBFDEAD, dtype=np.uint32).view(np.float32)


def algorithmic_bytes(wl: Workload, inputs: Optional[Inputs] = None) -> int:
    """Bytes one launch must move, counting active (non-padded) rows only.

    x + out + conv_state window read (d_conv-1 columns) + committed window write
    (d_conv-1 columns) + rollback windows (dense: T*(d_conv-1), dedup: T+d_conv-2 per
    channel) + weight + bias (once).
    """
    xb = 4 if wl.x_dtype == "f32" else 2
    sb = 4 if wl.state_dtype == "f32" else 2
    once = wl.d_inner * wl.d_conv * xb + (wl.d_inner * xb if wl.bias else 0)
    if inputs is None:
        rows = [(wl.T, True)] * wl.n_seq
    else:
        lens = inputs.lengths
        act = np.ones(wl.n_seq, bool) if inputs.slot_idx is None else inputs.slot_idx >= 0
        init = np.ones(wl.n_seq, bool) if inputs.has_init is None else inputs.has_init != 0
        rows = [(int(lens[i]), bool(init[i])) for i in range(wl.n_seq) if act[i] and lens[i] > 0]
    total = 0
    for Ti, init in rows:
        if wl.prefill:
            # x and out, the starting window (when the row has one), the committed window
            per_chan = 2 * Ti * xb + (wl.win_cols * sb if init else 0) + wl.win_cols * sb
        else:
            win = Ti * wl.win_cols if wl.layout == "dense" else Ti + wl.d_conv - 2
            commit = 0 if wl.tree else wl.win_cols * sb
            per_chan = 2 * Ti * xb + wl.win_cols * sb + commit + win * sb
        total += wl.d_inner * per_chan
    return total + once


def restore_bytes(wl: Workload, inputs: Inputs) -> int:
    """Bytes an accepted-prefix restore must move: one window read and one state write of
    d_conv-1 columns per channel, for rows with a slot and an index >= 0."""
    sb = 4 if wl.state_dtype == "f32" else 2
    act = np.ones(wl.n_seq, bool) if inputs.slot_idx is None else inputs.slot_idx >= 0
    n = int((act & (inputs.restore_k >= 0)).sum())
    return n * wl.d_inner * 2 * wl.win_cols * sb


def l2_bytes(wl: Workload, inputs: Inputs) -> int:
    """Bytes the separate q|k L2 pass moves over all token rows it is given (every row
    of the packed x): the q|k channels, read and written once."""
    xb = 4 if wl.x_dtype == "f32" else 2
    tokens = int(np.prod(inputs.x.shape[:-1]))
    return 2 * tokens * wl.qk_channels * xb
