"""fp64 brute force of the verify conv, written from the whole-sequence definition.

Independent of the oracle's per-token loop: for each active row it concatenates the
initial window and all T inputs into one sequence u = [state[a..a+D-2] | x_0..x_{T-1}]
per channel, takes every width-D sliding window of u at once, and reads every
rollback window, the dedup row and the committed window as slices of u.  SiLU uses
the tanh form x * (1 + tanh(x/2)) / 2; the bf16 rounding compares exact distances to
the two neighbouring bf16 values instead of scaling.

Facts used (cited by page and section):
* windows after token t are u[t+1 .. t+D-1]; the dedup row is u[1 .. T+D-2], so step
  t's window is its columns t..t+D-2 (sglang PR 46184, "Motivation", "Modifications");
* conv_state ends holding the committed window u[T .. T+D-2], which equals the last
  snapshot (Atlas docs, fn gdn_verify_fused_conv_kn_batched);
* L2 is 1/sqrt(sum + eps) over each head of the q|k channels, V untouched (Atlas
  glm5next_kda/mod.rs, Glm5NextKdaConfig).
"""

from __future__ import annotations

import numpy as np
from numpy.lib.stride_tricks import sliding_window_view


def values(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def bits(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return a.astype(np.uint32)
    return np.ascontiguousarray(a).view(np.uint32).copy()


def x_bits_as_state(a: np.ndarray, x_dtype: str, state_dtype: str) -> np.ndarray:
    if x_dtype == state_dtype:
        return bits(a, x_dtype)
    assert x_dtype == "bf16" and state_dtype == "f32"
    return a.astype(np.uint32) << 16


def bf16_neighbours(y: np.ndarray):
    """The bf16 values just below and above |y| (as float64), elementwise, |y| finite."""
    ay = np.abs(y)
    f = ay.astype(np.float32)
    fb = f.view(np.uint32)
    lo = (fb & 0xFFFF0000).view(np.float32).astype(np.float64)
    # if truncation overshot (float rounding up past y), step down one bf16 ulp
    over = lo > ay
    lo_b = np.where(over, (fb & 0xFFFF0000) - 0x10000, fb & 0xFFFF0000).astype(np.uint32)
    lo = lo_b.view(np.float32).astype(np.float64)
    hi_b = (lo_b + 0x10000).astype(np.uint32)
    hi = hi_b.view(np.float32).astype(np.float64)
    hi = np.where(hi_b == 0x7F800000, 2.0 ** 128, hi)   # the step past the largest bf16
    return lo_b, lo, hi_b, hi


def round_bf16_exact(y: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, nearest with ties to even, by comparing exact distances."""
    y = np.asarray(y, dtype=np.float64)
    out = np.zeros(y.shape, np.uint16)
    sign = np.where(np.signbit(y), 0x8000, 0).astype(np.uint32)
    fin = np.isfinite(y)
    yf = np.where(fin, y, 0.0)
    lo_b, lo, hi_b, hi = bf16_neighbours(yf)
    ay = np.abs(yf)
    dlo, dhi = ay - lo, hi - ay          # exact (Sterbenz) for neighbouring values
    pick_hi = (dhi < dlo) | ((dhi == dlo) & ((lo_b >> 16) & 1 == 1))
    mag = np.where(pick_hi, hi_b, lo_b) >> 16
    mag = np.where(ay >= 2.0 ** 128, 0x7F80, mag)   # beyond float range: inf
    res = (sign | mag).astype(np.uint16)
    res = np.where(np.isnan(y), (sign | 0x7FC0).astype(np.uint16), res)
    res = np.where(np.isinf(y), (sign | 0x7F80).astype(np.uint16), res)
    out[...] = res
    return out


def silu(p: np.ndarray) -> np.ndarray:
    return p * (1.0 + np.tanh(p / 2.0)) / 2.0


def brute(x, weight, bias, conv_state, *, d_inner, qk_channels, head_dim, l2_eps,
          x_dtype, state_dtype, layout, slot_idx=None, num_accept_tokens=None):
    """Returns dict: pre (fp64), y (fp64), out bits, windows bits, conv_state bits.

    Arrays for padded rows / unreferenced slots hold None-equivalents: ``active`` lists
    the active rows and the slot of each.  Windows and state are returned as full
    arrays in the input's bit layout with untouched entries copied from ``conv_state``
    (state) or set to the sentinel 0xFFFFFFFF (windows).
    """
    n_seq, T, _ = x.shape
    D = weight.shape[1]
    W1 = D - 1
    C = d_inner
    n_slots, _, state_len = conv_state.shape
    xv = values(x[:, :, :C], x_dtype)
    xb = x_bits_as_state(x[:, :, :C], x_dtype, state_dtype)
    wv = values(weight, x_dtype)
    bv = values(bias, x_dtype) if bias is not None else np.zeros(C)
    sv = values(conv_state, state_dtype)
    sb = bits(conv_state, state_dtype)

    pre = np.full((n_seq, T, C), np.nan)
    y = np.full((n_seq, T, C), np.nan)
    state_after = sb.copy()
    if layout == "dense":
        win = np.full((n_slots, T, C, W1), 0xFFFFFFFF, np.uint64)
    else:
        win = np.full((n_slots, C, T + D - 2), 0xFFFFFFFF, np.uint64)
    active = []
    for i in range(n_seq):
        s = i if slot_idx is None else int(slot_idx[i])
        if s < 0:
            continue
        a = 0 if num_accept_tokens is None else int(num_accept_tokens[i])
        active.append((i, s))
        u = np.concatenate([sv[s, :, a:a + W1], xv[i].T], axis=1)        # [C, T+W1]
        ub = np.concatenate([sb[s, :, a:a + W1], xb[i].T], axis=1)
        sw = sliding_window_view(u, D, axis=1)                          # [C, T, D]
        p = (sw * wv[:, None, :]).sum(axis=2) + bv[:, None]             # [C, T]
        yy = silu(p)
        if qk_channels:
            h = yy[:qk_channels].reshape(qk_channels // head_dim, head_dim, T)
            ss = (h * h).sum(axis=1, keepdims=True)
            yy[:qk_channels] = (h / np.sqrt(ss + np.float64(np.float32(l2_eps)))).reshape(
                qk_channels, T)
        pre[i] = p.T
        y[i] = yy.T
        if layout == "dense":
            for t in range(T):
                win[s, t] = ub[:, t + 1:t + D]
        else:
            win[s] = ub[:, 1:T + D - 1]
        state_after[s, :, :W1] = ub[:, T:T + W1]
    if x_dtype == "bf16":
        out = round_bf16_exact(y)
    else:
        out = y.astype(np.float32)
    return {"pre": pre, "y": y, "out": out, "windows": win, "conv_state": state_after,
            "active": active}


def brute_general(x, weight, bias, conv_state, *, T, d_inner, qk_channels, head_dim, l2_eps,
                  x_dtype, state_dtype, layout="dense", slot_idx=None,
                  num_accept_tokens=None, cu_seqlens=None, parent=None, has_init=None,
                  do_l2=True, commit=True):
    """The general verify by paths instead of a rolling window.

    For token t of row i the input sequence is the row's starting window (the state
    columns a..a+D-2, or zeros for a row without an initial state) followed by x along
    the token's ancestor path ..., parent(parent(t)), parent(t), t (for a chain, every
    token before t).  The conv of token t is the dot product of the last D values of
    that sequence with the taps; its window is the last D-1 values.  Rows may be packed
    (``cu_seqlens``).  Windows are returned in the layout's shape with the sentinel
    0xFFFFFFFF where nothing is written; the state is the committed copy (chain only).
    """
    D = weight.shape[1]
    W1 = D - 1
    C = d_inner
    n_slots, _, state_len = conv_state.shape
    n_seq = len(cu_seqlens) - 1 if cu_seqlens is not None else x.shape[0]
    xv_all = values(x[..., :C], x_dtype)
    xb_all = x_bits_as_state(x[..., :C], x_dtype, state_dtype)
    wv = values(weight, x_dtype)
    bv = values(bias, x_dtype) if bias is not None else np.zeros(C)
    sv = values(conv_state, state_dtype)
    sb = bits(conv_state, state_dtype)
    pre = np.full((n_seq, T, C), np.nan)
    y = np.full((n_seq, T, C), np.nan)
    state_after = sb.copy()
    L = T + D - 2
    shape = {"dense": (n_slots, T, C, W1), "dedup": (n_slots, C, L),
             "dedup_t": (n_slots, L, C)}[layout]
    win = np.full(shape, 0xFFFFFFFF, np.uint64)
    active = []
    for i in range(n_seq):
        s = i if slot_idx is None else int(slot_idx[i])
        if s < 0:
            continue
        if cu_seqlens is not None:
            t0, Ti = int(cu_seqlens[i]), int(cu_seqlens[i + 1] - cu_seqlens[i])
            xv, xb = xv_all[t0:t0 + Ti], xb_all[t0:t0 + Ti]
        else:
            Ti = T
            xv, xb = xv_all[i], xb_all[i]
        if Ti == 0:
            continue
        a = 0 if num_accept_tokens is None else int(num_accept_tokens[i])
        init = True if has_init is None else bool(has_init[i])
        active.append((i, s))
        rv = sv[s, :, a:a + W1] if init else np.zeros((C, W1))
        rb = sb[s, :, a:a + W1] if init else np.zeros((C, W1), np.uint32)
        for t in range(Ti):
            path = [t]
            while True:
                q = path[-1]
                pq = (q - 1) if parent is None else int(parent[i, q])
                if pq < 0:
                    break
                path.append(pq)
            path = path[::-1]
            seqv = np.concatenate([rv, xv[path].T], axis=1)       # [C, W1 + len(path)]
            seqb = np.concatenate([rb, xb[path].T], axis=1)
            p = (seqv[:, -D:] * wv).sum(axis=1) + bv
            yy = silu(p)
            if qk_channels and do_l2:
                h = yy[:qk_channels].reshape(qk_channels // head_dim, head_dim)
                ss = (h * h).sum(axis=1, keepdims=True)
                yy[:qk_channels] = (h / np.sqrt(ss + np.float64(np.float32(l2_eps)))).reshape(-1)
            pre[i, t] = p
            y[i, t] = yy
            wnd = seqb[:, -W1:]
            if layout == "dense":
                win[s, t] = wnd
            elif layout == "dedup":
                win[s, :, t:t + W1] = wnd
            else:
                win[s, t:t + W1, :] = wnd.T
            if commit and t == Ti - 1:
                state_after[s, :, :W1] = wnd
    if x_dtype == "bf16":
        out = round_bf16_exact(np.where(np.isnan(y), 0.0, y))
    else:
        out = y.astype(np.float32)
    return {"pre": pre, "y": y, "out": out, "windows": win, "conv_state": state_after,
            "active": active}
