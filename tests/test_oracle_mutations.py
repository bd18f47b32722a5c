"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of the oracle's C source with one plausible mistake (a dropped
term, a wrong sign or index, a transposed operand, a wrong convention), built with
the host compiler into a temporary library.  The pins of ``oracle_pins.py`` are run
against it; at least one must fail.  Nothing here touches a GPU.
"""

import os

import pytest

import oracle
import oracle_pins
from oracle import build as obuild

SRC = open(obuild.SRC).read()

MUTANTS = [
    ("ignore_accept_offset",
     "st_base + (int64_t)c * p->state_len + a + j)", "st_base + (int64_t)c * p->state_len + j)"),
    ("drop_bias", "float acc = bias ? x_val(p, bias, c) : 0.0f;", "float acc = 0.0f;"),
    ("reversed_taps", "x_val(p, weight, (int64_t)c * D + w)",
     "x_val(p, weight, (int64_t)c * D + (D - 1 - w))"),
    ("mul_add_not_fma", "acc = fmaf(x_val(p, weight, (int64_t)c * D + w), v, acc);",
     "acc = (float)(x_val(p, weight, (int64_t)c * D + w) * v) + acc; acc = acc;"),
    ("silu_sign", "y[c] = pd / (1.0 + exp(-pd));", "y[c] = pd / (1.0 + exp(pd));"),
    ("l2_on_v_too", "e->do_l2) {\n                for (int h0 = 0; h0 < p->qk_channels; h0 += p->head_dim)",
     "e->do_l2) {\n                for (int h0 = 0; h0 + p->head_dim <= p->d_inner; h0 += p->head_dim)"),
    ("l2_max_eps", "double scale = 1.0 / sqrt(ss + (double)p->l2_eps);\n                    for (int c = h0; c < h0 + p->head_dim; ++c)\n                        y[c] *= scale;",
     "double scale = 1.0 / fmax(sqrt(ss), (double)p->l2_eps);\n                    for (int c = h0; c < h0 + p->head_dim; ++c)\n                        y[c] *= scale;"),
    ("l2_half_head", "for (int c = h0; c < h0 + p->head_dim; ++c)\n                        ss +=",
     "for (int c = h0; c < h0 + p->head_dim / 2; ++c)\n                        ss +="),
    ("l2_no_eps", "sqrt(ss + (double)p->l2_eps);\n                    for (int c = h0; c < h0 + p->head_dim; ++c)\n                        y[c] *= scale;",
     "sqrt(ss);\n                    for (int c = h0; c < h0 + p->head_dim; ++c)\n                        y[c] *= scale;"),
    ("dense_window_reversed", "((int64_t)t * C + c) * W1 + j;",
     "((int64_t)t * C + c) * W1 + (W1 - 1 - j);"),
    ("dedup_row_shift", "return base + (int64_t)c * L + t + j;",
     "return base + (int64_t)c * L + (t + j + 1) % L;"),
    ("commit_at_offset", "state_put(p, conv_state, st_base + (int64_t)c * p->state_len + j,\n                          last[",
     "state_put(p, conv_state, st_base + (int64_t)c * p->state_len + a + j,\n                          last["),
    ("window_not_shifted", "wc[j] = pc[j + 1];", "wc[j] = pc[j];"),
    ("ignore_slot", "        int s = slot_idx ? slot_idx[i] : i;\n        if (s < 0)\n            continue;               /* padded",
     "        int s = slot_idx ? (slot_idx[i] < 0 ? -1 : i) : i;\n        if (s < 0)\n            continue;               /* padded"),
    ("x_token_stride_ignored", "tok * p->x_tok_stride;", "tok * p->d_inner;"),
    ("widen_bf16_wrong", "p->state_bf16 ? (uint32_t)b : ((uint32_t)b << 16);",
     "p->state_bf16 ? (uint32_t)b : ((uint32_t)b << 15);"),
    ("round_ties_away", "double r = nearbyint(q);", "double r = round(q);"),
    ("round_truncate", "double r = nearbyint(q);", "double r = trunc(q);"),
    ("rounded_before_l2", "y[c] = pd / (1.0 + exp(-pd));",
     "y[c] = (double)bf16_to_float(orc_round_bf16(pd / (1.0 + exp(-pd))));"),
    ("f32_out_via_bf16", "((float *)out)[o_base + c] = orc_round_f32(y[c]);",
     "((float *)out)[o_base + c] = bf16_to_float(orc_round_bf16(y[c]));"),
    # the general loop: packed rows, trees, layouts, zero starts; restore; separate L2
    ("rows_t_as_rows", "return base + (int64_t)(t + j) * C + c;",
     "return base + (int64_t)c * L + t + j;"),
    ("rows_t_transposed_index", "return base + (int64_t)(t + j) * C + c;",
     "return base + (int64_t)(t + j) * C + (C - 1 - c);"),
    # (mutants stay in bounds: a planted mistake must not corrupt the test process)
    ("packed_tokens_reversed", "const int64_t tok = e->cu_seqlens ? (int64_t)e->cu_seqlens[i] + t : t;",
     "const int64_t tok = e->cu_seqlens ? (int64_t)e->cu_seqlens[i] + (Ti - 1 - t) : t;"),
    ("packed_last_token_dropped", "int Ti = e->cu_seqlens ? e->cu_seqlens[i + 1] - e->cu_seqlens[i] : T;\n        if (Ti == 0)",
     "int Ti = e->cu_seqlens ? e->cu_seqlens[i + 1] - e->cu_seqlens[i] - 1 : T;\n        if (Ti <= 0)"),
    ("tree_parent_ignored", "int pt = e->parent ? e->parent[(int64_t)i * e->parent_stride + t] : t - 1;",
     "int pt = t - 1;"),
    ("tree_parent_off_by_one", "int pt = e->parent ? e->parent[(int64_t)i * e->parent_stride + t] : t - 1;",
     "int pt = e->parent ? e->parent[(int64_t)i * e->parent_stride + t] - 1 : t - 1;"),
    ("commit_ignores_flag", "for (int c = 0; e->commit && c < C; ++c)", "for (int c = 0; c < C; ++c)"),
    ("zero_start_ignored", "init ? state_get(", "1 ? state_get("),
    ("restore_wrong_window", "state_get(p, windows, win_index(p, layout, s, k, c, j))",
     "state_get(p, windows, win_index(p, layout, s, k > 0 ? k - 1 : k + 1, c, j))"),
    ("restore_at_offset_one", "state_put(p, conv_state, st_base + (int64_t)c * p->state_len + j,\n                          state_get(",
     "state_put(p, conv_state, st_base + (int64_t)c * p->state_len + (j + 1) % (p->d_conv - 1),\n                          state_get("),
    ("l2norm_no_eps", "double scale = 1.0 / sqrt(ss + (double)p->l2_eps);\n            for",
     "double scale = 1.0 / sqrt(ss);\n            for"),
    ("l2norm_half_head", "for (int c = h0; c < h0 + p->head_dim; ++c) {\n                double v = (double)x_val(p, x, base + c);\n                ss",
     "for (int c = h0; c < h0 + p->head_dim / 2; ++c) {\n                double v = (double)x_val(p, x, base + c);\n                ss"),
    ("l2norm_on_v", "for (int h0 = 0; h0 < p->qk_channels; h0 += p->head_dim) {\n            double ss = 0.0;\n            for (int c = h0; c < h0 + p->head_dim; ++c) {",
     "for (int h0 = 0; h0 + p->head_dim <= p->d_inner; h0 += p->head_dim) {\n            double ss = 0.0;\n            for (int c = h0; c < h0 + p->head_dim; ++c) {"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    assert SRC.count(old) == 1, f"mutation anchor for {name} not unique in the oracle source"
    src = tmp_path / f"mut_{name}.c"
    src.write_text(SRC.replace(old, new))
    lib_path = obuild.build(str(src), str(tmp_path / f"mut_{name}.so"), quiet=True)
    lib = oracle.load(lib_path)
    failures = []
    for pin in oracle_pins.PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError) as e:
            failures.append(f"{pin.__name__}: {e}")
    assert failures, f"mutant {name} passed every pin"
    os.remove(lib_path)
