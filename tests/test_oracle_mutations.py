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
    ("l2_on_v_too", "for (int h0 = 0; h0 < p->qk_channels; h0 += p->head_dim)",
     "for (int h0 = 0; h0 + p->head_dim <= p->d_inner; h0 += p->head_dim)"),
    ("l2_max_eps", "double scale = 1.0 / sqrt(ss + (double)p->l2_eps);",
     "double scale = 1.0 / fmax(sqrt(ss), (double)p->l2_eps);"),
    ("l2_half_head", "for (int c = h0; c < h0 + p->head_dim; ++c)\n                        ss +=",
     "for (int c = h0; c < h0 + p->head_dim / 2; ++c)\n                        ss +="),
    ("l2_no_eps", "sqrt(ss + (double)p->l2_eps)", "sqrt(ss)"),
    ("dense_window_reversed", "((int64_t)t * C + c) * W1 + j;",
     "((int64_t)t * C + c) * W1 + (W1 - 1 - j);"),
    ("dedup_row_shift", "(int64_t)c * (T + D - 2) + t + j;",
     "(int64_t)c * (T + D - 2) + (t + j + 1) % (T + D - 2);"),
    ("commit_at_offset", "state_put(p, conv_state, st_base + (int64_t)c * p->state_len + j,",
     "state_put(p, conv_state, st_base + (int64_t)c * p->state_len + a + j,"),
    ("window_not_shifted", "wc[j] = wc[j + 1];", "wc[j] = wc[j];"),
    ("ignore_slot", "        int s = slot_idx ? slot_idx[i] : i;\n        if (s < 0)\n            continue;               /* padded",
     "        int s = slot_idx ? (slot_idx[i] < 0 ? -1 : i) : i;\n        if (s < 0)\n            continue;               /* padded"),
    ("x_token_stride_ignored", "(int64_t)t * p->x_tok_stride;", "(int64_t)t * p->d_inner;"),
    ("widen_bf16_wrong", "p->state_bf16 ? (uint32_t)b : ((uint32_t)b << 16);",
     "p->state_bf16 ? (uint32_t)b : ((uint32_t)b << 15);"),
    ("round_ties_away", "double r = nearbyint(q);", "double r = round(q);"),
    ("round_truncate", "double r = nearbyint(q);", "double r = trunc(q);"),
    ("rounded_before_l2", "y[c] = pd / (1.0 + exp(-pd));",
     "y[c] = (double)bf16_to_float(orc_round_bf16(pd / (1.0 + exp(-pd))));"),
    ("f32_out_via_bf16", "((float *)out)[o_base + c] = orc_round_f32(y[c]);",
     "((float *)out)[o_base + c] = bf16_to_float(orc_round_bf16(y[c]));"),
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
