/*
 * CPU oracle for the batched speculative-verify causal conv1d update.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the HIP
 * library is checked against.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the product path never does.  It
 * shares no header, helper or table with the HIP library.
 *
 * What it computes (one row i of the batch, skipped entirely when its slot is -1):
 *
 *   The per-token path that the fused verify launch replaces: for each draft
 *   position t = 0..T-1, one causal conv1d update of width D over the rolling
 *   window, SiLU, per-head L2 on the q|k channels, then a copy of the new window
 *   into the rollback buffer.  [Atlas docs, fn gdn_verify_fused_conv_kn_batched:
 *   the fused call covers every draft position in one launch and takes the place
 *   of K per-token conv-update-with-L2 calls, each followed by a window copy; the
 *   same function notes that the sequences' windows do not depend on each other.]
 *
 *   - window: D-1 columns of conv_state, read starting at column a =
 *     num_accept_tokens[i] (0 when absent).  [sglang PR 46184, "Modifications"
 *     (test coverage: a num_accept_tokens state offset) and "Accuracy Tests"
 *     (a tile that ignores num_accept_tokens fails the accept-offset cases).]
 *   - conv:   pre = bias[c] + sum_{w<D} W[c,w] * v[t+w], v = [window, x_0 .. x_{T-1}],
 *     W[c,D-1] multiplying the newest input; fp32, one correctly rounded fused
 *     multiply-add per tap in tap order.  [Atlas docs, same function: the fused
 *     kernel keeps the per-token path's numerics and accumulates in the same
 *     order; the fp32 accumulation is the stated precision of the method.]
 *   - SiLU:   y = pre / (1 + exp(-pre)), in fp64.  [Atlas glm5next_kda/mod.rs, module
 *     doc: the conv is followed by SiLU, then an L2 over q and k alone.]
 *   - L2:     for channels c < qk_channels, head h = c / head_dim:
 *     y <- y / sqrt(sum_{head} y^2 + l2_eps), in fp64.  V channels are untouched.
 *     [Atlas glm5next_kda/mod.rs, Glm5NextKdaConfig::l2_eps: the scale is
 *     1/sqrt(sum + eps) as in FLA, with no max(norm, eps) clamp; qk_channels() is
 *     2 * qkv_dim; the V channels are left as they are.]
 *   - out[i,t,c] = y rounded once to the output dtype (nearest, ties to even).
 *   - the window shifts by one: w <- (w[1..], x_t) in the state dtype.
 *   - the new window is copied into the rollback buffer:
 *       dense: win[s, t, c, j]   = w[j], j < D-1    ([T, dim, K-1] per slot)
 *       dedup: win[s, c, t + j]  = w[j], j < D-1    (one [dim, T+K-2] row per slot;
 *              overlapping columns are rewritten with the same value)
 *     [sglang PR 46184, "Motivation" (MambaPool's deduplicated [dim, T+K-2] row viewed
 *     as an overlapping [T, dim, K-1] window) and "Scope" (dense windows).]
 *   After the last token conv_state[s, c, 0..D-2] = w, the committed window; columns
 *   >= D-1 are left alone.  [Atlas docs, same function: after the call conv_state
 *   holds the window committed after the last draft position.]
 *
 * Readings where the pages are silent (each is also listed in the design notes):
 * the offset a is the value itself and the committed window goes to columns
 * 0..D-2; bias is added before SiLU; rounding to the output dtype happens once,
 * after L2; an (x=f32, state=bf16) pair is refused; copies move bit patterns.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_seq, n_tok, d_inner, d_conv;
    int32_t qk_channels, head_dim;
    float   l2_eps;
    int32_t x_bf16;        /* 1: x, weight, bias and out hold bf16 bit patterns; 0: f32 */
    int32_t state_bf16;    /* 1: conv_state and windows hold bf16; 0: f32 */
    int32_t n_slots, state_len;
    int64_t x_seq_stride, x_tok_stride;       /* elements */
    int64_t out_seq_stride, out_tok_stride;   /* elements */
    int64_t state_slot_stride;                /* elements; channel stride is state_len */
    int32_t dedup;         /* 0: dense windows, 1: deduplicated rows */
    int64_t win_slot_stride;                  /* elements */
} orc_problem;

enum { ORC_OK = 0, ORC_BAD = -1, ORC_NOMEM = -2 };

/* ---- scalar formats ---------------------------------------------------------------- */

static float bf16_to_float(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t float_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float bits_float(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round a double to the nearest bf16, ties to even, in one step (no detour through
 * float, which would round twice).  bf16 keeps 8 significant bits and float's
 * exponent range, so its quantum is 2^(e-7) for |y| in [2^e, 2^(e+1)), and 2^-133
 * below 2^-126 (subnormals). */
uint16_t orc_round_bf16(double y) {
    if (isnan(y))
        return (uint16_t)((signbit(y) ? 0x8000u : 0u) | 0x7FC0u);
    uint16_t sign = signbit(y) ? 0x8000u : 0u;
    double ay = fabs(y);
    if (isinf(ay))
        return sign | 0x7F80u;
    int e2;
    frexp(ay, &e2);                 /* ay = m * 2^e2, m in [0.5, 1)  => floor(log2 ay) = e2-1 */
    int qexp = (e2 - 1) - 7;
    if (qexp < -133)
        qexp = -133;
    double q = ldexp(ay, -qexp);    /* exact */
    double r = nearbyint(q);        /* default rounding mode: nearest, ties to even */
    double rv = ldexp(r, qexp);
    if (rv >= 0x1p128)
        return sign | 0x7F80u;
    float f = (float)rv;            /* exact: rv is a bf16 value */
    return (uint16_t)(sign | (float_bits(f) >> 16));
}

float orc_round_f32(double y) { return (float)y; }

/* ---- the per-token loop -------------------------------------------------------------- */

static int check_problem(const orc_problem *p) {
    if (p->n_seq < 0 || p->n_tok < 1 || p->d_inner < 0 || p->d_conv < 2)
        return ORC_BAD;
    if (p->qk_channels < 0 || p->qk_channels > p->d_inner)
        return ORC_BAD;
    if (p->qk_channels > 0 && (p->head_dim <= 0 || p->qk_channels % p->head_dim != 0))
        return ORC_BAD;
    if (p->state_len < p->d_conv - 1 || p->n_slots < 0)
        return ORC_BAD;
    if (p->x_bf16 == 0 && p->state_bf16 == 1)
        return ORC_BAD;             /* (f32 x, bf16 state) is not a supported pair */
    return ORC_OK;
}

/* x element as float, and as a bit pattern in the state dtype (exact widening). */
static float x_val(const orc_problem *p, const void *base, int64_t idx) {
    if (p->x_bf16)
        return bf16_to_float(((const uint16_t *)base)[idx]);
    return ((const float *)base)[idx];
}

static uint32_t x_as_state_bits(const orc_problem *p, const void *base, int64_t idx) {
    if (p->x_bf16) {
        uint16_t b = ((const uint16_t *)base)[idx];
        return p->state_bf16 ? (uint32_t)b : ((uint32_t)b << 16);
    }
    return float_bits(((const float *)base)[idx]);
}

static uint32_t state_get(const orc_problem *p, const void *base, int64_t idx) {
    return p->state_bf16 ? (uint32_t)((const uint16_t *)base)[idx]
                         : float_bits(((const float *)base)[idx]);
}

static void state_put(const orc_problem *p, void *base, int64_t idx, uint32_t bits) {
    if (p->state_bf16)
        ((uint16_t *)base)[idx] = (uint16_t)bits;
    else
        ((float *)base)[idx] = bits_float(bits);
}

static float state_bits_val(const orc_problem *p, uint32_t bits) {
    return p->state_bf16 ? bf16_to_float((uint16_t)bits) : bits_float(bits);
}

/*
 * Window layouts of the rollback buffer (T = p->n_tok, the buffer's token count):
 *   ORC_DENSE  win[s, t, c, j]                       [T, dim, K-1] per slot
 *   ORC_ROWS   win[s, c, t + j], row length T+K-2    one [dim, T+K-2] row per slot
 *   ORC_ROWS_T win[s, t + j, c]                      the same row stored time-major,
 *                                                    [T+K-2, dim] per slot
 * ORC_ROWS is MambaPool's deduplicated row; ORC_ROWS_T is its axis-0 layout seen
 * transposed: in both, one step along the view moves by the same stride as one
 * element along a window.  [sglang PR 46184, "Modifications": the tile store serves
 * every layout with that property, and its tests include the pool's window layout
 * along axis 0, transposed.]
 */
enum { ORC_DENSE = 0, ORC_ROWS = 1, ORC_ROWS_T = 2 };

static int64_t win_index(const orc_problem *p, int layout, int s, int t, int c, int j) {
    const int64_t C = p->d_inner, W1 = p->d_conv - 1, L = p->n_tok + p->d_conv - 2;
    const int64_t base = (int64_t)s * p->win_slot_stride;
    if (layout == ORC_DENSE)
        return base + ((int64_t)t * C + c) * W1 + j;
    if (layout == ORC_ROWS)
        return base + (int64_t)c * L + t + j;
    return base + (int64_t)(t + j) * C + c;
}

/*
 * The general per-token loop.  Beyond the plain batched verify it takes:
 *
 *   cu_seqlens [n_seq+1] or NULL: packed rows.  Row i holds T_i = cu[i+1]-cu[i] <= T
 *     tokens, token t at x/out index (cu[i] + t) * tok_stride (the seq strides are
 *     unused).  A row with T_i = 0 writes nothing.  [sglang PR 46184, "Related
 *     upstream work": packed variable-length rows, ragged tokens.]
 *   parent [n_seq, parent_stride] or NULL: tree verify.  Token t's window continues
 *     the window of token parent[i,t] (-1: the row's starting window) instead of
 *     token t-1's; the chain is parent[i,t] = t-1.  Tree windows are dense only and
 *     the call commits nothing to conv_state: the accepted path is known only after
 *     verification, and the restore below writes it.  [sglang PR 46184, "Scope" (tree
 *     verify keeps dense windows) and "Modifications" (the tile path is not used with
 *     a tree mask).]
 *   has_init [n_seq] or NULL: 0 starts row i from a zero window instead of its state
 *     (a prompt with no earlier state).
 *   do_l2 = 0 skips the per-head L2; windows = NULL writes no rollback windows; commit
 *     = 0 leaves conv_state alone.
 *
 * The arithmetic of each token is the plain verify's: conv + bias in fp32 FMAs in
 * tap order, SiLU and L2 in fp64, one rounding to the output dtype.
 */
typedef struct {
    int32_t layout;
    const int32_t *cu_seqlens;
    const int32_t *parent;
    int64_t parent_stride;
    const int32_t *has_init;
    int32_t do_l2;
    int32_t commit;
} orc_ext;

int orc_verify_general(const orc_problem *p, const orc_ext *e, const void *x,
                       const void *weight, const void *bias, void *conv_state,
                       const int32_t *slot_idx, const int32_t *num_accept_tokens,
                       void *out, void *windows, float *pre_dbg, double *y_dbg) {
    if (check_problem(p) != ORC_OK)
        return ORC_BAD;
    if (e->layout < ORC_DENSE || e->layout > ORC_ROWS_T)
        return ORC_BAD;
    if (e->parent && (e->layout != ORC_DENSE || e->commit))
        return ORC_BAD;
    const int D = p->d_conv, W1 = p->d_conv - 1, T = p->n_tok, C = p->d_inner;

    for (int i = 0; i < p->n_seq; ++i) {
        int s = slot_idx ? slot_idx[i] : i;
        int a = num_accept_tokens ? num_accept_tokens[i] : 0;
        if (s < 0)
            continue;
        if (s >= p->n_slots || a < 0 || a > p->state_len - W1)
            return ORC_BAD;
        int Ti = e->cu_seqlens ? e->cu_seqlens[i + 1] - e->cu_seqlens[i] : T;
        if (Ti < 0 || Ti > T)
            return ORC_BAD;
        for (int t = 0; e->parent && t < Ti; ++t) {
            int pt = e->parent[(int64_t)i * e->parent_stride + t];
            if (pt < -1 || pt >= t)
                return ORC_BAD;
        }
    }

    /* hist[t] = the window after token t; root = the row's starting window */
    const size_t cw = (size_t)(C > 0 ? C : 1) * (size_t)W1;
    uint32_t *root = malloc(sizeof(uint32_t) * cw);
    uint32_t *hist = malloc(sizeof(uint32_t) * cw * (size_t)T);
    double *y = malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    if (!root || !hist || !y) {
        free(root);
        free(hist);
        free(y);
        return ORC_NOMEM;
    }

    for (int i = 0; i < p->n_seq; ++i) {
        int s = slot_idx ? slot_idx[i] : i;
        if (s < 0)
            continue;               /* padded row: no write anywhere */
        int a = num_accept_tokens ? num_accept_tokens[i] : 0;
        int Ti = e->cu_seqlens ? e->cu_seqlens[i + 1] - e->cu_seqlens[i] : T;
        if (Ti == 0)
            continue;
        const int64_t st_base = (int64_t)s * p->state_slot_stride;
        const int init = e->has_init ? e->has_init[i] != 0 : 1;

        for (int c = 0; c < C; ++c)
            for (int j = 0; j < W1; ++j)
                root[(int64_t)c * W1 + j] =
                    init ? state_get(p, conv_state, st_base + (int64_t)c * p->state_len + a + j)
                         : 0u;

        for (int t = 0; t < Ti; ++t) {
            int pt = e->parent ? e->parent[(int64_t)i * e->parent_stride + t] : t - 1;
            const uint32_t *pw = pt < 0 ? root : hist + (size_t)pt * cw;
            uint32_t *nw = hist + (size_t)t * cw;
            const int64_t tok = e->cu_seqlens ? (int64_t)e->cu_seqlens[i] + t : t;
            const int64_t x_base = (e->cu_seqlens ? 0 : (int64_t)i * p->x_seq_stride) +
                                   tok * p->x_tok_stride;

            /* conv + bias, then SiLU, channel by channel */
            for (int c = 0; c < C; ++c) {
                float acc = bias ? x_val(p, bias, c) : 0.0f;
                for (int w = 0; w < D; ++w) {
                    float v = (w < W1) ? state_bits_val(p, pw[(int64_t)c * W1 + w])
                                       : x_val(p, x, x_base + c);
                    acc = fmaf(x_val(p, weight, (int64_t)c * D + w), v, acc);
                }
                if (pre_dbg)
                    pre_dbg[((int64_t)i * T + t) * C + c] = acc;
                double pd = (double)acc;
                y[c] = pd / (1.0 + exp(-pd));
            }

            /* per-head L2 over the q|k channels only */
            if (p->qk_channels > 0 && e->do_l2) {
                for (int h0 = 0; h0 < p->qk_channels; h0 += p->head_dim) {
                    double ss = 0.0;
                    for (int c = h0; c < h0 + p->head_dim; ++c)
                        ss += y[c] * y[c];
                    double scale = 1.0 / sqrt(ss + (double)p->l2_eps);
                    for (int c = h0; c < h0 + p->head_dim; ++c)
                        y[c] *= scale;
                }
            }

            const int64_t o_base = (e->cu_seqlens ? 0 : (int64_t)i * p->out_seq_stride) +
                                   tok * p->out_tok_stride;
            for (int c = 0; c < C; ++c) {
                if (y_dbg)
                    y_dbg[((int64_t)i * T + t) * C + c] = y[c];
                if (p->x_bf16)
                    ((uint16_t *)out)[o_base + c] = orc_round_bf16(y[c]);
                else
                    ((float *)out)[o_base + c] = orc_round_f32(y[c]);
            }

            /* the new window: the parent's shifted by one, x_t appended; then its copy
             * into the rollback buffer */
            for (int c = 0; c < C; ++c) {
                const uint32_t *pc = pw + (int64_t)c * W1;
                uint32_t *wc = nw + (int64_t)c * W1;
                for (int j = 0; j + 1 < W1; ++j)
                    wc[j] = pc[j + 1];
                wc[W1 - 1] = x_as_state_bits(p, x, x_base + c);
                for (int j = 0; windows && j < W1; ++j)
                    state_put(p, windows, win_index(p, e->layout, s, t, c, j), wc[j]);
            }
        }

        const uint32_t *last = hist + (size_t)(Ti - 1) * cw;
        for (int c = 0; e->commit && c < C; ++c)
            for (int j = 0; j < W1; ++j)
                state_put(p, conv_state, st_base + (int64_t)c * p->state_len + j,
                          last[(int64_t)c * W1 + j]);
    }
    free(root);
    free(hist);
    free(y);
    return ORC_OK;
}

/*
 * The plain batched verify: every row T tokens, chain windows in the dense or the
 * deduplicated-row layout, L2 on, the committed window written to conv_state.
 *
 * conv_state is updated in place; out and windows are written for active rows only.
 * pre_dbg (fp32) and y_dbg (fp64, after L2, before rounding), if not NULL, receive
 * [n_seq, T, d_inner] contiguous copies of the intermediate values for the
 * self-tests.  Returns ORC_BAD if the problem is malformed or a row's slot or offset
 * is out of range (nothing is written then), ORC_NOMEM on allocation failure.
 */
int orc_conv_verify(const orc_problem *p, const void *x, const void *weight,
                    const void *bias, void *conv_state, const int32_t *slot_idx,
                    const int32_t *num_accept_tokens, void *out, void *windows,
                    float *pre_dbg, double *y_dbg) {
    orc_ext e = {p->dedup ? ORC_ROWS : ORC_DENSE, NULL, NULL, 0, NULL, 1, 1};
    return orc_verify_general(p, &e, x, weight, bias, conv_state, slot_idx,
                              num_accept_tokens, out, windows, pre_dbg, y_dbg);
}

/*
 * Accepted-prefix restore: conv_state[s, c, 0..K-2] = window k of slot s, k =
 * win_index[i] (chain verify: the number of accepted tokens minus one; tree verify:
 * the position of the last accepted token).  k = -1 restores nothing for that row,
 * as does slot -1.  [sglang PR 46184, "Motivation": the window lets the accepted
 * prefix's conv state be restored after verify; Atlas glm5next_kda/mod.rs, decode_k:
 * the snapshot after row t is what a partial accept rewinds to.]
 */
int orc_restore(const orc_problem *p, int layout, void *conv_state, const void *windows,
                const int32_t *slot_idx, const int32_t *win_k) {
    if (check_problem(p) != ORC_OK || layout < ORC_DENSE || layout > ORC_ROWS_T)
        return ORC_BAD;
    const int W1 = p->d_conv - 1;
    for (int i = 0; i < p->n_seq; ++i) {
        int s = slot_idx ? slot_idx[i] : i;
        int k = win_k[i];
        if (s < 0 || k < 0)
            continue;
        if (s >= p->n_slots || k >= p->n_tok)
            return ORC_BAD;
    }
    for (int i = 0; i < p->n_seq; ++i) {
        int s = slot_idx ? slot_idx[i] : i;
        int k = win_k[i];
        if (s < 0 || k < 0)
            continue;
        const int64_t st_base = (int64_t)s * p->state_slot_stride;
        for (int c = 0; c < p->d_inner; ++c)
            for (int j = 0; j < W1; ++j)
                state_put(p, conv_state, st_base + (int64_t)c * p->state_len + j,
                          state_get(p, windows, win_index(p, layout, s, k, c, j)));
    }
    return ORC_OK;
}

/*
 * Separate per-head L2 over the q|k channels, in place, on rows of x (the prefill
 * conv's output): y <- y / sqrt(sum_head y^2 + eps) in fp64, rounded once to x's
 * dtype.  V channels are untouched.  [Atlas glm5next_kda/mod.rs, module doc: the
 * decode conv has the L2 fused in, the prefill conv does not and is followed by its
 * own L2 launch over q|k; the prefill body computes conv and SiLU only.]
 */
int orc_l2norm(const orc_problem *p, int64_t n_rows, int64_t row_stride, void *x) {
    if (p->qk_channels < 0 || p->qk_channels > p->d_inner ||
        (p->qk_channels > 0 && (p->head_dim <= 0 || p->qk_channels % p->head_dim)))
        return ORC_BAD;
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t base = r * row_stride;
        for (int h0 = 0; h0 < p->qk_channels; h0 += p->head_dim) {
            double ss = 0.0;
            for (int c = h0; c < h0 + p->head_dim; ++c) {
                double v = (double)x_val(p, x, base + c);
                ss += v * v;
            }
            double scale = 1.0 / sqrt(ss + (double)p->l2_eps);
            for (int c = h0; c < h0 + p->head_dim; ++c) {
                double v = (double)x_val(p, x, base + c) * scale;
                if (p->x_bf16)
                    ((uint16_t *)x)[base + c] = orc_round_bf16(v);
                else
                    ((float *)x)[base + c] = orc_round_f32(v);
            }
        }
    }
    return ORC_OK;
}
