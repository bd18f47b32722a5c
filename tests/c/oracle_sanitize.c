/* Runs the CPU oracle (oracle/conv_verify_oracle.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer on problems of every kind, each buffer a heap block of
 * exactly its size, so that any read or write past a buffer is reported: the chain
 * verify in both layouts, the general loop (three layouts, packed rows with empty rows,
 * trees, zero-start rows, no windows, no commit), the restore, the separate L2, and
 * the refusals (bad slot, bad offset, bad parent), which must write nothing.  Values
 * are drawn from a fixed linear congruential sequence; what is checked here is memory
 * and arithmetic safety and the return codes (the values are pinned elsewhere).
 * Test code only: it includes nothing from the HIP library. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t n_seq, n_tok, d_inner, d_conv;
    int32_t qk_channels, head_dim;
    float l2_eps;
    int32_t x_bf16, state_bf16;
    int32_t n_slots, state_len;
    int64_t x_seq_stride, x_tok_stride;
    int64_t out_seq_stride, out_tok_stride;
    int64_t state_slot_stride;
    int32_t dedup;
    int64_t win_slot_stride;
} orc_problem;

typedef struct {
    int32_t layout;
    const int32_t *cu_seqlens;
    const int32_t *parent;
    int64_t parent_stride;
    const int32_t *has_init;
    int32_t do_l2;
    int32_t commit;
} orc_ext;

int orc_verify_general(const orc_problem *p, const orc_ext *e, const void *x, const void *weight,
                       const void *bias, void *conv_state, const int32_t *slot_idx,
                       const int32_t *num_accept_tokens, void *out, void *windows, float *pre_dbg,
                       double *y_dbg);
int orc_conv_verify(const orc_problem *p, const void *x, const void *weight, const void *bias,
                    void *conv_state, const int32_t *slot_idx, const int32_t *num_accept_tokens,
                    void *out, void *windows, float *pre_dbg, double *y_dbg);
int orc_restore(const orc_problem *p, int layout, void *conv_state, const void *windows,
                const int32_t *slot_idx, const int32_t *win_k);
int orc_l2norm(const orc_problem *p, int64_t n_rows, int64_t row_stride, void *x);

static uint32_t lcg = 12345u;
static uint32_t rnd(void) {
    lcg = lcg * 1664525u + 1013904223u;
    return lcg >> 8;
}

static int fails = 0;
static void expect(const char *what, int got, int want) {
    printf("%-56s %5d (want %d)%s\n", what, got, want, got == want ? "" : "  MISMATCH");
    if (got != want) fails = 1;
}

/* a heap block of n elements of eb bytes, filled with small random values */
static void *block(size_t n, int eb) {
    void *p = malloc(n ? n * (size_t)eb : 1);
    for (size_t i = 0; i < n; ++i) {
        float v = (float)((int)(rnd() % 33) - 16) / 8.0f;
        if (eb == 4) {
            memcpy((char *)p + 4 * i, &v, 4);
        } else {
            uint32_t u;
            memcpy(&u, &v, 4);
            uint16_t b = (uint16_t)(u >> 16);
            memcpy((char *)p + 2 * i, &b, 2);
        }
    }
    return p;
}

/* one problem: T tokens, D width, layout, dtype pair, options */
static void run(const char *name, int n, int T, int C, int D, int layout, int xbf, int sbf,
                int offsets, int packed, int tree, int zero_start, int no_windows) {
    const int xb = xbf ? 2 : 4, sb = sbf ? 2 : 4, W1 = D - 1;
    const int slots = n + 2, SL = W1 + (offsets ? T - 1 : 0);
    const int L = T + W1 - 1;
    orc_problem p;
    memset(&p, 0, sizeof p);
    p.n_seq = n; p.n_tok = T; p.d_inner = C; p.d_conv = D;
    p.qk_channels = C / 2; p.head_dim = C / 4; p.l2_eps = 1e-6f;
    p.x_bf16 = xbf; p.state_bf16 = sbf; p.n_slots = slots; p.state_len = SL;
    p.state_slot_stride = (int64_t)C * SL;
    p.win_slot_stride = layout == 0 ? (int64_t)T * C * W1 : (int64_t)C * L;
    int32_t *cu = NULL, *parent = NULL, *has_init = NULL;
    size_t tokens = (size_t)n * T;
    if (packed) {
        cu = malloc(sizeof(int32_t) * (n + 1));
        cu[0] = 0;
        for (int i = 0; i < n; ++i) cu[i + 1] = cu[i] + (int32_t)(rnd() % (T + 1));   /* 0..T */
        tokens = (size_t)cu[n];
        p.x_tok_stride = p.out_tok_stride = C;
    } else {
        p.x_seq_stride = p.out_seq_stride = (int64_t)T * C;
        p.x_tok_stride = p.out_tok_stride = C;
    }
    if (tree) {
        parent = malloc(sizeof(int32_t) * (size_t)n * T);
        for (int i = 0; i < n; ++i)
            for (int t = 0; t < T; ++t) parent[i * T + t] = t == 0 ? -1 : (int32_t)(rnd() % (t + 1)) - 1;
    }
    if (zero_start) {
        has_init = malloc(sizeof(int32_t) * n);
        for (int i = 0; i < n; ++i) has_init[i] = (int32_t)(rnd() & 1);
    }
    int32_t *slot = malloc(sizeof(int32_t) * n), *nat = malloc(sizeof(int32_t) * n);
    for (int i = 0; i < n; ++i) {
        slot[i] = (rnd() % 5 == 0) ? -1 : (int32_t)(slots - 1 - i);   /* distinct, in range */
        nat[i] = offsets ? (int32_t)(rnd() % T) : 0;
    }
    void *x = block(tokens * C, xb), *w = block((size_t)C * D, xb), *b = block(C, xb);
    void *state = block((size_t)slots * C * SL, sb), *out = block(tokens * C, xb);
    void *win = no_windows ? NULL : block((size_t)slots * p.win_slot_stride, sb);
    float *pre = packed ? NULL : malloc(sizeof(float) * (size_t)n * T * C);
    double *y = packed ? NULL : malloc(sizeof(double) * (size_t)n * T * C);
    orc_ext e = {layout, cu, parent, T, has_init, 1, tree ? 0 : 1};
    int rc = orc_verify_general(&p, &e, x, w, b, state, slot, nat, out, win, pre, y);
    expect(name, rc, 0);
    if (!packed && !tree && !zero_start && layout < 2 && !no_windows) {
        p.dedup = layout;
        expect("  the chain entry point", orc_conv_verify(&p, x, w, b, state, slot, nat, out, win, pre, y), 0);
    }
    if (!no_windows) {
        int32_t *k = malloc(sizeof(int32_t) * n);
        for (int i = 0; i < n; ++i) {
            const int Ti = packed ? cu[i + 1] - cu[i] : T;
            k[i] = Ti ? (int32_t)(rnd() % (Ti + 1)) - 1 : -1;
        }
        expect("  restore", orc_restore(&p, layout, state, win, slot, k), 0);
        free(k);
    }
    expect("  separate L2 over out", orc_l2norm(&p, (int64_t)tokens, C, out), 0);
    /* refusals: a slot past the pool, an offset past the row, a parent from the future */
    int32_t s0 = slot[0];
    slot[0] = slots;
    expect("  refused: slot past the pool", orc_verify_general(&p, &e, x, w, b, state, slot, nat, out, win, NULL, NULL), -1);
    slot[0] = s0 < 0 ? 0 : s0;
    int32_t a0 = nat[0];
    nat[0] = SL - W1 + 1;
    expect("  refused: offset past the row", orc_verify_general(&p, &e, x, w, b, state, slot, nat, out, win, NULL, NULL), -1);
    nat[0] = a0;
    if (tree && T > 1 && (!packed || cu[1] - cu[0] > 1)) {
        parent[1] = 1;
        expect("  refused: parent not earlier", orc_verify_general(&p, &e, x, w, b, state, slot, nat, out, win, NULL, NULL), -1);
    }
    free(x); free(w); free(b); free(state); free(out); free(win); free(pre); free(y);
    free(slot); free(nat); free(cu); free(parent); free(has_init);
}

int main(void) {
    char name[128];
    for (int layout = 0; layout < 3; ++layout)
        for (int pair = 0; pair < 3; ++pair)
            for (int D = 2; D <= 4; ++D) {
                const int xbf = pair != 0, sbf = pair == 1;
                snprintf(name, sizeof name, "verify layout %d, x %s, state %s, D %d", layout,
                         xbf ? "bf16" : "f32", sbf ? "bf16" : "f32", D);
                run(name, 5, 7, 64, D, layout, xbf, sbf, 1, 0, 0, 0, 0);
                snprintf(name, sizeof name, "  packed rows (empty ones too), layout %d", layout);
                run(name, 6, 9, 32, D, layout, xbf, sbf, 1, 1, 0, 0, 0);
            }
    for (int pair = 0; pair < 3; ++pair) {
        const int xbf = pair != 0, sbf = pair == 1;
        run("tree", 4, 12, 64, 4, 0, xbf, sbf, 1, 0, 1, 0, 0);
        run("tree, packed rows", 5, 12, 32, 3, 0, xbf, sbf, 1, 1, 1, 0, 0);
        run("zero-start rows, no windows (the prefill form)", 4, 40, 32, 4, 0, xbf, sbf, 0, 1, 0, 1, 1);
        run("T 1", 3, 1, 16, 4, 1, xbf, sbf, 0, 0, 0, 0, 0);
        run("T 32, dense", 3, 32, 16, 4, 0, xbf, sbf, 1, 0, 0, 0, 0);
    }
    printf(fails ? "FAILED\n" : "ALL OK\n");
    return fails;
}
