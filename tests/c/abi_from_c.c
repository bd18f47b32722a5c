/* Uses the library through include/conv_verify.h from plain C (no GPU needed): ABI
 * version, launch geometry of a shape, refusals with their codes and detail strings,
 * and a call that validates its arguments before any launch.  Prints one line per check
 * and exits non-zero on the first mismatch. */
#include <stdio.h>
#include <string.h>

#include "conv_verify.h"

static int fails = 0;

static void expect(const char *what, int got, int want) {
    printf("%-40s %6d (want %d)%s\n", what, got, want, got == want ? "" : "  <-- MISMATCH");
    if (got != want) fails = 1;
}

static cv_shape_t headline(void) {
    cv_shape_t s;
    memset(&s, 0, sizeof s);
    s.n_seq = 128; s.T = 8; s.d_inner = 10240; s.d_conv = 4;
    s.qk_channels = 4096; s.head_dim = 128; s.l2_eps = 1e-6f;
    s.x_dtype = CV_BF16; s.state_dtype = CV_BF16; s.n_slots = 128; s.state_len = 3;
    s.x_seq_stride = 8 * 10240; s.x_tok_stride = 10240;
    s.out_seq_stride = 8 * 10240; s.out_tok_stride = 10240;
    s.state_slot_stride = 10240 * 3; s.win_slot_stride = 10240 * 10;
    return s;
}

int main(void) {
    expect("abi version", conv_verify_abi_version(), CONV_VERIFY_ABI_VERSION);
    cv_shape_t s = headline();
    cv_launch_info_t info;
    expect("describe rows", conv_verify_describe(CV_WIN_ROWS, &s, &info), CV_OK);
    expect("  workgroups", (int)info.workgroups, 128 * 40);
    expect("  threads", info.threads, 64);
    expect("  channels per wavefront", info.channels_per_wave, 256);
    expect("  token bucket", info.token_bucket, 8);
    expect("  head lanes", info.head_lanes, 32);
    expect("  token chunks", info.token_chunks, 1);
    expect("  no slot-first wait (one generation)", (info.flags & CV_LAUNCH_SLOT_FIRST) != 0, 0);
    expect("describe time-major rows", conv_verify_describe(CV_WIN_ROWS_T, &s, &info), CV_OK);
    expect("describe dense (rows-sized slots)", conv_verify_describe(CV_WIN_DENSE, &s, &info), CV_EINVAL);
    if (!strlen(conv_verify_last_error())) { puts("missing error detail"); fails = 1; }
    cv_shape_t bad = s;
    bad.T = 33;
    expect("T = 33", conv_verify_describe(CV_WIN_ROWS, &bad, &info), CV_ENOTSUP);
    bad = s;
    bad.head_dim = 132; bad.qk_channels = 396;   /* no block of whole heads is 16-byte sized */
    expect("head_dim 132", conv_verify_describe(CV_WIN_ROWS, &bad, &info), CV_ENOTSUP);
    bad = s;
    bad.head_dim = 96; bad.qk_channels = 960;    /* blocks of 2 heads, then 256-channel blocks */
    expect("head_dim 96", conv_verify_describe(CV_WIN_ROWS, &bad, &info), CV_OK);
    expect("  q|k in blocks of whole heads", (info.flags & CV_LAUNCH_HEAD_BLOCKS) != 0, 1);
    expect("  5 + 37 channel blocks", info.channel_blocks, 5 + 37);
    /* conv_state stored time-major: columns of >= d_inner elements, no state region in LDS */
    bad = s;
    bad.state_col_stride = 10240 - 8;
    expect("state columns overlap", conv_verify_describe(CV_WIN_ROWS, &bad, &info), CV_EINVAL);
    cv_launch_info_t cm, tm;
    bad = s;
    bad.state_len = 18; bad.state_slot_stride = 10240 * 18;
    expect("describe rows, 18-column channel-major state", conv_verify_describe(CV_WIN_ROWS, &bad, &cm), CV_OK);
    bad.state_col_stride = 10240;
    expect("describe rows, time-major state", conv_verify_describe(CV_WIN_ROWS, &bad, &tm), CV_OK);
    expect("  time-major state takes less LDS", tm.lds_bytes < cm.lds_bytes, 1);
    /* argument checks run before any HIP call: a NULL x is refused, nothing launched */
    expect("update with NULL x", conv_verify_update(&s, CV_WIN_ROWS, NULL, (void *)0x10000, NULL,
                                                    (void *)0x10000, NULL, NULL, NULL,
                                                    (void *)0x10000, (void *)0x10000, NULL),
           CV_EINVAL);
    expect("empty batch", conv_verify_update_dedup(&(cv_shape_t){.n_seq = 0, .T = 1, .d_inner = 8,
                                                   .d_conv = 4, .x_dtype = CV_BF16,
                                                   .state_dtype = CV_BF16, .state_len = 3},
                                                   NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                                   NULL, NULL),
           CV_OK);
    printf("strerror(EINVAL) = %s\n", conv_verify_strerror(CV_EINVAL));
    return fails;
}
