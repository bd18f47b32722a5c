/*
 * conv_verify.h - C ABI of the batched speculative-verify causal conv1d update,
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * One call = one kernel launch that, for every row i < n_seq of a batch of
 * speculative-decode chains and every draft position t < T, computes
 *
 *   pre[i,t,c] = bias[c] + sum_{w < D} weight[c,w] * v[t+w]       (depthwise, causal)
 *   y          = SiLU(pre) = pre / (1 + exp(-pre))
 *   y          = y / sqrt(sum_{c' in head(c)} y[c']^2 + l2_eps)   for c < qk_channels
 *   out[i,t,c] = y rounded once (nearest even) to the x dtype
 *
 * over the sequence v = [conv_state[s, c, a .. a+D-2], x[i,0,c], ..., x[i,T-1,c]]
 * with s = slot_idx[i] and a = num_accept_tokens[i], writes every per-token
 * rollback window (the window after consuming x_t is v[t+1 .. t+D-1]) and leaves
 * conv_state[s, c, 0 .. D-2] holding the committed window v[T .. T+D-2].
 *
 * Sources (page title, section):
 *  - Atlas docs, fn spark_model::layers::ops::gdn_verify_fused_conv_kn_batched: one
 *    launch covers every draft position of every sequence; the same launch writes each
 *    position's rollback snapshot to a strided buffer; afterwards conv_state holds the
 *    window committed after the last position (equal to the last snapshot); the
 *    arguments carry per-token and per-sequence strides; the sequences' windows do not
 *    interact.
 *  - sglang PR 46184 (dedup conv window tile store), "Motivation" and
 *    "Modifications": the deduplicated per-slot row [dim, T+K-2] viewed as an
 *    overlapping [T, dim, K-1] window with step stride == window stride, written
 *    once instead of per token; padded rows exit before any store; a
 *    num_accept_tokens state offset.  "Scope": dense [T, dim, K-1] windows.
 *  - Atlas glm5next_kda/mod.rs, Glm5NextKdaConfig: conv -> SiLU -> L2 on q|k only,
 *    FLA convention 1/sqrt(sum + eps), V never normalised, qk_channels = 2*heads*hd.
 *
 * Beyond that chain verify the library covers, with the same kernels family:
 *  - packed variable-length rows (cu_seqlens), sglang PR 46184, "Related upstream
 *    work" (packed ragged tokens in the verify kernel, so the tile store covers them);
 *  - the time-major row layout (MambaPool's window layout along axis 0: the
 *    channel-major rows transposed),
 *    sglang PR 46184, "Modifications" (test coverage);
 *  - tree verify (per-token parents, dense windows), sglang PR 46184, "Scope";
 *  - the accepted-prefix restore (window k -> conv_state), sglang PR 46184,
 *    "Motivation"; Atlas glm5next_kda/mod.rs, decode_k (snapshots a partial accept
 *    rewinds to);
 *  - the prefill conv (conv + SiLU, no L2, no windows) and the separate q|k L2 pass,
 *    Atlas glm5next_kda/mod.rs, module doc and the prefill body (the prefill conv
 *    computes conv and SiLU only; q|k get their L2 in a launch of their own).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every data pointer is a DEVICE pointer (HBM of the GPU current on the calling
 *    thread); only `shape` is a host pointer.  The caller owns every buffer.  The
 *    library allocates nothing, keeps no pointer after returning, performs no
 *    host<->device copy and never synchronizes: the call enqueues exactly one kernel
 *    on `hip_stream` (a hipStream_t; NULL = the null stream) and returns.
 *  - Thread-safe and stateless (apart from a thread-local error detail string).
 *  - All validation happens on the host before any HIP call; a call that returns an
 *    error has launched nothing and written nothing.  Faults inside the kernel can
 *    only surface at the caller's next synchronization of the stream.
 *  - Element layouts (strides in ELEMENTS, innermost dimension contiguous):
 *      x           [n_seq, T, d_inner]     x[i,t,c]   = x   + i*x_seq_stride   + t*x_tok_stride   + c
 *      out         [n_seq, T, d_inner]     out[i,t,c] = out + i*out_seq_stride + t*out_tok_stride + c
 *      weight      [d_inner, d_conv]       contiguous; weight[c, d_conv-1] multiplies x_t
 *      bias        [d_inner]               contiguous, or NULL (no bias)
 *      conv_state  [n_slots, d_inner, state_len] (channel-major, state_col_stride == 0):
 *                  state[s,c,k] = conv_state + s*state_slot_stride + c*state_len + k
 *                  or [n_slots, state_len, d_inner] (time-major, state_col_stride > 0):
 *                  state[s,c,k] = conv_state + s*state_slot_stride + k*state_col_stride + c
 *      slot_idx    [n_seq] int32 or NULL (row i uses slot i).  -1 marks a padded row.
 *      num_accept_tokens [n_seq] int32 or NULL (all 0): start column a of row i's window.
 *  - A padded row (slot -1) writes nothing at all: not out, not conv_state, not the
 *    windows.  Slots no row references are never touched.
 *  - Device-side preconditions (not checked on the host, which never reads device
 *    memory): the slots of non-padded rows are distinct; 0 <= a <= state_len-(d_conv-1).
 *    A row whose slot is >= n_slots or < -1, or whose a is out of that range, is
 *    skipped like a padded row (nothing written), so bad indices never address
 *    memory outside the buffers.  Two rows sharing a slot race.
 *  - Buffers must not overlap each other (x and weight/bias may).
 *  - Alignment (else CV_ENOTSUP): every pointer 16-byte aligned; d_inner, the x/out
 *    strides multiples of 16/sizeof(x element) (8 for bf16, 4 for fp32);
 *    state_slot_stride, state_col_stride and win_slot_stride multiples of 16 bytes;
 *    a head is reduced inside one wavefront: head_dim a multiple of 4 up to 256.  A
 *    head_dim that divides 256 (4, 8, ..., 256) tiles the 256-channel wavefronts; any
 *    other (12, 96, 192, ...) makes the q|k channels go in blocks of k whole heads, k
 *    the largest with k * head_dim <= 256 and a multiple of 16/min(sizeof(x element),
 *    sizeof(state element)), followed by 256-channel blocks from qk_channels on, so
 *    qk_channels must be such a multiple too (CV_LAUNCH_HEAD_BLOCKS).
 *  - LDS (else CV_ENOTSUP): with a channel-major conv_state, a 256-channel wavefront
 *    stages its [256, state_len] state region (and its weights, its window tiles) in
 *    LDS, at most 160 KiB (all of a gfx950 compute unit's): state_len up to 160 fp32 /
 *    320 bf16 columns.  A time-major conv_state is not staged (no such limit).
 *  - Which conv_state layout to pick: a channel-major row wider than the window
 *    (state_len > d_conv-1, as offsets need) puts window bytes in every 32-byte
 *    sector, so the kernels move such rows whole, read and written back; in the
 *    time-major layout a window is d_conv-1 contiguous columns of d_inner channels and
 *    only those move.
 *  - Numerics: the conv accumulates in fp32 as acc = bias (or +0); for w = 0..D-1:
 *    acc = fma(weight[c,w], v[t+w], acc), each step one correctly rounded fused
 *    multiply-add.  SiLU runs in fp32 in a form that neither overflows nor loses
 *    its subnormal results (p far below zero).  The L2 sums squares in fp32; a head
 *    whose sum leaves fp32's range (|y| from ~1.3e19, or tiny values with
 *    l2_eps < 2^-60) is summed again over a power-of-two rescaling of its values.
 *    One case is outside: l2_eps == 0 with a head whose sum of squares is below
 *    2^-256 (every value of the head subnormal) gives +-inf or NaN there.  Windows
 *    and conv_state are moved as bit patterns (bf16 -> fp32 widening is exact), so
 *    -0.0, subnormals and NaN payloads survive.
 *  - The window buffer is indexed by slot, like conv_state: it holds n_slots slots.
 */
#ifndef CONV_VERIFY_H
#define CONV_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 5: conv_verify_debug_count; launch info may report 4-wavefront workgroups
 *    (CV_LAUNCH_LINE_ALIGNED, threads 256).
 * 6: heads whose lane count is not a power of two (head_dim 12, 96, 192, ...), with
 *    CV_LAUNCH_HEAD_BLOCKS. */
#define CONV_VERIFY_ABI_VERSION 6

/* Only the entry points below are exported from the shared library. */
#define CV_API __attribute__((visibility("default")))

/* Element types. */
typedef enum cv_dtype { CV_F32 = 0, CV_BF16 = 1 } cv_dtype_t;

/* Return codes. */
#define CV_OK 0
#define CV_EINVAL (-22)      /* malformed arguments: NULL pointer, bad size or stride */
#define CV_ENOTSUP (-95)     /* well-formed but outside what the kernels implement */
#define CV_EHIP_BASE (-1000) /* launch failure: returns CV_EHIP_BASE - (int)hipError_t */

/* Rollback-window layouts (T = shape->T, W1 = d_conv - 1, L = T + W1 - 1):
 *   CV_WIN_DENSE  [n_slots, T, d_inner, W1]  win[s,t,c,j] = base + s*ws + (t*d_inner + c)*W1 + j
 *                                             = the window after consuming x_t
 *   CV_WIN_ROWS   [n_slots, d_inner, L]      row[s,c,k]   = base + s*ws + c*L + k = v[k+1]
 *   CV_WIN_ROWS_T [n_slots, L, d_inner]      row[s,k,c]   = base + s*ws + k*d_inner + c = v[k+1]
 * In both row layouts the window after consuming x_t is columns t .. t+W1-1: the view
 * [T, d_inner, W1] has step stride == window stride (sglang PR 46184, "Modifications").
 * ws = shape->win_slot_stride. */
typedef enum cv_layout { CV_WIN_DENSE = 0, CV_WIN_ROWS = 1, CV_WIN_ROWS_T = 2 } cv_layout_t;

/* Problem description (host memory, read during the call only). */
typedef struct cv_shape {
    int32_t n_seq;        /* rows in the batch, >= 0 (0: nothing to do, returns CV_OK)      */
    int32_t T;            /* draft positions per row, 1..32 (packed rows: the most a row
                             may hold, and the T of the window buffer's geometry);
                             conv_prefill: the longest prompt, >= 1                         */
    int32_t d_inner;      /* channels, >= 0 (0: nothing to do)                              */
    int32_t d_conv;       /* conv width D, 2..4                                             */
    int32_t qk_channels;  /* leading channels normalised per head, 0..d_inner; 0 = no L2    */
    int32_t head_dim;     /* channels per L2 head: qk_channels % head_dim == 0, head_dim a
                             multiple of 4 (channels per lane) and <= 256; see Alignment   */
    float l2_eps;         /* >= 0 and finite                                                */
    int32_t x_dtype;      /* cv_dtype_t of x, weight, bias and out                          */
    int32_t state_dtype;  /* cv_dtype_t of conv_state and the windows.  Supported pairs
                             (x, state): (F32, F32), (BF16, BF16), (BF16, F32)              */
    int32_t n_slots;      /* slots in the conv_state pool and in the window buffer, >= 0;
                             >= n_seq when slot_idx is NULL                                 */
    int32_t state_len;    /* columns per state channel, >= d_conv-1                         */
    int64_t x_seq_stride, x_tok_stride;      /* elements, >= 0                              */
    int64_t out_seq_stride, out_tok_stride;  /* elements; rows/tokens of out must not overlap */
    int64_t state_slot_stride;               /* elements, >= d_inner*state_len if n_slots>1 */
    int64_t win_slot_stride;                 /* elements of the window buffer per slot,
                                                >= its per-slot size if n_slots > 1         */
    int64_t state_col_stride;                /* 0: conv_state channel-major (a channel's
                                                state_len columns contiguous).  > 0:
                                                time-major, elements between columns,
                                                >= d_inner; then state_slot_stride >=
                                                (state_len-1)*state_col_stride + d_inner
                                                if n_slots > 1                              */
} cv_shape_t;

/*
 * Dense rollback windows (sglang PR 46184, "Scope": UnifiedMambaPool, KDA/Kimi-Linear;
 * Atlas gdn_verify_fused_conv_kn_batched's conv_state_inter).
 *
 *   snapshots [n_slots, T, d_inner, d_conv-1]:
 *     snapshots[s,t,c,j] = snapshots + s*win_slot_stride + (t*d_inner + c)*(d_conv-1) + j
 *                        = v[t+1+j]   (the window after consuming x_t; t = T-1 is the
 *                                      committed window)
 *
 * Returns CV_OK after enqueueing the launch, or an error code (nothing launched).
 */
CV_API int conv_verify_update_dense(const cv_shape_t *shape, const void *x, const void *weight,
                             const void *bias, void *conv_state, const int32_t *slot_idx,
                             const int32_t *num_accept_tokens, void *out, void *snapshots,
                             void *hip_stream);

/*
 * Deduplicated rollback windows (sglang PR 46184, "Motivation", "Modifications":
 * MambaPool's one row per slot, written once).
 *
 *   window_rows [n_slots, d_inner, T+d_conv-2]:
 *     rows[s,c,k] = window_rows + s*win_slot_stride + c*(T+d_conv-2) + k  = v[k+1]
 *   so the window after consuming x_t is columns t .. t+d_conv-2 of the row: the
 *   overlapping [T, d_inner, d_conv-1] view with step stride == window stride.
 *
 * Returns CV_OK after enqueueing the launch, or an error code (nothing launched).
 */
CV_API int conv_verify_update_dedup(const cv_shape_t *shape, const void *x, const void *weight,
                             const void *bias, void *conv_state, const int32_t *slot_idx,
                             const int32_t *num_accept_tokens, void *out, void *window_rows,
                             void *hip_stream);

/*
 * The general verify: any window layout, and optionally packed rows.
 *
 *   layout      cv_layout_t of `windows`.
 *   cu_seqlens  NULL, or [n_seq+1] int32 (device): packed rows.  Row i holds
 *               T_i = cu[i+1] - cu[i] tokens, token t at x[(cu[i]+t)*x_tok_stride + c]
 *               and out[(cu[i]+t)*out_tok_stride + c]; the seq strides are unused.  A
 *               row with T_i = 0 writes nothing (its state keeps its starting window
 *               where it was).  Its windows are those of t < T_i; in the row layouts
 *               it writes columns 0 .. T_i+W1-2 and leaves the rest of its row alone.
 *               Device-side precondition: non-decreasing offsets inside x and out; a
 *               row with T_i outside 0..T is skipped like a padded row.
 *
 * Without cu_seqlens, CV_WIN_DENSE is conv_verify_update_dense and CV_WIN_ROWS is
 * conv_verify_update_dedup.  Returns CV_OK after enqueueing the launch, or an error.
 */
CV_API int conv_verify_update(const cv_shape_t *shape, int32_t layout, const void *x,
                       const void *weight, const void *bias, void *conv_state,
                       const int32_t *slot_idx, const int32_t *num_accept_tokens,
                       const int32_t *cu_seqlens, void *out, void *windows, void *hip_stream);

/*
 * Tree verify (sglang PR 46184, "Scope": tree verify keeps per-token dense windows).
 *
 *   parent [n_seq, T] int32 (device), row stride T: parent[i,t] in -1 .. t-1.  Token
 *          t's conv runs over the window of its parent token (-1: the row's starting
 *          window, conv_state[s, c, a .. a+D-2]) followed by x_t, and its window is
 *          that window shifted by x_t; the chain is parent[i,t] = t-1.
 *   windows: CV_WIN_DENSE layout.  conv_state is only read: the accepted path is
 *          known after verification, and conv_verify_restore writes its window.
 *   cu_seqlens as in conv_verify_update (NULL: T tokens per row).  A row with a
 *          parent outside -1..t-1 is skipped (nothing written).
 */
CV_API int conv_verify_update_tree(const cv_shape_t *shape, const void *x, const void *weight,
                            const void *bias, const void *conv_state,
                            const int32_t *slot_idx, const int32_t *num_accept_tokens,
                            const int32_t *cu_seqlens, const int32_t *parent, void *out,
                            void *windows, void *hip_stream);

/*
 * Accepted-prefix restore (sglang PR 46184, "Motivation"; Atlas decode_k snapshots):
 * for each row i with slot s = slot_idx[i] >= 0 and k = window_index[i] >= 0,
 *   conv_state[s, c, 0 .. d_conv-2] = the window after consuming x_k, read from
 *   `windows` in `layout` (chain verify: k = accepted tokens - 1; tree verify: the
 *   position of the last accepted token).  Columns >= d_conv-1 are not written.
 * Uses shape fields n_seq, T (the window buffer's), d_inner, d_conv, state_dtype,
 * n_slots, state_len, state_slot_stride, state_col_stride, win_slot_stride (x fields
 * are ignored).
 * window_index [n_seq] int32 (device).  Rows with k >= T or a slot >= n_slots are
 * skipped.  One launch; returns CV_OK or an error (nothing launched).
 */
CV_API int conv_verify_restore(const cv_shape_t *shape, int32_t layout, void *conv_state,
                        const void *windows, const int32_t *slot_idx,
                        const int32_t *window_index, void *hip_stream);

/*
 * Prefill conv over packed prompts (Atlas glm5next_kda/mod.rs, prefill body: conv +
 * SiLU only; the L2 is a separate pass, conv_qk_l2norm).  Row i's T_i = cu[i+1]-cu[i]
 * tokens (0 <= T_i <= shape->T) run through the conv starting from its state window
 * conv_state[s, c, 0 .. D-2] (s = slot_idx[i], or i), or from zeros where
 * has_initial_state[i] == 0; out gets SiLU(conv + bias) rounded to the x dtype; the
 * last window is committed to conv_state[s, c, 0 .. D-2].  No rollback windows, no
 * L2 (qk_channels and head_dim are ignored).  has_initial_state may be NULL (all 1).
 * shape->T may exceed 32 here.
 */
CV_API int conv_prefill(const cv_shape_t *shape, const void *x, const void *weight, const void *bias,
                 void *conv_state, const int32_t *slot_idx, const int32_t *cu_seqlens,
                 const int32_t *has_initial_state, void *out, void *hip_stream);

/*
 * Separate per-head L2 over the q|k channels, in place: for each of n_rows rows of x
 * (row r at x + r*row_stride, channel stride 1) and each head of head_dim channels in
 * [0, qk_channels): y <- y / sqrt(sum_head y^2 + l2_eps) in fp32, rounded to the x
 * dtype.  Channels >= qk_channels are not touched.  Uses shape fields d_inner,
 * qk_channels, head_dim, l2_eps, x_dtype (head_dim as for the verify, its blocks of whole
 * heads a multiple of 16/sizeof(x element)).  CV_ENOTSUP if 2 consecutive rows span more
 * than 2 GiB (a wavefront takes 2 rows).
 */
CV_API int conv_qk_l2norm(const cv_shape_t *shape, int64_t n_rows, int64_t row_stride, void *x,
                   void *hip_stream);

/* Launch geometry the library would use for a shape (validation of the shape only;
 * pointers are not examined).  Lets a caller or a test check, on the host, what the
 * kernel and its grid will assume. */
typedef struct cv_launch_info {
    int64_t workgroups;        /* 1-D grid: n_seq * channel_blocks * token_chunks         */
    int32_t threads;           /* per workgroup: one 64-lane wavefront, or 4 (LINE_ALIGNED) */
    int32_t channel_blocks;    /* workgroups per row: ceil(d_inner / (channels_per_wave *  */
                               /* threads / 64)); with HEAD_BLOCKS the q|k blocks of whole */
                               /* heads, then ceil((d_inner - qk_channels) / 256)          */
    int32_t channels_per_wave; /* 64 lanes * channels per lane                             */
    int32_t channels_per_lane; /* 16 bytes of x per lane per token                         */
    int32_t token_bucket;      /* compile-time tokens per workgroup (>= T unless split)    */
    int32_t lds_bytes;         /* dynamic LDS per workgroup                                */
    int32_t head_lanes;        /* lanes per L2 head (0 when qk_channels == 0)              */
    int32_t token_chunks;      /* workgroups per (row, channel block) along T: 1, or, on a */
                               /* small grid, ceil(T / 4) - each row's tokens spread over  */
                               /* wavefronts, each computing its 4-token chunk (dense      */
                               /* chain verify: token_bucket 4; row layouts: chunk 0 also  */
                               /* writes the row block and the state)                      */
    int32_t flags;             /* CV_LAUNCH_* bits: how the launch moves its data          */
} cv_launch_info_t;

/* cv_launch_info_t.flags (host-side launch choices; none changes a result bit):
 *   STATE_TIME_MAJOR  the time-major conv_state build (state_col_stride > 0)
 *   SLOT_FIRST        with a slot table, a wavefront reads its row's slot before any
 *                     vector load, so padded rows load nothing (grids of more than
 *                     5,120 wavefronts: more than one resident generation)
 *   XCD_ORDER         work items follow MI355X's round-robin XCD dispatch so that a row's
 *                     channel blocks share one L2 (d_inner not a multiple of 256; and the
 *                     line-aligned build with a channel-major conv_state)
 *   LINE_ALIGNED      workgroups of 4 wavefronts over 1024 channels, whose store ranges
 *                     leave through LDS cut at 128-byte lines (bf16, time-major
 *                     conv_state, dedup rows, T 16, no token split)
 *   HEAD_BLOCKS       head_dim does not divide 256: the q|k channels go in blocks of
 *                     whole heads (see Alignment) and each head is summed by a segmented
 *                     scan across its lanes */
#define CV_LAUNCH_STATE_TIME_MAJOR 1
#define CV_LAUNCH_SLOT_FIRST 2
#define CV_LAUNCH_XCD_ORDER 4
#define CV_LAUNCH_LINE_ALIGNED 8
#define CV_LAUNCH_HEAD_BLOCKS 16

/* variant: a cv_layout_t, or CV_VARIANT_TREE for conv_verify_update_tree.  Returns
 * CV_OK or an error code. */
#define CV_VARIANT_TREE 3
CV_API int conv_verify_describe(int variant, const cv_shape_t *shape, cv_launch_info_t *info);

/* Static description of an error code (never NULL). */
CV_API const char *conv_verify_strerror(int code);

/* Detail of the last error returned on the calling thread (empty string if none). */
CV_API const char *conv_verify_last_error(void);

/* CONV_VERIFY_ABI_VERSION of the loaded library. */
CV_API int conv_verify_abi_version(void);

/* Test instrumentation, for the single-writer check of the outputs (no passage of the
 * pages defines it; it exists to show that every element is written by one store).
 * Only libconvverify_wc.so, the write-count build of the library (its verify kernels
 * for bf16 x and state, and every restore / prefill / L2 kernel), implements it; the
 * regular library returns CV_ENOTSUP.  Registers n (0..4) device ranges: range k covers
 * bytes[k] bytes from lo[k] (even), and counts[k] is a device array of bytes[k] / 2
 * uint32 counters, one per 2 bytes.  Every global store a later launch makes inside a
 * range adds 1 to the counter of each 2-byte unit it writes; stores outside all ranges
 * count nothing.  The caller owns every buffer and zeroes the counters; the ranges stay
 * registered (and must stay allocated) until the next call, n = 0 clears them.  The
 * counters are added to atomically, so launches of the write-count build run slower. */
CV_API int conv_verify_debug_count(int32_t n, const void *const *lo, const uint64_t *bytes,
                                   void *const *counts);

#ifdef __cplusplus
}
#endif

#endif /* CONV_VERIFY_H */
