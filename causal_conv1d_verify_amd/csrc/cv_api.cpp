// C-ABI entry points of the verify conv library: host-side validation, launch
// planning and error reporting.  Every check runs before any HIP call, so a call
// that fails has launched nothing and written nothing.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "conv_verify.h"
#include "cv_internal.h"

namespace {

thread_local char g_detail[512];

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return code;
}

int dtype_bytes(int32_t dt) {
    switch (dt) {
        case CV_F32: return 4;
        case CV_BF16: return 2;
        default: return 0;
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kSpanLimit = ((int64_t)1 << 31) - 16;   // buffer-resource offsets stay below 2^31
constexpr int kChw = cvimpl::kWave * cvimpl::kChannelsPerLane;

// Size arithmetic on caller-supplied values (all >= 0 where these are used), saturating
// at INT64_MAX instead of overflowing: the results are only compared against limits,
// so an absurd size is refused rather than wrapped into an acceptable one.
int64_t sat_mul(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}
int64_t sat_add(int64_t a, int64_t b) {
    int64_t r;
    return __builtin_add_overflow(a, b, &r) ? INT64_MAX : r;
}
// bytes spanned by `rows` rows `stride` elements apart, the last of `width` elements
int64_t span_bytes(int64_t rows, int64_t stride, int64_t width, int elem_bytes) {
    return sat_mul(sat_add(sat_mul(rows - 1, stride), width), elem_bytes);
}

// Checks shared by every entry point: dtypes, d_conv, channels, state geometry.
int check_common(const cv_shape_t *s, int *xb_out, int *sb_out) {
    if (!s) return fail(CV_EINVAL, "shape is NULL");
    if (s->n_seq < 0) return fail(CV_EINVAL, "n_seq (%d) < 0", s->n_seq);
    if (s->d_inner < 0) return fail(CV_EINVAL, "d_inner (%d) < 0", s->d_inner);
    if (s->T < 1) return fail(CV_EINVAL, "T (%d) < 1", s->T);
    if (s->d_conv < 1) return fail(CV_EINVAL, "d_conv (%d) < 1", s->d_conv);
    if (s->d_conv < 2 || s->d_conv > 4)
        return fail(CV_ENOTSUP, "d_conv (%d) outside 2..4", s->d_conv);
    const int xb = dtype_bytes(s->x_dtype), sb = dtype_bytes(s->state_dtype);
    if (!xb || !sb) return fail(CV_EINVAL, "unknown dtype (x %d, state %d)", s->x_dtype, s->state_dtype);
    if (!((xb == 4 && sb == 4) || (xb == 2 && sb == 2) || (xb == 2 && sb == 4)))
        return fail(CV_ENOTSUP, "dtype pair (x f32, state bf16) is not supported");
    // channels come in 16-byte units of the x dtype, so every wavefront's share of
    // every buffer is a whole number of 16-byte chunks
    const int align = 16 / xb;
    if (s->d_inner % align)
        return fail(CV_ENOTSUP, "d_inner (%d) must be a multiple of %d", s->d_inner, align);
    if (s->n_slots < 0) return fail(CV_EINVAL, "n_slots (%d) < 0", s->n_slots);
    const int W1 = s->d_conv - 1;
    if (s->state_len < W1)
        return fail(CV_EINVAL, "state_len (%d) < d_conv-1 (%d)", s->state_len, W1);
    if (s->state_slot_stride < 0 || s->win_slot_stride < 0)
        return fail(CV_EINVAL, "negative slot stride");
    const int64_t C = s->d_inner;
    const int64_t col = s->state_col_stride;
    if (col < 0) return fail(CV_EINVAL, "state_col_stride (%lld) < 0", (long long)col);
    if (col > 0 && col < C)
        return fail(CV_EINVAL, "state_col_stride (%lld) < d_inner: state columns overlap",
                    (long long)col);
    // elements one slot's state spans, in either layout
    const int64_t state_span = col > 0 ? sat_add(sat_mul(s->state_len - 1, col), C)
                                       : sat_mul(C, s->state_len);
    if (s->n_slots > 1 && s->state_slot_stride < state_span)
        return fail(CV_EINVAL, "state_slot_stride (%lld) < the %lld elements of a slot's state",
                    (long long)s->state_slot_stride, (long long)state_span);
    if (s->state_slot_stride % (16 / sb) || s->win_slot_stride % (16 / sb) || col % (16 / sb))
        return fail(CV_ENOTSUP, "state/window slot and state column strides must be multiples "
                                "of 16 bytes");
    if (sat_mul(state_span, sb) > kSpanLimit)
        return fail(CV_ENOTSUP, "a slot's state spans more than 2 GiB");
    *xb_out = xb;
    *sb_out = sb;
    return CV_OK;
}

// L2 head geometry: lanes per head, its log2 (-1 when not a power of two) and the
// channel blocks of q|k.  align: the channel multiple every block must start and end on
// (16 bytes of the narrower of the element types that move in 16-byte units).
int plan_heads(const cv_shape_t *s, int align, int *hl_log2, cvimpl::HeadBlocks *h) {
    using cvimpl::kWave;
    const int cpl = cvimpl::kChannelsPerLane;
    *hl_log2 = 0;
    *h = cvimpl::HeadBlocks{0, 0, 0};
    if (s->qk_channels < 0 || s->qk_channels > s->d_inner)
        return fail(CV_EINVAL, "qk_channels (%d) outside 0..d_inner", s->qk_channels);
    if (s->qk_channels == 0) return CV_OK;
    if (s->head_dim <= 0) return fail(CV_EINVAL, "head_dim (%d) <= 0", s->head_dim);
    if (s->qk_channels % s->head_dim)
        return fail(CV_EINVAL, "qk_channels (%d) %% head_dim (%d) != 0", s->qk_channels, s->head_dim);
    if (!std::isfinite(s->l2_eps) || s->l2_eps < 0.0f)
        return fail(CV_EINVAL, "l2_eps must be finite and >= 0");
    if (s->head_dim % cpl)
        return fail(CV_ENOTSUP, "head_dim (%d) must be a multiple of %d", s->head_dim, cpl);
    const int hl = s->head_dim / cpl;
    if (hl > kWave)
        return fail(CV_ENOTSUP, "head_dim (%d) > %d: a head is reduced inside one wavefront",
                    s->head_dim, kWave * cpl);
    h->head_lanes = hl;
    if ((hl & (hl - 1)) == 0) {   // the head tiles the 256-channel blocks
        while ((1 << *hl_log2) < hl) ++*hl_log2;
        return CV_OK;
    }
    *hl_log2 = -1;
    // blocks of k whole heads, each block (and q|k's end, where the 256-channel blocks
    // begin) on the channel multiple the kernels' 16-byte units need
    int k = kWave * cpl / s->head_dim;
    while (k > 0 && (k * s->head_dim) % align) --k;
    if (k == 0)
        return fail(CV_ENOTSUP, "head_dim (%d): no block of whole heads of at most %d channels "
                                "is a multiple of %d", s->head_dim, kWave * cpl, align);
    if (s->qk_channels % align)
        return fail(CV_ENOTSUP, "qk_channels (%d) must be a multiple of %d with head_dim %d",
                    s->qk_channels, align, s->head_dim);
    h->qk_block_ch = k * s->head_dim;
    h->qk_blocks = (s->qk_channels + h->qk_block_ch - 1) / h->qk_block_ch;
    return CV_OK;
}

// Channel blocks per row: uniform 256-channel blocks, or the q|k blocks of whole heads
// and 256-channel blocks from qk on.
int64_t row_blocks(const cv_shape_t *s, const cvimpl::HeadBlocks &h) {
    const int64_t rest = h.qk_blocks ? (int64_t)s->d_inner - s->qk_channels : s->d_inner;
    return h.qk_blocks + (rest + kChw - 1) / kChw;
}

int64_t win_per_slot(int layout, const cv_shape_t *s) {
    const int64_t C = s->d_inner, W1 = s->d_conv - 1, L = s->T + W1 - 1;
    return layout == cvimpl::kDense ? (int64_t)s->T * C * W1 : C * L;
}

// Shape-only validation and launch planning of a verify call.
int plan_verify(int layout, bool tree, bool packed, const cv_shape_t *s, cvimpl::Plan *plan) {
    using cvimpl::kMaxLds;
    using cvimpl::kMaxT;
    using cvimpl::kWave;
    int xb = 0, sb = 0;
    int rc = check_common(s, &xb, &sb);
    if (rc) return rc;
    if (layout < cvimpl::kDense || layout > cvimpl::kRowsT)
        return fail(CV_EINVAL, "unknown window layout %d", layout);
    if (tree && layout != cvimpl::kDense)
        return fail(CV_EINVAL, "tree verify writes dense windows");
    if (s->T > kMaxT) return fail(CV_ENOTSUP, "T (%d) > %d", s->T, kMaxT);
    int hl_log2 = 0;
    cvimpl::HeadBlocks heads;
    rc = plan_heads(s, 16 / (xb < sb ? xb : sb), &hl_log2, &heads);
    if (rc) return rc;
    if (s->x_seq_stride < 0 || s->x_tok_stride < 0 || s->out_seq_stride < 0 || s->out_tok_stride < 0)
        return fail(CV_EINVAL, "negative x/out stride");
    const int align = 16 / xb;
    const int W1 = s->d_conv - 1;
    const int64_t C = s->d_inner;
    if ((s->T > 1 || packed) && s->out_tok_stride < C)
        return fail(CV_EINVAL, "out_tok_stride (%lld) < d_inner: tokens of out overlap",
                    (long long)s->out_tok_stride);
    if (!packed && s->n_seq > 1 &&
        s->out_seq_stride < sat_add(sat_mul(s->T - 1, s->out_tok_stride), C))
        return fail(CV_EINVAL, "out_seq_stride (%lld) too small: rows of out overlap",
                    (long long)s->out_seq_stride);
    const int64_t wps = win_per_slot(layout, s);
    if (s->n_slots > 1 && s->win_slot_stride < wps)
        return fail(CV_EINVAL, "win_slot_stride (%lld) < %lld elements per slot",
                    (long long)s->win_slot_stride, (long long)wps);
    if (s->x_seq_stride % align || s->x_tok_stride % align || s->out_seq_stride % align ||
        s->out_tok_stride % align)
        return fail(CV_ENOTSUP, "x/out strides must be multiples of %d elements", align);

    const int64_t blocks = row_blocks(s, heads);
    const int64_t wg = blocks * (int64_t)s->n_seq;
    if (sat_mul(wg, kWave) > (int64_t)UINT32_MAX)
        return fail(CV_ENOTSUP, "grid of %lld workgroups exceeds the launch limit", (long long)wg);
    int tb = 1;                                  // token buckets: 1 2 4 8 16 24 32
    while (tb < s->T && tb < 16) tb *= 2;
    if (tb < s->T) tb = s->T <= 24 ? 24 : 32;
    // LDS: the wavefront's conv_state region [channels, state_len] passes through first;
    // afterwards the same allocation holds the rows tile (T+D-2 rows of the
    // wavefront's channels) or one or two dense snapshot slabs [channels, D-1] - after
    // the tree's v tile (D-1+bucket rows) in tree verify.
    const int pitch = cvimpl::tile_pitch(sb);
    // (a time-major conv_state moves by columns through registers, not through LDS)
    const int64_t region = s->state_col_stride ? 0 : (int64_t)kChw * s->state_len * sb;
    const int64_t slabs = (int64_t)kChw * W1 * sb * (s->T > 1 ? 2 : 1);
    int64_t later = 0;
    if (layout == cvimpl::kRows) {
        // T a bucket and fixed rows: the compile-time-length path stages the row block
        // [channels, T+D-2] lane by lane (in halves past kRowsStageBytes); otherwise the
        // tile of T+D-2 sequence positions
        const int64_t block = (int64_t)kChw * (s->T + s->d_conv - 2) * sb;
        if (!packed && s->T == tb)
            later = block > cvimpl::kRowsStageBytes ? block / 2 : block;
        else
            later = (int64_t)(s->T + s->d_conv - 2) * pitch;
    }
    // While the loads are in flight the weights [channels, d_conv] sit at the start of
    // LDS; the state region is written over them once they are read, and (packed rows,
    // rows layout) the stored row block follows the region.  Both are filled by direct
    // global->LDS loads, so their spans are whole load-instruction widths.
    const int64_t wspan = cvimpl::lds_dma_span(kChw * s->d_conv * xb);
    const int64_t first = region > wspan ? region : wspan;
    if (layout == cvimpl::kRows && packed) {
        // the stored row block of short packed rows, past the state region and the weights
        // (it is loaded with them)
        const int64_t image = (region > wspan ? region : wspan) +
                              cvimpl::lds_dma_span(kChw * (s->T + s->d_conv - 2) * sb);
        if (image > later) later = image;
    }
    if (layout == cvimpl::kDense) later = (tree ? (int64_t)(W1 + tb) * pitch : 0) + slabs;
    const int64_t lds = first > later ? first : later;
    if (lds > kMaxLds)
        return fail(CV_ENOTSUP, "kernel needs %lld bytes of LDS (> %d)", (long long)lds, kMaxLds);
    // Buffer resources span one row's bytes with a 32-bit size; lanes past d_inner use
    // the offset 2^31, so every span must stay below it.
    const int64_t x_span = span_bytes(s->T, s->x_tok_stride, C, xb);
    const int64_t o_span = span_bytes(s->T, s->out_tok_stride, C, xb);
    const int64_t w_span = wps * sb;
    if (x_span > kSpanLimit || o_span > kSpanLimit || w_span > kSpanLimit)
        return fail(CV_ENOTSUP, "a row spans more than 2 GiB (x %lld, out %lld, windows %lld bytes)",
                    (long long)x_span, (long long)o_span, (long long)w_span);

    // Token split (dense windows, chain verify): on a grid too small to fill the chip,
    // each row's tokens are spread over ceil(T / kSplitChunk) wavefronts per channel
    // block.  Their LDS: chunk 0's state region, the weights, two snapshot slabs.
    // Tree verify splits the same way along its own 4-token chunks (buckets past 8),
    // each wavefront still building the row's whole v tile.
    int chunks = 1;
    int64_t split_lds = 0;
    const int64_t dense_chunks = (s->T + cvimpl::kSplitChunk - 1) / cvimpl::kSplitChunk;
    if (layout == cvimpl::kDense && !tree && s->T >= 2 * cvimpl::kSplitChunk &&
        wg * dense_chunks <= cvimpl::kSplitMaxWaves) {
        split_lds = region + cvimpl::lds_dma_span(kChw * s->d_conv * xb) + 2 * (int64_t)kChw * W1 * sb;
        if (split_lds <= kMaxLds) chunks = (int)dense_chunks;
    }
    const bool tree_split = tree && wg < cvimpl::kTreeSplitBelowWaves && tb > 8;
    if (tree_split) chunks = (s->T + 3) / 4;
    // Row layouts: chunk 0 of a split row keeps the copies (state commit, row block).
    const bool rows_split = (layout == cvimpl::kRows || layout == cvimpl::kRowsT) && !tree &&
                            (tb == 8 || tb == 16) && s->T > 4 &&
                            wg * ((s->T + 3) / 4) <= cvimpl::kRowsSplitMaxWaves;
    if (rows_split) chunks = (s->T + 3) / 4;

    plan->layout = layout;
    plan->tree = tree ? 1 : 0;
    plan->x_bytes = xb;
    plan->state_bytes = sb;
    plan->d_conv = s->d_conv;
    const bool dense_split = chunks > 1 && layout == cvimpl::kDense && !tree;
    plan->token_bucket = dense_split ? cvimpl::kSplitChunk : tb;
    plan->token_chunks = chunks;
    // The 16-token bucket's lean build (5 wavefronts per SIMD, a few spilled registers)
    // pays only where LDS lets 5 wavefronts per SIMD be resident, and exists for bf16 x
    // and state with a channel-major conv_state only (time-major, the regular build's
    // pipelined loads measured 3% faster at d 10240 and 10200: 102.0 against 105.4 us).
    plan->lean = tb == 16 && chunks == 1 && lds <= cvimpl::kRowsStageBytes && xb == 2 &&
                 sb == 2 && s->state_col_stride == 0;
    plan->state_tm = s->state_col_stride != 0;
    plan->channels_per_lane = cvimpl::kChannelsPerLane;
    plan->channel_blocks = (int)blocks;
    plan->workgroups = wg * chunks;
    plan->lds_bytes = (int)(dense_split ? split_lds : lds);
    plan->head_lanes = heads.head_lanes;
    plan->hl_log2 = hl_log2;
    plan->heads = heads;
    plan->waves_per_group = 1;
    // The line-aligned build (bf16, row layout, full 16-token rows, no token split): 4-wavefront
    // workgroups take 1024 channels each and cut their shared store ranges at the
    // destination's 128-byte lines.  Where rows start off those lines, one wavefront per 256
    // channels splits a line at every wavefront boundary.  With a time-major state it is
    // taken always: stress shape d 10200 116-118 -> 106 us, and on aligned rows 1% faster
    // (d 10240: 103.4 -> 102.2 us).  With a channel-major state only where a store range (the
    // rows of out, the slots' state regions or row blocks) starts off lines - d 10200: 172.0
    // -> 160.3 us; x and out on lines, state and rows off them: 160.4 -> 155.0 us; but all on
    // lines 153.5 -> 158.7 us and bs128 T16 26.5 -> 30.7 us - and where its LDS allows 3
    // workgroups per compute unit (state_len <= 18 at bf16).
    // Its LDS: two exchange buffers of 4 tokens of out (after a channel-major state's staged
    // region, which holds the workgroup's region after up to 112 bytes of its first line),
    // or the workgroup's row block placed the same way.
    // (strides are >= 0 here; reduced first, so no product overflows)
    auto off = [](int64_t stride, int bytes) { return (stride % 128) * bytes % 128 != 0; };
    const bool off_lines = off(s->out_tok_stride, xb) ||
                           (s->n_seq > 1 && off(s->out_seq_stride, xb)) ||
                           (s->n_slots > 1 && (off(s->state_slot_stride, sb) || off(s->win_slot_stride, sb)));
    {
        constexpr int nw = cvimpl::kLineGroupWaves;
        const int64_t range = (int64_t)kChw * nw;
        const int64_t out_bufs = 2 * 4 * range * xb;
        const int64_t block = 128 + range * (s->T + s->d_conv - 2) * sb;
        const int64_t region = plan->state_tm ? 0 : 128 + range * s->state_len * sb;
        if (layout == cvimpl::kRows && !tree && !packed && s->T == 16 && chunks == 1 && xb == 2 &&
            sb == 2 && heads.qk_blocks == 0 &&
            (plan->state_tm ||
             (off_lines && (region + 15) / 16 * 16 + out_bufs <= cvimpl::kLineGroupMaxLds))) {
            const int64_t staged = (region + 15) / 16 * 16 + out_bufs;
            const int64_t la_lds = staged > block ? staged : block;
            plan->waves_per_group = nw;
            plan->lean = 0;
            plan->channel_blocks = (int)((C + range - 1) / range);
            plan->workgroups = (int64_t)plan->channel_blocks * s->n_seq;
            plan->lds_bytes = (int)la_lds;
        }
    }
    // Data-movement choices, each measured on MI355X (none changes a result bit):
    // a grid of more than one resident generation waits for the slot before loading x
    // (padded rows then load nothing); a partial last channel block leaves the rows'
    // buffers off 128-byte line boundaries, so neighbouring wavefronts share lines and a
    // row's blocks go to one XCD (time-major builds there also store with the default
    // cache policy, so the shared lines merge in L2: a.store_cached).
    plan->slot_first = plan->workgroups * plan->waves_per_group > cvimpl::kResidentWaves;
    // (the line-aligned build with a channel-major state, which merges the partial lines
    // of neighbouring workgroups in L2, runs them in XCD order too; with a time-major
    // state that order measured slower: 106.5 -> 108.3 us at d 10200)
    plan->xcd_remap = plan->waves_per_group == 1 ? s->d_inner % kChw != 0 : !plan->state_tm;
    return CV_OK;
}

const void *pick_verify(const cvimpl::Plan &plan) {
    using namespace cvimpl;
    const int d = plan.d_conv, tb = plan.token_bucket;
    const int build = plan.waves_per_group > 1 ? 2 : plan.lean ? 1 : 0;
    const int split = plan.token_chunks > 1 ? 1 : 0;
    const int v = plan.tree ? 3 : plan.layout;
    if (plan.token_chunks > 1 && !plan.tree && plan.layout == cvimpl::kDense)
        return pick_split(plan.x_bytes, plan.state_bytes, d, plan.state_tm);
#define CV_PICK_TM(xb, sb, tm)                                      \
    switch (v) {                                                    \
        case 0: return pick_kernel_##xb##_##sb##_0_##tm(d, tb, build, split); \
        case 1: return pick_kernel_##xb##_##sb##_1_##tm(d, tb, build, split); \
        case 2: return pick_kernel_##xb##_##sb##_2_##tm(d, tb, build, split); \
        case 3: return pick_kernel_##xb##_##sb##_3_##tm(d, tb, build, split); \
        default: return nullptr;                                    \
    }
#define CV_PICK_FOR(xb, sb) \
    if (plan.state_tm) { CV_PICK_TM(xb, sb, 1) } else { CV_PICK_TM(xb, sb, 0) }
    if (plan.x_bytes == 4 && plan.state_bytes == 4) { CV_PICK_FOR(4, 4) }
    if (plan.x_bytes == 2 && plan.state_bytes == 2) { CV_PICK_FOR(2, 2) }
    if (plan.x_bytes == 2 && plan.state_bytes == 4) { CV_PICK_FOR(2, 4) }
#undef CV_PICK_FOR
#undef CV_PICK_TM
    return nullptr;
}

// Enqueues one 1-D launch of workgroups of `waves` 64-lane wavefronts; returns CV_OK or
// the launch error.
template <typename Args>
int launch(const void *fn, int64_t workgroups, int lds_bytes, const Args &args, void *stream,
           int waves = 1) {
    if (!fn)
        return fail(CV_EHIP_BASE - (int)hipErrorInvalidDeviceFunction,
                    "no kernel compiled for this case");
    Args a = args;
    void *kargs[] = {&a};
    const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)workgroups), dim3(cvimpl::kWave * waves), kargs,
                                         (size_t)lds_bytes, (hipStream_t)stream);
    if (e != hipSuccess)
        return fail(CV_EHIP_BASE - (int)e, "kernel launch failed: %s", hipGetErrorString(e));
    return CV_OK;
}

int verify(int layout, bool tree, const cv_shape_t *s, const void *x, const void *weight,
           const void *bias, void *conv_state, const int32_t *slot_idx, const int32_t *nat,
           const int32_t *cu, const int32_t *parent, void *out, void *win, void *stream) {
    g_detail[0] = 0;
    cvimpl::Plan plan;
    int rc = plan_verify(layout, tree, cu != nullptr, s, &plan);
    if (rc) return rc;
    if (s->n_seq == 0 || s->d_inner == 0) return CV_OK;   // nothing to do, nothing launched
    if (!x || !weight || !conv_state || !out || !win)
        return fail(CV_EINVAL, "NULL data pointer (x %p, weight %p, conv_state %p, out %p, "
                               "windows %p)", x, weight, conv_state, out, win);
    if (tree && !parent) return fail(CV_EINVAL, "parent is NULL");
    if (!aligned16(x) || !aligned16(weight) || (bias && !aligned16(bias)) ||
        !aligned16(conv_state) || !aligned16(out) || !aligned16(win))
        return fail(CV_ENOTSUP, "data pointers must be 16-byte aligned");
    if (!slot_idx && s->n_slots < s->n_seq)
        return fail(CV_EINVAL, "n_slots (%d) < n_seq (%d) with identity slots", s->n_slots,
                    s->n_seq);

    cvimpl::KernelArgs a;
    a.x = x;
    a.weight = weight;
    a.bias = bias;
    a.state = conv_state;
    a.slot_idx = slot_idx;
    a.nat = nat;
    a.out = out;
    a.win = win;
    a.cu = cu;
    a.parent = parent;
    a.x_seq = s->x_seq_stride;
    a.x_tok = s->x_tok_stride;
    a.out_seq = s->out_seq_stride;
    a.out_tok = s->out_tok_stride;
    a.state_slot = s->state_slot_stride;
    a.win_slot = s->win_slot_stride;
    a.n_seq = s->n_seq;
    a.T = s->T;
    a.d_inner = s->d_inner;
    a.qk = s->qk_channels;
    a.n_slots = s->n_slots;
    a.state_len = s->state_len;
    a.channel_blocks = plan.channel_blocks;
    a.head_lanes_log2 = plan.hl_log2;
    a.heads = plan.heads;
    a.eps = s->l2_eps;
    a.token_chunks = plan.token_chunks;
    a.state_col = s->state_col_stride;
    a.slot_first = slot_idx != nullptr && plan.slot_first;
    a.xcd_remap = plan.xcd_remap;
    a.store_cached = plan.xcd_remap && plan.state_tm && plan.waves_per_group == 1;
    return launch(pick_verify(plan), plan.workgroups, plan.lds_bytes, a, stream,
                  plan.waves_per_group);
}

}  // namespace

extern "C" {

int conv_verify_update_dense(const cv_shape_t *shape, const void *x, const void *weight,
                             const void *bias, void *conv_state, const int32_t *slot_idx,
                             const int32_t *num_accept_tokens, void *out, void *snapshots,
                             void *hip_stream) {
    return verify(cvimpl::kDense, false, shape, x, weight, bias, conv_state, slot_idx,
                  num_accept_tokens, nullptr, nullptr, out, snapshots, hip_stream);
}

int conv_verify_update_dedup(const cv_shape_t *shape, const void *x, const void *weight,
                             const void *bias, void *conv_state, const int32_t *slot_idx,
                             const int32_t *num_accept_tokens, void *out, void *window_rows,
                             void *hip_stream) {
    return verify(cvimpl::kRows, false, shape, x, weight, bias, conv_state, slot_idx,
                  num_accept_tokens, nullptr, nullptr, out, window_rows, hip_stream);
}

int conv_verify_update(const cv_shape_t *shape, int32_t layout, const void *x,
                       const void *weight, const void *bias, void *conv_state,
                       const int32_t *slot_idx, const int32_t *num_accept_tokens,
                       const int32_t *cu_seqlens, void *out, void *windows, void *hip_stream) {
    return verify(layout, false, shape, x, weight, bias, conv_state, slot_idx,
                  num_accept_tokens, cu_seqlens, nullptr, out, windows, hip_stream);
}

int conv_verify_update_tree(const cv_shape_t *shape, const void *x, const void *weight,
                            const void *bias, const void *conv_state,
                            const int32_t *slot_idx, const int32_t *num_accept_tokens,
                            const int32_t *cu_seqlens, const int32_t *parent, void *out,
                            void *windows, void *hip_stream) {
    // conv_state is only read in tree verify (that kernel variant stores nothing to it)
    return verify(cvimpl::kDense, true, shape, x, weight, bias, const_cast<void *>(conv_state),
                  slot_idx, num_accept_tokens, cu_seqlens, parent, out, windows, hip_stream);
}

int conv_verify_restore(const cv_shape_t *s, int32_t layout, void *conv_state,
                        const void *windows, const int32_t *slot_idx,
                        const int32_t *window_index, void *hip_stream) {
    g_detail[0] = 0;
    int xb = 0, sb = 0;
    int rc = check_common(s, &xb, &sb);
    if (rc) return rc;
    if (layout < cvimpl::kDense || layout > cvimpl::kRowsT)
        return fail(CV_EINVAL, "unknown window layout %d", layout);
    if (s->T > cvimpl::kMaxT) return fail(CV_ENOTSUP, "T (%d) > %d", s->T, cvimpl::kMaxT);
    const int64_t wps = win_per_slot(layout, s);
    if (s->n_slots > 1 && s->win_slot_stride < wps)
        return fail(CV_EINVAL, "win_slot_stride (%lld) < %lld elements per slot",
                    (long long)s->win_slot_stride, (long long)wps);
    if (wps * sb > kSpanLimit) return fail(CV_ENOTSUP, "a slot's windows span more than 2 GiB");
    if (s->n_seq == 0 || s->d_inner == 0) return CV_OK;
    if (!conv_state || !windows || !window_index)
        return fail(CV_EINVAL, "NULL pointer (conv_state %p, windows %p, window_index %p)",
                    conv_state, windows, (const void *)window_index);
    if (!aligned16(conv_state) || !aligned16(windows))
        return fail(CV_ENOTSUP, "data pointers must be 16-byte aligned");
    if (!slot_idx && s->n_slots < s->n_seq)
        return fail(CV_EINVAL, "n_slots (%d) < n_seq (%d) with identity slots", s->n_slots, s->n_seq);
    const int64_t blocks = (s->d_inner + kChw - 1) / kChw;
    const int64_t wg = blocks * (int64_t)s->n_seq;
    if (sat_mul(wg, cvimpl::kWave) > (int64_t)UINT32_MAX)
        return fail(CV_ENOTSUP, "grid of %lld workgroups exceeds the launch limit", (long long)wg);
    // LDS: the channel-major window block (rows layout), then the state region; both
    // are filled by direct global->LDS loads, so their spans are whole load widths
    const int64_t lds =
        (layout == cvimpl::kRows ? cvimpl::lds_dma_span(kChw * (s->T + s->d_conv - 2) * sb) : 0) +
        (s->state_col_stride ? 0 : cvimpl::lds_dma_span((int64_t)kChw * s->state_len * sb));
    if (lds > cvimpl::kMaxLds)
        return fail(CV_ENOTSUP, "restore needs %lld bytes of LDS (> %d)", (long long)lds, cvimpl::kMaxLds);
    cvimpl::RestoreArgs a;
    a.state = conv_state;
    a.win = windows;
    a.slot_idx = slot_idx;
    a.widx = window_index;
    a.state_slot = s->state_slot_stride;
    a.win_slot = s->win_slot_stride;
    a.n_seq = s->n_seq;
    a.T = s->T;
    a.d_inner = s->d_inner;
    a.n_slots = s->n_slots;
    a.state_len = s->state_len;
    a.channel_blocks = (int)blocks;
    a.state_col = s->state_col_stride;
    return launch(cvimpl::pick_restore(sb, s->d_conv, layout, s->state_col_stride != 0), wg, (int)lds, a, hip_stream);
}

int conv_prefill(const cv_shape_t *s, const void *x, const void *weight, const void *bias,
                 void *conv_state, const int32_t *slot_idx, const int32_t *cu_seqlens,
                 const int32_t *has_initial_state, void *out, void *hip_stream) {
    g_detail[0] = 0;
    int xb = 0, sb = 0;
    int rc = check_common(s, &xb, &sb);
    if (rc) return rc;
    const int align = 16 / xb;
    const int64_t C = s->d_inner;
    if (s->x_tok_stride < C || s->out_tok_stride < C)
        return fail(CV_EINVAL, "x/out token strides must be >= d_inner");
    if (s->x_tok_stride % align || s->out_tok_stride % align)
        return fail(CV_ENOTSUP, "x/out token strides must be multiples of %d elements", align);
    const int64_t x_span = span_bytes(s->T, s->x_tok_stride, C, xb);
    const int64_t o_span = span_bytes(s->T, s->out_tok_stride, C, xb);
    if (x_span > kSpanLimit || o_span > kSpanLimit)
        return fail(CV_ENOTSUP, "a prompt spans more than 2 GiB");
    if (s->n_seq == 0 || s->d_inner == 0) return CV_OK;
    if (!x || !weight || !conv_state || !out || !cu_seqlens)
        return fail(CV_EINVAL, "NULL pointer (x %p, weight %p, conv_state %p, out %p, cu_seqlens %p)",
                    x, weight, conv_state, out, (const void *)cu_seqlens);
    if (!aligned16(x) || !aligned16(weight) || (bias && !aligned16(bias)) ||
        !aligned16(conv_state) || !aligned16(out))
        return fail(CV_ENOTSUP, "data pointers must be 16-byte aligned");
    if (!slot_idx && s->n_slots < s->n_seq)
        return fail(CV_EINVAL, "n_slots (%d) < n_seq (%d) with identity slots", s->n_slots, s->n_seq);
    // a chunk-0 wavefront's state region, then the weights (direct global->LDS loads)
    const int64_t lds = (s->state_col_stride ? 0 : (int64_t)kChw * s->state_len * sb) +
                        cvimpl::lds_dma_span(kChw * s->d_conv * xb);
    if (lds > cvimpl::kMaxLds)
        return fail(CV_ENOTSUP, "prefill needs %lld bytes of LDS (> %d)", (long long)lds, cvimpl::kMaxLds);
    const int64_t blocks = (C + kChw - 1) / kChw;
    const int64_t chunks = (s->T + cvimpl::kPrefillChunk - 1) / cvimpl::kPrefillChunk;
    const int64_t wg = sat_mul(sat_mul(blocks, chunks), s->n_seq);
    if (sat_mul(wg, cvimpl::kWave) > (int64_t)UINT32_MAX)
        return fail(CV_ENOTSUP, "grid of %lld workgroups exceeds the launch limit", (long long)wg);
    cvimpl::PrefillArgs a;
    a.x = x;
    a.weight = weight;
    a.bias = bias;
    a.state = conv_state;
    a.slot_idx = slot_idx;
    a.cu = cu_seqlens;
    a.has_init = has_initial_state;
    a.out = out;
    a.x_tok = s->x_tok_stride;
    a.out_tok = s->out_tok_stride;
    a.state_slot = s->state_slot_stride;
    a.n_seq = s->n_seq;
    a.T = s->T;
    a.d_inner = s->d_inner;
    a.n_slots = s->n_slots;
    a.state_len = s->state_len;
    a.channel_blocks = (int)blocks;
    a.chunks = (int)chunks;
    a.state_col = s->state_col_stride;
    return launch(cvimpl::pick_prefill(xb, sb, s->d_conv, s->state_col_stride != 0), wg, (int)lds, a, hip_stream);
}

int conv_qk_l2norm(const cv_shape_t *s, int64_t n_rows, int64_t row_stride, void *x,
                   void *hip_stream) {
    g_detail[0] = 0;
    if (!s) return fail(CV_EINVAL, "shape is NULL");
    const int xb = dtype_bytes(s->x_dtype);
    if (!xb) return fail(CV_EINVAL, "unknown x dtype %d", s->x_dtype);
    if (s->d_inner < 0) return fail(CV_EINVAL, "d_inner (%d) < 0", s->d_inner);
    int hl_log2 = 0;
    cvimpl::HeadBlocks heads;
    int rc = plan_heads(s, 16 / xb, &hl_log2, &heads);
    if (rc) return rc;
    if (n_rows < 0) return fail(CV_EINVAL, "n_rows (%lld) < 0", (long long)n_rows);
    if (row_stride < s->qk_channels) return fail(CV_EINVAL, "row_stride < qk_channels");
    if (row_stride % (16 / xb)) return fail(CV_ENOTSUP, "row_stride must be a multiple of %d", 16 / xb);
    if (s->qk_channels % (16 / xb))
        return fail(CV_ENOTSUP, "qk_channels must be a multiple of %d", 16 / xb);
    if (span_bytes(cvimpl::kL2Rows, row_stride, s->qk_channels, xb) > kSpanLimit)
        return fail(CV_ENOTSUP, "%d rows of x span more than 2 GiB", cvimpl::kL2Rows);
    if (n_rows == 0 || s->qk_channels == 0) return CV_OK;
    if (!x) return fail(CV_EINVAL, "x is NULL");
    if (!aligned16(x)) return fail(CV_ENOTSUP, "x must be 16-byte aligned");
    const int64_t blocks = heads.qk_blocks ? heads.qk_blocks : (s->qk_channels + kChw - 1) / kChw;
    const int64_t wg = sat_mul(blocks, n_rows / cvimpl::kL2Rows + (n_rows % cvimpl::kL2Rows != 0));
    if (sat_mul(wg, cvimpl::kWave) > (int64_t)UINT32_MAX)
        return fail(CV_ENOTSUP, "grid of %lld workgroups exceeds the launch limit", (long long)wg);
    cvimpl::L2Args a;
    a.x = x;
    a.row_stride = row_stride;
    a.n_rows = n_rows;
    a.qk = s->qk_channels;
    a.qk_blocks = (int)blocks;
    a.head_lanes_log2 = hl_log2;
    a.eps = s->l2_eps;
    a.heads = heads;
    return launch(cvimpl::pick_l2(xb), wg, 0, a, hip_stream);
}

int conv_verify_describe(int variant, const cv_shape_t *shape, cv_launch_info_t *info) {
    g_detail[0] = 0;
    if (!info) return fail(CV_EINVAL, "info is NULL");
    if (variant < 0 || variant > CV_VARIANT_TREE) return fail(CV_EINVAL, "unknown variant %d", variant);
    cvimpl::Plan plan;
    const bool tree = variant == CV_VARIANT_TREE;
    int rc = plan_verify(tree ? cvimpl::kDense : variant, tree, false, shape, &plan);
    if (rc) return rc;
    info->workgroups = plan.workgroups;
    info->threads = cvimpl::kWave * plan.waves_per_group;
    info->channel_blocks = plan.channel_blocks;
    info->channels_per_wave = cvimpl::kWave * plan.channels_per_lane;
    info->channels_per_lane = plan.channels_per_lane;
    info->token_bucket = plan.token_bucket;
    info->lds_bytes = plan.lds_bytes;
    info->head_lanes = plan.head_lanes;
    info->token_chunks = plan.token_chunks;
    info->flags = (plan.state_tm ? CV_LAUNCH_STATE_TIME_MAJOR : 0) |
                  (plan.slot_first ? CV_LAUNCH_SLOT_FIRST : 0) |
                  (plan.xcd_remap ? CV_LAUNCH_XCD_ORDER : 0) |
                  (plan.waves_per_group > 1 ? CV_LAUNCH_LINE_ALIGNED : 0) |
                  (plan.heads.qk_blocks ? CV_LAUNCH_HEAD_BLOCKS : 0);
    return CV_OK;
}

const char *conv_verify_strerror(int code) {
    if (code == CV_OK) return "success";
    if (code == CV_EINVAL) return "invalid argument";
    if (code == CV_ENOTSUP) return "not supported by the compiled kernels";
    if (code <= CV_EHIP_BASE) return "HIP kernel launch failed";
    return "unknown error";
}

const char *conv_verify_last_error(void) { return g_detail; }

int conv_verify_abi_version(void) { return CONV_VERIFY_ABI_VERSION; }

int conv_verify_debug_count(int32_t n, const void *const *lo, const uint64_t *bytes,
                            void *const *counts) {
    g_detail[0] = 0;
#ifdef CV_WRITE_COUNT
    if (n < 0 || n > 4) return fail(CV_EINVAL, "count ranges: n (%d) outside 0..4", n);
    if (n > 0 && (!lo || !bytes || !counts)) return fail(CV_EINVAL, "count ranges: NULL array");
    cvimpl::CountRanges c;
    std::memset(&c, 0, sizeof c);
    c.n = n;
    for (int k = 0; k < n; ++k) {
        if (!lo[k] || !counts[k] || bytes[k] % 2 != 0)
            return fail(CV_EINVAL, "count range %d: NULL pointer or odd size", k);
        c.lo[k] = (const char *)lo[k];
        c.bytes[k] = bytes[k];
        c.counts[k] = (uint32_t *)counts[k];
    }
    int (*const setters[])(const cvimpl::CountRanges &) = {
        cvimpl::count_ranges_set_2_2_0_0, cvimpl::count_ranges_set_2_2_1_0,
        cvimpl::count_ranges_set_2_2_2_0, cvimpl::count_ranges_set_2_2_3_0,
        cvimpl::count_ranges_set_2_2_0_1, cvimpl::count_ranges_set_2_2_1_1,
        cvimpl::count_ranges_set_2_2_2_1, cvimpl::count_ranges_set_2_2_3_1,
        cvimpl::count_ranges_set_aux};
    for (size_t i = 0; i < sizeof setters / sizeof setters[0]; ++i) {
        const int e = setters[i](c);
        if (e != 0)
            return fail(CV_EHIP_BASE - e, "count ranges: code object %zu: %s (%d)", i,
                        hipGetErrorName((hipError_t)e), e);
    }
    return CV_OK;
#else
    (void)n; (void)lo; (void)bytes; (void)counts;
    return fail(CV_ENOTSUP, "write counting exists only in the write-count build of the library");
#endif
}

}  // extern "C"

#ifdef CV_WRITE_COUNT
// The write-count build compiles the verify objects for bf16 x and state only: the
// pickers of the other dtype pairs find no kernel (the launch then fails cleanly).
namespace cvimpl {
#define CV_NO_PICKER(xb, sb, v, tm) \
    const void *pick_kernel_##xb##_##sb##_##v##_##tm(int, int, int, int) { return nullptr; }
#define CV_NO_PICKERS(xb, sb) CV_NO_PICKER(xb, sb, 0, 0) CV_NO_PICKER(xb, sb, 1, 0) \
    CV_NO_PICKER(xb, sb, 2, 0) CV_NO_PICKER(xb, sb, 3, 0) CV_NO_PICKER(xb, sb, 0, 1) \
    CV_NO_PICKER(xb, sb, 1, 1) CV_NO_PICKER(xb, sb, 2, 1) CV_NO_PICKER(xb, sb, 3, 1)
CV_NO_PICKERS(4, 4)
CV_NO_PICKERS(2, 4)
#undef CV_NO_PICKERS
#undef CV_NO_PICKER
}  // namespace cvimpl
#endif
