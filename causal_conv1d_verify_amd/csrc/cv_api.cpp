// C-ABI entry points of the verify conv library: host-side validation, launch
// planning and error reporting.  Every check runs before any HIP call, so a call
// that fails has launched nothing and written nothing.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

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

// Shape-only validation and launch planning.
int plan_shape(int dedup, const cv_shape_t *s, cvimpl::Plan *plan) {
    using cvimpl::kMaxLds;
    using cvimpl::kMaxT;
    using cvimpl::kWave;
    if (!s) return fail(CV_EINVAL, "shape is NULL");
    if (dedup != 0 && dedup != 1) return fail(CV_EINVAL, "dedup must be 0 or 1");
    if (s->n_seq < 0) return fail(CV_EINVAL, "n_seq (%d) < 0", s->n_seq);
    if (s->d_inner < 0) return fail(CV_EINVAL, "d_inner (%d) < 0", s->d_inner);
    if (s->T < 1) return fail(CV_EINVAL, "T (%d) < 1", s->T);
    if (s->T > kMaxT) return fail(CV_ENOTSUP, "T (%d) > %d", s->T, kMaxT);
    if (s->d_conv < 1) return fail(CV_EINVAL, "d_conv (%d) < 1", s->d_conv);
    if (s->d_conv < 2 || s->d_conv > 4)
        return fail(CV_ENOTSUP, "d_conv (%d) outside 2..4", s->d_conv);
    const int xb = dtype_bytes(s->x_dtype), sb = dtype_bytes(s->state_dtype);
    if (!xb || !sb) return fail(CV_EINVAL, "unknown dtype (x %d, state %d)", s->x_dtype, s->state_dtype);
    if (!((xb == 4 && sb == 4) || (xb == 2 && sb == 2) || (xb == 2 && sb == 4)))
        return fail(CV_ENOTSUP, "dtype pair (x f32, state bf16) is not supported");
    // channels and x/out strides come in 16-byte units of the x dtype, so every
    // wavefront's share of every buffer is a whole number of 16-byte chunks
    const int align = 16 / xb;
    const int cpl = cvimpl::kChannelsPerLane;
    if (s->d_inner % align)
        return fail(CV_ENOTSUP, "d_inner (%d) must be a multiple of %d", s->d_inner, align);
    if (s->qk_channels < 0 || s->qk_channels > s->d_inner)
        return fail(CV_EINVAL, "qk_channels (%d) outside 0..d_inner", s->qk_channels);
    int hl_log2 = 0, head_lanes = 0;
    if (s->qk_channels > 0) {
        if (s->head_dim <= 0) return fail(CV_EINVAL, "head_dim (%d) <= 0", s->head_dim);
        if (s->qk_channels % s->head_dim)
            return fail(CV_EINVAL, "qk_channels (%d) %% head_dim (%d) != 0", s->qk_channels,
                        s->head_dim);
        if (s->head_dim % cpl)
            return fail(CV_ENOTSUP, "head_dim (%d) must be a multiple of %d", s->head_dim, cpl);
        head_lanes = s->head_dim / cpl;
        if (head_lanes > kWave || (head_lanes & (head_lanes - 1)))
            return fail(CV_ENOTSUP, "head_dim / %d (%d) must be a power of two <= %d", cpl,
                        head_lanes, kWave);
        while ((1 << hl_log2) < head_lanes) ++hl_log2;
    }
    if (!std::isfinite(s->l2_eps) || s->l2_eps < 0.0f)
        return fail(CV_EINVAL, "l2_eps must be finite and >= 0");
    if (s->n_slots < 0) return fail(CV_EINVAL, "n_slots (%d) < 0", s->n_slots);
    const int W1 = s->d_conv - 1;
    if (s->state_len < W1)
        return fail(CV_EINVAL, "state_len (%d) < d_conv-1 (%d)", s->state_len, W1);
    if (s->x_seq_stride < 0 || s->x_tok_stride < 0 || s->out_seq_stride < 0 ||
        s->out_tok_stride < 0 || s->state_slot_stride < 0 || s->win_slot_stride < 0)
        return fail(CV_EINVAL, "negative stride");
    const int64_t C = s->d_inner;
    if (s->T > 1 && s->out_tok_stride < C)
        return fail(CV_EINVAL, "out_tok_stride (%lld) < d_inner: tokens of out overlap",
                    (long long)s->out_tok_stride);
    if (s->n_seq > 1 && s->out_seq_stride < (s->T - 1) * s->out_tok_stride + C)
        return fail(CV_EINVAL, "out_seq_stride (%lld) too small: rows of out overlap",
                    (long long)s->out_seq_stride);
    if (s->n_slots > 1 && s->state_slot_stride < C * s->state_len)
        return fail(CV_EINVAL, "state_slot_stride (%lld) < d_inner*state_len",
                    (long long)s->state_slot_stride);
    const int64_t win_per_slot =
        dedup ? C * (s->T + s->d_conv - 2) : (int64_t)s->T * C * W1;
    if (s->n_slots > 1 && s->win_slot_stride < win_per_slot)
        return fail(CV_EINVAL, "win_slot_stride (%lld) < %lld elements per slot",
                    (long long)s->win_slot_stride, (long long)win_per_slot);
    if (s->x_seq_stride % align || s->x_tok_stride % align || s->out_seq_stride % align ||
        s->out_tok_stride % align)
        return fail(CV_ENOTSUP, "x/out strides must be multiples of %d elements", align);
    if ((s->state_slot_stride * sb) % 16 || (s->win_slot_stride * sb) % 16)
        return fail(CV_ENOTSUP, "state/window slot strides must be multiples of 16 bytes");

    const int chw = kWave * cpl;
    const int64_t blocks = (C + chw - 1) / chw;
    const int64_t wg = blocks * (int64_t)s->n_seq;
    if (wg * kWave > (int64_t)UINT32_MAX)
        return fail(CV_ENOTSUP, "grid of %lld workgroups exceeds the launch limit", (long long)wg);
    int tb = 1;                                  // token buckets: 1 2 4 8 16 24 32
    while (tb < s->T && tb < 16) tb *= 2;
    if (tb < s->T) tb = s->T <= 24 ? 24 : 32;
    // LDS: the wavefront's conv_state region [channels, state_len] passes through first;
    // afterwards the same allocation holds the dedup tile (T+D-2 rows of the
    // wavefront's channels) or one or two dense snapshot slabs [channels, D-1].
    const int64_t region = (int64_t)kWave * cpl * s->state_len * sb;
    const int64_t later = dedup ? (int64_t)(s->T + s->d_conv - 2) * cvimpl::tile_pitch(sb)
                                : (int64_t)kWave * cpl * W1 * sb * (s->T > 1 ? 2 : 1);
    const int64_t lds = region > later ? region : later;
    if (lds > kMaxLds)
        return fail(CV_ENOTSUP, "kernel needs %lld bytes of LDS (> %d)", (long long)lds, kMaxLds);
    // Buffer resources span one row's bytes with a 32-bit size; lanes past d_inner use
    // the offset 2^31, so every span must stay below it.
    const int64_t lim = ((int64_t)1 << 31) - 16;
    const int64_t x_span = ((int64_t)(s->T - 1) * s->x_tok_stride + C) * xb;
    const int64_t o_span = ((int64_t)(s->T - 1) * s->out_tok_stride + C) * xb;
    const int64_t w_span = dedup ? C * (s->T + s->d_conv - 2) * sb : (int64_t)s->T * C * W1 * sb;
    const int64_t st_span = C * s->state_len * sb;
    if (x_span > lim || o_span > lim || w_span > lim || st_span > lim)
        return fail(CV_ENOTSUP, "a row spans more than 2 GiB (x %lld, out %lld, windows %lld, "
                                "state %lld bytes)", (long long)x_span, (long long)o_span,
                    (long long)w_span, (long long)st_span);

    plan->dedup = dedup;
    plan->x_bytes = xb;
    plan->state_bytes = sb;
    plan->d_conv = s->d_conv;
    plan->token_bucket = tb;
    plan->channels_per_lane = cpl;
    plan->channel_blocks = (int)blocks;
    plan->workgroups = wg;
    plan->lds_bytes = (int)lds;
    plan->head_lanes = head_lanes;
    (void)hl_log2;
    return CV_OK;
}

const void *pick_kernel(const cvimpl::Plan &plan) {
    using namespace cvimpl;
    const int xb = plan.x_bytes, sb = plan.state_bytes, d = plan.d_conv, tb = plan.token_bucket;
    if (xb == 4 && sb == 4) return plan.dedup ? pick_kernel_4_4_1(d, tb) : pick_kernel_4_4_0(d, tb);
    if (xb == 2 && sb == 2) return plan.dedup ? pick_kernel_2_2_1(d, tb) : pick_kernel_2_2_0(d, tb);
    if (xb == 2 && sb == 4) return plan.dedup ? pick_kernel_2_4_1(d, tb) : pick_kernel_2_4_0(d, tb);
    return nullptr;
}

// Enqueues the kernel; returns a hipError_t value (0 = success).
int launch(const cvimpl::Plan &plan, const cvimpl::KernelArgs &args, void *stream) {
    const void *fn = pick_kernel(plan);
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    cvimpl::KernelArgs a = args;
    void *kargs[] = {&a};
    return (int)hipLaunchKernel(fn, dim3((unsigned)plan.workgroups), dim3(cvimpl::kWave), kargs,
                                (size_t)plan.lds_bytes, (hipStream_t)stream);
}

int update(int dedup, const cv_shape_t *s, const void *x, const void *weight, const void *bias,
           void *conv_state, const int32_t *slot_idx, const int32_t *nat, void *out, void *win,
           void *stream) {
    g_detail[0] = 0;
    cvimpl::Plan plan;
    int rc = plan_shape(dedup, s, &plan);
    if (rc) return rc;
    if (s->n_seq == 0 || s->d_inner == 0) return CV_OK;   // nothing to do, nothing launched
    if (!x || !weight || !conv_state || !out || !win)
        return fail(CV_EINVAL, "NULL data pointer (x %p, weight %p, conv_state %p, out %p, "
                               "windows %p)", x, weight, conv_state, out, win);
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
    int hl_log2 = 0;
    while (plan.head_lanes && (1 << hl_log2) < plan.head_lanes) ++hl_log2;
    a.head_lanes_log2 = hl_log2;
    a.eps = s->l2_eps;
    int e = launch(plan, a, stream);
    if (e != 0)
        return fail(CV_EHIP_BASE - e, "kernel launch failed: %s",
                    hipGetErrorString(static_cast<hipError_t>(e)));
    return CV_OK;
}

}  // namespace

extern "C" {

int conv_verify_update_dense(const cv_shape_t *shape, const void *x, const void *weight,
                             const void *bias, void *conv_state, const int32_t *slot_idx,
                             const int32_t *num_accept_tokens, void *out, void *snapshots,
                             void *hip_stream) {
    return update(0, shape, x, weight, bias, conv_state, slot_idx, num_accept_tokens, out,
                  snapshots, hip_stream);
}

int conv_verify_update_dedup(const cv_shape_t *shape, const void *x, const void *weight,
                             const void *bias, void *conv_state, const int32_t *slot_idx,
                             const int32_t *num_accept_tokens, void *out, void *window_rows,
                             void *hip_stream) {
    return update(1, shape, x, weight, bias, conv_state, slot_idx, num_accept_tokens, out,
                  window_rows, hip_stream);
}

int conv_verify_describe(int dedup, const cv_shape_t *shape, cv_launch_info_t *info) {
    g_detail[0] = 0;
    if (!info) return fail(CV_EINVAL, "info is NULL");
    cvimpl::Plan plan;
    int rc = plan_shape(dedup, shape, &plan);
    if (rc) return rc;
    info->workgroups = plan.workgroups;
    info->threads = cvimpl::kWave;
    info->channel_blocks = plan.channel_blocks;
    info->channels_per_wave = cvimpl::kWave * plan.channels_per_lane;
    info->channels_per_lane = plan.channels_per_lane;
    info->token_bucket = plan.token_bucket;
    info->lds_bytes = plan.lds_bytes;
    info->head_lanes = plan.head_lanes;
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

}  // extern "C"
