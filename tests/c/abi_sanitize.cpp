// Drives the host side of the C ABI (cv_api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer, linked with hip_host_stub.cpp instead of the device code
// and the HIP runtime (no GPU, no launch: the stub records what would be launched).
//
//  1. fixed cases: the kernel each entry point picks, its grid and LDS, and the launch
//     choices (token split, slot-first, XCD order) for the bench workloads' shapes;
//  2. refusals: every call that must fail returns its code and launches nothing;
//  3. a launch failure is reported with its code and detail;
//  4. a fuzz of random shapes over the whole int32 / int64 range of every field through
//     every entry point: a refused call launches nothing, an accepted one launches one
//     grid that fits the hardware limits.
//
// Prints one line per fixed check, "MISMATCH" on a failure, and exits non-zero then.
// Test code only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>

#include "conv_verify.h"
#include "cv_internal.h"

extern "C" {
struct stub_launch {
    int count;
    int code;
    unsigned grid_x, block_x;
    size_t lds;
    unsigned char args[512];
};
extern stub_launch g_stub_launch;
extern int g_stub_launch_result;   // a hipError_t
}

static int fails = 0;

static void expect(const char *what, long long got, long long want) {
    std::printf("%-58s %12lld (want %lld)%s\n", what, got, want, got == want ? "" : "  MISMATCH");
    if (got != want) fails = 1;
}

// fake device pointers: 16-byte aligned, never dereferenced on the host
static void *const A = reinterpret_cast<void *>(0x7f0000100000ull);
static const int32_t *const I = reinterpret_cast<const int32_t *>(0x7f0000200000ull);

// build: 0 regular, 1 lean (5 wavefronts per SIMD), 2 line-aligned (4-wavefront workgroups)
static int verify_code(int xb, int sb, int variant, int tm, int d_conv, int bucket_idx, int build,
                       int split) {
    return ((xb * 2 + sb / 2 - 3) & 7) << 9 | ((variant * 2 + tm) & 7) << 6 | (d_conv & 7) << 3 |
           (bucket_idx & 7) | (build == 1 ? 1 << 13 : 0) | (build == 2 ? 1 << 17 : 0) |
           (split ? 1 << 12 : 0);
}

static int64_t wmul(int64_t a, int64_t b);

static cv_shape_t shape(int n_seq, int T, int d, int qk, int state_len, int col, int layout) {
    cv_shape_t s;
    std::memset(&s, 0, sizeof s);
    s.n_seq = n_seq; s.T = T; s.d_inner = d; s.d_conv = 4;
    s.qk_channels = qk; s.head_dim = 128; s.l2_eps = 1e-6f;
    s.x_dtype = CV_BF16; s.state_dtype = CV_BF16; s.n_slots = n_seq; s.state_len = state_len;
    s.x_seq_stride = wmul(T, d); s.x_tok_stride = d;
    s.out_seq_stride = wmul(T, d); s.out_tok_stride = d;
    s.state_col_stride = col;
    s.state_slot_stride = col ? wmul(col, state_len) : wmul(d, state_len);
    s.win_slot_stride = layout == CV_WIN_DENSE ? wmul(wmul(T, d), 3) : wmul(d, (int64_t)T + 2);
    return s;
}

static const cvimpl::KernelArgs &kargs() {
    return *reinterpret_cast<const cvimpl::KernelArgs *>(g_stub_launch.args);
}

static void fixed_cases() {
    // the headline: 128 x 10240, T 8, dedup rows, one resident generation
    cv_shape_t s = shape(128, 8, 10240, 4096, 3, 0, CV_WIN_ROWS);
    int n0 = g_stub_launch.count;
    expect("headline: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("headline: one launch", g_stub_launch.count - n0, 1);
    expect("headline: kernel (bf16 rows, D 4, bucket 8)", g_stub_launch.code,
           verify_code(2, 2, 1, 0, 4, 3, 0, 0));
    expect("headline: grid", g_stub_launch.grid_x, 128 * 40);
    expect("headline: block", g_stub_launch.block_x, 64);
    expect("headline: slot-first off (one generation)", kargs().slot_first, 0);
    expect("headline: XCD order off (aligned rows)", kargs().xcd_remap, 0);
    expect("headline: head lanes log2", kargs().head_lanes_log2, 5);
    expect("headline: channel blocks", kargs().channel_blocks, 40);

    // heads of 96 channels (24 lanes): q|k in blocks of 2 whole heads (192 channels), then
    // 256-channel blocks from qk on; the segmented head sums (head_lanes_log2 -1)
    s = shape(128, 8, 10240, 96 * 40, 3, 0, CV_WIN_ROWS);
    s.head_dim = 96;
    expect("heads 96: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("heads 96: grid", g_stub_launch.grid_x, 128 * (20 + 25));
    expect("heads 96: head lanes log2", kargs().head_lanes_log2, -1);
    expect("heads 96: head lanes", kargs().heads.head_lanes, 24);
    expect("heads 96: q|k blocks", kargs().heads.qk_blocks, 20);
    expect("heads 96: q|k block channels", kargs().heads.qk_block_ch, 192);
    // the same at T 16 with a time-major state: not the line-aligned build
    s = shape(512, 16, 10240, 96 * 40, 18, 10240, CV_WIN_ROWS);
    s.head_dim = 96;
    expect("heads 96 T16 tm: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("heads 96 T16 tm: block", g_stub_launch.block_x, 64);
    expect("heads 96 T16 tm: grid", g_stub_launch.grid_x, 512 * 45);
    // power-of-two heads keep the uniform blocks
    s = shape(128, 8, 10240, 4096, 3, 0, CV_WIN_ROWS);
    expect("heads 128: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("heads 128: uniform blocks", kargs().heads.qk_blocks, 0);

    // the stress problem, conv_state time-major: 512 rows x T 16, 18-column state: the
    // line-aligned build (4-wavefront workgroups over 1024 channels)
    s = shape(512, 16, 10240, 4096, 18, 10240, CV_WIN_ROWS);
    expect("stress tm: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("stress tm: kernel (line-aligned 16-token build, tm state)", g_stub_launch.code,
           verify_code(2, 2, 1, 1, 4, 4, 2, 0));
    expect("stress tm: grid", g_stub_launch.grid_x, 512 * 10);
    expect("stress tm: block", g_stub_launch.block_x, 256);
    expect("stress tm: slot-first on (four generations)", kargs().slot_first, 1);
    expect("stress tm: LDS = 128 + the workgroup's row block", g_stub_launch.lds, 128 + 1024 * 18 * 2);
    expect("stress tm: nt stores", kargs().store_cached, 0);
    expect("stress tm: identity slots never wait", (conv_verify_update_dedup(&s, A, A, A, A, nullptr, I, A, A, nullptr), kargs().slot_first), 0);
    // with 8 tokens: the regular build, one wavefront per 256 channels
    s = shape(512, 8, 10240, 4096, 18, 10240, CV_WIN_ROWS);
    expect("stress tm T8: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("stress tm T8: kernel (regular build)", g_stub_launch.code, verify_code(2, 2, 1, 1, 4, 3, 0, 0));
    expect("stress tm T8: grid", g_stub_launch.grid_x, 512 * 40);
    expect("stress tm T8: block", g_stub_launch.block_x, 64);

    // channel-major 18-column state at d 10200 (rows of out off 128-byte lines): the
    // line-aligned build, LDS for the workgroup's state region after one line and the
    // exchange buffers after it
    s = shape(512, 16, 10200, 4096, 18, 0, CV_WIN_ROWS);
    expect("stress d10200: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("stress d10200: kernel (line-aligned build, channel-major state)", g_stub_launch.code,
           verify_code(2, 2, 1, 0, 4, 4, 2, 0));
    expect("stress d10200: grid", g_stub_launch.grid_x, 512 * 10);
    expect("stress d10200: block", g_stub_launch.block_x, 256);
    expect("stress d10200: XCD order (neighbouring workgroups share an L2)", kargs().xcd_remap, 1);
    expect("stress d10200: LDS = 128 + the workgroup's state region + 16 KiB", g_stub_launch.lds,
           128 + 1024 * 18 * 2 + 16384);
    expect("stress d10200: nt stores (channel-major state)", kargs().store_cached, 0);
    // ... the same with x and out on lines (token stride 10240): the state regions and row
    // blocks are still off them (slot strides of 10200 x 18 elements): line-aligned
    s.x_tok_stride = s.out_tok_stride = 10240;
    s.x_seq_stride = s.out_seq_stride = wmul(16, 10240);
    expect("stress d10200 strided: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("stress d10200 strided: block", g_stub_launch.block_x, 256);
    expect("stress d10200 strided: grid", g_stub_launch.grid_x, 512 * 10);
    // ... and with every store range on lines: one wavefront per 256 channels, the state
    // region in LDS, XCD order
    s.state_slot_stride = wmul(10240, 18);
    s.win_slot_stride = wmul(10240, 18);
    expect("stress d10200 all on lines: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("stress d10200 all on lines: grid", g_stub_launch.grid_x, 512 * 40);
    expect("stress d10200 all on lines: XCD order on", kargs().xcd_remap, 1);
    expect("stress d10200 all on lines: LDS = the state region", g_stub_launch.lds, 256 * 18 * 2);
    // ... and at d 10240, channel-major: the regular build
    s = shape(512, 16, 10240, 4096, 18, 0, CV_WIN_ROWS);
    expect("stress cm: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("stress cm: regular 16-token build", g_stub_launch.code, verify_code(2, 2, 1, 0, 4, 4, 0, 0));
    expect("stress cm: block", g_stub_launch.block_x, 64);
    // time-major state at d 10200, T 16: the line-aligned build (rows of out and the
    // row blocks start off 128-byte lines): 4-wavefront workgroups over 1024 channels,
    // LDS for the workgroup's row block [1024, 18] after up to 112 bytes of its first
    // line, every store streamed
    s = shape(512, 16, 10200, 4096, 18, 10240, CV_WIN_ROWS);
    expect("stress d10200 tm: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("stress d10200 tm: kernel (line-aligned build)", g_stub_launch.code,
           verify_code(2, 2, 1, 1, 4, 4, 2, 0));
    expect("stress d10200 tm: grid = rows x ceil(d / 1024)", g_stub_launch.grid_x, 512 * 10);
    expect("stress d10200 tm: block of 4 wavefronts", g_stub_launch.block_x, 256);
    expect("stress d10200 tm: workgroups per row", kargs().channel_blocks, 10);
    expect("stress d10200 tm: LDS = 128 + the workgroup's row block", g_stub_launch.lds, 128 + 1024 * 18 * 2);
    expect("stress d10200 tm: slot-first on (20,480 wavefronts)", kargs().slot_first, 1);
    expect("stress d10200 tm: no XCD order", kargs().xcd_remap, 0);
    expect("stress d10200 tm: nt stores", kargs().store_cached, 0);
    // ... but not with 15 tokens, packed rows or fp32 x
    s = shape(512, 15, 10200, 4096, 18, 10240, CV_WIN_ROWS);
    expect("d10200 tm T15: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("d10200 tm T15: regular build", g_stub_launch.code, verify_code(2, 2, 1, 1, 4, 4, 0, 0));
    expect("d10200 tm T15: XCD order on", kargs().xcd_remap, 1);
    expect("d10200 tm T15: default-policy stores", kargs().store_cached, 1);
    expect("d10200 tm T15: one wavefront per workgroup", g_stub_launch.block_x, 64);
    {
        s = shape(512, 16, 10200, 4096, 18, 10240, CV_WIN_ROWS);
        expect("d10200 tm packed: rc", conv_verify_update(&s, CV_WIN_ROWS, A, A, A, A, I, I, I, A, A, nullptr), CV_OK);
        expect("d10200 tm packed: one wavefront per workgroup", g_stub_launch.block_x, 64);
    }
    s = shape(512, 16, 10200, 4096, 18, 10240, CV_WIN_ROWS);
    s.x_dtype = CV_F32; s.state_dtype = CV_F32;
    s.state_slot_stride = 10240 * 18; s.win_slot_stride = 10200 * 18;
    expect("d10200 tm f32: rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("d10200 tm f32: one wavefront per workgroup", g_stub_launch.block_x, 64);
    s = shape(512, 8, 10240, 4096, 18, 10240, CV_WIN_ROWS);
    expect("stress tm T8 (aligned rows): rc", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_OK);
    expect("stress tm T8 (aligned rows): nt stores", kargs().store_cached, 0);

    // the K=17 GDN verify: dense windows on a small grid take the token-split kernel
    s = shape(8, 17, 8192, 4096, 3, 0, CV_WIN_DENSE);
    expect("gdn k17: rc", conv_verify_update_dense(&s, A, A, nullptr, A, nullptr, nullptr, A, A, nullptr), CV_OK);
    expect("gdn k17: split kernel", (g_stub_launch.code >> 14) & 7, 1);
    expect("gdn k17: grid = rows x blocks x ceil(T/4)", g_stub_launch.grid_x, 8 * 32 * 5);
    expect("gdn k17: token chunks", kargs().token_chunks, 5);

    // the tree at the same shape spreads its 4-token chunks too
    s = shape(8, 17, 8192, 4096, 3, 0, CV_WIN_DENSE);
    expect("tree k17: rc", conv_verify_update_tree(&s, A, A, nullptr, A, nullptr, nullptr, nullptr, I, A, A, nullptr), CV_OK);
    expect("tree k17: kernel (tree variant, bucket 24)", g_stub_launch.code & 0xFFF,
           verify_code(2, 2, 3, 0, 4, 5, 0, 0) & 0xFFF);
    expect("tree k17: grid", g_stub_launch.grid_x, 8 * 32 * 5);

    // KDA T 1 with an fp32 state
    s = shape(256, 1, 12288, 8192, 3, 0, CV_WIN_DENSE);
    s.state_dtype = CV_F32;
    expect("kda: rc", conv_verify_update_dense(&s, A, A, nullptr, A, nullptr, nullptr, A, A, nullptr), CV_OK);
    expect("kda: kernel (bf16 x, f32 state, bucket 1)", g_stub_launch.code,
           verify_code(2, 4, 0, 0, 4, 0, 0, 0));
    expect("kda: grid", g_stub_launch.grid_x, 256 * 48);

    // restore, prefill and the separate L2
    s = shape(512, 16, 10240, 4096, 18, 10240, CV_WIN_ROWS);
    expect("restore: rc", conv_verify_restore(&s, CV_WIN_ROWS, A, A, I, I, nullptr), CV_OK);
    expect("restore: family", g_stub_launch.code >> 14, 2);
    expect("restore: grid", g_stub_launch.grid_x, 512 * 40);
    expect("restore: LDS = the rows block", g_stub_launch.lds, (256 * 18 * 2 + 1023) / 1024 * 1024);
    s = shape(512, 16, 10240, 4096, 18, 10240, CV_WIN_ROWS_T);
    expect("restore from time-major rows: rc", conv_verify_restore(&s, CV_WIN_ROWS_T, A, A, I, I, nullptr), CV_OK);
    expect("restore from time-major rows: grid", g_stub_launch.grid_x, 512 * 40);
    expect("restore from time-major rows: no LDS", g_stub_launch.lds, 0);
    s = shape(8, 2048, 10240, 4096, 3, 0, CV_WIN_DENSE);
    expect("prefill: rc", conv_prefill(&s, A, A, nullptr, A, nullptr, I, nullptr, A, nullptr), CV_OK);
    expect("prefill: family", g_stub_launch.code >> 14, 3);
    expect("prefill: grid = rows x chunks x blocks", g_stub_launch.grid_x, 8 * 128 * 40);
    expect("l2: rc", conv_qk_l2norm(&s, 12345, 10240, A, nullptr), CV_OK);
    expect("l2: family", g_stub_launch.code >> 14, 4);
    expect("l2: grid = row pairs x q|k blocks", g_stub_launch.grid_x, (12345 + 1) / 2 * 16);
}

static void refusals() {
    struct Case {
        const char *what;
        void (*mut)(cv_shape_t *);
        int code;
    };
    static const Case cases[] = {
        {"T 0", [](cv_shape_t *s) { s->T = 0; }, CV_EINVAL},
        {"T 33", [](cv_shape_t *s) { s->T = 33; }, CV_ENOTSUP},
        {"d_conv 5", [](cv_shape_t *s) { s->d_conv = 5; }, CV_ENOTSUP},
        {"d_conv 0", [](cv_shape_t *s) { s->d_conv = 0; }, CV_EINVAL},
        {"n_seq -1", [](cv_shape_t *s) { s->n_seq = -1; }, CV_EINVAL},
        {"d_inner not a multiple of 8", [](cv_shape_t *s) { s->d_inner = 1028; }, CV_ENOTSUP},
        {"qk % head_dim", [](cv_shape_t *s) { s->qk_channels = 1000; }, CV_EINVAL},
        {"head_dim 132", [](cv_shape_t *s) { s->head_dim = 132; s->qk_channels = 396; }, CV_ENOTSUP},
        {"head_dim 12, qk 36", [](cv_shape_t *s) { s->head_dim = 12; s->qk_channels = 36; }, CV_ENOTSUP},
        {"head_dim 260", [](cv_shape_t *s) { s->head_dim = 260; s->qk_channels = 520; }, CV_ENOTSUP},
        {"qk > d", [](cv_shape_t *s) { s->qk_channels = s->d_inner + 128; }, CV_EINVAL},
        {"eps NaN", [](cv_shape_t *s) { s->l2_eps = __builtin_nanf(""); }, CV_EINVAL},
        {"eps < 0", [](cv_shape_t *s) { s->l2_eps = -1.0f; }, CV_EINVAL},
        {"dtype pair (f32, bf16)", [](cv_shape_t *s) { s->x_dtype = CV_F32; }, CV_ENOTSUP},
        {"unknown dtype", [](cv_shape_t *s) { s->state_dtype = 7; }, CV_EINVAL},
        {"state_len < d_conv-1", [](cv_shape_t *s) { s->state_len = 2; }, CV_EINVAL},
        {"state slot stride short", [](cv_shape_t *s) { s->state_slot_stride -= 8; }, CV_EINVAL},
        {"window slot stride short", [](cv_shape_t *s) { s->win_slot_stride -= 8; }, CV_EINVAL},
        {"out tokens overlap", [](cv_shape_t *s) { s->out_tok_stride = 8; }, CV_EINVAL},
        {"x stride not 16-byte", [](cv_shape_t *s) { s->x_tok_stride += 4; }, CV_ENOTSUP},
        {"state columns overlap", [](cv_shape_t *s) { s->state_col_stride = s->d_inner - 8; }, CV_EINVAL},
        {"state column stride not 16-byte", [](cv_shape_t *s) { s->state_col_stride = s->d_inner + 4; s->state_slot_stride = (int64_t)(s->d_inner + 4) * 3 + 8; }, CV_ENOTSUP},
        {"state region past 160 KiB of LDS", [](cv_shape_t *s) { s->state_len = 400; s->state_slot_stride = (int64_t)s->d_inner * 400; }, CV_ENOTSUP},
        {"identity slots, too few", [](cv_shape_t *s) { s->n_slots = s->n_seq - 1; }, CV_EINVAL},
    };
    for (const Case &c : cases) {
        cv_shape_t s = shape(16, 8, 1024, 512, 3, 0, CV_WIN_ROWS);
        c.mut(&s);
        const int n0 = g_stub_launch.count;
        char what[96];
        std::snprintf(what, sizeof what, "refused: %s", c.what);
        expect(what, conv_verify_update_dedup(&s, A, A, A, A, nullptr, nullptr, A, A, nullptr), c.code);
        expect("  nothing launched", g_stub_launch.count - n0, 0);
        expect("  detail set", std::strlen(conv_verify_last_error()) > 0, 1);
    }
    cv_shape_t s = shape(16, 8, 1024, 512, 3, 0, CV_WIN_ROWS);
    const int n0 = g_stub_launch.count;
    expect("refused: NULL shape", conv_verify_update_dedup(nullptr, A, A, A, A, I, I, A, A, nullptr), CV_EINVAL);
    expect("refused: NULL x", conv_verify_update_dedup(&s, nullptr, A, A, A, I, I, A, A, nullptr), CV_EINVAL);
    expect("refused: misaligned out", conv_verify_update_dedup(&s, A, A, A, A, I, I, (char *)A + 8, A, nullptr), CV_ENOTSUP);
    expect("refused: unknown layout", conv_verify_update(&s, 7, A, A, A, A, I, I, nullptr, A, A, nullptr), CV_EINVAL);
    expect("refused: tree without parents", conv_verify_update_tree(&s, A, A, A, A, I, I, nullptr, nullptr, A, A, nullptr), CV_EINVAL);
    expect("refused: restore without indices", conv_verify_restore(&s, CV_WIN_ROWS, A, A, I, nullptr, nullptr), CV_EINVAL);
    expect("refused: prefill without cu_seqlens", conv_prefill(&s, A, A, A, A, I, nullptr, I, A, nullptr), CV_EINVAL);
    expect("refused: l2 with row_stride < qk", conv_qk_l2norm(&s, 4, 256, A, nullptr), CV_EINVAL);
    expect("refused calls launched nothing", g_stub_launch.count - n0, 0);
    expect("empty batch: no pointers needed", conv_verify_update_dedup(&(s.n_seq = 0, s), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), CV_OK);
    expect("  and nothing launched", g_stub_launch.count - n0, 0);
}

static void launch_failure() {
    cv_shape_t s = shape(16, 8, 1024, 512, 3, 0, CV_WIN_ROWS);
    g_stub_launch_result = 1;   // hipErrorInvalidValue
    expect("launch failure: code", conv_verify_update_dedup(&s, A, A, A, A, I, I, A, A, nullptr), CV_EHIP_BASE - 1);
    expect("  strerror names it", std::strstr(conv_verify_strerror(CV_EHIP_BASE - 1), "launch") != nullptr, 1);
    expect("  detail set", std::strlen(conv_verify_last_error()) > 0, 1);
    g_stub_launch_result = 0;
}

// ---- fuzz -------------------------------------------------------------------------------

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next() {   // xorshift64*
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}
static int32_t pick32(std::initializer_list<int32_t> common) {
    const uint64_t r = next();
    switch (r % 16) {
        case 0: return (int32_t)(uint32_t)(r >> 32);                                  // anything
        case 1: return (int32_t)((r >> 32) % 65536) - 8;                              // small
        case 2: return r & 64 ? INT32_MAX - (int32_t)((r >> 40) % 4) : INT32_MIN + (int32_t)((r >> 40) % 4);
        default: return *(common.begin() + (r >> 20) % common.size());
    }
}
static int64_t pick64(int64_t base) {
    const uint64_t r = next();
    switch (r % 16) {
        case 0: return (int64_t)r;
        case 1: return (int64_t)((uint64_t)base + (r >> 32) % 64 - 32);
        case 2: return r & 64 ? INT64_MAX - (int64_t)((r >> 40) % 4) : INT64_MIN;
        default: return base;
    }
}

// products that may wrap (the fuzz's own base values; the library sees only the result)
static int64_t wmul(int64_t a, int64_t b) { return (int64_t)((uint64_t)a * (uint64_t)b); }

static void fuzz(int iters) {
    long long accepted = 0, refused = 0, la = 0;
    for (int it = 0; it < iters; ++it) {
        cv_shape_t s = shape(pick32({1, 7, 64, 128, 512, 4096}), pick32({1, 2, 3, 8, 16, 17, 24, 32}),
                             pick32({8, 256, 1032, 10200, 10240}), 0, 3, 0, CV_WIN_ROWS);
        s.qk_channels = pick32({0, 128, 512, 4096});
        s.head_dim = pick32({4, 8, 64, 128, 256, 96});
        s.d_conv = pick32({2, 3, 4});
        s.state_len = pick32({1, 2, 3, 8, 18, 120});
        s.n_slots = pick32({s.n_seq, (int32_t)((uint32_t)s.n_seq + 1u), 0});
        s.x_dtype = pick32({CV_BF16, CV_F32});
        s.state_dtype = pick32({CV_BF16, CV_F32});
        s.l2_eps = (next() & 7) == 0 ? -1.0f : 1e-6f;
        const int64_t d = s.d_inner;
        s.x_tok_stride = pick64(d);
        s.x_seq_stride = pick64(wmul(s.T, d));
        s.out_tok_stride = pick64(d);
        s.out_seq_stride = pick64(wmul(s.T, d));
        s.state_col_stride = (next() & 1) ? 0 : pick64(d);
        s.state_slot_stride = pick64(s.state_col_stride ? wmul(s.state_col_stride, s.state_len)
                                                        : wmul(d, s.state_len));
        s.win_slot_stride = pick64(wmul(wmul(d, (int64_t)s.T + 2), 3));
        const int layout = (int)(next() % 13) / 4;   // 3 (rarely): an unknown layout
        const int n0 = g_stub_launch.count;
        int rc;
        const uint64_t which = next() % 7;
        cv_launch_info_t info;
        switch (which) {
            case 0: rc = conv_verify_update(&s, layout, A, A, A, A, I, I, nullptr, A, A, nullptr); break;
            case 1: rc = conv_verify_update(&s, layout, A, A, nullptr, A, I, I, I, A, A, nullptr); break;
            case 2: rc = conv_verify_update_tree(&s, A, A, A, A, I, I, nullptr, I, A, A, nullptr); break;
            case 3: rc = conv_verify_restore(&s, layout, A, A, I, I, nullptr); break;
            case 4: rc = conv_prefill(&s, A, A, A, A, I, I, I, A, nullptr); break;
            case 5: rc = conv_qk_l2norm(&s, pick64(100), pick64(d), A, nullptr); break;
            default: rc = conv_verify_describe(layout, &s, &info); break;
        }
        const int launched = g_stub_launch.count - n0;
        if (rc != CV_OK && rc != CV_EINVAL && rc != CV_ENOTSUP) {
            std::printf("fuzz %d: unexpected code %d  MISMATCH\n", it, rc);
            fails = 1;
        }
        if (rc != CV_OK && launched) {
            std::printf("fuzz %d: refused (%d) but launched  MISMATCH\n", it, rc);
            fails = 1;
        }
        if (rc == CV_OK && which != 6 && launched > 1) {
            std::printf("fuzz %d: %d launches  MISMATCH\n", it, launched);
            fails = 1;
        }
        if (launched && ((uint64_t)g_stub_launch.grid_x * 64 > UINT32_MAX || g_stub_launch.grid_x == 0 ||
                         g_stub_launch.lds > (size_t)cvimpl::kMaxLds || g_stub_launch.code < 0)) {
            std::printf("fuzz %d: launch outside the limits (grid %u, lds %zu, code %d)  MISMATCH\n", it,
                        g_stub_launch.grid_x, g_stub_launch.lds, g_stub_launch.code);
            fails = 1;
        }
        // the line-aligned build (and only it) takes 4-wavefront workgroups, for bf16 x and
        // state, dedup rows and 16 tokens (not split or packed; a channel-major state only
        // with a store range off lines); its grid covers each (row, 1024 channels) once and
        // its LDS holds a row block (and a channel-major state's region) after one line
        const bool la_code = launched && g_stub_launch.code >= 0 && (g_stub_launch.code & (1 << 17));
        if (launched && (g_stub_launch.block_x != 64 && g_stub_launch.block_x != 256)) {
            std::printf("fuzz %d: block %u  MISMATCH\n", it, g_stub_launch.block_x);
            fails = 1;
        }
        if (launched && la_code != (g_stub_launch.block_x == 256)) {
            std::printf("fuzz %d: line-aligned kernel with block %u  MISMATCH\n", it, g_stub_launch.block_x);
            fails = 1;
        }
        if (la_code && (s.x_dtype != CV_BF16 || s.state_dtype != CV_BF16 || s.T != 16 ||
                        (s.state_col_stride == 0 && s.out_tok_stride % 64 == 0 &&
                         (s.n_seq == 1 || s.out_seq_stride % 64 == 0) &&
                         (s.n_slots <= 1 ||
                          (s.state_slot_stride % 64 == 0 && s.win_slot_stride % 64 == 0))) ||
                        (s.state_col_stride == 0 &&
                         (g_stub_launch.lds < (size_t)(128 + 1024 * s.state_len * 2 + 16384) ||
                          g_stub_launch.lds * 3 > (size_t)cvimpl::kMaxLds)) ||
                        layout != CV_WIN_ROWS || which > 1 ||
                        (s.qk_channels > 0 && ((s.head_dim / 4) & (s.head_dim / 4 - 1))) ||
                        g_stub_launch.grid_x != (uint64_t)s.n_seq * ((d + 1023) / 1024) ||
                        g_stub_launch.lds < (size_t)(128 + 1024 * (s.T + s.d_conv - 2) * 2))) {
            std::printf("fuzz %d: line-aligned launch of an unexpected shape  MISMATCH\n", it);
            fails = 1;
        }
        (rc == CV_OK ? accepted : refused)++;
        la += la_code;
    }
    std::printf("fuzz: %d shapes, %lld accepted, %lld refused, %lld line-aligned\n", iters, accepted,
                refused, la);
}

int main(int argc, char **argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 200000;
    expect("abi version", conv_verify_abi_version(), CONV_VERIFY_ABI_VERSION);
    fixed_cases();
    refusals();
    launch_failure();
    fuzz(iters);
    std::printf(fails ? "FAILED\n" : "ALL OK\n");
    return fails;
}
