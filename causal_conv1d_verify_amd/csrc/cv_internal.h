// Internal interface between the C-ABI layer (cv_api.cpp) and the HIP kernels
// (cv_kernels.hip).  Not installed, not part of the public ABI.
#pragma once

#include <stdint.h>

namespace cvimpl {

constexpr int kWave = 64;        // lanes per wavefront on CDNA; one wavefront per workgroup
constexpr int kChannelsPerLane = 4;   // 256 channels per wavefront
constexpr int kMaxT = 32;        // largest token bucket compiled
// dynamic LDS a workgroup may request: gfx950 has 160 KiB of LDS per compute unit and
// one workgroup may take all of it
constexpr int kMaxLds = 163840;

// Rollback-window layouts.
enum WinLayout { kDense = 0, kRows = 1, kRowsT = 2 };

// Per-head L2 geometry shared by the kernels that normalise q|k.  A head of head_lanes
// lanes (head_dim / kChannelsPerLane) that is a power of two tiles every 256-channel
// wavefront, and the channel blocks are uniform: block b starts at channel b * 256.  A
// head of any other size would straddle wavefronts, so there the q|k channels go in
// qk_blocks blocks of qk_block_ch channels (a whole number of heads, at most 256, the
// last block possibly shorter), and the channels from qk on in 256-channel blocks after
// them.  qk_blocks == 0 selects the uniform blocks.
struct HeadBlocks {
    int32_t head_lanes;        // lanes per head (head_dim / kChannelsPerLane)
    int32_t qk_blocks;         // blocks of whole heads; 0: uniform 256-channel blocks
    int32_t qk_block_ch;       // channels per such block
};

// Kernel arguments, by value.  Strides are in elements.
struct KernelArgs {
    const void *x;
    const void *weight;
    const void *bias;          // nullable
    void *state;
    const int32_t *slot_idx;   // nullable
    const int32_t *nat;        // nullable (num_accept_tokens)
    void *out;
    void *win;                 // dense snapshots or dedup rows
    const int32_t *cu;         // nullable: packed rows, [n_seq+1] token offsets
    const int32_t *parent;     // tree: [n_seq, T] parent positions (-1: the row's start)
    int64_t x_seq, x_tok, out_seq, out_tok, state_slot, win_slot;
    int32_t n_seq, T, d_inner, qk, n_slots, state_len;
    int32_t channel_blocks;    // workgroups per row
    int32_t head_lanes_log2;   // log2(lanes per L2 head), -1 when that is not a power of
                               // two; unused when qk == 0
    float eps;
    int32_t token_chunks;      // token-split verify: workgroups per (row, channel block)
    int64_t state_col;         // 0: conv_state channel-major; else time-major column stride
    int32_t slot_first;        // read the slot before any vector load (padded rows load nothing)
    int32_t xcd_remap;         // work index from xcd_linear(blockIdx): a row's blocks on one XCD
    int32_t store_cached;      // time-major builds: stores with the default cache policy
    HeadBlocks heads;          // L2 head size and the channel blocks of q|k
};

// A launch of more wavefronts than the chip holds at once (256 CUs x 4 SIMDs x 5) runs
// in generations: there a wavefront waits for its row's slot before loading x, so the
// x of padded rows is never read; a launch that fits in one generation issues x first.
constexpr int64_t kResidentWaves = 5120;

// The rows layout's compile-time-length path stages a wavefront's row block in LDS in
// halves when the block is larger than this: 8 KiB per wavefront leaves LDS for 20
// resident wavefronts per compute unit (5 per SIMD).
constexpr int kRowsStageBytes = 8192;

// Wavefronts per workgroup of the line-aligned build (1024 consecutive channels), and
// the most LDS it may take with a channel-major state: 3 workgroups per compute unit
// (LDS is allocated in 512-byte units).
constexpr int kLineGroupWaves = 4;
constexpr int kLineGroupMaxLds = kMaxLds / 3 / 512 * 512;

// Token-split verify (dense windows): tokens per wavefront, and the grids it serves:
// at most kSplitMaxWaves wavefronts once split (measured at d 8192: T 8 gains up to 64
// rows, T 17 up to 32 rows, e.g. 10.4 -> 5.8 us at 8 rows; larger splits ran slower).
// Tree verify splits grids of fewer than kTreeSplitBelowWaves one-row wavefronts.
constexpr int kSplitChunk = 4;
constexpr int64_t kSplitMaxWaves = 5120;
constexpr int64_t kTreeSplitBelowWaves = 1024;
// Row layouts split a row's 4-token chunks (buckets 8 and 16) when the split grid has at
// most this many wavefronts (chunk 0 keeps the copies, since a row block is shared by
// all tokens).  Measured at d 10240: T 8 gains up to 32 rows (5.9 -> 5.1 us at 8 rows),
// T 16 up to 16 rows (8.2 -> 6.5 us at 8 rows); larger splits ran slower.
constexpr int64_t kRowsSplitMaxWaves = 2560;

// What the host decided to launch.
struct Plan {
    int layout;                // WinLayout
    int tree;                  // per-token parents (dense windows)
    int x_bytes, state_bytes;  // element sizes: (4,4), (2,2) or (2,4)
    int d_conv;                // 2..4
    int token_bucket;          // 1,2,4,8,16,24,32 >= T; kSplitChunk when split
    int token_chunks;          // wavefronts per (row, channel block) along T
    int lean;                  // 16-token bucket built for 5 wavefronts per SIMD
    int state_tm;              // conv_state time-major (the kernels' TM build)
    int slot_first;            // KernelArgs::slot_first when a slot table is passed
    int xcd_remap;             // KernelArgs::xcd_remap
    int channels_per_lane;     // kChannelsPerLane
    int channel_blocks;        // workgroups per row (each of waves_per_group wavefronts)
    int64_t workgroups;
    int lds_bytes;
    int head_lanes;
    int hl_log2;               // log2(head_lanes), -1 when not a power of two
    HeadBlocks heads;
    int waves_per_group;       // 1, or kLineGroupWaves for the line-aligned build
};

// Accepted-prefix restore: window widx[i] of row i's slot -> conv_state columns 0..D-2.
struct RestoreArgs {
    void *state;
    const void *win;
    const int32_t *slot_idx;   // nullable
    const int32_t *widx;       // [n_seq] window index per row (-1: nothing)
    int64_t state_slot, win_slot;
    int32_t n_seq, T, d_inner, n_slots, state_len;
    int32_t channel_blocks;
    int64_t state_col;         // 0: conv_state channel-major; else time-major column stride
};

// Prefill conv over packed prompts (conv + SiLU, no L2, no windows).
#ifndef CV_PREFILL_CHUNK
#define CV_PREFILL_CHUNK 16
#endif
constexpr int kPrefillChunk = CV_PREFILL_CHUNK;   // tokens per wavefront
struct PrefillArgs {
    const void *x;
    const void *weight;
    const void *bias;          // nullable
    void *state;
    const int32_t *slot_idx;   // nullable
    const int32_t *cu;         // [n_seq+1]
    const int32_t *has_init;   // nullable
    void *out;
    int64_t x_tok, out_tok, state_slot;
    int32_t n_seq, T, d_inner, n_slots, state_len;
    int32_t channel_blocks;
    int32_t chunks;            // token chunks per row: ceil(T / kPrefillChunk)
    int64_t state_col;         // 0: conv_state channel-major; else time-major column stride
};

// Separate per-head L2 over the q|k channels of token rows, in place.
struct L2Args {
    void *x;
    int64_t row_stride;
    int64_t n_rows;
    int32_t qk, qk_blocks, head_lanes_log2;   // qk_blocks: channel blocks per row
    float eps;
    HeadBlocks heads;          // as in KernelArgs (uniform: qk_blocks == 0)
};
// Token rows per wavefront of the separate L2.  On the prefill batch (12.4k rows of
// 4096 q|k channels) 1, 2, 4 and 8 rows measured 44.4, 35.6, 38.5 and 41.8 us.
constexpr int kL2Rows = 2;

// Bytes between consecutive rows of the dedup LDS tile: one wavefront's channels of
// one sequence position, plus 16 bytes so successive rows start on different banks.
constexpr int tile_pitch(int state_bytes) {
    return kWave * kChannelsPerLane * state_bytes + 16;
}

// LDS bytes to reserve for a block of `bytes` filled by direct global->LDS loads: each
// such load instruction writes kWave 16-byte chunks, whole, so the span is rounded up
// to a multiple of kWave * 16.
constexpr int64_t lds_dma_span(int64_t bytes) {
    return (bytes + kWave * 16 - 1) / (kWave * 16) * (kWave * 16);
}

// The write-count build only (a test library, compiled with CV_WRITE_COUNT): device
// ranges whose stores are counted, one 32-bit counter per 2 bytes of each range.
struct CountRanges {
    int32_t n;                 // ranges in use, 0..4
    const char *lo[4];
    uint64_t bytes[4];
    uint32_t *counts[4];
};
// Each code object holds its own copy of the ranges; these set it (write-count build,
// which compiles the verify objects for bf16 x and state only, and the aux object).
#define CV_DECLARE_COUNT_SET(v, tm) int count_ranges_set_2_2_##v##_##tm(const CountRanges &c);
CV_DECLARE_COUNT_SET(0, 0) CV_DECLARE_COUNT_SET(1, 0) CV_DECLARE_COUNT_SET(2, 0) CV_DECLARE_COUNT_SET(3, 0)
CV_DECLARE_COUNT_SET(0, 1) CV_DECLARE_COUNT_SET(1, 1) CV_DECLARE_COUNT_SET(2, 1) CV_DECLARE_COUNT_SET(3, 1)
#undef CV_DECLARE_COUNT_SET
int count_ranges_set_aux(const CountRanges &c);

// Kernel pickers, one per compiled (x bytes, state bytes, variant, state layout)
// object - variant 0 dense, 1 rows, 2 time-major rows, 3 tree; state layout 0
// channel-major, 1 time-major: the kernel for (d_conv, token bucket), or nullptr.
// build: 0 the regular build; 1 the 16-token bucket's build for 5 resident wavefronts per
// SIMD (lean); 2 the line-aligned build of kLineGroupWaves-wavefront workgroups (bf16,
// time-major state, row layout, 16 tokens).  split: the row layouts' token-split build
// (buckets 8 and 16).
#define CV_DECLARE_PICKERS_TM(xb, sb, tm)                                   \
    const void *pick_kernel_##xb##_##sb##_0_##tm(int d_conv, int token_bucket, int build, int split); \
    const void *pick_kernel_##xb##_##sb##_1_##tm(int d_conv, int token_bucket, int build, int split); \
    const void *pick_kernel_##xb##_##sb##_2_##tm(int d_conv, int token_bucket, int build, int split); \
    const void *pick_kernel_##xb##_##sb##_3_##tm(int d_conv, int token_bucket, int lean, int split);
#define CV_DECLARE_PICKERS(xb, sb) CV_DECLARE_PICKERS_TM(xb, sb, 0) CV_DECLARE_PICKERS_TM(xb, sb, 1)
CV_DECLARE_PICKERS(4, 4)
CV_DECLARE_PICKERS(2, 2)
CV_DECLARE_PICKERS(2, 4)
#undef CV_DECLARE_PICKERS
#undef CV_DECLARE_PICKERS_TM

// The kernels below take the state layout at compile time the same way (tm: 1 for a
// time-major conv_state).
const void *pick_restore(int state_bytes, int d_conv, int layout, int tm);
const void *pick_split(int x_bytes, int state_bytes, int d_conv, int tm);
const void *pick_prefill(int x_bytes, int state_bytes, int d_conv, int tm);
const void *pick_l2(int x_bytes);

}  // namespace cvimpl
