// Internal interface between the C-ABI layer (cv_api.cpp) and the HIP kernels
// (cv_kernels.hip).  Not installed, not part of the public ABI.
#pragma once

#include <stdint.h>

namespace cvimpl {

constexpr int kWave = 64;        // lanes per wavefront on CDNA; one wavefront per workgroup
constexpr int kChannelsPerLane = 4;   // 256 channels per wavefront
constexpr int kMaxT = 32;        // largest token bucket compiled
constexpr int kMaxLds = 65536;   // dynamic LDS a workgroup may request

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
    int64_t x_seq, x_tok, out_seq, out_tok, state_slot, win_slot;
    int32_t n_seq, T, d_inner, qk, n_slots, state_len;
    int32_t channel_blocks;    // workgroups per row
    int32_t head_lanes_log2;   // log2(lanes per L2 head); unused when qk == 0
    float eps;
};

// What the host decided to launch.
struct Plan {
    int dedup;                 // 0 dense, 1 dedup
    int x_bytes, state_bytes;  // element sizes: (4,4), (2,2) or (2,4)
    int d_conv;                // 2..4
    int token_bucket;          // 1,2,4,8,16,24,32 >= T
    int channels_per_lane;     // kChannelsPerLane
    int channel_blocks;
    int64_t workgroups;
    int lds_bytes;
    int head_lanes;
};

// Bytes between consecutive rows of the dedup LDS tile: one wavefront's channels of
// one sequence position, plus 16 bytes so successive rows start on different banks.
constexpr int tile_pitch(int state_bytes) {
    return kWave * kChannelsPerLane * state_bytes + 16;
}

// Kernel pickers, one per compiled (x bytes, state bytes, dedup) object: the kernel
// for (d_conv, token bucket), or nullptr.
const void *pick_kernel_4_4_0(int d_conv, int token_bucket);
const void *pick_kernel_4_4_1(int d_conv, int token_bucket);
const void *pick_kernel_2_2_0(int d_conv, int token_bucket);
const void *pick_kernel_2_2_1(int d_conv, int token_bucket);
const void *pick_kernel_2_4_0(int d_conv, int token_bucket);
const void *pick_kernel_2_4_1(int d_conv, int token_bucket);

}  // namespace cvimpl
