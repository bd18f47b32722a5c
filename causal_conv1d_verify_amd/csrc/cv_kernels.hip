// HIP kernels (gfx950 / CDNA4) for the batched speculative-verify causal conv1d
// update: depthwise width-D conv over [conv_state window | x_0..x_{T-1}], SiLU,
// per-head L2 on the q|k channels, every per-token rollback window (dense or
// deduplicated), and the committed window back into conv_state, for all n_seq rows
// and all T draft positions in one launch.
//
// What the pages fix (Atlas docs, fn gdn_verify_fused_conv_kn_batched; sglang PR
// 46184, "Motivation" / "Modifications"; Atlas glm5next_kda/mod.rs,
// Glm5NextKdaConfig) is restated in include/conv_verify.h.  This file is the MI355X
// design of it:
//
//  * One 64-lane wavefront per workgroup.  Lane l owns CPL = 16 / sizeof(x element)
//    consecutive channels (8 for bf16, 4 for fp32), so every per-token load of x and
//    every store of out is one 16-byte access per lane and one contiguous 1 KiB span
//    per wavefront.  The grid is 1-D: n_seq * ceil(d_inner / (64 * CPL)) workgroups.
//  * The whole window sequence v[0 .. T+D-2] of the lane's channels lives in
//    registers: all T loads of x are issued before the first use, and the token loop
//    is unrolled over a compile-time bucket TB >= T so every register index is static.
//  * The conv is one fused multiply-add per tap in tap order (bias first), the same
//    order as the per-token path it replaces, so the pre-activation is bit-identical
//    to a correctly rounded fp32 evaluation of that order.
//  * L2: with head_dim = H and CPL channels per lane a head spans H / CPL lanes
//    (16 at H = 128, bf16), a power of two; the sum of squares is a butterfly over
//    those lanes with DPP (quad_perm, row_half_mirror, row_mirror inside a 16-lane
//    row; ds_swizzle / bpermute beyond).  Every lane of a head ends with the same sum.
//  * Dense snapshots: the lane's CPL x (D-1) window elements of token t are
//    contiguous in memory, so they leave as 16-byte stores assembled in registers.
//  * Dedup rows: the row [d_inner, T+D-2] of a slot is contiguous per wavefront;
//    each sequence position is written once into an LDS tile (16-byte conflict-free
//    writes), then the wavefront streams the tile out in row order with 16-byte,
//    fully coalesced stores.  Nothing is written per token and nothing twice.
//  * conv_state: when its rows are exactly D-1 wide the lane's window is one
//    contiguous run (16-byte loads/stores); with wider rows (an accept offset) the
//    D-1 elements per channel are moved one by one.
//  * Windows and conv_state move as bit patterns; only the conv reads them as floats.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cv_internal.h"

namespace cvimpl {
namespace {

// ---- bit-pattern helpers (compile-time channel indices) ------------------------------

// Element `e` of a packed word array of EB-byte elements, as raw bits.
template <int EB>
__device__ __forceinline__ uint32_t elem_bits(const uint32_t *w, int e) {
    if constexpr (EB == 4) {
        return w[e];
    } else {
        return (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
    }
}

// Element `e` as a float (bf16 widening is exact).
template <int EB>
__device__ __forceinline__ float elem_val(const uint32_t *w, int e) {
    if constexpr (EB == 4) {
        return __uint_as_float(w[e]);
    } else {
        return __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
    }
}

// x-element bits re-expressed in the state element type (bf16 -> fp32 is exact).
template <int XB, int SB>
__device__ __forceinline__ uint32_t x_to_state_bits(uint32_t xbits) {
    if constexpr (XB == SB) {
        return xbits;
    } else {
        static_assert(XB == 2 && SB == 4, "only bf16 -> fp32 widening");
        return xbits << 16;
    }
}

__device__ __forceinline__ float silu(float p) {
    // p * sigmoid(p); v_exp_f32 and v_rcp_f32.  For p << 0 the exponential
    // saturates to +inf and the result is -0.
    return p * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(p * -1.4426950408889634f));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 2^hl_log2 lanes of an aligned lane group (all lanes active).  Each
// step adds the two halves of a group symmetrically, so all lanes of a group hold
// the bit-identical sum.
__device__ __forceinline__ float group_sum(float v, int hl_log2) {
    if (hl_log2 >= 1) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    if (hl_log2 >= 2) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    if (hl_log2 >= 3) v += dpp<0x141>(v);   // row_half_mirror: other quad of the 8
    if (hl_log2 >= 4) v += dpp<0x140>(v);   // row_mirror: other half of the 16-lane row
    if (hl_log2 >= 5)                       // lane ^ 16 inside 32 (ds_swizzle xor mode)
        v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
    if (hl_log2 >= 6) v += __shfl_xor(v, 32);
    return v;
}

// ---- the kernel -------------------------------------------------------------------------

template <int XB, int SB, int D, int TB, bool DEDUP>
__global__ __launch_bounds__(kWave) void cv_verify_kernel(KernelArgs p) {
    constexpr int CPL = 16 / XB;          // channels per lane
    constexpr int CHW = kWave * CPL;      // channels per wavefront
    constexpr int W1 = D - 1;             // window columns
    constexpr int SW = CPL * SB / 4;      // 32-bit words per state-typed column
    constexpr int CHUNK_W = CPL * W1 * SB / 4;   // words of a lane's window run
    static_assert(CHUNK_W % 4 == 0, "window runs are whole 16-byte units");

    extern __shared__ uint4 lds_tile[];

    const int lane = threadIdx.x;
    const int row = (int)(blockIdx.x / (unsigned)p.channel_blocks);
    const int cb = (int)(blockIdx.x - (unsigned)row * (unsigned)p.channel_blocks) * CHW;

    const int slot = p.slot_idx ? p.slot_idx[row] : row;
    const int a = p.nat ? p.nat[row] : 0;
    // Padded rows (slot -1) leave before any store; rows with an index that would
    // address outside the buffers are skipped the same way.
    if (slot < 0 || slot >= p.n_slots || a < 0 || a > p.state_len - W1) return;

    const int T = p.T;
    const int c0 = cb + lane * CPL;
    const bool on = c0 < p.d_inner;

    // ---- issue every global load up front --------------------------------------------
    uint32_t X[TB][4];   // x_t for the lane's CPL channels (16 bytes each)
    {
        const char *xr = (const char *)p.x + ((int64_t)row * p.x_seq + c0) * XB;
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (t < T && on) v = *(const uint4 *)(xr + (int64_t)t * p.x_tok * XB);
            X[t][0] = v.x; X[t][1] = v.y; X[t][2] = v.z; X[t][3] = v.w;
        }
    }

    char *srow = (char *)p.state + (int64_t)slot * p.state_slot * SB;
    const bool contiguous_state = p.state_len == W1;
    uint32_t S[W1 > 0 ? W1 : 1][SW];   // initial window columns v[0..W1-1]
    if (contiguous_state) {
        uint32_t run[CHUNK_W];
#pragma unroll
        for (int q = 0; q < CHUNK_W / 4; ++q) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (on) v = *(const uint4 *)(srow + (int64_t)c0 * W1 * SB + 16 * q);
            run[4 * q] = v.x; run[4 * q + 1] = v.y; run[4 * q + 2] = v.z; run[4 * q + 3] = v.w;
        }
        // run holds [ch][j]; regroup into columns [j][ch]
#pragma unroll
        for (int j = 0; j < W1; ++j) {
#pragma unroll
            for (int w = 0; w < SW; ++w) {
                if constexpr (SB == 4) {
                    S[j][w] = elem_bits<4>(run, w * W1 + j);
                } else {
                    S[j][w] = elem_bits<2>(run, (2 * w) * W1 + j) |
                              (elem_bits<2>(run, (2 * w + 1) * W1 + j) << 16);
                }
            }
        }
    } else {
        const char *rec = srow + ((int64_t)c0 * p.state_len + a) * SB;
#pragma unroll
        for (int j = 0; j < W1; ++j) {
#pragma unroll
            for (int w = 0; w < SW; ++w) {
                if constexpr (SB == 4) {
                    S[j][w] = on ? *(const uint32_t *)(rec + ((int64_t)w * p.state_len + j) * 4) : 0u;
                } else {
                    uint32_t lo = on ? *(const uint16_t *)(rec + ((int64_t)(2 * w) * p.state_len + j) * 2) : 0u;
                    uint32_t hi = on ? *(const uint16_t *)(rec + ((int64_t)(2 * w + 1) * p.state_len + j) * 2) : 0u;
                    S[j][w] = lo | (hi << 16);
                }
            }
        }
    }

    float wv[CPL][D];
    float bv[CPL];
    {
        uint32_t wr[CPL * D * XB / 4];
#pragma unroll
        for (int q = 0; q < D; ++q) {   // CPL*D*XB bytes = 16*D
            uint4 v = make_uint4(0, 0, 0, 0);
            if (on) v = *(const uint4 *)((const char *)p.weight + (int64_t)c0 * D * XB + 16 * q);
            wr[4 * q] = v.x; wr[4 * q + 1] = v.y; wr[4 * q + 2] = v.z; wr[4 * q + 3] = v.w;
        }
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
            for (int w = 0; w < D; ++w) wv[ch][w] = elem_val<XB>(wr, ch * D + w);
        uint4 bb = make_uint4(0, 0, 0, 0);
        if (p.bias && on) bb = *(const uint4 *)((const char *)p.bias + (int64_t)c0 * XB);
        const uint32_t br[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) bv[ch] = elem_val<XB>(br, ch);
    }

    // v[k] accessors: k < W1 -> initial window, else x_{k-W1}.  k is compile-time.
    auto val = [&](int k, int ch) -> float {
        return k < W1 ? elem_val<SB>(S[k < W1 ? k : 0], ch)
                      : elem_val<XB>(X[k < W1 ? 0 : k - W1], ch);
    };
    auto sbits = [&](int k, int ch) -> uint32_t {
        return k < W1 ? elem_bits<SB>(S[k < W1 ? k : 0], ch)
                      : x_to_state_bits<XB, SB>(elem_bits<XB>(X[k < W1 ? 0 : k - W1], ch));
    };
    // The lane's CPL x (D-1) run of window v[k0 .. k0+W1-1] ([ch][j] order), packed.
    auto window_run = [&](int k0, uint32_t *run) {
#pragma unroll
        for (int w = 0; w < CHUNK_W; ++w) {
            if constexpr (SB == 4) {
                run[w] = sbits(k0 + w % W1, w / W1);
            } else {
                const int e0 = 2 * w, e1 = 2 * w + 1;
                run[w] = sbits(k0 + e0 % W1, e0 / W1) | (sbits(k0 + e1 % W1, e1 / W1) << 16);
            }
        }
    };
    // Column v[k] in the state type (SW words).
    auto column = [&](int k, uint32_t *col) {
#pragma unroll
        for (int w = 0; w < SW; ++w) {
            if constexpr (SB == 4) {
                col[w] = sbits(k, w);
            } else {
                col[w] = sbits(k, 2 * w) | (sbits(k, 2 * w + 1) << 16);
            }
        }
    };

    const int pitch = tile_pitch(CPL, SB);
    char *tile = (char *)lds_tile;
    if constexpr (DEDUP) {
        // tile row r holds v[r+1]; rows 0..W1-2 come from the initial window
#pragma unroll
        for (int k = 1; k < W1; ++k) {
            uint32_t col[SW];
            column(k, col);
#pragma unroll
            for (int q = 0; q < SW / 4; ++q)
                *(uint4 *)(tile + (k - 1) * pitch + lane * (CPL * SB) + 16 * q) =
                    make_uint4(col[4 * q], col[4 * q + 1], col[4 * q + 2], col[4 * q + 3]);
        }
    }

    const bool wave_l2 = cb < p.qk;    // uniform: this wavefront holds q|k channels
    const bool lane_l2 = c0 < p.qk;
    char *orow = (char *)p.out + ((int64_t)row * p.out_seq + c0) * XB;
    char *wbase = (char *)p.win + (int64_t)slot * p.win_slot * SB;

#pragma unroll
    for (int t = 0; t < TB; ++t) {
        if (t < T) {   // uniform guard; the loop itself is fully unrolled
            float y[CPL];
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) {
                float acc = bv[ch];
#pragma unroll
                for (int w = 0; w < D; ++w) acc = __builtin_fmaf(wv[ch][w], val(t + w, ch), acc);
                y[ch] = silu(acc);
            }
            if (wave_l2) {
                float ss = 0.0f;
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) ss = __builtin_fmaf(y[ch], y[ch], ss);
                ss = group_sum(ss, p.head_lanes_log2);
                const float sc = __builtin_amdgcn_rsqf(ss + p.eps);
                if (lane_l2) {
#pragma unroll
                    for (int ch = 0; ch < CPL; ++ch) y[ch] *= sc;
                }
            }
            if (on) {
                uint32_t o[4];
                if constexpr (XB == 4) {
#pragma unroll
                    for (int ch = 0; ch < 4; ++ch) o[ch] = __float_as_uint(y[ch]);
                } else {
                    typedef float f2 __attribute__((ext_vector_type(2)));
                    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        f2 pr = {y[2 * w], y[2 * w + 1]};
                        o[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, b2));
                    }
                }
                *(uint4 *)(orow + (int64_t)t * p.out_tok * XB) = make_uint4(o[0], o[1], o[2], o[3]);
            }

            if constexpr (!DEDUP) {
                // dense snapshot t = v[t+1 .. t+W1]: the lane's run is contiguous
                if (on) {
                    uint32_t run[CHUNK_W];
                    window_run(t + 1, run);
                    char *dst = wbase + ((int64_t)t * p.d_inner + c0) * W1 * SB;
#pragma unroll
                    for (int q = 0; q < CHUNK_W / 4; ++q)
                        *(uint4 *)(dst + 16 * q) =
                            make_uint4(run[4 * q], run[4 * q + 1], run[4 * q + 2], run[4 * q + 3]);
                }
            } else {
                // x_t is v[t+W1], tile row t+W1-1
                uint32_t col[SW];
                column(t + W1, col);
#pragma unroll
                for (int q = 0; q < SW / 4; ++q)
                    *(uint4 *)(tile + (t + W1 - 1) * pitch + lane * (CPL * SB) + 16 * q) =
                        make_uint4(col[4 * q], col[4 * q + 1], col[4 * q + 2], col[4 * q + 3]);
            }

            if (t == T - 1 && on) {
                // committed window v[T .. T+W1-1] -> conv_state columns 0..W1-1
                if (contiguous_state) {
                    uint32_t run[CHUNK_W];
                    window_run(t + 1, run);
                    char *dst = srow + (int64_t)c0 * W1 * SB;
#pragma unroll
                    for (int q = 0; q < CHUNK_W / 4; ++q)
                        *(uint4 *)(dst + 16 * q) =
                            make_uint4(run[4 * q], run[4 * q + 1], run[4 * q + 2], run[4 * q + 3]);
                } else {
                    char *rec = srow + (int64_t)c0 * p.state_len * SB;
#pragma unroll
                    for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
                        for (int j = 0; j < W1; ++j) {
                            const uint32_t b = sbits(t + 1 + j, ch);
                            if constexpr (SB == 4)
                                *(uint32_t *)(rec + ((int64_t)ch * p.state_len + j) * 4) = b;
                            else
                                *(uint16_t *)(rec + ((int64_t)ch * p.state_len + j) * 2) = (uint16_t)b;
                        }
                }
            }
        }
    }

    if constexpr (DEDUP) {
        // Stream the tile out in the row layout [c][k], k < L = T+W1-1, 16 bytes per lane.
        __syncthreads();
        constexpr int EPC = 16 / SB;   // elements per 16-byte chunk
        const int L = T + W1 - 1;
        const int nch = min(CHW, p.d_inner - cb);
        const int nchunks = nch * L / EPC;   // exact: nch is a multiple of CPL
        char *dst = wbase + (int64_t)cb * L * SB;
        int e0 = lane * EPC;
        int c = e0 / L;
        int k = e0 - c * L;
        const int step_c = (kWave * EPC) / L;
        const int step_k = (kWave * EPC) - step_c * L;
        for (int q = lane; q < nchunks; q += kWave) {
            uint32_t w[4];
            int cc = c, kk = k;
#pragma unroll
            for (int m = 0; m < EPC; ++m) {
                uint32_t b;
                if constexpr (SB == 4)
                    b = *(const uint32_t *)(tile + kk * pitch + cc * 4);
                else
                    b = *(const uint16_t *)(tile + kk * pitch + cc * 2);
                if constexpr (SB == 4) {
                    w[m] = b;
                } else {
                    if (m & 1) w[m >> 1] |= b << 16; else w[m >> 1] = b;
                }
                if (++kk == L) { kk = 0; ++cc; }
            }
            *(uint4 *)(dst + (int64_t)q * 16) = make_uint4(w[0], w[1], w[2], w[3]);
            c += step_c;
            k += step_k;
            if (k >= L) { k -= L; ++c; }
        }
    }
}

// ---- dispatch table -------------------------------------------------------------------

using KernelFn = void (*)(KernelArgs);

template <int XB, int SB, int D, bool DEDUP>
KernelFn pick_bucket(int tb) {
    switch (tb) {
        case 1: return cv_verify_kernel<XB, SB, D, 1, DEDUP>;
        case 2: return cv_verify_kernel<XB, SB, D, 2, DEDUP>;
        case 4: return cv_verify_kernel<XB, SB, D, 4, DEDUP>;
        case 8: return cv_verify_kernel<XB, SB, D, 8, DEDUP>;
        case 16: return cv_verify_kernel<XB, SB, D, 16, DEDUP>;
        case 32: return cv_verify_kernel<XB, SB, D, 32, DEDUP>;
        default: return nullptr;
    }
}

template <int XB, int SB, bool DEDUP>
KernelFn pick_d(int d, int tb) {
    switch (d) {
        case 2: return pick_bucket<XB, SB, 2, DEDUP>(tb);
        case 3: return pick_bucket<XB, SB, 3, DEDUP>(tb);
        case 4: return pick_bucket<XB, SB, 4, DEDUP>(tb);
        default: return nullptr;
    }
}

template <bool DEDUP>
KernelFn pick_types(int xb, int sb, int d, int tb) {
    if (xb == 4 && sb == 4) return pick_d<4, 4, DEDUP>(d, tb);
    if (xb == 2 && sb == 2) return pick_d<2, 2, DEDUP>(d, tb);
    if (xb == 2 && sb == 4) return pick_d<2, 4, DEDUP>(d, tb);
    return nullptr;
}

}  // namespace

int launch(const Plan &plan, const KernelArgs &args, void *stream) {
    KernelFn fn = plan.dedup ? pick_types<true>(plan.x_bytes, plan.state_bytes, plan.d_conv,
                                                plan.token_bucket)
                             : pick_types<false>(plan.x_bytes, plan.state_bytes, plan.d_conv,
                                                 plan.token_bucket);
    if (!fn) return (int)hipErrorInvalidDeviceFunction;
    KernelArgs a = args;
    void *kargs[] = {&a};
    hipError_t e = hipLaunchKernel((const void *)fn, dim3((unsigned)plan.workgroups), dim3(kWave),
                                   kargs, (size_t)plan.lds_bytes, (hipStream_t)stream);
    return (int)e;
}

}  // namespace cvimpl
