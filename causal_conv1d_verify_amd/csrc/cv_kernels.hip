// HIP kernels (gfx950 / CDNA4) for the batched speculative-verify causal conv1d
// update: depthwise width-D conv over [conv_state window | x_0..x_{T-1}], SiLU,
// per-head L2 on the q|k channels, every per-token rollback window (dense or
// deduplicated), and the committed window back into conv_state, for all n_seq rows
// and all T draft positions in one launch.
//
// What the pages fix (Atlas docs, fn gdn_verify_fused_conv_kn_batched; sglang PR
// 46184, "Motivation" / "Modifications"; Atlas glm5next_kda/mod.rs,
// Glm5NextKdaConfig) is restated in include/conv_verify.h.  This file is the MI355X
// design of it.  The op moves ~3 bytes per flop, so the design is about HBM:
//
//  * One 64-lane wavefront per workgroup, 4 channels per lane, 256 channels per
//    wavefront; the 1-D grid is n_seq * ceil(d_inner / 256) workgroups.  (256-channel
//    blocks stream measurably faster on MI355X than 512-channel ones for this traffic
//    mix: twice the wavefronts keep more requests in flight.)
//  * Every global access is a lane-contiguous 8- or 16-byte buffer access with the
//    nt (streaming) policy: x and out per token, and every run of conv_state, the
//    dense snapshots and the dedup rows, which are staged through LDS so that they
//    too leave in lane-contiguous units.  Per-token offsets live in SGPRs.
//  * All loads (x for every token, conv_state, weights, bias) are issued before the
//    first barrier; after it the wavefront only stores, so no wait on a load is ever
//    stuck behind stores (vmcnt counts both).  Later LDS hand-offs use barriers that
//    order LDS only.
//  * The rollback windows and the committed state are pure copies of the inputs; they
//    are written first, and the arithmetic runs while they drain.
//  * The conv is one fused multiply-add per tap in tap order (bias first), the same
//    order as the per-token path it replaces, so the pre-activation is bit-identical
//    to a correctly rounded fp32 evaluation of that order.
//  * L2: a head of H channels spans H/4 lanes; its sum of squares is a butterfly with
//    DPP inside 16-lane rows (quad_perm, row_half_mirror, row_mirror) and ds_swizzle /
//    bpermute beyond; every lane of a head ends with the same sum.
//  * Windows and conv_state move as bit patterns; only the conv reads them as floats.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cv_internal.h"

namespace cvimpl {
namespace {

// ---- bit-pattern helpers (compile-time element indices) -----------------------------

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
    // p * sigmoid(p) with v_exp_f32 and v_rcp_f32.  For p << 0 the exponential
    // saturates to +inf and the result is -0.
    return p * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(p * -1.4426950408889634f));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sums over the 2^hl_log2 lanes of an aligned lane group (all lanes active), for each
// of G independent values at once: every stage is applied to all G values before the
// next, so their cross-lane latencies overlap.  Each step adds the two halves of a
// group symmetrically, so all lanes of a group hold the bit-identical sum.
template <int G>
__device__ __forceinline__ void group_sums(float (&v)[G], int hl_log2) {
    if (hl_log2 >= 1)   // quad_perm [1,0,3,2]: lane ^ 1
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] += dpp<0xB1>(v[g]);
    if (hl_log2 >= 2)   // quad_perm [2,3,0,1]: lane ^ 2
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] += dpp<0x4E>(v[g]);
    if (hl_log2 >= 3)   // row_half_mirror: the other quad of the 8
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] += dpp<0x141>(v[g]);
    if (hl_log2 >= 4)   // row_mirror: the other half of the 16-lane row
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] += dpp<0x140>(v[g]);
    if (hl_log2 >= 5)   // lane ^ 16 inside 32 (ds_swizzle xor mode)
#pragma unroll
        for (int g = 0; g < G; ++g)
            v[g] += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[g]), 0x401F));
    if (hl_log2 >= 6) {  // lane ^ 32
        const int src = (int)((threadIdx.x ^ 32u) << 2);
#pragma unroll
        for (int g = 0; g < G; ++g)
            v[g] += __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v[g])));
    }
}

// ---- raw buffer access ------------------------------------------------------------------
//
// Every global access goes through a buffer resource spanning exactly the bytes the
// wavefront may touch.  The per-token offset lives in an SGPR (soffset), the per-lane
// offset in a VGPR, so no 64-bit address arithmetic is repeated per token.  Lanes
// past the end of d_inner use the lane offset 0x80000000, which the hardware range
// check turns into a load of zeros / a dropped store.

using rsrc_t = __amdgpu_buffer_rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr uint32_t kOffLane = 0x80000000u;
// Cache policy of every global access: nt (streaming).  Each byte is read or written
// once per launch, so nothing is worth keeping in L2 or the Infinity Cache.
constexpr int kNT = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// NB-byte (8 or 16) global load / store of words d[0 .. NB/4).
template <int NB>
__device__ __forceinline__ void gload(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t *d) {
    if constexpr (NB == 16) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kNT);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else {
        static_assert(NB == 8, "8- or 16-byte accesses");
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kNT);
        d[0] = v.x; d[1] = v.y;
    }
}

template <int NB>
__device__ __forceinline__ void gstore(rsrc_t r, uint32_t voff, uint32_t soff, const uint32_t *s) {
    if constexpr (NB == 16) {
        const u32x4 v = {s[0], s[1], s[2], s[3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, kNT);
    } else {
        static_assert(NB == 8, "8- or 16-byte accesses");
        const u32x2 v = {s[0], s[1]};
        __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)voff, (int)soff, kNT);
    }
}

// A run of NB bytes (a multiple of 8) between registers and LDS, in the widest units
// that divide it.
template <int NB>
__device__ __forceinline__ void lds_write_run(char *p, const uint32_t *s) {
    static_assert(NB % 8 == 0, "runs are whole 8-byte units");
    if constexpr (NB % 16 == 0) {
#pragma unroll
        for (int q = 0; q < NB / 16; ++q)
            *(uint4 *)(p + 16 * q) = make_uint4(s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]);
    } else {
#pragma unroll
        for (int q = 0; q < NB / 8; ++q) *(uint2 *)(p + 8 * q) = make_uint2(s[2 * q], s[2 * q + 1]);
    }
}

template <int NB>
__device__ __forceinline__ void lds_read_run(const char *p, uint32_t *d) {
    static_assert(NB % 8 == 0, "runs are whole 8-byte units");
    if constexpr (NB % 16 == 0) {
#pragma unroll
        for (int q = 0; q < NB / 16; ++q) {
            const uint4 v = *(const uint4 *)(p + 16 * q);
            d[4 * q] = v.x; d[4 * q + 1] = v.y; d[4 * q + 2] = v.z; d[4 * q + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < NB / 8; ++q) {
            const uint2 v = *(const uint2 *)(p + 8 * q);
            d[2 * q] = v.x; d[2 * q + 1] = v.y;
        }
    }
}

template <int EB>
__device__ __forceinline__ uint32_t lds_get(const char *p) {
    if constexpr (EB == 4) return *(const uint32_t *)p;
    else return *(const uint16_t *)p;
}

template <int EB>
__device__ __forceinline__ void lds_put(char *p, uint32_t v) {
    if constexpr (EB == 4) *(uint32_t *)p = v;
    else *(uint16_t *)p = (uint16_t)v;
}

// Streams `chunks` 16-byte chunks from LDS (offset 0) to a buffer, lane-contiguous.
__device__ __forceinline__ void lds_to_global(const char *lds, int chunks, rsrc_t r, uint32_t soff,
                                              int lane) {
    for (int q = lane; q < chunks; q += kWave) {
        const uint4 v = *(const uint4 *)(lds + q * 16);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        gstore<16>(r, (uint32_t)q * 16u, soff, w4);
    }
}

// A wavefront-uniform int read through the constant address space, so it is a scalar
// load: it waits on its own counter, not behind the vector loads already in flight.
// Only for data no kernel writes while this one runs (slot indices, offsets).
__device__ __forceinline__ int scalar_read(const int32_t *p, int i) {
    return *((const __attribute__((address_space(4))) int32_t *)p + i);
}

// Orders LDS accesses across the workgroup (one wavefront) without waiting for the
// wavefront's global stores: __syncthreads() is a release fence for all memory, which
// would make every LDS hand-off wait for the writes issued before it to reach memory.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- the kernel -------------------------------------------------------------------------

template <int XB, int SB, int D, int TB, bool DEDUP>
__global__ __launch_bounds__(kWave) void cv_verify_kernel(KernelArgs p) {
    constexpr int CPL = kChannelsPerLane;     // channels per lane
    constexpr int CHW = kWave * CPL;          // channels per wavefront
    constexpr int W1 = D - 1;                 // window columns
    constexpr int VB = CPL * XB;              // bytes of x / out per lane per token (8 or 16)
    constexpr int XW = VB / 4;
    constexpr int SCB = CPL * SB;             // bytes of a state-typed column per lane
    constexpr int SW = SCB / 4;
    constexpr int RUNB = CPL * W1 * SB;       // bytes of a lane's [CPL][W1] window run
    constexpr int RUNW = RUNB / 4;
    constexpr int P = tile_pitch(SB);         // bytes per LDS tile row

    extern __shared__ uint4 lds_raw[];
    char *lds = (char *)lds_raw;

    const int lane = threadIdx.x;
    const int row = (int)(blockIdx.x / (unsigned)p.channel_blocks);
    const int cb = (int)(blockIdx.x - (unsigned)row * (unsigned)p.channel_blocks) * CHW;

    // The row's slot and offset are read now (scalar loads) and tested once the loads
    // that do not depend on them are on their way.
    const int slot = p.slot_idx ? scalar_read(p.slot_idx, row) : row;
    const int a = p.nat ? scalar_read(p.nat, row) : 0;

    const int T = p.T;
    const int SL = p.state_len;
    const int nch = min(CHW, p.d_inner - cb);   // channels of this wavefront
    const bool on = lane * CPL < nch;
    const uint32_t laneV = on ? (uint32_t)(lane * VB) : kOffLane;
    const bool contiguous_state = SL == W1;

    // ---- every load, issued up front -------------------------------------------------------
    // Raised wave priority while this wavefront issues its loads: when several
    // wavefronts of a SIMD are ready, the ones still issuing loads go first, so reads
    // enter the memory pipeline ahead of other wavefronts' stores.
    __builtin_amdgcn_s_setprio(3);
    const rsrc_t x_r = make_rsrc((const char *)p.x + ((int64_t)row * p.x_seq + cb) * XB,
                                 (uint32_t)(((int64_t)(T - 1) * p.x_tok + nch) * XB));
    uint32_t X[TB][XW];   // x_t for the lane's channels
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        if (t < T) {
            gload<VB>(x_r, laneV, (uint32_t)(t * p.x_tok * XB), X[t]);
        } else {
#pragma unroll
            for (int w = 0; w < XW; ++w) X[t][w] = 0u;
        }
    }

    uint32_t wr[XW * D];          // weights [CPL][D]
    uint32_t br[XW];              // bias [CPL]
    {
        const rsrc_t w_r = make_rsrc((const char *)p.weight + (int64_t)cb * D * XB,
                                     (uint32_t)(nch * D * XB));
        const uint32_t lw = on ? (uint32_t)(lane * VB * D) : kOffLane;
#pragma unroll
        for (int q = 0; q < D; ++q) gload<VB>(w_r, lw + VB * q, 0, wr + XW * q);
#pragma unroll
        for (int w = 0; w < XW; ++w) br[w] = 0u;
        if (p.bias) {
            const rsrc_t b_r = make_rsrc((const char *)p.bias + (int64_t)cb * XB,
                                         (uint32_t)(nch * XB));
            gload<VB>(b_r, laneV, 0, br);
        }
    }

    // Padded rows (slot -1) leave before any store; rows with an index that would
    // address outside the buffers are skipped the same way.  The loads above stay in
    // bounds for every row; wait for them before leaving.
    if (slot < 0 || slot >= p.n_slots || a < 0 || a > p.state_len - W1) {
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // conv_state: the wavefront's [nch, state_len] region is contiguous.  It comes in
    // whole (coalesced 16-byte loads, issued with the other loads) and is staged in
    // LDS; each lane picks its channels' window out of it, writes its committed window
    // back into it, and the region leaves whole - so every state byte is read once and
    // written once in lane-contiguous 16-byte units, whatever state_len and the offset
    // are.  (Direct global->LDS loads measured slower here than loads through VGPRs.)
    const rsrc_t st_r = make_rsrc((const char *)p.state + ((int64_t)slot * p.state_slot +
                                                           (int64_t)cb * SL) * SB,
                                  (uint32_t)(nch * SL * SB));
    const int rchunks = nch * SL * SB / 16;   // exact: nch * SB is a multiple of 16
    // chunks per lane, all in flight at once up to RJ; longer regions go in rounds
    constexpr int RJ = (W1 * SB + 3) / 4 > 12 ? (W1 * SB + 3) / 4 : 12;
    uint32_t sreg[RJ][4];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const int q = j * kWave + lane;
        if (j * kWave < rchunks) gload<16>(st_r, q < rchunks ? (uint32_t)q * 16u : kOffLane, 0, sreg[j]);
    }
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const int q = j * kWave + lane;
        if (j * kWave < rchunks && q < rchunks)
            *(uint4 *)(lds + q * 16) = make_uint4(sreg[j][0], sreg[j][1], sreg[j][2], sreg[j][3]);
    }
    for (int j0 = RJ; j0 * kWave < rchunks; j0 += RJ) {   // state_len beyond the in-flight set
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int q = (j0 + j) * kWave + lane;
            if ((j0 + j) * kWave < rchunks) gload<16>(st_r, q < rchunks ? (uint32_t)q * 16u : kOffLane, 0, sreg[j]);
        }
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int q = (j0 + j) * kWave + lane;
            if ((j0 + j) * kWave < rchunks && q < rchunks)
                *(uint4 *)(lds + q * 16) = make_uint4(sreg[j][0], sreg[j][1], sreg[j][2], sreg[j][3]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();

    uint32_t S[W1][SW];   // initial window columns v[0..W1-1], state-typed bits
    if (contiguous_state) {
        uint32_t run[RUNW];   // the lane's [CPL][W1] run
        lds_read_run<RUNB>(lds + lane * RUNB, run);
#pragma unroll
        for (int j = 0; j < W1; ++j)
#pragma unroll
            for (int w = 0; w < SW; ++w) {
                if constexpr (SB == 4) {
                    S[j][w] = elem_bits<4>(run, w * W1 + j);
                } else {
                    S[j][w] = elem_bits<2>(run, (2 * w) * W1 + j) |
                              (elem_bits<2>(run, (2 * w + 1) * W1 + j) << 16);
                }
            }
    } else {
        const char *rec = lds + (lane * CPL * SL + a) * SB;
#pragma unroll
        for (int j = 0; j < W1; ++j)
#pragma unroll
            for (int w = 0; w < SW; ++w) {
                if constexpr (SB == 4) {
                    S[j][w] = lds_get<4>(rec + (w * SL + j) * 4);
                } else {
                    S[j][w] = lds_get<2>(rec + ((2 * w) * SL + j) * 2) |
                              (lds_get<2>(rec + ((2 * w + 1) * SL + j) * 2) << 16);
                }
            }
    }

    float wv[CPL][D];
    float bv[CPL];
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
#pragma unroll
        for (int w = 0; w < D; ++w) wv[ch][w] = elem_val<XB>(wr, ch * D + w);
        bv[ch] = elem_val<XB>(br, ch);
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
    // The lane's [CPL][W1] run of the window v[k0 .. k0+W1-1], packed.
    auto window_run = [&](int k0, uint32_t *run) {
#pragma unroll
        for (int w = 0; w < RUNW; ++w) {
            if constexpr (SB == 4) {
                run[w] = sbits(k0 + w % W1, w / W1);
            } else {
                const int e0 = 2 * w, e1 = 2 * w + 1;
                run[w] = sbits(k0 + e0 % W1, e0 / W1) | (sbits(k0 + e1 % W1, e1 / W1) << 16);
            }
        }
    };
    // Column v[k] (the lane's CPL channels) in the state type.
    auto column = [&](int k, uint32_t *col) {
        if (k < W1) {
#pragma unroll
            for (int w = 0; w < SW; ++w) col[w] = S[k < W1 ? k : 0][w];
        } else if constexpr (XB == SB) {
#pragma unroll
            for (int w = 0; w < SW; ++w) col[w] = X[k < W1 ? 0 : k - W1][w];
        } else {
#pragma unroll
            for (int w = 0; w < SW; ++w)   // bf16 -> fp32 widening, channel w
                col[w] = x_to_state_bits<XB, SB>(elem_bits<XB>(X[k < W1 ? 0 : k - W1], w));
        }
    };

    // ---- conv + SiLU + per-head L2 -> out --------------------------------------------------
    // The arithmetic runs as soon as the inputs are in, before the copies below: while
    // the memory pipeline is still full of other wavefronts' traffic, a wavefront that
    // stores first would stall at its stores with its arithmetic still ahead of it.
    const bool wave_l2 = cb < p.qk;    // uniform: this wavefront holds q|k channels
    const bool lane_l2 = lane * CPL + cb < p.qk;
    const rsrc_t o_r = make_rsrc((char *)p.out + ((int64_t)row * p.out_seq + cb) * XB,
                                 (uint32_t)(((int64_t)(T - 1) * p.out_tok + nch) * XB));
    // Tokens go in chunks with no branch inside a chunk: x past T reads as zeros and
    // those tokens are computed but never stored.  The chunk's exponentials,
    // reciprocals and cross-lane sums are then independent and overlap.  Buckets up
    // to 8 are one chunk; larger ones use chunks of 4, which bounds the registers and
    // the work spent past T.
    constexpr int G = TB <= 8 ? TB : 4;
#pragma unroll
    for (int t0 = 0; t0 < TB; t0 += G) {
        if (t0 < T) {   // uniform guard; the loops are fully unrolled
            float y[G][CPL];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) {
                    float acc = bv[ch];
#pragma unroll
                    for (int w = 0; w < D; ++w)
                        acc = __builtin_fmaf(wv[ch][w], val(t0 + g + w, ch), acc);
                    y[g][ch] = silu(acc);
                }
            if (wave_l2) {
                float ss[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    ss[g] = 0.0f;
#pragma unroll
                    for (int ch = 0; ch < CPL; ++ch) ss[g] = __builtin_fmaf(y[g][ch], y[g][ch], ss[g]);
                }
                group_sums<G>(ss, p.head_lanes_log2);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float sc = lane_l2 ? __builtin_amdgcn_rsqf(ss[g] + p.eps) : 1.0f;
#pragma unroll
                    for (int ch = 0; ch < CPL; ++ch) y[g][ch] *= sc;
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int t = t0 + g;
                if (t < T) {
                    uint32_t o[XW];
                    if constexpr (XB == 4) {
#pragma unroll
                        for (int ch = 0; ch < CPL; ++ch) o[ch] = __float_as_uint(y[g][ch]);
                    } else {
                        typedef float f2 __attribute__((ext_vector_type(2)));
                        typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
                        for (int w = 0; w < XW; ++w) {
                            f2 pr = {y[g][2 * w], y[g][2 * w + 1]};
                            o[w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, b2));
                        }
                    }
                    gstore<VB>(o_r, laneV, (uint32_t)(t * p.out_tok * XB), o);
                }
            }
        }
    }
    // ---- committed window -> conv_state -----------------------------------------------------
    // v[T .. T+W1-1] into columns 0..W1-1 of the staged rows (each lane rewrites only
    // its own channels' records, after having read them above), then the region leaves.
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        if (t == T - 1) {
            if (contiguous_state) {
                uint32_t run[RUNW];
                window_run(t + 1, run);
                lds_write_run<RUNB>(lds + lane * RUNB, run);
            } else {
                char *rec = lds + lane * CPL * SL * SB;
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
                    for (int j = 0; j < W1; ++j)
                        lds_put<SB>(rec + (ch * SL + j) * SB, sbits(t + 1 + j, ch));
            }
        }
    }
    lds_barrier();
    lds_to_global(lds, rchunks, st_r, 0, lane);
    lds_barrier();   // the region's LDS is reused below

    // ---- rollback windows: pure copies of the inputs ---------------------------------------
    if constexpr (DEDUP) {
        const int L = T + W1 - 1;             // row length: v[1 .. T+W1-1]
        const rsrc_t row_r = make_rsrc(
            (char *)p.win + ((int64_t)slot * p.win_slot + (int64_t)cb * L) * SB,
            (uint32_t)(nch * L * SB));
        if (T == TB) {
            // Row length known at compile time: each lane assembles its channels' rows
            // ([CPL][LC], contiguous in the row layout) in registers into LDS at the
            // same offsets, and the wavefront streams the block out lane-contiguously.
            constexpr int LC = TB + W1 - 1;
            constexpr int LANEB = CPL * LC * SB;   // bytes of a lane's rows
            constexpr int CW = LANEB / 4;
            constexpr int PIECE = (LANEB % 16 == 0) ? 16 : 8;
            char *mine = lds + lane * LANEB;
#pragma unroll
            for (int q = 0; q < CW / (PIECE / 4); ++q) {
                uint32_t w4[PIECE / 4];
#pragma unroll
                for (int i = 0; i < PIECE / 4; ++i) {
                    const int wd = (PIECE / 4) * q + i;
                    if constexpr (SB == 4) {
                        w4[i] = sbits(wd % LC + 1, wd / LC);
                    } else {
                        const int e0 = 2 * wd, e1 = 2 * wd + 1;
                        w4[i] = sbits(e0 % LC + 1, e0 / LC) | (sbits(e1 % LC + 1, e1 / LC) << 16);
                    }
                }
                lds_write_run<PIECE>(mine + PIECE * q, w4);
            }
            lds_barrier();
            lds_to_global(lds, nch * LC * SB / 16, row_r, 0, lane);
        } else {
            // Tile row r holds v[r+1] for the wavefront's channels; rows 0..W1-2 come
            // from the initial window, the rest are x_0..x_{T-1}.
#pragma unroll
            for (int k = 1; k < W1 + TB; ++k) {
                if (k < W1 + T) {
                    uint32_t col[SW];
                    column(k, col);
                    lds_write_run<SCB>(lds + (k - 1) * P + lane * SCB, col);
                }
            }
            lds_barrier();
            // Stream the tile out in the row layout [c][k], k < L: chunk q of the
            // wavefront's contiguous row block holds elements e = q*EPC .. q*EPC+EPC-1,
            // element e = (channel e / L, column e % L) = tile row e % L, channel e / L.
            constexpr int EPC = 16 / SB;   // elements per 16-byte chunk
            const int nchunks = nch * L / EPC;   // exact: nch * SB is a multiple of 16
            const int e0 = lane * EPC;
            int cc = e0 / L;
            int kk = e0 - cc * L;
            const int dq = (kWave * EPC) / L;
            const int dr = kWave * EPC - dq * L;
            if (L >= EPC) {
                // a chunk spans at most two channels: columns kk.. of channel cc, then
                // columns 0.. of channel cc+1; each element is one LDS read at a fixed
                // row step from one of two bases
                for (int q = lane; q < nchunks; q += kWave) {
                    const int split = L - kk;
                    const uint32_t b1 = (uint32_t)(kk * P + cc * SB);
                    const uint32_t b2 = b1 + (uint32_t)SB - (uint32_t)(L * P);
                    uint32_t w[4];
#pragma unroll
                    for (int m = 0; m < EPC; ++m) {
                        const uint32_t b = lds_get<SB>(lds + ((m < split ? b1 : b2) + m * P));
                        if constexpr (SB == 4) {
                            w[m] = b;
                        } else {
                            if (m & 1) w[m >> 1] |= b << 16; else w[m >> 1] = b;
                        }
                    }
                    gstore<16>(row_r, (uint32_t)q * 16u, 0, w);
                    cc += dq;
                    kk += dr;
                    if (kk >= L) { kk -= L; ++cc; }
                }
            } else {
                for (int q = lane; q < nchunks; q += kWave) {
                    uint32_t w[4];
                    int c2 = cc, k2 = kk;
#pragma unroll
                    for (int m = 0; m < EPC; ++m) {
                        const uint32_t b = lds_get<SB>(lds + k2 * P + c2 * SB);
                        if constexpr (SB == 4) {
                            w[m] = b;
                        } else {
                            if (m & 1) w[m >> 1] |= b << 16; else w[m >> 1] = b;
                        }
                        if (++k2 == L) { k2 = 0; ++c2; }
                    }
                    gstore<16>(row_r, (uint32_t)q * 16u, 0, w);
                    cc += dq;
                    kk += dr;
                    while (kk >= L) { kk -= L; ++cc; }
                }
            }
        }
    } else {
        // Dense snapshot t = v[t+1 .. t+W1]: the wavefront's [nch, W1] slab is contiguous.
        // Lanes drop their [CPL][W1] runs into an LDS slab and the slab leaves in
        // lane-contiguous 16-byte units.  Two slabs alternate, so one barrier per
        // token orders both reuse hazards.
        constexpr int SLAB = CHW * W1 * SB;
        const int slab_chunks = nch * W1 * SB / 16;
        const rsrc_t snap_r = make_rsrc(
            (char *)p.win + ((int64_t)slot * p.win_slot + (int64_t)cb * W1) * SB,
            (uint32_t)(((int64_t)(T - 1) * p.d_inner * W1 + (int64_t)nch * W1) * SB));
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t < T) {
                char *slab = lds + (t & 1) * SLAB;
                uint32_t run[RUNW];
                window_run(t + 1, run);
                lds_write_run<RUNB>(slab + lane * RUNB, run);
                lds_barrier();
                lds_to_global(slab, slab_chunks, snap_r, (uint32_t)(t * p.d_inner * W1 * SB), lane);
            }
        }
    }

}

// ---- instantiation ----------------------------------------------------------------------
//
// This file is compiled once per (x dtype, state dtype, layout) with CV_XB, CV_SB and
// CV_DEDUP defined, so the instantiations build in parallel; each object exports one
// picker over (d_conv, token bucket).

template <int XB, int SB, int D, bool DEDUP>
const void *pick_bucket(int tb) {
    switch (tb) {
        case 1: return (const void *)cv_verify_kernel<XB, SB, D, 1, DEDUP>;
        case 2: return (const void *)cv_verify_kernel<XB, SB, D, 2, DEDUP>;
        case 4: return (const void *)cv_verify_kernel<XB, SB, D, 4, DEDUP>;
        case 8: return (const void *)cv_verify_kernel<XB, SB, D, 8, DEDUP>;
        case 16: return (const void *)cv_verify_kernel<XB, SB, D, 16, DEDUP>;
        case 24: return (const void *)cv_verify_kernel<XB, SB, D, 24, DEDUP>;
        case 32: return (const void *)cv_verify_kernel<XB, SB, D, 32, DEDUP>;
        default: return nullptr;
    }
}

}  // namespace

#if !defined(CV_XB) || !defined(CV_SB) || !defined(CV_DEDUP)
#error "compile with -DCV_XB=<2|4> -DCV_SB=<2|4> -DCV_DEDUP=<0|1>"
#endif

#define CV_PICK_NAME(xb, sb, dd) pick_kernel_##xb##_##sb##_##dd
#define CV_PICK(xb, sb, dd) CV_PICK_NAME(xb, sb, dd)

const void *CV_PICK(CV_XB, CV_SB, CV_DEDUP)(int d_conv, int token_bucket) {
    switch (d_conv) {
        case 2: return pick_bucket<CV_XB, CV_SB, 2, CV_DEDUP != 0>(token_bucket);
        case 3: return pick_bucket<CV_XB, CV_SB, 3, CV_DEDUP != 0>(token_bucket);
        case 4: return pick_bucket<CV_XB, CV_SB, 4, CV_DEDUP != 0>(token_bucket);
        default: return nullptr;
    }
}

}  // namespace cvimpl
