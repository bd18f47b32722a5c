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
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
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

// ---- raw buffer access ------------------------------------------------------------------
//
// Every global access goes through a buffer resource spanning exactly the bytes the
// wavefront may touch.  The per-token offset lives in an SGPR (soffset), the per-lane
// offset in a VGPR, so no 64-bit address arithmetic is repeated per token.  Lanes
// past the end of d_inner use the lane offset 0x80000000, which the hardware range
// check turns into a load of zeros / a dropped store.

using rsrc_t = __amdgpu_buffer_rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr uint32_t kOffLane = 0x80000000u;
// Cache policy of every global access: nt (streaming).  Each byte is read or written
// once per launch, so nothing is worth keeping in L2 or the Infinity Cache.
constexpr int kNT = 2;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ void load16(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t *d) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kNT);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
}

__device__ __forceinline__ void store16(rsrc_t r, uint32_t voff, uint32_t soff, const uint32_t *s) {
    const u32x4 v = {s[0], s[1], s[2], s[3]};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)voff, (int)soff, kNT);
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
    constexpr int CPL = 16 / XB;          // channels per lane
    constexpr int CHW = kWave * CPL;      // channels per wavefront
    constexpr int W1 = D - 1;             // window columns
    constexpr int SW = CPL * SB / 4;      // 32-bit words per state-typed column
    constexpr int RUNW = CPL * W1 * SB / 4;   // words of a lane's [ch][j] window run
    constexpr int P = tile_pitch(CPL, SB);    // bytes per LDS tile row
    static_assert(RUNW % 4 == 0 && SW % 4 == 0, "runs and columns are whole 16-byte units");

    extern __shared__ uint4 lds_raw[];
    char *lds = (char *)lds_raw;

    const int lane = threadIdx.x;
    const int row = (int)(blockIdx.x / (unsigned)p.channel_blocks);
    const int cb = (int)(blockIdx.x - (unsigned)row * (unsigned)p.channel_blocks) * CHW;

    const int slot = p.slot_idx ? p.slot_idx[row] : row;
    const int a = p.nat ? p.nat[row] : 0;
    // Padded rows (slot -1) leave before any store; rows with an index that would
    // address outside the buffers are skipped the same way.
    if (slot < 0 || slot >= p.n_slots || a < 0 || a > p.state_len - W1) return;

    const int T = p.T;
    const int SL = p.state_len;
    const int nch = min(CHW, p.d_inner - cb);       // channels of this wavefront
    const bool on = lane * CPL < nch;
    const uint32_t lane16 = on ? (uint32_t)lane * 16u : kOffLane;
    const bool contiguous_state = SL == W1;

    // ---- loads: x (registers), window, weights, bias ----------------------------------
    const rsrc_t x_r = make_rsrc((const char *)p.x + ((int64_t)row * p.x_seq + cb) * XB,
                                 (uint32_t)(((int64_t)(T - 1) * p.x_tok + nch) * XB));
    uint32_t X[TB][4];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        if (t < T) {
            load16(x_r, lane16, (uint32_t)(t * p.x_tok * XB), X[t]);
        } else {
            X[t][0] = X[t][1] = X[t][2] = X[t][3] = 0u;
        }
    }

    // weights and bias: loaded with everything else, before the first barrier, so no
    // load is outstanding once the stores start (vmcnt counts loads and stores together)
    uint32_t wr[4 * D];   // CPL*D*XB bytes = 16*D
    uint32_t br[4] = {0u, 0u, 0u, 0u};
    {
        const rsrc_t w_r = make_rsrc((const char *)p.weight + (int64_t)cb * D * XB,
                                     (uint32_t)(nch * D * XB));
        const uint32_t lw = on ? (uint32_t)lane * 16u * D : kOffLane;
#pragma unroll
        for (int q = 0; q < D; ++q) load16(w_r, lw + 16 * q, 0, wr + 4 * q);
        if (p.bias) {
            const rsrc_t b_r = make_rsrc((const char *)p.bias + (int64_t)cb * XB,
                                         (uint32_t)(nch * XB));
            load16(b_r, lane16, 0, br);
        }
    }

    // conv_state: the wavefront's [nch, state_len] region is contiguous.  It comes in
    // whole through LDS (direct loads, coalesced), each lane picks its channels'
    // window out of it, writes its committed window back into it, and the region
    // leaves whole (coalesced) - so every state byte is read once and written once
    // in full 16-byte lane-contiguous units, whatever state_len and the offset are.
    const rsrc_t st_r = make_rsrc((const char *)p.state + ((int64_t)slot * p.state_slot +
                                                           (int64_t)cb * SL) * SB,
                                  (uint32_t)(nch * SL * SB));
    const int rchunks = nch * SL * SB / 16;   // exact: nch * SB is a multiple of 16
    for (int j = 0; j * kWave < rchunks; ++j) {
        const int q = j * kWave + lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(st_r, (lds_void_t *)(lds + j * (kWave * 16)), 16,
                                                 q < rchunks ? q * 16 : (int)kOffLane, 0, 0, kNT);
    }
    __syncthreads();   // waits for the direct loads (and x): nothing has been stored yet
    uint32_t S[W1][SW];   // initial window columns v[0..W1-1], state-typed bits
    if (contiguous_state) {
        // the lane's [CPL][W1] run: RUNW/4 aligned 16-byte LDS reads
        uint32_t run[RUNW];
#pragma unroll
        for (int q = 0; q < RUNW / 4; ++q) {
            const uint4 v = *(const uint4 *)(lds + lane * (RUNW * 4) + 16 * q);
            run[4 * q] = v.x; run[4 * q + 1] = v.y; run[4 * q + 2] = v.z; run[4 * q + 3] = v.w;
        }
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
    // The lane's CPL x (D-1) run of the window v[k0 .. k0+W1-1] ([ch][j] order), packed.
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
    // Column v[k] in the state type (SW words).
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

    {
        // committed window v[T .. T+W1-1] into columns 0..W1-1 of the staged rows, then
        // the whole region goes back out.  Each lane rewrites only its own channels'
        // records, after having read them above.
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t == T - 1) {
                if (contiguous_state) {
                    uint32_t run[RUNW];
                    window_run(t + 1, run);
#pragma unroll
                    for (int q = 0; q < RUNW / 4; ++q)
                        *(uint4 *)(lds + lane * (RUNW * 4) + 16 * q) =
                            make_uint4(run[4 * q], run[4 * q + 1], run[4 * q + 2], run[4 * q + 3]);
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
        for (int q = lane; q < rchunks; q += kWave) {
            const uint4 v = *(const uint4 *)(lds + q * 16);
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
            store16(st_r, (uint32_t)q * 16u, 0, w4);
        }
        lds_barrier();   // the region's LDS is reused below
    }

    // ---- rollback windows: pure copies of the inputs, written before any arithmetic so
    // the stores drain while the wavefront computes --------------------------------------
    if constexpr (DEDUP) {
        const int L = T + W1 - 1;             // row length: v[1 .. T+W1-1]
        const rsrc_t row_r = make_rsrc(
            (char *)p.win + ((int64_t)slot * p.win_slot + (int64_t)cb * L) * SB,
            (uint32_t)(nch * L * SB));
        if (T == TB) {
            // Row length known at compile time: each lane assembles its channels' rows
            // ([CPL][LC], contiguous in the row layout) in registers, 16 bytes at a time,
            // into LDS at the same offsets, and the wavefront streams the block out in
            // lane-contiguous 16-byte units.
            constexpr int LC = TB + W1 - 1;
            constexpr int CW = CPL * LC * SB / 4;   // 32-bit words of a lane's rows
            char *mine = lds + lane * (CPL * LC * SB);
#pragma unroll
            for (int q = 0; q < CW / 4; ++q) {
                uint32_t w4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int wd = 4 * q + i;
                    if constexpr (SB == 4) {
                        w4[i] = sbits(wd % LC + 1, wd / LC);
                    } else {
                        const int e0 = 2 * wd, e1 = 2 * wd + 1;
                        w4[i] = sbits(e0 % LC + 1, e0 / LC) | (sbits(e1 % LC + 1, e1 / LC) << 16);
                    }
                }
                *(uint4 *)(mine + 16 * q) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
            }
            lds_barrier();
            const int nchunks = nch * LC * SB / 16;
            for (int q = lane; q < nchunks; q += kWave) {
                const uint4 v = *(const uint4 *)(lds + q * 16);
                const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                store16(row_r, (uint32_t)q * 16u, 0, w4);
            }
        } else {
        // Tile row r holds v[r+1] for the wavefront's channels (16-byte LDS writes);
        // rows 0..W1-2 come from the initial window, the rest are x_0..x_{T-1}.
#pragma unroll
        for (int k = 1; k < W1 + TB; ++k) {
            if (k < W1 + T) {
                uint32_t col[SW];
                column(k, col);
#pragma unroll
                for (int q = 0; q < SW / 4; ++q)
                    *(uint4 *)(lds + (k - 1) * P + lane * (CPL * SB) + 16 * q) =
                        make_uint4(col[4 * q], col[4 * q + 1], col[4 * q + 2], col[4 * q + 3]);
            }
        }
        lds_barrier();
        // Stream the tile out in the row layout [c][k], k < L: chunk q of the
        // wavefront's contiguous row block holds elements e = q*EPC .. q*EPC+EPC-1,
        // element e = (channel e / L, column e % L) = tile row e % L, channel e / L.
        constexpr int EPC = 16 / SB;   // elements per 16-byte chunk
        const int nchunks = nch * L / EPC;   // exact: nch is a multiple of CPL
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
                store16(row_r, (uint32_t)q * 16u, 0, w);
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
                store16(row_r, (uint32_t)q * 16u, 0, w);
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
#pragma unroll
                for (int q = 0; q < RUNW / 4; ++q)
                    *(uint4 *)(slab + lane * (RUNW * 4) + 16 * q) =
                        make_uint4(run[4 * q], run[4 * q + 1], run[4 * q + 2], run[4 * q + 3]);
                lds_barrier();
                const uint32_t soff = (uint32_t)(t * p.d_inner * W1 * SB);
                for (int q = lane; q < slab_chunks; q += kWave) {
                    const uint4 v = *(const uint4 *)(slab + q * 16);
                    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
                    store16(snap_r, (uint32_t)q * 16u, soff, w4);
                }
            }
        }
    }

    // ---- conv + SiLU + per-head L2 -> out --------------------------------------------------
    const bool wave_l2 = cb < p.qk;    // uniform: this wavefront holds q|k channels
    const bool lane_l2 = lane * CPL + cb < p.qk;
    const rsrc_t o_r = make_rsrc((char *)p.out + ((int64_t)row * p.out_seq + cb) * XB,
                                 (uint32_t)(((int64_t)(T - 1) * p.out_tok + nch) * XB));
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
            store16(o_r, lane16, (uint32_t)(t * p.out_tok * XB), o);
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
