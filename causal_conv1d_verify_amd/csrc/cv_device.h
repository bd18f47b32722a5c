// Device-side helpers shared by the HIP kernels of the library (verify, restore,
// prefill, L2): bit-pattern access to packed elements, SiLU, cross-lane sums, raw
// buffer loads/stores with the streaming policy, LDS runs and barriers.  Internal;
// included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cv_internal.h"

#ifdef CV_WRITE_COUNT
// The write-count build's ranges (see count_store below): one variable per code object,
// named by the including source (CV_COUNT_RANGES) so that no two objects share a symbol.
#ifndef CV_COUNT_RANGES
#error "a write-count build names its code object's count ranges (CV_COUNT_RANGES)"
#endif
__device__ cvimpl::CountRanges CV_COUNT_RANGES;
#endif

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

// SiLU(p) = p * sigmoid(p) with v_exp_f32 and v_rcp_f32, in a form with no overflow and
// no intermediate outside fp32's normal range.  With e = 2^q, q = -|p| * log2(e) <= 0:
// sigmoid(p) = 1 / (1 + e) for p >= 0 and e / (1 + e) for p < 0, so the reciprocal's
// argument stays in [1, 2].  Neither instruction returns a subnormal, and e leaves the
// normal range at p ~ -87.3, where SiLU(p) is still a normal fp32 (and bf16) value; so
// for q < -100 the exponential is taken 64 binades up (normal down to p ~ -131.7) and the
// product is scaled back by 2^-64 in the last multiply, which rounds into fp32's
// subnormals like any other multiply (denormals are enabled).  Below p ~ -131.7 the
// shifted exponential flushes to 0 and the result is -0: the exact value is then under
// 1e-55, far below half of fp32's smallest subnormal.  q + 64 is exact for q < -100.
// +-inf give +inf and NaN, and NaN stays NaN, as p / (1 + exp(-p)) does.
__device__ __forceinline__ float silu(float p) {
    const float q = __builtin_fabsf(p) * -1.4426950408889634f;
    const bool deep = q < -100.0f;
    const float e = __builtin_amdgcn_exp2f(deep ? q + 64.0f : q);   // 2^q, or 2^(q + 64)
    const float scale = deep ? 0x1p-64f : 1.0f;
    const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(e, scale, 1.0f));   // 1 / (1 + 2^q)
    return p < 0.0f ? ((p * e) * r) * scale : p * r;
}

// p * rcp(1 + 2^(-p log2 e)): five instructions, exact to the same bar as silu() while
// p >= kSiluFastMin (then 2^(-p log2 e) <= 2^125.5 and its reciprocal stays normal).
// Below it the reciprocal would flush to zero and the result become -0.
constexpr float kSiluFastMin = -87.0f;
__device__ __forceinline__ float silu_fast(float p) {
    return p * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(p * -1.4426950408889634f));
}

// SiLU over G token rows of pre-activations, in place, in the form FULL selects.
template <bool FULL, int G>
__device__ __forceinline__ void silu_rows(float (&v)[G][kChannelsPerLane]) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int ch = 0; ch < kChannelsPerLane; ++ch) v[g][ch] = FULL ? silu(v[g][ch]) : silu_fast(v[g][ch]);
}

// SiLU over G token rows, in place, choosing the form from the values themselves: the
// five-instruction one unless some value of the wavefront's rows lies below
// kSiluFastMin (one wavefront-uniform test per call).
template <int G>
__device__ __forceinline__ void silu_rows_checked(float (&v)[G][kChannelsPerLane]) {
    float lo = v[0][0];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int ch = 0; ch < kChannelsPerLane; ++ch) lo = __builtin_fminf(lo, v[g][ch]);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(lo < kSiluFastMin) == 0, 1))
        silu_rows<false, G>(v);
    else
        silu_rows<true, G>(v);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// v[i] + v[i ^ 16] and v[i] + v[i ^ 32] on every lane i, with gfx950's lane-swap
// instructions (plain VALU: no LDS round trip, no lane-address register).  With both
// operands v, the two results of a swap hold the lane pair {v[i], v[i ^ k]}, on both
// lanes of the pair in the same order, so both lanes get the bit-identical sum.
__device__ __forceinline__ float xor16_sum(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
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
    if (hl_log2 >= 5)   // lane ^ 16
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] = xor16_sum(v[g]);
    if (hl_log2 >= 6)   // lane ^ 32
#pragma unroll
        for (int g = 0; g < G; ++g) v[g] = xor32_sum(v[g]);
}

// Sums over groups of hl lanes where hl is not a power of two (3 <= hl <= 63): the groups
// start at lane 0 and follow one another, and the lanes past the last whole group form a
// shorter group of their own.  For G values at once, a segmented inclusive scan (step s
// adds the value s lanes down when that lane is in the same group, so after the steps
// s = 1, 2, 4, ... < hl a group's last lane holds the group's total, each value added once)
// is followed by a broadcast of that lane's total to its whole group, so all lanes of a
// group hold the bit-identical sum.  Lanes move through ds_bpermute (no LDS memory).
// All lanes active.
template <int G>
__device__ __forceinline__ void group_sums_any(float (&v)[G], int hl) {
    const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int first = lane - lane % hl;
    const int last = min(first + hl - 1, kWave - 1);
    for (int s = 1; s < hl; s *= 2) {   // (uniform)
        const bool take = lane - s >= first;
        const int src = (take ? lane - s : lane) * 4;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float t = __int_as_float(__builtin_amdgcn_ds_bpermute(src, __float_as_int(v[g])));
            v[g] = take ? v[g] + t : v[g];
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = __int_as_float(__builtin_amdgcn_ds_bpermute(last * 4, __float_as_int(v[g])));
}

// The first channel of channel block blk of a row and the end of its channels (before
// d_inner's end): uniform 256-channel blocks, or the q|k blocks of whole heads followed by
// 256-channel blocks from qk on (HeadBlocks).
__device__ __forceinline__ int block_first(const HeadBlocks &h, int blk, int qk, int d_inner, int &cend) {
    if (blk < h.qk_blocks) {
        const int c0 = blk * h.qk_block_ch;
        cend = min(c0 + h.qk_block_ch, qk);
        return c0;
    }
    cend = d_inner;
    return (h.qk_blocks ? qk : 0) + (blk - h.qk_blocks) * (kWave * kChannelsPerLane);
}

// group_sums for one value with every stage selected rather than branched on: the rare
// path of head_l2 uses it, where branches (and per-stage lane addresses) would hold
// registers across the whole token loop.
__device__ __forceinline__ float group_sum_sel(float v, int hl_log2) {
    float o = dpp<0xB1>(v);
    v = hl_log2 >= 1 ? v + o : v;
    o = dpp<0x4E>(v);
    v = hl_log2 >= 2 ? v + o : v;
    o = dpp<0x141>(v);
    v = hl_log2 >= 3 ? v + o : v;
    o = dpp<0x140>(v);
    v = hl_log2 >= 4 ? v + o : v;
    o = xor16_sum(v);
    v = hl_log2 >= 5 ? o : v;
    o = xor32_sum(v);
    v = hl_log2 >= 6 ? o : v;
    return v;
}

// Per-head L2 of G token rows held as y[g][channel], the lane's kChannelsPerLane
// channels: y <- y / sqrt(S + eps), S = sum_head y^2, on lanes with lane_l2 set (a head
// is the aligned group of 2^hl_log2 lanes, or with hl_log2 < 0 a group of hl lanes as in
// group_sums_any); other lanes keep y.  All lanes active.  ANY_HEAD false leaves the second
// form out of a build that only ever runs with power-of-two heads.
//
// S runs in fp32 (any reduction order) with v_rsq_f32.  That is accurate while
// S + eps <= 2^127 (no partial sum overflows) and either S >= 2^-100 (squares below
// 2^-126 lose bits, but are then at most 2^-42 of S) or eps >= 2^-60 (S is then at most
// 2^-40 of eps).  When a head of the wavefront is outside that range - |y| from ~1.3e19
// up, or tiny values with eps < 2^-60 - every head is summed again over y * f for a
// power of two f that brings its squares into range: 2^-70 after an overflow (|y f| <
// 2^58, so the sum stays below 2^124 and, as S >= 2^126, above 2^-14), 2^100 for a tiny
// S (every |y| < 2^-50, so the squares lie in [2^-98, 2^100) unless 0), and 1 for a head
// that was in range (the same sum, bit for bit).  The scale is then rsq(sum + eps f^2)
// * f; the multiply by 2^-70 rounds into fp32's subnormals when |y| nears fp32's maximum
// (still 17 or more significant bits, and |out| <= 1).  Where eps f^2 >= 2^127 the sum is
// below 2^-27 of it and the scale is rsq(eps).  Left out: eps = 0 with a head whose S is
// below 2^-256 (every value subnormal), whose scale exceeds fp32's range.  NaN and
// infinities give what y / sqrt(S + eps) gives.  The stages of the second sum are
// selected rather than branched on, so the rare path costs the common one no registers.
template <int G, bool ANY_HEAD = true>
__device__ __forceinline__ void head_l2(float (&y)[G][kChannelsPerLane], bool lane_l2,
                                        int hl_log2, int hl, float eps) {
    constexpr int CPL = kChannelsPerLane;
    float ss[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        ss[g] = 0.0f;
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) ss[g] = __builtin_fmaf(y[g][ch], y[g][ch], ss[g]);
    }
    if (!ANY_HEAD || hl_log2 >= 0)
        group_sums<G>(ss, hl_log2);
    else
        group_sums_any<G>(ss, hl);
    // in range: every S <= 2^126 (then S + eps <= 2^127 for eps <= 2^126; a larger eps
    // takes the second sum) and, unless eps >= 2^-60, every S >= 2^-100.  A NaN S gives
    // NaN either way, so the running max / min may drop it.
    const bool eps_swamps = eps >= 0x1p-60f;
    float hi = ss[0], lo = ss[0];
#pragma unroll
    for (int g = 1; g < G; ++g) {
        hi = __builtin_fmaxf(hi, ss[g]);
        lo = __builtin_fminf(lo, ss[g]);
    }
    const bool all_in = hi <= 0x1p126f && eps <= 0x1p126f && (eps_swamps || lo >= 0x1p-100f);
    float sc[G];
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(lane_l2 && !all_in) == 0, 1)) {
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = __builtin_amdgcn_rsqf(ss[g] + eps);
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            // f = 1 for a head in range: the same sum again, bit for bit
            const float f = !(ss[g] + eps <= 0x1p127f) ? 0x1p-70f
                            : (ss[g] >= 0x1p-100f || eps_swamps) ? 1.0f : 0x1p100f;
            float s = 0.0f;
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) {
                const float u = y[g][ch] * f;
                s = __builtin_fmaf(u, u, s);
            }
            if (!ANY_HEAD || hl_log2 >= 0) {
                s = group_sum_sel(s, hl_log2);
            } else {
                float one[1] = {s};
                group_sums_any<1>(one, hl);
                s = one[0];
            }
            const float ep = eps * f * f;
            // rsq(eps) is uniform: readfirstlane keeps it in a scalar register wherever
            // the compiler hoists it to
            const float r_eps = __builtin_bit_cast(
                float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, __builtin_amdgcn_rsqf(eps))));
            sc[g] = ep < 0x1p127f ? __builtin_amdgcn_rsqf(s + ep) * f : r_eps;
        }
    }
    if (lane_l2) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) y[g][ch] *= sc[g];
    }
}

// ---- raw buffer access ------------------------------------------------------------------
//
// Every global access goes through a buffer resource spanning exactly the bytes the
// wavefront may touch.  The per-token offset lives in an SGPR (soffset), the per-lane
// offset in a VGPR, so no 64-bit address arithmetic is repeated per token.  Lanes
// past the end of d_inner use the lane offset 0x80000000, which the hardware range
// check turns into a load of zeros / a dropped store.

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr uint32_t kOffLane = 0x80000000u;

#ifdef CV_WRITE_COUNT
// The write-count build (a library of its own, for tests): every global store also adds
// 1, per 2-byte unit it writes, to a counter of the registered range that holds it, so a
// test can check that each output element is written by exactly one store.  A resource
// then carries its base and size next to the hardware descriptor; the ranges live in one
// variable per code object (CV_COUNT_RANGES), set by the host through count_ranges_set_*.
struct rsrc_t {
    __amdgpu_buffer_rsrc_t r;
    const char *base;
    uint32_t bytes;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw(const rsrc_t &r) { return r.r; }
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return {__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                              0x00020000),
            (const char *)base, bytes};
}
// The stores the hardware drops (a lane at kOffLane, or past the resource) count nothing.
__device__ __forceinline__ void count_store(const rsrc_t &r, uint32_t voff, uint32_t soff, int nb) {
    const CountRanges &cr = ::CV_COUNT_RANGES;
    const uint64_t off = (uint64_t)voff + soff;
    if (off + (uint64_t)nb > r.bytes) return;
    const char *a = r.base + off;
    for (int k = 0; k < cr.n; ++k) {
        const char *lo = cr.lo[k];
        if (a >= lo && a + nb <= lo + cr.bytes[k]) {
            const uint64_t u = (uint64_t)(a - lo) / 2;
            for (int i = 0; i < nb / 2; ++i) atomicAdd(cr.counts[k] + u + i, 1u);
            return;
        }
    }
}
#else
using rsrc_t = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ rsrc_t raw(rsrc_t r) { return r; }
__device__ __forceinline__ void count_store(rsrc_t, uint32_t, uint32_t, int) {}
#endif
// Cache policy of the global accesses: nt (streaming).  Each byte of x, out, conv_state
// and the windows is read or written once per launch, so none of it is worth keeping
// in L2 or the Infinity Cache.  The weights (and bias) are the exception: every row's
// wavefronts read the same block, so their loads use the default policy (kKeep).
constexpr int kNT = 2;
constexpr int kKeep = 0;

#ifndef CV_WRITE_COUNT
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
#endif

// NB-byte (8 or 16) global load / store of words d[0 .. NB/4).
template <int NB, int POL = kNT>
__device__ __forceinline__ void gload(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t *d) {
    if constexpr (NB == 16) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(raw(r), (int)voff, (int)soff, POL);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    } else {
        static_assert(NB == 8, "8- or 16-byte accesses");
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(raw(r), (int)voff, (int)soff, POL);
        d[0] = v.x; d[1] = v.y;
    }
}

template <int NB, int POL = kNT>
__device__ __forceinline__ void gstore(rsrc_t r, uint32_t voff, uint32_t soff, const uint32_t *s) {
    if constexpr (NB == 16) {
        // The offset goes into the lane offset, the scalar offset stays 0: after a store of
        // more than 8 bytes whose scalar offset is an SGPR the compiler puts no wait state
        // before a VALU instruction that overwrites the store's data registers, and on
        // gfx950 the store then wrote that instruction's result for some lanes (the fourth
        // dword of lanes 12-15 of each 16-lane row, now and then: the widened fp32
        // columns of the time-major commit).  With an inline-constant scalar offset the
        // compiler inserts the wait.  kOffLane + soff stays out of range (soff < 2^31).
        const u32x4 v = {s[0], s[1], s[2], s[3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, raw(r), (int)(voff + soff), 0, POL);
    } else {
        static_assert(NB == 8, "8- or 16-byte accesses");
        const u32x2 v = {s[0], s[1]};
        __builtin_amdgcn_raw_buffer_store_b64(v, raw(r), (int)voff, (int)soff, POL);
    }
    count_store(r, voff, soff, NB);
}

// One EB-byte (2 or 4) element store, for the ends of rows that do not fill a chunk.
template <int EB, int POL = kNT>
__device__ __forceinline__ void gstore_elem(rsrc_t r, uint32_t voff, uint32_t bits) {
    if constexpr (EB == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(bits, raw(r), (int)voff, 0, POL);
    } else {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bits, raw(r), (int)voff, 0, POL);
    }
    count_store(r, voff, 0, EB);
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
template <int POL = kNT>
__device__ __forceinline__ void lds_to_global(const char *lds, int chunks, rsrc_t r, uint32_t soff,
                                              int lane) {
    for (int q = lane; q < chunks; q += kWave) {
        const uint4 v = *(const uint4 *)(lds + q * 16);
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
        gstore<16, POL>(r, (uint32_t)q * 16u, soff, w4);
    }
}

// A wavefront-uniform int read through the constant address space, so it is a scalar
// load: it waits on its own counter, not behind the vector loads already in flight.
// Only for data no kernel writes while this one runs (slot indices, offsets).
__device__ __forceinline__ int scalar_read(const int32_t *p, int i) {
    return *((const __attribute__((address_space(4))) int32_t *)p + i);
}

// Workgroups are handed to MI355X's 8 XCDs round-robin by index, and each XCD has an
// L2 of its own.  This maps the hardware index b of a grid of G workgroups to a linear
// work index so that each XCD takes one contiguous range of work indices (XCD x gets
// the indices b = x, x+8, ...; they map to consecutive work items): neighbouring
// channel blocks of a row then share one L2, and a cache line that straddles their
// boundary is fetched, merged and written back once.  A bijection on [0, G).
__device__ __forceinline__ unsigned xcd_linear(unsigned b, unsigned G) {
    const unsigned x = b % 8u, k = b / 8u, q = G / 8u, r = G % 8u;
    return x < r ? x * (q + 1u) + k : r * (q + 1u) + (x - r) * q + k;
}

// A contiguous block of `chunks` 16-byte chunks into LDS at dst by direct global->LDS
// loads: every load is issued before any completes, and no VGPR holds the data.  dst
// must have lds_dma_span(chunks * 16) bytes.  The caller waits (vmcnt) before reading.
__device__ __forceinline__ void block_to_lds(rsrc_t r, char *dst, int chunks, int lane) {
    for (int j = 0; j * kWave < chunks; ++j) {
        const int q = j * kWave + lane;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(raw(r), (lds_void_t *)(dst + j * kWave * 16), 16,
                                                 q < chunks ? (uint32_t)q * 16u : kOffLane, 0, 0,
                                                 kNT);
    }
}

// The s_waitcnt immediate that waits until at most n (0..63) vector memory operations
// of the wavefront are outstanding; expcnt and lgkmcnt are left at their maxima (not
// waited on).  gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
static_assert(vmcnt_imm(0) == 0x0F70 && vmcnt_imm(17) == 0x4F71, "s_waitcnt encoding");

// Orders LDS accesses across the workgroup (one wavefront) without waiting for the
// wavefront's global stores: __syncthreads() is a release fence for all memory, which
// would make every LDS hand-off wait for the writes issued before it to reach memory.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace
}  // namespace cvimpl
