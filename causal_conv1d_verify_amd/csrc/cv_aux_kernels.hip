// HIP kernels (gfx950) around the verify launch: the accepted-prefix restore, the
// prefill conv over packed prompts, and the separate per-head L2 over q|k.
//
//  * Restore (sglang PR 46184, "Motivation": the window lets the accepted prefix's
//    conv state be restored after verify): one wavefront per (row, 256 channels)
//    copies window k of the row's slot into conv_state columns 0..D-2.
//  * Prefill (Atlas glm5next_kda/mod.rs, prefill body: conv + SiLU only): one
//    wavefront per (row, 16-token chunk, 256 channels); the chunk's D-1 earlier inputs
//    come from x (or, for the first chunk, from the row's state window or zeros), and
//    the first chunk's wavefront also commits the row's last window - it is the one
//    that read the state, so the read and the write of a slot stay in one wavefront.
//  * L2 (same page, module doc: prefill L2 is a separate pass over q|k): one wavefront
//    per (token row, 256 q|k channels), the same cross-lane head sums as the verify.
//
// Every global access is a lane-contiguous 8/16-byte buffer access with the streaming
// policy; conv_state regions always move whole (see region_load).
#define CV_COUNT_RANGES cv_count_ranges_aux
#include "cv_device.h"
#include "cv_internal.h"

namespace cvimpl {
namespace {

constexpr int CPL = kChannelsPerLane;
constexpr int CHW = kWave * kChannelsPerLane;

// Element (ch, j) of a lane's packed [CPL][W1] run of SB-byte elements.
template <int SB, int W1>
__device__ __forceinline__ uint32_t run_elem(const uint32_t *run, int ch, int j) {
    return elem_bits<SB>(run, ch * W1 + j);
}

// A wavefront's conv_state region [nch, state_len] (contiguous) moves between HBM and
// LDS in coalesced 16-byte chunks.  State rows wider than the window are always read
// and written whole: writing only the window's bytes makes partial-sector writes,
// which measured about five times slower than moving the whole rows.
__device__ __forceinline__ void region_load(rsrc_t r, char *dst, int chunks, int lane) {
    constexpr int RJ = 8;   // chunks per lane in flight per round
    for (int j0 = 0; j0 * kWave < chunks; j0 += RJ) {
        uint32_t v[RJ][4];
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int q = (j0 + j) * kWave + lane;
            if ((j0 + j) * kWave < chunks) gload<16>(r, q < chunks ? (uint32_t)q * 16u : kOffLane, 0, v[j]);
        }
#pragma unroll
        for (int j = 0; j < RJ; ++j) {
            const int q = (j0 + j) * kWave + lane;
            if ((j0 + j) * kWave < chunks && q < chunks)
                *(uint4 *)(dst + q * 16) = make_uint4(v[j][0], v[j][1], v[j][2], v[j][3]);
        }
    }
}

// Columns 0..W1-1 of the lane's channels in the LDS copy of the region <- e.
template <int SB, int W1>
__device__ __forceinline__ void put_window(char *region, int SL, bool on, int lane,
                                           const uint32_t (&e)[CPL][W1]) {
    if (!on) return;
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
        for (int j = 0; j < W1; ++j) lds_put<SB>(region + ((lane * CPL + ch) * SL + j) * SB, e[ch][j]);
}

// Time-major conv_state (column k holds the d channels contiguously): column j of the
// window e[CPL][W1] as the lane's SCB bytes, stored at column j of the slot.
template <int SB, int W1>
__device__ __forceinline__ void store_window_columns(rsrc_t r, uint32_t lane_off, int64_t col_bytes,
                                                     const uint32_t (&e)[CPL][W1]) {
    constexpr int SW = CPL * SB / 4;
#pragma unroll
    for (int j = 0; j < W1; ++j) {
        uint32_t c[SW];
#pragma unroll
        for (int w = 0; w < SW; ++w)
            c[w] = SB == 4 ? e[w][j] : (e[2 * w][j] | (e[2 * w + 1][j] << 16));
        gstore<CPL * SB>(r, lane_off, (uint32_t)(j * col_bytes), c);
    }
}

// ... and the other way: columns c0 .. c0+W1-1 into e[CPL][W1] (loads in flight; the
// compiler waits where e is used).
template <int SB, int W1>
__device__ __forceinline__ void load_window_columns(rsrc_t r, uint32_t lane_off, int64_t col_bytes,
                                                    int c0, uint32_t (&e)[CPL][W1]) {
    constexpr int SW = CPL * SB / 4;
#pragma unroll
    for (int j = 0; j < W1; ++j) {
        uint32_t c[SW];
        gload<CPL * SB>(r, lane_off, (uint32_t)((c0 + j) * col_bytes), c);
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) e[ch][j] = elem_bits<SB>(c, ch);
    }
}

// A slot's time-major state columns as a buffer resource: state_len columns of
// `col` elements, the wavefront's nch channels at cb.
template <int SB>
__device__ __forceinline__ rsrc_t tm_state_rsrc(void *state, int64_t slot_off, int cb, int SL,
                                                int64_t col, int nch) {
    return make_rsrc((char *)state + (slot_off + cb) * SB, (uint32_t)(((int64_t)(SL - 1) * col + nch) * SB));
}

// ---- accepted-prefix restore ------------------------------------------------------------

// TM: conv_state time-major (p.state_col is the column stride), built separately.
template <int SB, int D, int LAYOUT, bool TM>
__global__ __launch_bounds__(kWave) void cv_restore_kernel(RestoreArgs p) {
    constexpr int W1 = D - 1;
    constexpr int SCB = CPL * SB;
    constexpr int SW = SCB / 4;
    constexpr int RUNB = CPL * W1 * SB;
    extern __shared__ uint4 lds_raw[];
    char *lds = (char *)lds_raw;

    const int lane = threadIdx.x;
    const int row = (int)(blockIdx.x / (unsigned)p.channel_blocks);
    const int cb = (int)(blockIdx.x - (unsigned)row * (unsigned)p.channel_blocks) * CHW;
    const int slot = p.slot_idx ? scalar_read(p.slot_idx, row) : row;
    const int k = scalar_read(p.widx, row);
    if (slot < 0 || slot >= p.n_slots || k < 0 || k >= p.T) return;
    const int nch = min(CHW, p.d_inner - cb);
    const bool on = lane * CPL < nch;

    uint32_t e[CPL][W1];   // the window's elements of the lane's channels, as bits
    if constexpr (LAYOUT == kDense) {
        // window k of the slot: the wavefront's [nch, W1] slab is contiguous
        const rsrc_t w_r = make_rsrc(
            (const char *)p.win + ((int64_t)slot * p.win_slot + ((int64_t)k * p.d_inner + cb) * W1) * SB,
            (uint32_t)(nch * W1 * SB));
        uint32_t run[RUNB / 4];
        const uint32_t lo = on ? (uint32_t)(lane * RUNB) : kOffLane;
#pragma unroll
        for (int q = 0; q < RUNB / 8; ++q) gload<8>(w_r, lo + 8 * q, 0, run + 2 * q);
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
            for (int j = 0; j < W1; ++j) e[ch][j] = run_elem<SB, W1>(run, ch, j);
    } else if constexpr (LAYOUT == kRows) {
        // columns k..k+W1-1 of each channel's row: every 32-byte sector of the
        // wavefront's row block holds some of them, so the block comes in whole
        // (coalesced) through LDS, together with the state region below, and each lane
        // picks its elements out
        const int LS = p.T + W1 - 1;
        const rsrc_t row_r = make_rsrc(
            (const char *)p.win + ((int64_t)slot * p.win_slot + (int64_t)cb * LS) * SB,
            (uint32_t)(nch * LS * SB));
        block_to_lds(row_r, lds, nch * LS * SB / 16, lane);
    } else {
        // time-major rows: column k+j holds the d channels contiguously
        const int LS = p.T + W1 - 1;
        const rsrc_t rt_r = make_rsrc(
            (const char *)p.win + ((int64_t)slot * p.win_slot + cb) * SB,
            (uint32_t)(((int64_t)(LS - 1) * p.d_inner + nch) * SB));
        const uint32_t laneS = on ? (uint32_t)(lane * SCB) : kOffLane;
#pragma unroll
        for (int j = 0; j < W1; ++j) {
            uint32_t col[SW];
            gload<SCB>(rt_r, laneS, (uint32_t)((k + j) * p.d_inner * SB), col);
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) e[ch][j] = elem_bits<SB>(col, ch);
        }
    }

    // the state region (channel-major): rows wider than the window come in whole first
    // (the window columns are then replaced in LDS), and the region leaves whole.
    // Time-major: the window's W1 columns are stored straight from registers.
    const int SL = p.state_len;
    constexpr bool tm = TM;
    const int rchunks = tm ? 0 : nch * SL * SB / 16;
    char *region = lds + (LAYOUT == kRows ? lds_dma_span(CHW * (p.T + W1 - 1) * SB) : 0);
    const rsrc_t st_r = make_rsrc(
        (char *)p.state + ((int64_t)slot * p.state_slot + (int64_t)cb * SL) * SB,
        (uint32_t)(nch * SL * SB));
    if (SL > W1 && !tm) block_to_lds(st_r, region, rchunks, lane);
    __builtin_amdgcn_s_waitcnt(0);   // every load above has landed (in LDS or VGPRs)
    lds_barrier();
    if constexpr (LAYOUT == kRows) {
        const int LS = p.T + W1 - 1;
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
            for (int j = 0; j < W1; ++j)
                e[ch][j] = on ? lds_get<SB>(lds + ((lane * CPL + ch) * LS + k + j) * SB) : 0u;
    }
    if constexpr (tm) {
        const rsrc_t stm_r = tm_state_rsrc<SB>(p.state, (int64_t)slot * p.state_slot, cb, SL,
                                               p.state_col, nch);
        store_window_columns<SB, W1>(stm_r, on ? (uint32_t)(lane * SCB) : kOffLane,
                                     p.state_col * SB, e);
        return;
    }
    put_window<SB, W1>(region, SL, on, lane, e);
    lds_barrier();
    lds_to_global(region, rchunks, st_r, 0, lane);
}

// ---- prefill conv -----------------------------------------------------------------------

template <int XB, int SB, int D, int TC, bool TM>
__global__ __launch_bounds__(kWave) void cv_prefill_kernel(PrefillArgs p) {
    constexpr int W1 = D - 1;
    constexpr int VB = CPL * XB;
    constexpr int XW = VB / 4;
    constexpr int G = 4;   // tokens per branch-free arithmetic chunk

    const int lane = threadIdx.x;
    const unsigned b = blockIdx.x;
    const unsigned r2 = b / (unsigned)p.channel_blocks;
    const int cb = (int)(b - r2 * (unsigned)p.channel_blocks) * CHW;
    const int row = (int)(r2 / (unsigned)p.chunks);
    const int chunk = (int)(r2 - (unsigned)row * (unsigned)p.chunks);

    const int c0 = scalar_read(p.cu, row);
    const int Ti = scalar_read(p.cu, row + 1) - c0;
    const int slot = p.slot_idx ? scalar_read(p.slot_idx, row) : row;
    const bool init = p.has_init ? scalar_read(p.has_init, row) != 0 : true;
    const int t0 = chunk * TC;
    if (Ti < 1 || Ti > p.T || t0 >= Ti || slot < 0 || slot >= p.n_slots) return;
    const int nt = min(TC, Ti - t0);
    const int nch = min(CHW, p.d_inner - cb);
    const bool on = lane * CPL < nch;
    const uint32_t laneV = on ? (uint32_t)(lane * VB) : kOffLane;
    const int SL = p.state_len;

    __builtin_amdgcn_s_setprio(3);
    const rsrc_t x_r = make_rsrc((const char *)p.x + ((int64_t)c0 * p.x_tok + cb) * XB,
                                 (uint32_t)(((int64_t)(Ti - 1) * p.x_tok + nch) * XB));
    uint32_t X[TC][XW];   // x_{t0+t}
#pragma unroll
    for (int t = 0; t < TC; ++t) {
        if (t < nt) {
            gload<VB>(x_r, laneV, (uint32_t)((t0 + t) * p.x_tok * XB), X[t]);
        } else {
#pragma unroll
            for (int w = 0; w < XW; ++w) X[t][w] = 0u;
        }
    }
    // Weights [nch][D] come into LDS past the state region by direct global->LDS
    // loads in lane-contiguous 16-byte chunks (a fraction of the cache-line accesses
    // of per-lane tap loads; every chunk's wavefront reads them).
    extern __shared__ uint4 lds_raw[];
    char *lds = (char *)lds_raw;
    constexpr bool tm = TM;   // time-major conv_state: nothing of it in LDS
    const int w_off = tm ? 0 : CHW * SL * SB;
    {
        const rsrc_t w_r = make_rsrc((const char *)p.weight + (int64_t)cb * D * XB,
                                     (uint32_t)(nch * D * XB));
        const int wchunks = nch * D * XB / 16;   // exact: nch * XB is a multiple of 16
        constexpr int WJ = (CHW * D * XB / 16 + kWave - 1) / kWave;
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            const int q = j * kWave + lane;
            if (j * kWave < wchunks)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    raw(w_r), (lds_void_t *)(lds + w_off + j * kWave * 16), 16,
                    q < wchunks ? (uint32_t)q * 16u : kOffLane, 0, 0, kKeep);
        }
    }
    uint32_t br[XW];
    {
#pragma unroll
        for (int w = 0; w < XW; ++w) br[w] = 0u;
        if (p.bias) {
            const rsrc_t b_r = make_rsrc((const char *)p.bias + (int64_t)cb * XB, (uint32_t)(nch * XB));
            gload<VB, kKeep>(b_r, laneV, 0, br);
        }
    }
    // The W1 inputs before token t0: x for later chunks; for the first chunk the
    // state window (columns 0..W1-1) or zeros.
    float hv[W1][CPL];
    uint32_t hs[W1][CPL];   // first chunk: the state window's bits (zero without one)
    const rsrc_t st_r = make_rsrc(
        (char *)p.state + ((int64_t)slot * p.state_slot + (int64_t)cb * SL) * SB,
        (uint32_t)(nch * SL * SB));
    const int rchunks = nch * SL * SB / 16;
    if (t0 > 0) {
#pragma unroll
        for (int j = 0; j < W1; ++j) {
            uint32_t h[XW];
            gload<VB>(x_r, laneV, (uint32_t)((t0 - W1 + j) * p.x_tok * XB), h);
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) {
                hv[j][ch] = elem_val<XB>(h, ch);
                hs[j][ch] = 0u;
            }
        }
    } else if constexpr (tm) {
        // the first chunk reads the window's W1 columns of the time-major state
        uint32_t e[CPL][W1];
        if (init) {
            load_window_columns<SB, W1>(
                tm_state_rsrc<SB>(p.state, (int64_t)slot * p.state_slot, cb, SL, p.state_col, nch),
                on ? (uint32_t)(lane * CPL * SB) : kOffLane, p.state_col * SB, 0, e);
        }
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
            for (int j = 0; j < W1; ++j) hs[j][ch] = init ? e[ch][j] : 0u;
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
            for (int j = 0; j < W1; ++j) {
                const uint32_t bits = hs[j][ch];
                hv[j][ch] = SB == 4 ? __uint_as_float(bits) : __uint_as_float(bits << 16);
            }
    } else {
        // the first chunk takes the wavefront's state region through LDS (coalesced):
        // its window is the halo, and the region goes back whole with the commit
        if (init || SL > W1) region_load(st_r, lds, rchunks, lane);
        lds_barrier();
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
            for (int j = 0; j < W1; ++j)
                hs[j][ch] = init && on ? lds_get<SB>(lds + ((lane * CPL + ch) * SL + j) * SB) : 0u;
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
            for (int j = 0; j < W1; ++j) {
                const uint32_t bits = hs[j][ch];
                hv[j][ch] = SB == 4 ? __uint_as_float(bits) : __uint_as_float(bits << 16);
            }
    }
    // The first chunk also commits the row's last window: the last W1 of
    // [start window | x_0 .. x_{Ti-1}].
    uint32_t cx[W1][XW];
    if (chunk == 0) {
#pragma unroll
        for (int j = 0; j < W1; ++j) {
            if (Ti - W1 + j >= 0) {
                gload<VB>(x_r, laneV, (uint32_t)((Ti - W1 + j) * p.x_tok * XB), cx[j]);
            } else {
#pragma unroll
                for (int w = 0; w < XW; ++w) cx[j][w] = 0u;
            }
        }
    }
    __builtin_amdgcn_s_setprio(0);

    lds_barrier();
    uint32_t wr[XW * D];   // the lane's weights [CPL][D] (zeros past d_inner)
    lds_read_run<VB * D>(lds + w_off + lane * VB * D, wr);
#pragma unroll
    for (int w = 0; w < XW * D; ++w) wr[w] = on ? wr[w] : 0u;
    float wv[CPL][D];
    float bv[CPL];
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
#pragma unroll
        for (int w = 0; w < D; ++w) wv[ch][w] = elem_val<XB>(wr, ch * D + w);
        bv[ch] = elem_val<XB>(br, ch);
    }
    // v[k]: k < W1 the inputs before t0, else x_{t0+k-W1}; k compile-time
    auto val = [&](int k, int ch) -> float {
        return k < W1 ? hv[k < W1 ? k : 0][ch] : elem_val<XB>(X[k < W1 ? 0 : k - W1], ch);
    };

    const rsrc_t o_r = make_rsrc((char *)p.out + ((int64_t)c0 * p.out_tok + cb) * XB,
                                 (uint32_t)(((int64_t)(Ti - 1) * p.out_tok + nch) * XB));
#pragma unroll
    for (int g0 = 0; g0 < TC; g0 += G) {
        if (g0 < nt) {
            float y[G][CPL];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) {
                    float acc = bv[ch];
#pragma unroll
                    for (int w = 0; w < D; ++w)
                        acc = __builtin_fmaf(wv[ch][w], val(g0 + g + w, ch), acc);
                    y[g][ch] = acc;
                }
            silu_rows_checked<G>(y);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (g0 + g < nt) {
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
                    gstore<VB>(o_r, laneV, (uint32_t)((t0 + g0 + g) * p.out_tok * XB), o);
                }
            }
        }
    }

    if (chunk == 0) {
        // u = [start window | x_0 ..]: the committed window is u[Ti .. Ti+W1-1]; an
        // element with u-index m < W1 is start window column m (rows shorter than W1).
        uint32_t e[CPL][W1];
#pragma unroll
        for (int j = 0; j < W1; ++j) {
            const int m = Ti + j;
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) {
                uint32_t v = x_to_state_bits<XB, SB>(elem_bits<XB>(cx[j], ch));
#pragma unroll
                for (int q = 0; q < W1; ++q)
                    if (m == q) v = hs[q][ch];
                e[ch][j] = v;
            }
        }
        if constexpr (tm) {
            store_window_columns<SB, W1>(
                tm_state_rsrc<SB>(p.state, (int64_t)slot * p.state_slot, cb, SL, p.state_col, nch),
                on ? (uint32_t)(lane * CPL * SB) : kOffLane, p.state_col * SB, e);
            return;
        }
        put_window<SB, W1>(lds, SL, on, lane, e);
        lds_barrier();
        lds_to_global(lds, rchunks, st_r, 0, lane);
    }
}

// ---- token-split verify (dense windows) --------------------------------------------------
//
// The verify of cv_verify_kernel with a row's T tokens spread over ceil(T / TC)
// wavefronts per 256 channels, for grids too small to fill the chip (a few rows of
// many draft tokens).  Tokens are independent given their D-1 predecessors, so chunk
// k computes out and the dense snapshots of tokens [k*TC, k*TC+TC) from x alone,
// with the D-1 tokens before the chunk as its halo; chunk 0 takes its halo from the
// state window at column a and is also the wavefront that commits the row's last
// window, so a slot's state read and write stay in one wavefront and chunks never
// race.  (Dense snapshots only: a channel-major row is shared by every chunk of a
// channel.)  Same arithmetic, same order, same rounding as the verify kernel.
template <int XB, int SB, int D, int TC, bool TM>
__global__ __launch_bounds__(kWave) void cv_split_kernel(KernelArgs p) {
    static_assert(TC >= D - 1, "the halo of a chunk must come from the chunk before");
    constexpr int W1 = D - 1;
    constexpr int VB = CPL * XB;
    constexpr int XW = VB / 4;
    constexpr int RUNB = CPL * W1 * SB;   // a lane's [CPL][W1] window run
    constexpr int RUNW = RUNB / 4;
    extern __shared__ uint4 lds_raw[];
    char *lds = (char *)lds_raw;

    const int lane = threadIdx.x;
    const unsigned b = blockIdx.x;
    const unsigned r2 = b / (unsigned)p.channel_blocks;
    int cend;   // the end of this block's channels
    const int cb = block_first(p.heads, (int)(b - r2 * (unsigned)p.channel_blocks), p.qk, p.d_inner, cend);
    const int row = (int)(r2 / (unsigned)p.token_chunks);
    const int chunk = (int)(r2 - (unsigned)row * (unsigned)p.token_chunks);

    const int slot = p.slot_idx ? scalar_read(p.slot_idx, row) : row;
    const int a = p.nat ? scalar_read(p.nat, row) : 0;
    int T = p.T;
    int64_t xrow = (int64_t)row * p.x_seq, orow = (int64_t)row * p.out_seq;
    if (p.cu) {
        const int c0 = scalar_read(p.cu, row);
        T = scalar_read(p.cu, row + 1) - c0;
        xrow = (int64_t)c0 * p.x_tok;
        orow = (int64_t)c0 * p.out_tok;
        if (T < 1 || T > p.T) return;
    }
    const int t0 = chunk * TC;
    if (t0 >= T) return;
    const int nt = min(TC, T - t0);
    const int SL = p.state_len;
    const int nch = min(CHW, cend - cb);
    const bool on = lane * CPL < nch;
    const uint32_t laneV = on ? (uint32_t)(lane * VB) : kOffLane;

    // ---- loads: the chunk's x and halo, the weights (LDS), bias, the commit's inputs
    __builtin_amdgcn_s_setprio(3);
    const rsrc_t x_r = make_rsrc((const char *)p.x + (xrow + cb) * XB,
                                 (uint32_t)(((int64_t)(T - 1) * p.x_tok + nch) * XB));
    uint32_t X[W1 + TC][XW];   // v[t0 + k] for k >= W1 (x_{t0+k-W1}); k < W1: the x halo
#pragma unroll
    for (int j = 0; j < TC; ++j) {
        if (j < nt) {
            gload<VB>(x_r, laneV, (uint32_t)((t0 + j) * p.x_tok * XB), X[W1 + j]);
        } else {
#pragma unroll
            for (int w = 0; w < XW; ++w) X[W1 + j][w] = 0u;
        }
    }
#pragma unroll
    for (int h = 0; h < W1; ++h) {
        if (chunk > 0) {
            gload<VB>(x_r, laneV, (uint32_t)((t0 - W1 + h) * p.x_tok * XB), X[h]);
        } else {
#pragma unroll
            for (int w = 0; w < XW; ++w) X[h][w] = 0u;
        }
    }
    constexpr bool tm = TM;   // time-major conv_state: nothing of it in LDS
    const int w_off = tm ? 0 : CHW * SL * SB;   // past chunk 0's state region
    {
        const rsrc_t w_r = make_rsrc((const char *)p.weight + (int64_t)cb * D * XB,
                                     (uint32_t)(nch * D * XB));
        const int wchunks = nch * D * XB / 16;   // exact: nch * XB is a multiple of 16
        constexpr int WJ = (CHW * D * XB / 16 + kWave - 1) / kWave;
#pragma unroll
        for (int j = 0; j < WJ; ++j) {
            const int q = j * kWave + lane;
            if (j * kWave < wchunks)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    raw(w_r), (lds_void_t *)(lds + w_off + j * kWave * 16), 16,
                    q < wchunks ? (uint32_t)q * 16u : kOffLane, 0, 0, kKeep);
        }
    }
    uint32_t br[XW];
#pragma unroll
    for (int w = 0; w < XW; ++w) br[w] = 0u;
    if (p.bias) {
        const rsrc_t b_r = make_rsrc((const char *)p.bias + (int64_t)cb * XB, (uint32_t)(nch * XB));
        gload<VB, kKeep>(b_r, laneV, 0, br);
    }
    // chunk 0 commits v[T .. T+W1-1]: x_{T-W1+j}, or start-window column T+j (T < W1)
    uint32_t cx[W1][XW];
#pragma unroll
    for (int j = 0; j < W1; ++j) {
        if (chunk == 0 && T - W1 + j >= 0) {
            gload<VB>(x_r, laneV, (uint32_t)((T - W1 + j) * p.x_tok * XB), cx[j]);
        } else {
#pragma unroll
            for (int w = 0; w < XW; ++w) cx[j][w] = 0u;
        }
    }
    // Padded rows (slot -1), and rows whose slot or offset would address outside the
    // buffers, write nothing; the loads above stay in bounds - wait for them and leave.
    if (slot < 0 || slot >= p.n_slots || a < 0 || a > SL - W1) {
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }
    const rsrc_t st_r = make_rsrc((char *)p.state + ((int64_t)slot * p.state_slot + (int64_t)cb * SL) * SB,
                                  (uint32_t)(nch * SL * SB));
    const int rchunks = tm ? 0 : nch * SL * SB / 16;
    const rsrc_t stm_r = tm_state_rsrc<SB>(p.state, (int64_t)slot * p.state_slot, cb, SL, p.state_col, nch);
    const uint32_t laneS = on ? (uint32_t)(lane * CPL * SB) : kOffLane;
    uint32_t tw[CPL][W1];   // time-major: chunk 0's start window, columns a..a+W1-1
    if constexpr (tm) {
        if (chunk == 0) load_window_columns<SB, W1>(stm_r, laneS, p.state_col * SB, a, tw);
    } else {
        if (chunk == 0) region_load(st_r, lds, rchunks, lane);   // the whole region, through LDS
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the weights have landed
    lds_barrier();

    uint32_t wr[XW * D];   // the lane's weights [CPL][D] (zeros past d_inner)
    lds_read_run<VB * D>(lds + w_off + lane * VB * D, wr);
#pragma unroll
    for (int w = 0; w < XW * D; ++w) wr[w] = on ? wr[w] : 0u;
    float wv[CPL][D];
    float bv[CPL];
#pragma unroll
    for (int ch = 0; ch < CPL; ++ch) {
#pragma unroll
        for (int w = 0; w < D; ++w) wv[ch][w] = elem_val<XB>(wr, ch * D + w);
        bv[ch] = elem_val<XB>(br, ch);
    }
    // the halo v[t0 .. t0+W1-1] as state-typed bits: the start window (chunk 0), else x
    uint32_t hs[W1][CPL];
#pragma unroll
    for (int j = 0; j < W1; ++j)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch)
            hs[j][ch] = chunk == 0 ? (tm ? tw[ch][j]
                                         : on ? lds_get<SB>(lds + ((lane * CPL + ch) * SL + a + j) * SB) : 0u)
                                   : x_to_state_bits<XB, SB>(elem_bits<XB>(X[j], ch));
    // v[t0 + k], k compile-time: the halo (exact in either type) or x
    auto val = [&](int k, int ch) -> float {
        if (k < W1) {
            const uint32_t bits = hs[k < W1 ? k : 0][ch];
            return SB == 4 ? __uint_as_float(bits) : __uint_as_float(bits << 16);
        }
        return elem_val<XB>(X[k], ch);
    };
    auto sbits = [&](int k, int ch) -> uint32_t {
        return k < W1 ? hs[k < W1 ? k : 0][ch] : x_to_state_bits<XB, SB>(elem_bits<XB>(X[k], ch));
    };

    // ---- conv + SiLU + per-head L2 -> out (one branch-free chunk)
    float y[TC][CPL];
#pragma unroll
    for (int g = 0; g < TC; ++g)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) {
            float acc = bv[ch];
#pragma unroll
            for (int w = 0; w < D; ++w) acc = __builtin_fmaf(wv[ch][w], val(g + w, ch), acc);
            y[g][ch] = acc;
        }
    silu_rows_checked<TC>(y);
    if (cb < p.qk)   // uniform: this wavefront holds q|k channels
        head_l2<TC>(y, on && lane * CPL + cb < p.qk, p.head_lanes_log2, p.heads.head_lanes, p.eps);
    const rsrc_t o_r = make_rsrc((char *)p.out + (orow + cb) * XB,
                                 (uint32_t)(((int64_t)(T - 1) * p.out_tok + nch) * XB));
#pragma unroll
    for (int g = 0; g < TC; ++g) {
        if (g < nt) {
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
            gstore<VB>(o_r, laneV, (uint32_t)((t0 + g) * p.out_tok * XB), o);
        }
    }

    // ---- chunk 0: the committed window into the staged region, which leaves whole
    if (chunk == 0) {
        uint32_t e[CPL][W1];
#pragma unroll
        for (int j = 0; j < W1; ++j) {
            const int m = T + j;   // v index; m < W1: start-window column m
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) {
                uint32_t v = x_to_state_bits<XB, SB>(elem_bits<XB>(cx[j], ch));
#pragma unroll
                for (int q = 0; q < W1; ++q)
                    if (m == q) v = hs[q][ch];
                e[ch][j] = v;
            }
        }
        if constexpr (tm) {
            store_window_columns<SB, W1>(stm_r, laneS, p.state_col * SB, e);
        } else {
            put_window<SB, W1>(lds, SL, on, lane, e);
            lds_barrier();
            lds_to_global(lds, rchunks, st_r, 0, lane);
        }
    }

    // ---- dense snapshots of the chunk's tokens: snapshot t = v[t+1 .. t+W1]; the
    // wavefront's [nch, W1] slab is contiguous and leaves through one of two
    // alternating LDS slabs in lane-contiguous 16-byte units
    constexpr int SLAB = CHW * W1 * SB;
    char *slabs = lds + w_off + lds_dma_span(CHW * D * XB);
    const int slab_chunks = nch * W1 * SB / 16;   // exact: nch * SB is a multiple of 16
    const rsrc_t snap_r = make_rsrc(
        (char *)p.win + ((int64_t)slot * p.win_slot + (int64_t)cb * W1) * SB,
        (uint32_t)(((int64_t)(T - 1) * p.d_inner * W1 + (int64_t)nch * W1) * SB));
#pragma unroll
    for (int g = 0; g < TC; ++g) {
        if (g < nt) {
            uint32_t run[RUNW];   // [CPL][W1], channel-major
#pragma unroll
            for (int w = 0; w < RUNW; ++w) {
                if constexpr (SB == 4) {
                    run[w] = sbits(g + 1 + w % W1, w / W1);
                } else {
                    const int e0 = 2 * w, e1 = 2 * w + 1;
                    run[w] = sbits(g + 1 + e0 % W1, e0 / W1) | (sbits(g + 1 + e1 % W1, e1 / W1) << 16);
                }
            }
            char *slab = slabs + (g & 1) * SLAB;
            lds_write_run<RUNB>(slab + lane * RUNB, run);
            lds_barrier();
            lds_to_global(slab, slab_chunks, snap_r, (uint32_t)((t0 + g) * p.d_inner * W1 * SB), lane);
        }
    }
}

// ---- separate per-head L2 over q|k -------------------------------------------------------

template <int XB>
__global__ __launch_bounds__(kWave) void cv_l2_kernel(L2Args p) {
    constexpr int VB = CPL * XB;
    constexpr int XW = VB / 4;
    constexpr int R = kL2Rows;   // token rows of this wavefront, all loads in flight together
    const int lane = threadIdx.x;
    const int64_t rb = (int64_t)(blockIdx.x / (unsigned)p.qk_blocks);
    int cend;   // the end of this block's channels (the q|k blocks end at qk)
    const int cb = block_first(p.heads, (int)(blockIdx.x - (unsigned)rb * (unsigned)p.qk_blocks), p.qk,
                               p.qk, cend);
    const int64_t r0 = rb * R;
    const int nr = (int)min((int64_t)R, p.n_rows - r0);   // >= 1: the grid covers the rows once
    const int nch = min(CHW, cend - cb);
    const bool on = lane * CPL < nch;
    const uint32_t laneV = on ? (uint32_t)(lane * VB) : kOffLane;
    const rsrc_t x_r = make_rsrc((char *)p.x + (r0 * p.row_stride + cb) * XB,
                                 (uint32_t)(((int64_t)(nr - 1) * p.row_stride + nch) * XB));
    uint32_t w[R][XW];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < nr) {
            gload<VB>(x_r, laneV, (uint32_t)(r * p.row_stride * XB), w[r]);
        } else {
#pragma unroll
            for (int q = 0; q < XW; ++q) w[r][q] = 0u;
        }
    }
    float y[R][CPL];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) y[r][ch] = elem_val<XB>(w[r], ch);
    // a head never straddles the block's end (a block holds whole heads), so lanes past
    // it form groups of their own; they store nothing
    head_l2<R>(y, on, p.head_lanes_log2, p.heads.head_lanes, p.eps);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < nr) {
            uint32_t o[XW];
            if constexpr (XB == 4) {
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) o[ch] = __float_as_uint(y[r][ch]);
            } else {
                typedef float f2 __attribute__((ext_vector_type(2)));
                typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
                for (int q = 0; q < XW; ++q) {
                    f2 pr = {y[r][2 * q], y[r][2 * q + 1]};
                    o[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, b2));
                }
            }
            gstore<VB>(x_r, laneV, (uint32_t)(r * p.row_stride * XB), o);
        }
    }
}

template <int SB, int LAYOUT, bool TM>
const void *restore_for(int d_conv) {
    switch (d_conv) {
        case 2: return (const void *)cv_restore_kernel<SB, 2, LAYOUT, TM>;
        case 3: return (const void *)cv_restore_kernel<SB, 3, LAYOUT, TM>;
        case 4: return (const void *)cv_restore_kernel<SB, 4, LAYOUT, TM>;
        default: return nullptr;
    }
}

template <int SB, bool TM>
const void *restore_layout(int d_conv, int layout) {
    if (layout == kDense) return restore_for<SB, kDense, TM>(d_conv);
    if (layout == kRows) return restore_for<SB, kRows, TM>(d_conv);
    if (layout == kRowsT) return restore_for<SB, kRowsT, TM>(d_conv);
    return nullptr;
}

template <int XB, int SB, bool TM>
const void *split_for(int d_conv) {
    switch (d_conv) {
        case 2: return (const void *)cv_split_kernel<XB, SB, 2, kSplitChunk, TM>;
        case 3: return (const void *)cv_split_kernel<XB, SB, 3, kSplitChunk, TM>;
        case 4: return (const void *)cv_split_kernel<XB, SB, 4, kSplitChunk, TM>;
        default: return nullptr;
    }
}

template <int XB, int SB, bool TM>
const void *prefill_for(int d_conv) {
    switch (d_conv) {
        case 2: return (const void *)cv_prefill_kernel<XB, SB, 2, kPrefillChunk, TM>;
        case 3: return (const void *)cv_prefill_kernel<XB, SB, 3, kPrefillChunk, TM>;
        case 4: return (const void *)cv_prefill_kernel<XB, SB, 4, kPrefillChunk, TM>;
        default: return nullptr;
    }
}

}  // namespace

#ifdef CV_WRITE_COUNT
int count_ranges_set_aux(const CountRanges &c) {
    void *dst = nullptr;
    const hipError_t e = hipGetSymbolAddress(&dst, HIP_SYMBOL(CV_COUNT_RANGES));
    if (e != hipSuccess) return (int)e;
    return (int)hipMemcpy(dst, &c, sizeof c, hipMemcpyHostToDevice);
}
#endif

const void *pick_restore(int state_bytes, int d_conv, int layout, int tm) {
    if (state_bytes == 4) return tm ? restore_layout<4, true>(d_conv, layout) : restore_layout<4, false>(d_conv, layout);
    if (state_bytes == 2) return tm ? restore_layout<2, true>(d_conv, layout) : restore_layout<2, false>(d_conv, layout);
    return nullptr;
}

const void *pick_split(int x_bytes, int state_bytes, int d_conv, int tm) {
    if (x_bytes == 4 && state_bytes == 4) return tm ? split_for<4, 4, true>(d_conv) : split_for<4, 4, false>(d_conv);
    if (x_bytes == 2 && state_bytes == 2) return tm ? split_for<2, 2, true>(d_conv) : split_for<2, 2, false>(d_conv);
    if (x_bytes == 2 && state_bytes == 4) return tm ? split_for<2, 4, true>(d_conv) : split_for<2, 4, false>(d_conv);
    return nullptr;
}

const void *pick_prefill(int x_bytes, int state_bytes, int d_conv, int tm) {
    if (x_bytes == 4 && state_bytes == 4) return tm ? prefill_for<4, 4, true>(d_conv) : prefill_for<4, 4, false>(d_conv);
    if (x_bytes == 2 && state_bytes == 2) return tm ? prefill_for<2, 2, true>(d_conv) : prefill_for<2, 2, false>(d_conv);
    if (x_bytes == 2 && state_bytes == 4) return tm ? prefill_for<2, 4, true>(d_conv) : prefill_for<2, 4, false>(d_conv);
    return nullptr;
}

const void *pick_l2(int x_bytes) {
    if (x_bytes == 4) return (const void *)cv_l2_kernel<4>;
    if (x_bytes == 2) return (const void *)cv_l2_kernel<2>;
    return nullptr;
}

}  // namespace cvimpl
