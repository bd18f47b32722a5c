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
//    wavefront; the 1-D grid is n_seq * ceil(d_inner / 256) workgroups (with heads that
//    do not divide 256 channels, the q|k blocks hold whole heads instead).  (256-channel
//    blocks stream measurably faster on MI355X than 512-channel ones for this traffic
//    mix: twice the wavefronts keep more requests in flight.)  The line-aligned 16-token
//    build groups 4 such wavefronts over 1024 channels, so that the store ranges they
//    share leave through LDS cut at 128-byte lines (see verify_body's NW).
//  * Every global access is a lane-contiguous 8- or 16-byte buffer access: x and out
//    per token, the columns of a time-major conv_state and of time-major rows, and
//    every run of a channel-major conv_state, the dense snapshots and the dedup rows,
//    which are staged through LDS so that they too leave in lane-contiguous units.
//    Per-token offsets live in SGPRs.  Loads and stores use the nt (streaming) policy,
//    except the weights and bias, which every row's wavefronts read, and the stores of
//    time-major builds on rows that start off 128-byte lines (default policy).
//  * All loads (weights, bias, x for every token, conv_state) are issued up front,
//    with raised wave priority.  Most builds then wait for all of them once, so that no
//    wait on a load is ever stuck behind stores (vmcnt counts both in issue order).
//    The time-major builds of more than one token chunk instead compute each chunk as
//    its x lands, chunk 0 (the one that takes the conv_state window, whose loads go
//    out last) at the end.  LDS hand-offs use barriers that order LDS only.
//  * The arithmetic runs in branch-free token chunks; the rollback windows and the
//    committed state (pure copies of the inputs) follow.
//  * The conv is one fused multiply-add per tap in tap order (bias first), the same
//    order as the per-token path it replaces, so the pre-activation is bit-identical
//    to a correctly rounded fp32 evaluation of that order.
//  * L2: a head of H channels spans H/4 lanes; its sum of squares is a butterfly with
//    DPP inside 16-lane rows (quad_perm, row_half_mirror, row_mirror) and gfx950 lane
//    swaps (permlane16/32) beyond; every lane of a head ends with the same sum.  A head
//    whose lane count is not a power of two would straddle wavefronts: there the q|k
//    channels go in blocks of whole heads (block_first) and each head's sum is a
//    segmented scan across its lanes (group_sums_any).
//  * Windows and conv_state move as bit patterns; only the conv reads them as floats.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#define CV_COUNT_RANGES_NAME(xb, sb, v, tm) cv_count_ranges_##xb##_##sb##_##v##_##tm
#define CV_COUNT_RANGES_OF(xb, sb, v, tm) CV_COUNT_RANGES_NAME(xb, sb, v, tm)
#define CV_COUNT_RANGES CV_COUNT_RANGES_OF(CV_XB, CV_SB, CV_VARIANT, CV_TM)
#include "cv_device.h"
#include "cv_internal.h"

namespace cvimpl {
namespace {

// ---- the kernel -------------------------------------------------------------------------

// LAYOUT: kDense, kRows or kRowsT (rollback windows); TREE: per-token parents (dense
// windows, nothing committed).  Packed rows (p.cu) are a runtime option of every variant.
// WPE > 0 asks the register allocator for WPE resident wavefronts per SIMD: the
// 16-token bucket is built a second time that way (at most 102 VGPRs, a few spilled),
// for launches whose LDS allows 5 per SIMD, so that a 128-row grid stays resident in
// one generation.
// SPLIT (row layouts, buckets 8 and 16): on a small grid a row's 4-token chunks go to
// p.token_chunks wavefronts.  Each computes out for its own chunk only; chunk 0 also
// does every copy (the state commit and the row block, which is shared by all the
// row's tokens), so the arithmetic on each wavefront's path is a quarter to a half.
// TM: conv_state time-major (p.state_col is the column stride), a build of its own so
// that neither layout's path costs the other registers.
// NW: wavefronts per workgroup.  NW 4 is the line-aligned build (time-major state, row
// layout, full 16-token rows): the workgroup's 4 wavefronts take 1024 consecutive
// channels, and every store range they share (a token of out, a column of the state,
// the row block) goes through LDS and leaves cut at the destination's 128-byte lines, so
// that only the workgroup's two end lines of each range are written in part.  Where rows
// start off those lines, one wavefront per 256 channels splits a line between two
// wavefronts' stores at every wavefront boundary: a streaming probe of the stress
// traffic at d 10200 ran 132.6 us that way and 113.2 us line-aligned, against 108.4 us
// at d 10240; the verify itself went from 116-118 to 106 us there.
// SPOL: the cache policy of every store (the kernel below picks it).
template <int XB, int SB, int D, int TB, int LAYOUT, bool TREE, int WPE, bool SPLIT, bool TM, int NW,
          int SPOL>
__device__ __forceinline__ void verify_body(const KernelArgs &p) {
    static_assert(!TREE || LAYOUT == kDense, "tree windows are dense");
    static_assert(!SPLIT || (!TREE && LAYOUT != kDense), "dense chains split in cv_split_kernel");
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
    // Tokens go in chunks with no branch inside a chunk: buckets up to 8 are one chunk;
    // larger ones use chunks of 4, which bounds the registers and the work past T.
    constexpr int G = TB <= 8 && !SPLIT ? TB : 4;
    // A time-major build of more than one token chunk starts computing as its loads
    // land, rather than after all of them: the compiler's waits before each use count
    // outstanding loads (and stores) in issue order.  Its loads therefore go out in a
    // fixed number, whatever T and the bias, so that those counts are exact on every
    // path: every x token of the bucket (those past T as out-of-range loads, which read
    // zeros) and the bias (out of range when there is none).  The chunks
    // that take no state column (tokens W1 and later) go first; the state's W1 column
    // loads are issued once the first of them has its results, so that they are not
    // held in registers through it, and land while the other chunks compute.
    constexpr bool PIPE = TM && !TREE && !SPLIT && G < TB;
    constexpr bool LA = NW > 1;
    static_assert(!LA || (!TREE && !SPLIT && G < TB && LAYOUT == kRows && TB == 16 && WPE == 0 &&
                          XB == SB),
                  "the line-aligned build: row layout, 16-token rows");
    // The line-aligned build with a channel-major state: the 4 wavefronts' state regions
    // lie side by side in LDS as the workgroup's one contiguous region, placed after the
    // bytes of its first 128-byte line that precede it; the exchange buffers of out follow
    // the region, which stays staged through the arithmetic, takes the committed window
    // in the copy phase and leaves cut at lines.
    constexpr bool LACM = LA && !TM;
    constexpr int RANGE = NW * CHW;           // channels of a workgroup

    extern __shared__ uint4 lds_raw[];
    char *lds = (char *)lds_raw;

    const int tid = threadIdx.x;
    const int lane = LA ? tid % kWave : tid;
    const int wave = LA ? __builtin_amdgcn_readfirstlane(tid / kWave) : 0;
    const unsigned bid = p.xcd_remap ? xcd_linear(blockIdx.x, gridDim.x) : blockIdx.x;
    const int r2 = (int)(bid / (unsigned)p.channel_blocks);
    const int blk = (int)(bid - (unsigned)r2 * (unsigned)p.channel_blocks);
    // (the line-aligned build runs with uniform blocks only)
    int cend = p.d_inner;                       // the end of this block's channels
    const int cbg = LA ? blk * RANGE : block_first(p.heads, blk, p.qk, p.d_inner, cend);
    const int cb = cbg + wave * CHW;            // this wavefront's first channel
    // Tree verify on a small grid spreads a row's token chunks over p.token_chunks
    // wavefronts: each one builds the row's whole v tile (a token's ancestors may be
    // any earlier token) and computes and writes only its own chunk of tokens.
    int row = r2, chunk = 0;
    if constexpr (TREE || SPLIT) {
        row = r2 / p.token_chunks;
        chunk = r2 - row * p.token_chunks;
    }
    const bool copier = !SPLIT || chunk == 0;   // this wavefront does the copies

    // The row's slot and offset are read now (scalar loads) and tested once the loads
    // that do not depend on them are on their way.
    const int slot = p.slot_idx ? scalar_read(p.slot_idx, row) : row;
    const int a = p.nat ? scalar_read(p.nat, row) : 0;

    // Tokens of this row and where they start.  Packed rows take both from cu_seqlens;
    // an empty row (or one outside 1..T) has nothing to compute and writes nothing.
    int T = p.T;
    int64_t xrow = (int64_t)row * p.x_seq, orow = (int64_t)row * p.out_seq;
    if (p.cu) {
        const int c0 = scalar_read(p.cu, row);
        T = scalar_read(p.cu, row + 1) - c0;
        xrow = (int64_t)c0 * p.x_tok;
        orow = (int64_t)c0 * p.out_tok;
        if (T < 1 || T > p.T) return;
    }
    if constexpr (TREE || SPLIT) {
        if (chunk * G >= T) return;   // a split row's chunk past its tokens
    }
    if constexpr (LA) {
        if (p.cu || T != TB) return;   // launched for full unpacked rows only
    }
    if (p.slot_first) {
        if (slot < 0) return;   // a padded row on a multi-generation grid: no load at all
    }
    const int SL = p.state_len;
    // channels of this wavefront (none for the last wavefronts of a line-aligned
    // workgroup past d_inner: they take part in the workgroup's exchanges only)
    const int nch = max(0, min(CHW, cend - cb));
    const int nchg = min(RANGE, p.d_inner - cbg);   // channels of the workgroup
    const bool on = lane * CPL < nch;
    const uint32_t laneV = on ? (uint32_t)(lane * VB) : kOffLane;
    const bool contiguous_state = SL == W1;

    // ---- every load, issued up front -------------------------------------------------------
    // Raised wave priority while this wavefront issues its loads: when several
    // wavefronts of a SIMD are ready, the ones still issuing loads go first, so reads
    // enter the memory pipeline ahead of other wavefronts' stores.
    __builtin_amdgcn_s_setprio(3);

    // Weights [nch][D]: the wavefront's block is contiguous, and comes into LDS by
    // direct global->LDS loads in lane-contiguous 16-byte chunks.  Per-lane loads of
    // each lane's D taps would touch D/2..D times as many cache lines per instruction;
    // the weights are read by every row's wavefront, so those extra line accesses were
    // a measurable share of the launch.  They land at the start of LDS and go to VGPRs
    // once every load has landed, before the state region is written over them: the
    // two share LDS, which keeps the wavefront's LDS (and so its occupancy) that of the
    // state region alone.  A direct load fills kWave * 16 bytes of LDS per instruction,
    // so the weights' LDS is reserved in whole multiples of that.
    // A pipelined build loads each lane's weights straight into VGPRs instead (its
    // contiguous [CPL][D] run, in 16- or 8-byte loads): the compiler cannot count a
    // global->LDS load's completion precisely, and would wait for every load before
    // reading the weights from LDS.
    uint32_t wr[XW * D];   // the lane's weights [CPL][D] (zeros past d_inner)
    {
        const rsrc_t w_r = make_rsrc((const char *)p.weight + (int64_t)cb * D * XB,
                                     (uint32_t)(nch * D * XB));
        if constexpr (PIPE || LA) {
            constexpr int WP = VB * D % 16 == 0 ? 16 : 8;   // bytes per load
#pragma unroll
            for (int j = 0; j < VB * D / WP; ++j)
                gload<WP, kKeep>(w_r, on ? (uint32_t)(lane * VB * D + WP * j) : kOffLane, 0,
                                 wr + WP / 4 * j);
        } else {
            const int wchunks = nch * D * XB / 16;   // exact: nch * XB is a multiple of 16
            constexpr int WJ = (CHW * D * XB / 16 + kWave - 1) / kWave;
#pragma unroll
            for (int j = 0; j < WJ; ++j) {
                const int q = j * kWave + lane;
                if (j * kWave < wchunks)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        raw(w_r), (lds_void_t *)(lds + j * kWave * 16), 16,
                        q < wchunks ? (uint32_t)q * 16u : kOffLane, 0, 0, kKeep);
            }
        }
    }
    uint32_t br[XW];              // bias [CPL]
    {
#pragma unroll
        for (int w = 0; w < XW; ++w) br[w] = 0u;
        if (PIPE || p.bias) {
            // without a bias: a resource of no bytes (every lane out of range, zeros)
            const rsrc_t b_r = make_rsrc(p.bias ? (const char *)p.bias + (int64_t)cb * XB
                                                : (const char *)p.weight,
                                         p.bias ? (uint32_t)(nch * XB) : 0u);
            gload<VB, kKeep>(b_r, laneV, 0, br);
        }
    }
    const rsrc_t x_r = make_rsrc((const char *)p.x + (xrow + cb) * XB,
                                 (uint32_t)(((int64_t)(T - 1) * p.x_tok + nch) * XB));
    uint32_t X[TB][XW];   // x_t for the lane's channels
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        // a split row's later chunks need only their tokens and the W1 before them
        const bool need = copier || (t >= chunk * G - W1 && t < chunk * G + G);
        if constexpr (PIPE) {   // tokens past T: out-of-range loads of zeros
            gload<VB>(x_r, t < T ? laneV : kOffLane, t < T ? (uint32_t)(t * p.x_tok * XB) : 0u, X[t]);
        } else if (t < T && need) {
            gload<VB>(x_r, laneV, (uint32_t)(t * p.x_tok * XB), X[t]);
        } else {
#pragma unroll
            for (int w = 0; w < XW; ++w) X[t][w] = 0u;
        }
    }

    // Padded rows (slot -1) leave before any store; rows with an index that would
    // address outside the buffers are skipped the same way.  The loads above stay in
    // bounds for every row; wait for them before leaving.
    if (slot < 0 || slot >= p.n_slots || a < 0 || a > p.state_len - W1) {
        __builtin_amdgcn_s_waitcnt(0);
        return;
    }

    // conv_state, channel-major: the wavefront's [nch, state_len] region is contiguous.
    // It comes in whole (coalesced 16-byte loads, issued with the other loads) and is
    // staged in LDS; each lane picks its channels' window out of it, writes its
    // committed window back into it, and the region leaves whole - so every state byte
    // is read once and written once in lane-contiguous 16-byte units, whatever
    // state_len and the offset are.  (Direct global->LDS loads measured no faster here
    // than loads through VGPRs.)
    // Time-major: column k holds the d channels contiguously, so the window is W1
    // lane-contiguous column loads at columns a.., like x, and the commit W1 column
    // stores at columns 0..W1-1; the other columns are never touched.
    constexpr bool tm = TM;
    const rsrc_t st_r = make_rsrc((const char *)p.state + ((int64_t)slot * p.state_slot +
                                                           (int64_t)cb * SL) * SB,
                                  (uint32_t)(nch * SL * SB));
    const rsrc_t stm_r = make_rsrc((const char *)p.state + ((int64_t)slot * p.state_slot + cb) * SB,
                                   (uint32_t)(((int64_t)(SL - 1) * p.state_col + nch) * SB));
    const uint32_t laneS = on ? (uint32_t)(lane * SCB) : kOffLane;
    uint32_t S[W1][SW];   // initial window columns v[0..W1-1], state-typed bits
    auto load_state_columns = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < W1; ++j) {
            if (copier) {
                gload<SCB>(stm_r, laneS, (uint32_t)((int64_t)(a + j) * p.state_col * SB), S[j]);
            } else {
#pragma unroll
                for (int w = 0; w < SW; ++w) S[j][w] = 0u;
            }
        }
    };
    if constexpr (tm && !PIPE) load_state_columns();
    // exact: nch * SB is a multiple of 16; a split row's other chunks take no state
    const int rchunks = copier && !tm ? nch * SL * SB / 16 : 0;
    // line-aligned, channel-major: where this wavefront's region sits in LDS
    const int64_t sreg_off = ((int64_t)slot * p.state_slot + (int64_t)cbg * SL) * SB;   // bytes
    const int s_delta = LACM ? (int)(((uint64_t)(uintptr_t)p.state + (uint64_t)sreg_off) & 127u) : 0;
    char *const rgn = lds + (LACM ? s_delta + wave * CHW * SL * SB : 0);
    // chunks per lane, all in flight at once up to RJ; longer regions go in rounds
    constexpr int RJ = (W1 * SB + 3) / 4 > 12 ? (W1 * SB + 3) / 4 : 12;
    uint32_t sreg[RJ][4];
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const int q = j * kWave + lane;
        if (j * kWave < rchunks) gload<16>(st_r, q < rchunks ? (uint32_t)q * 16u : kOffLane, 0, sreg[j]);
    }
    // Packed rows shorter than the buffer's rows (row layout): the slot's stored row block
    // comes into LDS too (the copy phase rewrites its columns below the row's length and
    // stores it whole).  Builds that wait for every load at once load it here, with the
    // others, past both the weights and the state region; pipelined builds, whose waits
    // count loads in issue order, load it in the copy phase.
    constexpr bool IMG_EARLY = LAYOUT == kRows && !PIPE && !LA;
    constexpr int WSPAN = (CHW * D * XB + kWave * 16 - 1) / (kWave * 16) * (kWave * 16);
    const int img_off = IMG_EARLY ? max(tm ? 0 : CHW * SL * SB, WSPAN) : (tm ? 0 : CHW * SL * SB);
    const bool row_image = LAYOUT == kRows && p.cu != nullptr && T < p.T && copier;
    if constexpr (IMG_EARLY) {
        if (row_image) {
            const int LS = p.T + W1 - 1;
            block_to_lds(make_rsrc((char *)p.win + ((int64_t)slot * p.win_slot + (int64_t)cb * LS) * SB,
                                   (uint32_t)(nch * LS * SB)),
                         lds + img_off, nch * LS * SB / 16, lane);
        }
    }
    int par = -1;   // tree: lane t < T holds parent[row, t] (loaded with the rest)
    if constexpr (TREE) {
        if (lane < T) par = p.parent[(int64_t)row * p.T + lane];
    }
    if constexpr (!PIPE) {
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): every load above has landed
        if constexpr (!LA) {
            lds_read_run<VB * D>(lds + lane * VB * D, wr);   // (LDS accesses run in order)
#pragma unroll
            for (int w = 0; w < XW * D; ++w) wr[w] = on ? wr[w] : 0u;
        }
    }
#pragma unroll
    for (int j = 0; j < RJ; ++j) {
        const int q = j * kWave + lane;
        if (j * kWave < rchunks && q < rchunks)
            *(uint4 *)(rgn + q * 16) = make_uint4(sreg[j][0], sreg[j][1], sreg[j][2], sreg[j][3]);
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
                *(uint4 *)(rgn + q * 16) = make_uint4(sreg[j][0], sreg[j][1], sreg[j][2], sreg[j][3]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();

    // Channel-major state: each lane picks its window out of the staged region.
    auto window_from_lds = [&]() __attribute__((always_inline)) {
        if (contiguous_state) {
            uint32_t run[RUNW];   // the lane's [CPL][W1] run
            lds_read_run<RUNB>(rgn + lane * RUNB, run);
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
            const char *rec = rgn + (lane * CPL * SL + a) * SB;
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
    };
    if constexpr (!TM) window_from_lds();   // time-major: the window came in with the loads

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

    // ---- tree: the v tile and each token's ancestor columns ---------------------------------
    // Tile row k of LDS holds v[k] (k < W1: the starting window, else x_{k-W1}) for the
    // wavefront's channels, in the state type.  vidx[m] of lane t is the v index of
    // the value m steps back along token t's path: m = 0 is x_t itself; a step past the
    // root lands in the starting window.  Token t's taps are then v[vidx[W1]], ...,
    // v[vidx[1]], x_t and its window is v[vidx[W1-1]], ..., v[vidx[0]].
    constexpr int TILE = TREE ? (W1 + TB) * P : 0;   // LDS bytes of the tile
    int vidx[D];
    if constexpr (TREE) {
        if (__builtin_amdgcn_ballot_w64(lane < T && (par < -1 || par >= lane)))
            return;   // a malformed tree: nothing written for this row
        lds_barrier();   // every lane has read its window out of the state region
#pragma unroll
        for (int k = 0; k < W1 + TB; ++k) {
            if (k < W1 + T) {
                uint32_t col[SW];
                column(k, col);
                lds_write_run<SCB>(lds + k * P + lane * SCB, col);
            }
        }
        vidx[0] = W1 + lane;
#pragma unroll
        for (int m = 1; m <= W1; ++m) {
            const int up = __builtin_amdgcn_ds_bpermute((par < 0 ? lane : par) << 2, vidx[m - 1]);
            vidx[m] = par < 0 ? W1 - m : up;
        }
        lds_barrier();
    }
    // Token t's v index m steps back, uniform across the wavefront (t compile-time).
    auto tree_idx = [&](int t, int m) -> int {
        return __builtin_amdgcn_readfirstlane(__builtin_amdgcn_readlane(vidx[m], t));
    };
    // The lane's CPL channels of tile row k, in the state type.
    auto tile_col = [&](int k, uint32_t *col) { lds_read_run<SCB>(lds + k * P + lane * SCB, col); };

    // ---- conv + SiLU + per-head L2 -> out --------------------------------------------------
    // The arithmetic runs as soon as the inputs are in, before the copies below: while
    // the memory pipeline is still full of other wavefronts' traffic, a wavefront that
    // stores first would stall at its stores with its arithmetic still ahead of it.
    const bool wave_l2 = cb < p.qk;    // uniform: this wavefront holds q|k channels
    const bool lane_l2 = on && lane * CPL + cb < p.qk;
    const rsrc_t o_r = make_rsrc((char *)p.out + (orow + cb) * XB,
                                 (uint32_t)(((int64_t)(T - 1) * p.out_tok + nch) * XB));
    // Line-aligned build: N contiguous ranges of nb <= NW * kWave * U bytes each, range i
    // at byte soff0 + i * soff_step of the resource r (whose base address is base), staged
    // in LDS at src + i * src_step.  The workgroup's threads take consecutive U-byte units
    // starting at the 128-byte line that holds a range's first byte, so each store
    // instruction covers whole lines except at the range's two ends; the units of the
    // range's last, partial line beyond those (at most 120 bytes, so threads of wavefront
    // 0 only) go in a second store.  Units outside the range are dropped (kOffLane).  All
    // LDS reads go first, then the stores.
    // With a channel-major state the units of a range's two partial lines are stored with
    // the default policy (and the workgroups run in XCD order): the neighbouring workgroup,
    // on the same XCD, writes the rest of such a line, and the two halves merge in L2
    // instead of reaching HBM as two partial writes (stress d 10200: 159.9 -> 156.7 us).
    // With a time-major state both measured slower (106.5 -> 108.3 / 110.3 us).
    constexpr int PASS = NW * kWave;            // threads of the workgroup
    constexpr int PPOL = LACM ? kKeep : SPOL;   // the store policy of partial lines
    auto la_store = [&](auto n_ranges, const char *src, int src_step, rsrc_t r, uint64_t base,
                        uint32_t soff0, uint32_t soff_step, int nb) __attribute__((always_inline)) {
        constexpr int N = decltype(n_ranges)::value;
        constexpr int U = VB;
        uint32_t v[N][U / 4], v2[N][U / 4], off[N], offp[N], off2[N];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const uint32_t soff = soff0 + (uint32_t)i * soff_step;
            const int delta = (int)((base + soff) & 127u);
            const int o = tid * U - delta;
            const int o2 = o + PASS * U;
            const bool ok = o >= 0 && o < nb, ok2 = o2 < nb;
            // the unit lies in the range's first or last line, and that line is partial
            const bool part = (delta != 0 && o < 128 - delta) ||
                              (((delta + nb) & 127) != 0 && o >= ((delta + nb) & ~127) - delta);
            lds_read_run<U>(src + i * src_step + (ok ? o : 0), v[i]);
            lds_read_run<U>(src + i * src_step + (ok2 ? o2 : 0), v2[i]);
            off[i] = ok && (PPOL == SPOL || !part) ? (uint32_t)o : kOffLane;
            offp[i] = ok && part ? (uint32_t)o : kOffLane;
            off2[i] = ok2 ? (uint32_t)o2 : kOffLane;
        }
#pragma unroll
        for (int i = 0; i < N; ++i) gstore<U, SPOL>(r, off[i], soff0 + (uint32_t)i * soff_step, v[i]);
        if constexpr (PPOL != SPOL) {
#pragma unroll
            for (int i = 0; i < N; ++i) gstore<U, PPOL>(r, offp[i], soff0 + (uint32_t)i * soff_step, v[i]);
        }
        if (wave == 0) {   // (the last line: partial)
#pragma unroll
            for (int i = 0; i < N; ++i) gstore<U, PPOL>(r, off2[i], soff0 + (uint32_t)i * soff_step, v2[i]);
        }
    };
    // The same for an even number N of ranges in 16-byte units, two ranges per store
    // instruction: range 2i+j goes to the threads j * PASS/2 .. (j+1) * PASS/2 - 1, and its
    // last partial line (units past PASS/2) to the first lanes of wavefronts 0 and NW/2.
    // The halves of the workgroup store different ranges, so each lane's offset holds its
    // range's soff; the partial lines take PPOL as above.  (Out, time-major state: stress
    // d 10200 107.1 -> 105.5 us; channel-major: 154.9 -> 153.8 us; d 10240 unchanged
    // within the spread.)
    auto la_store16 = [&](auto n_ranges, const char *src, int src_step, rsrc_t r, uint64_t base,
                          uint32_t soff0, uint32_t soff_step, int nb) __attribute__((always_inline)) {
        constexpr int N = decltype(n_ranges)::value;
        constexpr int HP = PASS / 2;               // threads per range
        static_assert(N % 2 == 0 && NW % 2 == 0, "pairs of ranges over two halves");
        const int j = tid / HP, k = tid % HP;
        uint32_t v[N / 2][4], v2[N / 2][4], off[N / 2], offp[N / 2], off2[N / 2];
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const int rg = 2 * i + j;
            const uint32_t soff = soff0 + (uint32_t)rg * soff_step;
            const int delta = (int)((base + soff) & 127u);
            const int o = k * 16 - delta;
            const int o2 = o + HP * 16;
            const bool ok = o >= 0 && o < nb, ok2 = o2 < nb;
            const bool part = (delta != 0 && o < 128 - delta) ||
                              (((delta + nb) & 127) != 0 && o >= ((delta + nb) & ~127) - delta);
            lds_read_run<16>(src + rg * src_step + (ok ? o : 0), v[i]);
            lds_read_run<16>(src + rg * src_step + (ok2 ? o2 : 0), v2[i]);
            off[i] = ok && (PPOL == SPOL || !part) ? soff + (uint32_t)o : kOffLane;
            offp[i] = ok && part ? soff + (uint32_t)o : kOffLane;
            off2[i] = ok2 ? soff + (uint32_t)o2 : kOffLane;
        }
#pragma unroll
        for (int i = 0; i < N / 2; ++i) gstore<16, SPOL>(r, off[i], 0u, v[i]);
        if constexpr (PPOL != SPOL) {
#pragma unroll
            for (int i = 0; i < N / 2; ++i) gstore<16, PPOL>(r, offp[i], 0u, v[i]);
        }
        if (wave % (NW / 2) == 0) {
#pragma unroll
            for (int i = 0; i < N / 2; ++i) gstore<16, PPOL>(r, off2[i], 0u, v2[i]);
        }
    };
    // A contiguous range of nb bytes staged in LDS at src + delta (delta: the offset of the
    // range's first byte in its 128-byte line), stored in 16-byte units from that line on.
    auto la_store_block = [&](const char *src, rsrc_t r, int delta, int nb) __attribute__((always_inline)) {
        for (int k = tid * 16; k < delta + nb; k += PASS * 16) {
            const int o = k - delta;
            uint32_t w[4];
            lds_read_run<16>(src + (o >= 0 ? k : 0), w);
            const bool part = k < 128 || k >= ((delta + nb) & ~127);   // first or last line
            gstore<16, SPOL>(r, o >= 0 && (PPOL == SPOL || !part) ? (uint32_t)o : kOffLane, 0, w);
            if constexpr (PPOL != SPOL) gstore<16, PPOL>(r, o >= 0 && part ? (uint32_t)o : kOffLane, 0, w);
        }
    };
    constexpr int OUT_ROW = LA ? RANGE * XB : 0;   // LDS bytes of one token of out (workgroup)
    // where the exchange buffers start: after a channel-major state's staged region
    const int ob_base = LACM ? (128 + RANGE * SL * SB + 15) / 16 * 16 : 0;
    const rsrc_t og_r = make_rsrc((char *)p.out + (orow + cbg) * XB,
                                  (uint32_t)(((int64_t)(T - 1) * p.out_tok + nchg) * XB));
    // Tokens go in chunks of G with no branch inside a chunk: x past T reads as zeros
    // and those tokens are computed but never stored.  The chunk's exponentials,
    // reciprocals and cross-lane sums are then independent and overlap.
    // tree, split: this wavefront's chunk only (the chunks are the G-token chunks)
    auto mine = [&](int t) { return (!TREE && !SPLIT) || p.token_chunks == 1 || t / G == chunk; };
    // after_math runs between a chunk's arithmetic and its stores
    auto do_chunk = [&](int t0, auto after_math) __attribute__((always_inline)) {
        float y[G][CPL];
        uint32_t tv[TREE ? G : 1][W1][SW];   // tree: the taps before x_t, from the tile
        if constexpr (TREE) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int w = 0; w < W1; ++w)
                    if (t0 + g < T) tile_col(tree_idx(t0 + g, W1 - w), tv[g][w]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) {
                float acc = bv[ch];
#pragma unroll
                for (int w = 0; w < D; ++w) {
                    float v;
                    if constexpr (TREE)
                        v = w < W1 ? elem_val<SB>(tv[g][w < W1 ? w : 0], ch) : val(t0 + g + W1, ch);
                    else
                        v = val(t0 + g + w, ch);
                    acc = __builtin_fmaf(wv[ch][w], v, acc);
                }
                y[g][ch] = acc;
            }
        silu_rows_checked<G>(y);
        // (the line-aligned build runs with power-of-two heads only: it leaves the
        // segmented head sums out, which kept its time-major build at 3 waves per SIMD,
        // measured 1.2% faster at the stress shape than 4)
        if (wave_l2) head_l2<G, !LA>(y, lane_l2, p.head_lanes_log2, p.heads.head_lanes, p.eps);
        after_math();
        // line-aligned: the chunk's out goes through one of two LDS buffers (alternate
        // chunks), so one barrier per chunk orders both the hand-off and the reuse
        char *ob = lds + ob_base + ((t0 / G) & 1) * (G * OUT_ROW);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = t0 + g;
            if (LA || t < T) {
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
                if constexpr (LA)
                    lds_write_run<VB>(ob + g * OUT_ROW + tid * VB, o);
                else
                    gstore<VB, SPOL>(o_r, laneV, (uint32_t)(t * p.out_tok * XB), o);
            }
        }
        if constexpr (LA) {   // (full rows: every token of the chunk is below T)
            lds_barrier();
            // (16-byte units need 16-byte aligned ranges: x, out and their strides are)
            if constexpr (XB == 2)
                la_store16(std::integral_constant<int, G>(), ob, OUT_ROW, og_r,
                           (uint64_t)(uintptr_t)p.out + (uint64_t)(orow + cbg) * XB,
                           (uint32_t)(t0 * p.out_tok * XB), (uint32_t)(p.out_tok * XB), nchg * XB);
            else
                la_store(std::integral_constant<int, G>(), ob, OUT_ROW, og_r,
                         (uint64_t)(uintptr_t)p.out + (uint64_t)(orow + cbg) * XB,
                         (uint32_t)(t0 * p.out_tok * XB), (uint32_t)(p.out_tok * XB), nchg * XB);
        }
    };
    // Channel-major line-aligned build, copy phase: the committed window v[TB .. TB+W1-1]
    // (full rows) into the staged region, then the workgroup's region leaves whole.
    auto lacm_commit = [&]() __attribute__((always_inline)) {
        if (contiguous_state) {
            uint32_t run[RUNW];
            window_run(TB, run);
            lds_write_run<RUNB>(rgn + lane * RUNB, run);
        } else {
            char *rec = rgn + lane * CPL * SL * SB;
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
                for (int j = 0; j < W1; ++j) lds_put<SB>(rec + (ch * SL + j) * SB, sbits(TB + j, ch));
        }
        lds_barrier();
        la_store_block(lds, make_rsrc((char *)p.state + sreg_off, (uint32_t)(nchg * SL * SB)), s_delta,
                       nchg * SL * SB);
    };
    auto nothing = []() {};
    if constexpr (PIPE) {
        // The chunks from C0 on take no window column (their tokens are >= W1): they go
        // first, the chunks before C0 last.  The state's loads go out after chunk HC's
        // arithmetic: C0 where registers allow, the last chunk in the build for 5
        // wavefronts per SIMD, where holding the state columns any longer would spill
        // them (and the spill store would wait for every load).  A packed row may have
        // no token in chunk HC: the loads then go out there all the same.
        constexpr int NC = TB / G, C0 = (W1 + G - 1) / G, HC = WPE > 0 ? NC - 1 : C0;
        static_assert(C0 < NC, "a pipelined build has a chunk that takes no window column");
#pragma unroll
        for (int c = C0; c < HC; ++c)
            if (c * G < T) do_chunk(c * G, nothing);
        if (HC * G < T) do_chunk(HC * G, load_state_columns);
        else load_state_columns();
#pragma unroll
        for (int c = HC + 1; c < NC; ++c)
            if (c * G < T) do_chunk(c * G, nothing);
#pragma unroll
        for (int c = 0; c < C0; ++c)
            if (c == 0 || c * G < T) do_chunk(c * G, nothing);
    } else {
#pragma unroll
        for (int t0 = 0; t0 < TB; t0 += G)   // uniform guard; the loops are fully unrolled
            if (t0 < T && mine(t0)) do_chunk(t0, nothing);
    }
    if constexpr (SPLIT) {
        if (!copier) return;   // its chunk of out is stored; the copies are chunk 0's
    }
    if constexpr (LACM) lacm_commit();
    if constexpr (!TREE && !LACM) {
        // Channel-major state, the 16-token build for 5 wavefronts per SIMD: the window
        // is read out of LDS again here (the region is untouched until the commit below),
        // so that it is not held in registers through chunks 1 and later, which take no
        // window column; the memory clobber keeps the compiler from reusing the first
        // read.  Holding it there spilled it, and every reload waited for all stores
        // issued before it (bs128 T16: 28.7 -> 27.1 us).  Builds with registers to spare
        // keep it (the second read cost the T 8 shapes 2-5%).
        if constexpr (!TM && WPE > 0) {
            asm volatile("" ::: "memory");
            window_from_lds();
        }
        // ---- committed window -> conv_state -----------------------------------------------------
        // v[T .. T+W1-1] into columns 0..W1-1 of the staged rows (each lane rewrites only
        // its own channels' records, after having read them above), then the region leaves.
    #pragma unroll
        for (int t = 0; t < TB; ++t) {
            if (t == T - 1) {
                if constexpr (LA) {
                    // through the LDS buffer that the last chunk did not use (the chunk
                    // before it did, and every wavefront has passed the last chunk's
                    // barrier since reading it)
                    constexpr int NC = TB / G, C0 = (W1 + G - 1) / G;
                    constexpr int LASTC = C0 - 1, PREVC = C0 >= 2 ? C0 - 2 : NC - 1;
                    static_assert((LASTC & 1) != (PREVC & 1) && W1 * RANGE * SB <= G * OUT_ROW,
                                  "the commit's LDS buffer");
                    char *sbuf = lds + ((LASTC & 1) ^ 1) * (G * OUT_ROW);
    #pragma unroll
                    for (int j = 0; j < W1; ++j) {
                        uint32_t col[SW];
                        column(t + 1 + j, col);
                        lds_write_run<SCB>(sbuf + j * RANGE * SB + tid * SCB, col);
                    }
                    lds_barrier();
                    const rsrc_t sg_r = make_rsrc(
                        (char *)p.state + ((int64_t)slot * p.state_slot + cbg) * SB,
                        (uint32_t)(((int64_t)(SL - 1) * p.state_col + nchg) * SB));
                    la_store(std::integral_constant<int, W1>(), sbuf, RANGE * SB, sg_r,
                             (uint64_t)(uintptr_t)p.state +
                                 (uint64_t)((int64_t)slot * p.state_slot + cbg) * SB,
                             0u, (uint32_t)(p.state_col * SB), nchg * SB);
                } else if (tm) {
    #pragma unroll
                    for (int j = 0; j < W1; ++j) {
                        uint32_t col[SW];
                        column(t + 1 + j, col);
                        gstore<SCB, SPOL>(stm_r, laneS, (uint32_t)((int64_t)j * p.state_col * SB), col);
                    }
                } else if (contiguous_state) {
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
        if (!tm) {
            lds_barrier();
            lds_to_global<SPOL>(lds, rchunks, st_r, 0, lane);
            lds_barrier();   // the region's LDS is reused below
        }
    }

    // ---- rollback windows: pure copies of the inputs ---------------------------------------
    if constexpr (LAYOUT == kRows && LA) {
        // Line-aligned build (full rows: T == p.T == TB).  The workgroup's row block
        // [nchg][LC] is one contiguous range: each lane's rows [CPL][LC] go into LDS at
        // their offset in it, after the bytes of the range's first line that precede the
        // range, and the workgroup stores it in 16-byte units from that line on.
        constexpr int LC = TB + W1 - 1;
        constexpr int LANEB = CPL * LC * SB;   // bytes of a lane's rows
        constexpr int CW = LANEB / 4;
        constexpr int PIECE = (LANEB % 16 == 0) ? 16 : 8;
        const int64_t S = ((int64_t)slot * p.win_slot + (int64_t)cbg * LC) * SB;
        const int delta = (int)(((uint64_t)(uintptr_t)p.win + (uint64_t)S) & 127u);
        const int nb = nchg * LC * SB;
        lds_barrier();   // every wavefront has stored the commit out of LDS
        if (on) {
            char *mine = lds + delta + tid * LANEB;
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
        }
        lds_barrier();
        la_store_block(lds, make_rsrc((char *)p.win + S, (uint32_t)nb), delta, nb);
    } else if constexpr (LAYOUT == kRows) {
        const int L = T + W1 - 1;             // columns this row writes: v[1 .. T+W1-1]
        const int LS = p.T + W1 - 1;          // columns per channel in the buffer
        const rsrc_t row_r = make_rsrc(
            (char *)p.win + ((int64_t)slot * p.win_slot + (int64_t)cb * LS) * SB,
            (uint32_t)(nch * LS * SB));
        // Packed rows shorter than the buffer's: the slot's row block, as stored, is in LDS
        // (loaded with the other loads, or here in pipelined builds: there a global->LDS
        // load still outstanding at a later LDS access would make the compiler wait for
        // every store issued before it); each lane writes its channels' columns below L
        // into it, and the block leaves whole: the columns past L keep their bits, and
        // every store stays a coalesced 16-byte one.
        if (row_image) {
            constexpr int LC = TB + W1 - 1;   // >= LS
            char *img = lds + img_off;
            if constexpr (!IMG_EARLY) {
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): earlier LDS accesses are done
                block_to_lds(row_r, img, nch * LS * SB / 16, lane);
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the block has landed
            }
            if (on) {
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch)
#pragma unroll
                    for (int k = 0; k < LC; ++k)
                        if (k < L) lds_put<SB>(img + ((lane * CPL + ch) * LS + k) * SB, sbits(k + 1, ch));
            }
            lds_barrier();
            lds_to_global<SPOL>(img, nch * LS * SB / 16, row_r, 0, lane);
        } else if (T == TB && L == LS) {
            // Row length known at compile time: each lane assembles its channels' rows
            // ([CPL][LC], contiguous in the row layout) in registers into LDS at the
            // same offsets, and the wavefront streams the block out lane-contiguously.
            // A block over kRowsStageBytes goes in two halves of the lanes, so the
            // wavefront's LDS does not cap the number of resident wavefronts.
            constexpr int LC = TB + W1 - 1;
            constexpr int LANEB = CPL * LC * SB;   // bytes of a lane's rows
            constexpr int CW = LANEB / 4;
            constexpr int PIECE = (LANEB % 16 == 0) ? 16 : 8;
            constexpr int HALVES = kWave * LANEB > kRowsStageBytes ? 2 : 1;
            constexpr int HL = kWave / HALVES;     // lanes per half
#pragma unroll
            for (int h = 0; h < HALVES; ++h) {
                if (lane / HL == h) {
                    char *mine = lds + (lane % HL) * LANEB;
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
                }
                lds_barrier();
                const int c0 = h * HL * CPL;       // the half's first channel
                const int hch = min(HL * CPL, nch - c0);
                if (hch > 0) lds_to_global<SPOL>(lds, hch * LC * SB / 16, row_r, (uint32_t)(c0 * LC * SB), lane);
                if (h + 1 < HALVES) lds_barrier();
            }
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
            // Stream the tile out in the row layout [c][k], k < LS: chunk q of the
            // wavefront's contiguous row block holds elements e = q*EPC .. q*EPC+EPC-1,
            // element e = (channel e / LS, column e % LS) = tile row e % LS, channel e / LS.
            constexpr int EPC = 16 / SB;   // elements per 16-byte chunk
            const int nchunks = nch * LS / EPC;   // exact: nch * SB is a multiple of 16
            const int e0 = lane * EPC;
            int cc = e0 / LS;
            int kk = e0 - cc * LS;
            const int dq = (kWave * EPC) / LS;
            const int dr = kWave * EPC - dq * LS;
            if (L == LS && L >= EPC) {
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
                    gstore<16, SPOL>(row_r, (uint32_t)q * 16u, 0, w);
                    cc += dq;
                    kk += dr;
                    if (kk >= L) { kk -= L; ++cc; }
                }
            } else {
                // Short rows (L < EPC), or a packed row shorter than the buffer's rows:
                // columns >= L are not this call's to write, so chunks that reach
                // past L store only their columns below it.
                for (int q = lane; q < nchunks; q += kWave) {
                    uint32_t w[4] = {0u, 0u, 0u, 0u};
                    uint32_t valid = 0;
                    int c2 = cc, k2 = kk;
#pragma unroll
                    for (int m = 0; m < EPC; ++m) {
                        const bool ok = k2 < L;
                        const uint32_t b = ok ? lds_get<SB>(lds + k2 * P + c2 * SB) : 0u;
                        valid |= (ok ? 1u : 0u) << m;
                        if constexpr (SB == 4) {
                            w[m] = b;
                        } else {
                            if (m & 1) w[m >> 1] |= b << 16; else w[m >> 1] = b;
                        }
                        if (++k2 == LS) { k2 = 0; ++c2; }
                    }
                    if (valid == (1u << EPC) - 1u) {
                        gstore<16, SPOL>(row_r, (uint32_t)q * 16u, 0, w);
                    } else if (valid) {
#pragma unroll
                        for (int m = 0; m < EPC; ++m) {
                            if ((valid >> m) & 1u) {
                                const uint32_t bits = SB == 4 ? w[m] : (w[m >> 1] >> ((m & 1) * 16)) & 0xFFFFu;
                                gstore_elem<SB, SPOL>(row_r, (uint32_t)(q * 16 + m * SB), bits);
                            }
                        }
                    }
                    cc += dq;
                    kk += dr;
                    while (kk >= LS) { kk -= LS; ++cc; }
                }
            }
        }
    } else if constexpr (LAYOUT == kRowsT) {
        // Time-major rows: buffer column k (= v[k+1]) holds the d channels contiguously,
        // so each lane stores its CPL channels of every column straight from registers.
        const int L = T + W1 - 1;
        const int LS = p.T + W1 - 1;
        const uint32_t laneS = on ? (uint32_t)(lane * SCB) : kOffLane;
        const rsrc_t rt_r = make_rsrc(
            (char *)p.win + ((int64_t)slot * p.win_slot + cb) * SB,
            (uint32_t)(((int64_t)(LS - 1) * p.d_inner + nch) * SB));
#pragma unroll
        for (int k = 1; k < W1 + TB; ++k) {
            if (k - 1 < L) {
                uint32_t col[SW];
                column(k, col);
                gstore<SCB, SPOL>(rt_r, laneS, (uint32_t)((k - 1) * p.d_inner * SB), col);
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
            if (t < T && mine(t)) {
                char *slab = lds + TILE + (t & 1) * SLAB;
                uint32_t run[RUNW];
                if constexpr (TREE) {
                    uint32_t cols[W1][SW];   // the window's columns, oldest first
#pragma unroll
                    for (int j = 0; j < W1; ++j) tile_col(tree_idx(t, W1 - 1 - j), cols[j]);
#pragma unroll
                    for (int w = 0; w < RUNW; ++w) {   // [CPL][W1] run, channel-major
                        if constexpr (SB == 4) {
                            run[w] = cols[w % W1][w / W1];
                        } else {
                            const int e0 = 2 * w, e1 = 2 * w + 1;
                            const uint32_t lo = (cols[e0 % W1][(e0 / W1) >> 1] >> (((e0 / W1) & 1) * 16)) & 0xFFFFu;
                            const uint32_t hi = (cols[e1 % W1][(e1 / W1) >> 1] >> (((e1 / W1) & 1) * 16)) & 0xFFFFu;
                            run[w] = lo | (hi << 16);
                        }
                    }
                } else {
                    window_run(t + 1, run);
                }
                lds_write_run<RUNB>(slab + lane * RUNB, run);
                lds_barrier();
                lds_to_global<SPOL>(slab, slab_chunks, snap_r, (uint32_t)(t * p.d_inner * W1 * SB), lane);
            }
        }
    }

}

// The kernel: verify_body with the nt store policy, or - time-major builds where rows
// start off 128-byte lines (p.store_cached) - with the default one: neighbouring
// wavefronts then share the lines at their boundaries, and a line kept in L2 is merged
// there before it leaves instead of being streamed out in pieces (measured at d 10200:
// 119.2 -> 116.7 us, HBM traffic 1.039 -> 1.027x the algorithmic bytes).  Both bodies sit
// in one kernel behind a wavefront-uniform branch, so the launch and the register count
// are those of one body.
// The line-aligned build (NW 4) streams every store: its store ranges leave in whole lines.
template <int XB, int SB, int D, int TB, int LAYOUT, bool TREE, int WPE, bool SPLIT, bool TM, int NW = 1>
__global__ __launch_bounds__(kWave * NW) __attribute__((amdgpu_waves_per_eu(WPE > 0 ? WPE : 1)))
void cv_verify_kernel(KernelArgs p) {
    if constexpr (TM && NW == 1) {
        if (p.store_cached) {
            verify_body<XB, SB, D, TB, LAYOUT, TREE, WPE, SPLIT, TM, NW, 0>(p);
            return;
        }
    }
    verify_body<XB, SB, D, TB, LAYOUT, TREE, WPE, SPLIT, TM, NW, kNT>(p);
}

// ---- instantiation ----------------------------------------------------------------------
//
// This file is compiled once per (x bytes, state bytes, variant, state layout) with
// CV_XB, CV_SB, CV_VARIANT (0 dense, 1 rows, 2 time-major rows, 3 tree with dense
// windows) and CV_TM (1: time-major conv_state) defined, so the instantiations build
// in parallel; each object exports one picker over (d_conv, token bucket).
// build: 0 the regular build, 1 the 16-token build for 5 wavefronts per SIMD (lean),
// 2 the line-aligned build of 4-wavefront workgroups (16 tokens).
template <int XB, int SB, int D, int LAYOUT, bool TREE, bool TM>
const void *pick_bucket(int tb, int build, bool split) {
    const bool lean = build == 1;
    if constexpr (!TREE && LAYOUT != kDense) {
        if (split) {
            if (tb == 8) return (const void *)cv_verify_kernel<XB, SB, D, 8, LAYOUT, TREE, 0, true, TM>;
            if (tb == 16) return (const void *)cv_verify_kernel<XB, SB, D, 16, LAYOUT, TREE, 0, true, TM>;
            return nullptr;
        }
    }
    switch (tb) {
        case 1: return (const void *)cv_verify_kernel<XB, SB, D, 1, LAYOUT, TREE, 0, false, TM>;
        case 2: return (const void *)cv_verify_kernel<XB, SB, D, 2, LAYOUT, TREE, 0, false, TM>;
        case 4: return (const void *)cv_verify_kernel<XB, SB, D, 4, LAYOUT, TREE, 0, false, TM>;
        case 8: return (const void *)cv_verify_kernel<XB, SB, D, 8, LAYOUT, TREE, 0, false, TM>;
        case 16:
            if constexpr (XB == 2 && SB == 2 && LAYOUT == kRows && !TREE) {
                if (build == 2) return (const void *)cv_verify_kernel<XB, SB, D, 16, LAYOUT, TREE, 0, false, TM, 4>;
            }
            // the 5-wavefront build exists for bf16 x and state with a channel-major
            // conv_state only: elsewhere it spills heavily, or (time-major) the regular
            // build's pipelined loads measured faster
            if constexpr (XB == 2 && SB == 2 && !TM) {
                if (lean) return (const void *)cv_verify_kernel<XB, SB, D, 16, LAYOUT, TREE, 5, false, TM>;
            }
            return (const void *)cv_verify_kernel<XB, SB, D, 16, LAYOUT, TREE, 0, false, TM>;
        case 24: return (const void *)cv_verify_kernel<XB, SB, D, 24, LAYOUT, TREE, 0, false, TM>;
        case 32: return (const void *)cv_verify_kernel<XB, SB, D, 32, LAYOUT, TREE, 0, false, TM>;
        default: return nullptr;
    }
}

}  // namespace

#if !defined(CV_XB) || !defined(CV_SB) || !defined(CV_VARIANT) || !defined(CV_TM)
#error "compile with -DCV_XB=<2|4> -DCV_SB=<2|4> -DCV_VARIANT=<0..3> -DCV_TM=<0|1>"
#endif

#define CV_PICK_NAME(xb, sb, v, tm) pick_kernel_##xb##_##sb##_##v##_##tm
#define CV_PICK(xb, sb, v, tm) CV_PICK_NAME(xb, sb, v, tm)

#ifdef CV_WRITE_COUNT
#define CV_COUNT_SET_NAME(xb, sb, v, tm) count_ranges_set_##xb##_##sb##_##v##_##tm
#define CV_COUNT_SET(xb, sb, v, tm) CV_COUNT_SET_NAME(xb, sb, v, tm)
int CV_COUNT_SET(CV_XB, CV_SB, CV_VARIANT, CV_TM)(const CountRanges &c) {
    void *dst = nullptr;
    const hipError_t e = hipGetSymbolAddress(&dst, HIP_SYMBOL(CV_COUNT_RANGES));
    if (e != hipSuccess) return (int)e;
    return (int)hipMemcpy(dst, &c, sizeof c, hipMemcpyHostToDevice);
}
#endif

const void *CV_PICK(CV_XB, CV_SB, CV_VARIANT, CV_TM)(int d_conv, int token_bucket, int build, int split) {
    constexpr int layout = CV_VARIANT == 3 ? kDense : CV_VARIANT;
    constexpr bool tree = CV_VARIANT == 3;
    constexpr bool tm = CV_TM != 0;
    switch (d_conv) {
        case 2: return pick_bucket<CV_XB, CV_SB, 2, layout, tree, tm>(token_bucket, build, split != 0);
        case 3: return pick_bucket<CV_XB, CV_SB, 3, layout, tree, tm>(token_bucket, build, split != 0);
        case 4: return pick_bucket<CV_XB, CV_SB, 4, layout, tree, tm>(token_bucket, build, split != 0);
        default: return nullptr;
    }
}

}  // namespace cvimpl
