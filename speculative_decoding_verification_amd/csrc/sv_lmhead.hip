// gfx950 kernels of LM-head-fused verification.
//
// What is computed: the acceptance rule of speculative sampling (NgramRL
// essay "AI 开始抄自己的作业——而且抄得理直气壮", section "投机解码：让草稿先跑，
// 考官殿后") with the target's and the draft's logits formed from their hidden
// states and output-layer weights inside the call, l_i(y) = h_i . w_y.
// Greedy (T == 0) never stores the [B][k+1][V] logits: the target's
// choice is its lowest-index argmax, a draft token is kept iff it equals it.
// Sampling (T > 0): p = softmax(l_t / T), q = softmax(l_d / T); x_i is kept iff
// u_i q_i(x_i) < p_i(x_i); at the first rejection r a token is drawn from
// max(0, p_r - q_r), after full acceptance from p_k.
//
// Kernels:
//  k_lmhead_gemm<MODE>  a bf16 GEMM H . W^T on the matrix cores
//                    (v_mfma_f32_32x32x16_bf16, fp32 accumulation) whose
//                    epilogue reduces each 256 x 256 tile: per row (max,
//                    lowest index) for greedy; for sampling per row the
//                    softmax statistics (m, s) and the logit of the row's
//                    draft token, with the fp32 logits stored for the draws
//                    (writes that fit in the memory bandwidth the
//                    matrix-bound GEMM leaves idle).
//                    One launch can hold two GEMMs (target rows against the
//                    target's output layer, draft rows against the draft's).
//                    Each of the 8 wavefronts computes a 128 x 64 block.  K
//                    is staged 64 at a time through two LDS buffers, filled by
//                    direct-to-LDS loads (global_load_lds_dwordx4: no staging
//                    registers, no LDS-write instructions) into unpadded
//                    128-byte rows whose 16-byte pieces are XOR-swizzled by
//                    row, so fragment reads hit distinct banks.  A slice is
//                    four 16-deep MFMA groups; between the MFMAs of one group
//                    the wavefront reads the next group's fragments, or issues
//                    the loads of the slice after next, in a fixed interleave,
//                    so that the matrix pipe is not left waiting behind a
//                    burst of memory instructions; one wait and one barrier
//                    per slice, before the last group, whose MFMAs overlap the
//                    reads of the next slice's first fragments.  The grid is
//                    persistent, one workgroup per compute unit, each taking
//                    every G-th item: all workgroups advance through the items
//                    in step, and the items a die (XCD) takes in one step are
//                    consecutive, so the row tiles of one vocabulary tile run
//                    side by side on one die and share its weight rows in that
//                    die's L2.
//  k_lmhead_finish   greedy, per sequence: the rows' argmaxes from the
//                    partials, the decisions on one lane per position.
//  k_lmhead_decide   sampling, per sequence: (m, Z) of every row from the
//                    partials, p(x_i), q(x_i), the tests and the first
//                    rejection; which rows the draw needs.
//  k_lmhead_draw     sampling, per sequence: the draw from the residual (or
//                    from p_k) over the stored logits of target row r (or k)
//                    and draft row r, by inverting the cumulative weight in
//                    ascending token order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "specverify.h"
#include "sv_lmhead.h"

namespace sv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kLmMaxRows = SV_MAX_DRAFT + 1;  // positions of one sequence


__device__ __forceinline__ float neg_inf_f() { return -__builtin_inff(); }

// Larger value wins; equal values: lower index wins.
__device__ __forceinline__ void better(float& v, int& i, float ov, int oi) {
    if (ov > v || (ov == v && oi < i)) {
        v = ov;
        i = oi;
    }
}

template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, true));
}

template <int CTRL>
__device__ __forceinline__ int dppi(int x) {
    return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xf, 0xf, true);
}

// (max, lowest index) over the 32 lanes of each half-wave (lanes 0-31 and
// 32-63 reduce separately); the result on every lane of the half.
__device__ __forceinline__ void half_wave_argmax(float& v, int& i) {
    better(v, i, dppf<0xb1>(v), dppi<0xb1>(i));    // quad_perm [1,0,3,2]
    better(v, i, dppf<0x4e>(v), dppi<0x4e>(i));    // quad_perm [2,3,0,1]
    better(v, i, dppf<0x124>(v), dppi<0x124>(i));  // row_ror 4
    better(v, i, dppf<0x128>(v), dppi<0x128>(i));  // row_ror 8
    better(v, i, __shfl_xor(v, 16), __shfl_xor(i, 16));
}

// Maximum and sum over the 32 lanes of each half-wave, fixed order.
__device__ __forceinline__ float half_wave_max(float v) {
    v = fmaxf(v, dppf<0xb1>(v));
    v = fmaxf(v, dppf<0x4e>(v));
    v = fmaxf(v, dppf<0x124>(v));
    v = fmaxf(v, dppf<0x128>(v));
    return fmaxf(v, __shfl_xor(v, 16));
}

__device__ __forceinline__ float half_wave_sum(float v) {
    v += dppf<0xb1>(v);
    v += dppf<0x4e>(v);
    v += dppf<0x124>(v);
    v += dppf<0x128>(v);
    return v + __shfl_xor(v, 16);
}


// The token whose logit statistics row m captures (-1: none).
__device__ __forceinline__ int row_token(const LmPlan& pl, int tokens, int m) {
    int x = -1;
    if (tokens == kLmTargetTokens) {
        const int i = m % (pl.k + 1);
        if (i < pl.k) x = pl.tokens[static_cast<int64_t>(m / (pl.k + 1)) * pl.k + i];
    } else if (tokens == kLmDraftTokens) {
        x = pl.tokens[m];
    }
    return (x >= 0 && x < pl.vocab) ? x : -1;
}

template <int MODE>
__global__ __launch_bounds__(kLmThreads, kLmBlocksPerCu) void k_lmhead_gemm(LmPlan pl) {
    constexpr int FM = kLmWaveM / 32;  // 32 x 32 fragments per wavefront block
    constexpr int FN = kLmWaveN / 32;
    constexpr int WAVES_M = kLmBM / kLmWaveM;
    constexpr int WAVES_N = kLmBN / kLmWaveN;
    static_assert(WAVES_M * WAVES_N * 64 == kLmThreads, "one wavefront per block of the tile");
    constexpr int ROWS_PER_PASS = kLmThreads / (kLmBK / 8);  // tile rows one pass of 16-byte pieces covers
    constexpr int PA = kLmBM / ROWS_PER_PASS;                 // direct-to-LDS loads per wavefront and slice: A
    constexpr int PB = kLmBN / ROWS_PER_PASS;                 // and B
    static_assert(PA * ROWS_PER_PASS == kLmBM && PB * ROWS_PER_PASS == kLmBN, "whole passes");
    static_assert(kLmBK == 64 && kLmThreads == 512, "a load of 64 lanes fills 8 rows of 8 pieces; 8 wavefronts");
    static_assert(kLmHiddenMultiple % kLmBK == 0, "whole K slices");
    // two stages, each buffer its own array (so the compiler can tell a
    // direct-to-LDS load into one from reads of the other); rows of 64 bf16
    // (128 B) unpadded, 16-byte pieces XOR-swizzled by row: piece s of row r
    // sits at slot s ^ (r & 7)
    __shared__ __attribute__((aligned(16))) uint16_t sa0[kLmBM * kLmBK];
    __shared__ __attribute__((aligned(16))) uint16_t sa1[kLmBM * kLmBK];
    __shared__ __attribute__((aligned(16))) uint16_t sb0[kLmBN * kLmBK];
    __shared__ __attribute__((aligned(16))) uint16_t sb1[kLmBN * kLmBK];
    __shared__ float cand_v[WAVES_N][kLmBM];  // argmax max, statistics m
    __shared__ int cand_i[WAVES_N][kLmBM];    // argmax index
    __shared__ float cand_s[WAVES_N][kLmBM];  // statistics s
    __shared__ int stok[kLmBM];               // statistics: each row's token

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WAVES_M;  // row block of the tile
    const int wn = wave / WAVES_M;  // column block of the tile
    const int D = pl.hidden;
    const int kblocks = D / kLmBK;
    const int64_t items = pl.items;
    const int G = gridDim.x;  // a multiple of kXcds
    // Blocks are dealt to the XCDs by index mod 8: give each die a run of
    // consecutive items per step.
    const int slot = (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;

    // Rows past the end of H or W are read as the last row (their results
    // are never written or are masked out), so no load is guarded.
    //
    // Direct-to-LDS piece q of a wavefront: 64 lanes write 1 KiB contiguous,
    // tile rows (8q + wave) * 8 + lane / 8, slot lane % 8, which holds the
    // row's K piece (lane % 8) ^ (lane / 8).
    const int drow = (lane >> 3);
    const int dseg = (lane & 7) ^ (lane >> 3);

    for (int64_t item = slot; item < items; item += G) {
        // The GEMM this item belongs to (fields picked one by one: indexing
        // the argument's array with a varying index would copy it to scratch).
        const bool g1 = pl.n_gemms > 1 && item >= pl.g[1].item0;
        const uint16_t* const ga = g1 ? pl.g[1].a : pl.g[0].a;
        const uint16_t* const gw = g1 ? pl.g[1].w : pl.g[0].w;
        const int g_rows = g1 ? pl.g[1].rows : pl.g[0].rows;
        const int g_mt = g1 ? pl.g[1].m_tiles : pl.g[0].m_tiles;
        const int g_out0 = g1 ? pl.g[1].out_row0 : pl.g[0].out_row0;
        const int64_t li = item - (g1 ? pl.g[1].item0 : pl.g[0].item0);
        const int mt = static_cast<int>(li % g_mt);
        const int nt = static_cast<int>(li / g_mt);
        const int m0 = mt * kLmBM;
        const int n0 = nt * kLmBN;
        const uint16_t* const a_base = ga;
        const uint16_t* const b_base = gw + static_cast<int64_t>(n0) * D;
        const int b_last = pl.vocab - 1 - n0;
        // A offsets are absolute (rows x hidden < 2^31 is checked on the
        // host), W offsets are from the tile's first row.
        uint32_t a_off[PA], b_off[PB];
#pragma unroll
        for (int q = 0; q < PA; ++q) {
            const int m = min(m0 + (q * 8 + wave) * 8 + drow, g_rows - 1);
            a_off[q] = static_cast<uint32_t>(m * D + dseg * 8);
        }
#pragma unroll
        for (int q = 0; q < PB; ++q)
            b_off[q] = static_cast<uint32_t>(min((q * 8 + wave) * 8 + drow, b_last) * D + dseg * 8);
        floatx16_t acc[FM][FN];
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

        static_assert(kLmBK == 64, "four 16-deep MFMA groups per slice");
        constexpr int NMF = FM * FN;     // MFMAs per group
        constexpr int NRD = FM + FN;     // fragment reads per group
        constexpr int NGL = PA + PB;     // global loads (and LDS writes) per slice
        static_assert(2 * NMF >= NRD && NMF >= NGL, "interleave slots");
        bf16x8_t f0a[FM], f0b[FN], f1a[FM], f1b[FN];
#define LM_FRAGS(FA, FB, SA, SB, KS)                                                        \
    {                                                                                       \
        const int kp_ = (KS) * 2 + (lane >> 5);                                             \
        _Pragma("unroll") for (int mi = 0; mi < FM; ++mi) {                                 \
            const int r_ = wm * kLmWaveM + mi * 32 + (lane & 31);                           \
            FA[mi] = *reinterpret_cast<const bf16x8_t*>(&SA[r_ * kLmBK + ((kp_ ^ (r_ & 7)) << 3)]); \
        }                                                                                   \
        _Pragma("unroll") for (int ni = 0; ni < FN; ++ni) {                                 \
            const int r_ = wn * kLmWaveN + ni * 32 + (lane & 31);                           \
            FB[ni] = *reinterpret_cast<const bf16x8_t*>(&SB[r_ * kLmBK + ((kp_ ^ (r_ & 7)) << 3)]); \
        }                                                                                   \
    }
#define LM_DMA(SA, SB, K0)                                                                  \
    {                                                                                       \
        _Pragma("unroll") for (int q = 0; q < PA; ++q)                                      \
            __builtin_amdgcn_global_load_lds((const void*)(a_base + (K0) + a_off[q]),       \
                (__attribute__((address_space(3))) void*)(SA + (q * 8 + wave) * 512), 16, 0, 0); \
        _Pragma("unroll") for (int q = 0; q < PB; ++q)                                      \
            __builtin_amdgcn_global_load_lds((const void*)(b_base + (K0) + b_off[q]),       \
                (__attribute__((address_space(3))) void*)(SB + (q * 8 + wave) * 512), 16, 0, 0); \
    }
#define LM_MFMA(FA, FB)                                                                     \
    {                                                                                       \
        _Pragma("unroll") for (int mi = 0; mi < FM; ++mi)                                   \
            _Pragma("unroll") for (int ni = 0; ni < FN; ++ni)                               \
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[mi], FB[ni], acc[mi][ni], 0, 0, 0); \
    }
// After each MFMA of a group: up to two fragment reads (READS), one direct-to-LDS load (LOADS), one LDS write (WRITES).
#define LM_INTERLEAVE(READS, LOADS, WRITES)                                                 \
    {                                                                                       \
        _Pragma("unroll") for (int t = 0; t < NMF; ++t) {                                   \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                              \
            if ((READS) && 2 * t < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  \
            if ((READS) && 2 * t + 1 < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); \
            if ((LOADS) && t < NGL) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      \
            if ((WRITES) && t < NGL) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);     \
        }                                                                                   \
    }

        // Two stages: the direct-to-LDS loads of slice kb+2 go out in group 3
        // of slice kb, into the buffer slice kb has just finished with; one
        // wait for this wavefront's loads and one barrier per slice.
        __syncthreads();  // the previous item's readers of the buffers and of cand are done
        if (MODE == kLmStats) {
            const int g_tok = g1 ? pl.g[1].tokens : pl.g[0].tokens;
            for (int r = tid; r < kLmBM; r += kLmThreads)
                stok[r] = m0 + r < g_rows ? row_token(pl, g_tok, m0 + r) : -1;
        }
        LM_DMA(sa0, sb0, 0);
        LM_DMA(sa1, sb1, min(1, kblocks - 1) * kLmBK);
        __builtin_amdgcn_s_waitcnt(0x0F70 | NGL);  // vmcnt(NGL): slice 0 has landed
        __syncthreads();
        LM_FRAGS(f0a, f0b, sa0, sb0, 0);
#define LM_SLICE(CA, CB, NA, NB, KB)                                                        \
    {                                                                                       \
        const int kload_ = min((KB) + 2, kblocks - 1) * kLmBK;                              \
        __builtin_amdgcn_sched_barrier(0);                                                  \
        LM_FRAGS(f1a, f1b, CA, CB, 1);                                                      \
        LM_MFMA(f0a, f0b);                                                                  \
        LM_INTERLEAVE(true, false, false);                                                  \
        __builtin_amdgcn_sched_barrier(0);                                                  \
        LM_FRAGS(f0a, f0b, CA, CB, 2);                                                      \
        LM_MFMA(f1a, f1b);                                                                  \
        LM_INTERLEAVE(true, false, false);                                                  \
        __builtin_amdgcn_sched_barrier(0);                                                  \
        LM_FRAGS(f1a, f1b, CA, CB, 3);                                                      \
        LM_MFMA(f0a, f0b);                                                                  \
        LM_INTERLEAVE(true, false, false);                                                  \
        __builtin_amdgcn_sched_barrier(0);                                                  \
        __builtin_amdgcn_s_waitcnt(0x0F70);  /* vmcnt(0): slice KB+1 has landed */          \
        __syncthreads();                                                                    \
        LM_FRAGS(f0a, f0b, NA, NB, 0);                                                      \
        LM_DMA(CA, CB, kload_);                                                             \
        LM_MFMA(f1a, f1b);                                                                  \
        LM_INTERLEAVE(true, true, false);                                                   \
    }
        for (int kb = 0; kb < kblocks; kb += 2) {
            LM_SLICE(sa0, sb0, sa1, sb1, kb);
            if (kb + 1 < kblocks) LM_SLICE(sa1, sb1, sa0, sb0, kb + 1);
        }
#undef LM_SLICE
        __builtin_amdgcn_sched_barrier(0);
#undef LM_INTERLEAVE
#undef LM_MFMA
#undef LM_FRAGS
#undef LM_DMA

        // Epilogue: accumulator j of lane l holds row 8(j/4) + 4(l/32) + j%4
        // of a 32 x 32 block, column l % 32.  Statistics mode first stores
        // the logits (each half-wave writes 128 contiguous bytes of a row,
        // non-temporal: they are read once, by the draws, after the GEMM).
        // The writes add about 8% to the GEMM (all workgroups write at the
        // same time and the next tile's loads queue behind them); forming
        // the draw rows again took a second GEMM of one row tile per
        // vocabulary tile, which cost more.
        if (MODE == kLmStats) {
#pragma unroll
            for (int mi = 0; mi < FM; ++mi)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int m = m0 + wm * kLmWaveM + mi * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
                    float* const out = pl.logits + static_cast<int64_t>(g_out0 + m) * pl.vocab;
#pragma unroll
                    for (int ni = 0; ni < FN; ++ni) {
                        const int col = n0 + wn * kLmWaveN + ni * 32 + (lane & 31);
                        if (m < g_rows && col < pl.vocab) __builtin_nontemporal_store(acc[mi][ni][j], out + col);
                    }
                }
        }
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int row = wm * kLmWaveM + mi * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
                if (MODE == kLmArgmax) {
                    float v = neg_inf_f();
                    int idx = INT_MAX;
#pragma unroll
                    for (int ni = 0; ni < FN; ++ni) {
                        const int col = n0 + wn * kLmWaveN + ni * 32 + (lane & 31);
                        if (col < pl.vocab) better(v, idx, acc[mi][ni][j], col);
                    }
                    half_wave_argmax(v, idx);
                    if ((lane & 31) == 0) {
                        cand_v[wn][row] = v;
                        cand_i[wn][row] = idx;
                    }
                } else {
                    const int tok = stok[row];
                    float v[FN];
                    float mx = neg_inf_f();
#pragma unroll
                    for (int ni = 0; ni < FN; ++ni) {
                        const int col = n0 + wn * kLmWaveN + ni * 32 + (lane & 31);
                        v[ni] = col < pl.vocab ? acc[mi][ni][j] * pl.c2 : neg_inf_f();
                        mx = fmaxf(mx, v[ni]);
                        if (col == tok && m0 + row < g_rows) pl.lx[g_out0 + m0 + row] = acc[mi][ni][j];
                    }
                    mx = half_wave_max(mx);
                    float sum = 0.f;
#pragma unroll
                    for (int ni = 0; ni < FN; ++ni) sum += v[ni] == neg_inf_f() ? 0.f : exp2f(v[ni] - mx);
                    sum = half_wave_sum(sum);
                    if ((lane & 31) == 0) {
                        cand_v[wn][row] = mx;
                        cand_s[wn][row] = sum;
                    }
                }
            }
        }
        __syncthreads();
        for (int r = tid; r < kLmBM; r += kLmThreads) {
            const int m = m0 + r;
            if (m >= g_rows) continue;
            const int64_t at = static_cast<int64_t>(g_out0 + m) * pl.n_parts + nt;
            if (MODE == kLmArgmax) {
                float v = cand_v[0][r];
                int idx = cand_i[0][r];
#pragma unroll
                for (int c = 1; c < WAVES_N; ++c) better(v, idx, cand_v[c][r], cand_i[c][r]);
                pl.part_v[at] = v;
                pl.part_i[at] = idx;
            } else {
                float mx = cand_v[0][r];
#pragma unroll
                for (int c = 1; c < WAVES_N; ++c) mx = fmaxf(mx, cand_v[c][r]);
                float sum = 0.f;
#pragma unroll
                for (int c = 0; c < WAVES_N; ++c) sum += cand_s[c][r] * exp2f(cand_v[c][r] - mx);
                pl.part_v[at] = mx;
                pl.part_s[at] = sum;
            }
        }
    }
}

// One workgroup per sequence: each wavefront reduces the partials of every
// fourth row (four independent loads per lane in flight), then wavefront 0
// decides every position on one lane.
constexpr int kFinishThreads = 256;

__global__ __launch_bounds__(kFinishThreads) void k_lmhead_finish(LmPlan pl) {
    __shared__ int g_row[kLmMaxRows];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int k = pl.k;
    const int n = pl.n_parts;
    for (int i = wave; i <= k; i += kFinishThreads / 64) {
        const int64_t row = static_cast<int64_t>(b) * (k + 1) + i;
        const float* pv = pl.part_v + row * n;
        const int32_t* pi = pl.part_i + row * n;
        float v = neg_inf_f();
        int idx = INT_MAX;
        for (int c0 = 0; c0 < n; c0 += 256) {
            float tv[4];
            int ti[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * 64 + lane;
                tv[u] = c < n ? pv[c] : neg_inf_f();
                ti[u] = c < n ? pi[c] : INT_MAX;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) better(v, idx, tv[u], ti[u]);
        }
        half_wave_argmax(v, idx);
        better(v, idx, __shfl_xor(v, 32), __shfl_xor(idx, 32));
        if (lane == 0) {
            g_row[i] = idx;
            if (pl.argmax_out) pl.argmax_out[row] = idx;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    const bool active = lane < k;
    int x = 0;
    if (active) x = pl.tokens[static_cast<int64_t>(b) * k + lane];
    const int my_g = active ? g_row[lane] : -1;
    const bool bad = active && (x < 0 || x >= pl.vocab);
    const bool invalid = __ballot(bad) != 0ull;
    const uint64_t mismatch = __ballot(active && x != my_g);
    const int r = invalid ? -1 : (mismatch ? __builtin_ctzll(mismatch) : k);
    const int g_r = r < 0 ? -1 : g_row[r];
    int32_t* out = pl.out_tokens + static_cast<int64_t>(b) * (k + 1);
    for (int j = lane; j <= k; j += 64) {
        if (invalid) out[j] = -1;
        else if (j < r) out[j] = x;
        else if (j == r) out[j] = g_r;
        else out[j] = -1;
    }
    if (lane == 0) pl.accepted_len[b] = r;
}

// Sampling, per sequence: (m, Z) of target rows 0..k and draft rows
// 0..k-1 from their partials (one wavefront per row, rows round-robin), then
// on one lane per position p(x_i), q(x_i) and the test u_i q < p.
__global__ __launch_bounds__(kFinishThreads) void k_lmhead_decide(LmPlan pl) {
    __shared__ float row_m[2 * kLmMaxRows], row_z[2 * kLmMaxRows];  // target rows 0..k, then draft rows
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int k = pl.k;
    const int n = pl.n_parts;
    for (int t = wave; t < 2 * k + 1; t += kFinishThreads / 64) {
        const int64_t row = t <= k ? static_cast<int64_t>(b) * (k + 1) + t
                                   : pl.rows_t + static_cast<int64_t>(b) * k + (t - k - 1);
        const float* pm = pl.part_v + row * n;
        const float* ps = pl.part_s + row * n;
        float mx = neg_inf_f();
        for (int c0 = 0; c0 < n; c0 += 256) {
            float tv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * 64 + lane;
                tv[u] = c < n ? pm[c] : neg_inf_f();
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) mx = fmaxf(mx, tv[u]);
        }
        mx = half_wave_max(mx);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        float z = 0.f;
        for (int c0 = 0; c0 < n; c0 += 256) {
            float tm[4], tz[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = c0 + u * 64 + lane;
                tm[u] = c < n ? pm[c] : mx;
                tz[u] = c < n ? ps[c] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) z += tz[u] * exp2f(tm[u] - mx);
        }
        z = half_wave_sum(z);
        z += __shfl_xor(z, 32);
        if (lane == 0) {
            row_m[t] = mx;
            row_z[t] = z;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const bool active = lane < k;
        int x = 0;
        float p = 0.f, q = 0.f;
        bool keep = false;
        if (active) {
            x = pl.tokens[static_cast<int64_t>(b) * k + lane];
            const float lt = pl.lx[static_cast<int64_t>(b) * (k + 1) + lane];
            const float ld = pl.lx[pl.rows_t + static_cast<int64_t>(b) * k + lane];
            // log2 p(x) and log2 q(x): the test u q < p is taken in the log
            // domain, where p and q far below the smallest float still compare.
            const float lp = lt * pl.c2 - row_m[lane] - log2f(row_z[lane]);
            const float lq = ld * pl.c2 - row_m[k + 1 + lane] - log2f(row_z[k + 1 + lane]);
            p = exp2f(lp);
            q = exp2f(lq);
            const float u = pl.uniforms[static_cast<int64_t>(b) * (k + 1) + lane];
            keep = (u > 0.f ? log2f(u) : neg_inf_f()) + lq < lp;
        }
        const bool bad = active && (x < 0 || x >= pl.vocab);
        const bool invalid = __ballot(bad) != 0ull;
        const uint64_t rejected = __ballot(active && !keep);
        const int r = invalid ? -1 : (rejected ? __builtin_ctzll(rejected) : k);
        if (pl.probs_out && active) {
            pl.probs_out[(static_cast<int64_t>(b) * k + lane) * 2] = invalid ? __builtin_nanf("") : p;
            pl.probs_out[(static_cast<int64_t>(b) * k + lane) * 2 + 1] = invalid ? __builtin_nanf("") : q;
        }
        int32_t* out = pl.out_tokens + static_cast<int64_t>(b) * (k + 1);
        for (int j = lane; j <= k; j += 64) {
            if (invalid || j > r) out[j] = -1;
            else if (j < r) out[j] = x;  // j < r <= k: lane j holds x_j
            // j == r: the draw writes it
        }
        if (lane == 0) {
            pl.accepted_len[b] = r;
            LmSeqDraw d;
            d.r = r;
            const int rt = max(r, 0);
            const int rd = min(max(r, 0), k - 1);
            d.mt = row_m[rt];
            d.zt = row_z[rt];
            d.md = row_m[k + 1 + rd];
            d.zd = row_z[k + 1 + rd];
            d.pad[0] = d.pad[1] = d.pad[2] = 0;
            pl.seq[b] = d;
        }
    }
}

// Sampling, per sequence: the draw at the first rejection r from
// max(0, p_r - q_r), or after full acceptance from p_k, over the draw rows'
// logits, inverting the cumulative weight in ascending token order.  The
// row is cut into segments of 1024 consecutive tokens (lane l of a
// wavefront takes tokens l, l+64, ..., so every load is coalesced); a
// segment's weight is a wavefront sum; the segments' running sum finds the
// segment holding u * total, and one wavefront scans that segment in order.
constexpr int kDrawThreads = 1024;
constexpr int kDrawWaves = kDrawThreads / 64;
constexpr int kDrawSeg = 1024;                                    // tokens per segment
constexpr int kDrawMaxSegs = ((1 << 24) + kDrawSeg - 1) / kDrawSeg;  // V <= 2^24

__device__ __forceinline__ float wave_sum(float v) {
    v = half_wave_sum(v);
    return v + __shfl_xor(v, 32);
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_prefix(float v) {
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
        const float o = __shfl_up(v, sh);
        if ((threadIdx.x & 63) >= sh) v += o;
    }
    return v;
}

__global__ __launch_bounds__(kDrawThreads) void k_lmhead_draw(LmPlan pl) {
    __shared__ float seg_sum[kDrawMaxSegs];
    __shared__ float s_total;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const LmSeqDraw d = pl.seq[b];
    const int k = pl.k;
    const int r = d.r;
    if (r < 0) return;  // invalid token: the decision step wrote -1 everywhere
    const int V = pl.vocab;
    // target row r (k after full acceptance) and draft row r of the stored logits
    const float* lt = pl.logits + (static_cast<int64_t>(b) * (k + 1) + r) * V;
    const float* ld = pl.logits + (pl.rows_t + static_cast<int64_t>(b) * k + min(r, k - 1)) * V;
    const float c2 = pl.c2;
    const float inv_zt = 1.f / d.zt, inv_zd = 1.f / d.zd;
    const int nseg = (V + kDrawSeg - 1) / kDrawSeg;
    bool residual = r < k;
    constexpr int PER_LANE = kDrawSeg / 64;
    // A segment's weights, lane l holding tokens l + 64 i (i < PER_LANE);
    // every load of the segment is issued before any is used.
    auto seg_weights = [&](int sg, float* w) {
        float a[PER_LANE], c[PER_LANE];
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
            const int y = min(sg * kDrawSeg + i * 64 + lane, V - 1);
            a[i] = lt[y];
            c[i] = residual ? ld[y] : 0.f;
        }
        // p and q rounded on their own before the difference (no fused
        // multiply-subtract): equal rows give exactly zero residual weight.
#pragma unroll
        for (int i = 0; i < PER_LANE; ++i) {
#pragma clang fp contract(off)
            const bool in = sg * kDrawSeg + i * 64 + lane < V;
            const float pt = exp2f(fmaf(a[i], c2, -d.mt)) * inv_zt;
            const float qd = residual ? exp2f(fmaf(c[i], c2, -d.md)) * inv_zd : 0.f;
            w[i] = in ? (pt > qd ? pt - qd : 0.f) : 0.f;
        }
    };
    for (int pass = 0; pass < 2; ++pass) {
        for (int sg = wave; sg < nseg; sg += kDrawWaves) {
            float w[PER_LANE];
            seg_weights(sg, w);
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) acc += w[i];
            acc = wave_sum(acc);
            if (lane == 0) seg_sum[sg] = acc;
        }
        __syncthreads();
        if (wave == 0) {
            // the running sum over the segments in ascending order, 64 at a time
            float c = 0.f;
            for (int c0 = 0; c0 < nseg; c0 += 64) {
                const float pre = wave_prefix(c0 + lane < nseg ? seg_sum[c0 + lane] : 0.f);
                c += __shfl(pre, 63);
            }
            if (lane == 0) s_total = c;
        }
        __syncthreads();
        const bool retry = residual && !(s_total > 0.f);
        __syncthreads();  // every thread has read s_total (and wave 0 seg_sum) before a second pass
        if (!retry) break;
        residual = false;  // an all-zero residual (p_r == q_r): draw from p_r
    }
    if (wave != 0) return;
    const float theta = pl.uniforms[static_cast<int64_t>(b) * (k + 1) + k] * s_total;
    // The first segment whose inclusive running sum exceeds theta, and the
    // running sum before it (the same operations as the total's).
    int sg = -1;
    float base = 0.f;
    {
        float c = 0.f;
        for (int c0 = 0; c0 < nseg && sg < 0; c0 += 64) {
            const float v = c0 + lane < nseg ? seg_sum[c0 + lane] : 0.f;
            const float pre = wave_prefix(v);
            const uint64_t crossed = __ballot(v > 0.f && c + pre > theta);
            if (crossed) {
                const int L = __builtin_ctzll(crossed);
                const float before = __shfl(pre, L > 0 ? L - 1 : 0);
                sg = c0 + L;
                base = L > 0 ? c + before : c;
            }
            c += __shfl(pre, 63);
        }
    }
    if (sg < 0) {
        // rounding left theta at or past the total: the last segment with
        // weight, whose last positive token is taken
        sg = nseg - 1;
        while (sg > 0 && !(seg_sum[sg] > 0.f)) --sg;
        base = -__builtin_inff();
    }
    int ystar = -1, last_pos = -1;
    float c = base;
    float w[PER_LANE];
    seg_weights(sg, w);
    for (int i = 0; i < PER_LANE && ystar < 0; ++i) {
        const float pre = wave_prefix(w[i]);
        const uint64_t crossed = __ballot(w[i] > 0.f && c + pre > theta);
        const uint64_t pos = __ballot(w[i] > 0.f);
        if (pos) last_pos = sg * kDrawSeg + i * 64 + 63 - __builtin_clzll(pos);
        if (crossed) ystar = sg * kDrawSeg + i * 64 + __builtin_ctzll(crossed);
        c += __shfl(pre, 63);
    }
    if (ystar < 0) ystar = last_pos >= 0 ? last_pos : min(V - 1, sg * kDrawSeg);
    if (lane == 0) pl.out_tokens[static_cast<int64_t>(b) * (k + 1) + r] = ystar;
}

}  // namespace

namespace {

// As many workgroups as the compute units hold at once, a multiple of the
// XCD count, no more than there are items.
hipError_t gemm_grid(const LmPlan& pl, unsigned* grid) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int64_t g = std::max<int64_t>(kXcds, static_cast<int64_t>(cus) * kLmBlocksPerCu / kXcds * kXcds);
    g = std::min<int64_t>(g, (pl.items + kXcds - 1) / kXcds * kXcds);
    *grid = static_cast<unsigned>(g);
    return hipSuccess;
}

template <int MODE>
hipError_t launch_gemm(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    unsigned grid = 0;
    hipError_t e = gemm_grid(pl, &grid);
    if (e != hipSuccess) return e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev0, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_lmhead_gemm<MODE>, dim3(grid), dim3(kLmThreads), 0, stream, pl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev0 && ev1) e = hipEventRecord(ev1, stream);
    return e;
}

}  // namespace

hipError_t launch_lmhead_greedy(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    hipError_t e = launch_gemm<kLmArgmax>(pl, stream, ev0, ev1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lmhead_finish, dim3(static_cast<unsigned>(pl.batch)), dim3(kFinishThreads), 0, stream, pl);
    return hipGetLastError();
}

hipError_t launch_lmhead_sample(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    hipError_t e = launch_gemm<kLmStats>(pl, stream, ev0, ev1);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lmhead_decide, dim3(static_cast<unsigned>(pl.batch)), dim3(kFinishThreads), 0, stream, pl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lmhead_draw, dim3(static_cast<unsigned>(pl.batch)), dim3(kDrawThreads), 0, stream, pl);
    return hipGetLastError();
}

}  // namespace sv
