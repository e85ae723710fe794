// gfx950 kernels of LM-head-fused greedy verification.
//
// What is computed: the T == 0 reading of the acceptance rule (NgramRL essay
// "AI 开始抄自己的作业——而且抄得理直气壮", section "投机解码：让草稿先跑，
// 考官殿后"), with the target's logits formed from its hidden states and
// output-layer weights inside the kernel: l_i(y) = h_i . w_y.  The target's
// choice at a position is its lowest-index argmax; a draft token is kept iff
// it equals that choice; the chain stops at the first mismatch, where the
// target's choice is the committed token.  The logits never reach memory.
//
// Kernels:
//  k_lmhead_argmax   a bf16 GEMM H . W^T on the matrix cores
//                    (v_mfma_f32_32x32x16_bf16, fp32 accumulation) with an
//                    argmax epilogue.  A work item is a 256 x 256 tile (hidden
//                    rows x vocabulary columns); each of the 8 wavefronts
//                    computes a 128 x 64 block.  K is staged through two LDS
//                    buffers 64 at a time.  A slice is four 16-deep MFMA
//                    groups; between the MFMAs of one group the wavefront reads
//                    the next group's fragments, writes the next slice (held in
//                    registers) to the other buffer, or issues the global loads
//                    of the slice after it, in a fixed interleave, so that the
//                    matrix pipe is not left waiting behind a burst of memory
//                    instructions; one barrier per slice, before the last group,
//                    whose MFMAs overlap the reads of the next slice's first
//                    fragments.  The epilogue reduces the tile to (max, lowest
//                    index) per row: one partial per row and vocabulary tile.
//                    The grid is persistent, one workgroup per compute unit,
//                    each taking every G-th item: all workgroups advance
//                    through the items in step, and the items a die (XCD)
//                    takes in one step are consecutive, so the row tiles of
//                    one vocabulary tile run side by side on one die and share
//                    its weight rows in that die's L2.
//  k_lmhead_finish   per sequence: combines its rows' partials, decides every
//                    position on one lane, writes accepted_len and
//                    out_tokens.
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

constexpr int kLdsStride = kLmBK + 8;  // bf16 per staged row: 16 bytes of padding shift the banks row to row

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

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__global__ __launch_bounds__(kLmThreads, kLmBlocksPerCu) void k_lmhead_argmax(LmPlan pl) {
    constexpr int FM = kLmWaveM / 32;  // 32 x 32 fragments per wavefront block
    constexpr int FN = kLmWaveN / 32;
    constexpr int WAVES_M = kLmBM / kLmWaveM;
    constexpr int WAVES_N = kLmBN / kLmWaveN;
    static_assert(WAVES_M * WAVES_N * 64 == kLmThreads, "one wavefront per block of the tile");
    constexpr int ROWS_PER_PASS = kLmThreads / (kLmBK / 8);  // tile rows one pass of 16-byte pieces covers
    constexpr int PA = kLmBM / ROWS_PER_PASS;                 // pieces per thread: A
    constexpr int PB = kLmBN / ROWS_PER_PASS;                 // and B
    static_assert(PA * ROWS_PER_PASS == kLmBM && PB * ROWS_PER_PASS == kLmBN, "whole passes");
    static_assert(kLmHiddenMultiple % kLmBK == 0, "whole K slices");
    __shared__ __attribute__((aligned(16))) uint16_t sa[2][kLmBM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2][kLmBN * kLdsStride];
    __shared__ float cand_v[WAVES_N][kLmBM];
    __shared__ int cand_i[WAVES_N][kLmBM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % WAVES_M;  // row block of the tile
    const int wn = wave / WAVES_M;  // column block of the tile
    const int D = pl.hidden;
    const int kblocks = D / kLmBK;
    const int64_t items = lmhead_items(pl);
    const int G = gridDim.x;  // a multiple of kXcds
    // Blocks are dealt to the XCDs by index mod 8: give each die a run of
    // consecutive items per step.
    const int slot = (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;

    // Piece q of a thread: tile row tid / 4 + ROWS_PER_PASS q, K segment
    // tid % 4 (8 bf16 each).  Rows past the end of H or W are read as the
    // last row (their results are never written or are masked out), so no
    // load is guarded.
    const int prow = tid / (kLmBK / 8);
    const int pseg = tid % (kLmBK / 8);
    uint16_t* const sa_st = &sa[0][prow * kLdsStride + pseg * 8];
    uint16_t* const sb_st = &sb[0][prow * kLdsStride + pseg * 8];

    for (int64_t item = slot; item < items; item += G) {
        const int mt = static_cast<int>(item % pl.m_tiles);
        const int nt = static_cast<int>(item / pl.m_tiles);
        const int m0 = mt * kLmBM;
        const int n0 = nt * kLmBN;
        const uint16_t* const a_base = pl.hidden_states + static_cast<int64_t>(m0) * D;
        const uint16_t* const b_base = pl.weight + static_cast<int64_t>(n0) * D;
        const int a_last = pl.rows - 1 - m0;
        const int b_last = pl.vocab - 1 - n0;
        uint32_t a_off[PA], b_off[PB];  // elements from the tile's base, < 256 * 65536
#pragma unroll
        for (int q = 0; q < PA; ++q) a_off[q] = static_cast<uint32_t>(min(prow + q * ROWS_PER_PASS, a_last) * D + pseg * 8);
#pragma unroll
        for (int q = 0; q < PB; ++q) b_off[q] = static_cast<uint32_t>(min(prow + q * ROWS_PER_PASS, b_last) * D + pseg * 8);
        floatx16_t acc[FM][FN];
#pragma unroll
        for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

        uint4 ra[PA], rb[PB];
        static_assert(kLmBK == 64, "four 16-deep MFMA groups per slice");
        constexpr int NMF = FM * FN;     // MFMAs per group
        constexpr int NRD = FM + FN;     // fragment reads per group
        constexpr int NGL = PA + PB;     // global loads (and LDS writes) per slice
        static_assert(2 * NMF >= NRD && NMF >= NGL, "interleave slots");
        bf16x8_t f0a[FM], f0b[FN], f1a[FM], f1b[FN];
#define LM_FRAGS(FA, FB, BUF, KS)                                                           \
    {                                                                                       \
        const int kcol_ = (KS) * 16 + 8 * (lane >> 5);                                      \
        _Pragma("unroll") for (int mi = 0; mi < FM; ++mi)                                   \
            FA[mi] = *reinterpret_cast<const bf16x8_t*>(&sa[BUF][(wm * kLmWaveM + mi * 32 + (lane & 31)) * kLdsStride + kcol_]); \
        _Pragma("unroll") for (int ni = 0; ni < FN; ++ni)                                   \
            FB[ni] = *reinterpret_cast<const bf16x8_t*>(&sb[BUF][(wn * kLmWaveN + ni * 32 + (lane & 31)) * kLdsStride + kcol_]); \
    }
#define LM_MFMA(FA, FB)                                                                     \
    {                                                                                       \
        _Pragma("unroll") for (int mi = 0; mi < FM; ++mi)                                   \
            _Pragma("unroll") for (int ni = 0; ni < FN; ++ni)                               \
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(FA[mi], FB[ni], acc[mi][ni], 0, 0, 0); \
    }
// After each MFMA of a group: up to two fragment reads (READS), one global load (LOADS), one LDS write (WRITES).
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

        // Pipeline over K slices with two LDS buffers: slice kb+1 is written
        // to the other buffer during group 2 of step kb, a barrier follows,
        // and group 3 reads the first fragments of slice kb+1 and issues the
        // global loads of slice kb+2 while its MFMAs run.
#pragma unroll
        for (int q = 0; q < PA; ++q) ra[q] = ld16(a_base + a_off[q]);
#pragma unroll
        for (int q = 0; q < PB; ++q) rb[q] = ld16(b_base + b_off[q]);
        __syncthreads();  // the previous item's readers of the buffers and of cand are done
#pragma unroll
        for (int q = 0; q < PA; ++q) *reinterpret_cast<uint4*>(sa_st + q * ROWS_PER_PASS * kLdsStride) = ra[q];
#pragma unroll
        for (int q = 0; q < PB; ++q) *reinterpret_cast<uint4*>(sb_st + q * ROWS_PER_PASS * kLdsStride) = rb[q];
        {
            const int k1 = min(1, kblocks - 1) * kLmBK;
#pragma unroll
            for (int q = 0; q < PA; ++q) ra[q] = ld16(a_base + k1 + a_off[q]);
#pragma unroll
            for (int q = 0; q < PB; ++q) rb[q] = ld16(b_base + k1 + b_off[q]);
        }
        __syncthreads();
        LM_FRAGS(f0a, f0b, 0, 0);
        for (int kb = 0; kb < kblocks; ++kb) {
            const int cur = kb & 1;
            const int nxt = cur ^ 1;
            const int kload = min(kb + 2, kblocks - 1) * kLmBK;  // clamped: the last steps reload a slice nobody reads
            __builtin_amdgcn_sched_barrier(0);
            // group 0: reads of group 1
            LM_FRAGS(f1a, f1b, cur, 1);
            LM_MFMA(f0a, f0b);
            LM_INTERLEAVE(true, false, false);
            __builtin_amdgcn_sched_barrier(0);
            // group 1: reads of group 2
            LM_FRAGS(f0a, f0b, cur, 2);
            LM_MFMA(f1a, f1b);
            LM_INTERLEAVE(true, false, false);
            __builtin_amdgcn_sched_barrier(0);
            // group 2: reads of group 3, slice kb+1 (staged in registers) to the other buffer
            LM_FRAGS(f1a, f1b, cur, 3);
#pragma unroll
            for (int q = 0; q < PA; ++q)
                *reinterpret_cast<uint4*>(sa_st + (nxt * kLmBM + q * ROWS_PER_PASS) * kLdsStride) = ra[q];
#pragma unroll
            for (int q = 0; q < PB; ++q)
                *reinterpret_cast<uint4*>(sb_st + (nxt * kLmBN + q * ROWS_PER_PASS) * kLdsStride) = rb[q];
            LM_MFMA(f0a, f0b);
            LM_INTERLEAVE(true, false, true);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();  // slice kb+1 visible; every read of this buffer done
            // group 3: first fragments of slice kb+1, global loads of slice kb+2
            LM_FRAGS(f0a, f0b, nxt, 0);
#pragma unroll
            for (int q = 0; q < PA; ++q) ra[q] = ld16(a_base + kload + a_off[q]);
#pragma unroll
            for (int q = 0; q < PB; ++q) rb[q] = ld16(b_base + kload + b_off[q]);
            LM_MFMA(f1a, f1b);
            LM_INTERLEAVE(true, true, false);
        }
        __builtin_amdgcn_sched_barrier(0);
#undef LM_INTERLEAVE
#undef LM_MFMA
#undef LM_FRAGS

        // Epilogue: accumulator j of lane l holds row 8(j/4) + 4(l/32) + j%4
        // of a 32 x 32 block, column l % 32.
#pragma unroll
        for (int mi = 0; mi < FM; ++mi) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float v = neg_inf_f();
                int idx = INT_MAX;
#pragma unroll
                for (int ni = 0; ni < FN; ++ni) {
                    const int col = n0 + wn * kLmWaveN + ni * 32 + (lane & 31);
                    if (col < pl.vocab) better(v, idx, acc[mi][ni][j], col);
                }
                half_wave_argmax(v, idx);
                const int row = wm * kLmWaveM + mi * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
                if ((lane & 31) == 0) {
                    cand_v[wn][row] = v;
                    cand_i[wn][row] = idx;
                }
            }
        }
        __syncthreads();
        for (int r = tid; r < kLmBM; r += kLmThreads) {
            const int m = m0 + r;
            if (m < pl.rows) {
                float v = cand_v[0][r];
                int idx = cand_i[0][r];
#pragma unroll
                for (int c = 1; c < WAVES_N; ++c) better(v, idx, cand_v[c][r], cand_i[c][r]);
                pl.part_v[static_cast<int64_t>(m) * pl.n_parts + nt] = v;
                pl.part_i[static_cast<int64_t>(m) * pl.n_parts + nt] = idx;
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

}  // namespace

hipError_t launch_lmhead(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    hipError_t e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev0, stream);
        if (e != hipSuccess) return e;
    }
    // As many workgroups as the compute units hold at once, a multiple of
    // the XCD count, no more than there are items.
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t items = lmhead_items(pl);
    int64_t grid = std::max<int64_t>(kXcds, static_cast<int64_t>(cus) * kLmBlocksPerCu / kXcds * kXcds);
    grid = std::min<int64_t>(grid, (items + kXcds - 1) / kXcds * kXcds);
    hipLaunchKernelGGL(k_lmhead_argmax, dim3(static_cast<unsigned>(grid)), dim3(kLmThreads), 0, stream, pl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev1, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_lmhead_finish, dim3(static_cast<unsigned>(pl.batch)), dim3(kFinishThreads), 0, stream, pl);
    return hipGetLastError();
}

}  // namespace sv
