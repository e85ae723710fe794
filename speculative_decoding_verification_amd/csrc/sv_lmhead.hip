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
//                    argmax epilogue.  A workgroup owns 128 hidden rows and a
//                    run of 8 vocabulary tiles of 128; per tile it stages
//                    32-wide slices of K for both operands in LDS (double
//                    buffered), each wave computes a 64 x 64 block, and the
//                    epilogue folds the tile into a running (max, lowest
//                    index) per row.  The run's result is one partial per row.
//                    Workgroups of one vocabulary run sit on one XCD (grid
//                    index = XCD + 8 * slot), so the run's weight rows are
//                    fetched into that XCD's L2 once for all its row tiles.
//  k_lmhead_finish   per sequence: combines its rows' partials, decides every
//                    position on one lane, writes accepted_len and
//                    out_tokens.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "sv_lmhead.h"

namespace sv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kLdsStride = kLmBK + 8;  // bf16 per staged row: 80 bytes, shifts banks row to row

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

__global__ __launch_bounds__(kLmThreads) void k_lmhead_argmax(LmPlan pl) {
    __shared__ __attribute__((aligned(16))) uint16_t sa[2][kLmBM * kLdsStride];
    __shared__ __attribute__((aligned(16))) uint16_t sb[2][kLmBN * kLdsStride];
    __shared__ float cand_v[2][kLmBM];
    __shared__ int cand_i[2][kLmBM];
    __shared__ float run_v[kLmBM];
    __shared__ int run_i[kLmBM];

    // Grid index -> (vocabulary run ng, row tile mt); all row tiles of a run
    // share an XCD (blocks are spread over the 8 XCDs by index mod 8).
    const int x = blockIdx.x;
    const int slot = x / kXcds;
    const int mt = slot % pl.m_tiles;
    const int ng = (slot / pl.m_tiles) * kXcds + x % kXcds;
    if (ng >= pl.n_runs) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1;   // 64-row half of the tile
    const int wn = wave >> 1;  // 64-column half of the tile
    const int m0 = mt * kLmBM;
    const int D = pl.hidden;
    const int kblocks = D / kLmBK;

    for (int r = tid; r < kLmBM; r += kLmThreads) {
        run_v[r] = neg_inf_f();
        run_i[r] = INT_MAX;
    }

    // Global -> LDS: 512 16-byte pieces per operand tile, two per thread.
    // Piece c: row c / 4, K segment c % 4 (8 bf16 each).
    int a_row[2], seg[2];
    const uint16_t* a_src[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = tid + q * kLmThreads;
        a_row[q] = c >> 2;
        seg[q] = c & 3;
        const int m = m0 + a_row[q];
        a_src[q] = m < pl.rows ? pl.hidden_states + static_cast<int64_t>(m) * D + seg[q] * 8 : nullptr;
    }
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);

    for (int nt = 0; nt < kLmRunTiles; ++nt) {
        const int n0 = (ng * kLmRunTiles + nt) * kLmBN;
        if (n0 >= pl.vocab) break;
        const uint16_t* b_src[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int n = n0 + a_row[q];
            b_src[q] = n < pl.vocab ? pl.weight + static_cast<int64_t>(n) * D + seg[q] * 8 : nullptr;
        }
        floatx16_t acc[2][2];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

        uint4 ra[2], rb[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            ra[q] = a_src[q] ? ld16(a_src[q]) : zero;
            rb[q] = b_src[q] ? ld16(b_src[q]) : zero;
        }
        __syncthreads();  // the previous tile's readers of buffer 0 are done
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            *reinterpret_cast<uint4*>(&sa[0][a_row[q] * kLdsStride + seg[q] * 8]) = ra[q];
            *reinterpret_cast<uint4*>(&sb[0][a_row[q] * kLdsStride + seg[q] * 8]) = rb[q];
        }
        __syncthreads();

        for (int kb = 0; kb < kblocks; ++kb) {
            const int cur = kb & 1;
            const bool more = kb + 1 < kblocks;
            if (more) {
                const int koff = (kb + 1) * kLmBK;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    ra[q] = a_src[q] ? ld16(a_src[q] + koff) : zero;
                    rb[q] = b_src[q] ? ld16(b_src[q] + koff) : zero;
                }
            }
#pragma unroll
            for (int ks = 0; ks < kLmBK / 16; ++ks) {
                const int kcol = ks * 16 + 8 * (lane >> 5);
                bf16x8_t fa[2], fb[2];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi) {
                    const int row = wm * 64 + mi * 32 + (lane & 31);
                    fa[mi] = *reinterpret_cast<const bf16x8_t*>(&sa[cur][row * kLdsStride + kcol]);
                }
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int row = wn * 64 + ni * 32 + (lane & 31);
                    fb[ni] = *reinterpret_cast<const bf16x8_t*>(&sb[cur][row * kLdsStride + kcol]);
                }
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
            }
            if (more) {
                const int nxt = cur ^ 1;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    *reinterpret_cast<uint4*>(&sa[nxt][a_row[q] * kLdsStride + seg[q] * 8]) = ra[q];
                    *reinterpret_cast<uint4*>(&sb[nxt][a_row[q] * kLdsStride + seg[q] * 8]) = rb[q];
                }
            }
            __syncthreads();
        }

        // Epilogue: accumulator j of lane l holds row 8(j/4) + 4(l/32) + j%4
        // of a 32 x 32 block, column l % 32.
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float v = neg_inf_f();
                int idx = INT_MAX;
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) {
                    const int col = n0 + wn * 64 + ni * 32 + (lane & 31);
                    if (col < pl.vocab) better(v, idx, acc[mi][ni][j], col);
                }
                half_wave_argmax(v, idx);
                const int row = wm * 64 + mi * 32 + 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
                if ((lane & 31) == 0) {
                    cand_v[wn][row] = v;
                    cand_i[wn][row] = idx;
                }
            }
        }
        __syncthreads();
        for (int r = tid; r < kLmBM; r += kLmThreads) {
            float v = run_v[r];
            int idx = run_i[r];
            better(v, idx, cand_v[0][r], cand_i[0][r]);
            better(v, idx, cand_v[1][r], cand_i[1][r]);
            run_v[r] = v;
            run_i[r] = idx;
        }
        // (the next tile's first barrier orders these updates before reuse)
    }
    __syncthreads();
    for (int r = tid; r < kLmBM; r += kLmThreads) {
        const int m = m0 + r;
        if (m < pl.rows) {
            pl.part_v[static_cast<int64_t>(m) * pl.n_runs + ng] = run_v[r];
            pl.part_i[static_cast<int64_t>(m) * pl.n_runs + ng] = run_i[r];
        }
    }
}

// One wavefront per sequence: row argmaxes from the partials, then the
// decisions on lane i for position i.
__global__ __launch_bounds__(64) void k_lmhead_finish(LmPlan pl) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int k = pl.k;
    const int n_rows = k + 1;
    int my_g = -1;    // lane i: the choice at position i < k
    int g_last = -1;  // the choice at position k (after full acceptance)
    for (int i = 0; i < n_rows; ++i) {
        const int64_t row = static_cast<int64_t>(b) * n_rows + i;
        float v = neg_inf_f();
        int idx = INT_MAX;
        for (int c = lane; c < pl.n_runs; c += 64) better(v, idx, pl.part_v[row * pl.n_runs + c], pl.part_i[row * pl.n_runs + c]);
        half_wave_argmax(v, idx);
        const float v2 = __shfl_xor(v, 32);
        const int i2 = __shfl_xor(idx, 32);
        better(v, idx, v2, i2);
        if (lane == i) my_g = idx;
        if (i == k) g_last = idx;
        if (pl.argmax_out && lane == 0) pl.argmax_out[row] = idx;
    }
    const bool active = lane < k;
    int x = 0;
    if (active) x = pl.tokens[static_cast<int64_t>(b) * k + lane];
    const bool bad = active && (x < 0 || x >= pl.vocab);
    const bool invalid = __ballot(bad) != 0ull;
    const uint64_t mismatch = __ballot(active && x != my_g);
    const int r = invalid ? -1 : (mismatch ? __builtin_ctzll(mismatch) : k);
    const int g_r = r < 0 ? -1 : (r == k ? g_last : __shfl(my_g, r));
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

int64_t lmhead_grid_blocks(const LmPlan& pl) {
    const int64_t groups = (static_cast<int64_t>(pl.n_runs) + kXcds - 1) / kXcds;
    return groups * kXcds * pl.m_tiles;
}

hipError_t launch_lmhead(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    hipError_t e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev0, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_lmhead_argmax, dim3(static_cast<unsigned>(lmhead_grid_blocks(pl))), dim3(kLmThreads), 0,
                       stream, pl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev1, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_lmhead_finish, dim3(static_cast<unsigned>(pl.batch)), dim3(64), 0, stream, pl);
    return hipGetLastError();
}

}  // namespace sv
