// Launch interface of the LM-head-fused greedy verification kernels
// (sv_lmhead.hip).  Host code builds an LmPlan and calls launch_lmhead.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace sv {

constexpr int kLmBM = 128;        // hidden rows per workgroup tile
constexpr int kLmBN = 128;        // vocabulary columns per tile
constexpr int kLmBK = 32;         // K slice staged in LDS per step
constexpr int kLmThreads = 256;   // 4 wavefronts, each a 64 x 64 block of the tile
constexpr int kLmRunTiles = 8;    // vocabulary tiles one workgroup walks (its "run")
constexpr int kXcds = 8;          // accelerator complex dies of gfx950

struct LmPlan {
    const uint16_t* hidden_states;  // [rows][hidden] bf16
    const uint16_t* weight;         // [vocab][hidden] bf16
    const int32_t* tokens;          // [batch][k]
    int32_t* accepted_len;          // [batch]
    int32_t* out_tokens;            // [batch][k+1]
    int32_t* argmax_out;            // [rows] or null
    float* part_v;                  // workspace: [rows][n_runs] run maxima
    int32_t* part_i;                // workspace: [rows][n_runs] their lowest indices
    int32_t rows;                   // batch * (k + 1)
    int32_t batch;
    int32_t k;
    int32_t vocab;
    int32_t hidden;                 // multiple of kLmBK
    int32_t m_tiles;                // ceil(rows / kLmBM)
    int32_t n_runs;                 // ceil(ceil(vocab / kLmBN) / kLmRunTiles)
};

// Blocks of the GEMM launch (a multiple of kXcds).
int64_t lmhead_grid_blocks(const LmPlan& pl);

// Enqueues the GEMM + argmax launch and the per-sequence finisher on
// `stream`.  When both events are given they bracket the GEMM launch.
hipError_t launch_lmhead(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace sv
