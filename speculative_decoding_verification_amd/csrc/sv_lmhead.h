// Launch interface of the LM-head-fused greedy verification kernels
// (sv_lmhead.hip).  Host code builds an LmPlan and calls launch_lmhead.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace sv {

constexpr int kLmBM = 256;        // hidden rows per workgroup tile
constexpr int kLmBN = 256;        // vocabulary columns per tile
constexpr int kLmBK = 64;         // K slice staged in LDS per step
constexpr int kLmWaveM = 128;     // rows of one wavefront's block of the tile
constexpr int kLmWaveN = 64;     // columns of one wavefront's block
constexpr int kLmThreads = 512;   // 8 wavefronts in a 2 x 4 arrangement
constexpr int kLmBlocksPerCu = 1; // workgroups one compute unit holds (LDS and registers)
constexpr int kLmHiddenMultiple = 64;  // the hidden sizes accepted (a multiple of kLmBK)
constexpr int kXcds = 8;          // accelerator complex dies of gfx950

struct LmPlan {
    const uint16_t* hidden_states;  // [rows][hidden] bf16
    const uint16_t* weight;         // [vocab][hidden] bf16
    const int32_t* tokens;          // [batch][k]
    int32_t* accepted_len;          // [batch]
    int32_t* out_tokens;            // [batch][k+1]
    int32_t* argmax_out;            // [rows] or null
    float* part_v;                  // workspace: [rows][n_parts] tile maxima
    int32_t* part_i;                // workspace: [rows][n_parts] their lowest indices
    int32_t rows;                   // batch * (k + 1)
    int32_t batch;
    int32_t k;
    int32_t vocab;
    int32_t hidden;                 // multiple of kLmBK
    int32_t m_tiles;                // ceil(rows / kLmBM)
    int32_t n_tiles;                // ceil(vocab / kLmBN)
    int32_t n_parts;                // partials per row: one per vocabulary tile
};

// Host: tile counts of a plan whose rows and vocab are set.
inline void lmhead_shape(LmPlan* pl) {
    pl->m_tiles = (pl->rows + kLmBM - 1) / kLmBM;
    pl->n_tiles = (pl->vocab + kLmBN - 1) / kLmBN;
    pl->n_parts = pl->n_tiles;
}

// Tiles (work items) of one call.
__host__ __device__ inline int64_t lmhead_items(const LmPlan& pl) { return static_cast<int64_t>(pl.m_tiles) * pl.n_tiles; }

// Enqueues the GEMM + argmax launch (a persistent grid of one workgroup per
// compute unit of the current device) and the per-sequence finisher on
// `stream`.  When both events are given they bracket the GEMM launch.
hipError_t launch_lmhead(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace sv
