// Launch interface of the LM-head-fused verification kernels (sv_lmhead.hip).
// Host code builds an LmPlan and calls launch_lmhead_greedy or
// launch_lmhead_sample.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace sv {

constexpr int kLmBM = 256;        // hidden rows per workgroup tile
constexpr int kLmBN = 256;        // vocabulary columns per tile
constexpr int kLmBK = 64;         // K slice staged in LDS per step
constexpr int kLmWaveM = 128;     // rows of one wavefront's block of the tile
constexpr int kLmWaveN = 64;      // columns of one wavefront's block
constexpr int kLmThreads = 512;   // 8 wavefronts in a 2 x 4 arrangement
constexpr int kLmBlocksPerCu = 1; // workgroups one compute unit holds (LDS and registers)
constexpr int kLmHiddenMultiple = 64;  // the hidden sizes accepted (a multiple of kLmBK)
constexpr int kXcds = 8;          // accelerator complex dies of gfx950

// What the GEMM's epilogue makes of a 256 x 256 tile of logits.
enum LmMode : int32_t {
    kLmArgmax = 0,  // per row: (max, lowest index)
    kLmStats = 1    // per row: m = max l c2, s = sum 2^(l c2 - m); the logit of the row's token; and the
                    // logits themselves, fp32
};

// Which token's logit a statistics row captures.
enum LmTokens : int32_t {
    kLmNoTokens = 0,
    kLmTargetTokens = 1,  // row m = b(k+1) + i: token x_i for i < k, none at i = k
    kLmDraftTokens = 2    // row m = b k + i: token x_i
};

// One GEMM of a launch: rows of A (hidden states) times W^T.
struct LmGemm {
    const uint16_t* a;  // hidden states, bf16, hidden-contiguous
    const uint16_t* w;  // [vocab][hidden] bf16
    int32_t rows;       // rows this GEMM computes
    int32_t m_tiles;    // ceil(rows / kLmBM)
    int64_t item0;      // its first work item in the launch
    int32_t out_row0;   // its first row in the per-row outputs
    int32_t tokens;     // LmTokens (statistics mode)
};

// Per-sequence result of the decision step of sampling verification.
struct LmSeqDraw {
    int32_t r;     // first rejection (k: none; -1: invalid token)
    float mt, zt;  // target row at the draw: p(y) = 2^(l(y) c2 - mt) / zt
    float md, zd;  // draft row at r (r < k)
    int32_t pad[3];
};

struct LmPlan {
    LmGemm g[2];
    int32_t n_gemms;
    int32_t mode;                   // LmMode of the GEMM launch
    int64_t items;                  // work items over all GEMMs
    const int32_t* tokens;          // [batch][k]
    const float* uniforms;          // [batch][k+1] (sampling)
    int32_t* accepted_len;          // [batch]
    int32_t* out_tokens;            // [batch][k+1]
    int32_t* argmax_out;            // [batch (k+1)] or null (greedy)
    float* probs_out;               // [batch][k][2] or null (sampling)
    float* part_v;                  // workspace [rows][n_parts]: argmax max, or statistics m
    int32_t* part_i;                // workspace [rows][n_parts]: argmax index (greedy)
    float* part_s;                  // workspace [rows][n_parts]: statistics s (sampling)
    float* lx;                      // workspace [rows]: the logit of the row's token (sampling)
    LmSeqDraw* seq;                 // workspace [batch] (sampling)
    float* logits;                  // workspace [rows_t + rows_d][vocab], fp32 (sampling): every row's logits
    int32_t batch;
    int32_t k;
    int32_t vocab;
    int32_t hidden;                 // multiple of kLmHiddenMultiple
    int32_t n_tiles;                // ceil(vocab / kLmBN)
    int32_t n_parts;                // partials per row: one per vocabulary tile
    int32_t rows_t;                 // target rows: batch (k+1)
    float c2;                       // log2(e) / T (sampling)
};

// Host: tile counts and item ranges of the GEMMs whose rows are set.
inline void lmhead_layout(LmPlan* pl) {
    pl->n_tiles = (pl->vocab + kLmBN - 1) / kLmBN;
    pl->n_parts = pl->n_tiles;
    int64_t item = 0;
    for (int i = 0; i < pl->n_gemms; ++i) {
        pl->g[i].m_tiles = (pl->g[i].rows + kLmBM - 1) / kLmBM;
        pl->g[i].item0 = item;
        item += static_cast<int64_t>(pl->g[i].m_tiles) * pl->n_tiles;
    }
    pl->items = item;
}

// Greedy verification: the argmax GEMM over the target rows (bracketed by
// the events when both are given), then the per-sequence finisher.
hipError_t launch_lmhead_greedy(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

// Sampling verification: the statistics GEMM over target and draft rows
// (bracketed by the events; it also stores every row's logits), the
// decision step, then the draws from the stored rows.
hipError_t launch_lmhead_sample(const LmPlan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);

}  // namespace sv
