// Internal interface between the C-ABI layer (sv_api.cpp) and the gfx950
// kernels (sv_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>

#include "sv_grid.h"

namespace sv {

// One wavefront streams one "chunk" of a logit row: 64 lanes x 8 vectors of
// 16 bytes = 8 KiB, i.e. 2048 fp32 or 4096 bf16 logits.
constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kVecPerLane = 8;
constexpr int kChunkBytes = kWave * kVecPerLane * 16;

inline int chunk_elems(int elem_bytes) { return kChunkBytes / elem_bytes; }

// Per-sequence sampling modes written by the accept kernel.
enum SampleMode : int32_t {
    kModeDone = 0,     // nothing left to draw (greedy, invalid token, VAT)
    kModeBonus = 1,    // all k kept: draw from target row k
    kModeOneHot = 2,   // one-hot draft rejected at r: draw from p_r without x_r
    kModeResidual = 3  // draft logits rejected at r: draw from max(0, p_r - q_r)
};

// Tagged words the decision finisher of a sequence leaves for the residual
// and bonus roles (see kTagFirst).
enum DecisionWord : int32_t {
    kDecRMode = 0,  // (r + 2) | mode << 16; r = -1 invalid token, -2 timed out
    kDecMt = 1,     // max of target row r (residual)
    kDecZt = 2,     // Z of target row r
    kDecMd = 3,     // max of draft row r
    kDecZd = 4,     // Z of draft row r
    kDecU = 5,      // the uniform of the draw
    kDecWords = 8
};

// Everything the kernels of one call need.  Global row numbering (row_mz,
// row_stats_out): target rows 0 .. rows_t-1 (sequence b, position i ->
// b*target_rows_per_seq + i), then draft rows rows_t .. rows_t+rows_d-1
// (b, i -> rows_t + b*k + i).  Within a sequence, local row j < n_t is target
// position j and j >= n_t is draft position j - n_t.
struct Plan {
    int32_t batch;            // B (verify) or N (VAT)
    int32_t k;
    int32_t vocab;
    int32_t elem_bytes;       // 4 fp32, 2 bf16
    int32_t target_rows_per_seq;  // k+1 (verify) or k (VAT)
    int32_t chunks;           // P = ceil(V / chunk)
    int32_t chunk;            // elements per chunk
    // Per sequence, the chunk partials hold local rows: target positions
    // 0..k-1, then draft positions 0..k-1 (when draft logits are read), then
    // the bonus row (target position k, verification only).
    int32_t dec_rows;         // rows the decision reads: k or 2k
    int32_t rows_per_seq;     // dec_rows + (1 if there is a bonus row)
    int32_t words_per_seq;    // hand-off words of one sequence in `partials`
    bool has_resid;           // draft logits at T > 0: residual roles exist
    bool has_bonus;           // verification (not VAT): bonus roles exist
    int32_t nc_dec, nc_bonus, nc_res;  // chunks per worker wavefront
    int32_t eager_bonus_from; // sequences b >= this read their bonus row without waiting for the decision
    bool two_deep_polls;      // finishers keep two reads of their words in flight (grids of one residency)
    uint32_t tag;             // this call's tag of hand-off words
    int64_t rows_t;
    int64_t rows_d;           // 0 for one-hot drafts and T == 0
    bool vec;                 // 16-byte loads allowed (aligned rows)
    bool greedy;              // T == 0
    bool onehot;
    bool vat;
    bool vat_loss;            // VAT with the training loss: workers read chunk pairs
    float temperature;
    float c2;                 // log2(e) / T
    float decay;

    const void* target;
    const void* draft;
    const int32_t* tokens;
    const float* uniforms;

    int32_t* accepted_len;
    int32_t* out_tokens;
    uint8_t* mask;
    int32_t* first_reject;
    float* weights;
    float* probs_out;
    float* row_stats_out;
    const int32_t* hard_tokens;  // VAT loss: the target's sampled token per position
    float hard_weight;
    float* soft_ce;           // [N][k] -sum_y p(y) ln q(y)
    float* hard_ce;           // [N][k] -ln q(h)
    float* block_loss;        // [N] sum_i w_i (soft_i + hard_weight * hard_i)

    // workspace regions
    uint64_t* partials;       // [B][R_s][P][2] tagged words (m, s) or (max, index);
                              // VAT loss: [B][k][P][5] (pair partials)
    uint64_t* resid;          // [B][P] tagged residual masses
    uint64_t* dec;            // [B][kDecWords] tagged decision words

    TaskGrid grid;            // role of every block of the launch
};

// Blocks the GPU keeps resident at once (256 CUs x ~5 workgroups of 256
// threads): the lag, in blocks, between a sequence's worker blocks and its
// finisher block.
constexpr int64_t kResidentBlocks = 1280;

// Chunks each worker wavefront streams, one after the other.  Two per wave
// for large calls: block dispatch (on the order of 150-200 blocks per
// microsecond) would otherwise bound the grid; one per wave for small calls,
// where the drain of long-lived blocks at the end dominates.  Residual
// workers read two rows per chunk and take one chunk pair per wave.
constexpr int kChunksPerWave = 2;
constexpr int kChunksPerWaveSmall = 1;
constexpr int64_t kSmallCallChunks = 4 * kWavesPerBlock * kResidentBlocks;
constexpr int kChunksPerWaveResid = 1;
constexpr int kChunksPerWaveBonus = 2;

// Values handed between blocks inside a kernel travel as 64-bit words,
// written and read whole (single-copy atomic): 32 data bits and a 32-bit tag
// that names the call.  Tags run 1 .. 2^32 - 1 over the calls a process makes;
// a zero-filled slot matches none.  A reader polls until every word it needs
// carries its call's tag, so no slot needs clearing between calls.
constexpr uint32_t kTagFirst = 1u;
constexpr uint32_t kTagCount = 0xffffffffu;

// Staging capacity of a finisher block in LDS: 32-bit words of partials.
constexpr int kStageWords = 4096;

struct WorkspaceLayout {
    size_t partials, resid, dec, total;
};

// partial_words: tagged words of chunk partials over the whole call.
WorkspaceLayout workspace_layout(int64_t partial_words, int64_t batch, int64_t chunks);

// Words per chunk pair of the VAT loss: (m_t, s_t, m_d, s_d, x).
constexpr int kPairWords = 5;

// Enqueue the whole path on `stream`.  Returns hipSuccess or the first error.
hipError_t launch_path(const Plan& plan, hipStream_t stream, hipEvent_t probe_start, hipEvent_t probe_stop);

// Histogram of accepted lengths into hist[0 .. k+3] (one block).
hipError_t launch_accept_hist(const int32_t* acc, int32_t batch, int32_t k, int32_t* hist, hipStream_t stream);

// The VAT loss gradient with respect to the draft logits (sv_vat_loss_grad).
struct GradPlan {
    const void* target;       // [rows][V] logits, elem_bytes each
    const void* draft;        // [rows][V]
    const int32_t* hard;      // [rows] hard tokens
    const float* weights;     // [rows] VAT weights
    const float* row_stats;   // [2 rows][2]: (m/T, Z), target rows then draft rows
    float* grad;              // [rows][V] out
    int64_t rows;             // N k
    int64_t items;            // rows * chunks
    int32_t vocab;
    int32_t chunks;           // ceil(V / chunk)
    int32_t elem_bytes;
    bool vec;                 // 16-byte rows and pointers
    float c2;                 // log2(e) / T
    float inv_t;              // 1 / T
    float hard_weight;
};

hipError_t launch_vat_grad(const GradPlan& g, hipStream_t stream, hipEvent_t probe_start, hipEvent_t probe_stop);

}  // namespace sv
