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

// Specialisations of the verification kernel: which rows a call streams and
// which roles its grid holds are fixed per specialisation, so each carries
// only its own code.
enum PathMode : int32_t {
    kPathSample = 0,     // verification with draft logits, T > 0
    kPathOneHot = 1,     // verification with one-hot drafts, T > 0
    kPathGreedy = 2,     // verification, T == 0
    kPathVat = 3,        // VAT labels, T > 0
    kPathVatGreedy = 4,  // VAT labels, T == 0
    kPathVatLoss = 5,    // VAT labels, weights and loss
};

// Everything the kernels of one call need.  Global row numbering (row_mz,
// row_stats_out): target rows 0 .. rows_t-1 (sequence b, position i ->
// b*target_rows_per_seq + i), then draft rows rows_t .. rows_t+rows_d-1
// (b, i -> rows_t + b*k + i).  Within a sequence, local row j < dec_rows is
// position j / halves, its target row when j % halves == 0 and its draft
// row otherwise; local row dec_rows is the bonus row (target position k).
struct Plan {
    int32_t batch;            // B (verify) or N (VAT)
    int32_t k;
    int32_t vocab;
    int32_t elem_bytes;       // 4 fp32, 2 bf16
    int32_t target_rows_per_seq;  // k+1 (verify) or k (VAT)
    int32_t chunks;           // P = ceil(V / chunk)
    int32_t chunk;            // elements per chunk
    int32_t path;             // PathMode
    int32_t halves;           // rows per position among the decision rows: 2 with draft logits, else 1
    int32_t dec_rows;         // k * halves (VAT loss: k chunk-pair rows)
    int32_t rows_per_seq;     // dec_rows + (1 if there is a bonus row)
    int32_t words_per_seq;    // chunk words of one sequence (two per row chunk; VAT loss: five per pair)
    int32_t segs;             // S: segments per row, one per decision worker block
    int32_t seg_chunks;       // chunks per segment (four wavefronts x nc_dec)
    int32_t seg_words_per_seq;  // segment words of one sequence: rows_per_seq * S * 2
    int32_t nc_dec, nc_res;   // chunks per worker wavefront
    int32_t eager_bonus_from; // sequences b >= this read their bonus row without deciding first
    int32_t pos_major;        // decision worker blocks ordered position-major over all sequences
    int32_t window;           // > 0 (window mode): no row after a known rejection is read; unless the
                              // previous call on the workspace rejected every sequence at position 0,
                              // every other row is read at once, else the rows of position i >= window
                              // only once the sequence's accepted prefix a has i < window +
                              // kWindowGrowth * a
    // Flags are 32-bit: a byte-sized field at an unaligned offset of the
    // kernel argument block is read with a vector load (a memory round trip
    // at the start of every block) instead of a scalar one.
    int32_t two_deep_polls;   // (nearly) the whole grid resident at once: poll with short sleeps
    int32_t vec;              // 16-byte loads allowed (aligned rows)
    int32_t greedy;           // T == 0
    uint32_t tag;             // this call's tag of hand-off words
    int64_t rows_t;
    int64_t rows_d;           // 0 for one-hot drafts and T == 0
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
    uint64_t* chunkw;         // [B][rows_per_seq][P][2] tagged chunk partials (m, s) or (max, index);
                              // VAT loss: [B][k][P][5] (pair partials)
    uint64_t* segw;           // [B][rows_per_seq][S][2] tagged segment partials (not for the VAT loss)
    uint64_t* resid;          // [B][P + 3] tagged residual masses, then the decision word (r + 2), the
                              // progress word (window mode: positions accepted while none is rejected)
                              // and the history word (window mode: r + 2 of the last call, any tag)

    TaskGrid grid;            // role of every block of the launch
};

// Residency: the lags between a sequence's worker blocks and its finisher
// block are about one residency of blocks, the device's compute units times
// the blocks of k_verify each holds (verify_blocks_per_cu, from the
// occupancy calculator; kMinBlocksPerCu is what the kernel's launch bounds
// guarantee).  kDefaultComputeUnits stands in only if the device query fails.
constexpr int kMinBlocksPerCu = 5;
constexpr int kDefaultComputeUnits = 256;

// Blocks of k_verify<EB, VEC, path> one compute unit holds at once (0 on failure).
int verify_blocks_per_cu(int elem_bytes, bool vec, int path);

// Small one-hot and greedy calls whose rows need not all be read (see
// Plan::window): positions whose rows are always read at once, and how fast
// the read-ahead grows with the accepted prefix.
constexpr int kRowWindow = 1;
constexpr int kWindowGrowth = 2;

// Chunks each worker wavefront streams, one after the other.  Two per wave
// for large calls: block dispatch (on the order of 150-200 blocks per
// microsecond) would otherwise bound the grid; one per wave for small calls
// (at most kSmallCallWaves chunks per resident block), where the drain of
// long-lived blocks at the end dominates.  Residual workers read two rows
// per chunk and take one chunk pair per wave.
constexpr int kChunksPerWave = 2;
constexpr int kChunksPerWaveSmall = 1;
constexpr int64_t kSmallCallWaves = 4 * kWavesPerBlock;
constexpr int kChunksPerWaveResid = 1;

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
    size_t chunkw, segw, resid, total;
};

// chunk_words / seg_words: tagged words of chunk and segment partials over
// the whole call.
WorkspaceLayout workspace_layout(int64_t chunk_words, int64_t seg_words, int64_t batch, int64_t chunks);

// Words per chunk pair of the VAT loss: (m_t, s_t, m_d, s_d, x).
constexpr int kPairWords = 5;

// Enqueue the whole path on `stream`.  Returns hipSuccess or the first error.
hipError_t launch_path(const Plan& plan, hipStream_t stream, hipEvent_t probe_start, hipEvent_t probe_stop);

// Size of the built-in workspace of sv_verify_noalloc (SV_NOALLOC_SCRATCH_BYTES).
constexpr size_t kNoAllocScratchBytes = size_t{8} << 20;

// Device address of the current device's built-in workspace, set up (address
// looked up, zero-filled by a kernel on `stream`) on the first call per
// device.
hipError_t noalloc_scratch(hipStream_t stream, void** ptr);

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
    int32_t vec;              // 16-byte rows and pointers
    float c2;                 // log2(e) / T
    float inv_t;              // 1 / T
    float hard_weight;
};

hipError_t launch_vat_grad(const GradPlan& g, hipStream_t stream, hipEvent_t probe_start, hipEvent_t probe_stop);

// Speed-of-light references (sv_sol.hip): a plain read of nvec 16-byte
// vectors, and a read of two arrays of nvec 16-byte vectors with one fp32
// array of the same element count written.
hipError_t launch_sol_read(const void* data, int64_t nvec, uint32_t* sink, hipStream_t stream);
hipError_t launch_sol_read_write(const void* a, const void* b, float* out, int64_t nvec, int elem_bytes,
                                 hipStream_t stream);

}  // namespace sv
