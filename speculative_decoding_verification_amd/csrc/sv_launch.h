// Internal interface between the C-ABI layer (sv_api.cpp) and the gfx950
// kernels (sv_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>

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

struct SeqState {
    int32_t r;     // first rejection (k if none), -1 invalid
    int32_t mode;  // SampleMode
    int32_t x_r;   // draft token at r (one-hot exclusion)
    int32_t pad;
};

// Everything the kernels of one call need.  Row numbering: target rows
// 0 .. rows_t-1 (sequence b, position i -> b*target_rows_per_seq + i), then
// draft rows rows_t .. rows_t+rows_d-1 (b, i -> rows_t + b*k + i).
struct Plan {
    int32_t batch;            // B (verify) or N (VAT)
    int32_t k;
    int32_t vocab;
    int32_t elem_bytes;       // 4 fp32, 2 bf16
    int32_t target_rows_per_seq;  // k+1 (verify) or k (VAT)
    int32_t chunks;           // P = ceil(V / chunk)
    int32_t chunk;            // elements per chunk
    int64_t rows_t;
    int64_t rows_d;           // 0 for one-hot drafts and T == 0
    bool vec;                 // 16-byte loads allowed (aligned rows)
    bool greedy;              // T == 0
    bool onehot;
    bool vat;
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

    // workspace regions
    float2* partials;         // [rows][P]
    float2* row_mz;           // [rows]
    SeqState* seq;            // [B]
    float* resid;             // [B][P]
};

struct WorkspaceLayout {
    size_t partials, row_mz, seq, resid, total;
};

WorkspaceLayout workspace_layout(int64_t rows, int64_t batch, int64_t chunks);

// Enqueue the whole path on `stream`.  Returns hipSuccess or the first error.
hipError_t launch_path(const Plan& plan, hipStream_t stream, hipEvent_t probe_start, hipEvent_t probe_stop);

}  // namespace sv
