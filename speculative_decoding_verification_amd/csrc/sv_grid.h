// Task grid of the verification kernel: which role each block of the single
// launch plays, and for which sequence.
//
// The grid is a sequence of groups.  Phase A group g holds, in this order:
//   decision workers of sequence g           (w_dec blocks, if g < B)
//   the decision finisher of g - lag_a       (1 block, if that sequence exists)
//   residual workers of g - lag_a - lag_r    (w_res blocks, draft logits at T > 0)
//   the residual finisher of g - lag_a - lag_r - lag_f   (1 block)
// and phase B group h (verification only):
//   bonus workers of sequence h              (w_bonus blocks, if h < B)
//   the bonus finisher of h - lag_b          (1 block)
// A role only waits on roles of the same sequence placed before it, so with
// blocks dispatched in index order every wait ends; the one exception is a
// grid of about one residency whose decision finishers are all placed first
// (fin_first): they wait on workers dispatched after them, which always find
// a slot since the finishers hold at most an eighth of them.  The lags (in groups)
// place a finisher about one residency of blocks behind the blocks it waits
// on, so finishers run while later sequences stream.
//
// Group composition is constant between the breakpoints 0, B, lag_a, ...,
// so the grid is stored as a few segments of equal groups and a block's role
// is found with one scan over the segments and one division: no search, and
// only values that arrive as kernel arguments.
//
// This header is plain C++ (no HIP types): the host builds the segments, the
// kernels decode with the same function, and host tests can check the
// decoding of every block of a grid.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define SV_HOST_DEVICE __host__ __device__
#else
#define SV_HOST_DEVICE
#endif

namespace sv {

enum RoleKind : int32_t {
    kDecWorker = 0,     // one chunk per wavefront of the decision rows (target 0..k-1, draft 0..k-1)
    kDecFinisher = 1,   // per sequence: (m, Z), p(x), q(x), accept test, first rejection
    kResWorker = 2,     // residual mass of chunks of the rejected row pair
    kResFinisher = 3,   // per sequence: the residual draw
    kBonusWorker = 4,   // chunks of the bonus row (target position k)
    kBonusFinisher = 5  // per sequence: the bonus row's statistics and draw
};

enum RoleBits : int32_t {
    kBitDecWorker = 1 << kDecWorker,
    kBitDecFinisher = 1 << kDecFinisher,
    kBitResWorker = 1 << kResWorker,
    kBitResFinisher = 1 << kResFinisher,
    kBitBonusWorker = 1 << kBonusWorker,
    kBitBonusFinisher = 1 << kBonusFinisher
};

struct Role {
    int32_t kind;
    int32_t seq;
    int32_t index;  // worker index within the sequence
};

constexpr int kMaxSegments = 13;  // the finishers placed first, phase A at most 8, phase B at most 4

// A run of groups with the same roles.
struct Segment {
    int32_t first_block;   // grid index of the run's first block
    int32_t first_group;   // g (phase A) or h (phase B) of the run's first group
    int32_t group_blocks;  // blocks per group
    int32_t roles;         // RoleBits of every group in the run
    float inv_group_blocks;
};

struct TaskGrid {
    int32_t batch;
    int32_t w_dec, w_res, w_bonus;     // worker blocks per sequence of each kind
    int32_t lag_a, lag_r, lag_f, lag_b;  // in groups
    int32_t n_segments;
    int32_t total_blocks;
    int32_t fin_first;  // 1: the B decision finishers are blocks 0 .. B-1, before every worker
    Segment seg[kMaxSegments];
};

// q = x / d for 0 <= x < 2^31, d >= 1, from a rounded reciprocal and exact
// integer corrections.
SV_HOST_DEVICE inline int32_t grid_div(int32_t x, int32_t d, float inv_d) {
    int32_t q = static_cast<int32_t>(static_cast<float>(x) * inv_d);
    while (q > 0 && static_cast<int64_t>(q) * d > x) --q;
    while (static_cast<int64_t>(q + 1) * d <= x) ++q;
    return q;
}

SV_HOST_DEVICE inline Role decode_role(const TaskGrid& tg, int32_t blk) {
    // The segment holding blk: the last one that starts at or before it.
    int32_t fb = tg.seg[0].first_block, fg = tg.seg[0].first_group, gb = tg.seg[0].group_blocks;
    int32_t roles = tg.seg[0].roles;
    float inv = tg.seg[0].inv_group_blocks;
#pragma unroll
    for (int s = 1; s < kMaxSegments; ++s) {
        if (s < tg.n_segments && blk >= tg.seg[s].first_block) {
            fb = tg.seg[s].first_block;
            fg = tg.seg[s].first_group;
            gb = tg.seg[s].group_blocks;
            roles = tg.seg[s].roles;
            inv = tg.seg[s].inv_group_blocks;
        }
    }
    const int32_t x = blk - fb;
    const int32_t q = grid_div(x, gb, inv);
    int32_t o = x - q * gb;
    const int32_t g = fg + q;
    Role r{kResFinisher, 0, 0};
    if (roles & kBitDecWorker) {
        if (o < tg.w_dec) return Role{kDecWorker, g, o};
        o -= tg.w_dec;
    }
    if (roles & kBitDecFinisher) {
        if (o == 0) return Role{kDecFinisher, g - tg.lag_a, 0};
        o -= 1;
    }
    if (roles & kBitResWorker) {
        if (o < tg.w_res) return Role{kResWorker, g - tg.lag_a - tg.lag_r, o};
        o -= tg.w_res;
    }
    if (roles & kBitResFinisher) return Role{kResFinisher, g - tg.lag_a - tg.lag_r - tg.lag_f, 0};
    if (roles & kBitBonusWorker) {
        if (o < tg.w_bonus) return Role{kBonusWorker, g, o};
        o -= tg.w_bonus;
    }
    if (roles & kBitBonusFinisher) return Role{kBonusFinisher, g - tg.lag_b, 0};
    return r;  // not reached for a block inside the grid
}

// Host: the grid of one call.  dec_items = decision-row chunks per sequence,
// chunks = chunks per row; a worker block covers `per_block_dec` chunks of
// decision rows, `per_block_bonus` chunks of the bonus row and
// `per_block_res` chunk pairs of the residual; the lags are derived from the
// number of blocks the device keeps resident.  Returns false if the grid
// does not fit the limits.  With allow_fin_first, a grid whose decision
// workers all come before its first finisher (one residency) places the
// decision finishers first when they take at most an eighth of the resident
// blocks.
bool plan_task_grid(int32_t batch, int64_t dec_items, int64_t chunks, bool has_resid, bool has_bonus,
                    int64_t per_block_dec, int64_t per_block_bonus, int64_t per_block_res, int64_t resident_blocks,
                    TaskGrid* tg, bool allow_fin_first = false);

// Host: the segments of a grid.  Returns false if the grid does not fit the
// limits (more than 2^31 - 1 blocks, or lags outside [0, B]).
bool build_task_grid(int32_t batch, int32_t w_dec, int32_t w_res, int32_t w_bonus, bool has_resid, bool has_bonus,
                     int32_t lag_a, int32_t lag_r, int32_t lag_f, int32_t lag_b, TaskGrid* tg, bool fin_first = false);

}  // namespace sv
