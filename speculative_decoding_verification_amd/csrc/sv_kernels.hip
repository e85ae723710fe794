// gfx950 (CDNA4) kernels of libspecverify.
//
// What is computed (NgramRL essay "AI 开始抄自己的作业", section "投机解码：
// 让草稿先跑，考官殿后": acceptance with probability min(1, p/q), cut at the
// first rejection, the target's own token drawn from the residual or, after
// full acceptance, from its last distribution; VAT write-up "让AI草稿模型学会
// “照镜子”", sections "VAT怎么把“验收规则”塞进训练里" and "第二件事，改权重分配
// 的锚点": the same rule on training blocks, labels and first-rejection-
// anchored weights).
//
// One call is one launch of k_verify<EB, VEC, MODE> (one specialisation per
// path: sampling with draft logits, one-hot drafts, greedy, VAT labels, VAT
// greedy, VAT loss), a grid of 256-thread blocks, each of which decodes its
// role from its block index (a "task grid").  The roles:
//  decision worker   one segment of one row per block: each wavefront streams
//                    nc 8 KiB chunks of the row (non-temporal 16-byte
//                    coalesced loads), the chunk's max and sum of
//                    exp2((l - m) * log2(e)/T) (at T == 0: max and lowest
//                    index), DPP wave reductions; one tagged word pair per
//                    chunk, then one merged pair per segment.  Workers never
//                    wait, except in small one-hot and greedy calls (window
//                    mode), where the rows of later positions are read only
//                    as the accepted prefix comes near them.
//  decision finisher per sequence: `decide` (shared by every role that needs
//                    the first rejection r) combines the segment partials
//                    into (m, Z) per row as the rows complete, gathers
//                    p(x_i), q(x_i), tests u*q < p position by position and
//                    stops at the first rejection; then the accepted prefix
//                    or VAT labels and weights, and the one-hot residual draw
//                    (p_r without x_r) inline.
//  residual worker   draft logits at T > 0 only: decides, then the residual
//                    mass max(0, p_r - q_r) of one chunk pair per wavefront.
//  residual finisher decides, then the residual draw (chunk prefix scan, then
//                    one chunk).
//  bonus worker      streams the target row at position k (the bonus row)
//                    when it can be needed.
//  bonus finisher    decides, the bonus row's statistics and, after full
//                    acceptance, the draw.
// Blocks run in index order within the grid closely enough that each role only
// ever waits on blocks with smaller indices (small grids place their decision
// finishers first, where they take few slots), and finishers are placed about
// one residency behind the workers they wait on, so that they overlap the
// streaming of later sequences instead of stalling it.  Every wait is bounded
// (about a second); a sequence whose wait runs out reports -2.  Hand-off words
// carry a per-call tag in their upper half, so the workspace needs no clearing
// between calls and no fence is ever issued.
//
// Draws: block prefix scan over the chunk masses finds the chunk holding the
// draw, then an LDS block scan of that one chunk finds the token.  No
// floating-point atomics and fixed reduction orders: bitwise reproducible.
//
// Also here: k_vat_grad, the gradient of the VAT loss with respect to the
// draft logits (one streaming pass over both rows, from the row statistics
// the loss pass wrote), and k_accept_hist, the histogram of accepted lengths.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kMaxDraft = 64;
constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ const char* row_base(const void* p, int64_t row, int64_t V, int eb) {
    return static_cast<const char*>(p) + (row * V) * eb;
}

// ------------------------------------------------------------------ elements

template <int EB>
struct Elem;

template <>
struct Elem<4> {
    static constexpr int kPerVec = 4;
    static constexpr uint32_t kNegInfWord = 0xff800000u;
    __device__ static float at(const char* row, int64_t i) {
        return reinterpret_cast<const float*>(row)[i];
    }
    __device__ static void decode(const uint4& v, float* o) {
        o[0] = __uint_as_float(v.x);
        o[1] = __uint_as_float(v.y);
        o[2] = __uint_as_float(v.z);
        o[3] = __uint_as_float(v.w);
    }
};

template <>
struct Elem<2> {
    static constexpr int kPerVec = 8;
    static constexpr uint32_t kNegInfWord = 0xff80ff80u;
    __device__ static float at(const char* row, int64_t i) {
        return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(row)[i]) << 16);
    }
    // A 32-bit word holds logit 2j in its low half and 2j+1 in its high half;
    // a bf16 is the high half of the fp32 with the same value.
    __device__ static void decode(const uint4& v, float* o) {
        o[0] = __uint_as_float(v.x << 16);
        o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16);
        o[3] = __uint_as_float(v.y & 0xffff0000u);
        o[4] = __uint_as_float(v.z << 16);
        o[5] = __uint_as_float(v.z & 0xffff0000u);
        o[6] = __uint_as_float(v.w << 16);
        o[7] = __uint_as_float(v.w & 0xffff0000u);
    }
};

template <int EB>
struct Chunk {
    static constexpr int kPerLane = kVecPerLane * Elem<EB>::kPerVec;  // logits per lane
    static constexpr int kElems = kWave * kPerLane;                   // logits per chunk
    static constexpr int kPerThread = kElems / kBlock;                // chunk scan: per thread
};

// Streaming loads of logits are non-temporal: every logit is read once, and
// keeping the stream out of the caches' normal replacement measurably raises
// the read rate on gfx950 (about 6.2 -> 7.0 TB/s for a plain 428 MB read).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Loads chunk [start, start+len) of one row into the lanes of a wavefront.
// Vector layout: lane l holds vectors l, l+64, ..., l+448 (coalesced 1 KiB per
// instruction).  Scalar layout (unaligned rows): lane l holds logits l, l+64, ...
// Missing logits (ragged last chunk) read as -inf.
template <int EB, bool VEC>
__device__ __forceinline__ void load_chunk(const char* row, int64_t start, int len, int lane,
                                           float (&v)[Chunk<EB>::kPerLane]) {
    constexpr int PV = Elem<EB>::kPerVec;
    if constexpr (VEC) {
        const uint4* p = reinterpret_cast<const uint4*>(row + start * EB);
        uint4 raw[kVecPerLane];
        if (len == Chunk<EB>::kElems) {
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) raw[j] = load_stream(p + j * kWave + lane);
        } else {
            const int nvec = len / PV;  // rows are whole vectors on this path
            const uint32_t ni = Elem<EB>::kNegInfWord;
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                const int idx = j * kWave + lane;
                raw[j] = idx < nvec ? load_stream(p + idx) : make_uint4(ni, ni, ni, ni);
            }
        }
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) Elem<EB>::decode(raw[j], &v[j * PV]);
    } else {
#pragma unroll
        for (int e = 0; e < Chunk<EB>::kPerLane; ++e) {
            const int idx = e * kWave + lane;
            v[e] = idx < len ? Elem<EB>::at(row, start + idx) : neg_inf();
        }
    }
}

// Position inside the chunk of v[e] as laid out by load_chunk.
template <int EB, bool VEC>
__device__ __forceinline__ int chunk_index(int e, int lane) {
    constexpr int PV = Elem<EB>::kPerVec;
    if constexpr (VEC) {
        return ((e / PV) * kWave + lane) * PV + (e % PV);
    } else {
        return e * kWave + lane;
    }
}

// ------------------------------------------------------------------ reductions
//
// Cross-lane work uses DPP (data-parallel primitives: a VALU operand read
// from another lane of the same 16-lane row, or broadcast across rows) and
// v_readlane, never the LDS permute path, so a wave reduction is a dozen
// dependent VALU instructions.

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf, bool BOUND_ZERO = true>
__device__ __forceinline__ float dpp(float old, float src) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, ROW_MASK, BANK_MASK, BOUND_ZERO));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int old, int src) {
    return __builtin_amdgcn_update_dpp(old, src, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ float readlane(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

constexpr int kDppQuadSwap1 = 0xb1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4e;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;
constexpr int kDppWaveShr1 = 0x138;

// Maximum over the wave, on every lane (max is exact in any order).
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<kDppQuadSwap1>(v, v));
    v = fmaxf(v, dpp<kDppQuadSwap2>(v, v));
    v = fmaxf(v, dpp<kDppRowRor4>(v, v));
    v = fmaxf(v, dpp<kDppRowRor8>(v, v));
    return fmaxf(fmaxf(readlane(v, 0), readlane(v, 16)), fmaxf(readlane(v, 32), readlane(v, 48)));
}

// Sum over the wave, the same bits on every lane: row sums within each
// 16-lane row, then the four row sums read from lanes 0, 16, 32, 48 and
// added in that order.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<kDppQuadSwap1>(v, v);
    v += dpp<kDppQuadSwap2>(v, v);
    v += dpp<kDppRowRor4>(v, v);
    v += dpp<kDppRowRor8>(v, v);
    return ((readlane(v, 0) + readlane(v, 16)) + readlane(v, 32)) + readlane(v, 48);
}

// Integer maximum / minimum over the wave, on every lane.
__device__ __forceinline__ int wave_max_i(int v) {
    v = max(v, dpp_i<kDppQuadSwap1>(v, v));
    v = max(v, dpp_i<kDppQuadSwap2>(v, v));
    v = max(v, dpp_i<kDppRowRor4>(v, v));
    v = max(v, dpp_i<kDppRowRor8>(v, v));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

__device__ __forceinline__ int wave_min_i(int v) {
    v = min(v, dpp_i<kDppQuadSwap1>(v, v));
    v = min(v, dpp_i<kDppQuadSwap2>(v, v));
    v = min(v, dpp_i<kDppRowRor4>(v, v));
    v = min(v, dpp_i<kDppRowRor8>(v, v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Block-wide "any": a ballot per wave, one LDS flag per wave, a barrier.
// (flags: kWavesPerBlock ints of LDS.)  Whole block.
__device__ __forceinline__ bool block_any(bool pred, int* flags) {
    const bool w = __ballot(pred) != 0ull;
    if ((threadIdx.x & (kWave - 1)) == 0) flags[threadIdx.x / kWave] = w;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int q = 0; q < kWavesPerBlock; ++q) any |= flags[q];
    __syncthreads();
    return any != 0;
}

// Larger value wins; equal values: lower index wins.  Result on every lane.
__device__ __forceinline__ void argmax_step(float& best, int& idx, float ob, int oi) {
    if (ob > best || (ob == best && oi < idx)) {
        best = ob;
        idx = oi;
    }
}

__device__ __forceinline__ void wave_argmax(float& best, int& idx) {
    argmax_step(best, idx, dpp<kDppQuadSwap1>(best, best), dpp_i<kDppQuadSwap1>(idx, idx));
    argmax_step(best, idx, dpp<kDppQuadSwap2>(best, best), dpp_i<kDppQuadSwap2>(idx, idx));
    argmax_step(best, idx, dpp<kDppRowRor4>(best, best), dpp_i<kDppRowRor4>(idx, idx));
    argmax_step(best, idx, dpp<kDppRowRor8>(best, best), dpp_i<kDppRowRor8>(idx, idx));
    float b = readlane(best, 0);
    int i = __builtin_amdgcn_readlane(idx, 0);
    argmax_step(b, i, readlane(best, 16), __builtin_amdgcn_readlane(idx, 16));
    argmax_step(b, i, readlane(best, 32), __builtin_amdgcn_readlane(idx, 32));
    argmax_step(b, i, readlane(best, 48), __builtin_amdgcn_readlane(idx, 48));
    best = b;
    idx = i;
}

// Scale of a row with max m: returns mc = m*c2 rounded, and sets corr so that
// exp2(fma(l, c2, -mc)) * corr == exp2((l - m) * c2) up to one rounding of the
// exponent (corr = exp2(-(m*c2 - mc)), the rounding error of mc being exact).
__device__ __forceinline__ float row_scale(float m, float c2, float& corr) {
    const float mc = m * c2;
    corr = exp2_hw(-fmaf(m, c2, -mc));
    return mc;
}

// Merges (m, s) pairs where s = sum exp2((l - m) * c2) over disjoint sets.
__device__ __forceinline__ void wave_merge_ms(float& m, float& s, float c2) {
    const float M = wave_max(m);
    const float scaled = (m == neg_inf()) ? 0.f : s * exp2_hw((m - M) * c2);
    s = wave_sum(scaled);
    m = M;
}

// Inclusive prefix sum over the wave: Hillis-Steele within 16-lane rows
// (shifts 1, 2, 4, 8), then row 0's total into row 1 and row 2's into row 3
// (row_bcast:15), then rows 0-1's total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ float wave_incl_scan(float x) {
    x += dpp<kDppRowShr1>(0.f, x);
    x += dpp<kDppRowShr2>(0.f, x);
    x += dpp<kDppRowShr4>(0.f, x);
    x += dpp<kDppRowShr8>(0.f, x);
    x += dpp<kDppRowBcast15, 0xa, 0xf, false>(0.f, x);
    x += dpp<kDppRowBcast31, 0xc, 0xf, false>(0.f, x);
    return x;
}

// Inclusive scan over a workgroup of kBlock threads; returns the inclusive
// value, writes the exclusive one (the inclusive value of the previous
// thread, bit for bit) and the block total.  Fixed order.
__device__ __forceinline__ float block_scan(float v, float& excl, float& total, float* s_wt) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const float incl = wave_incl_scan(v);
    const float wexcl = dpp<kDppWaveShr1>(0.f, incl);  // lane 0 reads 0
    if (lane == kWave - 1) s_wt[wave] = incl;
    __syncthreads();
    float prefix = 0.f;
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
        if (w < wave) prefix += s_wt[w];
        tot += s_wt[w];
    }
    __syncthreads();
    excl = prefix + wexcl;
    total = tot;
    return prefix + incl;
}

__device__ __forceinline__ float block_sum(float v, float* s_wt) {
    float excl, total;
    block_scan(v, excl, total, s_wt);
    return total;
}

// ------------------------------------------------------------------ layout

template <int EB>
__device__ __forceinline__ const char* row_of(const Plan& pl, int64_t grow) {
    return grow < pl.rows_t ? row_base(pl.target, grow, pl.vocab, EB)
                            : row_base(pl.draft, grow - pl.rows_t, pl.vocab, EB);
}

// ------------------------------------------------------------------ chunk partials

// (m, s) of one chunk: m = max raw logit, s = sum of exp2((l - m) * c2) with
// c2 = log2(e)/T, i.e. the sum of exp(l/T - m/T).
template <int EB, bool VEC>
__device__ __forceinline__ float2 chunk_stats(const char* rp, int64_t start, int len, int lane, float c2) {
    float v[Chunk<EB>::kPerLane];
    load_chunk<EB, VEC>(rp, start, len, lane, v);
    float m = v[0];
#pragma unroll
    for (int e = 1; e < Chunk<EB>::kPerLane; ++e) m = fmaxf(m, v[e]);
    m = wave_max(m);
    float s = 0.f;
    if (m != neg_inf()) {
        // fma(v, c2, -mc) = (v - m) * c2 + dlt, rounded once, where
        // dlt = m*c2 - mc is the (exactly representable) rounding error of
        // mc: a factor exp2(dlt) common to the whole chunk, removed below.
        const float mc = m * c2;
        const float dlt = fmaf(m, c2, -mc);
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int e = 0; e < Chunk<EB>::kPerLane; e += 4) {
            a0 += exp2_hw(fmaf(v[e + 0], c2, -mc));
            a1 += exp2_hw(fmaf(v[e + 1], c2, -mc));
            a2 += exp2_hw(fmaf(v[e + 2], c2, -mc));
            a3 += exp2_hw(fmaf(v[e + 3], c2, -mc));
        }
        s = ((a0 + a1) + (a2 + a3)) * exp2_hw(-dlt);
    }
    return make_float2(m, wave_sum(s));
}

// (max, lowest index of the max within the row) of one chunk, T == 0.
template <int EB, bool VEC>
__device__ __forceinline__ float2 chunk_argmax(const char* rp, int64_t start, int len, int lane) {
    float v[Chunk<EB>::kPerLane];
    load_chunk<EB, VEC>(rp, start, len, lane, v);
    // Ascending index order within the lane, strict '>' keeps the first max.
    float best = v[0];
    int bi = chunk_index<EB, VEC>(0, lane);
#pragma unroll
    for (int e = 1; e < Chunk<EB>::kPerLane; ++e) {
        if (v[e] > best) {
            best = v[e];
            bi = chunk_index<EB, VEC>(e, lane);
        }
    }
    wave_argmax(best, bi);
    return make_float2(best, __int_as_float(static_cast<int>(start) + bi));
}

// ------------------------------------------------------------------ hand-off words

// Worker blocks hand values to a finisher block of the same kernel through
// tagged 64-bit words (see kTagFirst).  Writes are device-scope atomic
// stores: write-through to the device-coherent level (sc1), so nothing is
// left dirty in an XCD's L2 and workers never wait.  The finisher reads with
// device-scope atomic loads and polls until every word carries the call's
// tag; no release/acquire fence (an L2 writeback or invalidate) is needed.
__device__ __forceinline__ void put_word(uint64_t* p, uint32_t data, uint32_t tag) {
    __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | data, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t get_word(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t word_data(uint64_t w) { return static_cast<uint32_t>(w); }

// Chunk partial i of a sequence: words 2i (m or max) and 2i+1 (s or index).
__device__ __forceinline__ void put_partial(uint64_t* seq_words, int i, float2 v, uint32_t tag) {
    put_word(seq_words + 2 * i, __float_as_uint(v.x), tag);
    put_word(seq_words + 2 * i + 1, __float_as_uint(v.y), tag);
}

// A finisher gives up after about a second of polling (the wall clock runs at
// 100 MHz): it cannot happen when blocks are dispatched in grid order, and it
// turns any other case into an error code instead of a hung kernel.  Roles
// that wait on a sequence's decision wait twice as long: its finisher comes
// earlier in the grid, so by then it has either published the decision or
// reported its own timeout (it owns accepted_len; a draw owns only its token).
constexpr uint64_t kPollTimeoutTicks = 1ull << 27;
constexpr uint64_t kDecisionTimeoutTicks = 2 * kPollTimeoutTicks;

// Two-deep polls: each thread reads at most kPollPer of the words.
constexpr int kPollPer = 6;

__device__ __forceinline__ void poll_read(const uint64_t* words, int n, uint64_t (&w)[kPollPer]) {
#pragma unroll
    for (int j = 0; j < kPollPer; ++j) {
        const int i = threadIdx.x + j * kBlock;
        w[j] = i < n ? get_word(words + i) : 0ull;
    }
}

// Whether one of this thread's words lacks the tag; stages the others' data.
__device__ __forceinline__ bool poll_missing(int n, uint32_t tag, uint32_t* stage, const uint64_t (&w)[kPollPer]) {
    bool missing = false;
#pragma unroll
    for (int j = 0; j < kPollPer; ++j) {
        const int i = threadIdx.x + j * kBlock;
        if (i < n) {
            if (static_cast<uint32_t>(w[j] >> 32) != tag) missing = true;
            else if (stage) stage[i] = word_data(w[j]);
        }
    }
    return missing;
}

// Polls the n words at `words` until all carry `tag`; with `stage` (n <=
// kStageWords) their data is left in stage[0..n).  Whole block (flags: the
// block's LDS vote slots).  Returns false on timeout.
//
// With `two_deep` (n <= kPollPer * kBlock) the next read of the words goes
// out before the current one is checked and voted on, so a word is seen about
// half a memory round trip sooner.  That pays when the whole grid is resident
// at once; under a full stream the extra reads cost as much as they save, so
// larger calls read once per round.
__device__ __forceinline__ bool collect(const uint64_t* words, int n, uint32_t tag, uint32_t* stage, int* flags,
                                        bool two_deep, uint64_t timeout = kPollTimeoutTicks) {
    const uint64_t t0 = wall_clock64();
    if (two_deep && n <= kPollPer * kBlock) {
        uint64_t wa[kPollPer], wb[kPollPer];
        poll_read(words, n, wa);
        for (;;) {
            __builtin_amdgcn_s_sleep(4);
            poll_read(words, n, wb);
            if (!block_any(poll_missing(n, tag, stage, wa), flags)) return true;
            if (block_any(wall_clock64() - t0 > timeout, flags)) return false;
            __builtin_amdgcn_s_sleep(4);
            poll_read(words, n, wa);
            if (!block_any(poll_missing(n, tag, stage, wb), flags)) return true;
            if (block_any(wall_clock64() - t0 > timeout, flags)) return false;
        }
    }
    for (;;) {
        bool missing = false;
        for (int i = threadIdx.x; i < n; i += kBlock) {
            const uint64_t w = get_word(words + i);
            if (static_cast<uint32_t>(w >> 32) != tag) missing = true;
            else if (stage) stage[i] = word_data(w);
        }
        if (!block_any(missing, flags)) return true;
        // waves read the clock at slightly different times: decide together
        if (block_any(wall_clock64() - t0 > timeout, flags)) return false;
        __builtin_amdgcn_s_sleep(8);
    }
}

// Chunk partials of a sequence, staged in LDS or read from the words.
struct PartialSrc {
    const uint32_t* stage;
    const uint64_t* words;
    __device__ __forceinline__ float2 get(int i) const {
        if (stage) return make_float2(__uint_as_float(stage[2 * i]), __uint_as_float(stage[2 * i + 1]));
        return make_float2(__uint_as_float(word_data(get_word(words + 2 * i))),
                           __uint_as_float(word_data(get_word(words + 2 * i + 1))));
    }
};

struct TailShared {
    uint32_t stage[kStageWords];   // staged hand-off words
    float2 segp[kWavesPerBlock * kChunksPerWave];  // a segment's chunk partials (decision and bonus workers)
    float2 mz[2 * kMaxDraft + 1];  // (m, Z) or (max, argmax) of the sequence's rows
    float xs[kMaxDraft];           // VAT loss: sum_y p(y) (l_d(y) - m_d) c2, times Z_t
    float wt[kWavesPerBlock];      // block scan scratch
    int vote[kWavesPerBlock];      // block_any scratch
    int wlast[kWavesPerBlock];     // per-wave last positive position (draws)
    int wsel[kWavesPerBlock];      // per-wave selected position (draws)
    float prev_mass;               // running mass before the selected chunk
    int sel;
    int last_pos;
    int r;
    int mode;
    int x_r;
    float l_x;
    int ahead;                     // window mode: last position read without waiting
    int known;                     // window mode: r from the decision word, k while undecided
};

// ------------------------------------------------------------------ sampling

struct ResidW {
    float c2, mt, izt, md, izd;  // mt, md: row max * c2 (rounded); izt, izd: corr / Z
    __device__ __forceinline__ float operator()(float lt, float ld) const {
        // p and q rounded on their own before the difference (no fused
        // multiply-subtract): equal rows give exactly zero residual mass.
#pragma clang fp contract(off)
        const float p = exp2_hw(fmaf(lt, c2, -mt)) * izt;
        const float q = exp2_hw(fmaf(ld, c2, -md)) * izd;
        return fmaxf(0.f, p - q);
    }
};

__device__ __forceinline__ ResidW make_resid_w(float2 mzt, float2 mzd, float c2) {
    ResidW w;
    float ct, cd;
    w.c2 = c2;
    w.mt = row_scale(mzt.x, c2, ct);
    w.izt = ct / mzt.y;
    w.md = row_scale(mzd.x, c2, cd);
    w.izd = cd / mzd.y;
    return w;
}

// The distribution the token is drawn from, as weights over token ids.
struct DrawRow {
    int mode;                 // kModeBonus (plain target row), kModeOneHot, kModeResidual
    const char* rt;           // target row
    const char* rd;           // draft row (residual only)
    PartialSrc part;          // chunk partials of the target row at part_base + c
    int part_base;
    const uint32_t* rstage;   // residual chunk masses, staged ...
    const uint64_t* rwords;   // ... or as words
    float c2, mt, corr, mrow; // target row: mt = max*c2 rounded, corr (row_scale), mrow = max
    int excl;                 // one-hot: excluded token, else -1
    float lx;                 // one-hot: target logit of the excluded token
    ResidW rw;
};

// Logits [i0, i0 + kPerThread) of a chunk for thread t (i0 = t*kPerThread);
// -inf past the end of the row.
template <int EB, bool VEC>
__device__ __forceinline__ void load_run(const char* row, int64_t cstart, int clen, float (&v)[Chunk<EB>::kPerThread]) {
    constexpr int PT = Chunk<EB>::kPerThread;
    constexpr int PV = Elem<EB>::kPerVec;
    const int i0 = threadIdx.x * PT;
    if constexpr (VEC) {
        if (i0 + PT <= clen) {  // 32 contiguous, 16-byte aligned bytes
            const uint4* p = reinterpret_cast<const uint4*>(row + (cstart + i0) * EB);
            const uint4 a = p[0];
            const uint4 b = p[1];
            Elem<EB>::decode(a, &v[0]);
            Elem<EB>::decode(b, &v[PV]);
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < PT; ++e) v[e] = i0 + e < clen ? Elem<EB>::at(row, cstart + i0 + e) : neg_inf();
}

// Weights in the distribution of `d` of a thread's run of logits, from the
// target (lt) and, for residuals, draft (ld) logits of that run.
template <int EB>
__device__ __forceinline__ void run_weights(const DrawRow& d, int64_t cstart, const float (&lt)[Chunk<EB>::kPerThread],
                                            const float (&ld)[Chunk<EB>::kPerThread],
                                            float (&w)[Chunk<EB>::kPerThread]) {
    constexpr int PT = Chunk<EB>::kPerThread;
    if (d.mode == kModeResidual) {
#pragma unroll
        for (int e = 0; e < PT; ++e) w[e] = d.rw(lt[e], ld[e]);
    } else {
        const int64_t i0 = cstart + threadIdx.x * PT;
#pragma unroll
        for (int e = 0; e < PT; ++e)
            w[e] = (i0 + e == d.excl) ? 0.f : exp2_hw(fmaf(lt[e], d.c2, -d.mt)) * d.corr;
    }
}

// Loads the run of chunk `c` this thread needs for the weights of `d`.
template <int EB, bool VEC>
__device__ __forceinline__ void load_runs(const DrawRow& d, int c, int64_t V, float (&lt)[Chunk<EB>::kPerThread],
                                          float (&ld)[Chunk<EB>::kPerThread]) {
    constexpr int CH = Chunk<EB>::kElems;
    const int64_t cstart = static_cast<int64_t>(c) * CH;
    const int clen = static_cast<int>(min(static_cast<int64_t>(CH), V - cstart));
    load_run<EB, VEC>(d.rt, cstart, clen, lt);
    if (d.mode == kModeResidual) load_run<EB, VEC>(d.rd, cstart, clen, ld);
}

// Mass of chunk c in the units of the weights: residual masses as computed,
// plain target rows from the chunk partials (relative to the row max), with
// x_r's chunk recomputed without x_r for one-hot drafts.
__device__ __forceinline__ float chunk_mass(const DrawRow& d, int c, int cx, float mass_cx) {
    if (d.mode == kModeResidual)
        return __uint_as_float(d.rstage ? d.rstage[c] : word_data(get_word(d.rwords + c)));
    if (c == cx) return mass_cx;
    const float2 pc = d.part.get(d.part_base + c);
    return pc.x == neg_inf() ? 0.f : pc.y * exp2_hw((pc.x - d.mrow) * d.c2);
}

// The chunk a draw falls in: `cs`, with the threshold `th` left inside it
// (open_end: rounding left no chunk above the threshold, take the last
// positive weight of chunk cs).
struct DrawPick {
    int cs;
    float th;
    bool open_end;
    int cx;         // one-hot: chunk of the excluded token, else -1
    float mass_cx;  // one-hot: its mass without that token
};

// Draw rule: the smallest id y whose running weight exceeds u times the
// total weight, in ascending id order.  First step: the chunk, from a block
// prefix scan over the chunk masses.  Whole block.
template <int EB, bool VEC>
__device__ __forceinline__ DrawPick draw_select(const DrawRow& d, float u, int P, int64_t V, TailShared& sh) {
    constexpr int CH = Chunk<EB>::kElems;
    constexpr int PT = Chunk<EB>::kPerThread;
    const int tid = threadIdx.x;
    DrawPick pk;
    pk.cx = -1;
    pk.mass_cx = 0.f;
    if (d.mode == kModeOneHot) {
        pk.cx = d.excl / CH;
        float lt[PT], ld[PT], w[PT];
        load_runs<EB, VEC>(d, pk.cx, V, lt, ld);
        run_weights<EB>(d, static_cast<int64_t>(pk.cx) * CH, lt, ld, w);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < PT; ++e) sum += w[e];
        pk.mass_cx = block_sum(sum, sh.wt);
    }
    // Pass 1: total mass, as the carry of the same tiled scan pass 2 runs.
    float carry = 0.f;
    for (int base = 0; base < P; base += kBlock) {
        const int c = base + tid;
        const float v = c < P ? chunk_mass(d, c, pk.cx, pk.mass_cx) : 0.f;
        float excl, total;
        block_scan(v, excl, total, sh.wt);
        carry = carry + total;
    }
    const float theta = u * carry;
    // Pass 2: the chunk whose running mass first exceeds theta.
    if (tid == 0) {
        sh.sel = INT_MAX;
        sh.last_pos = -1;
    }
    __syncthreads();
    carry = 0.f;
    for (int base = 0; base < P; base += kBlock) {
        const int c = base + tid;
        const float v = c < P ? chunk_mass(d, c, pk.cx, pk.mass_cx) : 0.f;
        float excl, total;
        const float incl = block_scan(v, excl, total, sh.wt);
        if (c < P) {
            const float C = carry + incl;
            const float prev = carry + excl;
            if (C > theta && prev <= theta) {
                sh.sel = c;  // unique: the running mass is non-decreasing
                sh.prev_mass = prev;
            }
        }
        const int wl = wave_max_i(c < P && v > 0.f ? c : -1);
        if ((tid & (kWave - 1)) == 0 && wl >= 0) atomicMax(&sh.last_pos, wl);
        carry = carry + total;
        __syncthreads();
        if (sh.sel != INT_MAX) break;
    }
    pk.open_end = sh.sel == INT_MAX;
    if (pk.open_end) {
        pk.cs = sh.last_pos >= 0 ? sh.last_pos : P - 1;
        pk.th = 0.f;
    } else {
        pk.cs = sh.sel;
        pk.th = theta - sh.prev_mass;
    }
    __syncthreads();
    return pk;
}

// Chunk selection when P <= 64 (lane c holds the mass of chunk c, 0 beyond
// P), done by one wave with a DPP prefix scan and ballots: no block barrier,
// so every wave can compute it redundantly.
__device__ __forceinline__ DrawPick wave_pick(float mass, float u, int P) {
    const int lane = threadIdx.x & (kWave - 1);
    const float incl = wave_incl_scan(mass);
    const float excl = dpp<kDppWaveShr1>(0.f, incl);  // lane c: running mass before chunk c
    const float theta = u * readlane(incl, kWave - 1);
    const uint64_t hit = __ballot(lane < P && incl > theta && excl <= theta);
    DrawPick pk;
    pk.cx = -1;
    pk.mass_cx = 0.f;
    if (hit) {
        pk.cs = __builtin_ctzll(hit);  // unique: the running mass is non-decreasing
        pk.th = theta - readlane(excl, pk.cs);
        pk.open_end = false;
    } else {
        const uint64_t pos = __ballot(lane < P && mass > 0.f);
        pk.cs = pos ? 63 - __builtin_clzll(pos) : P - 1;
        pk.th = 0.f;
        pk.open_end = true;
    }
    return pk;
}

// Second step: the token inside chunk pk.cs, from this thread's weights of
// its run of that chunk (block scan: DPP within waves, LDS across them).
// Whole block; returns the token on every thread.
template <int EB>
__device__ __forceinline__ int draw_scan(const DrawPick& pk, const float (&w)[Chunk<EB>::kPerThread], TailShared& sh) {
    constexpr int CH = Chunk<EB>::kElems;
    constexpr int PT = Chunk<EB>::kPerThread;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    float my_sum = 0.f;
    int my_last = -1;
#pragma unroll
    for (int e = 0; e < PT; ++e) {
        my_sum += w[e];
        if (w[e] > 0.f) my_last = tid * PT + e;
    }
    const float incl = wave_incl_scan(my_sum);
    if (lane == kWave - 1) sh.wt[wave] = incl;
    const int wl = wave_max_i(my_last);
    if (lane == 0) sh.wlast[wave] = wl;
    __syncthreads();
    float prefix = 0.f;
#pragma unroll
    for (int q = 0; q < kWavesPerBlock; ++q)
        if (q < wave) prefix += sh.wt[q];
    const float excl = prefix + dpp<kDppWaveShr1>(0.f, incl);
    int pick = INT_MAX;
    if (!pk.open_end && excl + my_sum > pk.th) {
        float run = excl;
#pragma unroll
        for (int e = 0; e < PT; ++e) {
            run += w[e];
            if (pick == INT_MAX && w[e] > 0.f && run > pk.th) pick = tid * PT + e;
        }
    }
    pick = wave_min_i(pick);
    if (lane == 0) sh.wsel[wave] = pick;
    __syncthreads();
    int sel = INT_MAX, last = -1;
#pragma unroll
    for (int q = 0; q < kWavesPerBlock; ++q) {
        sel = min(sel, sh.wsel[q]);
        last = max(last, sh.wlast[q]);
    }
    const int y = sel != INT_MAX ? sel : (last >= 0 ? last : 0);
    __syncthreads();
    return pk.cs * CH + y;
}

// The chunk of a draw from `d` (whole block).  P <= 64: lane c of every wave
// holds the mass of chunk c and each wave picks redundantly (DPP prefix scan,
// ballot; no barrier).  A one-hot draw needs x_r's chunk without x_r: its
// partial minus x_r's weight when that difference keeps the draw's accuracy
// (the chunk holds at most 8 times the mass left to draw from, so the
// difference's rounding, about 2^-22 of the chunk, stays below 2^-19 of the
// total), else the chunk summed again without x_r.  P > 64: the tiled
// block-level selection.
template <int EB, bool VEC>
__device__ __forceinline__ DrawPick pick_chunk(const DrawRow& d, float u, int P, int64_t V, TailShared& sh) {
    constexpr int CH = Chunk<EB>::kElems;
    constexpr int PT = Chunk<EB>::kPerThread;
    if (P > kWave) return draw_select<EB, VEC>(d, u, P, V, sh);
    const int lane = threadIdx.x & (kWave - 1);
    float mass = lane < P ? chunk_mass(d, lane, -1, 0.f) : 0.f;
    int cx = -1;
    float mass_cx = 0.f;
    if (d.mode == kModeOneHot) {
        cx = d.excl / CH;
        const float part = readlane(mass, cx);
        const float wx = exp2_hw(fmaf(d.lx, d.c2, -d.mt)) * d.corr;
        const float left = wave_sum(mass) - wx;  // the mass the draw is from
        if (part <= 8.f * left) {
            // a remainder within twice its rounding of zero is taken as zero
            mass_cx = part - wx > 0x1p-21f * part ? part - wx : 0.f;
        } else {
            float lt[PT], ld[PT], w[PT];
            load_runs<EB, VEC>(d, cx, V, lt, ld);
            run_weights<EB>(d, static_cast<int64_t>(cx) * CH, lt, ld, w);
            float sum = 0.f;
#pragma unroll
            for (int e = 0; e < PT; ++e) sum += w[e];
            mass_cx = block_sum(sum, sh.wt);
        }
        if (lane == cx) mass = mass_cx;
    }
    DrawPick pk = wave_pick(mass, u, P);
    pk.cx = cx;
    pk.mass_cx = mass_cx;
    return pk;
}

// Draws one token from the weights of `d` with uniform u.  Whole block;
// returns the token on every thread.
template <int EB, bool VEC>
__device__ __forceinline__ int draw_token(const DrawRow& d, float u, int P, int64_t V, TailShared& sh) {
    constexpr int CH = Chunk<EB>::kElems;
    constexpr int PT = Chunk<EB>::kPerThread;
    const DrawPick pk = pick_chunk<EB, VEC>(d, u, P, V, sh);
    float lt[PT], ld[PT], w[PT];
    load_runs<EB, VEC>(d, pk.cs, V, lt, ld);
    run_weights<EB>(d, static_cast<int64_t>(pk.cs) * CH, lt, ld, w);
    return draw_scan<EB>(pk, w, sh);
}

// ------------------------------------------------------------------ specialisations

template <int MODE>
struct PathTraits {
    static constexpr bool greedy = MODE == kPathGreedy || MODE == kPathVatGreedy;
    static constexpr bool vat = MODE == kPathVat || MODE == kPathVatGreedy || MODE == kPathVatLoss;
    static constexpr bool loss = MODE == kPathVatLoss;
    static constexpr bool onehot = MODE == kPathOneHot;
    static constexpr bool resid = MODE == kPathSample;      // residual draws after a rejection
    static constexpr bool bonus = !vat;                      // the bonus row and its draw
    static constexpr int halves = (MODE == kPathSample || MODE == kPathVat) ? 2 : 1;
};

// ------------------------------------------------------------------ rows and words

// Global row (the numbering of row_stats_out) of local row j of sequence b.
__device__ __forceinline__ int64_t global_row(const Plan& pl, int b, int j) {
    if (j < pl.dec_rows) {
        const int i = j / pl.halves;
        if (j == i * pl.halves) return static_cast<int64_t>(b) * pl.target_rows_per_seq + i;
        return pl.rows_t + static_cast<int64_t>(b) * pl.k + i;
    }
    return static_cast<int64_t>(b) * pl.target_rows_per_seq + pl.k;
}

// Chunk words of sequence b: two per chunk of each local row, row-major.
__device__ __forceinline__ uint64_t* chunk_words(const Plan& pl, int b) {
    return pl.chunkw + static_cast<int64_t>(b) * pl.words_per_seq;
}

// Segment words of sequence b: two per segment of each local row, row-major.
__device__ __forceinline__ uint64_t* seg_words(const Plan& pl, int b) {
    return pl.segw + static_cast<int64_t>(b) * pl.seg_words_per_seq;
}

// Residual masses of sequence b (one per chunk), then its decision word
// (r + 2, from the decision finisher, for the workers that wait for it),
// its progress word (window mode: the positions accepted so far while no
// rejection is known) and its history word (window mode: r + 2 of the last
// call that used the workspace, whatever its tag; 0 before any).
__device__ __forceinline__ uint64_t* resid_words(const Plan& pl, int b) {
    return pl.resid + static_cast<int64_t>(b) * (pl.chunks + 3);
}

__device__ __forceinline__ uint64_t* decision_word(const Plan& pl, int b) { return resid_words(pl, b) + pl.chunks; }

__device__ __forceinline__ uint64_t* progress_word(const Plan& pl, int b) {
    return resid_words(pl, b) + pl.chunks + 1;
}

__device__ __forceinline__ uint64_t* history_word(const Plan& pl, int b) {
    return resid_words(pl, b) + pl.chunks + 2;
}

// Window mode: the last position whose row is read without waiting.  Only
// kRowWindow - 1 if the previous call on the workspace rejected the first
// draft token of every sequence (the rows after it were all useless then,
// and acceptance carries over from one decoding step to the next); else k,
// every row and the bonus row.  In the same round of loads (wave 1), what
// sequence b's decision word says: `known` = its r, or k while undecided.
// Whole block.
__device__ __forceinline__ int read_ahead(const Plan& pl, int b, TailShared& sh, int& known) {
    if (threadIdx.x >= kWave && threadIdx.x < 2 * kWave) {
        const int lane = static_cast<int>(threadIdx.x) - kWave;
        const uint64_t d = get_word(decision_word(pl, b));
        bool other = false;
        for (int i = lane; i < pl.batch; i += kWave) other |= word_data(get_word(history_word(pl, i))) != 2u;
        const bool any = __ballot(other) != 0ull;
        if (lane == 0) {
            sh.ahead = any ? pl.k : pl.window - 1;
            sh.known = static_cast<uint32_t>(d >> 32) == pl.tag ? static_cast<int>(word_data(d)) - 2 : pl.k;
        }
    }
    __syncthreads();
    known = sh.known;
    return sh.ahead;
}

// Window mode: whether the row of position pos of sequence b is read.  One
// lane of wave 1 polls the sequence's decision and progress words until the
// decision is known (read if r >= pos: the bonus row after full acceptance)
// or the accepted prefix a has pos < window + kWindowGrowth * a.  Returns 0
// (never used), 1 (read) or 2 (the wait ran out: read anyway).  The wait is
// a quarter of the decision finisher's, so that a finisher whose rows were
// held back still receives them before its own wait runs out.  Whole block.
__device__ __forceinline__ int released(const Plan& pl, int b, int pos, TailShared& sh) {
    if (threadIdx.x == kWave) {
        const uint64_t t0 = wall_clock64();
        int go;
        for (;;) {
            const uint64_t d = get_word(decision_word(pl, b));
            const uint64_t a = get_word(progress_word(pl, b));
            if (static_cast<uint32_t>(d >> 32) == pl.tag) {
                go = static_cast<int>(word_data(d)) - 2 >= pos ? 1 : 0;
                break;
            }
            if (static_cast<uint32_t>(a >> 32) == pl.tag &&
                pos < kWindowGrowth * static_cast<int>(word_data(a)) + pl.window) {
                go = 1;
                break;
            }
            if (wall_clock64() - t0 > kPollTimeoutTicks / 4) {
                go = 2;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        sh.r = go;
    }
    __syncthreads();
    return sh.r;
}

// ------------------------------------------------------------------ workers

// Merges chunk partials (m, s) -- or (max, index) at T == 0 -- in order.
__device__ __forceinline__ float2 merge_partial(float2 a, float2 b, bool greedy, float c2) {
    if (greedy) {
        float best = a.x;
        int idx = __float_as_int(a.y);
        argmax_step(best, idx, b.x, __float_as_int(b.y));
        return make_float2(best, __int_as_float(idx));
    }
    if (b.x == neg_inf()) return a;
    if (a.x == neg_inf()) return b;
    const float m = fmaxf(a.x, b.x);
    return make_float2(m, a.y * exp2_hw((a.x - m) * c2) + b.y * exp2_hw((b.x - m) * c2));
}

// One segment of local row j of sequence b: wavefront w streams chunks
// c0 + w + 4n (n < nc_dec) of the segment, each handed off as two chunk
// words; after one barrier, thread 0 merges the segment's chunk partials in
// chunk order and hands off the segment partial as two segment words.  The
// decision steps poll segment words only (a few per row); the draws and the
// bonus finisher read the chunk words of the one row they use.  With more
// than one chunk per wave, every hand-off store waits for the barrier and
// comes from wave 0 (see below).  Whole block.
template <int EB, bool VEC, int MODE>
__device__ __forceinline__ void stream_segment(const Plan& pl, int b, int j, int s, TailShared& sh) {
    using Tr = PathTraits<MODE>;
    const bool defer = pl.nc_dec > 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int P = pl.chunks;
    const int c0 = s * pl.seg_chunks;
    const int c1 = min(P, c0 + pl.seg_chunks);
    const char* rp = row_of<EB>(pl, global_row(pl, b, j));
    uint64_t* cw = chunk_words(pl, b) + static_cast<int64_t>(j) * P * 2;
#pragma unroll 1
    for (int n = 0; n < pl.nc_dec; ++n) {
        const int c = c0 + wave + n * kWavesPerBlock;
        if (c >= c1) break;
        const int64_t start = static_cast<int64_t>(c) * Chunk<EB>::kElems;
        const int len = static_cast<int>(min(static_cast<int64_t>(Chunk<EB>::kElems), pl.vocab - start));
        const float2 part = Tr::greedy ? chunk_argmax<EB, VEC>(rp, start, len, lane)
                                       : chunk_stats<EB, VEC>(rp, start, len, lane, pl.c2);
        if (lane == 0) {
            // one chunk per wave: its word at once; more: after all of the
            // block's loads (a wave's write-through stores share the memory
            // counter with its loads, so a store between two chunks would
            // make the second chunk's wait cover the store's acknowledgement)
            if (!defer) put_partial(cw, c, part, pl.tag);
            sh.segp[c - c0] = part;
        }
    }
    __syncthreads();
    if (defer && threadIdx.x > 0 && threadIdx.x < c1 - c0)
        put_partial(cw, c0 + static_cast<int>(threadIdx.x), sh.segp[threadIdx.x], pl.tag);
    if (threadIdx.x == 0) {
        if (defer) put_partial(cw, c0, sh.segp[0], pl.tag);
        float2 acc = sh.segp[0];
        for (int q = 1; q < c1 - c0; ++q) acc = merge_partial(acc, sh.segp[q], Tr::greedy, pl.c2);
        put_partial(seg_words(pl, b) + static_cast<int64_t>(j) * pl.segs * 2, s, acc, pl.tag);
    }
}

// Residual mass of chunk [start, start+len) of a target/draft row pair, in
// the wavefront's chunk layout.  The vector path reads half the chunk at a
// time and decodes in registers, keeping the kernel's register budget at the
// streaming pass's.
template <int EB, bool VEC>
__device__ __forceinline__ float chunk_resid_mass(const char* rt, const char* rd, int64_t start, int len, int lane,
                                                  const ResidW& wf) {
    float s = 0.f;
    if constexpr (VEC) {
        constexpr int PV = Elem<EB>::kPerVec;
        constexpr int kHalf = kVecPerLane / 2;
        const uint4* pt = reinterpret_cast<const uint4*>(rt + start * EB);
        const uint4* pd = reinterpret_cast<const uint4*>(rd + start * EB);
        const int nvec = len / PV;
        const uint32_t ni = Elem<EB>::kNegInfWord;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4 at[kHalf], ad[kHalf];
#pragma unroll
            for (int j = 0; j < kHalf; ++j) {
                const int idx = (h * kHalf + j) * kWave + lane;
                at[j] = idx < nvec ? load_stream(pt + idx) : make_uint4(ni, ni, ni, ni);
                ad[j] = idx < nvec ? load_stream(pd + idx) : make_uint4(ni, ni, ni, ni);
            }
#pragma unroll
            for (int j = 0; j < kHalf; ++j) {
                float ft[PV], fd[PV];
                Elem<EB>::decode(at[j], ft);
                Elem<EB>::decode(ad[j], fd);
#pragma unroll
                for (int e = 0; e < PV; ++e) s += wf(ft[e], fd[e]);
            }
        }
    } else {
        for (int e = 0; e < Chunk<EB>::kPerLane; ++e) {
            const int idx = e * kWave + lane;
            if (idx < len) s += wf(Elem<EB>::at(rt, start + idx), Elem<EB>::at(rd, start + idx));
        }
    }
    return wave_sum(s);
}

// ------------------------------------------------------------------ VAT loss partials
//
// The loss needs, per position, the target's (m, Z), the draft's (m, Z) and
// sum_y p(y) (l_d(y) - m_d) c2, the expectation under p of the draft's
// log2-probability up to its normaliser.  A chunk pair contributes
// (m_t, s_t, m_d, s_d, x) with x = sum_y 2^((l_t(y) - m_t) c2) (l_d(y) - m_d) c2
// over its tokens; pairs merge by rescaling to the larger maxima.

struct PairPart {
    float mt, st;  // target: max raw logit, sum of 2^((l - mt) c2)
    float md, sd;  // draft: the same
    float x;       // cross term, <= 0, relative to (mt, md)
};

__device__ __forceinline__ PairPart pair_empty() { return PairPart{neg_inf(), 0.f, neg_inf(), 0.f, 0.f}; }

// Commutative in its arguments bit for bit (sums of two terms, maxima), so a
// DPP butterfly leaves the same value on both lanes of every exchange.
__device__ __forceinline__ PairPart pair_merge(const PairPart& a, const PairPart& b, float c2) {
    PairPart r;
    r.mt = fmaxf(a.mt, b.mt);
    r.md = fmaxf(a.md, b.md);
    const float fa = a.st > 0.f ? exp2_hw((a.mt - r.mt) * c2) : 0.f;
    const float fb = b.st > 0.f ? exp2_hw((b.mt - r.mt) * c2) : 0.f;
    const float ga = a.sd > 0.f ? exp2_hw((a.md - r.md) * c2) : 0.f;
    const float gb = b.sd > 0.f ? exp2_hw((b.md - r.md) * c2) : 0.f;
    r.st = a.st * fa + b.st * fb;
    r.sd = a.sd * ga + b.sd * gb;
    const float xa = a.st > 0.f ? fa * fmaf((a.md - r.md) * c2, a.st, a.x) : 0.f;
    const float xb = b.st > 0.f ? fb * fmaf((b.md - r.md) * c2, b.st, b.x) : 0.f;
    r.x = xa + xb;
    return r;
}

template <int CTRL>
__device__ __forceinline__ PairPart dpp_pair(const PairPart& v) {
    return PairPart{dpp<CTRL>(v.mt, v.mt), dpp<CTRL>(v.st, v.st), dpp<CTRL>(v.md, v.md), dpp<CTRL>(v.sd, v.sd),
                    dpp<CTRL>(v.x, v.x)};
}

__device__ __forceinline__ PairPart readlane_pair(const PairPart& v, int l) {
    return PairPart{readlane(v.mt, l), readlane(v.st, l), readlane(v.md, l), readlane(v.sd, l), readlane(v.x, l)};
}

// Merge over the wave; the same bits on every lane.
__device__ __forceinline__ PairPart wave_merge_pair(PairPart v, float c2) {
    v = pair_merge(v, dpp_pair<kDppQuadSwap1>(v), c2);
    v = pair_merge(v, dpp_pair<kDppQuadSwap2>(v), c2);
    v = pair_merge(v, dpp_pair<kDppRowRor4>(v), c2);
    v = pair_merge(v, dpp_pair<kDppRowRor8>(v), c2);
    const PairPart lo = pair_merge(readlane_pair(v, 0), readlane_pair(v, 16), c2);
    const PairPart hi = pair_merge(readlane_pair(v, 32), readlane_pair(v, 48), c2);
    return pair_merge(lo, hi, c2);
}

// One lane's part of n target/draft logit pairs (fetched twice by `get`).
template <typename Get>
__device__ __forceinline__ PairPart lane_pair(int n, Get get, float c2) {
    float mt = neg_inf(), md = neg_inf();
#pragma unroll
    for (int e = 0; e < n; ++e) {
        const float2 v = get(e);
        mt = fmaxf(mt, v.x);
        md = fmaxf(md, v.y);
    }
    PairPart p{mt, 0.f, md, 0.f, 0.f};
    float ct = 1.f, cd = 1.f;
    const float mtc = mt != neg_inf() ? row_scale(mt, c2, ct) : 0.f;
    const float mdc = md != neg_inf() ? row_scale(md, c2, cd) : 0.f;
    float st = 0.f, sd = 0.f, x = 0.f;
#pragma unroll
    for (int e = 0; e < n; ++e) {
        const float2 v = get(e);
        const float w = mt != neg_inf() ? exp2_hw(fmaf(v.x, c2, -mtc)) : 0.f;
        st += w;
        if (w > 0.f) x = fmaf(w, (v.y - md) * c2, x);
        sd += md != neg_inf() ? exp2_hw(fmaf(v.y, c2, -mdc)) : 0.f;
    }
    p.st = st * ct;
    p.sd = sd * cd;
    p.x = x * ct;
    return p;
}

// Pair partials of chunk c of target row i and draft row i of block b (the
// wave's merged result; put_pair publishes it).  Whole wave.
template <int EB, bool VEC>
__device__ __forceinline__ PairPart stream_pair(const Plan& pl, int b, int i, int c) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t V = pl.vocab;
    const char* rt = row_base(pl.target, static_cast<int64_t>(b) * pl.k + i, V, EB);
    const char* rd = row_base(pl.draft, static_cast<int64_t>(b) * pl.k + i, V, EB);
    const int64_t start = static_cast<int64_t>(c) * Chunk<EB>::kElems;
    const int len = static_cast<int>(min(static_cast<int64_t>(Chunk<EB>::kElems), V - start));
    const float c2 = pl.c2;
    PairPart acc = pair_empty();
    if constexpr (VEC) {
        // Two 16-byte vectors of each row per step keeps the decoded values
        // of both rows within the register budget of the streaming loop.
        constexpr int PV = Elem<EB>::kPerVec;
        constexpr int kStep = 2;
        const uint4* pt = reinterpret_cast<const uint4*>(rt + start * EB);
        const uint4* pd = reinterpret_cast<const uint4*>(rd + start * EB);
        const int nvec = len / PV;
        const uint32_t ni = Elem<EB>::kNegInfWord;
        uint4 at[kVecPerLane], ad[kVecPerLane];
#pragma unroll
        for (int j = 0; j < kVecPerLane; ++j) {
            const int idx = j * kWave + lane;
            at[j] = idx < nvec ? load_stream(pt + idx) : make_uint4(ni, ni, ni, ni);
            ad[j] = idx < nvec ? load_stream(pd + idx) : make_uint4(ni, ni, ni, ni);
        }
#pragma unroll
        for (int h = 0; h < kVecPerLane; h += kStep) {
            float ft[kStep * PV], fd[kStep * PV];
#pragma unroll
            for (int j = 0; j < kStep; ++j) {
                Elem<EB>::decode(at[h + j], &ft[j * PV]);
                Elem<EB>::decode(ad[h + j], &fd[j * PV]);
            }
            acc = pair_merge(acc, lane_pair(kStep * PV, [&](int e) { return make_float2(ft[e], fd[e]); }, c2), c2);
        }
    } else {
        constexpr int kStep = 8;
#pragma unroll 1
        for (int e0 = 0; e0 < Chunk<EB>::kPerLane; e0 += kStep) {
            float ft[kStep], fd[kStep];
#pragma unroll
            for (int e = 0; e < kStep; ++e) {
                const int idx = (e0 + e) * kWave + lane;
                ft[e] = idx < len ? Elem<EB>::at(rt, start + idx) : neg_inf();
                fd[e] = idx < len ? Elem<EB>::at(rd, start + idx) : neg_inf();
            }
            acc = pair_merge(acc, lane_pair(kStep, [&](int e) { return make_float2(ft[e], fd[e]); }, c2), c2);
        }
    }
    return wave_merge_pair(acc, c2);
}

// The five tagged words of a chunk pair's partials (one lane).
__device__ __forceinline__ void put_pair(const Plan& pl, int b, int li, const PairPart& acc) {
    uint64_t* w = chunk_words(pl, b) + static_cast<int64_t>(li) * kPairWords;
    put_word(w + 0, __float_as_uint(acc.mt), pl.tag);
    put_word(w + 1, __float_as_uint(acc.st), pl.tag);
    put_word(w + 2, __float_as_uint(acc.md), pl.tag);
    put_word(w + 3, __float_as_uint(acc.sd), pl.tag);
    put_word(w + 4, __float_as_uint(acc.x), pl.tag);
}

// ------------------------------------------------------------------ finishers

// Marks a sequence whose decision's wait ran out (see kPollTimeoutTicks).
// Only the decision finisher, which owns these outputs, calls it.
template <int MODE>
__device__ __forceinline__ void fail_sequence(const Plan& pl, int b) {
    using Tr = PathTraits<MODE>;
    const int k = pl.k;
    for (int j = threadIdx.x; j <= k; j += kBlock) {
        if constexpr (Tr::vat) {
            if (j < k) {
                pl.mask[static_cast<int64_t>(b) * k + j] = 0;
                pl.weights[static_cast<int64_t>(b) * k + j] = 0.f;
            }
        } else {
            pl.out_tokens[static_cast<int64_t>(b) * (k + 1) + j] = -1;
        }
    }
    if (threadIdx.x == 0) {
        if constexpr (Tr::vat) pl.first_reject[b] = -2;
        else pl.accepted_len[b] = -2;
    }
}

// Row (m, Z) -- or (max, argmax) at T == 0 -- of local row j from its P
// partials; one wave.  Result on every lane.
__device__ __forceinline__ float2 combine_row(const PartialSrc& src, int j, int P, bool greedy, float c2) {
    const int lane = threadIdx.x & (kWave - 1);
    if (greedy) {
        float best = neg_inf();
        int bi = INT_MAX;
        for (int c = lane; c < P; c += kWave) {
            const float2 pc = src.get(j * P + c);
            argmax_step(best, bi, pc.x, __float_as_int(pc.y));
        }
        wave_argmax(best, bi);
        return make_float2(best, __int_as_float(bi));
    }
    float m = neg_inf(), s = 0.f;
    for (int c = lane; c < P; c += kWave) {
        const float2 pc = src.get(j * P + c);
        if (pc.x == neg_inf()) continue;
        if (pc.x > m) {
            s = (m == neg_inf() ? 0.f : s * exp2_hw((m - pc.x) * c2)) + pc.y;
            m = pc.x;
        } else {
            s += pc.y * exp2_hw((pc.x - m) * c2);
        }
    }
    wave_merge_ms(m, s, c2);
    return make_float2(m, s);
}

// (m, Z) -- or (max, argmax) at T == 0 -- of local rows [j0, j1) from their
// P partials each: every row on the 16 lanes of one DPP row (16 rows per pass
// over the block), a lane merging partials sub, sub+16, ... in order, then
// four DPP steps inside the row.  No readlane and no cross-row step.  Lane 0
// of each row writes mz[j].  Whole block.
__device__ __forceinline__ void combine_rows(const PartialSrc& src, int j0, int j1, int P, bool greedy, float c2,
                                             float2* mz) {
    const int sub = threadIdx.x & 15;
    for (int jb = j0; jb < j1; jb += kBlock / 16) {
        const int j = jb + static_cast<int>(threadIdx.x / 16);
        const bool on = j < j1;
        if (greedy) {
            float best = neg_inf();
            int bi = INT_MAX;
            if (on) {
                for (int c = sub; c < P; c += 16) {
                    const float2 pc = src.get(j * P + c);
                    argmax_step(best, bi, pc.x, __float_as_int(pc.y));
                }
            }
            argmax_step(best, bi, dpp<kDppQuadSwap1>(best, best), dpp_i<kDppQuadSwap1>(bi, bi));
            argmax_step(best, bi, dpp<kDppQuadSwap2>(best, best), dpp_i<kDppQuadSwap2>(bi, bi));
            argmax_step(best, bi, dpp<kDppRowRor4>(best, best), dpp_i<kDppRowRor4>(bi, bi));
            argmax_step(best, bi, dpp<kDppRowRor8>(best, best), dpp_i<kDppRowRor8>(bi, bi));
            if (on && sub == 0) mz[j] = make_float2(best, __int_as_float(bi));
        } else {
            float m = neg_inf(), s = 0.f;
            if (on) {
                for (int c = sub; c < P; c += 16) {
                    const float2 pc = src.get(j * P + c);
                    if (pc.x == neg_inf()) continue;
                    if (pc.x > m) {
                        s = (m == neg_inf() ? 0.f : s * exp2_hw((m - pc.x) * c2)) + pc.y;
                        m = pc.x;
                    } else {
                        s += pc.y * exp2_hw((pc.x - m) * c2);
                    }
                }
            }
            float M = fmaxf(m, dpp<kDppQuadSwap1>(m, m));
            M = fmaxf(M, dpp<kDppQuadSwap2>(M, M));
            M = fmaxf(M, dpp<kDppRowRor4>(M, M));
            M = fmaxf(M, dpp<kDppRowRor8>(M, M));
            float t = m == neg_inf() ? 0.f : s * exp2_hw((m - M) * c2);
            t += dpp<kDppQuadSwap1>(t, t);
            t += dpp<kDppQuadSwap2>(t, t);
            t += dpp<kDppRowRor4>(t, t);
            t += dpp<kDppRowRor8>(t, t);
            if (on && sub == 0) mz[j] = make_float2(M, t);
        }
    }
}

__device__ __forceinline__ void write_row_stats(const Plan& pl, int64_t grow, float2 res) {
    if (!pl.row_stats_out) return;
    pl.row_stats_out[2 * grow] = pl.greedy ? res.x : res.x / pl.temperature;
    pl.row_stats_out[2 * grow + 1] = pl.greedy ? static_cast<float>(__float_as_int(res.y)) : res.y;
}

// Block-wide minimum of one int per thread.  Whole block.
__device__ __forceinline__ int block_min(int v, int* flags) {
    const int w = wave_min_i(v);
    if ((threadIdx.x & (kWave - 1)) == 0) flags[threadIdx.x / kWave] = w;
    __syncthreads();
    int m = flags[0];
#pragma unroll
    for (int q = 1; q < kWavesPerBlock; ++q) m = min(m, flags[q]);
    __syncthreads();
    return m;
}

// Per-position values a decision needs, held by wave 0 (lane i: position i).
struct PosRegs {
    int x;         // draft token
    float u;       // the uniform of its test
    float lt, ld;  // target and draft logits at the token (T > 0)
    float p, q;    // p_i(x_i), q_i(x_i) once the position is tested
    bool active;   // wave 0, lane < k
    bool bad;      // token outside [0, V)
};

// Loads that do not depend on any partial, issued before the polling: the
// token and uniform of each position, and (T > 0) the logits at the token
// (index clamped into the row; an invalid token flags the sequence).
template <int EB, int MODE>
__device__ __forceinline__ PosRegs load_positions(const Plan& pl, int b) {
    using Tr = PathTraits<MODE>;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = pl.k;
    const int64_t V = pl.vocab;
    PosRegs pr;
    pr.x = 0;
    pr.u = pr.lt = pr.ld = 0.f;
    pr.p = pr.q = __builtin_nanf("");
    pr.active = threadIdx.x < kWave && lane < k;
    if (pr.active) {
        pr.x = pl.tokens[static_cast<int64_t>(b) * k + lane];
        if (!Tr::greedy) pr.u = pl.uniforms[static_cast<int64_t>(b) * (Tr::vat ? k : k + 1) + lane];
    }
    pr.bad = pr.active && (pr.x < 0 || pr.x >= pl.vocab);
    if (!Tr::greedy && pr.active) {
        const int xc = min(max(pr.x, 0), pl.vocab - 1);
        pr.lt = Elem<EB>::at(row_base(pl.target, static_cast<int64_t>(b) * pl.target_rows_per_seq + lane, V, EB), xc);
        if (Tr::halves == 2) pr.ld = Elem<EB>::at(row_base(pl.draft, static_cast<int64_t>(b) * k + lane, V, EB), xc);
    }
    return pr;
}

// The test of position i (wave 0, lane i): u q(x) < p(x), taken in the log2
// domain so that probabilities below the fp32 range still decide correctly;
// at T == 0, x_i == the row's lowest-index argmax.  Sets pr.p, pr.q.
template <int MODE>
__device__ __forceinline__ bool test_position(const Plan& pl, const TailShared& sh, PosRegs& pr, int i) {
    using Tr = PathTraits<MODE>;
    constexpr int H = Tr::halves;
    if constexpr (Tr::greedy) {
        const bool keep = pr.x == __float_as_int(sh.mz[i * H].y);
        pr.p = keep ? 1.f : 0.f;
        pr.q = 1.f;
        return keep;
    } else {
        const float2 mzt = sh.mz[i * H];
        const float lp = (pr.lt - mzt.x) * pl.c2 - log2_hw(mzt.y);
        float lq = 0.f;
        if constexpr (H == 2) {
            const float2 mzd = sh.mz[i * H + 1];
            lq = (pr.ld - mzd.x) * pl.c2 - log2_hw(mzd.y);
        }
        pr.p = exp2_hw(lp);
        pr.q = exp2_hw(lq);
        return log2_hw(pr.u) + lq < lp;
    }
}

// The decision of sequence b, taken by every block that needs it (decision
// finisher, residual and bonus roles), so that none of them waits on
// another: polls the sequence's segment words, and as soon as all segments
// of the next positions are there combines their rows and tests them in
// order; stops at the first rejection unless every position is asked for
// (`all`: row statistics or probabilities of every position).  Returns r in
// [0, k] (k: all kept), -1 (a token outside [0, V)) or -2 (the wait ran
// out); leaves the combined rows in sh.mz (local row numbering) and the
// tested positions' p_i(x_i), q_i(x_i) in pr.  With `row0_chunks` (one-hot
// window mode) position 0 is decided from row 0's chunk words instead of its
// segment words, staged in sh.stage after the segment words for a draw at
// r = 0.  Whole block.
template <int EB, bool VEC, int MODE>
__device__ __forceinline__ int decide(const Plan& pl, int b, TailShared& sh, bool all, PosRegs& pr, uint64_t timeout,
                                      bool progress = false, bool row0_chunks = false) {
    using Tr = PathTraits<MODE>;
    constexpr int H = Tr::halves;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = pl.k;
    const int S = pl.segs;
    const int per_pos = 2 * H * S;
    const int n_words = k * per_pos;
    const uint64_t* words = seg_words(pl, b);
    const bool staged = n_words <= kStageWords;
    const PartialSrc src{staged ? sh.stage : nullptr, words};
    if (threadIdx.x < kWave) {
        const bool invalid = __ballot(pr.bad) != 0ull;
        if (lane == 0) sh.r = invalid ? -1 : k;
    }
    __syncthreads();
    int r = sh.r;
    if (r < 0) return -1;
    int done = 0;
    const uint64_t t0 = wall_clock64();
    if (row0_chunks) {
        // One poll of the row's chunk words (one per chunk) rather than of
        // its segment words: the same arrival, and a rejection at 0 then
        // draws from words already staged.
        const int P = pl.chunks;
        uint32_t* cst = sh.stage + n_words;
        if (!collect(chunk_words(pl, b), 2 * P, pl.tag, cst, sh.vote, false, timeout)) return -2;
        combine_rows(PartialSrc{cst, nullptr}, 0, 1, P, Tr::greedy, pl.c2, sh.mz);
        __syncthreads();
        if (threadIdx.x < kWave) {
            bool keep = true;
            if (lane == 0) keep = test_position<MODE>(pl, sh, pr, 0);
            if (lane == 0 && !keep) sh.r = 0;
        }
        __syncthreads();
        r = sh.r;
        done = 1;
        if (progress && r == k && done < k && threadIdx.x == kWave)
            put_word(progress_word(pl, b), static_cast<uint32_t>(done), pl.tag);
        if (done == k || (r < k && !all)) return r;
    }
    for (;;) {
        int miss = k;  // first position with a segment word not yet there
        for (int w = done * per_pos + static_cast<int>(threadIdx.x); w < n_words; w += kBlock) {
            const uint64_t v = get_word(words + w);
            if (static_cast<uint32_t>(v >> 32) != pl.tag) miss = min(miss, w / per_pos);
            else if (staged) sh.stage[w] = word_data(v);
        }
        const int f = block_min(miss, sh.vote);
        if (f > done) {
            combine_rows(src, done * H, f * H, S, Tr::greedy, pl.c2, sh.mz);
            __syncthreads();
            if (threadIdx.x < kWave) {
                const bool in = lane >= done && lane < f;
                bool keep = true;
                if (in) keep = test_position<MODE>(pl, sh, pr, lane);
                const uint64_t rej = __ballot(in && !keep);
                if (lane == 0 && rej && r == k) sh.r = __builtin_ctzll(rej);
            }
            __syncthreads();
            r = sh.r;
            done = f;
            // window mode: the accepted prefix so far, for the workers of
            // the next positions
            if (progress && r == k && done < k && threadIdx.x == kWave)
                put_word(progress_word(pl, b), static_cast<uint32_t>(done), pl.tag);
        }
        if (done == k || (r < k && !all)) return r;
        // waves read the clock at slightly different times: decide together
        if (block_any(wall_clock64() - t0 > timeout, sh.vote)) return -2;
        __builtin_amdgcn_s_sleep(4);
    }
}

// The draw of a one-hot draft rejected at r: target row r without x_r.
template <int EB>
__device__ __forceinline__ DrawRow onehot_row(const Plan& pl, int b, int r, const PartialSrc& src, float m_r, int x_r,
                                              float l_x) {
    DrawRow d;
    d.mode = kModeOneHot;
    d.rt = row_base(pl.target, static_cast<int64_t>(b) * pl.target_rows_per_seq + r, pl.vocab, EB);
    d.rd = nullptr;
    d.part = src;
    d.part_base = 0;
    d.rstage = nullptr;
    d.rwords = nullptr;
    d.c2 = pl.c2;
    d.mrow = m_r;
    d.mt = row_scale(m_r, pl.c2, d.corr);
    d.excl = x_r;
    d.lx = l_x;
    return d;
}

// accepted_len and out_tokens of a sequence, stored by wave 0 of its
// decision finisher (lane i holds x_i): x_0..x_{r-1}, -1 after r, and at r
// the greedy argmax or `token` (a one-hot draw); a residual or bonus token at
// r is stored by the block that draws it.
template <int MODE>
__device__ __forceinline__ void publish_outputs(const Plan& pl, int b, int r, int x, int token, const TailShared& sh) {
    using Tr = PathTraits<MODE>;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = pl.k;
    int32_t* out = pl.out_tokens + static_cast<int64_t>(b) * (k + 1);
    for (int j = lane; j <= k; j += kWave) {
        if (r < 0) out[j] = -1;
        else if (j < r) out[j] = x;  // j < r <= k <= 64 here, so j == lane
        else if (j > r) out[j] = -1;
        else if (Tr::greedy && r < k) out[j] = __float_as_int(sh.mz[r].y);
        else if (Tr::onehot && r < k) out[j] = token;
    }
    if (lane == 0) pl.accepted_len[b] = r;
}

// Decision finisher of sequence b: the outputs that depend on rows 0..k-1
// (accepted prefix, VAT labels and weights, probabilities, row statistics)
// and the one-hot draw.
template <int EB, bool VEC, int MODE>
__device__ __forceinline__ void decision_finisher(const Plan& pl, int b, TailShared& sh) {
    using Tr = PathTraits<MODE>;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = pl.k;
    const int P = pl.chunks;
    const int64_t V = pl.vocab;
    PosRegs pr = load_positions<EB, MODE>(pl, b);
    const float u_draw = Tr::onehot ? pl.uniforms[static_cast<int64_t>(b) * (k + 1) + k] : 0.f;
    const bool all = pl.probs_out || pl.row_stats_out;
    // window mode: the accepted prefix is published only while the
    // read-ahead is limited (a store would delay this wave's next poll)
    int known;
    bool limited = false;
    if constexpr (Tr::bonus && Tr::halves == 1) limited = pl.window && read_ahead(pl, b, sh, known) < pl.k;
    // One-hot window mode: position 0 from row 0's chunk words (staged after
    // the segment words, if they fit)
    const int seg_n = k * 2 * pl.segs;
    const bool row0 = Tr::onehot && pl.window && !all && seg_n + 2 * P <= kStageWords;
    const int r = decide<EB, VEC, MODE>(pl, b, sh, all, pr, kPollTimeoutTicks, limited, row0);
    if (r == -2) {
        fail_sequence<MODE>(pl, b);
        return;
    }
    if (pl.row_stats_out && r >= 0)
        for (int j = threadIdx.x; j < pl.dec_rows; j += kBlock) write_row_stats(pl, global_row(pl, b, j), sh.mz[j]);
    const bool draws = Tr::onehot && r >= 0 && r < k;
    // r for the bonus workers that read the bonus row only after full
    // acceptance, and for the window's workers (after the one-hot draw when
    // there is one and no worker waits for it: see below).
    if (Tr::bonus && (!draws || pl.window) && threadIdx.x == kWave) {
        put_word(decision_word(pl, b), static_cast<uint32_t>(r + 2), pl.tag);
        if (pl.window) put_word(history_word(pl, b), static_cast<uint32_t>(r + 2), pl.tag);
    }
    if (threadIdx.x < kWave) {
        const int i = lane;
        if (pl.probs_out && pr.active) {
            pl.probs_out[2 * (static_cast<int64_t>(b) * k + i)] = pr.p;
            pl.probs_out[2 * (static_cast<int64_t>(b) * k + i) + 1] = pr.q;
        }
        if constexpr (Tr::vat) {
            const bool invalid = r < 0;
            if (pr.active) {
                const int64_t o = static_cast<int64_t>(b) * k + i;
                pl.mask[o] = static_cast<uint8_t>(!invalid && i < r);
                // decay^(i-r) in fp64, rounded once to fp32
                pl.weights[o] = invalid ? 0.f
                                        : (i < r ? 1.f
                                                 : static_cast<float>(pow(static_cast<double>(pl.decay),
                                                                          static_cast<double>(i - r))));
            }
            if (lane == 0) pl.first_reject[b] = r;
        } else {
            // A one-hot draw is taken by this block before anything else is
            // stored: loads behind this wave's write-through stores would
            // wait for their acknowledgements as well.
            if (!draws) {
                publish_outputs<MODE>(pl, b, r, pr.x, -1, sh);
            } else {
                const int x_r = __builtin_amdgcn_readlane(pr.x, r);
                const float l_x = readlane(pr.lt, r);
                if (lane == 0) {
                    sh.x_r = x_r;
                    sh.l_x = l_x;
                }
            }
        }
    }
    if constexpr (Tr::onehot) {
        if (!draws) return;
        // chunk partials of target row r (local row r), tags checked
        const uint64_t* cw = chunk_words(pl, b) + static_cast<int64_t>(r) * P * 2;
        const float m_r = sh.mz[r].x;
        bool ok = true;
        PartialSrc src{sh.stage + seg_n, cw};  // a rejection at 0 in window mode: staged by decide
        if (!(row0 && r == 0)) {
            const bool cstaged = 2 * P <= kStageWords;
            ok = collect(cw, 2 * P, pl.tag, cstaged ? sh.stage : nullptr, sh.vote, false);
            src = PartialSrc{cstaged ? sh.stage : nullptr, cw};
        } else {
            __syncthreads();  // sh.x_r and sh.l_x, written by wave 0, for every wave (collect's barrier otherwise)
        }
        const DrawRow d = onehot_row<EB>(pl, b, r, src, m_r, sh.x_r, sh.l_x);
        const int y = ok ? draw_token<EB, VEC>(d, u_draw, P, V, sh) : -2;
        if (threadIdx.x < kWave) publish_outputs<MODE>(pl, b, r, pr.x, y, sh);
        if (threadIdx.x == kWave && !pl.window) put_word(decision_word(pl, b), static_cast<uint32_t>(r + 2), pl.tag);
    }
}

// Residual worker `w` of sequence b: decides, and if the sequence rejected
// at r, the mass of max(0, p_r - q_r) over one chunk pair per wavefront.
template <int EB, bool VEC, int MODE>
__device__ __forceinline__ void residual_worker(const Plan& pl, int b, int w, TailShared& sh) {
    PosRegs pr = load_positions<EB, MODE>(pl, b);
    const int r = decide<EB, VEC, MODE>(pl, b, sh, false, pr, kDecisionTimeoutTicks);
    if (r < 0 || r >= pl.k) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int P = pl.chunks;
    const int64_t V = pl.vocab;
    const ResidW wf = make_resid_w(sh.mz[2 * r], sh.mz[2 * r + 1], pl.c2);
    const char* rt = row_base(pl.target, static_cast<int64_t>(b) * pl.target_rows_per_seq + r, V, EB);
    const char* rd = row_base(pl.draft, static_cast<int64_t>(b) * pl.k + r, V, EB);
    const int base = w * kWavesPerBlock * pl.nc_res + static_cast<int>(threadIdx.x / kWave);
    // the masses go out after all of the wave's loads (see stream_segment)
    float mass[kChunksPerWaveResid];
#pragma unroll
    for (int n = 0; n < kChunksPerWaveResid; ++n) {
        const int c = base + n * kWavesPerBlock;
        mass[n] = 0.f;
        if (n < pl.nc_res && c < P) {
            const int64_t start = static_cast<int64_t>(c) * Chunk<EB>::kElems;
            const int len = static_cast<int>(min(static_cast<int64_t>(Chunk<EB>::kElems), V - start));
            mass[n] = chunk_resid_mass<EB, VEC>(rt, rd, start, len, lane, wf);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int n = 0; n < kChunksPerWaveResid; ++n) {
            const int c = base + n * kWavesPerBlock;
            if (n < pl.nc_res && c < P) put_word(resid_words(pl, b) + c, __float_as_uint(mass[n]), pl.tag);
        }
    }
}

// Residual finisher of sequence b: decides, and draws the target's token at
// r < k from the residual masses.
template <int EB, bool VEC, int MODE>
__device__ __forceinline__ void residual_finisher(const Plan& pl, int b, TailShared& sh) {
    const int P = pl.chunks;
    const int k = pl.k;
    const int64_t V = pl.vocab;
    PosRegs pr = load_positions<EB, MODE>(pl, b);
    const float u_draw = pl.uniforms[static_cast<int64_t>(b) * (k + 1) + k];
    // a decision that never comes is reported by the decision finisher
    const int r = decide<EB, VEC, MODE>(pl, b, sh, false, pr, kDecisionTimeoutTicks);
    if (r < 0 || r >= k) return;
    const float2 mzt = sh.mz[2 * r], mzd = sh.mz[2 * r + 1];
    int32_t* token = pl.out_tokens + static_cast<int64_t>(b) * (k + 1) + r;
    uint64_t* rwords = resid_words(pl, b);
    const bool staged = P <= kStageWords;
    if (!collect(rwords, P, pl.tag, staged ? sh.stage : nullptr, sh.vote, pl.two_deep_polls)) {
        if (threadIdx.x == 0) *token = -2;
        return;
    }
    DrawRow d;
    d.mode = kModeResidual;
    d.rt = row_base(pl.target, static_cast<int64_t>(b) * pl.target_rows_per_seq + r, V, EB);
    d.rd = row_base(pl.draft, static_cast<int64_t>(b) * k + r, V, EB);
    d.part = PartialSrc{nullptr, nullptr};
    d.part_base = 0;
    d.rstage = staged ? sh.stage : nullptr;
    d.rwords = rwords;
    d.c2 = pl.c2;
    d.mrow = mzt.x;
    d.mt = row_scale(mzt.x, pl.c2, d.corr);
    d.excl = -1;
    d.lx = 0.f;
    d.rw = make_resid_w(mzt, mzd, pl.c2);
    // A residual that rounds to zero mass (only possible through rounding,
    // since a rejection has probability TV(p, q)): draw from p_r instead,
    // from target row r's chunk partials, collected (tags checked) here.
    float zsum = 0.f;
    for (int cc = threadIdx.x; cc < P; cc += kBlock) zsum += chunk_mass(d, cc, -1, 0.f);
    if (!block_any(zsum > 0.f, sh.vote)) {
        const uint64_t* pw = chunk_words(pl, b) + static_cast<int64_t>(2 * r) * P * 2;
        const bool pstaged = 2 * P <= kStageWords;
        if (!collect(pw, 2 * P, pl.tag, pstaged ? sh.stage : nullptr, sh.vote, false)) {
            if (threadIdx.x == 0) *token = -2;
            return;
        }
        d.mode = kModeBonus;
        d.part = PartialSrc{pstaged ? sh.stage : nullptr, pw};
    }
    const int y = draw_token<EB, VEC>(d, u_draw, P, V, sh);
    if (threadIdx.x == 0) *token = y;
}

// Bonus worker of sequence b, segment s of the bonus row (target position
// k).  It is read only when the sequence kept all k drafts (or when every
// row's statistics are asked for), except for the last sequences, whose
// decisions come late: they read it at once.  The others wait for the
// decision finisher's word rather than deciding themselves: one word against
// the sequence's segment words and their combination, for blocks whose
// decision is long taken when they run.
template <int EB, bool VEC, int MODE>
__device__ __forceinline__ void bonus_worker(const Plan& pl, int b, int s, TailShared& sh) {
    if (pl.window) {
        // window mode: not after a known rejection; with the read-ahead
        // limited, once the accepted prefix comes near position k or after
        // full acceptance
        int known;
        const int ahead = read_ahead(pl, b, sh, known);
        if (known != pl.k || (ahead < pl.k && released(pl, b, pl.k, sh) == 0)) return;
    } else if (!pl.row_stats_out && b < pl.eager_bonus_from) {
        if (!collect(decision_word(pl, b), 1, pl.tag, sh.stage, sh.vote, false, kDecisionTimeoutTicks)) return;
        if (static_cast<int>(sh.stage[0]) - 2 != pl.k) return;
    } else if (!pl.row_stats_out && pl.grid.fin_first) {
        // Finishers placed first have often decided by now: one look at the
        // decision word, and no read of a row that a rejection makes useless.
        if (threadIdx.x == 0) {
            const uint64_t w = get_word(decision_word(pl, b));
            sh.stage[0] = static_cast<uint32_t>(w >> 32) == pl.tag ? word_data(w) : 0u;
        }
        __syncthreads();
        const uint32_t d = sh.stage[0];
        if (d != 0u && static_cast<int>(d) - 2 != pl.k) return;
    }
    stream_segment<EB, VEC, MODE>(pl, b, pl.dec_rows, s, sh);
}

// Bonus finisher of sequence b: decides; the statistics of target row k
// and, when all k drafts were kept, the token drawn from it (its argmax at
// T == 0).
template <int EB, bool VEC, int MODE>
__device__ __forceinline__ void bonus_finisher(const Plan& pl, int b, TailShared& sh) {
    using Tr = PathTraits<MODE>;
    const int lane = threadIdx.x & (kWave - 1);
    const int k = pl.k;
    const int P = pl.chunks;
    const int64_t V = pl.vocab;
    PosRegs pr = load_positions<EB, MODE>(pl, b);
    const float u_draw = Tr::greedy ? 0.f : pl.uniforms[static_cast<int64_t>(b) * (k + 1) + k];
    const int r = decide<EB, VEC, MODE>(pl, b, sh, false, pr, kDecisionTimeoutTicks);
    if (r < 0 || (r != k && !pl.row_stats_out)) return;
    int32_t* token = pl.out_tokens + static_cast<int64_t>(b) * (k + 1) + k;
    // The row's chunk partials, combined directly: the draw needs them
    // anyway, so one wait covers the row's statistics and the draw.
    const uint64_t* cw = chunk_words(pl, b) + static_cast<int64_t>(pl.dec_rows) * P * 2;
    const bool cstaged = 2 * P <= kStageWords;
    const PartialSrc src{cstaged ? sh.stage : nullptr, cw};
    if (!collect(cw, 2 * P, pl.tag, src.stage ? sh.stage : nullptr, sh.vote, pl.two_deep_polls)) {
        if (r == k && threadIdx.x == 0) *token = -2;
        return;
    }
    if (threadIdx.x < kWave) {
        const float2 res = combine_row(src, 0, P, Tr::greedy, pl.c2);
        if (lane == 0) {
            sh.mz[0] = res;
            write_row_stats(pl, global_row(pl, b, pl.dec_rows), res);
        }
    }
    __syncthreads();
    if (r != k) return;
    if constexpr (Tr::greedy) {
        if (threadIdx.x == 0) *token = __float_as_int(sh.mz[0].y);
    } else {
        const float m_k = sh.mz[0].x;
        DrawRow d;
        d.mode = kModeBonus;
        d.rt = row_base(pl.target, static_cast<int64_t>(b) * pl.target_rows_per_seq + k, V, EB);
        d.rd = nullptr;
        d.part = PartialSrc{cstaged ? sh.stage : nullptr, cw};
        d.part_base = 0;
        d.rstage = nullptr;
        d.rwords = nullptr;
        d.c2 = pl.c2;
        d.mrow = m_k;
        d.mt = row_scale(m_k, pl.c2, d.corr);
        d.excl = -1;
        d.lx = 0.f;
        const int y = draw_token<EB, VEC>(d, u_draw, P, V, sh);
        if (threadIdx.x == 0) *token = y;
    }
}

// VAT loss finisher of block b: the pair partials of each position, combined
// by one wave per position; then on wave 0, one lane per position: the
// simulated acceptance, labels and weights (as the decision finisher), the soft
// and hard terms and the block's weighted loss.
template <int EB, bool VEC>
__device__ __forceinline__ void vat_loss_finisher(const Plan& pl, int b, TailShared& sh) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int k = pl.k;
    const int P = pl.chunks;
    const int64_t V = pl.vocab;
    const float c2 = pl.c2;
    const int64_t o = static_cast<int64_t>(b) * k;

    // Token and logit loads that need no partials go out first.
    const bool active = wave == 0 && lane < k;
    int x = 0, h = 0;
    float u = 0.f, lt = 0.f, ld = 0.f, ldh = 0.f;
    if (active) {
        x = pl.tokens[o + lane];
        h = pl.hard_tokens[o + lane];
        u = pl.uniforms[o + lane];
    }
    const bool bad = active && (x < 0 || x >= pl.vocab || h < 0 || h >= pl.vocab);
    if (active) {
        const int xc = min(max(x, 0), pl.vocab - 1);
        const int hc = min(max(h, 0), pl.vocab - 1);
        const char* rt = row_base(pl.target, o + lane, V, EB);
        const char* rd = row_base(pl.draft, o + lane, V, EB);
        lt = Elem<EB>::at(rt, xc);
        ld = Elem<EB>::at(rd, xc);
        ldh = Elem<EB>::at(rd, hc);
    }

    // Position i on wave i % 4: lanes poll their chunks' five words.
    const uint64_t* words = chunk_words(pl, b);
    bool timed_out = false;
    const uint64_t t0 = wall_clock64();
    for (int i = wave; i < k; i += kWavesPerBlock) {
        PairPart acc = pair_empty();
        for (int c0 = 0; c0 < P && !timed_out; c0 += kWave) {
            const int c = c0 + lane;
            const uint64_t* w = words + (static_cast<int64_t>(i) * P + c) * kPairWords;
            uint32_t d[kPairWords] = {0u, 0u, 0u, 0u, 0u};
            for (;;) {
                bool missing = false;
                if (c < P) {
#pragma unroll
                    for (int q = 0; q < kPairWords; ++q) {
                        const uint64_t v = get_word(w + q);
                        if (static_cast<uint32_t>(v >> 32) != pl.tag) missing = true;
                        d[q] = word_data(v);
                    }
                }
                if (__ballot(missing) == 0ull) break;
                if (wall_clock64() - t0 > kPollTimeoutTicks) {
                    timed_out = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
            if (c < P)
                acc = pair_merge(acc, PairPart{__uint_as_float(d[0]), __uint_as_float(d[1]), __uint_as_float(d[2]),
                                               __uint_as_float(d[3]), __uint_as_float(d[4])}, c2);
        }
        acc = wave_merge_pair(acc, c2);
        if (lane == 0) {
            sh.mz[i] = make_float2(acc.mt, acc.st);
            sh.mz[k + i] = make_float2(acc.md, acc.sd);
            sh.xs[i] = acc.x;
            write_row_stats(pl, o + i, make_float2(acc.mt, acc.st));
            write_row_stats(pl, pl.rows_t + o + i, make_float2(acc.md, acc.sd));
        }
    }
    if (block_any(timed_out, sh.vote)) {
        fail_sequence<kPathVatLoss>(pl, b);
        for (int j = threadIdx.x; j < k; j += kBlock) {
            pl.soft_ce[o + j] = __builtin_nanf("");
            pl.hard_ce[o + j] = __builtin_nanf("");
        }
        if (threadIdx.x == 0) pl.block_loss[b] = __builtin_nanf("");
        return;
    }
    if (wave != 0) return;

    const int i = lane;
    const bool invalid = __ballot(bad) != 0ull;
    bool keep = false;
    float p = __builtin_nanf(""), q = __builtin_nanf("");
    float log2zd = 0.f;
    if (!invalid && active) {
        const float2 mzt = sh.mz[i], mzd = sh.mz[k + i];
        const float lp = (lt - mzt.x) * c2 - log2_hw(mzt.y);
        log2zd = log2_hw(mzd.y);
        const float lq = (ld - mzd.x) * c2 - log2zd;
        keep = log2_hw(u) + lq < lp;
        p = exp2_hw(lp);
        q = exp2_hw(lq);
    }
    const uint64_t kept = __ballot(keep);
    const uint64_t lowk = (k == 64) ? ~0ull : ((1ull << k) - 1ull);
    const uint64_t rej = ~kept & lowk;
    const int r = invalid ? -1 : (rej ? __builtin_ctzll(rej) : k);
    float contrib = 0.f;
    if (active) {
        float wi = 0.f, soft = __builtin_nanf(""), hard = __builtin_nanf("");
        if (!invalid) {
            wi = i < r ? 1.f
                       : static_cast<float>(pow(static_cast<double>(pl.decay), static_cast<double>(i - r)));
            const float2 mzt = sh.mz[i], mzd = sh.mz[k + i];
            // -sum p ln q = ln2 (log2 Z_d - sum_y p(y) (l_d(y) - m_d) c2)
            soft = kLn2 * (log2zd - sh.xs[i] / mzt.y);
            hard = kLn2 * (log2zd - (ldh - mzd.x) * c2);
            contrib = wi * fmaf(pl.hard_weight, hard, soft);
        }
        pl.mask[o + i] = static_cast<uint8_t>(!invalid && i < r);
        pl.weights[o + i] = wi;
        pl.soft_ce[o + i] = soft;
        pl.hard_ce[o + i] = hard;
        if (pl.probs_out) {
            pl.probs_out[2 * (o + i)] = p;
            pl.probs_out[2 * (o + i) + 1] = q;
        }
    }
    const float total = wave_sum(contrib);
    if (lane == 0) {
        pl.first_reject[b] = r;
        pl.block_loss[b] = invalid ? __builtin_nanf("") : total;
    }
}

// ------------------------------------------------------------------ kernel

// Five resident blocks per CU (five waves per SIMD, kMinBlocksPerCu): the
// register budget the streaming loop is written for (at most 102 VGPRs).
template <int EB, bool VEC, int MODE>
__global__ __launch_bounds__(kBlock, kMinBlocksPerCu) void k_verify(Plan pl) {
    using Tr = PathTraits<MODE>;
    __shared__ TailShared sh;
    const Role role = decode_role(pl.grid, static_cast<int32_t>(blockIdx.x));
    int b = role.seq;
    switch (role.kind) {
        case kDecWorker: {
            if constexpr (Tr::loss) {
                // Step n: the block's waves take chunk pairs base + n*4 + wave
                // (pair index li = i * P + c); the words go out after both
                // steps' loads (see stream_segment).
                static_assert(kChunksPerWave <= 2, "two steps at most");
                const int items = pl.dec_rows * pl.chunks;
                const int li0 = role.index * kWavesPerBlock * pl.nc_dec + static_cast<int>(threadIdx.x / kWave);
                const int li1 = li0 + kWavesPerBlock;
                const bool has1 = pl.nc_dec > 1 && li1 < items;
                if (li0 < items) {
                    const PairPart p0 = stream_pair<EB, VEC>(pl, b, li0 / pl.chunks, li0 % pl.chunks);
                    PairPart p1 = p0;
                    if (has1) p1 = stream_pair<EB, VEC>(pl, b, li1 / pl.chunks, li1 % pl.chunks);
                    if ((threadIdx.x & (kWave - 1)) == 0) {
                        put_pair(pl, b, li0, p0);
                        if (has1) put_pair(pl, b, li1, p1);
                    }
                }
            } else {
                // Block `index` of sequence b: segment index % S of local
                // row index / S.  When every decision worker block comes
                // before every finisher (one residency), the blocks are
                // taken position-major over all sequences instead, so that
                // the rows of early positions arrive first and decisions
                // that stop at an early rejection finish while the rest
                // streams.
                int idx = role.index;
                if (pl.pos_major) {
                    const int64_t q = static_cast<int64_t>(b) * pl.grid.w_dec + idx;
                    const int64_t t = q / pl.segs;
                    const int s = static_cast<int>(q - t * pl.segs);
                    b = static_cast<int>(t % pl.batch);
                    idx = static_cast<int>(t / pl.batch) * pl.segs + s;
                }
                const int j = idx / pl.segs;
                const int s = idx - j * pl.segs;
                // Window mode: the row of position j >= window is not read
                // after a known rejection before it, and beyond the
                // read-ahead only once released.
                if (Tr::bonus && Tr::halves == 1 && pl.window && j >= pl.window) {
                    int known;
                    const int ahead = read_ahead(pl, b, sh, known);
                    if (known < j || (j > ahead && released(pl, b, j, sh) == 0)) return;
                }
                stream_segment<EB, VEC, MODE>(pl, b, j, s, sh);
            }
            return;
        }
        case kBonusWorker:
            if constexpr (Tr::bonus) bonus_worker<EB, VEC, MODE>(pl, b, role.index, sh);
            return;
        case kDecFinisher:
            if constexpr (Tr::loss) vat_loss_finisher<EB, VEC>(pl, b, sh);
            else decision_finisher<EB, VEC, MODE>(pl, b, sh);
            return;
        case kResWorker:
            if constexpr (Tr::resid) residual_worker<EB, VEC, MODE>(pl, b, role.index, sh);
            return;
        case kResFinisher:
            if constexpr (Tr::resid) residual_finisher<EB, VEC, MODE>(pl, b, sh);
            return;
        default:
            if constexpr (Tr::bonus) bonus_finisher<EB, VEC, MODE>(pl, b, sh);
            return;
    }
}

// ------------------------------------------------------------------ dispatch

template <int EB, bool VEC, int MODE>
hipError_t launch_typed(const Plan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    hipError_t e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev0, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_verify<EB, VEC, MODE>), dim3(static_cast<unsigned>(pl.grid.total_blocks)), dim3(kBlock), 0,
                       stream, pl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev1, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int EB, bool VEC>
hipError_t launch_mode(const Plan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    switch (pl.path) {
        case kPathSample: return launch_typed<EB, VEC, kPathSample>(pl, stream, ev0, ev1);
        case kPathOneHot: return launch_typed<EB, VEC, kPathOneHot>(pl, stream, ev0, ev1);
        case kPathGreedy: return launch_typed<EB, VEC, kPathGreedy>(pl, stream, ev0, ev1);
        case kPathVat: return launch_typed<EB, VEC, kPathVat>(pl, stream, ev0, ev1);
        case kPathVatGreedy: return launch_typed<EB, VEC, kPathVatGreedy>(pl, stream, ev0, ev1);
        case kPathVatLoss: return launch_typed<EB, VEC, kPathVatLoss>(pl, stream, ev0, ev1);
        default: return hipErrorInvalidValue;
    }
}

template <int EB, bool VEC, int MODE>
int blocks_per_cu_typed() {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_verify<EB, VEC, MODE>, kBlock, 0) != hipSuccess) return 0;
    return n;
}

template <int EB, bool VEC>
int blocks_per_cu_mode(int path) {
    switch (path) {
        case kPathSample: return blocks_per_cu_typed<EB, VEC, kPathSample>();
        case kPathOneHot: return blocks_per_cu_typed<EB, VEC, kPathOneHot>();
        case kPathGreedy: return blocks_per_cu_typed<EB, VEC, kPathGreedy>();
        case kPathVat: return blocks_per_cu_typed<EB, VEC, kPathVat>();
        case kPathVatGreedy: return blocks_per_cu_typed<EB, VEC, kPathVatGreedy>();
        case kPathVatLoss: return blocks_per_cu_typed<EB, VEC, kPathVatLoss>();
        default: return 0;
    }
}

}  // namespace

// ------------------------------------------------------------------ VAT loss gradient

namespace {

// d(block loss)/d l_d(y) = w_i/T ((1 + lambda) q(y) - p(y) - lambda [y == h_i])
// for one (row, chunk) item per wavefront, in blocks of two wavefronts, one
// item each: the shape of the plain two-reads-one-write stream that ran
// fastest, with the chunk's loads all in flight before its first store and
// few enough registers for many wavefronts per SIMD.  p and q come from the
// logits and the row statistics (m/T, Z) that sv_vat_loss wrote:
// p(y) = 2^(l(y) c2 - (m/T) log2(e)) / Z.  A row of weight 0 is written as
// zeros without reading its logits.
constexpr int kGradBlock = 128;
constexpr int kGradWaves = kGradBlock / kWave;

template <int EB, bool VEC>
__global__ __launch_bounds__(kGradBlock) void k_vat_grad(GradPlan g) {
    constexpr int PV = Elem<EB>::kPerVec;
    constexpr int CH = Chunk<EB>::kElems;
    const int lane = threadIdx.x & (kWave - 1);
    // the item is the wavefront's: row parameters come through scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int64_t item = static_cast<int64_t>(blockIdx.x) * kGradWaves + wave;
    if (item >= g.items) return;
    int64_t row;
    int c;
    if (g.items <= INT_MAX) {
        const uint32_t it = static_cast<uint32_t>(item), nc = static_cast<uint32_t>(g.chunks);
        const uint32_t r32 = it / nc;
        row = r32;
        c = static_cast<int>(it - r32 * nc);
    } else {
        row = item / g.chunks;
        c = static_cast<int>(item - row * g.chunks);
    }
    const int64_t V = g.vocab;
    const float log2e = 1.4426950408889634f;
    const int start = c * CH;
    const int len = min(CH, static_cast<int>(V) - start);
    float* const out = g.grad + row * V + start;
    // the row's parameters, all loads issued together before the first use
    const float w = g.weights[row];
    const float2 st = *reinterpret_cast<const float2*>(g.row_stats + 2 * row);
    const float2 sd = *reinterpret_cast<const float2*>(g.row_stats + 2 * (g.rows + row));
    const int hard = g.hard[row];
    // an empty statement that takes all five: the loads are not sunk below
    // the weight test, so one wait covers them
    asm volatile("" ::"s"(w), "s"(st.x), "s"(st.y), "s"(sd.x), "s"(sd.y), "s"(hard));
    const float s = w * g.inv_t;
    const float aq = s * (1.f + g.hard_weight), hh = s * g.hard_weight;
    const float mt2 = st.x * log2e, izt = 1.f / st.y;
    const float md2 = sd.x * log2e, izd = 1.f / sd.y;
    const int64_t hard_at = static_cast<int64_t>(hard) - start;
    const int hx = hard_at >= 0 && hard_at < CH ? static_cast<int>(hard_at) : -1;  // its place in the chunk
    const auto grad_of = [&](float lt, float ld, int idx) {
        const float p = exp2_hw(fmaf(lt, g.c2, -mt2)) * izt;
        const float q = exp2_hw(fmaf(ld, g.c2, -md2)) * izd;
        return fmaf(aq, q, -s * p) - (idx == hx ? hh : 0.f);
    };
    const char* rt = row_base(g.target, row, V, EB) + static_cast<int64_t>(start) * EB;
    const char* rd = row_base(g.draft, row, V, EB) + static_cast<int64_t>(start) * EB;
    if constexpr (VEC) {
        typedef float f32x4_t __attribute__((ext_vector_type(4)));
        const int nvec = len / PV;
        const uint4* pt = reinterpret_cast<const uint4*>(rt);
        const uint4* pd = reinterpret_cast<const uint4*>(rd);
        f32x4_t* dst = reinterpret_cast<f32x4_t*>(out);
        if (w == 0.f) {
            const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                const int idx = j * kWave + lane;
                if (idx < nvec) {
#pragma unroll
                    for (int e = 0; e < PV; e += 4) __builtin_nontemporal_store(z, dst + (idx * PV + e) / 4);
                }
            }
            return;
        }
        // a whole chunk (every row's but the last) takes no per-vector tests,
        // so its loads issue back to back
        const auto run = [&](auto whole) {
            constexpr bool kWhole = decltype(whole)::value;
            uint4 at[kVecPerLane], ad[kVecPerLane];
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                const int idx = j * kWave + lane;
                at[j] = kWhole || idx < nvec ? load_stream(pt + idx) : make_uint4(0u, 0u, 0u, 0u);
                ad[j] = kWhole || idx < nvec ? load_stream(pd + idx) : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                const int idx = j * kWave + lane;
                if (!kWhole && idx >= nvec) continue;
                float ft[PV], fd[PV];
                Elem<EB>::decode(at[j], ft);
                Elem<EB>::decode(ad[j], fd);
#pragma unroll
                for (int e = 0; e < PV; e += 4) {
                    const f32x4_t v = {grad_of(ft[e], fd[e], idx * PV + e),
                                       grad_of(ft[e + 1], fd[e + 1], idx * PV + e + 1),
                                       grad_of(ft[e + 2], fd[e + 2], idx * PV + e + 2),
                                       grad_of(ft[e + 3], fd[e + 3], idx * PV + e + 3)};
                    __builtin_nontemporal_store(v, dst + (idx * PV + e) / 4);
                }
            }
        };
        if (nvec == kWave * kVecPerLane)
            run(std::true_type{});
        else
            run(std::false_type{});
    } else {
        for (int e = 0; e < Chunk<EB>::kPerLane; ++e) {
            const int idx = e * kWave + lane;
            if (idx >= len) break;
            out[idx] = w != 0.f ? grad_of(Elem<EB>::at(rt, idx), Elem<EB>::at(rd, idx), idx) : 0.f;
        }
    }
}

template <int EB, bool VEC>
hipError_t launch_grad_typed(const GradPlan& g, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    const int64_t blocks = (g.items + kGradWaves - 1) / kGradWaves;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipError_t e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev0, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_vat_grad<EB, VEC>), dim3(static_cast<unsigned>(blocks)), dim3(kGradBlock), 0, stream, g);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev0 && ev1) e = hipEventRecord(ev1, stream);
    return e;
}

}  // namespace

hipError_t launch_vat_grad(const GradPlan& g, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (g.items == 0) return hipSuccess;
    if (g.elem_bytes == 2)
        return g.vec ? launch_grad_typed<2, true>(g, stream, ev0, ev1) : launch_grad_typed<2, false>(g, stream, ev0, ev1);
    return g.vec ? launch_grad_typed<4, true>(g, stream, ev0, ev1) : launch_grad_typed<4, false>(g, stream, ev0, ev1);
}

// ------------------------------------------------------------------ acceptance telemetry

namespace {

// Counts of the accepted lengths of one call: bins 0..k, then -1 (invalid
// token), -2 (wait timed out), anything else.  One block; integer LDS
// atomics, so the counts are exact.
__global__ __launch_bounds__(kBlock) void k_accept_hist(const int32_t* acc, int32_t batch, int32_t k, int32_t* hist) {
    __shared__ int counts[kMaxDraft + 4];
    const int nb = k + 4;
    for (int j = threadIdx.x; j < nb; j += kBlock) counts[j] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < batch; i += kBlock) {
        const int v = acc[i];
        const int bin = (v >= 0 && v <= k) ? v : (v == -1 ? k + 1 : (v == -2 ? k + 2 : k + 3));
        atomicAdd(&counts[bin], 1);
    }
    __syncthreads();
    for (int j = threadIdx.x; j < nb; j += kBlock) hist[j] = counts[j];
}

}  // namespace

hipError_t launch_accept_hist(const int32_t* acc, int32_t batch, int32_t k, int32_t* hist, hipStream_t stream) {
    hipLaunchKernelGGL(k_accept_hist, dim3(1), dim3(kBlock), 0, stream, acc, batch, k, hist);
    return hipGetLastError();
}

int verify_blocks_per_cu(int elem_bytes, bool vec, int path) {
    if (elem_bytes == 2) return vec ? blocks_per_cu_mode<2, true>(path) : blocks_per_cu_mode<2, false>(path);
    return vec ? blocks_per_cu_mode<4, true>(path) : blocks_per_cu_mode<4, false>(path);
}

// ------------------------------------------------------------------ built-in scratch

namespace {

// The workspace of sv_verify_noalloc: one array per device, in the code
// object's own device memory, held until the process ends.  Host code never
// uses the array's name as an address (it is a host-side stand-in): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Zero-fill of a buffer of 16-byte words (the scratch starts at zero, so
// that no hand-off word in it carries a live call tag).
__global__ __launch_bounds__(kBlock) void k_fill_zero(uint4* p, int64_t n) {
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kBlock)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kMaxScratchDevices = 64;

struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};

ScratchSlot g_scratch[kMaxScratchDevices];

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&] {
        void* p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err != hipSuccess) return;
        // Cleared once with a kernel on the first call's stream, ordered
        // before that call's own launch; later calls leave it ready (tags).
        constexpr int64_t n = kNoAllocScratchBytes / 16;
        hipLaunchKernelGGL(k_fill_zero, dim3(1024), dim3(kBlock), 0, stream, static_cast<uint4*>(p), n);
        slot.err = hipGetLastError();
        if (slot.err == hipSuccess) slot.ptr = p;
    });
    if (slot.err != hipSuccess) return slot.err;
    *ptr = slot.ptr;
    return hipSuccess;
}

hipError_t launch_path(const Plan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (pl.batch == 0) return hipSuccess;
    if (pl.elem_bytes == 2) {
        return pl.vec ? launch_mode<2, true>(pl, stream, ev0, ev1) : launch_mode<2, false>(pl, stream, ev0, ev1);
    }
    return pl.vec ? launch_mode<4, true>(pl, stream, ev0, ev1) : launch_mode<4, false>(pl, stream, ev0, ev1);
}

}  // namespace sv
