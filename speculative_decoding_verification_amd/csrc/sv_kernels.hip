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
// Kernels (one call: k_stream, then k_residual when draft logits are read at
// T > 0):
//  k_stream    the HBM-bound pass.  Worker blocks: one wavefront per (row,
//              8 KiB chunk), sequence-major, 16-byte coalesced loads, the
//              chunk's max and sum of exp2((l - m) * log2(e)/T) (or, at T == 0,
//              max and lowest index), wave butterfly reductions, one partial
//              handed off as tagged words; workers never wait.  Finisher
//              blocks, one per sequence, sit in the same grid about one
//              residency behind their sequence's workers, so they run while
//              later sequences stream: poll and stage the partials in LDS,
//              combine them into (m, Z) per row, p(x_i) and q(x_i), the test
//              u*q < p on one lane per position, wave ballot -> first rejection
//              r, accepted prefix or VAT labels and weights, and the draw
//              itself when it needs no second pass over the logits (bonus token
//              from the chunk masses; one-hot residual = p_r without x_r).
//  k_residual  only for draft logits at T > 0: worker blocks compute the
//              residual mass max(0, p_r - q_r) of each chunk of a rejected row
//              pair; the sequence's finisher block draws the token.
//
// Draws: block prefix scan over the chunk masses finds the chunk holding the
// draw, then an LDS block scan of that one chunk finds the token.  No
// floating-point atomics and fixed reduction orders: bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>

#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kMaxDraft = 64;

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
            for (int j = 0; j < kVecPerLane; ++j) raw[j] = p[j * kWave + lane];
        } else {
            const int nvec = len / PV;  // rows are whole vectors on this path
            const uint32_t ni = Elem<EB>::kNegInfWord;
#pragma unroll
            for (int j = 0; j < kVecPerLane; ++j) {
                const int idx = j * kWave + lane;
                raw[j] = idx < nvec ? p[idx] : make_uint4(ni, ni, ni, ni);
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

// Global row of local row j of sequence b (j < n_t: target position j; else
// draft position j - n_t).
__device__ __forceinline__ int64_t global_row(const Plan& pl, int b, int j) {
    const int n_t = pl.target_rows_per_seq;
    return j < n_t ? static_cast<int64_t>(b) * n_t + j : pl.rows_t + static_cast<int64_t>(b) * pl.k + (j - n_t);
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
__device__ __forceinline__ uint32_t canon_nan(uint32_t bits) {
    return ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu)) ? 0x7fc00000u : bits;
}

__device__ __forceinline__ void put_word(uint64_t* p, uint32_t data, uint32_t tag) {
    __hip_atomic_store(p, (static_cast<uint64_t>(tag) << 32) | data, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t get_word(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t word_data(uint64_t w) { return static_cast<uint32_t>(w); }

// Chunk partial i of a sequence: words 2i (m or max) and 2i+1 (s or index).
__device__ __forceinline__ void put_partial(uint64_t* seq_words, int i, float2 v, bool index_in_y, uint32_t tag) {
    put_word(seq_words + 2 * i, canon_nan(__float_as_uint(v.x)), tag);
    put_word(seq_words + 2 * i + 1, index_in_y ? __float_as_uint(v.y) : canon_nan(__float_as_uint(v.y)), tag);
}

// A finisher gives up after about a second of polling (the wall clock runs at
// 100 MHz): it cannot happen when blocks are dispatched in grid order, and it
// turns any other case into an error code instead of a hung kernel.
constexpr uint64_t kPollTimeoutTicks = 1ull << 27;

// Polls the n words at `words` until all carry `tag`; with `stage` (n <=
// kStageWords) their data is left in stage[0..n).  Whole block.  Returns
// false on timeout.
__device__ bool collect(const uint64_t* words, int n, uint32_t tag, uint32_t* stage) {
    const uint64_t t0 = wall_clock64();
    for (;;) {
        int missing = 0;
        for (int i = threadIdx.x; i < n; i += kBlock) {
            const uint64_t w = get_word(words + i);
            if (static_cast<uint32_t>(w >> 32) != tag) missing = 1;
            else if (stage) stage[i] = word_data(w);
        }
        if (!__syncthreads_or(missing)) return true;
        if (wall_clock64() - t0 > kPollTimeoutTicks) return false;
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

// Block roles of a grid with W worker blocks per sequence and one finisher
// block per sequence, the finisher of sequence b placed after the workers of
// sequence b + L (or at the end).  With blocks dispatched in grid order, all
// workers a finisher waits for were dispatched before it.
struct Role {
    int seq;
    int worker;  // worker index within the sequence, -1 for the finisher
};

__device__ __forceinline__ Role decode_role(int64_t blk, int B, int W, int L) {
    const int64_t head = static_cast<int64_t>(L) * W;
    Role r;
    if (blk < head) {
        r.seq = static_cast<int>(blk / W);
        r.worker = static_cast<int>(blk - static_cast<int64_t>(r.seq) * W);
        return r;
    }
    const int64_t rel = blk - head;
    const int64_t mid = static_cast<int64_t>(B - L) * (W + 1);
    if (rel < mid) {
        const int g = L + static_cast<int>(rel / (W + 1));
        const int pos = static_cast<int>(rel - static_cast<int64_t>(g - L) * (W + 1));
        if (pos < W) {
            r.seq = g;
            r.worker = pos;
        } else {
            r.seq = g - L;
            r.worker = -1;
        }
        return r;
    }
    r.seq = B - L + static_cast<int>(rel - mid);
    r.worker = -1;
    return r;
}

struct TailShared {
    uint32_t stage[kStageWords];   // staged hand-off words
    float2 mz[2 * kMaxDraft + 1];  // (m, Z) or (max, argmax) of the sequence's rows
    float wt[kWavesPerBlock];      // block scan scratch
    float prev_mass;               // running mass before the selected chunk
    float u_draw;
    int sel;
    int last_pos;
    int r;
    int mode;
    int x_r;
};

// ------------------------------------------------------------------ sampling

struct ResidW {
    float c2, mt, izt, md, izd;  // mt, md: row max * c2 (rounded); izt, izd: corr / Z
    __device__ __forceinline__ float operator()(float lt, float ld) const {
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
__device__ DrawPick draw_select(const DrawRow& d, float u, int P, int64_t V, TailShared& sh) {
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
            if (v > 0.f) atomicMax(&sh.last_pos, c);
        }
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
__device__ int draw_scan(const DrawPick& pk, const float (&w)[Chunk<EB>::kPerThread], TailShared& sh) {
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
    if (tid == 0) {
        sh.sel = INT_MAX;
        sh.last_pos = -1;
    }
    __syncthreads();
    float prefix = 0.f;
#pragma unroll
    for (int q = 0; q < kWavesPerBlock; ++q)
        if (q < wave) prefix += sh.wt[q];
    const float excl = prefix + dpp<kDppWaveShr1>(0.f, incl);
    if (my_last >= 0) atomicMax(&sh.last_pos, my_last);
    if (!pk.open_end && excl + my_sum > pk.th) {
        float run = excl;
        int pick = -1;
#pragma unroll
        for (int e = 0; e < PT; ++e) {
            run += w[e];
            if (pick < 0 && w[e] > 0.f && run > pk.th) pick = tid * PT + e;
        }
        if (pick >= 0) atomicMin(&sh.sel, pick);
    }
    __syncthreads();
    const int y = sh.sel != INT_MAX ? sh.sel : (sh.last_pos >= 0 ? sh.last_pos : 0);
    __syncthreads();
    return pk.cs * CH + y;
}

// The chunk of a draw from `d`: one wave-level pick when P <= 64, else the
// tiled block-level selection.  Whole block.
template <int EB, bool VEC>
__device__ DrawPick pick_chunk(const DrawRow& d, float u, int P, int64_t V, TailShared& sh) {
    constexpr int CH = Chunk<EB>::kElems;
    constexpr int PT = Chunk<EB>::kPerThread;
    if (P > kWave) return draw_select<EB, VEC>(d, u, P, V, sh);
    int cx = -1;
    float mass_cx = 0.f;
    if (d.mode == kModeOneHot) {
        cx = d.excl / CH;
        float lt[PT], ld[PT], w[PT];
        load_runs<EB, VEC>(d, cx, V, lt, ld);
        run_weights<EB>(d, static_cast<int64_t>(cx) * CH, lt, ld, w);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < PT; ++e) sum += w[e];
        mass_cx = block_sum(sum, sh.wt);
    }
    const int lane = threadIdx.x & (kWave - 1);
    const float mass = lane < P ? chunk_mass(d, lane, cx, mass_cx) : 0.f;
    DrawPick pk = wave_pick(mass, u, P);
    pk.cx = cx;
    pk.mass_cx = mass_cx;
    return pk;
}

// Draws one token from the weights of `d` with uniform u.  Whole block.
template <int EB, bool VEC>
__device__ int draw_token(const DrawRow& d, float u, int P, int64_t V, TailShared& sh) {
    constexpr int CH = Chunk<EB>::kElems;
    constexpr int PT = Chunk<EB>::kPerThread;
    const DrawPick pk = pick_chunk<EB, VEC>(d, u, P, V, sh);
    float lt[PT], ld[PT], w[PT];
    load_runs<EB, VEC>(d, pk.cs, V, lt, ld);
    run_weights<EB>(d, static_cast<int64_t>(pk.cs) * CH, lt, ld, w);
    return draw_scan<EB>(pk, w, sh);
}

// ------------------------------------------------------------------ sequence tail

// Outputs of a sequence whose finisher timed out waiting for its workers.
__device__ void fail_sequence(const Plan& pl, int b) {
    const int k = pl.k;
    for (int j = threadIdx.x; j <= k; j += kBlock) {
        if (pl.vat) {
            if (j < k) {
                pl.mask[static_cast<int64_t>(b) * k + j] = 0;
                pl.weights[static_cast<int64_t>(b) * k + j] = 0.f;
            }
        } else {
            pl.out_tokens[static_cast<int64_t>(b) * (k + 1) + j] = -1;
        }
    }
    if (threadIdx.x == 0) {
        if (pl.vat) {
            pl.first_reject[b] = -2;
        } else {
            pl.accepted_len[b] = -2;
            ResidJob job{};
            job.r = -2;
            job.mode = kModeDone;
            pl.jobs[b] = job;
        }
    }
}

// Row (m, Z) -- or (max, argmax) at T == 0 -- of local row j from its chunk
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
    if (P <= kWave) {
        if (lane < P) {
            const float2 pc = src.get(j * P + lane);
            m = pc.x;
            s = pc.y;
        }
    } else {
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
    }
    wave_merge_ms(m, s, c2);
    return make_float2(m, s);
}

// Everything after the streaming pass for sequence b, run by its finisher block.
template <int EB, bool VEC>
__device__ void finish_sequence(const Plan& pl, int b, TailShared& sh) {
    constexpr int CH = Chunk<EB>::kElems;
    constexpr int PT = Chunk<EB>::kPerThread;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int k = pl.k;
    const int n_t = pl.target_rows_per_seq;
    const int R_s = pl.rows_per_seq;
    const int P = pl.chunks;
    const int64_t V = pl.vocab;
    const float c2 = pl.c2;
    const int n_u = pl.vat ? k : k + 1;
    const int items = R_s * P;
    const uint64_t* words = pl.partials + static_cast<int64_t>(b) * items * 2;
    const bool sampling = !pl.vat && !pl.greedy;

    // Loads that do not depend on the partials go out before the polling, all
    // issued back to back (no branch on a loaded value): one lane per position
    // loads its token, uniform and the two logits at the token (index clamped
    // into the row; an invalid token flags the sequence below).
    const bool active = wave == 0 && lane < k;
    int x = 0;
    float lt = 0.f, ld = 0.f, u = 0.f;
    if (active) {
        x = pl.tokens[static_cast<int64_t>(b) * k + lane];
        if (!pl.greedy) u = pl.uniforms[static_cast<int64_t>(b) * n_u + lane];
    }
    const bool bad = active && (x < 0 || x >= pl.vocab);
    if (active && !pl.greedy) {
        const int xc = min(max(x, 0), pl.vocab - 1);
        lt = Elem<EB>::at(row_base(pl.target, static_cast<int64_t>(b) * n_t + lane, V, EB), xc);
        if (!pl.onehot) ld = Elem<EB>::at(row_base(pl.draft, static_cast<int64_t>(b) * k + lane, V, EB), xc);
    }
    const float u_draw = sampling ? pl.uniforms[static_cast<int64_t>(b) * (k + 1) + k] : 0.f;

    const bool staged = 2 * items <= kStageWords;
    if (!collect(words, 2 * items, pl.tag, staged ? sh.stage : nullptr)) {
        fail_sequence(pl, b);
        return;
    }
    const PartialSrc src{staged ? sh.stage : nullptr, words};

    // Combine the chunk partials of every row of the sequence.
    for (int j = wave; j < R_s; j += kWavesPerBlock) {
        const float2 res = combine_row(src, j, P, pl.greedy, c2);
        if (lane == 0) {
            const int64_t grow = global_row(pl, b, j);
            sh.mz[j] = res;
            pl.row_mz[grow] = res;
            if (pl.row_stats_out) {
                pl.row_stats_out[2 * grow] = pl.greedy ? res.x : res.x / pl.temperature;
                pl.row_stats_out[2 * grow + 1] = pl.greedy ? static_cast<float>(__float_as_int(res.y)) : res.y;
            }
        }
    }
    __syncthreads();

    // The bonus token (drawn from target row k if all k drafts are kept) needs
    // only row k's partials: pick its chunk now and start loading that chunk,
    // so the loads overlap the accept decisions below.
    DrawRow db;
    DrawPick pb;
    float lt_b[PT], ld_b[PT];
    if (sampling) {
        db.mode = kModeBonus;
        db.rt = row_base(pl.target, static_cast<int64_t>(b) * n_t + k, V, EB);
        db.rd = nullptr;
        db.part = src;
        db.part_base = k * P;
        db.rstage = nullptr;
        db.rwords = nullptr;
        db.c2 = c2;
        db.mrow = sh.mz[k].x;
        db.mt = row_scale(db.mrow, c2, db.corr);
        db.excl = -1;
        pb = pick_chunk<EB, VEC>(db, u_draw, P, V, sh);
        load_runs<EB, VEC>(db, pb.cs, V, lt_b, ld_b);
    }

    if (wave == 0) {
        const int i = lane;
        const bool invalid = __ballot(bad) != 0ull;
        bool keep = false;
        float p = __builtin_nanf(""), q = __builtin_nanf("");
        if (!invalid && active) {
            if (pl.greedy) {
                keep = (x == __float_as_int(sh.mz[i].y));
                p = keep ? 1.f : 0.f;
                q = 1.f;
            } else {
                // The test u*q < p, taken in the log2 domain so that
                // probabilities below the fp32 range still decide correctly.
                const float lp = (lt - sh.mz[i].x) * c2 - log2_hw(sh.mz[i].y);
                const float lq = pl.onehot ? 0.f : (ld - sh.mz[n_t + i].x) * c2 - log2_hw(sh.mz[n_t + i].y);
                keep = log2_hw(u) + lq < lp;
                p = exp2_hw(lp);
                q = exp2_hw(lq);
            }
        }
        const uint64_t kept = __ballot(keep);
        const uint64_t lowk = (k == 64) ? ~0ull : ((1ull << k) - 1ull);
        const uint64_t rej = ~kept & lowk;
        const int r = invalid ? -1 : (rej ? __builtin_ctzll(rej) : k);

        if (pl.probs_out && active) {
            pl.probs_out[2 * (static_cast<int64_t>(b) * k + i)] = p;
            pl.probs_out[2 * (static_cast<int64_t>(b) * k + i) + 1] = q;
        }
        int mode = kModeDone;
        if (pl.vat) {
            if (active) {
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
            if (!invalid && !pl.greedy) mode = r == k ? kModeBonus : (pl.onehot ? kModeOneHot : kModeResidual);
            const int x_r = (r >= 0 && r < k) ? __builtin_amdgcn_readlane(x, r) : -1;
            const int g_r = (pl.greedy && r >= 0) ? __float_as_int(sh.mz[r].y) : -1;
            int32_t* out = pl.out_tokens + static_cast<int64_t>(b) * (k + 1);
            for (int j = lane; j <= k; j += kWave) {
                int val = -1;
                if (!invalid) {
                    if (j < r) val = x;          // j < r <= k <= 64 here, so j == lane
                    else if (j == r) val = g_r;  // T > 0: the draw overwrites it
                }
                out[j] = val;
            }
            if (lane == 0) {
                pl.accepted_len[b] = r;
                ResidJob job{};
                job.r = r;
                job.mode = mode;
                if (mode == kModeResidual) {
                    job.u = u_draw;
                    job.mzt = sh.mz[r];
                    job.mzd = sh.mz[n_t + r];
                }
                pl.jobs[b] = job;
                sh.r = r;
                sh.x_r = x_r;
            }
        }
        if (lane == 0) sh.mode = mode;
    }
    __syncthreads();

    const int mode = sh.mode;
    if (mode == kModeBonus) {
        float w[PT];
        run_weights<EB>(db, static_cast<int64_t>(pb.cs) * CH, lt_b, ld_b, w);
        const int y = draw_scan<EB>(pb, w, sh);
        if (threadIdx.x == 0) pl.out_tokens[static_cast<int64_t>(b) * (k + 1) + k] = y;
    } else if (mode == kModeOneHot) {
        const int r = sh.r;
        DrawRow d;
        d.mode = kModeOneHot;
        d.rt = row_base(pl.target, static_cast<int64_t>(b) * n_t + r, V, EB);
        d.rd = nullptr;
        d.part = src;
        d.part_base = r * P;
        d.rstage = nullptr;
        d.rwords = nullptr;
        d.c2 = c2;
        d.mrow = sh.mz[r].x;
        d.mt = row_scale(d.mrow, c2, d.corr);
        d.excl = sh.x_r;
        const int y = draw_token<EB, VEC>(d, u_draw, P, V, sh);
        if (threadIdx.x == 0) pl.out_tokens[static_cast<int64_t>(b) * (k + 1) + r] = y;
    }
}

// ------------------------------------------------------------------ kernels

template <int EB, bool VEC>
__global__ __launch_bounds__(kBlock) void k_stream(Plan pl) {
    __shared__ TailShared sh;
    const Role role = decode_role(blockIdx.x, pl.batch, pl.wg_per_seq_a, pl.lag_a);
    const int b = role.seq;
    if (role.worker >= 0) {
        const int lane = threadIdx.x & (kWave - 1);
        const int P = pl.chunks;
        const int items = pl.rows_per_seq * P;
        const int li = role.worker * kWavesPerBlock + static_cast<int>(threadIdx.x / kWave);
        if (li >= items) return;
        const int j = li / P;
        const int c = li - j * P;
        const char* rp = row_of<EB>(pl, global_row(pl, b, j));
        const int64_t start = static_cast<int64_t>(c) * Chunk<EB>::kElems;
        const int len = static_cast<int>(min(static_cast<int64_t>(Chunk<EB>::kElems), pl.vocab - start));
        const float2 part = pl.greedy ? chunk_argmax<EB, VEC>(rp, start, len, lane)
                                      : chunk_stats<EB, VEC>(rp, start, len, lane, pl.c2);
        if (lane == 0) put_partial(pl.partials + static_cast<int64_t>(b) * items * 2, li, part, pl.greedy, pl.tag);
        return;
    }
    finish_sequence<EB, VEC>(pl, b, sh);
}

// Residual mass of each chunk of a rejected row pair; the sequence's finisher
// block draws the token.
template <int EB, bool VEC>
__global__ __launch_bounds__(kBlock) void k_residual(Plan pl) {
    __shared__ TailShared sh;
    const Role role = decode_role(blockIdx.x, pl.batch, pl.wg_per_seq_b, pl.lag_b);
    const int b = role.seq;
    const ResidJob job = pl.jobs[b];
    if (job.mode != kModeResidual) return;  // workers and finisher of the sequence agree
    const int P = pl.chunks;
    const int k = pl.k;
    const int64_t V = pl.vocab;
    const int64_t trow = static_cast<int64_t>(b) * pl.target_rows_per_seq + job.r;
    const int64_t drow = static_cast<int64_t>(b) * k + job.r;
    const ResidW wf = make_resid_w(job.mzt, job.mzd, pl.c2);
    uint64_t* rwords = pl.resid + static_cast<int64_t>(b) * P;
    if (role.worker >= 0) {
        const int lane = threadIdx.x & (kWave - 1);
        const int c = role.worker * kWavesPerBlock + static_cast<int>(threadIdx.x / kWave);
        if (c >= P) return;
        const int64_t start = static_cast<int64_t>(c) * Chunk<EB>::kElems;
        const int len = static_cast<int>(min(static_cast<int64_t>(Chunk<EB>::kElems), V - start));
        float vt[Chunk<EB>::kPerLane];
        float vd[Chunk<EB>::kPerLane];
        load_chunk<EB, VEC>(row_base(pl.target, trow, V, EB), start, len, lane, vt);
        load_chunk<EB, VEC>(row_base(pl.draft, drow, V, EB), start, len, lane, vd);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < Chunk<EB>::kPerLane; ++e) s += wf(vt[e], vd[e]);
        s = wave_sum(s);
        if (lane == 0) put_word(rwords + c, canon_nan(__float_as_uint(s)), pl.tag);
        return;
    }
    const bool staged = P <= kStageWords;
    if (!collect(rwords, P, pl.tag, staged ? sh.stage : nullptr)) {
        fail_sequence(pl, b);
        return;
    }
    DrawRow d;
    d.mode = kModeResidual;
    d.rt = row_base(pl.target, trow, V, EB);
    d.rd = row_base(pl.draft, drow, V, EB);
    d.part = PartialSrc{nullptr, pl.partials + static_cast<int64_t>(b) * pl.rows_per_seq * P * 2};
    d.part_base = job.r * P;
    d.rstage = staged ? sh.stage : nullptr;
    d.rwords = rwords;
    d.c2 = pl.c2;
    d.mrow = job.mzt.x;
    d.mt = row_scale(job.mzt.x, pl.c2, d.corr);
    d.excl = -1;
    d.rw = wf;
    // A residual that rounds to zero mass (only possible through rounding,
    // since a rejection has probability TV(p, q)): draw from p_r instead.
    float zsum = 0.f;
    for (int cc = threadIdx.x; cc < P; cc += kBlock) zsum += chunk_mass(d, cc, -1, 0.f);
    if (!__syncthreads_or(zsum > 0.f)) d.mode = kModeBonus;
    const int y = draw_token<EB, VEC>(d, job.u, P, V, sh);
    if (threadIdx.x == 0) pl.out_tokens[static_cast<int64_t>(b) * (k + 1) + job.r] = y;
}

// ------------------------------------------------------------------ dispatch

template <int EB, bool VEC>
hipError_t launch_typed(const Plan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    hipError_t e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev0, stream);
        if (e != hipSuccess) return e;
    }
    const unsigned grid_a = static_cast<unsigned>(static_cast<int64_t>(pl.batch) * (pl.wg_per_seq_a + 1));
    hipLaunchKernelGGL((k_stream<EB, VEC>), dim3(grid_a), dim3(kBlock), 0, stream, pl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev1, stream);
        if (e != hipSuccess) return e;
    }
    if (pl.vat || pl.greedy || pl.onehot) return hipSuccess;
    const unsigned grid_b = static_cast<unsigned>(static_cast<int64_t>(pl.batch) * (pl.wg_per_seq_b + 1));
    hipLaunchKernelGGL((k_residual<EB, VEC>), dim3(grid_b), dim3(kBlock), 0, stream, pl);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_path(const Plan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    if (pl.batch == 0) return hipSuccess;
    if (pl.elem_bytes == 2) {
        return pl.vec ? launch_typed<2, true>(pl, stream, ev0, ev1) : launch_typed<2, false>(pl, stream, ev0, ev1);
    }
    return pl.vec ? launch_typed<4, true>(pl, stream, ev0, ev1) : launch_typed<4, false>(pl, stream, ev0, ev1);
}

}  // namespace sv
