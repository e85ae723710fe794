// gfx950 (CDNA4) kernels of libspecverify.
//
// Path (batched verification, NgramRL essay "AI 开始抄自己的作业", section
// "投机解码：让草稿先跑，考官殿后"; VAT write-up "让AI草稿模型学会“照镜子”",
// sections "VAT怎么把“验收规则”塞进训练里" and "第二件事，改权重分配的锚点"):
//
//  k_row_stats     one wavefront per (row, 8 KiB chunk): 16-byte coalesced
//                  loads, chunk max and sum of exp2((l - m) * log2e/T), wave
//                  butterfly reductions, one (m, s) partial per chunk.  This is
//                  the kernel that streams every logit once (HBM bound).
//  k_row_argmax    T == 0: the same stream, (max, lowest index) per chunk.
//  k_accept        one workgroup per sequence: combines the chunk partials of
//                  its rows into (m, Z), gathers p(x_i), q(x_i), runs the test
//                  u*q < p on one lane per position, finds the first rejection
//                  with a wave ballot, writes the accepted prefix (or the VAT
//                  labels and weights) and the sampling mode.
//  k_residual_mass for sequences rejected with draft logits: per chunk of the
//                  rejected row pair, sum of max(0, p - q).
//  k_sample        one workgroup per sequence that still needs a token: chunk
//                  masses -> block prefix scan -> the one chunk holding the
//                  draw -> LDS block scan of that chunk -> the token.
//
// No floating-point atomics and fixed reduction orders: bitwise reproducible.
#include <hip/hip_runtime.h>

#include <climits>

#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kMaxDraft = 64;
constexpr int kMaxChunks = 8192;  // V <= 2^24 with 2048-element fp32 chunks

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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Butterfly: every lane ends with the same bits (a+b == b+a in IEEE).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Larger value wins; equal values: lower index wins.
__device__ __forceinline__ void wave_argmax(float& best, int& idx) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o, kWave);
        const int oi = __shfl_xor(idx, o, kWave);
        if (ob > best || (ob == best && oi < idx)) {
            best = ob;
            idx = oi;
        }
    }
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

// Inclusive scan over a workgroup of kBlock threads; returns the inclusive
// value, writes the exclusive one and the block total.  Fixed order.
__device__ __forceinline__ float block_scan(float v, float& excl, float& total, float* s_wt) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    float incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    float wexcl = __shfl_up(incl, 1, kWave);
    if (lane == 0) wexcl = 0.f;
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

// ------------------------------------------------------------------ kernel 1

// (m, s) partial of one (row, chunk): m = max raw logit, s = sum of
// exp2((l - m) * c2) with c2 = log2(e)/T, i.e. sum of exp(l/T - m/T).
template <int EB, bool VEC>
__global__ __launch_bounds__(kBlock) void k_row_stats(const void* target, const void* draft, int64_t rows_t,
                                                      int64_t n_items, int P, int64_t V, float c2,
                                                      float2* __restrict__ partials) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
    if (item >= n_items) return;
    const int64_t row = item / P;
    const int c = static_cast<int>(item - row * P);
    const char* rp = row < rows_t ? row_base(target, row, V, EB) : row_base(draft, row - rows_t, V, EB);
    const int64_t start = static_cast<int64_t>(c) * Chunk<EB>::kElems;
    const int len = static_cast<int>(min(static_cast<int64_t>(Chunk<EB>::kElems), V - start));

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
    s = wave_sum(s);
    if (lane == 0) partials[item] = make_float2(m, s);
}

// (max, lowest index of the max) of one (row, chunk), T == 0.
template <int EB, bool VEC>
__global__ __launch_bounds__(kBlock) void k_row_argmax(const void* target, int64_t n_items, int P, int64_t V,
                                                       float2* __restrict__ partials) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
    if (item >= n_items) return;
    const int64_t row = item / P;
    const int c = static_cast<int>(item - row * P);
    const char* rp = row_base(target, row, V, EB);
    const int64_t start = static_cast<int64_t>(c) * Chunk<EB>::kElems;
    const int len = static_cast<int>(min(static_cast<int64_t>(Chunk<EB>::kElems), V - start));

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
    if (lane == 0) partials[item] = make_float2(best, __int_as_float(static_cast<int>(start) + bi));
}

// ------------------------------------------------------------------ kernel 2

// log2 of p(x) = exp((l(x) - m)/T) / Z for a row with statistics (m, Z).
template <int EB>
__device__ __forceinline__ float log2_prob_of(const void* logits, int64_t row, int64_t V, int x, float2 mz,
                                              float c2) {
    const float l = Elem<EB>::at(row_base(logits, row, V, EB), x);
    return (l - mz.x) * c2 - log2_hw(mz.y);
}

template <int EB>
__global__ __launch_bounds__(kBlock) void k_accept(Plan pl) {
    __shared__ float2 s_mz[2 * kMaxDraft + 1];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int k = pl.k;
    const int n_t = pl.target_rows_per_seq;
    const int n_d = pl.rows_d ? k : 0;
    const int64_t V = pl.vocab;
    const float c2 = pl.c2;

    // Combine the chunk partials of every row of this sequence.
    for (int j = wave; j < n_t + n_d; j += kWavesPerBlock) {
        const int64_t row = j < n_t ? static_cast<int64_t>(b) * n_t + j
                                    : pl.rows_t + static_cast<int64_t>(b) * k + (j - n_t);
        const float2* part = pl.partials + row * pl.chunks;
        float2 res;
        float2 stat;
        if (pl.greedy) {
            float best = neg_inf();
            int bi = INT_MAX;
            for (int c = lane; c < pl.chunks; c += kWave) {
                const float2 pc = part[c];
                const int ic = __float_as_int(pc.y);
                if (pc.x > best || (pc.x == best && ic < bi)) {
                    best = pc.x;
                    bi = ic;
                }
            }
            wave_argmax(best, bi);
            res = make_float2(best, __int_as_float(bi));
            stat = make_float2(best, static_cast<float>(bi));
        } else {
            float m = neg_inf(), s = 0.f;
            for (int c = lane; c < pl.chunks; c += kWave) {
                const float2 pc = part[c];
                if (pc.x == neg_inf()) continue;
                if (pc.x > m) {
                    s = (m == neg_inf() ? 0.f : s * exp2_hw((m - pc.x) * c2)) + pc.y;
                    m = pc.x;
                } else {
                    s += pc.y * exp2_hw((pc.x - m) * c2);
                }
            }
            wave_merge_ms(m, s, c2);
            res = make_float2(m, s);
            stat = make_float2(m / pl.temperature, s);
        }
        if (lane == 0) {
            s_mz[j] = res;
            pl.row_mz[row] = res;
            if (pl.row_stats_out) {
                pl.row_stats_out[2 * row] = stat.x;
                pl.row_stats_out[2 * row + 1] = stat.y;
            }
        }
    }
    __syncthreads();
    if (wave != 0) return;

    // One lane per draft position.
    const int i = lane;
    const bool active = i < k;
    const int x = active ? pl.tokens[static_cast<int64_t>(b) * k + i] : 0;
    const bool bad = active && (x < 0 || x >= pl.vocab);
    const bool invalid = __ballot(bad) != 0ull;
    const int n_u = pl.vat ? k : k + 1;
    bool keep = false;
    float p = __builtin_nanf(""), q = __builtin_nanf("");
    if (!invalid && active) {
        const int64_t trow = static_cast<int64_t>(b) * n_t + i;
        if (pl.greedy) {
            keep = (x == __float_as_int(s_mz[i].y));
            p = keep ? 1.f : 0.f;
            q = 1.f;
        } else {
            // The test u*q < p, taken in the log2 domain so that probabilities
            // below the fp32 range still decide correctly (log2(0) = -inf).
            const float lp = log2_prob_of<EB>(pl.target, trow, V, x, s_mz[i], c2);
            const float lq = pl.onehot ? 0.f
                                       : log2_prob_of<EB>(pl.draft, static_cast<int64_t>(b) * k + i, V, x,
                                                          s_mz[n_t + i], c2);
            const float u = pl.uniforms[static_cast<int64_t>(b) * n_u + i];
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
        return;
    }

    const int x_r = (r >= 0 && r < k) ? __shfl(x, r, kWave) : -1;
    const int g_r = (pl.greedy && r >= 0) ? __float_as_int(s_mz[r].y) : -1;
    int32_t* out = pl.out_tokens + static_cast<int64_t>(b) * (k + 1);
    for (int j = lane; j <= k; j += kWave) {
        int val = -1;
        if (!invalid) {
            if (j < r) val = x;  // j < r <= k < 64 here, so j == lane
            else if (j == r) val = g_r;  // non-greedy: filled in by k_sample
        }
        out[j] = val;
    }
    if (lane == 0) {
        pl.accepted_len[b] = r;
        SeqState st;
        st.r = r;
        st.x_r = x_r;
        st.pad = 0;
        if (invalid || pl.greedy) st.mode = kModeDone;
        else if (r == k) st.mode = kModeBonus;
        else st.mode = pl.onehot ? kModeOneHot : kModeResidual;
        pl.seq[b] = st;
    }
}

// ------------------------------------------------------------------ kernel 3

struct ResidW {
    float c2, mt, izt, md, izd;  // mt, md: row max * c2; izt, izd: 1/Z
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

// Residual mass max(0, p_r - q_r) of one chunk of a rejected row pair.
template <int EB, bool VEC>
__global__ __launch_bounds__(kBlock) void k_residual_mass(Plan pl) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t item = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x / kWave);
    const int P = pl.chunks;
    if (item >= static_cast<int64_t>(pl.batch) * P) return;
    const int b = static_cast<int>(item / P);
    const int c = static_cast<int>(item - static_cast<int64_t>(b) * P);
    const SeqState st = pl.seq[b];
    if (st.mode != kModeResidual) return;
    const int64_t V = pl.vocab;
    const int64_t trow = static_cast<int64_t>(b) * pl.target_rows_per_seq + st.r;
    const int64_t drow = static_cast<int64_t>(b) * pl.k + st.r;
    const ResidW wf = make_resid_w(pl.row_mz[trow], pl.row_mz[pl.rows_t + drow], pl.c2);
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
    if (lane == 0) pl.resid[static_cast<int64_t>(b) * P + c] = s;
}

// ------------------------------------------------------------------ kernel 4

// Weight of token y in the distribution the draw is taken from.
struct DrawRow {
    int mode;        // kModeBonus (plain target row), kModeOneHot, kModeResidual
    const char* rt;  // target row
    const char* rd;  // draft row (residual only)
    float c2, mt;    // mt = row max * c2 rounded (bonus / one-hot)
    float corr;      // exact correction of that rounding (see row_scale)
    int excl;        // one-hot: excluded token, else -1
    ResidW rw;
};

template <int EB>
__device__ __forceinline__ float draw_weight(const DrawRow& d, int64_t y) {
    if (d.mode == kModeResidual) return d.rw(Elem<EB>::at(d.rt, y), Elem<EB>::at(d.rd, y));
    if (y == d.excl) return 0.f;
    return exp2_hw(fmaf(Elem<EB>::at(d.rt, y), d.c2, -d.mt)) * d.corr;
}

// Chunk masses of a plain target row from its k_row_stats partials, in the
// units of draw_weight (relative to the row max).
__device__ __forceinline__ float mass_from_partial(float2 pc, float row_max, float c2) {
    return pc.x == neg_inf() ? 0.f : pc.y * exp2_hw((pc.x - row_max) * c2);
}

// In-place inclusive prefix of s_mass[0..P) with tiles of kBlock and a carry.
__device__ __forceinline__ void scan_masses(float* s_mass, int P, float* s_wt) {
    float carry = 0.f;
    for (int base = 0; base < P; base += kBlock) {
        const int c = base + threadIdx.x;
        const float v = c < P ? s_mass[c] : 0.f;
        float excl, total;
        const float incl = block_scan(v, excl, total, s_wt);
        if (c < P) s_mass[c] = carry + incl;
        carry = carry + total;
        __syncthreads();
    }
}

template <int EB>
__global__ __launch_bounds__(kBlock) void k_sample(Plan pl) {
    __shared__ float s_mass[kMaxChunks];
    __shared__ float s_wt[kWavesPerBlock];
    __shared__ int s_sel;
    __shared__ int s_last;
    const int b = blockIdx.x;
    const SeqState st = pl.seq[b];
    if (st.mode == kModeDone) return;
    const int tid = threadIdx.x;
    const int k = pl.k;
    const int P = pl.chunks;
    const int CH = Chunk<EB>::kElems;
    const int64_t V = pl.vocab;
    const float c2 = pl.c2;
    const int r = st.r;
    const float u = pl.uniforms[static_cast<int64_t>(b) * (k + 1) + k];

    DrawRow d;
    d.mode = st.mode;
    d.c2 = c2;
    d.excl = st.mode == kModeOneHot ? st.x_r : -1;
    int64_t trow = static_cast<int64_t>(b) * pl.target_rows_per_seq + (st.mode == kModeBonus ? k : r);
    d.rt = row_base(pl.target, trow, V, EB);
    d.rd = nullptr;
    float2 mzt = pl.row_mz[trow];
    d.mt = row_scale(mzt.x, c2, d.corr);
    if (st.mode == kModeResidual) {
        const int64_t drow = static_cast<int64_t>(b) * k + r;
        d.rd = row_base(pl.draft, drow, V, EB);
        d.rw = make_resid_w(mzt, pl.row_mz[pl.rows_t + drow], c2);
    }

    // Chunk masses.
    for (int pass = 0; pass < 2; ++pass) {
        if (d.mode == kModeResidual) {
            for (int c = tid; c < P; c += kBlock) s_mass[c] = pl.resid[static_cast<int64_t>(b) * P + c];
        } else {
            const float2* part = pl.partials + trow * P;
            for (int c = tid; c < P; c += kBlock) s_mass[c] = mass_from_partial(part[c], mzt.x, c2);
        }
        __syncthreads();
        if (d.mode == kModeOneHot) {
            // Recompute the chunk holding x_r without it (avoids cancellation).
            const int cx = d.excl / CH;
            const int64_t cstart = static_cast<int64_t>(cx) * CH;
            const int clen = static_cast<int>(min(static_cast<int64_t>(CH), V - cstart));
            float part_sum = 0.f;
            for (int e = 0; e < Chunk<EB>::kPerThread; ++e) {
                const int idx = tid * Chunk<EB>::kPerThread + e;
                if (idx < clen) part_sum += draw_weight<EB>(d, cstart + idx);
            }
            const float tot = block_sum(part_sum, s_wt);
            if (tid == 0) s_mass[cx] = tot;
            __syncthreads();
        }
        scan_masses(s_mass, P, s_wt);
        // A residual that rounds to zero mass: draw from p_r instead.
        if (pass == 0 && d.mode == kModeResidual && !(s_mass[P - 1] > 0.f)) {
            d.mode = kModeBonus;
            __syncthreads();
            continue;
        }
        break;
    }

    const float zw = s_mass[P - 1];
    const float theta = u * zw;
    if (tid == 0) {
        s_sel = INT_MAX;
        s_last = -1;
    }
    __syncthreads();
    for (int c = tid; c < P; c += kBlock) {
        const float prev = c ? s_mass[c - 1] : 0.f;
        if (s_mass[c] > theta && prev <= theta) atomicMin(&s_sel, c);
        if (s_mass[c] > prev) atomicMax(&s_last, c);
    }
    __syncthreads();
    int cs = s_sel;
    float th = 0.f;
    bool open_end = false;  // rounding left no chunk above theta: take the last positive weight
    if (cs == INT_MAX) {
        cs = s_last >= 0 ? s_last : P - 1;
        open_end = true;
    } else {
        th = theta - (cs ? s_mass[cs - 1] : 0.f);
    }
    __syncthreads();

    // Scan the chosen chunk: thread t owns kPerThread consecutive logits.
    const int64_t cstart = static_cast<int64_t>(cs) * CH;
    const int clen = static_cast<int>(min(static_cast<int64_t>(CH), V - cstart));
    float w[Chunk<EB>::kPerThread];
    float st_sum = 0.f;
    int my_last = -1;
#pragma unroll
    for (int e = 0; e < Chunk<EB>::kPerThread; ++e) {
        const int idx = tid * Chunk<EB>::kPerThread + e;
        w[e] = idx < clen ? draw_weight<EB>(d, cstart + idx) : 0.f;
        st_sum += w[e];
        if (w[e] > 0.f) my_last = idx;
    }
    float excl, total;
    block_scan(st_sum, excl, total, s_wt);
    if (tid == 0) {
        s_sel = INT_MAX;
        s_last = -1;
    }
    __syncthreads();
    if (my_last >= 0) atomicMax(&s_last, my_last);
    int pick = -1;
    if (!open_end && excl + st_sum > th) {
        float run = excl;
#pragma unroll
        for (int e = 0; e < Chunk<EB>::kPerThread; ++e) {
            run += w[e];
            if (pick < 0 && w[e] > 0.f && run > th) pick = tid * Chunk<EB>::kPerThread + e;
        }
        if (pick >= 0) atomicMin(&s_sel, pick);
    }
    __syncthreads();
    if (tid == 0) {
        int y = s_sel != INT_MAX ? s_sel : (s_last >= 0 ? s_last : 0);
        pl.out_tokens[static_cast<int64_t>(b) * (k + 1) + r] = static_cast<int32_t>(cstart + y);
    }
}

// ------------------------------------------------------------------ dispatch

inline unsigned grid_for_waves(int64_t waves) {
    return static_cast<unsigned>((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}

template <int EB, bool VEC>
hipError_t launch_typed(const Plan& pl, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    const int64_t rows = pl.rows_t + pl.rows_d;
    const int64_t items = rows * pl.chunks;
    if (ev0 && ev1) {
        hipError_t e = hipEventRecord(ev0, stream);
        if (e != hipSuccess) return e;
    }
    if (pl.greedy) {
        hipLaunchKernelGGL((k_row_argmax<EB, VEC>), dim3(grid_for_waves(items)), dim3(kBlock), 0, stream,
                           pl.target, items, pl.chunks, static_cast<int64_t>(pl.vocab), pl.partials);
    } else {
        hipLaunchKernelGGL((k_row_stats<EB, VEC>), dim3(grid_for_waves(items)), dim3(kBlock), 0, stream,
                           pl.target, pl.draft, pl.rows_t, items, pl.chunks, static_cast<int64_t>(pl.vocab),
                           pl.c2, pl.partials);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ev0 && ev1) {
        e = hipEventRecord(ev1, stream);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_accept<EB>), dim3(pl.batch), dim3(kBlock), 0, stream, pl);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pl.vat || pl.greedy) return hipSuccess;
    if (!pl.onehot) {
        hipLaunchKernelGGL((k_residual_mass<EB, VEC>), dim3(grid_for_waves(static_cast<int64_t>(pl.batch) * pl.chunks)),
                           dim3(kBlock), 0, stream, pl);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_sample<EB>), dim3(pl.batch), dim3(kBlock), 0, stream, pl);
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
