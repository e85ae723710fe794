/*
 * oracle.c -- plain fp64 CPU reference for batched speculative-sampling
 * verification and verification-aware training (VAT) labels.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file; only the test suite, the package smoke check and the
 * bench's CPU-baseline leg do.  It shares no code, header, table or helper
 * with the HIP library: it has its own bf16 decode, its own softmax and its
 * own sampler, written as the plain definitions, one row at a time, in fp64,
 * with no blocking, fusion or reordering.
 *
 * Sources (page title, then section):
 *  [NG1] "AI 开始抄自己的作业——而且抄得理直气壮" (zhichai.net NgramRL essay),
 *        section "投机解码：让草稿先跑，考官殿后": the draft proposes k tokens,
 *        one target forward scores every position, a proposed token x is kept
 *        with probability min(1, pi(x|c)/q(x|c)), the chain is cut at the first
 *        rejection, the target supplies one token there, drawn from the residual
 *        (target mass minus what the draft already proposed).  Worked numbers:
 *        q=0.9, pi=0.95 -> kept for sure; q=0.9, pi=0.1 -> kept ~1 time in 9.
 *  [NG2] same page, section "考官坐镇：为什么抄作业不算作弊": the same rule
 *        and residual resampling make the output distribution exactly the
 *        target's.
 *  [NR1] "NgramRL：用Rollout历史加速RL后训练的推测解码新方案" (kongchang.com),
 *        section "一个被忽视的草稿源": verification accepts the matching prefix
 *        and drops everything after the first mismatch; section
 *        "自适应 fan-out 预取": the step's outcome is the pair (accepted length j,
 *        token b supplied by the target).
 *  [VAT1] "让AI草稿模型学会“照镜子”" (VAT news write-up), section
 *        "VAT怎么把“验收规则”塞进训练里": training simulates the inference-time
 *        acceptance rule; every position from the first rejection on is
 *        labelled as rejected.
 *  [VAT2] same page, section "第二件事，改权重分配的锚点": positions before the
 *        first rejection get full weight; the usual decay curve (EAGLE-3: 0.8
 *        to the power position-1) restarts at the first rejection.  The end of
 *        that section: the drafter's loss combines soft-label distillation
 *        from the target's output distribution with hard-label supervision
 *        from the token the target actually sampled.
 *
 * Readings where the pages leave a step open (each also listed in the design
 * notes of the repository):
 *  - acceptance is tested as u*q(x) < p(x) with u uniform in [0,1): the event
 *    has probability min(1, p/q) and needs no division;
 *  - softmax at temperature T>0 is p(y) = exp(l(y)/T - m)/Z with
 *    m = max_y l(y)/T, Z = sum_y exp(l(y)/T - m);
 *  - T == 0 is greedy: the target's choice is its first (lowest-id) argmax;
 *    a draft token is kept iff it equals that choice; the target's token at
 *    the first mismatch (or after full acceptance) is that argmax;
 *  - the residual at a rejected position r is w(y) = max(0, p_r(y)-q_r(y));
 *    after full acceptance the bonus token is drawn from the target row k;
 *    a one-hot draft is q = indicator of the draft token;
 *  - sampling from w with uniform u takes the smallest id y whose running
 *    sum exceeds u*sum(w) (ascending id); if none does (only through
 *    rounding) the largest id with w>0; if sum(w) == 0 the row p_r is used;
 *  - uniforms: u[b][i] for i<k drives test i, u[b][k] the single draw;
 *  - positions after the committed token are -1 in out_tokens;
 *  - a token outside [0,V) flags the whole sequence: accepted_len = -1,
 *    out_tokens all -1;
 *  - VAT weight at the rejected position itself is decay^0 = 1; no rejection
 *    gives first_reject = k and all weights 1.
 *  - LM-head greedy verification (orc_lm_head_greedy): the logits are the
 *    product of the hidden state with the output layer's weights, formed in
 *    fp64 from their bf16 values; the rest is the T == 0 rule above.
 *  - LM-head verification at T > 0 (orc_lm_head_logits, then orc_verify on
 *    ORC_F64 rows): target logits from the target's hidden states and output
 *    layer, draft logits from the draft's hidden states and its output layer,
 *    both formed in fp64 from bf16 values; the rest is the rule above.
 *  - VAT loss (orc_vat_loss): at every position the soft term is the cross
 *    entropy of the draft's distribution against the target's at the same
 *    temperature, -sum_y p(y) ln q(y); the hard term is -ln q(h) for the
 *    target's sampled token h; the block's loss is
 *    sum_i w_i (soft_i + hard_weight * hard_i) with the VAT weights w_i.
 *    Natural logarithms (nats).  T must be > 0 (both distributions are
 *    needed).  A block with a draft or hard token outside [0,V) is flagged:
 *    first_reject -1, mask 0, weights 0, soft/hard/loss NaN.
 *  - VAT loss gradient (orc_vat_loss_grad): the derivative of the block loss
 *    with respect to the draft logits, the weights held fixed (they are the
 *    labels of the simulated verification); derived from the definition above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* logits already in fp64 (formed by orc_lm_head_logits) */

int orc_abi_version(void) { return 1; }

/* bfloat16 is the top half of an IEEE-754 binary32: 1 sign bit, 8 exponent
 * bits (bias 127), 7 fraction bits.  Decoded field by field into fp64. */
double orc_decode_bf16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 7) & 0xFF;
    int frac = bits & 0x7F;
    double mag;
    if (expo == 0xFF) {
        mag = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        mag = ldexp((double)frac / 128.0, -126); /* subnormal */
    } else {
        mag = ldexp(1.0 + (double)frac / 128.0, expo - 127);
    }
    return sign ? -mag : mag;
}

/* IEEE binary32 decoded field by field (same layout with 23 fraction bits). */
static double decode_f32(uint32_t bits) {
    int sign = (bits >> 31) & 1;
    int expo = (bits >> 23) & 0xFF;
    uint32_t frac = bits & 0x7FFFFF;
    double mag;
    if (expo == 0xFF) {
        mag = frac ? NAN : INFINITY;
    } else if (expo == 0) {
        mag = ldexp((double)frac / 8388608.0, -126);
    } else {
        mag = ldexp(1.0 + (double)frac / 8388608.0, expo - 127);
    }
    return sign ? -mag : mag;
}

double orc_decode_f32(uint32_t bits) { return decode_f32(bits); }

/* Copy row `row` (V logits) of a row-major [rows][V] array into fp64. */
static void load_row(const void* base, int dtype, int64_t row, int64_t V, double* out) {
    int64_t y;
    if (dtype == ORC_BF16) {
        const uint16_t* p = (const uint16_t*)base + row * V;
        for (y = 0; y < V; ++y) out[y] = orc_decode_bf16(p[y]);
    } else if (dtype == ORC_F64) {
        const double* p = (const double*)base + row * V;
        for (y = 0; y < V; ++y) out[y] = p[y];
    } else {
        const uint32_t* p = (const uint32_t*)base + row * V;
        for (y = 0; y < V; ++y) out[y] = decode_f32(p[y]);
    }
}

/* Softmax at temperature T > 0 [NG1]: p(y) = exp(l(y)/T - m) / Z. */
void orc_softmax(const double* l, int64_t V, double T, double* p, double* m_out, double* z_out) {
    int64_t y;
    double m = -INFINITY, z = 0.0;
    for (y = 0; y < V; ++y) {
        double s = l[y] / T;
        if (s > m) m = s;
    }
    for (y = 0; y < V; ++y) {
        p[y] = exp(l[y] / T - m);
        z += p[y];
    }
    for (y = 0; y < V; ++y) p[y] /= z;
    if (m_out) *m_out = m;
    if (z_out) *z_out = z;
}

/* First (lowest-id) argmax, comparing the decoded values exactly. */
int64_t orc_argmax(const double* l, int64_t V) {
    int64_t y, best = 0;
    for (y = 1; y < V; ++y)
        if (l[y] > l[best]) best = y;
    return best;
}

/* Probability that a proposed token with target prob p and draft prob q is
 * kept [NG1]: min(1, p/q).  q == 0 (the draft could not have proposed it):
 * the test u*q < p keeps it iff p > 0. */
double orc_accept_prob(double p, double q) {
    if (q <= 0.0) return p > 0.0 ? 1.0 : 0.0;
    return p / q < 1.0 ? p / q : 1.0;
}

/* The acceptance event for one uniform draw u in [0,1): kept iff u*q < p,
 * which happens with probability min(1, p/q) [NG1]. */
int orc_accept(double u, double p, double q) { return u * q < p; }

/* Residual after a rejection [NG1]: what is left of the target distribution
 * once the part the draft proposed is taken away, w = max(0, p - q). */
void orc_residual(const double* p, const double* q, int64_t V, double* w) {
    int64_t y;
    for (y = 0; y < V; ++y) w[y] = p[y] - q[y] > 0.0 ? p[y] - q[y] : 0.0;
}

/* Draw from the (unnormalised) weights w with uniform u by inverting the
 * cumulative sum in ascending id order: smallest y with C(y) > u*Z, Z = sum w.
 * `margin` (may be NULL) receives the distance of u*Z from the nearer end of
 * the chosen interval [C(y-1), C(y)), divided by Z. */
int64_t orc_inverse_cdf(const double* w, int64_t V, double u, double* margin) {
    int64_t y, last_pos = -1;
    double z = 0.0, c = 0.0, theta;
    for (y = 0; y < V; ++y) z += w[y];
    theta = u * z;
    for (y = 0; y < V; ++y) {
        double prev = c;
        c += w[y];
        if (w[y] > 0.0) last_pos = y;
        if (c > theta) {
            if (margin) {
                double a = theta - prev, b = c - theta;
                *margin = (a < b ? a : b) / z;
            }
            return y;
        }
    }
    if (margin) *margin = 0.0;
    return last_pos >= 0 ? last_pos : V - 1;
}

static int tokens_valid(const int32_t* x, int32_t k, int64_t V) {
    int32_t i;
    for (i = 0; i < k; ++i)
        if (x[i] < 0 || (int64_t)x[i] >= V) return 0;
    return 1;
}

/*
 * Batched verification of B sequences with k draft tokens each.
 *   target [B][k+1][V], draft [B][k][V] (ignored if onehot or T == 0),
 *   tokens [B][k], u [B][k+1].
 * Outputs: accepted_len [B], out_tokens [B][k+1].
 * Optional diagnostics (NULL to skip), all fp64:
 *   probs [B][k][2]         (p_i(x_i), q_i(x_i));  T == 0: ([x_i == g_i], 1)
 *   target_mz [B][k+1][2]   (m, Z) of every target row; T == 0: (max l, argmax)
 *   draft_mz [B][k][2]      (m, Z) of every draft row (NaN if not read)
 *   accept_margin [B][k]    u_i - p_i/q_i (+inf for T == 0)
 *   sample_margin [B]       distance of the draw from its interval's ends
 * Returns 0, or -1 on bad arguments (nothing written).
 */
int orc_verify(int64_t B, int32_t k, int64_t V, int32_t dtype, int32_t onehot, double T,
               const void* target, const void* draft, const int32_t* tokens, const float* u,
               int32_t* accepted_len, int32_t* out_tokens, double* probs, double* target_mz,
               double* draft_mz, double* accept_margin, double* sample_margin) {
    int64_t b, y;
    int32_t i;
    int greedy = (T == 0.0);
    int use_draft = !greedy && !onehot;
    double *lt, *ld, *p, *q, *w, *prow_k;
    if (B < 0 || k < 1 || V < 1 || T < 0.0 || !(T == T)) return -1;
    if (!target || !tokens || !accepted_len || !out_tokens) return -1;
    if (use_draft && !draft) return -1;
    if (!greedy && !u) return -1;
    lt = (double*)malloc(sizeof(double) * V);
    ld = (double*)malloc(sizeof(double) * V);
    p = (double*)malloc(sizeof(double) * V * (k + 1)); /* p_0..p_k */
    q = (double*)malloc(sizeof(double) * V * k);       /* q_0..q_{k-1} */
    w = (double*)malloc(sizeof(double) * V);
    if (!lt || !ld || !p || !q || !w) {
        free(lt); free(ld); free(p); free(q); free(w);
        return -1;
    }
    for (b = 0; b < B; ++b) {
        const int32_t* x = tokens + b * k;
        const float* ub = greedy ? NULL : u + b * (k + 1);
        int32_t* out = out_tokens + b * (k + 1);
        int32_t r = k;
        int64_t ystar;
        double smargin = INFINITY;
        if (!tokens_valid(x, k, V)) {
            accepted_len[b] = -1;
            for (i = 0; i <= k; ++i) out[i] = -1;
            if (probs) for (i = 0; i < 2 * k; ++i) probs[b * 2 * k + i] = NAN;
            if (accept_margin) for (i = 0; i < k; ++i) accept_margin[b * k + i] = NAN;
            if (sample_margin) sample_margin[b] = NAN;
            if (target_mz) for (i = 0; i < 2 * (k + 1); ++i) target_mz[b * 2 * (k + 1) + i] = NAN;
            if (draft_mz) for (i = 0; i < 2 * k; ++i) draft_mz[b * 2 * k + i] = NAN;
            continue;
        }
        if (greedy) {
            /* T == 0: keep x_i while it equals the target's argmax g_i. */
            int64_t* g = (int64_t*)malloc(sizeof(int64_t) * (k + 1));
            if (!g) {
                free(lt); free(ld); free(p); free(q); free(w);
                return -1;
            }
            for (i = 0; i <= k; ++i) {
                load_row(target, dtype, b * (k + 1) + i, V, lt);
                g[i] = orc_argmax(lt, V);
                if (target_mz) {
                    target_mz[(b * (k + 1) + i) * 2 + 0] = lt[g[i]];
                    target_mz[(b * (k + 1) + i) * 2 + 1] = (double)g[i];
                }
            }
            for (i = 0; i < k; ++i) {
                int keep = (x[i] == g[i]);
                if (probs) {
                    probs[(b * k + i) * 2 + 0] = keep ? 1.0 : 0.0;
                    probs[(b * k + i) * 2 + 1] = 1.0;
                }
                if (accept_margin) accept_margin[b * k + i] = INFINITY;
                if (draft_mz) {
                    draft_mz[(b * k + i) * 2 + 0] = NAN;
                    draft_mz[(b * k + i) * 2 + 1] = NAN;
                }
                if (!keep && r == k) r = i;
            }
            ystar = g[r];
            free(g);
        } else {
            /* Target and draft distributions at every position. */
            for (i = 0; i <= k; ++i) {
                double m, z;
                load_row(target, dtype, b * (k + 1) + i, V, lt);
                orc_softmax(lt, V, T, p + (int64_t)i * V, &m, &z);
                if (target_mz) {
                    target_mz[(b * (k + 1) + i) * 2 + 0] = m;
                    target_mz[(b * (k + 1) + i) * 2 + 1] = z;
                }
            }
            for (i = 0; i < k; ++i) {
                double* qi = q + (int64_t)i * V;
                if (onehot) {
                    for (y = 0; y < V; ++y) qi[y] = 0.0;
                    qi[x[i]] = 1.0;
                    if (draft_mz) {
                        draft_mz[(b * k + i) * 2 + 0] = NAN;
                        draft_mz[(b * k + i) * 2 + 1] = NAN;
                    }
                } else {
                    double m, z;
                    load_row(draft, dtype, b * k + i, V, ld);
                    orc_softmax(ld, V, T, qi, &m, &z);
                    if (draft_mz) {
                        draft_mz[(b * k + i) * 2 + 0] = m;
                        draft_mz[(b * k + i) * 2 + 1] = z;
                    }
                }
            }
            /* Sequential test, cut at the first rejection [NG1][NR1]. */
            for (i = 0; i < k; ++i) {
                double pi = p[(int64_t)i * V + x[i]];
                double qi = q[(int64_t)i * V + x[i]];
                if (probs) {
                    probs[(b * k + i) * 2 + 0] = pi;
                    probs[(b * k + i) * 2 + 1] = qi;
                }
                if (accept_margin) {
                    if (qi > 0.0) accept_margin[b * k + i] = (double)ub[i] - pi / qi;
                    else accept_margin[b * k + i] = pi > 0.0 ? -INFINITY : INFINITY;
                }
            }
            for (i = 0; i < k; ++i) {
                if (!orc_accept((double)ub[i], p[(int64_t)i * V + x[i]], q[(int64_t)i * V + x[i]])) {
                    r = i;
                    break;
                }
            }
            /* The target's own token at r [NG1]: residual after a rejection,
             * the plain target row after full acceptance. */
            if (r < k) {
                double zw = 0.0;
                orc_residual(p + (int64_t)r * V, q + (int64_t)r * V, V, w);
                for (y = 0; y < V; ++y) zw += w[y];
                if (zw == 0.0) /* only reachable through rounding */
                    for (y = 0; y < V; ++y) w[y] = p[(int64_t)r * V + y];
            } else {
                prow_k = p + (int64_t)k * V;
                for (y = 0; y < V; ++y) w[y] = prow_k[y];
            }
            ystar = orc_inverse_cdf(w, V, (double)ub[k], &smargin);
        }
        accepted_len[b] = r;
        for (i = 0; i < r; ++i) out[i] = x[i];
        out[r] = (int32_t)ystar;
        for (i = r + 1; i <= k; ++i) out[i] = -1;
        if (sample_margin) sample_margin[b] = smargin;
    }
    free(lt); free(ld); free(p); free(q); free(w);
    return 0;
}

/*
 * Verification-aware training labels for N draft blocks of k positions
 * [VAT1][VAT2].  target [N][k][V] (no bonus row), draft [N][k][V] (ignored at
 * T == 0), tokens [N][k], u [N][k].
 * Outputs: mask [N][k] (1 = accepted: position before the first rejection),
 * first_reject [N] (k if none), weights [N][k] (1 before r, decay^(i-r) from
 * r on; decay^0 = 1).
 * Optional fp64 diagnostics as in orc_verify (probs [N][k][2], target_mz
 * [N][k][2], draft_mz [N][k][2], accept_margin [N][k]).
 * A block with a token outside [0,V): first_reject = -1, mask 0, weights 0.
 */
int orc_vat(int64_t N, int32_t k, int64_t V, int32_t dtype, double T, double decay,
            const void* target, const void* draft, const int32_t* tokens, const float* u,
            uint8_t* mask, int32_t* first_reject, double* weights, double* probs,
            double* target_mz, double* draft_mz, double* accept_margin) {
    int64_t n;
    int32_t i;
    int greedy = (T == 0.0);
    double *lt, *ld, *p, *q;
    if (N < 0 || k < 1 || V < 1 || T < 0.0 || !(T == T) || !(decay == decay)) return -1;
    if (!target || !tokens || !mask || !first_reject || !weights) return -1;
    if (!greedy && (!draft || !u)) return -1;
    lt = (double*)malloc(sizeof(double) * V);
    ld = (double*)malloc(sizeof(double) * V);
    p = (double*)malloc(sizeof(double) * V);
    q = (double*)malloc(sizeof(double) * V);
    if (!lt || !ld || !p || !q) {
        free(lt); free(ld); free(p); free(q);
        return -1;
    }
    for (n = 0; n < N; ++n) {
        const int32_t* x = tokens + n * k;
        int32_t r = k;
        if (!tokens_valid(x, k, V)) {
            first_reject[n] = -1;
            for (i = 0; i < k; ++i) {
                mask[n * k + i] = 0;
                weights[n * k + i] = 0.0;
                if (probs) { probs[(n * k + i) * 2] = NAN; probs[(n * k + i) * 2 + 1] = NAN; }
                if (accept_margin) accept_margin[n * k + i] = NAN;
                if (target_mz) { target_mz[(n * k + i) * 2] = NAN; target_mz[(n * k + i) * 2 + 1] = NAN; }
                if (draft_mz) { draft_mz[(n * k + i) * 2] = NAN; draft_mz[(n * k + i) * 2 + 1] = NAN; }
            }
            continue;
        }
        /* Simulated verification: the inference-time rule, position by
         * position; the first failure fixes r [VAT1]. */
        for (i = 0; i < k; ++i) {
            int keep;
            load_row(target, dtype, n * k + i, V, lt);
            if (greedy) {
                int64_t g = orc_argmax(lt, V);
                keep = (x[i] == g);
                if (probs) { probs[(n * k + i) * 2] = keep ? 1.0 : 0.0; probs[(n * k + i) * 2 + 1] = 1.0; }
                if (target_mz) { target_mz[(n * k + i) * 2] = lt[g]; target_mz[(n * k + i) * 2 + 1] = (double)g; }
                if (draft_mz) { draft_mz[(n * k + i) * 2] = NAN; draft_mz[(n * k + i) * 2 + 1] = NAN; }
                if (accept_margin) accept_margin[n * k + i] = INFINITY;
            } else {
                double mt, zt, md, zd, pi, qi;
                load_row(draft, dtype, n * k + i, V, ld);
                orc_softmax(lt, V, T, p, &mt, &zt);
                orc_softmax(ld, V, T, q, &md, &zd);
                pi = p[x[i]];
                qi = q[x[i]];
                keep = orc_accept((double)u[n * k + i], pi, qi);
                if (probs) { probs[(n * k + i) * 2] = pi; probs[(n * k + i) * 2 + 1] = qi; }
                if (target_mz) { target_mz[(n * k + i) * 2] = mt; target_mz[(n * k + i) * 2 + 1] = zt; }
                if (draft_mz) { draft_mz[(n * k + i) * 2] = md; draft_mz[(n * k + i) * 2 + 1] = zd; }
                if (accept_margin) {
                    if (qi > 0.0) accept_margin[n * k + i] = (double)u[n * k + i] - pi / qi;
                    else accept_margin[n * k + i] = pi > 0.0 ? -INFINITY : INFINITY;
                }
            }
            if (!keep && r == k) r = i;
        }
        first_reject[n] = r;
        /* Labels and first-rejection-anchored weights [VAT1][VAT2]. */
        for (i = 0; i < k; ++i) {
            mask[n * k + i] = (uint8_t)(i < r);
            weights[n * k + i] = i < r ? 1.0 : pow(decay, (double)(i - r));
        }
    }
    free(lt); free(ld); free(p); free(q);
    return 0;
}

/* VAT training loss of each block [VAT2]: the labels and weights of orc_vat,
 * then per position the soft term -sum_y p(y) ln q(y) and the hard term
 * -ln q(h_i), and the weighted block loss.  p, q: softmax at temperature T. */
int orc_vat_loss(int64_t N, int32_t k, int64_t V, int32_t dtype, double T, double decay, double hard_weight,
                 const void* target, const void* draft, const int32_t* tokens, const float* u,
                 const int32_t* hard_tokens, uint8_t* mask, int32_t* first_reject, double* weights,
                 double* soft, double* hard, double* block_loss) {
    int64_t n, y;
    int32_t i;
    double *lt, *ld, *p, *q;
    if (N < 0 || k < 1 || V < 1 || !(T > 0.0) || !(decay == decay) || !(hard_weight == hard_weight)) return -1;
    if (!target || !draft || !tokens || !u || !hard_tokens || !soft || !hard || !block_loss) return -1;
    if (orc_vat(N, k, V, dtype, T, decay, target, draft, tokens, u, mask, first_reject, weights, 0, 0, 0, 0))
        return -1;
    lt = (double*)malloc(sizeof(double) * V);
    ld = (double*)malloc(sizeof(double) * V);
    p = (double*)malloc(sizeof(double) * V);
    q = (double*)malloc(sizeof(double) * V);
    if (!lt || !ld || !p || !q) {
        free(lt); free(ld); free(p); free(q);
        return -1;
    }
    for (n = 0; n < N; ++n) {
        const int32_t* h = hard_tokens + n * k;
        double total = 0.0;
        if (first_reject[n] < 0 || !tokens_valid(h, k, V)) {
            first_reject[n] = -1;
            for (i = 0; i < k; ++i) {
                mask[n * k + i] = 0;
                weights[n * k + i] = 0.0;
                soft[n * k + i] = NAN;
                hard[n * k + i] = NAN;
            }
            block_loss[n] = NAN;
            continue;
        }
        for (i = 0; i < k; ++i) {
            double mt, zt, md, zd, ce = 0.0;
            load_row(target, dtype, n * k + i, V, lt);
            load_row(draft, dtype, n * k + i, V, ld);
            orc_softmax(lt, V, T, p, &mt, &zt);
            orc_softmax(ld, V, T, q, &md, &zd);
            /* ln q(y) = l_d(y)/T - md - ln zd */
            for (y = 0; y < V; ++y) {
                if (p[y] > 0.0) ce -= p[y] * (ld[y] / T - md - log(zd));
            }
            soft[n * k + i] = ce;
            hard[n * k + i] = -(ld[h[i]] / T - md - log(zd));
            total += weights[n * k + i] * (ce + hard_weight * hard[n * k + i]);
        }
        block_loss[n] = total;
    }
    free(lt); free(ld); free(p); free(q);
    return 0;
}

/* Gradient of the VAT block loss of orc_vat_loss with respect to the draft
 * logits [VAT2], the VAT weights held fixed (they are per-position labels of
 * the simulated verification, not functions of the logits).  With
 * q = softmax(l_d/T), p = softmax(l_t/T) and ln q(z) = l_d(z)/T - logsumexp:
 *   d(-sum_z p(z) ln q(z)) / d l_d(y) = (q(y) - p(y)) / T,
 *   d(-ln q(h)) / d l_d(y)             = (q(y) - [y == h]) / T,
 * so grad[n][i][y] = w_i / T * ((1 + hard_weight) q(y) - p(y) - hard_weight [y == h_i]).
 * Inputs: the logits as for orc_vat_loss, hard tokens [N][k], the weights
 * [N][k] that orc_vat_loss returned.  A position of weight 0 (a flagged
 * block, or decay 0 after the first rejection) has an all-zero row. */
int orc_vat_loss_grad(int64_t N, int32_t k, int64_t V, int32_t dtype, double T, double hard_weight,
                      const void* target, const void* draft, const int32_t* hard_tokens, const double* weights,
                      double* grad) {
    int64_t n, y;
    int32_t i;
    double *lt, *ld, *p, *q;
    if (N < 0 || k < 1 || V < 1 || !(T > 0.0) || !(hard_weight == hard_weight)) return -1;
    if (!target || !draft || !hard_tokens || !weights || !grad) return -1;
    lt = (double*)malloc(sizeof(double) * V);
    ld = (double*)malloc(sizeof(double) * V);
    p = (double*)malloc(sizeof(double) * V);
    q = (double*)malloc(sizeof(double) * V);
    if (!lt || !ld || !p || !q) {
        free(lt); free(ld); free(p); free(q);
        return -1;
    }
    for (n = 0; n < N; ++n) {
        for (i = 0; i < k; ++i) {
            const int64_t row = n * k + i;
            const double w = weights[row];
            double* g = grad + row * V;
            double mt, zt, md, zd, s;
            int64_t h;
            if (w == 0.0) {
                for (y = 0; y < V; ++y) g[y] = 0.0;
                continue;
            }
            h = hard_tokens[row];
            load_row(target, dtype, row, V, lt);
            load_row(draft, dtype, row, V, ld);
            orc_softmax(lt, V, T, p, &mt, &zt);
            orc_softmax(ld, V, T, q, &md, &zd);
            s = w / T;
            for (y = 0; y < V; ++y)
                g[y] = s * ((1.0 + hard_weight) * q[y] - p[y] - (y == h ? hard_weight : 0.0));
        }
    }
    free(lt); free(ld); free(p); free(q);
    return 0;
}

/* LM-head greedy verification (the T = 0 reading of [NG1], with the logits
 * formed from hidden states): logits l_i(y) = sum_d h_i[d] w_y[d] in fp64 from
 * bf16 hidden states h [B][k+1][D] and output-layer weights w [V][D]; the
 * target's choice g_i is the lowest-index argmax; a draft token is kept iff it
 * equals g_i; r = first mismatch (k if none); out = x_0..x_{r-1}, g_r, -1...
 * Also returns every row's argmax and the gap between its two largest logits
 * (the margin a rounding of the logits would have to overcome).
 * Each weight row is decoded once and dotted with every hidden row of the
 * call (each dot product is the plain sequential fp64 sum over d); tokens
 * are visited in ascending id, so the first strict maximum is the lowest. */
int orc_lm_head_greedy(int64_t B, int32_t k, int64_t V, int64_t D, const uint16_t* hidden, const uint16_t* weight,
                       const int32_t* tokens, int32_t* accepted_len, int32_t* out_tokens, int32_t* argmax_out,
                       double* top2_gap) {
    int64_t b, y, d, row;
    int32_t i;
    const int64_t rows = B * (k + 1);
    double *h, *wy, *best, *second;
    int64_t* g;
    if (B < 0 || k < 1 || V < 1 || D < 1 || !hidden || !weight || !tokens || !accepted_len || !out_tokens) return -1;
    h = (double*)malloc(sizeof(double) * (rows * D + D + 2 * rows + 1));
    g = (int64_t*)malloc(sizeof(int64_t) * (rows + 1));
    if (!h || !g) {
        free(h);
        free(g);
        return -1;
    }
    wy = h + rows * D;
    best = wy + D;
    second = best + rows;
    for (row = 0; row < rows; ++row) {
        for (d = 0; d < D; ++d) h[row * D + d] = orc_decode_bf16(hidden[row * D + d]);
        best[row] = -INFINITY;
        second[row] = -INFINITY;
        g[row] = 0;
    }
    for (y = 0; y < V; ++y) {
        for (d = 0; d < D; ++d) wy[d] = orc_decode_bf16(weight[y * D + d]);
        for (row = 0; row < rows; ++row) {
            const double* hr = h + row * D;
            double s = 0.0;
            for (d = 0; d < D; ++d) s += hr[d] * wy[d];
            if (s > best[row]) {
                second[row] = best[row];
                best[row] = s;
                g[row] = y;
            } else if (s > second[row]) {
                second[row] = s;
            }
        }
    }
    for (b = 0; b < B; ++b) {
        const int32_t* x = tokens + b * k;
        const int64_t r0 = b * (k + 1);
        int32_t r = k;
        for (i = 0; i <= k; ++i) {
            if (argmax_out) argmax_out[r0 + i] = (int32_t)g[r0 + i];
            if (top2_gap) top2_gap[r0 + i] = best[r0 + i] - second[r0 + i];
        }
        if (!tokens_valid(x, k, V)) {
            accepted_len[b] = -1;
            for (i = 0; i <= k; ++i) out_tokens[r0 + i] = -1;
            continue;
        }
        for (i = 0; i < k; ++i) {
            if (x[i] != g[r0 + i]) {
                r = i;
                break;
            }
        }
        accepted_len[b] = r;
        for (i = 0; i <= k; ++i) {
            if (i < r) out_tokens[r0 + i] = x[i];
            else if (i == r) out_tokens[r0 + i] = (int32_t)g[r0 + i];  /* the target's token */
            else out_tokens[r0 + i] = -1;
        }
    }
    free(h);
    free(g);
    return 0;
}

/* Logits formed from hidden states: out[row][y] = sum_d h_row[d] w_y[d] in
 * fp64 from bf16 hidden states h [rows][D] and output-layer weights w [V][D]
 * (no bias).  Each weight row is decoded once and dotted with every hidden
 * row; each dot product is the plain sequential sum over d.  With T > 0 the
 * verification rule then runs on these rows unchanged (orc_verify with
 * ORC_F64 logits). */
int orc_lm_head_logits(int64_t rows, int64_t V, int64_t D, const uint16_t* hidden, const uint16_t* weight,
                       double* out) {
    int64_t r, y, d;
    double *h, *wy;
    if (rows < 0 || V < 1 || D < 1 || !hidden || !weight || !out) return -1;
    h = (double*)malloc(sizeof(double) * (rows * D + D + 1));
    if (!h) return -1;
    wy = h + rows * D;
    for (r = 0; r < rows; ++r)
        for (d = 0; d < D; ++d) h[r * D + d] = orc_decode_bf16(hidden[r * D + d]);
    for (y = 0; y < V; ++y) {
        for (d = 0; d < D; ++d) wy[d] = orc_decode_bf16(weight[y * D + d]);
        for (r = 0; r < rows; ++r) {
            const double* hr = h + r * D;
            double s = 0.0;
            for (d = 0; d < D; ++d) s += hr[d] * wy[d];
            out[r * V + y] = s;
        }
    }
    free(h);
    return 0;
}
