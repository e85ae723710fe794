/*
 * specverify.h -- C ABI of libspecverify: batched lossless speculative-sampling
 * verification and verification-aware-training (VAT) labels on MI355X (gfx950).
 *
 * What the operations compute (sources: page title, then section):
 *
 *  sv_verify   -- "AI 开始抄自己的作业——而且抄得理直气壮" (NgramRL essay,
 *                 zhichai.net), section "投机解码：让草稿先跑，考官殿后":
 *                 for each sequence the draft proposes k tokens x_0..x_{k-1};
 *                 one target forward gives k+1 next-token distributions; token
 *                 x_i is kept with probability min(1, p_i(x_i)/q_i(x_i)); the
 *                 chain stops at the first rejection r, where the target
 *                 supplies one token drawn from the residual max(0, p_r - q_r)
 *                 renormalised; if all k are kept the target supplies a bonus
 *                 token from its last distribution p_k.  Same page, section
 *                 "考官坐镇：为什么抄作业不算作弊": the result is distributed
 *                 exactly as sampling from the target alone.
 *                 "NgramRL：用Rollout历史加速RL后训练的推测解码新方案"
 *                 (kongchang.com), section "自适应 fan-out 预取": the outcome
 *                 of one step is (accepted length j, target-supplied token b),
 *                 here (accepted_len[b], out_tokens[b][accepted_len[b]]).
 *
 *  sv_vat_labels -- "让AI草稿模型学会“照镜子”：训练时就知道自己会不会被打回"
 *                 (VAT write-up), section "VAT怎么把“验收规则”塞进训练里":
 *                 training runs the same acceptance rule on each draft block
 *                 and labels every position from the first rejection on as
 *                 rejected; section "第二件事，改权重分配的锚点": positions
 *                 before the first rejection r get weight 1 and the decay
 *                 curve restarts at r (weight decay^(i-r) for i >= r).
 *
 *  sv_accept_histogram, sv_draft_len_init, sv_draft_len_update --
 *                 EfficientRollout write-up (qunfachuanzhen.com), section
 *                 "四、自适应草稿长度": the draft length is picked from a fixed
 *                 set (5, 7, 9, 11 in the experiments), starting from the
 *                 shortest; after every training step the block efficiency
 *                 (tokens a draft-verify cycle commits) is measured; the
 *                 length moves up when two consecutive steps run close to
 *                 the current length's limit, down when they run too low,
 *                 and waits two steps so that one noisy step moves nothing.
 *                 NgramRL summary, section "自适应 fan-out 预取": the
 *                 distribution P(j) of accepted lengths is the statistic a
 *                 prefetcher plans with; the histogram is that distribution.
 *
 *  sv_vat_loss -- the same page and sections, with the end of section
 *                 "第二件事，改权重分配的锚点": the drafter's training loss
 *                 combines soft-label distillation from the target's output
 *                 distribution with hard-label supervision from the token the
 *                 target actually sampled.  Per position: soft term
 *                 -sum_y p(y) ln q(y) (cross entropy of the draft against the
 *                 target), hard term -ln q(h); per block:
 *                 sum_i w_i (soft_i + hard_weight * hard_i) with the VAT
 *                 weights w_i.  Labels, weights and losses come from one pass
 *                 over the logits.
 *
 * Readings this library takes where the pages leave a step open:
 *  - p = softmax(target_logits / T), q = softmax(draft_logits / T), one T;
 *  - acceptance: x_i is kept iff u[b][i] * q_i(x_i) < p_i(x_i);
 *  - the single draw uses u[b][k] and inverts the cumulative weight in
 *    ascending token id: smallest y with C(y) > u * C(V-1);
 *  - T == 0 is greedy: the target's choice g_i is the first (lowest-id)
 *    maximum of the raw logits; x_i is kept iff x_i == g_i; the target's token
 *    is g_r; uniforms and draft logits are not read;
 *  - one-hot drafts (SV_DRAFT_ONEHOT): q_i is the indicator of x_i, so x_i is
 *    kept iff u < p_i(x_i) and the residual is p_r with x_r removed;
 *  - positions of out_tokens after accepted_len are -1.
 *
 * Conventions shared by every entry point:
 *  - Shapes are row-major with the vocabulary contiguous.  Logits are either
 *    IEEE binary32 (SV_F32) or bfloat16 (SV_BF16, the top half of binary32).
 *  - Ownership: every array is caller-owned DEVICE memory on the current HIP
 *    device; descriptors, probe records and size out-parameters are host
 *    memory.  The library allocates nothing and keeps no per-call state.
 *  - Asynchrony: compute entry points enqueue kernels on `stream` and return;
 *    outputs are valid once the stream reaches that point.
 *  - Errors: arguments are checked on the host before anything is enqueued;
 *    on any error nothing is launched and no output or workspace byte is
 *    touched.  A failed launch returns SV_ERR_HIP (a workspace used by a call
 *    that returned SV_ERR_HIP must be zero-filled again before reuse).
 *  - Workspace queries (`*_workspace_bytes`) return the bytes a call with
 *    that descriptor needs; a valid descriptor always needs at least 256, so
 *    0 means the descriptor is NULL or invalid (the compute call then
 *    returns the reason).
 *  - Inside one call, blocks hand partial results to later blocks of the same
 *    grid through the workspace and wait for them with a bounded poll (about
 *    one second).  If a wait runs out (it cannot while the device dispatches
 *    blocks in grid order, as gfx950 does), the kernel still ends normally and
 *    the block that owns the affected output reports it: accepted_len = -2
 *    (first_reject = -2, mask 0, weights 0 for VAT) when the wait for a
 *    sequence's partials ran out, out_tokens[b][accepted_len[b]] = -2 when the
 *    wait of the draw of the target's token ran out.
 *  - Data checks done on the device: a sequence (block) holding a draft token
 *    outside [0, V) is flagged (accepted_len = -1 / first_reject = -1, its
 *    out_tokens -1, mask 0, weights 0) and never indexes memory with that
 *    token.  Uniforms outside [0,1), NaN logits or rows that are all -inf
 *    give unspecified (but in-bounds) results.
 *  - Tagged workspaces (sv_verify, sv_vat_labels, sv_vat_loss and their _ex
 *    forms, which may share one workspace): allocate it on the device and
 *    zero-fill it once before first use; every call that returns SV_OK leaves
 *    it ready for the next call.  Each call tags the words it hands between
 *    blocks with a call number from a process-wide 64-bit counter (mapped to
 *    1 .. 2^32 - 1, so two consecutive calls never share a number and a
 *    zero-filled word matches none).  The number is a kernel argument, so
 *    these calls cannot be captured into a HIP graph (every replay would
 *    reuse it): they return SV_ERR_CAPTURING while `stream` is capturing.  A
 *    buffer that anything else has written since (the LM-head entry points
 *    included) must be zero-filled again before one of them uses it.  Calls
 *    that use the same workspace must not overlap in time.  sv_verify also
 *    keeps each sequence's first rejection in the workspace: small one-hot
 *    and greedy calls read it back to decide how early they read the rows of
 *    later positions, which changes their speed, never their results.  The
 *    LM-head entry points and sv_vat_loss_grad hand nothing between blocks
 *    through tags and may be captured.
 *  - Determinism: results are bitwise reproducible for identical inputs (no
 *    floating-point atomics; fixed reduction orders).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_ABI_VERSION 7
#define SV_MAX_DRAFT 64 /* k is limited to one 64-lane wavefront */
#define SV_MAX_DRAFT_CHOICES 8

/* Status codes.  The first seven are the core contract of sv_verify and
 * sv_vat_labels; the later ones belong to options and entry points beyond it. */
typedef enum sv_status {
    SV_OK = 0,
    SV_ERR_NULL_ARG = 1,          /* a required pointer is NULL */
    SV_ERR_BAD_SHAPE = 2,         /* B/N < 0, k outside [1,64], V outside [1, 2^24], or size overflow */
    SV_ERR_BAD_DTYPE = 3,         /* dtype not SV_F32 / SV_BF16 */
    SV_ERR_BAD_TEMPERATURE = 4,   /* T not 0 and not a finite value >= 1e-4 */
    SV_ERR_WORKSPACE_TOO_SMALL = 5,
    SV_ERR_HIP = 6,               /* a kernel launch, event record or stream query failed */
    SV_ERR_BAD_DRAFT_KIND = 7,    /* draft_kind not SV_DRAFT_LOGITS / SV_DRAFT_ONEHOT */
    SV_ERR_BAD_DECAY = 8,         /* VAT decay not in [0, 1] */
    SV_ERR_BAD_HARD_WEIGHT = 9,   /* VAT loss hard_weight not finite and >= 0 */
    SV_ERR_BAD_CONTROL = 10,      /* draft-length controller thresholds out of range */
    SV_ERR_MISALIGNED = 11,       /* an array that must be 16-byte aligned is not */
    SV_ERR_CAPTURING = 12,        /* a tagged call on a stream that is being captured into a graph */
    SV_ERR_SCRATCH_TOO_SMALL = 13 /* sv_verify_noalloc: the call needs more than SV_NOALLOC_SCRATCH_BYTES */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

typedef enum sv_draft_kind { SV_DRAFT_LOGITS = 0, SV_DRAFT_ONEHOT = 1 } sv_draft_kind;

/* Shape and options of one sv_verify call. */
typedef struct sv_verify_desc {
    int32_t B;                 /* sequences, >= 0 (0: nothing to do) */
    int32_t k;                 /* draft positions per sequence, in [1, 64] */
    int32_t V;                 /* vocabulary size, >= 1 */
    sv_dtype dtype;            /* of both logit arrays */
    sv_draft_kind draft_kind;  /* draft logits, or one-hot draft (tokens only) */
    float temperature;         /* T: 0 (greedy) or finite >= 1e-4 */
} sv_verify_desc;

/* Shape and options of one sv_vat_labels call. */
typedef struct sv_vat_desc {
    int32_t N;                 /* draft blocks, >= 0 */
    int32_t k;                 /* positions per block, in [1, 64] */
    int32_t V;                 /* vocabulary size, >= 1 */
    sv_dtype dtype;
    float temperature;         /* T: 0 (greedy labels) or finite >= 1e-4 */
    float decay;               /* weight decay per position after the first rejection, in [0, 1] */
} sv_vat_desc;

/* Shape and options of one sv_vat_loss / sv_vat_loss_grad call. */
typedef struct sv_vat_loss_desc {
    int32_t N;                 /* draft blocks, >= 0 */
    int32_t k;                 /* positions per block, in [1, 64] */
    int32_t V;                 /* vocabulary size, >= 1 */
    sv_dtype dtype;
    float temperature;         /* T: finite >= 1e-4 (both distributions are needed) */
    float decay;               /* as for sv_vat_desc, in [0, 1] */
    float hard_weight;         /* weight of the hard-label term, finite >= 0 */
} sv_vat_loss_desc;

/* Shape of one sv_verify_lm_head_greedy call. */
typedef struct sv_lm_head_desc {
    int32_t B;                 /* sequences, >= 0 */
    int32_t k;                 /* draft positions, in [1, 64] */
    int32_t V;                 /* rows of the output layer, in [1, 2^24] */
    int32_t D;                 /* hidden size, a multiple of 64 in [64, 65536] */
} sv_lm_head_desc;

/* Shape and options of one sv_verify_lm_head call (sampling). */
typedef struct sv_lm_head_sample_desc {
    int32_t B;                 /* sequences, >= 0 */
    int32_t k;                 /* draft positions, in [1, 64] */
    int32_t V;                 /* rows of each output layer, in [1, 2^24] */
    int32_t D;                 /* hidden size, a multiple of 64 in [64, 65536] */
    float temperature;         /* T: finite >= 1e-4 (T == 0 is sv_verify_lm_head_greedy) */
} sv_lm_head_sample_desc;

/* Optional instrumentation of one call (host memory, may be NULL): two HIP
 * events, both non-NULL, recorded on `stream` immediately before and after
 * the call's main kernel (sv_verify, sv_vat_labels, sv_vat_loss: its single
 * launch; sv_vat_loss_grad: its single launch; the LM-head calls: the GEMM). */
typedef struct sv_probe {
    hipEvent_t start;
    hipEvent_t stop;
} sv_probe;

/* Returns SV_ABI_VERSION of the built library. */
int sv_abi_version(void);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* sv_status_str(sv_status status);

/* Workspace bytes sv_verify needs for `desc` (0: desc NULL or invalid). */
size_t sv_verify_workspace_bytes(const sv_verify_desc* desc);

/*
 * Batched verification.  Source: NgramRL essay, section "投机解码：让草稿先跑，
 * 考官殿后" (acceptance rule, truncation, residual / bonus token); NgramRL
 * summary, section "自适应 fan-out 预取" (outcome pair).
 *
 *  target_logits  device, [B][k+1][V] dtype: target logits at positions 0..k
 *  draft_logits   device, [B][k][V] dtype; read only when draft_kind is
 *                 SV_DRAFT_LOGITS and T > 0 (may be NULL otherwise)
 *  draft_tokens   device, [B][k] int32: proposed tokens, expected in [0, V)
 *  uniforms       device, [B][k+1] float32 in [0,1): column i < k drives test i,
 *                 column k the single residual / bonus draw; unused (may be
 *                 NULL) at T == 0
 *  accepted_len   device out, [B] int32 in [0, k] (-1: invalid token, -2: wait
 *                 timed out)
 *  out_tokens     device out, [B][k+1] int32: x_0..x_{r-1}, then the target's
 *                 token at r, then -1
 *  probs_out      device out or NULL, [B][k][2] float32: (p_i(x_i), q_i(x_i))
 *                 for every position (T == 0: ([x_i == g_i], 1))
 *  workspace      device, >= sv_verify_workspace_bytes(desc) bytes, zero-filled
 *                 once (see "Tagged workspaces" above)
 *  stream         HIP stream the kernel is enqueued on (0 = null stream)
 *
 * Errors (nothing launched): SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE,
 * SV_ERR_BAD_DTYPE, SV_ERR_BAD_TEMPERATURE, SV_ERR_BAD_DRAFT_KIND,
 * SV_ERR_WORKSPACE_TOO_SMALL, SV_ERR_CAPTURING.  Launch failure: SV_ERR_HIP.
 */
sv_status sv_verify(const sv_verify_desc* desc, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len,
                    int32_t* out_tokens, float* probs_out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * sv_verify with two additions (same source):
 *  row_stats_out  device out or NULL, [B(k+1) + B k][2] float32, target rows
 *                 then draft rows (one-hot or T == 0: target rows only):
 *                 (m, Z) with m = max_y l(y)/T and Z = sum_y exp(l(y)/T - m);
 *                 at T == 0: (max_y l(y), first argmax as a float)
 *  probe          host, NULL or the events that bracket the kernel launch
 * Errors as for sv_verify, plus SV_ERR_HIP if an event record fails.
 */
sv_status sv_verify_ex(const sv_verify_desc* desc, const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len,
                       int32_t* out_tokens, float* probs_out, float* row_stats_out, const sv_probe* probe,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the workspace built into the library for sv_verify_noalloc. */
#define SV_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * sv_verify without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory at the call (tight serving
 * loops, harnesses that forbid allocation).  The hand-off words live in an
 * array of SV_NOALLOC_SCRATCH_BYTES built into the library, one per device,
 * held until the process ends; the first call on a device looks its address
 * up and zero-fills it with a kernel on `stream`.  Arguments, outputs and
 * errors are those of sv_verify, plus SV_ERR_SCRATCH_TOO_SMALL when
 * sv_verify_workspace_bytes(desc) exceeds SV_NOALLOC_SCRATCH_BYTES (nothing
 * launched; about 4 MB covers B = 320, k = 7, V = 151936 bf16 logits).
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (different streams, or host threads) race and must not
 * be issued; calls in order on one stream are safe.  Not capturable
 * (SV_ERR_CAPTURING), as for the other tagged calls.
 */
sv_status sv_verify_noalloc(const sv_verify_desc* desc, const void* target_logits, const void* draft_logits,
                            const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len,
                            int32_t* out_tokens, float* probs_out, hipStream_t stream);

/* Workspace bytes sv_vat_labels needs for `desc` (0: NULL or invalid). */
size_t sv_vat_workspace_bytes(const sv_vat_desc* desc);

/*
 * VAT labels.  Source: VAT write-up, sections "VAT怎么把“验收规则”塞进训练里"
 * (simulated verification, labels) and "第二件事，改权重分配的锚点" (weights).
 *
 *  target_logits  device, [N][k][V] dtype: target logits at the k drafted
 *                 positions of each block (no bonus row)
 *  draft_logits   device, [N][k][V] dtype (unused, may be NULL, at T == 0)
 *  draft_tokens   device, [N][k] int32
 *  uniforms       device, [N][k] float32 in [0,1) (unused at T == 0)
 *  accept_mask    device out, [N][k] uint8: 1 before the first rejection, else 0
 *  first_reject   device out, [N] int32: r in [0,k], k = no rejection (-1: invalid
 *                 token, -2: wait timed out)
 *  weights        device out, [N][k] float32: 1 for i < r, decay^(i-r) for i >= r
 *  probs_out      device out or NULL, [N][k][2] float32 (p_i(x_i), q_i(x_i))
 *  workspace, workspace_bytes, stream: as for sv_verify
 *
 * Errors as for sv_verify (SV_ERR_BAD_DRAFT_KIND excepted), plus
 * SV_ERR_BAD_DECAY.
 */
sv_status sv_vat_labels(const sv_vat_desc* desc, const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms, uint8_t* accept_mask,
                        int32_t* first_reject, float* weights, float* probs_out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * sv_vat_labels with row_stats_out (device out or NULL, [N k + N k][2]
 * float32, target rows then draft rows, as for sv_verify_ex) and a probe.
 */
sv_status sv_vat_labels_ex(const sv_vat_desc* desc, const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, const float* uniforms, uint8_t* accept_mask,
                           int32_t* first_reject, float* weights, float* probs_out, float* row_stats_out,
                           const sv_probe* probe, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes sv_vat_loss needs for `desc` (0: NULL or invalid; T == 0
 * is invalid here). */
size_t sv_vat_loss_workspace_bytes(const sv_vat_loss_desc* desc);

/*
 * VAT labels, weights and the weighted training loss in one pass.  Source:
 * VAT write-up, sections "VAT怎么把“验收规则”塞进训练里" and
 * "第二件事，改权重分配的锚点" (labels, weights; soft plus hard labels).
 *
 *  target_logits, draft_logits  device, [N][k][V] dtype (both required)
 *  draft_tokens   device, [N][k] int32: the draft's proposals (simulated test)
 *  uniforms       device, [N][k] float32 in [0,1)
 *  hard_tokens    device, [N][k] int32: the target's sampled token at each
 *                 position (the hard label), expected in [0, V)
 *  accept_mask, first_reject, weights: as for sv_vat_labels
 *  soft_ce        device out, [N][k] float32: -sum_y p_i(y) ln q_i(y) (nats)
 *  hard_ce        device out, [N][k] float32: -ln q_i(h_i)
 *  block_loss     device out, [N] float32: sum_i w_i (soft_i + hard_weight hard_i)
 *  probs_out      device out or NULL, [N][k][2] float32 (p_i(x_i), q_i(x_i))
 *  row_stats_out  device out or NULL, [N k + N k][2] float32, as for
 *                 sv_vat_labels_ex (sv_vat_loss_grad consumes it)
 *  probe          host, NULL or the events that bracket the kernel launch
 *  workspace, workspace_bytes, stream: as for sv_verify
 *
 * A block holding a draft or hard token outside [0, V) gets first_reject -1,
 * mask 0, weights 0 and NaN losses.  Draft logits of -inf where the target
 * has positive mass make the exact soft or hard term +inf; the returned
 * value is then unspecified.
 * Errors as for sv_vat_labels, plus SV_ERR_BAD_HARD_WEIGHT.
 */
sv_status sv_vat_loss(const sv_vat_loss_desc* desc, const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms, const int32_t* hard_tokens,
                      uint8_t* accept_mask, int32_t* first_reject, float* weights, float* soft_ce, float* hard_ce,
                      float* block_loss, float* probs_out, float* row_stats_out, const sv_probe* probe,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gradient of the VAT training loss with respect to the draft logits, for
 * the backward pass of drafter training.  Source: VAT write-up, section
 * "第二件事，改权重分配的锚点" (the weighted soft-plus-hard-label loss that
 * sv_vat_loss computes); the derivative is taken with the VAT weights held
 * fixed, as labels of the simulated verification:
 *   grad[n][i][y] = w_i / T * ((1 + hard_weight) q_i(y) - p_i(y) - hard_weight [y == h_i]),
 * p_i = softmax(l_t/T), q_i = softmax(l_d/T).  It consumes what sv_vat_loss
 * wrote for the same logits and descriptor (its weights and row_stats_out).
 *
 *  desc           as for sv_vat_loss (decay unused here)
 *  target_logits, draft_logits  device, [N][k][V] dtype
 *  hard_tokens    device, [N][k] int32, as for sv_vat_loss
 *  weights        device, [N][k] float32: the weights sv_vat_loss wrote
 *  row_stats      device, [N k + N k][2] float32: sv_vat_loss's row_stats_out
 *  grad           device out, [N][k][V] float32 (16-byte aligned with V a
 *                 multiple of 4 for the vector path; any alignment works)
 *  probe          host, NULL or the events that bracket the kernel
 *  stream         HIP stream
 *
 * A position of weight 0 (a flagged block, or decay 0 after the first
 * rejection) gets a row of zeros and its logits are not read.  One streaming
 * kernel: reads both logit rows once and writes the gradient row once.
 * Errors (nothing launched): SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE,
 * SV_ERR_BAD_DTYPE, SV_ERR_BAD_TEMPERATURE (T == 0 included),
 * SV_ERR_BAD_HARD_WEIGHT.  Launch failure: SV_ERR_HIP.
 */
sv_status sv_vat_loss_grad(const sv_vat_loss_desc* desc, const void* target_logits, const void* draft_logits,
                           const int32_t* hard_tokens, const float* weights, const float* row_stats, float* grad,
                           const sv_probe* probe, hipStream_t stream);

/* Workspace bytes sv_verify_lm_head_greedy needs for `desc` (0: NULL or
 * invalid). */
size_t sv_lm_head_workspace_bytes(const sv_lm_head_desc* desc);

/*
 * Greedy (T == 0) verification with the target's logits formed from its
 * final hidden states and output-layer weights inside the call, so that the
 * [B][k+1][V] logits never reach memory.  Source: NgramRL essay, section
 * "投机解码：让草稿先跑，考官殿后" (the rule, read at T == 0 as above: the
 * target's choice is its lowest-index argmax, a draft token is kept iff it
 * equals it); the target's logit at a position is the dot product of the
 * hidden state with the output layer's row of that token.  EfficientRollout
 * write-up, section "二、量化压缩：从大模型里“变”出一个代笔助理": in the tail
 * phase most of a forward's time goes to loading dense weights, the output
 * (LM-head) layer among them; this call reads that layer once for all
 * B(k+1) positions.
 *
 *  hidden_states  device, [B][k+1][D] bfloat16, 16-byte aligned: the target's
 *                 final hidden state at positions 0..k
 *  weight         device, [V][D] bfloat16, 16-byte aligned: output layer,
 *                 row y gives token y's logit
 *  draft_tokens   device, [B][k] int32, expected in [0, V)
 *  accepted_len   device out, [B] int32 in [0, k] (-1: invalid token)
 *  out_tokens     device out, [B][k+1] int32, as for sv_verify
 *  argmax_out     device out or NULL, [B][k+1] int32: every position's
 *                 choice (written for invalid sequences too)
 *  probe          host, NULL or the events that bracket the GEMM launch
 *  workspace      device, >= sv_lm_head_workspace_bytes bytes (needs no
 *                 clearing: every byte read is written earlier in the call)
 *  stream         HIP stream the two kernels are enqueued on
 *
 * Arithmetic: bf16 x bf16 products accumulated in fp32 on the matrix cores;
 * the accumulation order differs from a sequential sum, so a position whose
 * two largest logits lie within rounding of each other may pick either.
 * Errors (nothing launched): SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE (also when
 * B(k+1) D >= 2^31), SV_ERR_MISALIGNED, SV_ERR_WORKSPACE_TOO_SMALL.  Launch
 * failure: SV_ERR_HIP.
 */
sv_status sv_verify_lm_head_greedy(const sv_lm_head_desc* desc, const void* hidden_states, const void* weight,
                                   const int32_t* draft_tokens, int32_t* accepted_len, int32_t* out_tokens,
                                   int32_t* argmax_out, const sv_probe* probe, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes sv_verify_lm_head needs for `desc` (0: NULL or invalid):
 * about (2k+1) (8 B ceil(V/256) + 4 B V) per sequence (every row's fp32
 * logits dominate: 856 MB at B = 128, k = 5, V = 151936). */
size_t sv_lm_head_sample_workspace_bytes(const sv_lm_head_sample_desc* desc);

/*
 * Speculative-sampling verification (T > 0) with the target's and the
 * draft's logits formed from their hidden states and output layers inside
 * the call.  Source: NgramRL essay, section "投机解码：让草稿先跑，考官殿后"
 * (the rule, as for sv_verify with draft logits: p = softmax(l_t / T),
 * q = softmax(l_d / T), x_i kept iff u_i q_i(x_i) < p_i(x_i), the draw at the
 * first rejection from max(0, p_r - q_r) renormalised, or from p_k after full
 * acceptance, with u[b][k], inverting the cumulative weight in ascending
 * token order).  Logits: l(y) = h . w_y, bf16 inputs, fp32 accumulation.  The
 * softmax statistics of every row come from one pass over both output layers,
 * whose epilogue also writes every row's fp32 logits into the workspace
 * (the GEMM is bound by the matrix cores, so the writes cost little memory
 * time); the draw then reads its two rows (target row r, or k, and draft
 * row r) from there instead of forming them again.
 *
 *  target_hidden  device, [B][k+1][D] bf16, 16-byte aligned
 *  target_weight  device, [V][D] bf16, 16-byte aligned
 *  draft_hidden   device, [B][k][D] bf16, 16-byte aligned
 *  draft_weight   device, [V][D] bf16, 16-byte aligned (may be target_weight)
 *  draft_tokens   device, [B][k] int32, expected in [0, V)
 *  uniforms       device, [B][k+1] float32 in [0,1), as for sv_verify
 *  accepted_len   device out, [B] int32 in [0, k] (-1: invalid token)
 *  out_tokens     device out, [B][k+1] int32, as for sv_verify
 *  probs_out      device out or NULL, [B][k][2] float32 (p_i(x_i), q_i(x_i))
 *  probe          host, NULL or the events that bracket the statistics GEMM
 *  workspace      device, >= sv_lm_head_sample_workspace_bytes bytes (needs no
 *                 clearing)
 *
 * Errors (nothing launched): SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE,
 * SV_ERR_BAD_TEMPERATURE, SV_ERR_MISALIGNED, SV_ERR_WORKSPACE_TOO_SMALL.
 * Launch failure: SV_ERR_HIP.
 */
sv_status sv_verify_lm_head(const sv_lm_head_sample_desc* desc, const void* target_hidden, const void* target_weight,
                            const void* draft_hidden, const void* draft_weight, const int32_t* draft_tokens,
                            const float* uniforms, int32_t* accepted_len, int32_t* out_tokens, float* probs_out,
                            const sv_probe* probe, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Histogram of accepted lengths (device in, device out).
 *  accepted_len  device, [B] int32 as written by sv_verify
 *  hist          device out, [k + 4] int32: hist[j] = #sequences with
 *                accepted_len == j for j in [0, k]; hist[k+1] = #(-1, invalid
 *                token); hist[k+2] = #(-2, wait timed out); hist[k+3] = #other
 * Counts are exact.  One small kernel on `stream`.
 * Errors: SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE (B < 0 or k outside [1, 64]),
 * SV_ERR_HIP.
 */
sv_status sv_accept_histogram(const int32_t* accepted_len, int32_t batch, int32_t k, int32_t* hist,
                              hipStream_t stream);

/* State of the draft-length controller: host memory, owned by the caller. */
typedef struct sv_draft_len_ctl {
    int32_t n_choices;                      /* 1 .. SV_MAX_DRAFT_CHOICES */
    int32_t choices[SV_MAX_DRAFT_CHOICES];  /* strictly increasing draft lengths in [1, 64] */
    int32_t index;                          /* current choice (starts at 0, the shortest) */
    float up_frac;                          /* move up when efficiency >= up_frac * (k+1) ... */
    float down_frac;                        /* move down when efficiency <= down_frac * (k+1) ... */
    int32_t patience;                       /* ... on this many consecutive steps */
    int32_t up_streak, down_streak;
    float last_efficiency;                  /* the last step's block efficiency */
} sv_draft_len_ctl;

/* Initialises `ctl` (host).  0 <= down_frac < up_frac <= 1, patience >= 1.
 * Errors: SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE (choices), SV_ERR_BAD_CONTROL. */
sv_status sv_draft_len_init(sv_draft_len_ctl* ctl, const int32_t* choices, int32_t n_choices, float up_frac,
                            float down_frac, int32_t patience);

/* One step of the controller (host).  hist: HOST copy of sv_accept_histogram's
 * output for a step run at draft length k (= the current choice).  Block
 * efficiency = sum_j (j+1) hist[j] / sum_j hist[j] over j in [0, k] (accepted
 * drafts plus the target's token, per cycle; at most k+1).  Writes the draft
 * length for the next step to *next_k.  A histogram with no valid sequence
 * changes nothing.  Errors: SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE (k is not the
 * current choice). */
sv_status sv_draft_len_update(sv_draft_len_ctl* ctl, const int32_t* hist, int32_t k, int32_t* next_k);

/*
 * Speed-of-light references (measurement only; no passage of the pages
 * defines them).  Plain streaming kernels with the memory traffic of the
 * calls above and none of their arithmetic, so that a call's duration can be
 * stated as a fraction of the fastest pass over the same bytes on the same
 * device.
 *
 * sv_sol_read: reads `bytes` bytes at `data` (device) once with 16-byte
 * non-temporal loads, the traffic of sv_verify and sv_vat_labels (every
 * logit read once, only small outputs written).
 *  data   device, 16-byte aligned; bytes a multiple of 16 (0: nothing runs)
 *  sink   device, one uint32; written only if the XOR of the words one lane
 *         loads equals a fixed constant (it keeps the loads from being
 *         optimised away)
 * Errors: SV_ERR_NULL_ARG, SV_ERR_MISALIGNED (data or bytes not 16-byte
 * multiples), SV_ERR_BAD_SHAPE (too large for one launch), SV_ERR_HIP.
 */
sv_status sv_sol_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * sv_sol_read_write: out[i] = a[i] - b[i] in fp32 for i in [0, n): two logit
 * arrays read, one fp32 array written, the traffic of sv_vat_loss_grad
 * (target and draft logits in, the gradient out).
 *  a, b   device, [n] elements of `dtype`, 16-byte aligned
 *  out    device, [n] fp32, 16-byte aligned; may not overlap a or b
 *  n      a multiple of 4 (SV_F32) or 8 (SV_BF16); 0: nothing runs
 * Errors: SV_ERR_NULL_ARG, SV_ERR_BAD_DTYPE, SV_ERR_MISALIGNED (pointers or
 * n), SV_ERR_BAD_SHAPE (n < 0 or too large for one launch), SV_ERR_HIP.
 */
sv_status sv_sol_read_write(const void* a, const void* b, float* out, int64_t n, sv_dtype dtype,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
