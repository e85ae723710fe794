// C ABI of libspecverify: host-side argument checks, workspace planning and
// dispatch to the gfx950 kernels.  Every check runs before anything is
// enqueued, so an error return leaves all outputs and the workspace untouched.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include "sv_launch.h"
#include "sv_lmhead.h"
#include "specverify.h"

namespace sv {

namespace {

constexpr int64_t kMaxVocab = int64_t{1} << 24;
constexpr float kMinTemperature = 1e-4f;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool temperature_ok(float t) { return t == 0.f || (std::isfinite(t) && t >= kMinTemperature); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tag of this call's hand-off words (see kTagFirst): consecutive calls get
// consecutive tags, so words left by an earlier call never match.
uint32_t next_tag() {
    static std::atomic<uint32_t> calls{0};
    return kTagFirst + calls.fetch_add(1u, std::memory_order_relaxed) % kTagCount;
}

struct Shape {
    int64_t batch, k, vocab;
    int elem_bytes;
    int64_t target_rows_per_seq;
    int64_t rows_t, rows_d;
    int64_t chunk, chunks;
    bool greedy, onehot, vat;
    bool loss;  // VAT with the training loss
};

// Shared checks of both entry points.  `draft_kind` is SV_DRAFT_LOGITS for VAT.
sv_status check_shape(int32_t batch, int32_t k, int32_t vocab, int32_t dtype, int32_t draft_kind,
                      float temperature, bool vat, Shape* s) {
    if (batch < 0 || k < 1 || k > SV_MAX_DRAFT || vocab < 1 || vocab > kMaxVocab) return SV_ERR_BAD_SHAPE;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_BAD_DTYPE;
    if (!temperature_ok(temperature)) return SV_ERR_BAD_TEMPERATURE;
    if (draft_kind != SV_DRAFT_LOGITS && draft_kind != SV_DRAFT_ONEHOT) return SV_ERR_BAD_DRAFT_KIND;
    s->batch = batch;
    s->k = k;
    s->vocab = vocab;
    s->elem_bytes = dtype == SV_BF16 ? 2 : 4;
    s->greedy = temperature == 0.f;
    s->onehot = draft_kind == SV_DRAFT_ONEHOT;
    s->vat = vat;
    s->loss = false;
    s->target_rows_per_seq = vat ? k : k + 1;
    s->rows_t = s->batch * s->target_rows_per_seq;
    s->rows_d = (s->greedy || s->onehot) ? 0 : s->batch * k;
    s->chunk = chunk_elems(s->elem_bytes);
    s->chunks = ceil_div(vocab, s->chunk);
    // Byte offsets of the largest logit array must fit in int64.
    const double bytes = static_cast<double>(s->rows_t + s->batch * k) * vocab * s->elem_bytes;
    if (bytes > 4.0e18) return SV_ERR_BAD_SHAPE;
    return SV_OK;
}

// Tagged words of chunk partials: two per row chunk, or five per chunk pair
// for the VAT loss.
int64_t partial_words(const Shape& s) {
    return s.loss ? s.batch * s.k * s.chunks * kPairWords : (s.rows_t + s.rows_d) * s.chunks * 2;
}

size_t workspace_bytes_for(const Shape& s) {
    return workspace_layout(partial_words(s), s.batch, s.chunks).total;
}

bool fill_plan(const Shape& s, float temperature, float decay, Plan* pl) {
    pl->batch = static_cast<int32_t>(s.batch);
    pl->k = static_cast<int32_t>(s.k);
    pl->vocab = static_cast<int32_t>(s.vocab);
    pl->elem_bytes = s.elem_bytes;
    pl->target_rows_per_seq = static_cast<int32_t>(s.target_rows_per_seq);
    pl->chunks = static_cast<int32_t>(s.chunks);
    pl->chunk = static_cast<int32_t>(s.chunk);
    // The VAT loss streams k chunk-pair "rows" (target row i with draft row i).
    pl->dec_rows = static_cast<int32_t>(s.loss ? s.k : s.k + (s.rows_d ? s.k : 0));
    pl->has_bonus = !s.vat;
    pl->has_resid = !s.vat && !s.greedy && !s.onehot;
    pl->rows_per_seq = pl->dec_rows + (pl->has_bonus ? 1 : 0);
    pl->vat_loss = s.loss;
    pl->words_per_seq = static_cast<int32_t>(s.loss ? s.k * s.chunks * kPairWords : pl->rows_per_seq * s.chunks * 2);
    const bool small = s.batch * pl->dec_rows * s.chunks <= kSmallCallChunks;
    pl->nc_dec = small ? kChunksPerWaveSmall : kChunksPerWave;
    pl->two_deep_polls = small;
    pl->nc_res = kChunksPerWaveResid;
    pl->nc_bonus = std::min(pl->nc_dec, kChunksPerWaveBonus);
    if (!plan_task_grid(pl->batch, static_cast<int64_t>(pl->dec_rows) * s.chunks, s.chunks, pl->has_resid,
                        pl->has_bonus, kWavesPerBlock * pl->nc_dec, kWavesPerBlock * pl->nc_bonus,
                        kWavesPerBlock * pl->nc_res, kResidentBlocks, &pl->grid))
        return false;
    // The decisions of the sequences in the last residency of phase A come
    // after the bonus phase has started; their bonus rows are read without
    // waiting, so that reading them is not added to the end of the chain.
    pl->eager_bonus_from = std::max(0, pl->batch - pl->grid.lag_a);
    pl->rows_t = s.rows_t;
    pl->rows_d = s.rows_d;
    pl->greedy = s.greedy;
    pl->onehot = s.onehot;
    pl->vat = s.vat;
    pl->temperature = temperature;
    pl->c2 = s.greedy ? 0.f : static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
    pl->decay = decay;
    return true;
}

void carve_workspace(const Shape& s, void* ws, Plan* pl) {
    const WorkspaceLayout L = workspace_layout(partial_words(s), s.batch, s.chunks);
    char* base = static_cast<char*>(ws);
    pl->partials = reinterpret_cast<uint64_t*>(base + L.partials);
    pl->resid = reinterpret_cast<uint64_t*>(base + L.resid);
    pl->dec = reinterpret_cast<uint64_t*>(base + L.dec);
    pl->tag = next_tag();
}

// LM-head verification: shape checks and workspace layouts.
constexpr int64_t kMaxHidden = 65536;
constexpr int64_t kMaxRowElems = 0x7fffffffLL;  // hidden-state offsets are 32-bit

struct LmShape {
    int64_t batch, k, vocab, hidden, rows_t, rows_d, n_tiles;
};

sv_status check_lm_shape(int32_t batch, int32_t k, int32_t vocab, int32_t hidden, LmShape* s) {
    if (batch < 0 || k < 1 || k > SV_MAX_DRAFT || vocab < 1 || vocab > kMaxVocab || hidden < kLmHiddenMultiple ||
        hidden > kMaxHidden || hidden % kLmHiddenMultiple != 0)
        return SV_ERR_BAD_SHAPE;
    s->batch = batch;
    s->k = k;
    s->vocab = vocab;
    s->hidden = hidden;
    s->rows_t = s->batch * (k + 1);
    s->rows_d = s->batch * k;
    s->n_tiles = ceil_div(vocab, kLmBN);
    if (s->rows_t * s->hidden > kMaxRowElems) return SV_ERR_BAD_SHAPE;
    return SV_OK;
}

// Greedy: argmax partials (value and index) per target row and vocabulary tile.
size_t lm_greedy_workspace_bytes(const LmShape& s) {
    const size_t n = static_cast<size_t>(s.rows_t * s.n_tiles);
    return align_up(n * sizeof(float)) + align_up(n * sizeof(int32_t));
}

struct LmSampleLayout {
    size_t part_m, part_s, lx, seq, logits, total;
};

// Sampling: (m, s) partials per target and draft row and tile, the token
// logits, the per-sequence draw records and every row's fp32 logits.
LmSampleLayout lm_sample_layout(const LmShape& s) {
    LmSampleLayout L;
    const size_t rows = static_cast<size_t>(s.rows_t + s.rows_d);
    const size_t n = rows * static_cast<size_t>(s.n_tiles);
    size_t off = 0;
    L.part_m = off;
    off = align_up(off + n * sizeof(float));
    L.part_s = off;
    off = align_up(off + n * sizeof(float));
    L.lx = off;
    off = align_up(off + rows * sizeof(float));
    L.seq = off;
    off = align_up(off + static_cast<size_t>(s.batch) * sizeof(LmSeqDraw));
    L.logits = off;
    off = align_up(off + rows * static_cast<size_t>(s.vocab) * sizeof(float));
    L.total = off;
    return L;
}

void lm_common(const LmShape& s, LmPlan* pl) {
    pl->batch = static_cast<int32_t>(s.batch);
    pl->k = static_cast<int32_t>(s.k);
    pl->vocab = static_cast<int32_t>(s.vocab);
    pl->hidden = static_cast<int32_t>(s.hidden);
    pl->rows_t = static_cast<int32_t>(s.rows_t);
}

LmGemm lm_gemm(const void* a, const void* w, int64_t rows, int64_t out_row0, int32_t tokens) {
    LmGemm g{};
    g.a = static_cast<const uint16_t*>(a);
    g.w = static_cast<const uint16_t*>(w);
    g.rows = static_cast<int32_t>(rows);
    g.out_row0 = static_cast<int32_t>(out_row0);
    g.tokens = tokens;
    return g;
}

}  // namespace

WorkspaceLayout workspace_layout(int64_t partial_words, int64_t batch, int64_t chunks) {
    WorkspaceLayout L;
    size_t off = 0;
    L.partials = off;
    off = align_up(off + static_cast<size_t>(partial_words) * sizeof(uint64_t));
    L.resid = off;
    off = align_up(off + static_cast<size_t>(batch * chunks) * sizeof(uint64_t));
    L.dec = off;
    off = align_up(off + static_cast<size_t>(batch) * kDecWords * sizeof(uint64_t));
    L.total = off;
    return L;
}

}  // namespace sv

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_str(int status) {
    switch (status) {
        case SV_OK: return "SV_OK";
        case SV_ERR_NULL_ARG: return "SV_ERR_NULL_ARG: a required pointer is NULL";
        case SV_ERR_BAD_SHAPE: return "SV_ERR_BAD_SHAPE: batch < 0, k outside [1,64], vocab outside [1,2^24] or size overflow";
        case SV_ERR_BAD_DTYPE: return "SV_ERR_BAD_DTYPE: dtype must be SV_F32 or SV_BF16";
        case SV_ERR_BAD_TEMPERATURE: return "SV_ERR_BAD_TEMPERATURE: temperature must be 0 or finite and >= 1e-4";
        case SV_ERR_BAD_DRAFT_KIND: return "SV_ERR_BAD_DRAFT_KIND: draft_kind must be SV_DRAFT_LOGITS or SV_DRAFT_ONEHOT";
        case SV_ERR_BAD_HARD_WEIGHT: return "SV_ERR_BAD_HARD_WEIGHT: hard_weight must be finite and >= 0";
        case SV_ERR_BAD_CONTROL: return "SV_ERR_BAD_CONTROL: need 0 <= down_frac < up_frac <= 1";
        case SV_ERR_WORKSPACE_TOO_SMALL: return "SV_ERR_WORKSPACE_TOO_SMALL: workspace_bytes below the size query";
        case SV_ERR_BAD_DECAY: return "SV_ERR_BAD_DECAY: decay must be in [0, 1]";
        case SV_ERR_HIP: return "SV_ERR_HIP: a HIP launch or event record failed";
        case SV_ERR_MISALIGNED: return "SV_ERR_MISALIGNED: hidden_states and weight must be 16-byte aligned";
        default: return "unknown status";
    }
}

sv_status sv_verify_workspace_size(const sv_verify_desc* desc, size_t* bytes) {
    if (!desc || !bytes) return SV_ERR_NULL_ARG;
    sv::Shape s;
    const sv_status st = sv::check_shape(desc->batch, desc->num_draft, desc->vocab, desc->dtype, desc->draft_kind,
                                         desc->temperature, false, &s);
    if (st != SV_OK) return st;
    *bytes = sv::workspace_bytes_for(s);
    return SV_OK;
}

sv_status sv_verify(const sv_verify_desc* desc, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len, int32_t* out_tokens,
                    float* probs_out, float* row_stats_out, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::Shape s;
    sv_status st = sv::check_shape(desc->batch, desc->num_draft, desc->vocab, desc->dtype, desc->draft_kind,
                                   desc->temperature, false, &s);
    if (st != SV_OK) return st;
    if (s.batch == 0) return SV_OK;
    if (!target_logits || !draft_tokens || !accepted_len || !out_tokens) return SV_ERR_NULL_ARG;
    if (!s.greedy && !uniforms) return SV_ERR_NULL_ARG;
    if (s.rows_d && !draft_logits) return SV_ERR_NULL_ARG;
    const size_t need = sv::workspace_bytes_for(s);
    if (!workspace) return SV_ERR_NULL_ARG;
    if (workspace_bytes < need) return SV_ERR_WORKSPACE_TOO_SMALL;

    sv::Plan pl{};
    if (!sv::fill_plan(s, desc->temperature, 0.f, &pl)) return SV_ERR_BAD_SHAPE;
    pl.vec = (s.vocab * s.elem_bytes) % 16 == 0 && sv::aligned16(target_logits) &&
             (!s.rows_d || sv::aligned16(draft_logits));
    pl.target = target_logits;
    pl.draft = s.rows_d ? draft_logits : nullptr;
    pl.tokens = draft_tokens;
    pl.uniforms = uniforms;
    pl.accepted_len = accepted_len;
    pl.out_tokens = out_tokens;
    pl.probs_out = probs_out;
    pl.row_stats_out = row_stats_out;
    sv::carve_workspace(s, workspace, &pl);
    const hipError_t e = sv::launch_path(pl, stream, desc->probe_start, desc->probe_stop);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_vat_workspace_size(const sv_vat_desc* desc, size_t* bytes) {
    if (!desc || !bytes) return SV_ERR_NULL_ARG;
    sv::Shape s;
    const sv_status st = sv::check_shape(desc->blocks, desc->num_draft, desc->vocab, desc->dtype, SV_DRAFT_LOGITS,
                                         desc->temperature, true, &s);
    if (st != SV_OK) return st;
    if (!(desc->decay >= 0.f && desc->decay <= 1.f)) return SV_ERR_BAD_DECAY;
    *bytes = sv::workspace_bytes_for(s);
    return SV_OK;
}

sv_status sv_vat_labels(const sv_vat_desc* desc, const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms, uint8_t* accept_mask,
                        int32_t* first_reject, float* weights, float* probs_out, float* row_stats_out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::Shape s;
    sv_status st = sv::check_shape(desc->blocks, desc->num_draft, desc->vocab, desc->dtype, SV_DRAFT_LOGITS,
                                   desc->temperature, true, &s);
    if (st != SV_OK) return st;
    if (!(desc->decay >= 0.f && desc->decay <= 1.f)) return SV_ERR_BAD_DECAY;
    if (s.batch == 0) return SV_OK;
    if (!target_logits || !draft_tokens || !accept_mask || !first_reject || !weights) return SV_ERR_NULL_ARG;
    if (!s.greedy && (!uniforms || !draft_logits)) return SV_ERR_NULL_ARG;
    const size_t need = sv::workspace_bytes_for(s);
    if (!workspace) return SV_ERR_NULL_ARG;
    if (workspace_bytes < need) return SV_ERR_WORKSPACE_TOO_SMALL;

    sv::Plan pl{};
    if (!sv::fill_plan(s, desc->temperature, desc->decay, &pl)) return SV_ERR_BAD_SHAPE;
    pl.vec = (s.vocab * s.elem_bytes) % 16 == 0 && sv::aligned16(target_logits) &&
             (!s.rows_d || sv::aligned16(draft_logits));
    pl.target = target_logits;
    pl.draft = s.rows_d ? draft_logits : nullptr;
    pl.tokens = draft_tokens;
    pl.uniforms = uniforms;
    pl.mask = accept_mask;
    pl.first_reject = first_reject;
    pl.weights = weights;
    pl.probs_out = probs_out;
    pl.row_stats_out = row_stats_out;
    sv::carve_workspace(s, workspace, &pl);
    const hipError_t e = sv::launch_path(pl, stream, desc->probe_start, desc->probe_stop);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_vat_loss_workspace_size(const sv_vat_loss_desc* desc, size_t* bytes) {
    if (!desc || !bytes) return SV_ERR_NULL_ARG;
    sv::Shape s;
    const sv_status st = sv::check_shape(desc->blocks, desc->num_draft, desc->vocab, desc->dtype, SV_DRAFT_LOGITS,
                                         desc->temperature, true, &s);
    if (st != SV_OK) return st;
    if (s.greedy) return SV_ERR_BAD_TEMPERATURE;
    if (!(desc->decay >= 0.f && desc->decay <= 1.f)) return SV_ERR_BAD_DECAY;
    if (!(desc->hard_weight >= 0.f && std::isfinite(desc->hard_weight))) return SV_ERR_BAD_HARD_WEIGHT;
    s.loss = true;
    *bytes = sv::workspace_bytes_for(s);
    return SV_OK;
}

sv_status sv_vat_loss(const sv_vat_loss_desc* desc, const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms, const int32_t* hard_tokens,
                      uint8_t* accept_mask, int32_t* first_reject, float* weights, float* soft_ce, float* hard_ce,
                      float* block_loss, float* probs_out, float* row_stats_out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::Shape s;
    sv_status st = sv::check_shape(desc->blocks, desc->num_draft, desc->vocab, desc->dtype, SV_DRAFT_LOGITS,
                                   desc->temperature, true, &s);
    if (st != SV_OK) return st;
    if (s.greedy) return SV_ERR_BAD_TEMPERATURE;
    if (!(desc->decay >= 0.f && desc->decay <= 1.f)) return SV_ERR_BAD_DECAY;
    if (!(desc->hard_weight >= 0.f && std::isfinite(desc->hard_weight))) return SV_ERR_BAD_HARD_WEIGHT;
    s.loss = true;
    if (s.batch == 0) return SV_OK;
    if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !hard_tokens || !accept_mask ||
        !first_reject || !weights || !soft_ce || !hard_ce || !block_loss)
        return SV_ERR_NULL_ARG;
    const size_t need = sv::workspace_bytes_for(s);
    if (!workspace) return SV_ERR_NULL_ARG;
    if (workspace_bytes < need) return SV_ERR_WORKSPACE_TOO_SMALL;

    sv::Plan pl{};
    if (!sv::fill_plan(s, desc->temperature, desc->decay, &pl)) return SV_ERR_BAD_SHAPE;
    pl.vec = (s.vocab * s.elem_bytes) % 16 == 0 && sv::aligned16(target_logits) && sv::aligned16(draft_logits);
    pl.target = target_logits;
    pl.draft = draft_logits;
    pl.tokens = draft_tokens;
    pl.uniforms = uniforms;
    pl.mask = accept_mask;
    pl.first_reject = first_reject;
    pl.weights = weights;
    pl.probs_out = probs_out;
    pl.row_stats_out = row_stats_out;
    pl.hard_tokens = hard_tokens;
    pl.hard_weight = desc->hard_weight;
    pl.soft_ce = soft_ce;
    pl.hard_ce = hard_ce;
    pl.block_loss = block_loss;
    sv::carve_workspace(s, workspace, &pl);
    const hipError_t e = sv::launch_path(pl, stream, desc->probe_start, desc->probe_stop);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_accept_histogram(const int32_t* accepted_len, int32_t batch, int32_t k, int32_t* hist,
                              hipStream_t stream) {
    if (batch < 0 || k < 1 || k > SV_MAX_DRAFT) return SV_ERR_BAD_SHAPE;
    if (!hist || (batch > 0 && !accepted_len)) return SV_ERR_NULL_ARG;
    const hipError_t e = sv::launch_accept_hist(accepted_len, batch, k, hist, stream);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_vat_loss_grad(const sv_vat_loss_desc* desc, const void* target_logits, const void* draft_logits,
                           const int32_t* hard_tokens, const float* weights, const float* row_stats, float* grad,
                           hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::Shape s;
    const sv_status st = sv::check_shape(desc->blocks, desc->num_draft, desc->vocab, desc->dtype, SV_DRAFT_LOGITS,
                                         desc->temperature, true, &s);
    if (st != SV_OK) return st;
    if (s.greedy) return SV_ERR_BAD_TEMPERATURE;
    if (!(desc->hard_weight >= 0.f && std::isfinite(desc->hard_weight))) return SV_ERR_BAD_HARD_WEIGHT;
    if (s.batch == 0) return SV_OK;
    if (!target_logits || !draft_logits || !hard_tokens || !weights || !row_stats || !grad) return SV_ERR_NULL_ARG;
    sv::GradPlan g{};
    g.target = target_logits;
    g.draft = draft_logits;
    g.hard = hard_tokens;
    g.weights = weights;
    g.row_stats = row_stats;
    g.grad = grad;
    g.rows = s.batch * s.k;
    g.vocab = static_cast<int32_t>(s.vocab);
    g.chunks = static_cast<int32_t>(s.chunks);
    g.items = g.rows * s.chunks;
    g.elem_bytes = s.elem_bytes;
    g.vec = (s.vocab * s.elem_bytes) % 16 == 0 && s.vocab % 4 == 0 && sv::aligned16(target_logits) &&
            sv::aligned16(draft_logits) && sv::aligned16(grad);
    g.c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(desc->temperature));
    g.inv_t = static_cast<float>(1.0 / static_cast<double>(desc->temperature));
    g.hard_weight = desc->hard_weight;
    const hipError_t e = sv::launch_vat_grad(g, stream, desc->probe_start, desc->probe_stop);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_lm_head_workspace_size(const sv_lm_head_desc* desc, size_t* bytes) {
    if (!desc || !bytes) return SV_ERR_NULL_ARG;
    sv::LmShape s;
    const sv_status st = sv::check_lm_shape(desc->batch, desc->num_draft, desc->vocab, desc->hidden, &s);
    if (st != SV_OK) return st;
    *bytes = sv::lm_greedy_workspace_bytes(s);
    return SV_OK;
}

sv_status sv_verify_lm_head_greedy(const sv_lm_head_desc* desc, const void* hidden_states, const void* weight,
                                   const int32_t* draft_tokens, int32_t* accepted_len, int32_t* out_tokens,
                                   int32_t* argmax_out, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::LmShape s;
    const sv_status st = sv::check_lm_shape(desc->batch, desc->num_draft, desc->vocab, desc->hidden, &s);
    if (st != SV_OK) return st;
    if (s.batch == 0) return SV_OK;
    if (!hidden_states || !weight || !draft_tokens || !accepted_len || !out_tokens || !workspace)
        return SV_ERR_NULL_ARG;
    if (!sv::aligned16(hidden_states) || !sv::aligned16(weight)) return SV_ERR_MISALIGNED;
    if (workspace_bytes < sv::lm_greedy_workspace_bytes(s)) return SV_ERR_WORKSPACE_TOO_SMALL;
    sv::LmPlan pl{};
    sv::lm_common(s, &pl);
    pl.g[0] = sv::lm_gemm(hidden_states, weight, s.rows_t, 0, sv::kLmNoTokens);
    pl.n_gemms = 1;
    pl.mode = sv::kLmArgmax;
    sv::lmhead_layout(&pl);
    pl.tokens = draft_tokens;
    pl.accepted_len = accepted_len;
    pl.out_tokens = out_tokens;
    pl.argmax_out = argmax_out;
    char* base = static_cast<char*>(workspace);
    const size_t n = static_cast<size_t>(s.rows_t * s.n_tiles);
    pl.part_v = reinterpret_cast<float*>(base);
    pl.part_i = reinterpret_cast<int32_t*>(base + sv::align_up(n * sizeof(float)));
    const hipError_t e = sv::launch_lmhead_greedy(pl, stream, desc->probe_start, desc->probe_stop);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_lm_head_sample_workspace_size(const sv_lm_head_sample_desc* desc, size_t* bytes) {
    if (!desc || !bytes) return SV_ERR_NULL_ARG;
    sv::LmShape s;
    const sv_status st = sv::check_lm_shape(desc->batch, desc->num_draft, desc->vocab, desc->hidden, &s);
    if (st != SV_OK) return st;
    if (!(desc->temperature > 0.f) || !sv::temperature_ok(desc->temperature)) return SV_ERR_BAD_TEMPERATURE;
    *bytes = sv::lm_sample_layout(s).total;
    return SV_OK;
}

sv_status sv_verify_lm_head(const sv_lm_head_sample_desc* desc, const void* target_hidden, const void* target_weight,
                            const void* draft_hidden, const void* draft_weight, const int32_t* draft_tokens,
                            const float* uniforms, int32_t* accepted_len, int32_t* out_tokens, float* probs_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::LmShape s;
    const sv_status st = sv::check_lm_shape(desc->batch, desc->num_draft, desc->vocab, desc->hidden, &s);
    if (st != SV_OK) return st;
    if (!(desc->temperature > 0.f) || !sv::temperature_ok(desc->temperature)) return SV_ERR_BAD_TEMPERATURE;
    if (s.batch == 0) return SV_OK;
    if (!target_hidden || !target_weight || !draft_hidden || !draft_weight || !draft_tokens || !uniforms ||
        !accepted_len || !out_tokens || !workspace)
        return SV_ERR_NULL_ARG;
    if (!sv::aligned16(target_hidden) || !sv::aligned16(target_weight) || !sv::aligned16(draft_hidden) ||
        !sv::aligned16(draft_weight))
        return SV_ERR_MISALIGNED;
    const sv::LmSampleLayout L = sv::lm_sample_layout(s);
    if (workspace_bytes < L.total) return SV_ERR_WORKSPACE_TOO_SMALL;
    char* base = static_cast<char*>(workspace);
    sv::LmPlan stats{};
    sv::lm_common(s, &stats);
    stats.tokens = draft_tokens;
    stats.uniforms = uniforms;
    stats.accepted_len = accepted_len;
    stats.out_tokens = out_tokens;
    stats.probs_out = probs_out;
    stats.part_v = reinterpret_cast<float*>(base + L.part_m);
    stats.part_s = reinterpret_cast<float*>(base + L.part_s);
    stats.lx = reinterpret_cast<float*>(base + L.lx);
    stats.seq = reinterpret_cast<sv::LmSeqDraw*>(base + L.seq);
    stats.logits = reinterpret_cast<float*>(base + L.logits);
    stats.c2 = static_cast<float>(1.4426950408889634 / static_cast<double>(desc->temperature));
    stats.g[0] = sv::lm_gemm(target_hidden, target_weight, s.rows_t, 0, sv::kLmTargetTokens);
    stats.g[1] = sv::lm_gemm(draft_hidden, draft_weight, s.rows_d, s.rows_t, sv::kLmDraftTokens);
    stats.n_gemms = 2;
    stats.mode = sv::kLmStats;
    sv::lmhead_layout(&stats);
    const hipError_t e = sv::launch_lmhead_sample(stats, stream, desc->probe_start, desc->probe_stop);
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
