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

// Tag of this call's hand-off words (see kTagFirst).  The counter is 64-bit
// and tags run through 1 .. 2^32 - 1 in turn, so consecutive calls never
// share a tag (a 32-bit counter would repeat tag 1 across its wrap).
uint32_t next_tag() {
    static std::atomic<uint64_t> calls{0};
    return kTagFirst + static_cast<uint32_t>(calls.fetch_add(1u, std::memory_order_relaxed) % kTagCount);
}

// Tagged calls bake their tag into the kernel arguments, so a captured graph
// would replay it; they refuse a stream that is being captured.
sv_status capture_check(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e == hipErrorStreamCaptureImplicit) return SV_ERR_CAPTURING;
    if (e != hipSuccess) return SV_ERR_HIP;
    return cs == hipStreamCaptureStatusNone ? SV_OK : SV_ERR_CAPTURING;
}

struct Shape {
    int64_t batch, k, vocab;
    int elem_bytes;
    int64_t target_rows_per_seq;
    int64_t rows_t, rows_d;
    int64_t chunk, chunks;
    bool greedy, onehot, vat;
    bool loss;  // VAT with the training loss
    int path() const {
        if (loss) return kPathVatLoss;
        if (vat) return greedy ? kPathVatGreedy : kPathVat;
        if (greedy) return kPathGreedy;
        return onehot ? kPathOneHot : kPathSample;
    }
};

// Blocks of k_verify the current device holds at once: its compute units
// times the kernel's occupancy per unit (queried once per device).
int64_t resident_blocks(const Shape& s, bool vec) {
    constexpr int kMaxDevices = 64;
    constexpr int kPaths = kPathVatLoss + 1;
    static std::atomic<int64_t> cache[kMaxDevices][2][2][kPaths];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
    const int e = s.elem_bytes == 2 ? 1 : 0, v = vec ? 1 : 0, m = s.path();
    if (dev >= 0) {
        const int64_t c = cache[dev][e][v][m].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = kDefaultComputeUnits;
    const int per_cu = verify_blocks_per_cu(s.elem_bytes, vec, m);
    const int64_t r = static_cast<int64_t>(cus) * (per_cu > 0 ? per_cu : kMinBlocksPerCu);
    if (dev >= 0) cache[dev][e][v][m].store(r, std::memory_order_relaxed);
    return r;
}

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

// Chunks per wavefront of the decision and bonus workers.
int chunks_per_wave(const Shape& s, int64_t resident) {
    const int64_t dec_rows = s.loss ? s.k : s.k * (s.rows_d ? 2 : 1);
    return s.batch * dec_rows * s.chunks <= kSmallCallWaves * resident ? kChunksPerWaveSmall : kChunksPerWave;
}

// Segments per row: one per decision worker block of four wavefronts.
int64_t segments(const Shape& s, int nc) { return ceil_div(s.chunks, kWavesPerBlock * nc); }

int64_t rows_per_seq(const Shape& s) {
    const int64_t dec_rows = s.loss ? s.k : s.k * (s.rows_d ? 2 : 1);
    return dec_rows + (s.vat ? 0 : 1);
}

// Tagged words: two per row chunk (five per chunk pair for the VAT loss),
// two per row segment, one residual mass per chunk.  The workspace is sized
// for the larger segment count (one chunk per wavefront), so that it does
// not depend on the device.
WorkspaceLayout layout_for(const Shape& s) {
    const int64_t chunk_words = s.loss ? s.batch * s.k * s.chunks * kPairWords : s.batch * rows_per_seq(s) * s.chunks * 2;
    const int64_t seg_words = s.loss ? 0 : s.batch * rows_per_seq(s) * segments(s, kChunksPerWaveSmall) * 2;
    return workspace_layout(chunk_words, seg_words, s.batch, s.chunks);
}

size_t workspace_bytes_for(const Shape& s) { return layout_for(s).total; }

bool fill_plan(const Shape& s, float temperature, float decay, bool vec, Plan* pl) {
    const int64_t resident = resident_blocks(s, vec);
    pl->batch = static_cast<int32_t>(s.batch);
    pl->k = static_cast<int32_t>(s.k);
    pl->vocab = static_cast<int32_t>(s.vocab);
    pl->elem_bytes = s.elem_bytes;
    pl->target_rows_per_seq = static_cast<int32_t>(s.target_rows_per_seq);
    pl->chunks = static_cast<int32_t>(s.chunks);
    pl->chunk = static_cast<int32_t>(s.chunk);
    pl->path = s.path();
    // The VAT loss streams k chunk-pair "rows" (target row i with draft row i).
    pl->halves = (!s.loss && s.rows_d) ? 2 : 1;
    pl->dec_rows = static_cast<int32_t>(s.loss ? s.k : s.k * pl->halves);
    const bool has_bonus = !s.vat;
    const bool has_resid = !s.vat && !s.greedy && !s.onehot;
    pl->rows_per_seq = static_cast<int32_t>(rows_per_seq(s));
    const int nc = chunks_per_wave(s, resident);
    pl->nc_dec = nc;
    pl->nc_res = kChunksPerWaveResid;
    pl->seg_chunks = kWavesPerBlock * nc;
    pl->segs = static_cast<int32_t>(s.loss ? 1 : segments(s, nc));
    pl->words_per_seq = static_cast<int32_t>(s.loss ? s.k * s.chunks * kPairWords : pl->rows_per_seq * s.chunks * 2);
    pl->seg_words_per_seq = static_cast<int32_t>(s.loss ? 0 : pl->rows_per_seq * pl->segs * 2);
    // A decision worker block covers one segment of one row (VAT loss: 4 nc
    // chunk pairs); a bonus worker one segment of the bonus row.
    const int64_t per_block = kWavesPerBlock * nc;
    const int64_t dec_items = s.loss ? s.k * s.chunks : static_cast<int64_t>(pl->dec_rows) * pl->segs * per_block;
    if (!plan_task_grid(pl->batch, dec_items, s.chunks, has_resid, has_bonus, per_block, per_block,
                        kWavesPerBlock * pl->nc_res, resident, &pl->grid, !s.loss))
        return false;
    // Every decision worker block before every finisher: position-major.
    pl->pos_major = !s.loss && pl->grid.lag_a >= pl->batch;
    // Small one-hot and greedy calls whose statistics are not asked for: the
    // rows after a sequence's first rejection are never used (window mode).
    // The decision finishers come first and the rows position-major, so a
    // decision is often known before the blocks of later rows start: those
    // then read nothing.  When the previous call on this workspace rejected
    // the first draft token of every sequence (acceptance carries over from
    // one decoding step to the next), only the rows of the first kRowWindow
    // positions are read at once, and any other row only once the decision
    // finisher's accepted prefix comes near it.
    pl->window = (s.onehot || s.greedy) && !s.vat && !pl->probs_out && !pl->row_stats_out && pl->pos_major &&
                         pl->grid.fin_first && s.k > kRowWindow
                     ? kRowWindow
                     : 0;
    // Short polling sleeps only when (nearly) the whole grid is resident at
    // once: no stream is left for the extra reads to slow down.  A quarter
    // of a residency over is allowed for the finisher and bonus blocks that
    // follow a one-residency stream.
    pl->two_deep_polls = pl->grid.total_blocks <= resident + resident / 4;
    // The decisions of the sequences in the last residency of phase A come
    // after the bonus phase has started; their bonus rows are read without
    // deciding first, so that reading them is not added to the end of the
    // chain.
    pl->eager_bonus_from = std::max(0, pl->batch - pl->grid.lag_a);
    pl->rows_t = s.rows_t;
    pl->rows_d = s.rows_d;
    pl->greedy = s.greedy;
    pl->temperature = temperature;
    pl->c2 = s.greedy ? 0.f : static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
    pl->decay = decay;
    return true;
}

void carve_workspace(const Shape& s, void* ws, Plan* pl) {
    const WorkspaceLayout L = layout_for(s);
    char* base = static_cast<char*>(ws);
    pl->chunkw = reinterpret_cast<uint64_t*>(base + L.chunkw);
    pl->segw = reinterpret_cast<uint64_t*>(base + L.segw);
    pl->resid = reinterpret_cast<uint64_t*>(base + L.resid);
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

WorkspaceLayout workspace_layout(int64_t chunk_words, int64_t seg_words, int64_t batch, int64_t chunks) {
    WorkspaceLayout L;
    size_t off = 0;
    L.chunkw = off;
    off = align_up(off + static_cast<size_t>(chunk_words) * sizeof(uint64_t));
    L.segw = off;
    off = align_up(off + static_cast<size_t>(seg_words) * sizeof(uint64_t));
    L.resid = off;
    off = align_up(off + static_cast<size_t>(batch * (chunks + 3)) * sizeof(uint64_t));
    L.total = off;
    return L;
}

}  // namespace sv

namespace sv {
namespace {

// A valid descriptor always needs at least this many workspace bytes, so a
// size query can report an invalid one as 0.
constexpr size_t kMinWorkspace = 256;

size_t query_bytes(size_t need) { return std::max(need, kMinWorkspace); }

hipEvent_t probe_start(const sv_probe* p) { return p && p->start && p->stop ? p->start : nullptr; }
hipEvent_t probe_stop(const sv_probe* p) { return p && p->start && p->stop ? p->stop : nullptr; }

sv_status verify_shape(const sv_verify_desc* desc, Shape* s) {
    if (!desc) return SV_ERR_NULL_ARG;
    return check_shape(desc->B, desc->k, desc->V, desc->dtype, desc->draft_kind, desc->temperature, false, s);
}

sv_status vat_shape(const sv_vat_desc* desc, Shape* s) {
    if (!desc) return SV_ERR_NULL_ARG;
    const sv_status st = check_shape(desc->N, desc->k, desc->V, desc->dtype, SV_DRAFT_LOGITS, desc->temperature,
                                     true, s);
    if (st != SV_OK) return st;
    if (!(desc->decay >= 0.f && desc->decay <= 1.f)) return SV_ERR_BAD_DECAY;
    return SV_OK;
}

sv_status vat_loss_shape(const sv_vat_loss_desc* desc, Shape* s) {
    if (!desc) return SV_ERR_NULL_ARG;
    const sv_status st = check_shape(desc->N, desc->k, desc->V, desc->dtype, SV_DRAFT_LOGITS, desc->temperature,
                                     true, s);
    if (st != SV_OK) return st;
    if (s->greedy) return SV_ERR_BAD_TEMPERATURE;
    if (!(desc->decay >= 0.f && desc->decay <= 1.f)) return SV_ERR_BAD_DECAY;
    if (!(desc->hard_weight >= 0.f && std::isfinite(desc->hard_weight))) return SV_ERR_BAD_HARD_WEIGHT;
    s->loss = true;
    return SV_OK;
}

// Workspace check, plan, tag and launch shared by the tagged entry points.
sv_status launch_tagged(const Shape& s, float temperature, float decay, void* workspace, size_t workspace_bytes,
                        const sv_probe* probe, hipStream_t stream, Plan* pl) {
    if (!workspace) return SV_ERR_NULL_ARG;
    if (workspace_bytes < workspace_bytes_for(s)) return SV_ERR_WORKSPACE_TOO_SMALL;
    const sv_status cs = capture_check(stream);
    if (cs != SV_OK) return cs;
    const bool vec = (s.vocab * s.elem_bytes) % 16 == 0 && aligned16(pl->target) &&
                     (!pl->draft || aligned16(pl->draft));
    if (!fill_plan(s, temperature, decay, vec, pl)) return SV_ERR_BAD_SHAPE;
    pl->vec = vec;
    carve_workspace(s, workspace, pl);
    const hipError_t e = launch_path(*pl, stream, probe_start(probe), probe_stop(probe));
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status verify_impl(const sv_verify_desc* desc, const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len, int32_t* out_tokens,
                      float* probs_out, float* row_stats_out, const sv_probe* probe, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    Shape s;
    const sv_status st = verify_shape(desc, &s);
    if (st != SV_OK) return st;
    if (s.batch == 0) return SV_OK;
    if (!target_logits || !draft_tokens || !accepted_len || !out_tokens) return SV_ERR_NULL_ARG;
    if (!s.greedy && !uniforms) return SV_ERR_NULL_ARG;
    if (s.rows_d && !draft_logits) return SV_ERR_NULL_ARG;
    Plan pl{};
    pl.target = target_logits;
    pl.draft = s.rows_d ? draft_logits : nullptr;
    pl.tokens = draft_tokens;
    pl.uniforms = uniforms;
    pl.accepted_len = accepted_len;
    pl.out_tokens = out_tokens;
    pl.probs_out = probs_out;
    pl.row_stats_out = row_stats_out;
    return launch_tagged(s, desc->temperature, 0.f, workspace, workspace_bytes, probe, stream, &pl);
}

sv_status vat_impl(const sv_vat_desc* desc, const void* target_logits, const void* draft_logits,
                   const int32_t* draft_tokens, const float* uniforms, uint8_t* accept_mask, int32_t* first_reject,
                   float* weights, float* probs_out, float* row_stats_out, const sv_probe* probe, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
    Shape s;
    const sv_status st = vat_shape(desc, &s);
    if (st != SV_OK) return st;
    if (s.batch == 0) return SV_OK;
    if (!target_logits || !draft_tokens || !accept_mask || !first_reject || !weights) return SV_ERR_NULL_ARG;
    if (!s.greedy && (!uniforms || !draft_logits)) return SV_ERR_NULL_ARG;
    Plan pl{};
    pl.target = target_logits;
    pl.draft = s.rows_d ? draft_logits : nullptr;
    pl.tokens = draft_tokens;
    pl.uniforms = uniforms;
    pl.mask = accept_mask;
    pl.first_reject = first_reject;
    pl.weights = weights;
    pl.probs_out = probs_out;
    pl.row_stats_out = row_stats_out;
    return launch_tagged(s, desc->temperature, desc->decay, workspace, workspace_bytes, probe, stream, &pl);
}

}  // namespace
}  // namespace sv

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char* sv_status_str(sv_status status) {
    switch (status) {
        case SV_OK: return "SV_OK";
        case SV_ERR_NULL_ARG: return "SV_ERR_NULL_ARG: a required pointer is NULL";
        case SV_ERR_BAD_SHAPE: return "SV_ERR_BAD_SHAPE: batch < 0, k outside [1,64], vocab outside [1,2^24] or size overflow";
        case SV_ERR_BAD_DTYPE: return "SV_ERR_BAD_DTYPE: dtype must be SV_F32 or SV_BF16";
        case SV_ERR_BAD_TEMPERATURE: return "SV_ERR_BAD_TEMPERATURE: temperature must be 0 or finite and >= 1e-4";
        case SV_ERR_WORKSPACE_TOO_SMALL: return "SV_ERR_WORKSPACE_TOO_SMALL: workspace_bytes below the size query";
        case SV_ERR_HIP: return "SV_ERR_HIP: a HIP launch, event record or stream query failed";
        case SV_ERR_BAD_DRAFT_KIND: return "SV_ERR_BAD_DRAFT_KIND: draft_kind must be SV_DRAFT_LOGITS or SV_DRAFT_ONEHOT";
        case SV_ERR_BAD_DECAY: return "SV_ERR_BAD_DECAY: decay must be in [0, 1]";
        case SV_ERR_BAD_HARD_WEIGHT: return "SV_ERR_BAD_HARD_WEIGHT: hard_weight must be finite and >= 0";
        case SV_ERR_BAD_CONTROL: return "SV_ERR_BAD_CONTROL: need 0 <= down_frac < up_frac <= 1";
        case SV_ERR_MISALIGNED: return "SV_ERR_MISALIGNED: hidden_states and weight must be 16-byte aligned";
        case SV_ERR_CAPTURING: return "SV_ERR_CAPTURING: tagged calls cannot be captured into a HIP graph";
        case SV_ERR_SCRATCH_TOO_SMALL:
            return "SV_ERR_SCRATCH_TOO_SMALL: the call needs more than the built-in workspace (SV_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

size_t sv_verify_workspace_bytes(const sv_verify_desc* desc) {
    sv::Shape s;
    if (sv::verify_shape(desc, &s) != SV_OK) return 0;
    return sv::query_bytes(sv::workspace_bytes_for(s));
}

sv_status sv_verify(const sv_verify_desc* desc, const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len, int32_t* out_tokens,
                    float* probs_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return sv::verify_impl(desc, target_logits, draft_logits, draft_tokens, uniforms, accepted_len, out_tokens,
                           probs_out, nullptr, nullptr, workspace, workspace_bytes, stream);
}

sv_status sv_verify_ex(const sv_verify_desc* desc, const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len,
                       int32_t* out_tokens, float* probs_out, float* row_stats_out, const sv_probe* probe,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return sv::verify_impl(desc, target_logits, draft_logits, draft_tokens, uniforms, accepted_len, out_tokens,
                           probs_out, row_stats_out, probe, workspace, workspace_bytes, stream);
}

sv_status sv_verify_noalloc(const sv_verify_desc* desc, const void* target_logits, const void* draft_logits,
                            const int32_t* draft_tokens, const float* uniforms, int32_t* accepted_len,
                            int32_t* out_tokens, float* probs_out, hipStream_t stream) {
    static_assert(sv::kNoAllocScratchBytes == SV_NOALLOC_SCRATCH_BYTES, "scratch size");
    sv::Shape s;
    const sv_status st = sv::verify_shape(desc, &s);
    if (st != SV_OK) return st;
    if (s.batch == 0) return SV_OK;
    if (sv::workspace_bytes_for(s) > sv::kNoAllocScratchBytes) return SV_ERR_SCRATCH_TOO_SMALL;
    if (!target_logits || !draft_tokens || !accepted_len || !out_tokens) return SV_ERR_NULL_ARG;
    if (!s.greedy && !uniforms) return SV_ERR_NULL_ARG;
    if (s.rows_d && !draft_logits) return SV_ERR_NULL_ARG;
    const sv_status cs = sv::capture_check(stream);
    if (cs != SV_OK) return cs;
    void* scratch = nullptr;
    if (sv::noalloc_scratch(stream, &scratch) != hipSuccess) return SV_ERR_HIP;
    return sv::verify_impl(desc, target_logits, draft_logits, draft_tokens, uniforms, accepted_len, out_tokens,
                           probs_out, nullptr, nullptr, scratch, sv::kNoAllocScratchBytes, stream);
}

size_t sv_vat_workspace_bytes(const sv_vat_desc* desc) {
    sv::Shape s;
    if (sv::vat_shape(desc, &s) != SV_OK) return 0;
    return sv::query_bytes(sv::workspace_bytes_for(s));
}

sv_status sv_vat_labels(const sv_vat_desc* desc, const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, const float* uniforms, uint8_t* accept_mask,
                        int32_t* first_reject, float* weights, float* probs_out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
    return sv::vat_impl(desc, target_logits, draft_logits, draft_tokens, uniforms, accept_mask, first_reject,
                        weights, probs_out, nullptr, nullptr, workspace, workspace_bytes, stream);
}

sv_status sv_vat_labels_ex(const sv_vat_desc* desc, const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, const float* uniforms, uint8_t* accept_mask,
                           int32_t* first_reject, float* weights, float* probs_out, float* row_stats_out,
                           const sv_probe* probe, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    return sv::vat_impl(desc, target_logits, draft_logits, draft_tokens, uniforms, accept_mask, first_reject,
                        weights, probs_out, row_stats_out, probe, workspace, workspace_bytes, stream);
}

size_t sv_vat_loss_workspace_bytes(const sv_vat_loss_desc* desc) {
    sv::Shape s;
    if (sv::vat_loss_shape(desc, &s) != SV_OK) return 0;
    return sv::query_bytes(sv::workspace_bytes_for(s));
}

sv_status sv_vat_loss(const sv_vat_loss_desc* desc, const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, const float* uniforms, const int32_t* hard_tokens,
                      uint8_t* accept_mask, int32_t* first_reject, float* weights, float* soft_ce, float* hard_ce,
                      float* block_loss, float* probs_out, float* row_stats_out, const sv_probe* probe,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    sv::Shape s;
    const sv_status st = sv::vat_loss_shape(desc, &s);
    if (st != SV_OK) return st;
    if (s.batch == 0) return SV_OK;
    if (!target_logits || !draft_logits || !draft_tokens || !uniforms || !hard_tokens || !accept_mask ||
        !first_reject || !weights || !soft_ce || !hard_ce || !block_loss)
        return SV_ERR_NULL_ARG;
    sv::Plan pl{};
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
    return sv::launch_tagged(s, desc->temperature, desc->decay, workspace, workspace_bytes, probe, stream, &pl);
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
                           const sv_probe* probe, hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::Shape s;
    const sv_status st = sv::check_shape(desc->N, desc->k, desc->V, desc->dtype, SV_DRAFT_LOGITS,
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
    const hipError_t e = sv::launch_vat_grad(g, stream, sv::probe_start(probe), sv::probe_stop(probe));
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

size_t sv_lm_head_workspace_bytes(const sv_lm_head_desc* desc) {
    if (!desc) return 0;
    sv::LmShape s;
    if (sv::check_lm_shape(desc->B, desc->k, desc->V, desc->D, &s) != SV_OK) return 0;
    return sv::query_bytes(sv::lm_greedy_workspace_bytes(s));
}

sv_status sv_verify_lm_head_greedy(const sv_lm_head_desc* desc, const void* hidden_states, const void* weight,
                                   const int32_t* draft_tokens, int32_t* accepted_len, int32_t* out_tokens,
                                   int32_t* argmax_out, const sv_probe* probe, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::LmShape s;
    const sv_status st = sv::check_lm_shape(desc->B, desc->k, desc->V, desc->D, &s);
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
    const hipError_t e = sv::launch_lmhead_greedy(pl, stream, sv::probe_start(probe), sv::probe_stop(probe));
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

size_t sv_lm_head_sample_workspace_bytes(const sv_lm_head_sample_desc* desc) {
    if (!desc) return 0;
    sv::LmShape s;
    if (sv::check_lm_shape(desc->B, desc->k, desc->V, desc->D, &s) != SV_OK) return 0;
    if (!(desc->temperature > 0.f) || !sv::temperature_ok(desc->temperature)) return 0;
    return sv::query_bytes(sv::lm_sample_layout(s).total);
}

sv_status sv_verify_lm_head(const sv_lm_head_sample_desc* desc, const void* target_hidden, const void* target_weight,
                            const void* draft_hidden, const void* draft_weight, const int32_t* draft_tokens,
                            const float* uniforms, int32_t* accepted_len, int32_t* out_tokens, float* probs_out,
                            const sv_probe* probe, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!desc) return SV_ERR_NULL_ARG;
    sv::LmShape s;
    const sv_status st = sv::check_lm_shape(desc->B, desc->k, desc->V, desc->D, &s);
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
    const hipError_t e = sv::launch_lmhead_sample(stats, stream, sv::probe_start(probe), sv::probe_stop(probe));
    return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}

sv_status sv_sol_read(const void* data, size_t bytes, uint32_t* sink, hipStream_t stream) {
    if (bytes == 0) return SV_OK;
    if (!data || !sink) return SV_ERR_NULL_ARG;
    if (!sv::aligned16(data) || bytes % 16 != 0) return SV_ERR_MISALIGNED;
    if (bytes / 16 > (size_t{1} << 40)) return SV_ERR_BAD_SHAPE;
    const hipError_t e = sv::launch_sol_read(data, static_cast<int64_t>(bytes / 16), sink, stream);
    return e == hipSuccess ? SV_OK : (e == hipErrorInvalidValue ? SV_ERR_BAD_SHAPE : SV_ERR_HIP);
}

sv_status sv_sol_read_write(const void* a, const void* b, float* out, int64_t n, sv_dtype dtype,
                            hipStream_t stream) {
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_BAD_DTYPE;
    if (n < 0 || n > (int64_t{1} << 42)) return SV_ERR_BAD_SHAPE;
    if (n == 0) return SV_OK;
    if (!a || !b || !out) return SV_ERR_NULL_ARG;
    const int per_vec = dtype == SV_F32 ? 4 : 8;
    if (!sv::aligned16(a) || !sv::aligned16(b) || !sv::aligned16(out) || n % per_vec != 0) return SV_ERR_MISALIGNED;
    const hipError_t e = sv::launch_sol_read_write(a, b, out, n / per_vec, dtype == SV_F32 ? 4 : 2, stream);
    return e == hipSuccess ? SV_OK : (e == hipErrorInvalidValue ? SV_ERR_BAD_SHAPE : SV_ERR_HIP);
}

}  // extern "C"
