// Host construction of the task grid (see sv_grid.h).  Plain C++.
#include "sv_grid.h"

#include <algorithm>
#include <vector>

namespace sv {
namespace {

struct PhaseRoles {
    bool a;  // phase A (decision, residual) or phase B (bonus)
    bool df;  // phase A holds the decision finishers (not placed first)
    int32_t batch, w_dec, w_res, w_bonus;
    bool has_resid;
    int32_t lag_a, lag_r, lag_f, lag_b;

    bool in(int64_t s) const { return s >= 0 && s < batch; }

    int32_t roles(int64_t g) const {
        int32_t r = 0;
        if (a) {
            if (in(g)) r |= kBitDecWorker;
            if (df && in(g - lag_a)) r |= kBitDecFinisher;
            if (has_resid && in(g - lag_a - lag_r)) r |= kBitResWorker;
            if (has_resid && in(g - lag_a - lag_r - lag_f)) r |= kBitResFinisher;
        } else {
            if (in(g)) r |= kBitBonusWorker;
            if (in(g - lag_b)) r |= kBitBonusFinisher;
        }
        return r;
    }

    int64_t blocks(int32_t r) const {
        int64_t n = 0;
        if (r & kBitDecWorker) n += w_dec;
        if (r & kBitDecFinisher) n += 1;
        if (r & kBitResWorker) n += w_res;
        if (r & kBitResFinisher) n += 1;
        if (r & kBitBonusWorker) n += w_bonus;
        if (r & kBitBonusFinisher) n += 1;
        return n;
    }
};

}  // namespace

bool build_task_grid(int32_t batch, int32_t w_dec, int32_t w_res, int32_t w_bonus, bool has_resid, bool has_bonus,
                     int32_t lag_a, int32_t lag_r, int32_t lag_f, int32_t lag_b, TaskGrid* tg, bool fin_first) {
    *tg = TaskGrid{};
    tg->fin_first = fin_first ? 1 : 0;
    tg->batch = batch;
    tg->w_dec = w_dec;
    tg->w_res = has_resid ? w_res : 0;
    tg->w_bonus = has_bonus ? w_bonus : 0;
    tg->lag_a = lag_a;
    tg->lag_r = has_resid ? lag_r : 0;
    tg->lag_f = has_resid ? lag_f : 0;
    tg->lag_b = has_bonus ? lag_b : 0;
    const int32_t lags[4] = {tg->lag_a, tg->lag_r, tg->lag_f, tg->lag_b};
    for (int32_t l : lags)
        if (l < 0 || l > batch) return false;
    if (batch < 1 || w_dec < 1 || (has_resid && w_res < 1) || (has_bonus && w_bonus < 1)) return false;

    int64_t next_block = 0;
    int n = 0;
    if (fin_first) {
        // one finisher per group, decoded as sequence g - lag_a = 0 .. B-1
        Segment& s = tg->seg[n++];
        s.first_block = 0;
        s.first_group = tg->lag_a;
        s.group_blocks = 1;
        s.roles = kBitDecFinisher;
        s.inv_group_blocks = 1.0f;
        next_block = batch;
    }
    for (int phase = 0; phase < 2; ++phase) {
        if (phase == 1 && !has_bonus) break;
        const PhaseRoles pr{phase == 0, !fin_first, batch, w_dec, tg->w_res, tg->w_bonus, has_resid,
                            tg->lag_a, tg->lag_r, tg->lag_f, tg->lag_b};
        const int64_t B = batch;
        std::vector<int64_t> bp;
        int64_t groups;
        if (phase == 0) {
            const int64_t la = tg->lag_a, lr = tg->lag_r, lf = tg->lag_f;
            groups = B + la + (has_resid ? lr + lf : 0);
            bp = {0, B, la, la + B};
            if (has_resid) {
                bp.insert(bp.end(), {la + lr, la + lr + B, la + lr + lf, la + lr + lf + B});
            }
        } else {
            groups = B + tg->lag_b;
            bp = {0, B, tg->lag_b, tg->lag_b + B};
        }
        bp.push_back(groups);
        std::sort(bp.begin(), bp.end());
        bp.erase(std::unique(bp.begin(), bp.end()), bp.end());
        int64_t prev_end = -1;  // end group of this phase's last segment
        for (size_t i = 0; i + 1 < bp.size(); ++i) {
            const int64_t g0 = bp[i], g1 = bp[i + 1];
            if (g0 < 0 || g0 >= groups || g1 <= g0) continue;
            const int32_t r = pr.roles(g0);
            const int64_t per = pr.blocks(r);
            if (per == 0) continue;
            // extend the previous segment when it continues with the same roles
            if (prev_end == g0 && tg->seg[n - 1].roles == r) {
                next_block += per * (g1 - g0);
                prev_end = g1;
                if (next_block > 0x7fffffffLL) return false;
                continue;
            }
            prev_end = g1;
            if (n == kMaxSegments) return false;
            Segment& s = tg->seg[n++];
            s.first_block = static_cast<int32_t>(next_block);
            s.first_group = static_cast<int32_t>(g0);
            s.group_blocks = static_cast<int32_t>(per);
            s.roles = r;
            s.inv_group_blocks = 1.0f / static_cast<float>(per);
            next_block += per * (g1 - g0);
            if (next_block > 0x7fffffffLL) return false;
        }
    }
    tg->n_segments = n;
    tg->total_blocks = static_cast<int32_t>(next_block);
    return n > 0;
}

bool plan_task_grid(int32_t batch, int64_t dec_items, int64_t chunks, bool has_resid, bool has_bonus,
                    int64_t per_block_dec, int64_t per_block_bonus, int64_t per_block_res, int64_t resident_blocks,
                    TaskGrid* tg, bool allow_fin_first) {
    const auto ceil_div = [](int64_t a, int64_t b) { return (a + b - 1) / b; };
    if (batch < 1 || dec_items < 1 || chunks < 1 || per_block_dec < 1 || per_block_bonus < 1 || per_block_res < 1)
        return false;
    const int64_t w_dec = ceil_div(dec_items, per_block_dec);
    const int64_t w_res = has_resid ? ceil_div(chunks, per_block_res) : 0;
    const int64_t w_bonus = has_bonus ? ceil_div(chunks, per_block_bonus) : 0;
    if (w_dec > 0x7fffffffLL || w_res > 0x7fffffffLL || w_bonus > 0x7fffffffLL) return false;
    // A finisher goes about one residency of blocks after its workers; the
    // residual workers go with the decision finisher (each decides for
    // itself), the residual finisher half a residency after them.
    const int64_t group_a = w_dec + 1 + (has_resid ? w_res + 1 : 0);
    const auto lag = [&](int64_t blocks, int64_t group) {
        return static_cast<int32_t>(std::min<int64_t>(batch, ceil_div(blocks, group)));
    };
    const int32_t lag_a = lag(resident_blocks, group_a);
    const int32_t lag_r = 0;
    const int32_t lag_f = has_resid ? lag(resident_blocks / 2, group_a) : 0;
    const int32_t lag_b = has_bonus ? lag(resident_blocks, w_bonus + 1) : 0;
    const bool fin_first = allow_fin_first && lag_a >= batch && static_cast<int64_t>(batch) * 8 <= resident_blocks;
    return build_task_grid(batch, static_cast<int32_t>(w_dec), static_cast<int32_t>(w_res),
                           static_cast<int32_t>(w_bonus), has_resid, has_bonus, lag_a, lag_r, lag_f, lag_b, tg,
                           fin_first);
}

}  // namespace sv
