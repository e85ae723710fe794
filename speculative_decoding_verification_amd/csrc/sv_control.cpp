// Host-side draft-length controller (see sv_draft_len_update in
// specverify.h).  Plain C++: no device code, no allocation.
#include <cmath>

#include "specverify.h"

extern "C" {

sv_status sv_draft_len_init(sv_draft_len_ctl* ctl, const int32_t* choices, int32_t n_choices, float up_frac,
                            float down_frac, int32_t patience) {
    if (!ctl || !choices) return SV_ERR_NULL_ARG;
    if (n_choices < 1 || n_choices > SV_MAX_DRAFT_CHOICES || patience < 1) return SV_ERR_BAD_SHAPE;
    for (int32_t i = 0; i < n_choices; ++i) {
        if (choices[i] < 1 || choices[i] > SV_MAX_DRAFT) return SV_ERR_BAD_SHAPE;
        if (i > 0 && choices[i] <= choices[i - 1]) return SV_ERR_BAD_SHAPE;
    }
    if (!(std::isfinite(up_frac) && std::isfinite(down_frac) && down_frac >= 0.f && down_frac < up_frac &&
          up_frac <= 1.f))
        return SV_ERR_BAD_CONTROL;
    *ctl = sv_draft_len_ctl{};
    ctl->n_choices = n_choices;
    for (int32_t i = 0; i < n_choices; ++i) ctl->choices[i] = choices[i];
    ctl->index = 0;
    ctl->up_frac = up_frac;
    ctl->down_frac = down_frac;
    ctl->patience = patience;
    ctl->last_efficiency = 0.f;
    return SV_OK;
}

sv_status sv_draft_len_update(sv_draft_len_ctl* ctl, const int32_t* hist, int32_t k, int32_t* next_k) {
    if (!ctl || !hist || !next_k) return SV_ERR_NULL_ARG;
    if (ctl->n_choices < 1 || ctl->index < 0 || ctl->index >= ctl->n_choices || k != ctl->choices[ctl->index])
        return SV_ERR_BAD_SHAPE;
    // Block efficiency: tokens committed per verify cycle (the accepted
    // drafts plus the target's own token), over the valid sequences.
    double n = 0.0, tokens = 0.0;
    for (int32_t j = 0; j <= k; ++j) {
        n += hist[j];
        tokens += static_cast<double>(j + 1) * hist[j];
    }
    if (n > 0.0) {
        const double eff = tokens / n;
        ctl->last_efficiency = static_cast<float>(eff);
        const double top = static_cast<double>(k + 1);
        if (eff >= ctl->up_frac * top) {
            ctl->up_streak += 1;
            ctl->down_streak = 0;
        } else if (eff <= ctl->down_frac * top) {
            ctl->down_streak += 1;
            ctl->up_streak = 0;
        } else {
            ctl->up_streak = 0;
            ctl->down_streak = 0;
        }
        if (ctl->up_streak >= ctl->patience && ctl->index + 1 < ctl->n_choices) {
            ctl->index += 1;
            ctl->up_streak = ctl->down_streak = 0;
        } else if (ctl->down_streak >= ctl->patience && ctl->index > 0) {
            ctl->index -= 1;
            ctl->up_streak = ctl->down_streak = 0;
        }
    }
    *next_k = ctl->choices[ctl->index];
    return SV_OK;
}

}  // extern "C"
