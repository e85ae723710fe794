// Host-side probe of the kernel's task grid, for tests/test_task_grid.py:
// builds a grid with the library's own planner and decodes every block with
// the same function the kernel uses.  Compiled with the host compiler only.
#include <stdint.h>

#include "sv_grid.h"

extern "C" int32_t probe_plan(int32_t batch, int64_t dec_items, int64_t chunks, int32_t has_resid, int32_t has_bonus,
                              int64_t per_block_dec, int64_t per_block_bonus, int64_t per_block_res, int64_t resident,
                              int32_t allow_fin_first, int32_t* params) {
    sv::TaskGrid tg;
    if (!sv::plan_task_grid(batch, dec_items, chunks, has_resid != 0, has_bonus != 0, per_block_dec, per_block_bonus,
                            per_block_res, resident, &tg, allow_fin_first != 0))
        return -1;
    params[0] = tg.w_dec;
    params[1] = tg.w_res;
    params[2] = tg.w_bonus;
    params[3] = tg.lag_a;
    params[4] = tg.lag_r;
    params[5] = tg.lag_f;
    params[6] = tg.lag_b;
    params[7] = tg.n_segments;
    params[8] = tg.fin_first;
    return tg.total_blocks;
}

extern "C" int32_t probe_decode(int32_t batch, int32_t w_dec, int32_t w_res, int32_t w_bonus, int32_t has_resid,
                                int32_t has_bonus, int32_t lag_a, int32_t lag_r, int32_t lag_f, int32_t lag_b,
                                int32_t fin_first, int32_t* kind, int32_t* seq, int32_t* index, int32_t cap) {
    sv::TaskGrid tg;
    if (!sv::build_task_grid(batch, w_dec, w_res, w_bonus, has_resid != 0, has_bonus != 0, lag_a, lag_r, lag_f,
                             lag_b, &tg, fin_first != 0))
        return -1;
    if (tg.total_blocks > cap) return -2;
    for (int32_t b = 0; b < tg.total_blocks; ++b) {
        const sv::Role r = sv::decode_role(tg, b);
        kind[b] = r.kind;
        seq[b] = r.seq;
        index[b] = r.index;
    }
    return tg.total_blocks;
}
