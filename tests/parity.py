"""Shared helpers of the GPU parity tests: upload a seeded workload, run the
HIP path through the C ABI, run the oracle on the same arrays, compare.

Comparison rules (the tolerance is the one the verification target states):
 - per-row statistics m = max l/T and Z, and p(x_i), q(x_i): within 1e-5
   relative of the fp64 oracle;
 - greedy (T == 0) row maxima and argmaxes, accepted lengths and tokens: exact;
 - T > 0 accepted lengths and tokens: exact, except where a tested position has
   |u - p/q| < 1e-5 (the fp32 and fp64 decisions may legitimately differ
   there; the sequence is compared only before that position and counted), or
   where the single draw u*Z lies within 1e-5*Z of an end of the oracle's
   chosen interval (counted; the rest of the sequence still compared).
"""
from __future__ import annotations

import numpy as np

BAND = 1e-5
RTOL = 1e-5
# VAT loss terms are log-sum-exp differences in fp32: their error is relative
# (1e-5) for typical values and absolute near zero (log2 of a sum close to 1
# resolves to about one ulp of 1.0, 1.2e-7; the floor allows a few of them).
LOSS_ATOL = 1e-6
# fp32 outputs cannot hold probabilities below the smallest normal float (the
# hardware exp2 flushes subnormal results): an absolute floor for p(x), q(x).
FLT_MIN = float(np.finfo(np.float32).tiny)


def pooled(fn, idx, workers=None):
    """fn(one-element index array) for every element of idx on a thread pool
    (the oracle's C calls run without Python's lock), the per-element
    results (oracle result objects) joined along their first axis."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    idx = np.asarray(idx)
    workers = workers or max(1, min(16, os.cpu_count() or 1, len(idx)))
    with ThreadPoolExecutor(workers) as ex:
        parts = list(ex.map(lambda i: fn(idx[i:i + 1]), range(len(idx))))
    if isinstance(parts[0], np.ndarray):
        return np.concatenate(parts, axis=0)
    cls = type(parts[0])

    def join(name):
        vals = [getattr(q, name, None) for q in parts]
        return None if vals[0] is None else np.concatenate(vals, axis=0)

    return cls(**{name: join(name) for name in cls.__slots__})


def to_torch(a, device):
    import torch

    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def run_verify_gpu(wl, device, temperature=None, onehot=None):
    import speculative_decoding_verification_amd as sv

    cfg = wl.config
    T = cfg.T if temperature is None else temperature
    oh = cfg.onehot if onehot is None else onehot
    t = to_torch(wl.target, device)
    d = to_torch(wl.draft, device) if (wl.draft is not None and not oh and T != 0.0) else None
    x = to_torch(wl.tokens, device)
    u = to_torch(wl.uniforms, device)
    res = sv.verify(t, d, x, u, T, onehot=oh, return_probs=True, return_row_stats=True)
    out = {name: getattr(res, name).cpu().numpy() for name in ("accepted_len", "out_tokens", "probs", "row_stats")}
    # Without row statistics the library skips the bonus rows that no draw
    # needs; the decisions and tokens must not change.
    lean = sv.verify(t, d, x, u, T, onehot=oh)
    assert np.array_equal(lean.accepted_len.cpu().numpy(), out["accepted_len"]), "accepted_len differs without row stats"
    assert np.array_equal(lean.out_tokens.cpu().numpy(), out["out_tokens"]), "out_tokens differ without row stats"
    return out


def run_vat_gpu(wl, device, temperature=None, decay=None):
    import speculative_decoding_verification_amd as sv

    cfg = wl.config
    T = cfg.T if temperature is None else temperature
    dec = cfg.decay if decay is None else decay
    t = to_torch(wl.target, device)
    d = to_torch(wl.draft, device) if T != 0.0 else None
    x = to_torch(wl.tokens, device)
    u = to_torch(wl.uniforms, device) if T != 0.0 else None
    res = sv.vat_labels(t, d, x, u, T, dec, return_probs=True, return_row_stats=True)
    out = {name: getattr(res, name).cpu().numpy()
           for name in ("accept_mask", "first_reject", "weights", "probs", "row_stats")}
    # The same call without the optional outputs gives the same labels.
    lean = sv.vat_labels(t, d, x, u, T, dec)
    for name in ("accept_mask", "first_reject", "weights"):
        assert np.array_equal(getattr(lean, name).cpu().numpy(), out[name]), name + " differs without probs"
    return out


def _close(a, b, rtol=RTOL, atol=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    ok = both_inf | (np.abs(a - b) <= atol + rtol * np.abs(b))
    return ok


def _assert_close(name, got, want, rtol=RTOL, atol=0.0):
    ok = _close(got, want, rtol, atol)
    if not np.all(ok):
        bad = np.argwhere(~ok)[:5]
        detail = ["%s: got %r want %r" % (tuple(i), got[tuple(i)], want[tuple(i)]) for i in bad]
        raise AssertionError("%s: %d of %d outside tolerance; e.g. %s" % (name, int((~ok).sum()), ok.size,
                                                                      "; ".join(detail)))


def check_row_stats(gpu_stats, orc_t_mz, orc_d_mz, greedy, rows_d_present):
    """Rows of sequences the oracle flags for an invalid token carry NaN there
    and are not compared (the library still reports their statistics)."""
    t = orc_t_mz.reshape(-1, 2)
    nt = t.shape[0]
    g_t = gpu_stats[:nt]
    keep = ~np.isnan(t[:, 0])
    t, g_t = t[keep], g_t[keep]
    if greedy:
        assert np.array_equal(g_t[:, 0].astype(np.float64), t[:, 0]), "greedy row max differs"
        assert np.array_equal(g_t[:, 1].astype(np.int64), t[:, 1].astype(np.int64)), "greedy argmax differs"
        return
    _assert_close("target m", g_t[:, 0], t[:, 0], atol=1e-6)
    _assert_close("target Z", g_t[:, 1], t[:, 1])
    if rows_d_present:
        d = orc_d_mz.reshape(-1, 2)
        g_d = gpu_stats[nt:nt + d.shape[0]]
        keep = ~np.isnan(d[:, 0])
        d, g_d = d[keep], g_d[keep]
        _assert_close("draft m", g_d[:, 0], d[:, 0], atol=1e-6)
        _assert_close("draft Z", g_d[:, 1], d[:, 1])


def compare_verify(gpu, orc, k, V, greedy, seq_index=None, band=BAND, rtol=RTOL):
    """Asserts parity; returns counts of ambiguous positions and draws.
    `band` and `rtol` default to the logits-input tolerances; paths that form
    the logits themselves in fp32 pass wider ones."""
    acc_g, out_g = gpu["accepted_len"], gpu["out_tokens"]
    B = acc_g.shape[0]
    rows = np.arange(B) if seq_index is None else seq_index
    valid = orc.accepted_len[rows] >= 0
    # probabilities of valid sequences
    pg = gpu["probs"][valid]
    po = orc.probs[rows][valid]
    if greedy:
        assert np.array_equal(pg.astype(np.float64), po), "greedy probs differ"
    else:
        _assert_close("p(x)", pg[..., 0], po[..., 0], rtol=rtol, atol=FLT_MIN)
        _assert_close("q(x)", pg[..., 1], po[..., 1], rtol=rtol, atol=FLT_MIN)
    amb_accept = 0
    amb_sample = 0
    for j, b in enumerate(rows):
        ro = int(orc.accepted_len[b])
        rg = int(acc_g[j])
        if ro < 0:
            assert rg == -1 and np.all(out_g[j] == -1), (b, rg)
            continue
        assert 0 <= rg <= k, (b, rg)
        assert np.all(out_g[j, rg + 1:] == -1), (b, out_g[j])
        assert 0 <= out_g[j, rg] < V, (b, out_g[j])
        tested = range(min(ro + 1, k))
        amb = [i for i in tested if abs(orc.accept_margin[b, i]) < band]
        if amb and not greedy:
            i0 = amb[0]
            amb_accept += 1
            assert rg >= i0, (b, rg, i0)
            n = min(rg, ro)
            assert np.array_equal(out_g[j, :n], orc.out_tokens[b, :n]), b
            continue
        assert rg == ro, ("accepted_len", int(b), rg, ro, orc.accept_margin[b])
        assert np.array_equal(out_g[j, :ro], orc.out_tokens[b, :ro]), b
        if not greedy and orc.sample_margin[b] < band:
            amb_sample += 1
            continue
        assert out_g[j, ro] == orc.out_tokens[b, ro], ("token", int(b), int(out_g[j, ro]),
                                                      int(orc.out_tokens[b, ro]), orc.sample_margin[b])
    return {"sequences": len(rows), "ambiguous_accept": amb_accept, "ambiguous_sample": amb_sample}


def compare_vat(gpu, orc, k, decay, greedy, blk_index=None):
    """`orc` must have been run with the fp32 value of decay the C ABI receives."""
    decay = float(np.float32(decay))
    fr_g = gpu["first_reject"]
    N = fr_g.shape[0]
    rows = np.arange(N) if blk_index is None else blk_index
    valid = orc.first_reject[rows] >= 0
    pg = gpu["probs"][valid]
    po = orc.probs[rows][valid]
    if greedy:
        assert np.array_equal(pg.astype(np.float64), po)
    else:
        _assert_close("p(x)", pg[..., 0], po[..., 0], atol=FLT_MIN)
        _assert_close("q(x)", pg[..., 1], po[..., 1], atol=FLT_MIN)
    amb = 0
    i = np.arange(k)
    for j, n in enumerate(rows):
        ro = int(orc.first_reject[n])
        rg = int(fr_g[j])
        if ro < 0:
            assert rg == -1 and np.all(gpu["accept_mask"][j] == 0) and np.all(gpu["weights"][j] == 0)
            continue
        # labels and weights follow the GPU's own r exactly (closed form)
        assert np.array_equal(gpu["accept_mask"][j], (i < rg).astype(np.uint8)), n
        want_w = np.where(i < rg, 1.0, np.power(float(decay), np.maximum(i - rg, 0).astype(np.float64)))
        _assert_close("weights", gpu["weights"][j], want_w, rtol=1e-7, atol=0.0)
        tested = range(min(ro + 1, k))
        a = [p for p in tested if abs(orc.accept_margin[n, p]) < BAND]
        if a and not greedy:
            amb += 1
            assert rg >= a[0]
            continue
        assert rg == ro, ("first_reject", int(n), rg, ro)
        _assert_close("weights vs oracle", gpu["weights"][j], orc.weights[n], rtol=1e-7)
        assert np.array_equal(gpu["accept_mask"][j], orc.accept_mask[n])
    return {"blocks": len(rows), "ambiguous_accept": amb}


def run_vat_loss_gpu(wl, device, temperature=None, decay=None, hard_weight=1.0, hard=None):
    import speculative_decoding_verification_amd as sv

    cfg = wl.config
    T = cfg.T if temperature is None else temperature
    dec = cfg.decay if decay is None else decay
    h = wl.hard_tokens if hard is None else hard
    res = sv.vat_loss(to_torch(wl.target, device), to_torch(wl.draft, device), to_torch(wl.tokens, device),
                      to_torch(wl.uniforms, device), to_torch(h, device), T, dec, hard_weight,
                      return_probs=True, return_row_stats=True)
    return {name: getattr(res, name).cpu().numpy()
            for name in ("accept_mask", "first_reject", "weights", "soft_ce", "hard_ce", "block_loss", "probs",
                         "row_stats")}


def compare_vat_loss(gpu, orc_loss, orc_lab, k, decay, hard_weight, blk_index=None):
    """Labels as compare_vat; soft and hard terms within RTOL of the oracle;
    the block loss equals the weighted sum of the oracle's terms under the
    GPU's own weights (RTOL), which must be the oracle's weights wherever the
    first rejection is not ambiguous.  `orc_lab` is orc.vat_labels on the same
    inputs (for the acceptance margins)."""
    decay = float(np.float32(decay))
    hard_weight = float(np.float32(hard_weight))
    fr_g = gpu["first_reject"]
    N = fr_g.shape[0]
    rows = np.arange(N) if blk_index is None else blk_index
    valid = orc_loss.first_reject[rows] >= 0
    _assert_close("soft", gpu["soft_ce"][valid], orc_loss.soft[rows][valid], atol=LOSS_ATOL)
    _assert_close("hard", gpu["hard_ce"][valid], orc_loss.hard[rows][valid], atol=LOSS_ATOL)
    amb = 0
    i = np.arange(k)
    for j, n in enumerate(rows):
        ro = int(orc_loss.first_reject[n])
        rg = int(fr_g[j])
        if ro < 0:
            assert rg == -1 and np.all(gpu["weights"][j] == 0) and np.isnan(gpu["block_loss"][j]), n
            assert np.all(np.isnan(gpu["soft_ce"][j])) and np.all(np.isnan(gpu["hard_ce"][j])), n
            continue
        assert 0 <= rg <= k, (n, rg)
        assert np.array_equal(gpu["accept_mask"][j], (i < rg).astype(np.uint8)), n
        want_w = np.where(i < rg, 1.0, np.power(decay, np.maximum(i - rg, 0).astype(np.float64)))
        _assert_close("weights", gpu["weights"][j], want_w, rtol=1e-7)
        want_loss = float(np.sum(want_w * (orc_loss.soft[n] + hard_weight * orc_loss.hard[n])))
        _assert_close("block loss", np.array([gpu["block_loss"][j]]), np.array([want_loss]), atol=k * LOSS_ATOL)
        tested = range(min(ro + 1, k))
        a = [p for p in tested if abs(orc_lab.accept_margin[n, p]) < BAND]
        if a:
            amb += 1
            assert rg >= a[0]
            continue
        assert rg == ro, ("first_reject", int(n), rg, ro)
    return {"blocks": len(rows), "ambiguous_accept": amb}
