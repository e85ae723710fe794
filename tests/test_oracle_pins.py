"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: a worked
example printed on a page, a closed form, an exact identity checked by
enumeration, a Monte-Carlo law with a stated tolerance, or a library routine
that computes the same quantity in a special case.  A plausible slip in the
oracle (a dropped term, a flipped comparison, a wrong index or an off-by-one
anchor) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import special, stats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_simplex(rng, V, zeros=0):
    p = rng.random(V) + 0.05
    if zeros:
        p[rng.choice(V, zeros, replace=False)] = 0.0
    return p / p.sum()


def _logits_from_probs(p):
    with np.errstate(divide="ignore"):
        return np.log(p).astype(np.float64)


# ----------------------------------------------------------------- bf16 decode

def test_bf16_decode_matches_torch_for_every_bit_pattern(orc):
    torch = pytest.importorskip("torch")
    bits = np.arange(65536, dtype=np.uint16)
    ours = orc.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


# ----------------------------------------------------------------- worked example

def test_worked_example_acceptance_probabilities(orc):
    g = _load_golden("worked_example_acceptance.json")
    for case in g["cases"]:
        a = orc.accept_prob(case["p_target"], case["q_draft"])
        assert abs(a - case["accept_prob"]) <= case["printed_tolerance"] + 1e-15, case


def test_worked_example_through_full_verify_v2(orc):
    """V=2: the draft proposes token 0 with q=0.9.  Target p(0)=0.95 keeps it for
    every u; target p(0)=0.1 keeps it for u < 1/9 and otherwise resamples the
    target's preferred token 1."""
    g = _load_golden("worked_example_acceptance.json")
    us = (np.arange(9000, dtype=np.float32) + 0.5) / 9000  # evenly spread uniforms in (0,1)
    for case in g["cases"]:
        p0, q0 = case["p_target"], case["q_draft"]
        pt = np.array([p0, 1 - p0])
        qd = np.array([q0, 1 - q0])
        B = us.size
        # k=1: target has rows for position 0 and the bonus position 1
        target = np.tile(np.stack([_logits_from_probs(pt), _logits_from_probs(pt)])[None], (B, 1, 1))
        draft = np.tile(_logits_from_probs(qd)[None, None], (B, 1, 1))
        tokens = np.zeros((B, 1), np.int32)
        u = np.stack([us, np.full(B, 0.5, np.float32)], axis=1).astype(np.float32)
        r = orc.verify(target.astype(np.float32), draft.astype(np.float32), tokens, u, 1.0)
        frac = r.accepted_len.mean()
        assert abs(frac - case["accept_prob"]) <= case["printed_tolerance"] + 2e-4, (case, frac)
        rejected = r.accepted_len == 0
        if rejected.any():
            # the residual max(0, p - q) is one-hot on token 1: every resample is 1
            assert np.all(r.out_tokens[rejected, 0] == 1)
            assert np.all(r.out_tokens[rejected, 1] == -1)
        acc = ~rejected
        assert np.all(r.out_tokens[acc, 0] == 0)


# ----------------------------------------------------------------- closed forms

def test_acceptance_rate_equals_one_minus_total_variation(orc):
    """x ~ q, kept w.p. min(1,p/q): E[kept] = sum_x min(p(x), q(x)) = 1 - TV(p,q)."""
    rng = np.random.default_rng(7)
    for trial in range(4):
        V = 6
        p = _rand_simplex(rng, V, zeros=trial % 2)
        q = _rand_simplex(rng, V, zeros=(trial // 2) % 2)
        B = 200_000
        x = rng.choice(V, size=B, p=q).astype(np.int32)[:, None]
        u = rng.random((B, 2), dtype=np.float32)
        lt = np.tile(np.stack([_logits_from_probs(p)] * 2)[None], (B, 1, 1)).astype(np.float32)
        ld = np.tile(_logits_from_probs(q)[None, None], (B, 1, 1)).astype(np.float32)
        r = orc.verify(lt, ld, x, u, 1.0)
        frac = r.accepted_len.mean()
        expect = np.minimum(p, q).sum()
        assert abs(expect - (1 - 0.5 * np.abs(p - q).sum())) < 1e-12
        sigma = math.sqrt(expect * (1 - expect) / B)
        assert abs(frac - expect) < 5 * sigma + 1e-6, (trial, frac, expect)


def test_residual_mass_is_total_variation(orc):
    rng = np.random.default_rng(3)
    for _ in range(50):
        V = int(rng.integers(2, 40))
        p, q = _rand_simplex(rng, V, zeros=1), _rand_simplex(rng, V)
        w = orc.residual(p, q)
        assert np.all(w >= 0)
        assert abs(w.sum() - 0.5 * np.abs(p - q).sum()) < 1e-12
        assert abs(w.sum() - (1 - np.minimum(p, q).sum())) < 1e-12


def test_losslessness_by_exact_enumeration(orc):
    """P(out = y) = q(y) a(y) + (1 - sum_x q(x) a(x)) w(y)/sum(w) equals p(y),
    a = accept_prob, w = residual: the output token is distributed as the target."""
    rng = np.random.default_rng(11)
    for V in range(2, 7):
        for _ in range(40):
            p = _rand_simplex(rng, V, zeros=int(rng.integers(0, V - 1)))
            q = _rand_simplex(rng, V, zeros=int(rng.integers(0, V - 1)))
            a = np.array([orc.accept_prob(p[y], q[y]) for y in range(V)])
            kept = q * a
            reject_mass = 1.0 - kept.sum()
            w = orc.residual(p, q)
            out = kept + (reject_mass * w / w.sum() if w.sum() > 0 else 0.0)
            assert np.allclose(out, p, atol=1e-12, rtol=0), (p, q, out)


def test_losslessness_chi_square_full_sampler(orc):
    """Monte Carlo through the whole batched path at V=8, k=3: among trials that
    reach position j, out[j] ~ p_j; P(accepted_len >= j) = prod_{i<j} alpha_i."""
    rng = np.random.default_rng(2024)
    V, k, B = 8, 3, 200_000
    P = np.stack([_rand_simplex(rng, V, zeros=1) for _ in range(k + 1)])
    Q = np.stack([_rand_simplex(rng, V, zeros=1 if i == 1 else 0) for i in range(k)])
    lt = np.tile(_logits_from_probs(P)[None], (B, 1, 1)).astype(np.float32)
    ld = np.tile(_logits_from_probs(Q)[None], (B, 1, 1)).astype(np.float32)
    # the fp32 logits round the probabilities; use the exactly decoded ones
    P = np.stack([orc.softmax(lt[0, i].astype(np.float64), 1.0)[0] for i in range(k + 1)])
    Q = np.stack([orc.softmax(ld[0, i].astype(np.float64), 1.0)[0] for i in range(k)])
    x = np.stack([rng.choice(V, size=B, p=Q[i]) for i in range(k)], axis=1).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    r = orc.verify(lt, ld, x, u, 1.0)
    L = r.accepted_len
    alpha = np.minimum(P[:k], Q).sum(axis=1)
    pvals = []
    for j in range(k + 1):
        reach = L >= j
        n = int(reach.sum())
        expect_reach = float(np.prod(alpha[:j]))
        sigma = math.sqrt(expect_reach * (1 - expect_reach) / B) if 0 < expect_reach < 1 else 0
        assert abs(n / B - expect_reach) < 5 * sigma + 1e-9, (j, n / B, expect_reach)
        counts = np.bincount(r.out_tokens[reach, j], minlength=V)
        support = P[j] > 0
        assert counts[~support].sum() == 0  # zero-probability tokens never emitted
        pvals.append(stats.chisquare(counts[support], n * P[j][support] / P[j][support].sum()).pvalue)
    assert min(pvals) > 1e-4 / len(pvals), pvals


# ----------------------------------------------------------------- special cases

def test_identical_draft_and_target_always_accepts(orc):
    rng = np.random.default_rng(5)
    B, k, V = 512, 5, 50
    lt = (3 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    ld = lt[:, :k].copy()
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    r = orc.verify(lt, ld, x, u, 0.7)
    assert np.all(r.accepted_len == k)
    assert np.array_equal(r.out_tokens[:, :k], x)


def test_onehot_draft_acceptance_is_target_prob(orc):
    """q = indicator of x: kept iff u < p(x); residual is p with x removed."""
    rng = np.random.default_rng(9)
    B, k, V = 4000, 1, 5
    lt = (2 * rng.standard_normal((1, k + 1, V))).astype(np.float32)
    lt = np.tile(lt, (B, 1, 1))
    x = np.full((B, 1), 2, np.int32)
    u = rng.random((B, 2), dtype=np.float32)
    r = orc.verify(lt, None, x, u, 1.0, onehot=True)
    p0 = orc.softmax(lt[0, 0].astype(np.float64), 1.0)[0]
    assert np.array_equal(r.accepted_len == 1, u[:, 0].astype(np.float64) < p0[2])
    assert np.allclose(r.probs[:, 0, 0], p0[2], rtol=1e-15)
    assert np.all(r.probs[:, 0, 1] == 1.0)
    rej = r.accepted_len == 0
    # resampled token never equals the rejected draft token, and follows the
    # library inverse CDF of p with x zeroed
    w = p0.copy()
    w[2] = 0.0
    cdf = np.cumsum(w)
    expect = np.searchsorted(cdf, u[rej, 1].astype(np.float64) * cdf[-1], side="right")
    assert np.array_equal(r.out_tokens[rej, 0], expect)
    assert not np.any(r.out_tokens[rej, 0] == 2)


def test_greedy_matches_numpy_argmax_with_ties(orc):
    rng = np.random.default_rng(13)
    B, k, V = 300, 4, 64
    # coarse values make ties common; numpy.argmax returns the first maximum
    lt = rng.integers(-4, 5, (B, k + 1, V)).astype(np.float32)
    g = np.argmax(lt, axis=2)
    x = np.where(rng.random((B, k)) < 0.7, g[:, :k], rng.integers(0, V, (B, k))).astype(np.int32)
    r = orc.verify(lt, None, x, None, 0.0)
    for b in range(B):
        mism = np.nonzero(x[b] != g[b, :k])[0]
        rr = int(mism[0]) if mism.size else k
        assert r.accepted_len[b] == rr
        assert list(r.out_tokens[b, :rr]) == list(x[b, :rr])
        assert r.out_tokens[b, rr] == g[b, rr]
        assert np.all(r.out_tokens[b, rr + 1:] == -1)
        assert np.array_equal(r.target_mz[b, :, 1], g[b])


def test_greedy_matches_numpy_argmax_bf16(orc):
    import workloads

    rng = np.random.default_rng(17)
    B, k, V = 50, 3, 3001
    bits = workloads.round_to_bf16_bits((4 * rng.standard_normal((B, k + 1, V))).astype(np.float32))
    vals = workloads.bf16_bits_to_f32(bits)
    g = np.argmax(vals, axis=2)
    x = g[:, :k].astype(np.int32).copy()
    x[::3, 1] = (x[::3, 1] + 1) % V
    r = orc.verify(bits, None, x, None, 0.0)
    assert np.array_equal(r.target_mz[:, :, 1].astype(np.int64), g)


def test_inverse_cdf_matches_searchsorted(orc):
    rng = np.random.default_rng(21)
    for _ in range(300):
        V = int(rng.integers(1, 200))
        w = rng.random(V) * (rng.random(V) < 0.7)
        if w.sum() == 0:
            w[int(rng.integers(0, V))] = 1.0
        u = float(rng.random(dtype=np.float32))
        y, margin = orc.inverse_cdf(w, u)
        cdf = np.cumsum(w)
        assert y == int(np.searchsorted(cdf, u * cdf[-1], side="right"))
        assert w[y] > 0
        assert margin >= 0


def test_inverse_cdf_never_picks_zero_weight_even_at_u_near_one(orc):
    w = np.array([0.0, 0.3, 0.0, 0.7, 0.0, 0.0])
    for u in [0.0, 0.2999, 0.3, 0.5, 0.9999999]:
        y, _ = orc.inverse_cdf(w, u)
        assert w[y] > 0


def test_softmax_matches_scipy(orc):
    rng = np.random.default_rng(23)
    for T in [1.0, 0.6, 0.01, 3.0]:
        l = 4 * rng.standard_normal(1000)
        l[::97] = -np.inf
        p, m, z = orc.softmax(l, T)
        assert np.allclose(p, special.softmax(l / T), rtol=1e-13, atol=0)
        assert abs(m + math.log(z) - special.logsumexp(l / T)) < 1e-12 * max(1.0, abs(m))
        assert m == np.max(l) / T
        assert np.all(p[::97] == 0)


def test_neg_inf_logits_are_never_emitted(orc):
    rng = np.random.default_rng(29)
    B, k, V = 2000, 2, 12
    lt = rng.standard_normal((B, k + 1, V)).astype(np.float32)
    ld = rng.standard_normal((B, k, V)).astype(np.float32)
    lt[:, :, 5:9] = -np.inf
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    r = orc.verify(lt, ld, x, u, 1.0)
    for b in range(B):
        L = r.accepted_len[b]
        assert not (5 <= r.out_tokens[b, L] < 9)


def test_invalid_token_flags_sequence(orc):
    rng = np.random.default_rng(31)
    B, k, V = 3, 3, 10
    lt = rng.standard_normal((B, k + 1, V)).astype(np.float32)
    ld = rng.standard_normal((B, k, V)).astype(np.float32)
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    x[1, 2] = V
    x[2, 0] = -1
    u = rng.random((B, k + 1), dtype=np.float32)
    r = orc.verify(lt, ld, x, u, 1.0)
    assert r.accepted_len[0] >= 0
    assert list(r.accepted_len[1:]) == [-1, -1]
    assert np.all(r.out_tokens[1:] == -1)


def test_temperature_scales_logits(orc):
    """softmax(l/T) at T is the T=1 softmax of l/T: the same verify result."""
    rng = np.random.default_rng(37)
    B, k, V, T = 64, 4, 300, 0.6
    lt = (4 * rng.standard_normal((B, k + 1, V))).astype(np.float64)
    ld = lt[:, :k] + 0.3 * rng.standard_normal((B, k, V))
    # choose T and logits so that l/T is exactly representable
    T = 0.5
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    a = orc.verify(lt.astype(np.float32), ld.astype(np.float32), x, u, T)
    b = orc.verify((lt / T).astype(np.float32), (ld / T).astype(np.float32), x, u, 1.0)
    np.testing.assert_array_equal(a.accepted_len, b.accepted_len)
    np.testing.assert_array_equal(a.out_tokens, b.out_tokens)


# ----------------------------------------------------------------- VAT

def _vat_inputs_with_reject_at(rs, k, V=4):
    """Blocks whose proposed token has p/q = 0.5 at every position; u = 0 keeps
    it, u = 0.9 rejects it.  Block n is built to reject first at rs[n]."""
    N = len(rs)
    p = np.array([0.2, 0.3, 0.25, 0.25])
    q = np.array([0.4, 0.2, 0.2, 0.2])
    lt = np.tile(_logits_from_probs(p)[None, None], (N, k, 1)).astype(np.float32)
    ld = np.tile(_logits_from_probs(q)[None, None], (N, k, 1)).astype(np.float32)
    x = np.zeros((N, k), np.int32)
    u = np.zeros((N, k), np.float32)
    for n, r in enumerate(rs):
        if r < k:
            u[n, r] = 0.9
            u[n, r + 1:] = np.linspace(0, 0.99, k - r - 1)
    return lt, ld, x, u


def test_vat_weighting_prose_examples(orc):
    g = _load_golden("vat_weighting_examples.json")
    decay = g["decay"]
    for case in g["cases"]:
        k, r = case["k"], case["first_reject"]
        lt, ld, x, u = _vat_inputs_with_reject_at([r], k)
        res = orc.vat_labels(lt, ld, x, u, 1.0, decay)
        assert res.first_reject[0] == r
        assert int(res.accept_mask[0].sum()) == case["accept_mask_ones"]
        assert np.all(res.accept_mask[0, :r] == 1) and np.all(res.accept_mask[0, r:] == 0)
        full = case["full_weight_positions"]
        assert np.all(res.weights[0, full] == 1.0)
        anchor = case["decay_anchor"]
        for i in range(anchor, k):
            assert res.weights[0, i] == pytest.approx(decay ** (i - anchor), rel=1e-15)
        if r == 0:
            # the fixed curve decaying from the first position: 0.8^(j-1), j 1-based
            j = np.arange(1, k + 1)
            assert np.allclose(res.weights[0], decay ** (j - 1), rtol=1e-15)


def test_vat_hard_cut_is_zero_decay(orc):
    k = 8
    lt, ld, x, u = _vat_inputs_with_reject_at([3], k)
    res = orc.vat_labels(lt, ld, x, u, 1.0, 0.0)
    assert list(res.weights[0]) == [1, 1, 1, 1, 0, 0, 0, 0]


def test_vat_labels_follow_inference_rule(orc):
    """The simulated verification is the inference-time rule: first_reject equals
    the accepted length of batched verification on the same rows and uniforms."""
    rng = np.random.default_rng(41)
    N, k, V = 400, 6, 40
    lt = (2 * rng.standard_normal((N, k + 1, V))).astype(np.float32)
    ld = (lt[:, :k] + 0.8 * rng.standard_normal((N, k, V))).astype(np.float32)
    x = rng.integers(0, V, (N, k)).astype(np.int32)
    u = rng.random((N, k + 1), dtype=np.float32)
    v = orc.verify(lt, ld, x, u, 0.8)
    t = orc.vat_labels(np.ascontiguousarray(lt[:, :k]), ld, x, np.ascontiguousarray(u[:, :k]), 0.8, 0.8)
    np.testing.assert_array_equal(v.accepted_len, t.first_reject)
    np.testing.assert_array_equal(t.accept_mask.sum(axis=1), t.first_reject)
    g = orc.verify(lt, None, x, None, 0.0)
    tg = orc.vat_labels(np.ascontiguousarray(lt[:, :k]), None, x, None, 0.0, 0.8)
    np.testing.assert_array_equal(g.accepted_len, tg.first_reject)


# ----------------------------------------------------------------- VAT loss

def _pq_block(rng, N, k, V, s_t=2.0, s_d=0.7):
    lt = (s_t * rng.standard_normal((N, k, V))).astype(np.float32)
    ld = (lt + s_d * rng.standard_normal((N, k, V))).astype(np.float32)
    x = rng.integers(0, V, (N, k)).astype(np.int32)
    h = rng.integers(0, V, (N, k)).astype(np.int32)
    u = rng.random((N, k), dtype=np.float32)
    return lt, ld, x, u, h


def test_vat_soft_term_with_identical_draft_is_the_target_entropy(orc):
    """q = p: the soft term is the Shannon entropy of p (scipy's entropy, in nats)."""
    rng = np.random.default_rng(50)
    lt, _, x, u, h = _pq_block(rng, 3, 5, 64)
    for T in (1.0, 0.7):
        res = orc.vat_loss(lt, lt, x, u, h, T, 0.8)
        for n in range(3):
            for i in range(5):
                p = special.softmax(lt[n, i].astype(np.float64) / T)
                assert res.soft[n, i] == pytest.approx(stats.entropy(p), rel=1e-12)


def test_vat_soft_term_is_entropy_plus_kl(orc):
    """Gibbs: -sum p ln q = H(p) + KL(p||q) >= H(p), KL from scipy's rel_entr."""
    rng = np.random.default_rng(51)
    lt, ld, x, u, h = _pq_block(rng, 4, 6, 97)
    T = 1.3
    res = orc.vat_loss(lt, ld, x, u, h, T, 0.8)
    for n in range(4):
        for i in range(6):
            p = special.softmax(lt[n, i].astype(np.float64) / T)
            q = special.softmax(ld[n, i].astype(np.float64) / T)
            kl = special.rel_entr(p, q).sum()
            assert kl > 0
            assert res.soft[n, i] == pytest.approx(stats.entropy(p) + kl, rel=1e-11)


def test_vat_uniform_draft_gives_log_v(orc):
    """A flat draft distribution costs ln V on both terms, whatever p is."""
    rng = np.random.default_rng(52)
    V = 1000
    lt, _, x, u, h = _pq_block(rng, 2, 3, V)
    ld = np.full_like(lt, 3.5)
    res = orc.vat_loss(lt, ld, x, u, h, 1.0, 0.8)
    assert np.allclose(res.soft, math.log(V), rtol=1e-13)
    assert np.allclose(res.hard, math.log(V), rtol=1e-13)


def test_vat_hard_term_is_log_softmax(orc):
    rng = np.random.default_rng(53)
    lt, ld, x, u, h = _pq_block(rng, 3, 4, 300)
    T = 0.6
    res = orc.vat_loss(lt, ld, x, u, h, T, 0.8)
    for n in range(3):
        for i in range(4):
            ls = special.log_softmax(ld[n, i].astype(np.float64) / T)
            assert res.hard[n, i] == pytest.approx(-ls[h[n, i]], rel=1e-12)


def test_vat_block_loss_weights_follow_first_rejection(orc):
    """Blocks built to reject first at r: the block loss is the first-rejection
    weighted sum of the two terms (weights 1 before r, decay^(i-r) from r)."""
    k, decay, lam = 7, 0.8, 0.5
    rs = [0, 3, k]
    lt, ld, x, u = _vat_inputs_with_reject_at(rs, k)
    h = np.tile(np.arange(k, dtype=np.int32) % 4, (len(rs), 1))
    res = orc.vat_loss(lt, ld, x, u, h, 1.0, decay, lam)
    # the distributions of the stored (fp32) logits
    p = special.softmax(lt[0, 0].astype(np.float64))
    q = special.softmax(ld[0, 0].astype(np.float64))
    soft = stats.entropy(p) + special.rel_entr(p, q).sum()
    for n, r in enumerate(rs):
        assert res.first_reject[n] == r
        i = np.arange(k)
        w = np.where(i < r, 1.0, decay ** np.maximum(i - r, 0))
        want = sum(w[j] * (soft + lam * -math.log(q[h[n, j]])) for j in range(k))
        assert res.block_loss[n] == pytest.approx(want, rel=1e-12)
        assert np.allclose(res.soft[n], soft, rtol=1e-12)


def test_vat_loss_temperature_scales_logits(orc):
    """Logits times T at temperature T give the T = 1 losses."""
    rng = np.random.default_rng(54)
    lt, ld, x, u, h = _pq_block(rng, 2, 4, 120)
    a = orc.vat_loss(lt.astype(np.float64).astype(np.float32), ld, x, u, h, 1.0, 0.8)
    T = 2.0  # a power of two keeps the scaled fp32 logits exact
    b = orc.vat_loss(lt * np.float32(T), ld * np.float32(T), x, u, h, T, 0.8)
    assert np.allclose(a.soft, b.soft, rtol=1e-13)
    assert np.allclose(a.hard, b.hard, rtol=1e-13)
    assert np.array_equal(a.first_reject, b.first_reject)


def test_vat_loss_labels_match_vat_labels_and_invalid_hard_token_flags(orc):
    rng = np.random.default_rng(55)
    lt, ld, x, u, h = _pq_block(rng, 5, 6, 50)
    h[2, 4] = 50
    res = orc.vat_loss(lt, ld, x, u, h, 1.0, 0.8)
    lab = orc.vat_labels(lt, ld, x, u, 1.0, 0.8)
    keep = np.arange(5) != 2
    assert np.array_equal(res.first_reject[keep], lab.first_reject[keep])
    assert np.array_equal(res.weights[keep], lab.weights[keep])
    assert res.first_reject[2] == -1 and np.all(res.weights[2] == 0)
    assert np.isnan(res.block_loss[2]) and np.all(np.isnan(res.soft[2]))
    assert np.all(np.isfinite(res.block_loss[keep]))


def test_vat_loss_grad_matches_central_differences_of_the_block_loss(orc):
    """The gradient against the block loss itself: a central difference of
    orc.vat_loss on fp64 logits, one draft logit at a time, with the
    acceptance outcome unchanged by the step (the weights are labels).  A
    dropped term, a wrong sign, a missing 1/T or the hard term on the wrong
    token fails this."""
    rng = np.random.default_rng(56)
    N, k, V, eps = 3, 4, 7, 1e-6
    lt, ld, x, u, h = _pq_block(rng, N, k, V)
    lt = lt.astype(np.float64)
    ld = ld.astype(np.float64)
    for T, lam, decay in ((1.0, 1.0, 0.8), (0.7, 0.5, 0.6), (1.6, 0.0, 0.8)):
        base = orc.vat_loss(lt, ld, x, u, h, T, decay, lam)
        g = orc.vat_loss_grad(lt, ld, h, base.weights, T, lam)
        checked = 0
        for n in range(N):
            for i in range(k):
                for y in range(V):
                    lp, lm = ld.copy(), ld.copy()
                    lp[n, i, y] += eps
                    lm[n, i, y] -= eps
                    a = orc.vat_loss(lt, lp, x, u, h, T, decay, lam)
                    b = orc.vat_loss(lt, lm, x, u, h, T, decay, lam)
                    if a.first_reject[n] != base.first_reject[n] or b.first_reject[n] != base.first_reject[n]:
                        continue
                    fd = (a.block_loss[n] - b.block_loss[n]) / (2 * eps)
                    assert g[n, i, y] == pytest.approx(fd, abs=2e-8), (T, lam, n, i, y)
                    checked += 1
        assert checked > 0.9 * N * k * V


def test_vat_loss_grad_rows_sum_to_zero_and_vanish_with_zero_weight(orc):
    """Softmax gradients sum to zero over the vocabulary ((1 + lam) - 1 - lam);
    positions of weight 0 (decay 0 after the first rejection, or a flagged
    block) have all-zero rows."""
    rng = np.random.default_rng(57)
    lt, ld, x, u, h = _pq_block(rng, 6, 5, 300)
    res = orc.vat_loss(lt, ld, x, u, h, 0.9, 0.0, 0.7)
    g = orc.vat_loss_grad(lt, ld, h, res.weights, 0.9, 0.7)
    assert np.allclose(g.sum(axis=2), 0.0, atol=1e-13)
    zero = res.weights == 0.0
    assert zero.any() and (~zero).any()
    assert np.all(g[zero] == 0.0)
    assert np.all(np.abs(g[~zero]).max(axis=1) > 0)


# ----------------------------------------------------------------- LM-head greedy verification

def _bf16_bits(a):
    a = np.ascontiguousarray(a, np.float32)
    u = a.view(np.uint32)
    # round to nearest even on the discarded half
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_vals(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_lm_head_logits_are_the_fp64_matmul(orc):
    rng = np.random.default_rng(70)
    B, k, V, D = 3, 4, 300, 96
    h = _bf16_bits(rng.standard_normal((B, k + 1, D)))
    w = _bf16_bits(rng.standard_normal((V, D)) * 0.3)
    logits = _bf16_vals(h) @ _bf16_vals(w).T            # numpy matmul in fp64
    x = np.argmax(logits[:, :k], axis=2).astype(np.int32)
    res = orc.lm_head_greedy(h, w, x)
    assert np.array_equal(res.argmax, np.argmax(logits, axis=2))
    srt = np.sort(logits, axis=2)
    assert np.allclose(res.top2_gap, srt[..., -1] - srt[..., -2], rtol=1e-9, atol=1e-12)
    assert np.all(res.accepted_len == k)
    assert np.array_equal(res.out_tokens[:, :k], x) and np.array_equal(res.out_tokens[:, k], res.argmax[:, k])


def test_lm_head_greedy_matches_logit_greedy_on_exact_integers(orc):
    """Small integer hidden states and weights make every logit an exact
    integer (ties included); the result must equal greedy verification on
    those logits, lowest index first among ties."""
    rng = np.random.default_rng(71)
    B, k, V, D = 40, 5, 64, 8
    h = _bf16_bits(rng.integers(-2, 3, (B, k + 1, D)).astype(np.float32))
    w = _bf16_bits(rng.integers(-2, 3, (V, D)).astype(np.float32))
    logits = (_bf16_vals(h) @ _bf16_vals(w).T).astype(np.float32)
    g = np.argmax(logits, axis=2)
    x = np.where(rng.random((B, k)) < 0.7, g[:, :k], rng.integers(0, V, (B, k))).astype(np.int32)
    res = orc.lm_head_greedy(h, w, x)
    ref = orc.verify(logits, None, x, None, 0.0)
    assert np.array_equal(res.accepted_len, ref.accepted_len)
    assert np.array_equal(res.out_tokens, ref.out_tokens)
    assert np.any(res.top2_gap == 0.0)   # ties occur and follow the lowest index


def test_lm_head_greedy_first_mismatch_and_invalid_token(orc):
    rng = np.random.default_rng(72)
    B, k, V, D = 2, 4, 50, 16
    h = _bf16_bits(rng.standard_normal((B, k + 1, D)))
    w = _bf16_bits(rng.standard_normal((V, D)))
    g = np.argmax(_bf16_vals(h) @ _bf16_vals(w).T, axis=2)
    x = g[:, :k].astype(np.int32).copy()
    x[0, 2] = (x[0, 2] + 1) % V
    x[1, 0] = V
    res = orc.lm_head_greedy(h, w, x)
    assert res.accepted_len[0] == 2
    assert list(res.out_tokens[0]) == [x[0, 0], x[0, 1], g[0, 2], -1, -1]
    assert res.accepted_len[1] == -1 and np.all(res.out_tokens[1] == -1)


def test_lm_head_logits_equal_the_fp64_matmul_and_integers_exactly(orc):
    rng = np.random.default_rng(73)
    h = _bf16_bits(rng.standard_normal((2, 3, 40)))
    w = _bf16_bits(rng.standard_normal((57, 40)) * 0.2)
    got = orc.lm_head_logits(h, w)
    assert got.shape == (2, 3, 57)
    assert np.allclose(got, _bf16_vals(h) @ _bf16_vals(w).T, rtol=1e-12, atol=1e-12)
    hi = _bf16_bits(rng.integers(-3, 4, (5, 16)).astype(np.float32))
    wi = _bf16_bits(rng.integers(-3, 4, (9, 16)).astype(np.float32))
    exact = _bf16_vals(hi).astype(np.int64) @ _bf16_vals(wi).astype(np.int64).T
    assert np.array_equal(orc.lm_head_logits(hi, wi), exact.astype(np.float64))


def test_f64_logits_run_the_same_rule_as_f32(orc):
    """fp64 rows holding fp32-representable values give bit-identical results
    to the same values passed as fp32."""
    rng = np.random.default_rng(74)
    B, k, V = 6, 4, 300
    t = (rng.standard_normal((B, k + 1, V)) * 3).astype(np.float32)
    d = (t[:, :k] + rng.standard_normal((B, k, V)).astype(np.float32) * 0.5).astype(np.float32)
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    a = orc.verify(t, d, x, u, 0.8)
    b = orc.verify(t.astype(np.float64), d.astype(np.float64), x, u, 0.8)
    for name in ("accepted_len", "out_tokens", "probs", "target_mz", "draft_mz"):
        assert np.array_equal(getattr(a, name), getattr(b, name), equal_nan=True), name


def test_lm_head_verify_with_the_target_as_draft_never_rejects(orc):
    """q = p makes every test u*q < p succeed (u < 1): all k drafts kept, and
    the bonus token is drawn from the target's last position."""
    rng = np.random.default_rng(75)
    B, k, V, D = 5, 3, 80, 24
    h = _bf16_bits(rng.standard_normal((B, k + 1, D)))
    w = _bf16_bits(rng.standard_normal((V, D)) * 0.4)
    x = rng.integers(0, V, (B, k)).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    res = orc.lm_head_verify(h, w, h[:, :k], w, x, u, 1.0)
    assert np.all(res.accepted_len == k)
    assert np.allclose(res.probs[..., 0], res.probs[..., 1], rtol=0, atol=0)
    lk = _bf16_vals(h[:, k]).astype(np.float64) @ _bf16_vals(w).astype(np.float64).T
    for b in range(B):
        p = np.exp(lk[b] - lk[b].max())
        c = np.cumsum(p)
        assert res.out_tokens[b, k] == int(np.searchsorted(c, u[b, k] * c[-1], side="right"))
