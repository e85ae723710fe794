"""GPU parity of LM-head-fused greedy verification (sv_verify_lm_head_greedy)
against the oracle's fp64 logits h . w_y.

Comparison rule: a position whose two largest fp64 logits differ by more than
GAP_BAND has one correct choice and the kernel must return it; a position
inside the band may return any token whose fp64 logit is within GAP_BAND of
the maximum (counted), and its sequence is compared only before it.  The
kernel sums bf16 products in fp32 (exact products, rounded sums): for the
hidden sizes here (D <= 4096, logits of size ~10) the expected rounding error
is ~1e-5, so GAP_BAND = 2e-3 leaves a margin of two orders of magnitude.
With small-integer inputs every logit is an exact integer in fp32 as well,
so ties are real and the lowest index must win exactly.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import pooled
from workloads import bf16_bits_to_f32, round_to_bf16_bits

pytestmark = pytest.mark.gpu

GAP_BAND = 2e-3


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import speculative_decoding_verification_amd as sv

    sv.load_library()
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf(a, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def _run_gpu(h, w, x, dev):
    import torch

    import speculative_decoding_verification_amd as sv

    res = sv.verify_lm_head_greedy(_bf(h, dev), _bf(w, dev), torch.from_numpy(np.ascontiguousarray(x)).to(dev),
                                   return_argmax=True)
    torch.cuda.synchronize()
    return res.accepted_len.cpu().numpy(), res.out_tokens.cpu().numpy(), res.argmax.cpu().numpy()


def _logit(h_row, w, y):
    return float(np.dot(bf16_bits_to_f32(h_row).astype(np.float64), bf16_bits_to_f32(w[y]).astype(np.float64)))


def _consistent(acc, out, am, x, V):
    """What holds at any size: decisions and tokens follow from the returned
    per-position choices."""
    B, k = x.shape
    for b in range(B):
        r = acc[b]
        if np.any((x[b] < 0) | (x[b] >= V)):
            assert r == -1 and np.all(out[b] == -1), b
            continue
        assert 0 <= r <= k, b
        assert np.array_equal(x[b, :r], am[b, :r]), b
        if r < k:
            assert x[b, r] != am[b, r], b
        assert np.array_equal(out[b, :r], x[b, :r]) and out[b, r] == am[b, r] and np.all(out[b, r + 1:] == -1), b


def _compare(h, w, x, got, orc, band=GAP_BAND, exact=False):
    acc, out, am = got
    B, k = x.shape
    V = w.shape[0]
    _consistent(acc, out, am, x, V)
    ambiguous = 0
    for b in range(B):
        cut = k + 1  # positions compared
        for i in range(k + 1):
            g_o = orc.argmax[b, i]
            if exact or orc.top2_gap[b, i] > band:
                assert am[b, i] == g_o, (b, i, am[b, i], g_o, orc.top2_gap[b, i])
            else:
                ambiguous += 1
                best = _logit(h[b, i], w, g_o)
                assert 0 <= am[b, i] < V and _logit(h[b, i], w, am[b, i]) >= best - band, (b, i)
                cut = min(cut, i)
        if cut > k:
            assert acc[b] == orc.accepted_len[b], b
            assert np.array_equal(out[b], orc.out_tokens[b]), b
        else:
            r_o = orc.accepted_len[b]
            if r_o >= 0 and r_o < cut:  # decided before the first ambiguous position
                assert acc[b] == r_o and np.array_equal(out[b], orc.out_tokens[b]), b
            elif r_o >= 0:  # the oracle accepted every position before the ambiguous one
                assert acc[b] >= cut and np.array_equal(out[b, :cut], x[b, :cut]), b
    return ambiguous


def _planted(B, k, V, D, hit=0.8, seed=11):
    cfg = workloads.LM_CONFIGS["lmhead_tiny"].scaled(B=B, k=k, V=V, D=D, hit=hit, seed=seed)
    return workloads.generate_lm_head(cfg)


@pytest.mark.parametrize("B,k,V,D", [
    (90, 5, 3000, 256),      # 3 row tiles (ragged), 12 vocabulary tiles (ragged)
    (1, 1, 1, 64),           # one token, one K slice
    (3, 64, 300, 64),        # longest draft (65 rows per sequence), V just over one tile
    (9, 16, 8193, 192),      # last vocabulary tile holds one column
    (40, 7, 2048, 4096),     # the full hidden size, two row tiles, V a multiple of the tile width
    (2, 3, 127, 64),         # V below one tile
])
def test_lm_head_reduced(dev, B, k, V, D):
    _say("case lm_head planted B=%d k=%d V=%d D=%d" % (B, k, V, D))
    wl = _planted(B, k, V, D)
    got = _run_gpu(wl.hidden, wl.weight, wl.tokens, dev)
    orc = oracle.lm_head_greedy(wl.hidden, wl.weight, wl.tokens)
    amb = _compare(wl.hidden, wl.weight, wl.tokens, got, orc)
    _say("  ambiguous positions: %d of %d; accepted mean %.2f" % (amb, B * (k + 1), float(np.mean(got[0]))))


def test_lm_head_unplanted_gaussian_logits(dev):
    """No planted margin: every argmax is the maximum of V Gaussian logits,
    gaps ~0.1; decisions still exact outside the band."""
    rng = np.random.default_rng(81)
    B, k, V, D = 24, 6, 5000, 512
    h = round_to_bf16_bits(rng.standard_normal((B, k + 1, D)).astype(np.float32))
    w = round_to_bf16_bits((rng.standard_normal((V, D)) / np.sqrt(D)).astype(np.float32))
    g = oracle.lm_head_greedy(h, w, np.zeros((B, k), np.int32)).argmax
    x = np.where(rng.random((B, k)) < 0.85, g[:, :k], rng.integers(0, V, (B, k))).astype(np.int32)
    _say("case lm_head unplanted B=%d k=%d V=%d D=%d" % (B, k, V, D))
    got = _run_gpu(h, w, x, dev)
    orc = oracle.lm_head_greedy(h, w, x)
    _compare(h, w, x, got, orc)


def test_lm_head_unplanted_full_vocabulary_and_hidden_size(dev):
    """No planted margin at the workloads' real sizes (V=151936, D=4096): every
    argmax is the maximum of 151936 Gaussian logits (top-two gaps of a few
    hundredths and below), summed over 4096 products; every row's argmax and
    every sequence's decision against the oracle."""
    rng = np.random.default_rng(83)
    B, k, V, D = 6, 5, 151936, 4096
    h = round_to_bf16_bits(rng.standard_normal((B, k + 1, D)).astype(np.float32))
    w = workloads.lm_head_weight(workloads.LM_CONFIGS["lmhead_selfdraft"])  # z / sqrt(D), [V][D] bf16
    assert w.shape == (V, D)
    every = np.arange(B)
    g = pooled(lambda i: oracle.lm_head_greedy(h[i], w, np.zeros((1, k), np.int32)), every).argmax
    x = np.where(rng.random((B, k)) < 0.85, g[:, :k], rng.integers(0, V, (B, k))).astype(np.int32)
    _say("case lm_head unplanted B=%d k=%d V=%d D=%d" % (B, k, V, D))
    got = _run_gpu(h, w, x, dev)
    orc = pooled(lambda i: oracle.lm_head_greedy(h[i], w, x[i]), every)
    amb = _compare(h, w, x, got, orc)
    _say("  ambiguous positions: %d of %d; smallest top-two gap %.3g" % (amb, B * (k + 1), float(orc.top2_gap.min())))


def test_lm_head_integer_ties_lowest_index(dev):
    """Integer inputs: every logit is exact in fp32 and ties are common; the
    lowest index must win, bit for bit."""
    rng = np.random.default_rng(82)
    B, k, V, D = 64, 5, 700, 64
    h = round_to_bf16_bits(rng.integers(-2, 3, (B, k + 1, D)).astype(np.float32))
    w = round_to_bf16_bits(rng.integers(-1, 2, (V, D)).astype(np.float32))
    g = oracle.lm_head_greedy(h, w, np.zeros((B, k), np.int32)).argmax
    x = np.where(rng.random((B, k)) < 0.8, g[:, :k], rng.integers(0, V, (B, k))).astype(np.int32)
    _say("case lm_head integer ties B=%d k=%d V=%d D=%d" % (B, k, V, D))
    got = _run_gpu(h, w, x, dev)
    orc = oracle.lm_head_greedy(h, w, x)
    assert np.sum(orc.top2_gap == 0.0) > 10
    _compare(h, w, x, got, orc, exact=True)
    assert np.array_equal(got[2], orc.argmax)


def test_lm_head_invalid_tokens_flag_sequence(dev):
    wl = _planted(6, 4, 900, 64)
    x = wl.tokens.copy()
    x[1, 3] = -5
    x[4, 0] = 900
    _say("case lm_head invalid tokens")
    got = _run_gpu(wl.hidden, wl.weight, x, dev)
    orc = oracle.lm_head_greedy(wl.hidden, wl.weight, x)
    _compare(wl.hidden, wl.weight, x, got, orc)
    assert got[0][1] == -1 and got[0][4] == -1


def test_lm_head_repeat_calls_are_bitwise_identical(dev):
    wl = _planted(40, 7, 4000, 128)
    _say("case lm_head determinism")
    a = _run_gpu(wl.hidden, wl.weight, wl.tokens, dev)
    b = _run_gpu(wl.hidden, wl.weight, wl.tokens, dev)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("name,seed", [("lmhead_selfdraft", 11), ("lmhead_grpo", 12)])
def test_lm_head_full_size_sampled(dev, name, seed):
    """Full workload on the GPU; every sequence checked for consistency, 8
    sequences (the first, the last and 6 drawn) against the oracle over the
    whole vocabulary."""
    cfg = workloads.LM_CONFIGS[name]
    _say("case lm_head full %s B=%d k=%d V=%d D=%d" % (name, cfg.B, cfg.k, cfg.V, cfg.D))
    wl = workloads.generate_lm_head(cfg)
    acc, out, am = _run_gpu(wl.hidden, wl.weight, wl.tokens, dev)
    _consistent(acc, out, am, wl.tokens, cfg.V)
    drawn = np.random.default_rng(seed).choice(np.arange(1, cfg.B - 1), 6, replace=False)
    idx = np.unique(np.concatenate([[0, cfg.B - 1], drawn]))
    orc = pooled(lambda i: oracle.lm_head_greedy(wl.hidden[i], wl.weight, wl.tokens[i]), idx)
    _compare(wl.hidden[idx], wl.weight, wl.tokens[idx], (acc[idx], out[idx], am[idx]), orc)
    # the planted margin makes the planted token the choice almost everywhere
    assert np.mean(am == wl.planted) > 0.99
    _say("  accepted mean %.3f" % float(np.mean(acc)))
