"""GPU parity of LM-head-fused sampling verification (sv_verify_lm_head)
against the oracle, which forms both sides' logits in fp64 and runs the same
rule.  The kernel's logits are fp32 sums of exact bf16 products: at D = 4096
and logits of size ~10 their error is ~1e-5, which moves p(x)/q(x) by a few
1e-5 / T.  Probabilities are therefore compared within 2e-4 relative, and a
test whose u lies within 2e-4 of p/q (or a draw within 2e-4 of an end of the
oracle's interval) is counted as ambiguous and compared only up to it.
At low temperature a residual max(0, p - q) between two near one-hot rows on
the same token is made of masses far below the logits' rounding (1e-10 at
T = 0.05); such draws are not determined by fp32 logits, so the
low-temperature case uses a draft whose rows peak elsewhere.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import pooled, compare_verify

pytestmark = pytest.mark.gpu

LM_BAND = 2e-4


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


def _run_gpu(wl, dev, T, idx=None):
    import torch

    import speculative_decoding_verification_amd as sv

    th, tw, dh, dw, x, u = workloads.lm_head_sample_to_device(wl, dev)
    res = sv.verify_lm_head(th, tw, dh, dw, x, u, T, return_probs=True)
    torch.cuda.synchronize()
    return {"accepted_len": res.accepted_len.cpu().numpy(), "out_tokens": res.out_tokens.cpu().numpy(),
            "probs": res.probs.cpu().numpy()}


def _oracle(wl, T, idx=None):
    sl = slice(None) if idx is None else np.asarray(idx)
    return oracle.lm_head_verify(wl.target_hidden[sl], wl.target_weight, wl.draft_hidden[sl], wl.draft_weight,
                                 wl.tokens[sl], wl.uniforms[sl], T)


def _case(dev, cfg, **changes):
    cfg = cfg.scaled(**changes)
    _say("case lm_head sample B=%d k=%d V=%d D=%d T=%g noise=%g wnoise=%g" % (
        cfg.B, cfg.k, cfg.V, cfg.D, cfg.T, cfg.draft_noise, cfg.draft_weight_noise))
    wl = workloads.generate_lm_head_sample(cfg)
    gpu = _run_gpu(wl, dev, cfg.T)
    orc = _oracle(wl, cfg.T)
    rep = compare_verify(gpu, orc, cfg.k, cfg.V, False, band=LM_BAND, rtol=LM_BAND)
    _say("  ", rep, "mean accepted %.2f" % float(np.mean(gpu["accepted_len"])))
    return gpu, orc


TINY = workloads.LM_CONFIGS["lmhead_sample_tiny"]


@pytest.mark.parametrize("B,k,V,D,T,noise,wnoise", [
    (90, 5, 3000, 256, 1.0, 0.3, 0.0),     # 3 target row tiles, ragged vocabulary tiles
    (90, 5, 3000, 256, 1.0, 2.0, 0.0),     # noisy draft: many rejections and residual draws
    (40, 7, 2048, 192, 0.6, 1.0, 0.1),     # the draft's own output layer
    (3, 64, 300, 64, 1.0, 1.5, 0.0),       # longest draft
    (1, 1, 1, 64, 1.0, 0.3, 0.0),          # one token
    (9, 16, 8193, 128, 2.0, 1.0, 0.05),    # last vocabulary tile holds one column
    (20, 3, 600, 64, 0.05, 3.0, 0.0),      # low temperature: near one-hot rows (distinct argmaxes)
])
def test_lm_head_sample_reduced(dev, B, k, V, D, T, noise, wnoise):
    plant = 8.0 if V <= 1000 else 10.0
    _case(dev, TINY, B=B, k=k, V=V, D=D, T=T, draft_noise=noise, draft_weight_noise=wnoise, plant=plant)


def test_lm_head_sample_invalid_tokens(dev):
    cfg = TINY.scaled(B=6, k=4, V=900, D=64, draft_noise=1.0)
    wl = workloads.generate_lm_head_sample(cfg)
    wl.tokens = wl.tokens.copy()
    wl.tokens[1, 2] = -3
    wl.tokens[4, 0] = 900
    _say("case lm_head sample invalid tokens")
    gpu = _run_gpu(wl, dev, cfg.T)
    orc = _oracle(wl, cfg.T)
    compare_verify(gpu, orc, cfg.k, cfg.V, False, band=LM_BAND, rtol=LM_BAND)
    assert gpu["accepted_len"][1] == -1 and gpu["accepted_len"][4] == -1
    assert np.all(gpu["out_tokens"][1] == -1) and np.all(gpu["out_tokens"][4] == -1)


def test_lm_head_sample_first_token_follows_the_target(dev):
    """Losslessness through the whole path: one position, the draft token
    drawn from q with numpy, the committed token must follow p (chi-square
    over many sequences that share one context)."""
    import torch

    import speculative_decoding_verification_amd as sv

    rng = np.random.default_rng(91)
    n, V, D = 40000, 12, 64
    ht = workloads.round_to_bf16_bits(rng.standard_normal((1, 2, D)).astype(np.float32))
    hd = workloads.round_to_bf16_bits(rng.standard_normal((1, 1, D)).astype(np.float32))
    w = workloads.round_to_bf16_bits((rng.standard_normal((V, D)) * 0.25).astype(np.float32))
    p = np.exp(oracle.lm_head_logits(ht[0, 0], w)); p /= p.sum()
    q = np.exp(oracle.lm_head_logits(hd[0, 0], w)); q /= q.sum()
    x = rng.choice(V, size=n, p=q).astype(np.int32).reshape(n, 1)
    u = rng.random((n, 2), dtype=np.float32)
    _say("case lm_head sample chi-square n=%d V=%d" % (n, V))

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    th = bf(np.repeat(ht, n, axis=0))
    dh = bf(np.repeat(hd, n, axis=0))
    wt = bf(w)
    res = sv.verify_lm_head(th, wt, dh, wt, torch.from_numpy(x).to(dev), torch.from_numpy(u).to(dev), 1.0)
    torch.cuda.synchronize()
    first = res.out_tokens.cpu().numpy()[:, 0]
    counts = np.bincount(first, minlength=V)
    expected = p * n
    chi2 = float(((counts - expected) ** 2 / expected).sum())
    # 11 degrees of freedom: the 0.999 quantile is 31.3
    assert chi2 < 31.3, (chi2, counts, expected)
    # and the draft was not already the target: the test has power
    assert float(np.abs(p - q).sum()) > 0.2


@pytest.mark.parametrize("name,seed", [("lmhead_sample_selfdraft", 21), ("lmhead_sample_grpo", 22)])
def test_lm_head_sample_full_size(dev, name, seed):
    cfg = workloads.LM_CONFIGS[name]
    _say("case lm_head sample full %s" % name)
    wl = workloads.generate_lm_head_sample(cfg)
    gpu = _run_gpu(wl, dev, cfg.T)
    acc = gpu["accepted_len"]
    assert np.all((acc >= 0) & (acc <= cfg.k))
    for b in range(cfg.B):
        r = acc[b]
        assert np.array_equal(gpu["out_tokens"][b, :r], wl.tokens[b, :r])
        assert 0 <= gpu["out_tokens"][b, r] < cfg.V and np.all(gpu["out_tokens"][b, r + 1:] == -1)
    # 8 sequences against the oracle: the first, the last and 6 drawn
    drawn = np.random.default_rng(seed).choice(np.arange(1, cfg.B - 1), 6, replace=False)
    idx = np.unique(np.concatenate([[0, cfg.B - 1], drawn]))
    orc = pooled(lambda i: _oracle(wl, cfg.T, i), idx)
    sub = {key: val[idx] for key, val in gpu.items()}
    rep = compare_verify(sub, orc, cfg.k, cfg.V, False, band=LM_BAND, rtol=LM_BAND)
    _say("  ", rep, "mean accepted %.3f" % float(np.mean(acc)))
