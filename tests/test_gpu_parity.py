"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases span several 8 KiB chunks and a ragged last chunk (V = 151936 is
37.09 bf16 chunks); the full-size cases are the five workloads at their
stated sizes, checked on every sequence where the oracle is fast and on a
sample otherwise.  Tolerances and ambiguity bands are described in parity.py.
"""
import sys

import numpy as np
import pytest

import oracle
import workloads
from parity import (check_row_stats, compare_vat, compare_vat_loss, compare_verify, pooled, run_vat_gpu,
                    run_vat_loss_gpu, run_verify_gpu, to_torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    import speculative_decoding_verification_amd as sv

    sv.load_library()  # fails loudly if the library is not built
    return torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _verify_case(wl, dev, T=None, onehot=None, seq_index=None):
    cfg = wl.config
    T = cfg.T if T is None else T
    oh = cfg.onehot if onehot is None else onehot
    _say("case verify %s B=%d k=%d V=%d %s T=%g onehot=%s" % (cfg.name, wl.n, cfg.k, cfg.V, cfg.dtype, T, oh))
    gpu = run_verify_gpu(wl, dev, temperature=T, onehot=oh)
    if seq_index is None:
        orc = oracle.verify(wl.target, wl.draft, wl.tokens, wl.uniforms, T, onehot=oh)
        check_row_stats(gpu["row_stats"], orc.target_mz, orc.draft_mz, T == 0.0, not oh and T != 0.0)
        rep = compare_verify(gpu, orc, cfg.k, cfg.V, T == 0.0)
    else:
        idx = np.asarray(seq_index)
        orc = pooled(lambda i: oracle.verify(wl.target[i], wl.draft[i] if wl.draft is not None else None,
                                             wl.tokens[i], wl.uniforms[i], T, onehot=oh), idx)
        gsub = {k: v[idx] for k, v in gpu.items() if k != "row_stats"}
        rows_per = cfg.k + 1
        st_t = gpu["row_stats"][: wl.n * rows_per].reshape(wl.n, rows_per, 2)[idx].reshape(-1, 2)
        st = st_t
        if not oh and T != 0.0:
            st_d = gpu["row_stats"][wl.n * rows_per:].reshape(wl.n, cfg.k, 2)[idx].reshape(-1, 2)
            st = np.concatenate([st_t, st_d])
        check_row_stats(st, orc.target_mz, orc.draft_mz, T == 0.0, not oh and T != 0.0)
        rep = compare_verify(gsub, orc, cfg.k, cfg.V, T == 0.0)
    _say("  parity ok:", rep)
    return gpu, rep


# ------------------------------------------------------------------ small cases

@pytest.mark.parametrize("name,changes", [
    ("tiny", {}),
    ("selfdraft", {"B": 8}),
    ("ngram_tail", {}),
    ("grpo", {"B": 6}),
    ("grpo_greedy", {"B": 16}),
])
def test_workloads_reduced(dev, name, changes):
    cfg = workloads.get_config(name).scaled(**changes)
    _verify_case(workloads.generate(cfg), dev)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_vat_reduced(dev, T):
    cfg = workloads.get_config("vat").scaled(B=12, T=T, draft_mode="sample" if T else "argmax")
    wl = workloads.generate(cfg)
    _say("case vat N=12 T=%g" % T)
    gpu = run_vat_gpu(wl, dev)
    orc = oracle.vat_labels(wl.target, wl.draft, wl.tokens, wl.uniforms, T, float(np.float32(cfg.decay)))
    check_row_stats(gpu["row_stats"], orc.target_mz, orc.draft_mz, T == 0.0, T != 0.0)
    _say("  parity ok:", compare_vat(gpu, orc, cfg.k, cfg.decay, T == 0.0))


# ------------------------------------------------------------------ VAT loss

def _vat_loss_case(cfg, dev, hard_weight=1.0, hard=None):
    wl = workloads.generate(cfg)
    h = wl.hard_tokens if hard is None else hard
    _say("case vat loss N=%d k=%d V=%d %s T=%g hard_weight=%g" % (cfg.B, cfg.k, cfg.V, cfg.dtype, cfg.T,
                                                                   hard_weight))
    gpu = run_vat_loss_gpu(wl, dev, hard_weight=hard_weight, hard=h)
    dec = float(np.float32(cfg.decay))
    orc = oracle.vat_loss(wl.target, wl.draft, wl.tokens, wl.uniforms, h, cfg.T, dec, float(np.float32(hard_weight)))
    lab = oracle.vat_labels(wl.target, wl.draft, wl.tokens, wl.uniforms, cfg.T, dec)
    valid = orc.first_reject >= 0
    if valid.any():
        check_row_stats(gpu["row_stats"], lab.target_mz, lab.draft_mz, False, True)
    _say("  parity ok:", compare_vat_loss(gpu, orc, lab, cfg.k, cfg.decay, hard_weight))
    return gpu, orc


@pytest.mark.parametrize("B,k,V,dtype,T,hw", [
    (12, 16, 128256, "f32", 1.0, 1.0),    # the VAT block shape, 12 blocks
    (6, 16, 151936, "bf16", 0.7, 0.5),    # bf16 rows, ragged last chunk
    (3, 5, 140000, "f32", 1.0, 2.0),      # 69 chunks: more than one pass of the lanes
    (20, 1, 3000, "f32", 1.3, 0.0),       # k = 1, no hard term
    (4, 7, 1001, "bf16", 1.0, 1.0),       # rows not 16-byte aligned: scalar loads
    (3, 64, 2500, "f32", 0.9, 1.0),       # k = 64
])
def test_vat_loss_reduced(dev, B, k, V, dtype, T, hw):
    cfg = workloads.Config("vatloss", "vat", B, k, V, dtype, T, 4.0, 0.25, "sample", 777)
    _vat_loss_case(cfg, dev, hard_weight=hw)


def test_vat_loss_invalid_hard_token_flags_block(dev):
    cfg = workloads.Config("vatloss", "vat", 5, 6, 4000, "f32", 1.0, 4.0, 0.25, "sample", 778)
    wl = workloads.generate(cfg)
    h = wl.hard_tokens.copy()
    h[1, 3] = cfg.V
    h[3, 0] = -1
    gpu, orc = _vat_loss_case(cfg, dev, hard=h)
    assert gpu["first_reject"][1] == -1 and gpu["first_reject"][3] == -1


# ------------------------------------------------------------------ VAT loss gradient

GRAD_RTOL = 2e-5


def _softmax_rows(a, T):
    from scipy import special

    return special.softmax(np.asarray(a, np.float64) / T, axis=-1)


def _logits_f64(a):
    return workloads.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def _compare_grad(g, target, draft, hard, weights, T, hw):
    """Element by element against the oracle's gradient for the GPU's own
    weights (the gradient takes them as given), within GRAD_RTOL of the size
    of the three terms w/T ((1 + hw) q, p, hw [y == h]) at each element."""
    T = float(np.float32(T))
    hw = float(np.float32(hw))
    w = weights.astype(np.float64)
    o = pooled(lambda i: oracle.vat_loss_grad(target[i], draft[i], hard[i], w[i], T, hw), np.arange(len(w)))
    p = _softmax_rows(_logits_f64(target), T)
    q = _softmax_rows(_logits_f64(draft), T)
    eh = np.zeros_like(p)
    N, k, V = p.shape
    np.put_along_axis(eh, np.clip(hard, 0, V - 1)[..., None].astype(np.int64), 1.0, axis=2)
    scale = (np.abs(w) / T)[..., None] * ((1 + hw) * q + p + hw * eh)
    err = np.abs(g.astype(np.float64) - o)
    bad = err > GRAD_RTOL * scale + 1e-30
    assert not bad.any(), (np.argwhere(bad)[:5], err[bad][:5], scale[bad][:5])
    assert np.all(g[w == 0.0] == 0.0)
    return float((err / np.maximum(scale, 1e-300)).max())


@pytest.mark.parametrize("B,k,V,dtype,T,hw,decay", [
    (12, 16, 128256, "f32", 1.0, 1.0, 0.8),    # the VAT block shape, 12 blocks
    (6, 16, 151936, "bf16", 0.7, 0.5, 0.8),    # bf16 rows, ragged last chunk
    (3, 5, 140000, "f32", 1.0, 2.0, 0.0),      # decay 0: zero rows after the first rejection
    (20, 1, 3000, "f32", 1.3, 0.0, 0.8),       # k = 1, no hard term
    (4, 7, 1001, "bf16", 1.0, 1.0, 0.8),       # rows not 16-byte aligned: scalar path
    (3, 64, 2502, "f32", 0.9, 1.0, 0.8),       # k = 64, V not a multiple of 4: scalar path
])
def test_vat_loss_grad_reduced(dev, B, k, V, dtype, T, hw, decay):
    import speculative_decoding_verification_amd as sv

    cfg = workloads.Config("vatgrad", "vat", B, k, V, dtype, T, 4.0, 0.25, "sample", 779)
    wl = workloads.generate(cfg)
    _say("case vat loss grad B=%d k=%d V=%d %s T=%g hw=%g decay=%g" % (B, k, V, dtype, T, hw, decay))
    t, d = to_torch(wl.target, dev), to_torch(wl.draft, dev)
    h = to_torch(wl.hard_tokens, dev)
    res = sv.vat_loss(t, d, to_torch(wl.tokens, dev), to_torch(wl.uniforms, dev), h, T, decay, hw,
                      return_row_stats=True)
    g = sv.vat_loss_grad(t, d, h, res.weights, res.row_stats, T, hw).cpu().numpy()
    w = res.weights.cpu().numpy()
    worst = _compare_grad(g, wl.target, wl.draft, wl.hard_tokens, w, T, hw)
    assert np.allclose(g.astype(np.float64).sum(axis=2), 0.0, atol=1e-5 * max(1.0, float(np.abs(w).max()) / T))
    _say("  grad parity ok, worst error / bound scale %.3g" % worst)


def test_vat_loss_grad_flagged_block_is_zero(dev):
    import speculative_decoding_verification_amd as sv

    cfg = workloads.Config("vatgrad", "vat", 5, 6, 4000, "f32", 1.0, 4.0, 0.25, "sample", 780)
    wl = workloads.generate(cfg)
    hard = wl.hard_tokens.copy()
    hard[2, 1] = cfg.V
    _say("case vat loss grad with a flagged block")
    t, d = to_torch(wl.target, dev), to_torch(wl.draft, dev)
    h = to_torch(hard, dev)
    res = sv.vat_loss(t, d, to_torch(wl.tokens, dev), to_torch(wl.uniforms, dev), h, 1.0, 0.8, 1.0,
                      return_row_stats=True)
    g = sv.vat_loss_grad(t, d, h, res.weights, res.row_stats, 1.0, 1.0).cpu().numpy()
    assert res.first_reject.cpu().numpy()[2] == -1
    assert np.all(g[2] == 0.0)
    _compare_grad(g, wl.target, wl.draft, hard, res.weights.cpu().numpy(), 1.0, 1.0)


def _custom(B, k, V, dtype, T, sigma_t=3.0, sigma_d=0.5, mode="sample", onehot=False, seed=900):
    return workloads.Config("custom", "verify", B, k, V, dtype, T, sigma_t, None if onehot else sigma_d,
                            mode if not onehot else "ngram", seed)


@pytest.mark.parametrize("B,k,V,dtype,T,onehot", [
    (5, 3, 1001, "bf16", 1.0, False),     # rows not 16-byte aligned: scalar loads
    (50, 2, 7, "f32", 1.0, False),        # V smaller than a vector
    (64, 1, 4096, "bf16", 1.0, False),    # exactly one chunk
    (3, 64, 5000, "f32", 0.8, False),     # k = 64: a full wavefront of positions
    (1, 16, 151936, "bf16", 1.0, False),  # B = 1
    (4, 5, 8200, "bf16", 0.01, False),    # sharp temperature, ragged 8-logit last chunk
    (6, 4, 3000, "f32", 1.0, True),       # one-hot draft, fp32
    (6, 4, 1001, "bf16", 1.0, True),      # one-hot draft, unaligned rows
    (20, 4, 2048, "f32", 0.0, False),     # greedy fp32, exactly one chunk
    (9, 3, 1001, "bf16", 0.0, False),     # greedy unaligned
    (32, 16, 151936, "bf16", 1.0, True),  # one-hot, several residencies: finishers behind their workers
    (2, 64, 151936, "bf16", 1.0, True),   # one-hot window mode, k = 64: position 0 from row 0's chunk words
    (1, 16, 600000, "f32", 1.0, True),    # one-hot window mode, 293 chunks staged beside the segment words
    (24, 3, 151936, "bf16", 0.7, False),  # sampling in one residency: finishers first, residual roles after
    (12, 5, 151936, "bf16", 0.0, False),  # greedy in one residency, finishers first
])
def test_edge_shapes(dev, B, k, V, dtype, T, onehot):
    cfg = _custom(B, k, V, dtype, T, onehot=onehot, mode="argmax" if T == 0 else "sample")
    _verify_case(workloads.generate(cfg), dev)


def _planted_rejections(rej, k, V, T, onehot, seed):
    """Each row has one planted maximum 40 above the rest, so the draft token
    is kept (argmax) or rejected (any other token) with certainty; sequence b
    first rejects at rej[b] (k: full acceptance, the bonus row)."""
    rng = np.random.default_rng(seed)
    B = len(rej)
    t = (2.0 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    g = rng.integers(0, V, (B, k + 1))
    t[np.arange(B)[:, None], np.arange(k + 1)[None, :], g] = 40.0
    bits = workloads.round_to_bf16_bits(t)
    x = g[:, :k].astype(np.int32).copy()
    for b, r in enumerate(rej):
        if r < k:
            x[b, r] = (g[b, r] + 1 + rng.integers(0, V - 1)) % V
    u = rng.random((B, k + 1), dtype=np.float32)
    cfg = _custom(B, k, V, "bf16", T, onehot=onehot, mode="argmax" if T == 0 else "sample")
    return workloads.Workload(cfg, 0, bits, None, x, u)


@pytest.mark.parametrize("T,onehot", [(0.0, False), (1.0, True)])
@pytest.mark.parametrize("rej", [(0, 2, 3, 5, 8, 13, 15, 16), (16, 16, 16, 16, 4, 6, 7, 12)])
def test_first_rejection_at_every_depth(dev, T, onehot, rej):
    """Small one-hot and greedy calls whose statistics are not asked for read
    every row at once, or, after a call on the same workspace that rejected
    every sequence's first token, the rows of later positions only as the
    accepted prefix comes near them.  First rejections at every depth and
    full acceptance, in both regimes: the call with statistics (every row
    read) matches the oracle, and the calls without match it bit for bit."""
    import torch

    import speculative_decoding_verification_amd as sv

    k, V = 16, 151936
    wl = _planted_rejections(rej, k, V, T, onehot, 81)
    gpu, _ = _verify_case(wl, dev)
    assert list(gpu["accepted_len"]) == list(rej)
    primer = _planted_rejections((0,) * len(rej), k, V, T, onehot, 82)
    ws = torch.zeros(8 << 20, dtype=torch.uint8, device=dev)

    def lean(w):
        t = to_torch(w.target, dev)
        return sv.verify(t, None, to_torch(w.tokens, dev), to_torch(w.uniforms, dev), T, onehot=onehot, workspace=ws)

    for first in (primer, wl):  # the second call reads every row: its predecessor accepted tokens
        out = lean(first)
        if first is primer:
            assert np.all(out.accepted_len.cpu().numpy() == 0)
        out = lean(wl)
        _say("  after %s:" % ("all-rejecting call" if first is primer else "accepting call"),
             list(out.accepted_len.cpu().numpy()))
        assert np.array_equal(out.accepted_len.cpu().numpy(), gpu["accepted_len"])
        assert np.array_equal(out.out_tokens.cpu().numpy(), gpu["out_tokens"])


def test_neg_inf_logits_and_greedy_ties(dev):
    rng = np.random.default_rng(77)
    B, k, V = 12, 4, 9000
    # coarse integer logits: many exact ties for the maximum; -inf blocks
    t = rng.integers(-3, 4, (B, k + 1, V)).astype(np.float32)
    t[:, :, 4096:6000] = -np.inf
    t[:, :, 7000:] = -np.inf
    d = t[:, :k] + rng.integers(-1, 2, (B, k, V)).astype(np.float32)
    bits_t = workloads.round_to_bf16_bits(t)
    bits_d = workloads.round_to_bf16_bits(d)
    g = np.argmax(t, axis=2)
    x = np.where(rng.random((B, k)) < 0.6, g[:, :k], rng.integers(0, 4096, (B, k))).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    cfg = _custom(B, k, V, "bf16", 1.0)
    wl = workloads.Workload(cfg, 0, bits_t, bits_d, x, u)
    _verify_case(wl, dev, T=0.0)
    gpu, _ = _verify_case(wl, dev, T=1.0)
    outs = gpu["out_tokens"][np.arange(B), np.maximum(gpu["accepted_len"], 0)]
    assert not np.any(((outs >= 4096) & (outs < 6000)) | (outs >= 7000))


@pytest.mark.parametrize("V,dtype", [(5000, "bf16"), (1001, "bf16"), (3000, "f32"), (151936, "bf16")])
def test_rejection_with_zero_residual_draws_from_target(dev, V, dtype):
    """Draft rows equal to the target rows and a draft token at a -inf logit:
    p(x) = q(x) = 0 rejects, and max(0, p - q) is zero everywhere, so the
    token comes from p_r (the degenerate-residual reading).  The kernel must
    round p and q on their own before the difference for the residual to be
    exactly zero.  V = 1001 bf16 rows are not 16-byte aligned (scalar loads);
    V = 151936 spans 38 chunks."""
    rng = np.random.default_rng(78)
    B, k = 10, 4
    t = (3.0 * rng.standard_normal((B, k + 1, V))).astype(np.float32)
    dead = np.arange(V // 3, V // 3 + max(V // 50, 4))
    t[:, :, dead] = -np.inf
    if dtype == "bf16":
        bits = workloads.round_to_bf16_bits(t)
        t_in, d_in = bits, bits[:, :k].copy()
        tf = workloads.bf16_bits_to_f32(bits)
    else:
        t_in, d_in = t, t[:, :k].copy()
        tf = t
    g = np.argmax(tf, axis=2)
    r = rng.integers(0, k, B)
    x = g[:, :k].astype(np.int32).copy()
    x[np.arange(B), r] = rng.choice(dead, B)
    u = rng.random((B, k + 1), dtype=np.float32)
    cfg = _custom(B, k, V, dtype, 1.0)
    wl = workloads.Workload(cfg, 0, t_in, d_in, x, u)
    gpu, _ = _verify_case(wl, dev)
    assert np.array_equal(gpu["accepted_len"], r)
    outs = gpu["out_tokens"][np.arange(B), r]
    assert not np.any(np.isin(outs, dead))


def test_invalid_tokens_flag_sequence(dev):
    cfg = _custom(6, 3, 2000, "f32", 1.0)
    wl = workloads.generate(cfg)
    wl.tokens[1, 2] = 2000
    wl.tokens[4, 0] = -7
    gpu, _ = _verify_case(wl, dev)
    assert list(gpu["accepted_len"][[1, 4]]) == [-1, -1]
    gpu0, _ = _verify_case(wl, dev, T=0.0)
    assert list(gpu0["accepted_len"][[1, 4]]) == [-1, -1]


def test_determinism_bitwise(dev):
    cfg = workloads.get_config("grpo").scaled(B=16)
    wl = workloads.generate(cfg)
    runs = [run_verify_gpu(wl, dev) for _ in range(3)]
    for r in runs[1:]:
        for key in runs[0]:
            assert np.array_equal(runs[0][key].view(np.uint8), r[key].view(np.uint8)), key


def test_two_streams_in_flight_match_one_stream(dev):
    """Calls on two streams at once, each with the workspace the binding keeps
    for its stream, give the results of the same calls made one at a time."""
    import speculative_decoding_verification_amd as sv
    import torch

    from parity import to_torch

    cases = [workloads.generate(workloads.get_config("grpo").scaled(B=24)),
             workloads.generate(_custom(40, 6, 20000, "bf16", 0.8, seed=901))]
    args = []
    for wl in cases:
        args.append((to_torch(wl.target, dev), to_torch(wl.draft, dev), to_torch(wl.tokens, dev),
                     to_torch(wl.uniforms, dev), wl.config.T))
    ref = [sv.verify(*a, return_row_stats=True) for a in args]
    ref = [(r.accepted_len.cpu().numpy(), r.out_tokens.cpu().numpy(), r.row_stats.cpu().numpy()) for r in ref]
    streams = [torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream(dev))
    outs = [[], []]
    for _ in range(4):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                outs[i].append(sv.verify(*args[i], return_row_stats=True))
    torch.cuda.synchronize(dev)
    for i in range(2):
        for r in outs[i]:
            assert np.array_equal(r.accepted_len.cpu().numpy(), ref[i][0])
            assert np.array_equal(r.out_tokens.cpu().numpy(), ref[i][1])
            assert np.array_equal(r.row_stats.cpu().numpy().view(np.uint32), ref[i][2].view(np.uint32))


def test_gpu_losslessness_chi_square(dev):
    """The HIP sampler's outputs follow the target: V=8, k=3, 200k sequences."""
    from scipy import stats

    import speculative_decoding_verification_amd as sv
    import torch

    rng = np.random.default_rng(4242)
    V, k, B = 8, 3, 200_000

    def simplex(z=0):
        p = rng.random(V) + 0.05
        if z:
            p[rng.choice(V, z, replace=False)] = 0
        return p / p.sum()

    with np.errstate(divide="ignore"):
        lt1 = np.log(np.stack([simplex(1) for _ in range(k + 1)])).astype(np.float32)
        ld1 = np.log(np.stack([simplex(int(i == 1)) for i in range(k)])).astype(np.float32)
    P = np.stack([oracle.softmax(lt1[i].astype(np.float64), 1.0)[0] for i in range(k + 1)])
    Q = np.stack([oracle.softmax(ld1[i].astype(np.float64), 1.0)[0] for i in range(k)])
    x = np.stack([rng.choice(V, size=B, p=Q[i]) for i in range(k)], axis=1).astype(np.int32)
    u = rng.random((B, k + 1), dtype=np.float32)
    _say("case chi-square V=8 k=3 B=200000")
    t = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(lt1, (B, k + 1, V)))).to(dev)
    d = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(ld1, (B, k, V)))).to(dev)
    res = sv.verify(t, d, to_torch(x, dev), to_torch(u, dev), 1.0)
    L = res.accepted_len.cpu().numpy()
    out = res.out_tokens.cpu().numpy()
    alpha = np.minimum(P[:k], Q).sum(axis=1)
    pv = []
    for j in range(k + 1):
        reach = L >= j
        n = int(reach.sum())
        er = float(np.prod(alpha[:j]))
        sig = np.sqrt(er * (1 - er) / B) if 0 < er < 1 else 0
        assert abs(n / B - er) < 5 * sig + 1e-9, (j, n / B, er)
        c = np.bincount(out[reach, j], minlength=V)
        sup = P[j] > 0
        assert c[~sup].sum() == 0
        pv.append(stats.chisquare(c[sup], n * P[j][sup] / P[j][sup].sum()).pvalue)
    _say("  chi-square p-values", pv)
    assert min(pv) > 1e-4 / len(pv)


# ------------------------------------------------------------------ full sizes

def test_full_selfdraft_all_sequences(dev):
    wl = workloads.generate(workloads.get_config("selfdraft"))
    _verify_case(wl, dev)


def test_full_ngram_tail(dev):
    wl = workloads.generate(workloads.get_config("ngram_tail"))
    _verify_case(wl, dev)


def test_full_grpo_sampled(dev):
    cfg = workloads.get_config("grpo")
    wl = workloads.generate(cfg)
    idx = np.random.default_rng(1).choice(cfg.B, 96, replace=False)
    idx.sort()
    _verify_case(wl, dev, seq_index=idx)


def test_full_grpo_greedy_all_sequences(dev):
    cfg = workloads.get_config("grpo_greedy")
    wl = workloads.generate(cfg, with_draft=True)
    _verify_case(wl, dev)


def test_full_vat_sampled(dev):
    import speculative_decoding_verification_amd as sv
    import torch

    cfg = workloads.get_config("vat")
    _say("case vat full N=2048 k=16 V=128256 f32 (33.6 GB, device-generated)")
    t, d, x, u = workloads.generate_on_device(cfg, dev)
    res = sv.vat_labels(t, d, x, u, cfg.T, cfg.decay, return_probs=True)
    torch.cuda.synchronize()
    fr = res.first_reject.cpu().numpy()
    mask = res.accept_mask.cpu().numpy()
    w = res.weights.cpu().numpy()
    i = np.arange(cfg.k)
    # every block: labels and weights follow its first rejection
    assert np.all((fr >= 0) & (fr <= cfg.k))
    assert np.array_equal(mask, (i[None, :] < fr[:, None]).astype(np.uint8))
    dec = float(np.float32(cfg.decay))
    want = np.where(i[None, :] < fr[:, None], 1.0, dec ** np.maximum(i[None, :] - fr[:, None], 0))
    assert np.allclose(w, want, rtol=1e-7, atol=0)
    idx = np.random.default_rng(5).choice(cfg.B, 64, replace=False)
    idx.sort()
    ti = torch.as_tensor(idx, device=dev)
    tl = t.index_select(0, ti).cpu().numpy()
    dl = d.index_select(0, ti).cpu().numpy()
    xs = x.index_select(0, ti).cpu().numpy()
    us = u.index_select(0, ti).cpu().numpy()
    dec = float(np.float32(cfg.decay))
    orc = pooled(lambda i: oracle.vat_labels(tl[i], dl[i], xs[i], us[i], cfg.T, dec), np.arange(len(idx)))
    gpu = {"first_reject": fr[idx], "accept_mask": mask[idx], "weights": w[idx],
           "probs": res.probs.cpu().numpy()[idx]}
    rep = compare_vat(gpu, orc, cfg.k, cfg.decay, False)
    _say("  parity ok:", rep, "mean first_reject", fr.mean())
    del t, d, x, u, res
    torch.cuda.empty_cache()


def test_full_vat_loss_sampled(dev):
    """The VAT workload (N=2048, k=16, V=128256, fp32) through sv_vat_loss, with
    the target's own samples as hard labels; sampled blocks against the oracle."""
    import speculative_decoding_verification_amd as sv
    import torch

    cfg = workloads.get_config("vat")
    _say("case vat loss full N=2048 k=16 V=128256 f32 (33.6 GB, device-generated)")
    t, d, x, u = workloads.generate_on_device(cfg, dev)
    h = workloads.hard_tokens_on_device(cfg, t, dev)
    res = sv.vat_loss(t, d, x, u, h, cfg.T, cfg.decay, 1.0)
    torch.cuda.synchronize()
    fr = res.first_reject.cpu().numpy()
    loss = res.block_loss.cpu().numpy()
    assert np.all((fr >= 0) & (fr <= cfg.k)) and np.all(np.isfinite(loss)) and np.all(loss > 0)
    idx = np.random.default_rng(6).choice(cfg.B, 64, replace=False)
    idx.sort()
    ti = torch.as_tensor(idx, device=dev)
    tl, dl = t.index_select(0, ti).cpu().numpy(), d.index_select(0, ti).cpu().numpy()
    xs, us, hs = (a.index_select(0, ti).cpu().numpy() for a in (x, u, h))
    dec = float(np.float32(cfg.decay))
    every = np.arange(len(idx))
    orc = pooled(lambda i: oracle.vat_loss(tl[i], dl[i], xs[i], us[i], hs[i], cfg.T, dec, 1.0), every)
    lab = pooled(lambda i: oracle.vat_labels(tl[i], dl[i], xs[i], us[i], cfg.T, dec), every)
    gpu = {"first_reject": fr[idx], "accept_mask": res.accept_mask.cpu().numpy()[idx],
           "weights": res.weights.cpu().numpy()[idx], "soft_ce": res.soft_ce.cpu().numpy()[idx],
           "hard_ce": res.hard_ce.cpu().numpy()[idx], "block_loss": loss[idx]}
    _say("  parity ok:", compare_vat_loss(gpu, orc, lab, cfg.k, cfg.decay, 1.0), "mean loss", loss.mean())
    del t, d, x, u, h, res
    torch.cuda.empty_cache()


def test_full_vat_loss_grad_sampled(dev):
    """The gradient of the VAT workload's loss (N=2048, k=16, V=128256, fp32:
    16.8 GB written): every row sums to zero, sampled blocks against the oracle."""
    import speculative_decoding_verification_amd as sv
    import torch

    cfg = workloads.get_config("vat")
    _say("case vat loss grad full N=2048 k=16 V=128256 f32 (device-generated)")
    t, d, x, u = workloads.generate_on_device(cfg, dev)
    h = workloads.hard_tokens_on_device(cfg, t, dev)
    res = sv.vat_loss(t, d, x, u, h, cfg.T, cfg.decay, 1.0, return_row_stats=True)
    g = sv.vat_loss_grad(t, d, h, res.weights, res.row_stats, cfg.T, 1.0)
    rs = g.sum(dim=2, dtype=torch.float64)
    torch.cuda.synchronize()
    assert float(rs.abs().max()) < 1e-4
    idx = np.random.default_rng(7).choice(cfg.B, 16, replace=False)
    idx.sort()
    ti = torch.as_tensor(idx, device=dev)
    gs = g.index_select(0, ti).cpu().numpy()
    tl, dl = t.index_select(0, ti).cpu().numpy(), d.index_select(0, ti).cpu().numpy()
    hs = h.index_select(0, ti).cpu().numpy()
    ws = res.weights.index_select(0, ti).cpu().numpy()
    worst = _compare_grad(gs, tl, dl, hs, ws, cfg.T, 1.0)
    _say("  grad parity ok on blocks", idx.tolist(), "worst error / bound scale %.3g" % worst)
    del t, d, x, u, h, res, g, rs
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ acceptance telemetry

def _hist_ref(acc, k):
    acc = np.asarray(acc, np.int64)
    h = np.zeros(k + 4, np.int64)
    valid = (acc >= 0) & (acc <= k)
    h[: k + 1] = np.bincount(acc[valid], minlength=k + 1)
    h[k + 1] = np.count_nonzero(acc == -1)
    h[k + 2] = np.count_nonzero(acc == -2)
    h[k + 3] = acc.size - h[: k + 3].sum()
    return h


@pytest.mark.parametrize("B,k", [(0, 5), (1, 1), (257, 7), (100003, 16), (4096, 64)])
def test_accept_histogram_exact(dev, B, k):
    import speculative_decoding_verification_amd as sv
    import torch

    _say("case accept histogram B=%d k=%d" % (B, k))
    rng = np.random.default_rng(B + k)
    acc = rng.integers(-3, k + 3, size=B).astype(np.int32)
    h = sv.accept_histogram(torch.from_numpy(acc).to(dev), k).cpu().numpy()
    assert np.array_equal(h, _hist_ref(acc, k))


def test_telemetry_after_verify_drives_the_controller(dev):
    import speculative_decoding_verification_amd as sv

    cfg = workloads.get_config("selfdraft").scaled(B=64)
    wl = workloads.generate(cfg)
    t, d, x, u = workloads.to_device(wl, dev)
    res = sv.verify(t, d, x, u, cfg.T)
    h = sv.accept_histogram(res.accepted_len, cfg.k).cpu().numpy()
    acc = res.accepted_len.cpu().numpy()
    assert np.array_equal(h, _hist_ref(acc, cfg.k))
    ctl = sv.DraftLengthController()
    ctl.update(h)
    assert ctl.efficiency == pytest.approx(float(np.mean(acc + 1)), rel=1e-6)
    _say("  block efficiency %.3f at k=%d" % (ctl.efficiency, cfg.k))
