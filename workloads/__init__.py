"""Seeded synthetic workloads for batched speculative-sampling verification.

The parity tests feed the same arrays to the HIP library and to the fp64
oracle, and the bench times the library on them.  This module holds none of
the verification arithmetic (no softmax, acceptance test, residual or
sampler): it draws Gaussian logits, rounds them to bfloat16, draws the draft
tokens (exponential race over the draft logits, i.e. the Gumbel-max trick, an
argmax, or an n-gram-style coin), and draws the host uniforms.

Every sequence (or VAT block) ``b`` is generated from its own PCG64 streams,
keyed by ``(seed, stream, b)``, so any subset of sequences of a configuration
can be regenerated on its own, bit for bit, and a reduced-batch variant holds
exactly the first sequences of the full one.

Workloads (shapes and value distributions as stated for each configuration;
logits stand in for the output of a target/draft forward, since the
verification step only ever sees logits):

=============  ======================================================================
tiny           B=4, k=4, V=1000, fp32, T=1; t = 3z, d = t + 0.3z', x ~ softmax(d/T)
selfdraft      B=128, k=5, V=151936, bf16, T=1; t = 4z, d = t + 0.1z', x ~ softmax(d/T)
ngram_tail     B=8, k=16, V=151936, bf16 target, one-hot draft, T=1; t = 5z;
               x = argmax t w.p. 0.9, else uniform over [0, V)
grpo           B=320, k=7, V=151936, bf16, T=0.6; t = 4z, d = t + 0.2z', x ~ softmax(d/T)
grpo_greedy    same logits as grpo, T=0; x = argmax d (lowest id)
vat            N=2048 blocks, k=16, V=128256, fp32, T=1, decay 0.8; t = 4z, d = t + 0.25z',
               x ~ softmax(d/T); target has k rows per block (no bonus row)
=============  ======================================================================

LM-head workloads (greedy verification with the logits formed from hidden
states ``h`` [B][k+1][D] and output-layer weights ``W`` [V][D], both bf16):
``W = z_w / sqrt(D)`` (so every logit h . w_y of an unplanted row is about
N(0, |h|^2 / D)), ``h = z + plant * W[t]`` for a planted token t per
position (t uniform over [0, V)), so that t is the likely argmax by a margin
of about ``plant``; draft token = t w.p. ``hit``, else uniform over [0, V).

=================  ===================================================================
lmhead_tiny        B=6, k=4, V=1000, D=128, plant 8, hit 0.8
lmhead_selfdraft   B=128, k=5, V=151936, D=4096, plant 8, hit 0.95
lmhead_grpo        B=320, k=7, V=151936, D=4096, plant 8, hit 0.9
=================  ===================================================================

Sampling (T > 0) LM-head workloads add the draft side: the draft's hidden
state at position i is the target's plus ``draft_noise`` * N(0, I) (bf16),
its output layer is the target's (a drafter that shares the output layer) or,
with ``draft_weight_noise`` > 0, the target's plus that much relative noise;
uniforms U[0,1) per sequence.  The planted margin is larger (14 at V=151936:
the planted token holds about 80% of the target's mass at T=1).

=======================  =============================================================
lmhead_sample_tiny       B=6, k=4, V=1000, D=128, T=1, plant 8, hit 0.8
lmhead_sample_selfdraft  B=128, k=5, V=151936, D=4096, T=1, plant 14, hit 0.95
lmhead_sample_grpo       B=320, k=7, V=151936, D=4096, T=0.6, plant 14, hit 0.9
=======================  =============================================================
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = ["Config", "Workload", "CONFIGS", "get_config", "generate", "generate_on_device", "to_device",
           "round_to_bf16_bits", "bf16_bits_to_f32", "LmHeadConfig", "LmHeadWorkload", "LM_CONFIGS",
           "lm_head_weight", "generate_lm_head", "lm_head_to_device", "LmHeadSampleWorkload",
           "generate_lm_head_sample", "lm_head_sample_to_device"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    kind: str            # "verify" or "vat"
    B: int               # sequences (verify) or draft blocks (vat)
    k: int               # draft positions
    V: int               # vocabulary
    dtype: str           # "f32" or "bf16"
    T: float             # temperature (0 = greedy)
    sigma_t: float       # target logits = sigma_t * N(0,1)
    sigma_d: Optional[float]  # draft logits = target + sigma_d * N(0,1); None = one-hot draft
    draft_mode: str      # "sample" | "argmax" | "ngram"
    seed_logits: int
    seed_draft: int = 1
    seed_u: int = 0
    decay: float = 0.8   # vat only
    ngram_hit: float = 0.9  # ngram only: probability that x is the target argmax

    @property
    def onehot(self) -> bool:
        return self.sigma_d is None

    @property
    def target_rows_per_seq(self) -> int:
        return self.k + 1 if self.kind == "verify" else self.k

    @property
    def n_uniforms(self) -> int:
        return self.k + 1 if self.kind == "verify" else self.k

    @property
    def reads_draft(self) -> bool:
        return (not self.onehot) and self.T != 0.0

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def algorithmic_bytes(self) -> int:
        """Every logit the path needs, read once (tokens/uniforms/outputs excluded)."""
        rows = self.B * self.target_rows_per_seq
        if self.reads_draft:
            rows += self.B * self.k
        return rows * self.V * self.elem_bytes

    def positions(self) -> int:
        return self.B * self.k

    def scaled(self, **changes) -> "Config":
        return dataclasses.replace(self, **changes)


CONFIGS = {
    "tiny": Config("tiny", "verify", 4, 4, 1000, "f32", 1.0, 3.0, 0.3, "sample", 100),
    "selfdraft": Config("selfdraft", "verify", 128, 5, 151936, "bf16", 1.0, 4.0, 0.1, "sample", 200),
    "ngram_tail": Config("ngram_tail", "verify", 8, 16, 151936, "bf16", 1.0, 5.0, None, "ngram", 300),
    "grpo": Config("grpo", "verify", 320, 7, 151936, "bf16", 0.6, 4.0, 0.2, "sample", 400),
    "grpo_greedy": Config("grpo_greedy", "verify", 320, 7, 151936, "bf16", 0.0, 4.0, 0.2, "argmax", 400),
    "vat": Config("vat", "vat", 2048, 16, 128256, "f32", 1.0, 4.0, 0.25, "sample", 500),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    config: Config
    lo: int                       # first sequence index held
    target: np.ndarray            # [n][rows][V] float32 or uint16 (bf16 bits)
    draft: Optional[np.ndarray]   # [n][k][V] or None (one-hot)
    tokens: np.ndarray            # [n][k] int32
    uniforms: np.ndarray          # [n][k+1] (verify) or [n][k] (vat) float32
    hard_tokens: Optional[np.ndarray] = None  # vat: [n][k] int32, the target's sampled tokens

    @property
    def n(self) -> int:
        return self.tokens.shape[0]


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(v) for v in key])))


def _as_values(stored: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(stored) if stored.dtype == np.uint16 else stored


def _one_sequence(cfg: Config, b: int, target_out, draft_out, tokens_out, u_out, i: int, hard_out=None) -> None:
    rows_t = cfg.target_rows_per_seq
    z = _rng(cfg.seed_logits, 0, b).standard_normal((rows_t, cfg.V), dtype=np.float32)
    t = (np.float32(cfg.sigma_t) * z).astype(np.float32)
    t_st = round_to_bf16_bits(t) if cfg.dtype == "bf16" else t
    target_out[i] = t_st
    d_st = None
    if not cfg.onehot:
        zd = _rng(cfg.seed_logits, 1, b).standard_normal((cfg.k, cfg.V), dtype=np.float32)
        d = (t[: cfg.k] + np.float32(cfg.sigma_d) * zd).astype(np.float32)
        d_st = round_to_bf16_bits(d) if cfg.dtype == "bf16" else d
        if draft_out is not None:
            draft_out[i] = d_st
    rx = _rng(cfg.seed_draft, b)
    if cfg.draft_mode == "sample":
        # Exponential race (Gumbel-max): argmax_y d(y)/T - log E(y), E ~ Exp(1),
        # picks y with probability proportional to exp(d(y)/T).
        dv = _as_values(d_st).astype(np.float64)
        e = rx.standard_exponential((cfg.k, cfg.V))
        tokens_out[i] = np.argmax(dv / cfg.T - np.log(e), axis=1)
    elif cfg.draft_mode == "argmax":
        tokens_out[i] = np.argmax(_as_values(d_st), axis=1)
    elif cfg.draft_mode == "ngram":
        hit = rx.random(cfg.k) < cfg.ngram_hit
        other = rx.integers(0, cfg.V, size=cfg.k)
        best = np.argmax(_as_values(t_st)[: cfg.k], axis=1)
        tokens_out[i] = np.where(hit, best, other)
    else:
        raise ValueError(cfg.draft_mode)
    u_out[i] = _rng(cfg.seed_u, b).random(cfg.n_uniforms, dtype=np.float32)
    if hard_out is not None:
        # the target's own sample at each position (exponential race at T)
        tv = _as_values(t_st).astype(np.float64)[: cfg.k]
        e = _rng(cfg.seed_draft + 1, b).standard_exponential((cfg.k, cfg.V))
        hard_out[i] = np.argmax(tv / cfg.T - np.log(e), axis=1)


def generate(cfg: Config, lo: int = 0, hi: Optional[int] = None, workers: Optional[int] = None,
             with_draft: bool = True) -> Workload:
    """Generate sequences [lo, hi) of ``cfg`` (all of them by default)."""
    hi = cfg.B if hi is None else hi
    assert 0 <= lo <= hi <= cfg.B
    n = hi - lo
    st_dtype = np.uint16 if cfg.dtype == "bf16" else np.float32
    target = np.empty((n, cfg.target_rows_per_seq, cfg.V), dtype=st_dtype)
    draft = None
    if with_draft and not cfg.onehot:
        draft = np.empty((n, cfg.k, cfg.V), dtype=st_dtype)
    tokens = np.empty((n, cfg.k), dtype=np.int32)
    u = np.empty((n, cfg.n_uniforms), dtype=np.float32)
    hard = np.empty((n, cfg.k), dtype=np.int32) if (cfg.kind == "vat" and cfg.T > 0) else None
    if workers is None:
        workers = max(1, min(16, os.cpu_count() or 1))
    jobs = [(cfg, lo + i, target, draft, tokens, u, i, hard) for i in range(n)]
    if workers == 1 or n <= 1:
        for j in jobs:
            _one_sequence(*j)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda j: _one_sequence(*j), jobs))
    return Workload(cfg, lo, target, draft, tokens, u, hard)


def generate_on_device(cfg: Config, device, slab: int = 64):
    """Device-side variant for workloads too large to draw on the host (the
    33.6 GB VAT case): the same distributions drawn by torch's generator on
    `device`, seeded per slab of `slab` sequences as (seed_logits, slab index).
    Returns torch tensors (target, draft, tokens, uniforms); a checker copies
    the sequences it samples back to the host and hands the oracle those bytes.
    """
    import torch

    rows_t = cfg.target_rows_per_seq
    st = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    target = torch.empty((cfg.B, rows_t, cfg.V), dtype=st, device=device)
    draft = None if cfg.onehot else torch.empty((cfg.B, cfg.k, cfg.V), dtype=st, device=device)
    tokens = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=device)
    uniforms = torch.empty((cfg.B, cfg.n_uniforms), dtype=torch.float32, device=device)
    for s0 in range(0, cfg.B, slab):
        s1 = min(cfg.B, s0 + slab)
        g = torch.Generator(device=device)
        g.manual_seed(int(cfg.seed_logits) * 1_000_003 + s0 // slab)
        t = cfg.sigma_t * torch.randn((s1 - s0, rows_t, cfg.V), generator=g, device=device, dtype=torch.float32)
        target[s0:s1] = t.to(st)
        if draft is not None:
            d = t[:, : cfg.k] + cfg.sigma_d * torch.randn((s1 - s0, cfg.k, cfg.V), generator=g, device=device,
                                                           dtype=torch.float32)
            draft[s0:s1] = d.to(st)
            dv = draft[s0:s1].float()
            if cfg.draft_mode == "sample":
                # fp64 draws: an Exp(1) draw of exactly 0 (which would always win
                # the race) has probability 2^-53 instead of 2^-24.
                e = torch.empty(dv.shape, dtype=torch.float64, device=device).exponential_(generator=g)
                tokens[s0:s1] = torch.argmax(dv.double() / cfg.T - torch.log(e), dim=2).to(torch.int32)
                del e
            elif cfg.draft_mode == "argmax":
                tokens[s0:s1] = torch.argmax(dv, dim=2).to(torch.int32)
            else:
                raise ValueError(cfg.draft_mode)
            del d, dv
        else:
            raise ValueError("device generation covers draft-logit workloads only")
        uniforms[s0:s1] = torch.rand((s1 - s0, cfg.n_uniforms), generator=g, device=device, dtype=torch.float32)
        del t
    return target, draft, tokens, uniforms


def hard_tokens_on_device(cfg: Config, target, device, slab: int = 64):
    """The target's own sample at each position of device-generated VAT
    blocks (exponential race at T over the stored logits), drawn by torch's
    generator per slab of `slab` blocks."""
    import torch

    hard = torch.empty((cfg.B, cfg.k), dtype=torch.int32, device=device)
    for s0 in range(0, cfg.B, slab):
        s1 = min(cfg.B, s0 + slab)
        g = torch.Generator(device=device)
        g.manual_seed(int(cfg.seed_logits) * 1_000_003 + 500_000 + s0 // slab)
        tv = target[s0:s1, : cfg.k].double()
        e = torch.empty(tv.shape, dtype=torch.float64, device=device).exponential_(generator=g)
        hard[s0:s1] = torch.argmax(tv / cfg.T - torch.log(e), dim=2).to(torch.int32)
        del tv, e
    return hard


def to_device(wl: Workload, device):
    """Copies a host workload to `device` as torch tensors (bf16 bits become
    torch.bfloat16).  Returns (target, draft or None, tokens, uniforms)."""
    import torch

    def up(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(a).to(device)

    return up(wl.target), up(wl.draft), up(wl.tokens), up(wl.uniforms)


@dataclasses.dataclass(frozen=True)
class LmHeadConfig:
    name: str
    B: int
    k: int
    V: int
    D: int
    plant: float = 8.0   # margin planted for the intended token of each position
    hit: float = 0.9     # probability that a draft token is the planted token
    seed: int = 11
    T: float = 0.0       # temperature (0: greedy workloads)
    draft_noise: float = 0.3         # draft hidden state = target's + draft_noise * N(0, I)
    draft_weight_noise: float = 0.0  # > 0: the draft's own output layer, W (1 + noise N(0,1))

    @property
    def rows(self) -> int:
        return self.B * (self.k + 1)

    def flops(self) -> int:
        """Multiply-adds of the logits, counted as 2 flops each."""
        return 2 * self.rows * self.V * self.D

    def scaled(self, **changes) -> "LmHeadConfig":
        return dataclasses.replace(self, **changes)


LM_CONFIGS = {
    "lmhead_tiny": LmHeadConfig("lmhead_tiny", 6, 4, 1000, 128, hit=0.8),
    "lmhead_selfdraft": LmHeadConfig("lmhead_selfdraft", 128, 5, 151936, 4096, hit=0.95),
    "lmhead_grpo": LmHeadConfig("lmhead_grpo", 320, 7, 151936, 4096, hit=0.9),
    "lmhead_sample_tiny": LmHeadConfig("lmhead_sample_tiny", 6, 4, 1000, 128, hit=0.8, T=1.0),
    "lmhead_sample_selfdraft": LmHeadConfig("lmhead_sample_selfdraft", 128, 5, 151936, 4096, plant=14.0,
                                            hit=0.95, T=1.0),
    "lmhead_sample_grpo": LmHeadConfig("lmhead_sample_grpo", 320, 7, 151936, 4096, plant=14.0, hit=0.9, T=0.6),
}

_W_SLAB = 4096  # weight rows drawn per generator stream


@dataclasses.dataclass
class LmHeadWorkload:
    config: LmHeadConfig
    hidden: np.ndarray    # [B][k+1][D] uint16 (bf16 bits)
    weight: np.ndarray    # [V][D] uint16
    tokens: np.ndarray    # [B][k] int32
    planted: np.ndarray   # [B][k+1] int32: the token each position was planted for


def lm_head_weight(cfg: LmHeadConfig, workers: Optional[int] = None) -> np.ndarray:
    """W [V][D] as bf16 bits; rows drawn in slabs of 4096, one stream each."""
    w = np.empty((cfg.V, cfg.D), dtype=np.uint16)
    scale = np.float32(1.0 / np.sqrt(cfg.D))

    def slab(s0):
        s1 = min(cfg.V, s0 + _W_SLAB)
        z = _rng(cfg.seed, 2, s0 // _W_SLAB).standard_normal((s1 - s0, cfg.D), dtype=np.float32)
        w[s0:s1] = round_to_bf16_bits(z * scale)

    starts = list(range(0, cfg.V, _W_SLAB))
    if workers is None:
        workers = max(1, min(16, os.cpu_count() or 1))
    if workers == 1 or len(starts) == 1:
        for s0 in starts:
            slab(s0)
    else:
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(slab, starts))
    return w


def generate_lm_head(cfg: LmHeadConfig, weight: Optional[np.ndarray] = None) -> LmHeadWorkload:
    """All B sequences of ``cfg``; sequence b draws from its own streams."""
    w = lm_head_weight(cfg) if weight is None else weight
    assert w.shape == (cfg.V, cfg.D) and w.dtype == np.uint16
    hidden = np.empty((cfg.B, cfg.k + 1, cfg.D), dtype=np.uint16)
    tokens = np.empty((cfg.B, cfg.k), dtype=np.int32)
    planted = np.empty((cfg.B, cfg.k + 1), dtype=np.int32)
    for b in range(cfg.B):
        r = _rng(cfg.seed, 0, b)
        t = r.integers(0, cfg.V, size=cfg.k + 1)
        z = r.standard_normal((cfg.k + 1, cfg.D), dtype=np.float32)
        hidden[b] = round_to_bf16_bits(z + np.float32(cfg.plant) * bf16_bits_to_f32(w[t]))
        planted[b] = t
        rx = _rng(cfg.seed, 1, b)
        hit = rx.random(cfg.k) < cfg.hit
        other = rx.integers(0, cfg.V, size=cfg.k)
        tokens[b] = np.where(hit, t[: cfg.k], other)
    return LmHeadWorkload(cfg, hidden, w, tokens, planted)


def lm_head_to_device(wl: LmHeadWorkload, device):
    """(hidden bf16, weight bf16, tokens int32) as torch tensors on `device`."""
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    return bf(wl.hidden), bf(wl.weight), torch.from_numpy(np.ascontiguousarray(wl.tokens)).to(device)


@dataclasses.dataclass
class LmHeadSampleWorkload:
    config: LmHeadConfig
    target_hidden: np.ndarray   # [B][k+1][D] uint16
    target_weight: np.ndarray   # [V][D] uint16
    draft_hidden: np.ndarray    # [B][k][D] uint16
    draft_weight: np.ndarray    # [V][D] uint16 (the target's array when shared)
    tokens: np.ndarray          # [B][k] int32
    uniforms: np.ndarray        # [B][k+1] float32
    planted: np.ndarray         # [B][k+1] int32


def generate_lm_head_sample(cfg: LmHeadConfig, weight: Optional[np.ndarray] = None) -> LmHeadSampleWorkload:
    """Target side as generate_lm_head; draft hidden states, the draft's
    output layer and the uniforms from streams of their own."""
    base = generate_lm_head(cfg, weight)
    w = base.weight
    if cfg.draft_weight_noise > 0.0:
        z = _rng(cfg.seed, 5).standard_normal(w.shape, dtype=np.float32)
        wd = round_to_bf16_bits(bf16_bits_to_f32(w) * (np.float32(1.0) + np.float32(cfg.draft_weight_noise) * z))
    else:
        wd = w
    hd = np.empty((cfg.B, cfg.k, cfg.D), dtype=np.uint16)
    u = np.empty((cfg.B, cfg.k + 1), dtype=np.float32)
    for b in range(cfg.B):
        z = _rng(cfg.seed, 3, b).standard_normal((cfg.k, cfg.D), dtype=np.float32)
        hd[b] = round_to_bf16_bits(bf16_bits_to_f32(base.hidden[b, : cfg.k]) + np.float32(cfg.draft_noise) * z)
        u[b] = _rng(cfg.seed, 4, b).random(cfg.k + 1, dtype=np.float32)
    return LmHeadSampleWorkload(cfg, base.hidden, w, hd, wd, base.tokens, u, base.planted)


def lm_head_sample_to_device(wl: LmHeadSampleWorkload, device):
    """(target_hidden, target_weight, draft_hidden, draft_weight, tokens,
    uniforms) on `device`; a shared output layer is uploaded once."""
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    th, tw = bf(wl.target_hidden), bf(wl.target_weight)
    dw = tw if wl.draft_weight is wl.target_weight else bf(wl.draft_weight)
    return (th, tw, bf(wl.draft_hidden), dw, torch.from_numpy(np.ascontiguousarray(wl.tokens)).to(device),
            torch.from_numpy(np.ascontiguousarray(wl.uniforms)).to(device))
