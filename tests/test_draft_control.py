"""Acceptance telemetry on the host: the draft-length controller of the
EfficientRollout write-up (section "四、自适应草稿长度"), checked against the
rule as that section states it, restated here in plain Python: a fixed set of
lengths, start at the shortest, move up after two consecutive steps whose
block efficiency is near the length's limit, down after two consecutive steps
that are too low, one noisy step moves nothing."""
import ctypes
import os

import numpy as np
import pytest

import speculative_decoding_verification_amd as sv

# A host-only build of the controller (the sanitizer run sets this).
_LIB = ctypes.CDLL(os.environ["SV_CONTROL_LIB"]) if os.environ.get("SV_CONTROL_LIB") else None


def controller(*args, **kw):
    return sv.DraftLengthController(*args, lib=_LIB, **kw)


def hist_for(k, lengths):
    """k+4 counts of the given accepted lengths."""
    h = np.zeros(k + 4, np.int32)
    for L in lengths:
        h[L] += 1
    return h


def hist_geometric(k, alpha, n=100000):
    """Expected counts (rounded) when each draft is kept with probability alpha."""
    p = np.array([alpha ** j * (1 - alpha) for j in range(k)] + [alpha ** k])
    h = np.zeros(k + 4, np.int32)
    h[: k + 1] = np.round(p * n).astype(np.int32)
    return h


class PlainRule:
    def __init__(self, choices, up, down, patience):
        self.choices, self.up, self.down, self.patience = list(choices), up, down, patience
        self.i, self.hi, self.lo = 0, 0, 0

    def step(self, hist):
        k = self.choices[self.i]
        counts = np.asarray(hist[: k + 1], np.float64)
        if counts.sum() == 0:
            return k
        eff = float((counts * np.arange(1, k + 2)).sum() / counts.sum())
        if eff >= self.up * (k + 1):
            self.hi, self.lo = self.hi + 1, 0
        elif eff <= self.down * (k + 1):
            self.hi, self.lo = 0, self.lo + 1
        else:
            self.hi = self.lo = 0
        if self.hi >= self.patience and self.i + 1 < len(self.choices):
            self.i, self.hi, self.lo = self.i + 1, 0, 0
        elif self.lo >= self.patience and self.i > 0:
            self.i, self.hi, self.lo = self.i - 1, 0, 0
        return self.choices[self.i]


def test_starts_short_and_climbs_after_two_good_steps():
    c = controller()
    assert c.k == 5
    good = hist_for(5, [5] * 9 + [4])      # efficiency 5.9 of 6
    assert c.update(good) == 5             # one step moves nothing
    assert c.update(good) == 7
    assert c.efficiency == pytest.approx(5.9)
    g7 = hist_for(7, [7] * 10)
    assert c.update(g7) == 7 and c.update(g7) == 9
    g9 = hist_for(9, [9] * 10)
    assert c.update(g9) == 9 and c.update(g9) == 11
    g11 = hist_for(11, [11] * 10)
    assert c.update(g11) == 11 and c.update(g11) == 11   # the longest choice stays


def test_one_noisy_step_moves_nothing_and_low_steps_step_down():
    c = controller()
    good = hist_for(5, [5] * 10)
    bad = hist_for(5, [0] * 10)            # efficiency 1 of 6
    c.update(good)
    assert c.update(bad) == 5              # the good streak is broken
    assert c.update(good) == 5
    assert c.update(good) == 7
    b7 = hist_for(7, [1] * 10)             # 2 of 8
    assert c.update(b7) == 7
    assert c.update(b7) == 5
    assert c.update(bad) == 5 and c.update(bad) == 5   # the shortest choice stays


def test_efficiency_of_geometric_acceptance():
    """Kept with probability alpha: E[tokens per cycle] = sum_{j=0..k} alpha^j."""
    for alpha in (0.5, 0.9, 0.96):
        c = controller()
        c.update(hist_geometric(5, alpha))
        assert c.efficiency == pytest.approx(sum(alpha ** j for j in range(6)), rel=1e-4)


def test_invalid_and_timed_out_sequences_are_not_counted():
    c = controller()
    h = hist_for(5, [5] * 4)
    h[6] = 100   # invalid tokens
    h[7] = 7     # timed out
    c.update(h)
    assert c.efficiency == pytest.approx(6.0)
    assert c.update(np.zeros(9, np.int32)) == 5     # no valid sequence: no change


def test_matches_the_plain_rule_on_random_runs():
    rng = np.random.default_rng(60)
    for trial in range(40):
        up = float(rng.uniform(0.6, 0.95))
        down = float(rng.uniform(0.1, up - 0.05))
        pat = int(rng.integers(1, 4))
        choices = sorted(rng.choice(np.arange(2, 20), size=int(rng.integers(1, 6)), replace=False).tolist())
        c = controller(choices, up, down, pat)
        plain = PlainRule(choices, np.float32(up), np.float32(down), pat)
        for step in range(60):
            k = c.k
            alpha = float(rng.uniform(0.0, 1.0))
            lengths = np.minimum(rng.geometric(1 - alpha, size=50) - 1, k) if alpha < 1 else np.full(50, k)
            h = hist_for(k, lengths.tolist())
            assert c.update(h) == plain.step(h), (trial, step)


def test_bad_arguments():
    with pytest.raises(sv.SVError):
        controller((5, 5, 7))            # not increasing
    with pytest.raises(sv.SVError):
        controller((5, 7), up_frac=0.4, down_frac=0.5)
    with pytest.raises(sv.SVError):
        controller((5, 70))              # beyond 64
    with pytest.raises(sv.SVError):
        controller(tuple(range(1, 10)))  # more than 8 choices
    c = controller()
    with pytest.raises(ValueError):
        c.update([1, 2])
