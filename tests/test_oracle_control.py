"""Pins for the oracle's gamma controller and ragged repacking
(oracle/control.py)."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import control

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_expected_tokens_matches_page_values():
    with open(os.path.join(GOLDEN, "expected_tokens.json")) as f:
        g = json.load(f)
    for v in g["values"]:
        assert abs(control.expected_tokens(v["alpha"], v["gamma"]) - v["value"]) <= v["tol"]
    assert control.expected_tokens(1.0, 4) == 5.0
    assert abs(control.expected_tokens(1 - 1e-12, 4) - 5.0) < 1e-9     # the limit
    assert control.expected_tokens(0.0, 7) == 1.0


def test_limiting_cases():
    c = control.GammaController(2, 8, 4, draft_ms_per_token=3.0, target_ms=20.0)
    assert c.optimal_gamma(0.0) == 2             # nothing accepted: least draft time
    free = control.GammaController(2, 8, 4, draft_ms_per_token=0.0, target_ms=20.0)
    for a in (0.1, 0.5, 0.9, 1.0):
        assert free.optimal_gamma(a) == 8        # free drafts: as deep as allowed
    dear = control.GammaController(1, 8, 4, draft_ms_per_token=1e6, target_ms=1.0)
    assert dear.optimal_gamma(0.95) == 1


def test_decision_is_monotone_in_alpha_and_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(40):
        lo = int(rng.integers(0, 4))
        hi = lo + int(rng.integers(0, 12))
        table = np.cumsum(rng.uniform(0.0, 2.0, hi + 1)) + rng.uniform(5, 30)   # grows with gamma
        c = control.GammaController(lo, hi, lo, draft_ms_per_token=float(rng.uniform(0.1, 5)),
                                    target_ms=list(table))
        prev = lo
        for a in np.linspace(0, 1, 41):
            g = c.optimal_gamma(a)
            rates = [control.expected_tokens(a, k) / (k * c.draft_ms + table[k]) for k in range(lo, hi + 1)]
            assert g == lo + int(np.argmax(rates))          # first maximum
            assert g >= prev - 0 or rates[g - lo] == rates[prev - lo]
            prev = g


def test_window_and_warm_up():
    c = control.GammaController(2, 8, 4, 2.0, 20.0)
    for _ in range(4):
        assert c.step(4, 0) == 4                 # fewer than 5 steps: keep gamma
    assert c.step(4, 0) == c.optimal_gamma(1.0)
    assert c.rolling_alpha() == 1.0
    assert c.step(-1, 0) == c.gamma and len(c.window) == 5   # refused rows record nothing
    for _ in range(control.WINDOW):
        c.step(0, 4)
    assert len(c.window) == control.WINDOW and c.rolling_alpha() == 0.0
    assert c.gamma == c.optimal_gamma(0.0)
    c.step(4, 0)
    assert abs(c.rolling_alpha() - 4 / (19 * 4 + 4)) < 1e-15   # the oldest step left the window


def test_page_defaults_pick_a_gamma_per_alpha():
    """The article's calibration (2 ms per draft token, 20 ms per target
    pass): tokens per second of each gamma, checked by hand-written sums."""
    c = control.GammaController()
    for a in (0.6, 0.8, 0.9):
        best = max(range(2, 9), key=lambda g: (sum(a ** k for k in range(g + 1)) / (2 * g + 20), -g))
        assert c.optimal_gamma(a) == best


def test_repack_hand_example():
    n = [2, -1, 0, 4]
    emitted = [[5, 6, 7, -1, -1], [-1] * 5, [9, -1, -1, -1, -1], [1, 2, 3, 4, 8]]
    r = control.repack(n, emitted, [10, 3, 7, 0])
    assert r["tokens"] == [5, 6, 7, 9, 1, 2, 3, 4, 8]
    assert r["offsets"] == [0, 3, 3, 4, 9]
    assert r["committed"] == [13, 3, 8, 5]
    assert r["order"] == [1, 2, 0, 3]            # counts 3, 0, 1, 5
    assert r["bin_offsets"] == [0, 1, 2, 2, 3, 3, 4]   # bins of counts 0 .. 5, then B
    assert r["width"] == 5 and r["waste"] == 4 * 5 - 9


@pytest.mark.parametrize("seed", range(10))
def test_repack_invariants(seed):
    rng = np.random.default_rng(seed)
    B, gamma = int(rng.integers(1, 60)), int(rng.integers(0, 9))
    n = rng.integers(-1, gamma + 1, B)
    emitted = np.full((B, gamma + 1), -1)
    for b in range(B):
        if n[b] >= 0:
            emitted[b, :n[b] + 1] = rng.integers(0, 1000, n[b] + 1)
    committed = rng.integers(0, 5000, B)
    r = control.repack(n, emitted, committed)
    counts = np.where(n >= 0, n + 1, 0)
    assert sorted(r["order"]) == list(range(B))
    oc = counts[r["order"]]
    assert (np.diff(oc) >= 0).all()
    for c in range(gamma + 2):      # stable: ids ascending inside a bin
        ids = np.array(r["order"][r["bin_offsets"][c]:r["bin_offsets"][c + 1]])
        assert (counts[ids] == c).all() and (np.diff(ids) > 0).all()
    assert r["offsets"][-1] == counts.sum() == len(r["tokens"])
    for b in range(B):
        assert r["tokens"][r["offsets"][b]:r["offsets"][b + 1]] == list(emitted[b, :counts[b]])
    assert (np.array(r["committed"]) == committed + counts).all()
    assert r["waste"] == B * counts.max() - counts.sum()
