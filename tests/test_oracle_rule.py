"""Pins for the oracle's acceptance rule (deterministic parts)."""

import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import (accept_test, inverse_cdf, nucleus_mask, spec_verify_from_logits,
                    verify_row, verify_row_greedy, warp_logits, warp_probs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- worked example

def test_worked_example_threshold_and_decisions():
    g = load("worked_example.json")
    pv = g["page_values"]
    ok, m = accept_test(pv["p_blue"], pv["q_blue"], pv["r_accept"])
    assert ok and abs(m - abs(pv["r_accept"] - pv["threshold"])) < 1e-12
    ok, m = accept_test(pv["p_blue"], pv["q_blue"], pv["r_reject"])
    assert not ok and abs(m - abs(pv["r_reject"] - pv["threshold"])) < 1e-12


def test_worked_example_correction_is_green():
    g = load("worked_example.json")
    p, q = np.array(g["p"]), np.array(g["q"])
    blue, green = g["vocab"].index("blue"), g["vocab"].index("green")
    res = oracle.rule.residual(p, q)
    assert np.allclose(res / res.sum(), g["residual_normalised"], atol=1e-15)
    for u in (0.0, 0.3, 0.999999):
        n, tok, _ = verify_row([p, p], [q], [blue], [(0.71, u), (0.5, 0.5)])
        assert (n, tok) == (0, green)
        n, tok, _ = verify_row([p, p], [q], [blue], [(0.42, u), (0.5, 0.5)])
        assert n == 1          # accepted, then a bonus from p at the next slot


# ---------------------------------------------------------------- top-p

def brute_force_nucleus(p, top_p):
    """Among all subsets with mass >= top_p: fewest tokens, then largest mass,
    then lexicographically smallest ids."""
    V = len(p)
    best = None
    for k in range(1, V + 1):
        for S in itertools.combinations(range(V), k):
            mass = sum(p[i] for i in S)
            if mass >= top_p - 1e-15:
                key = (-mass, S)
                if best is None or key < best[0]:
                    best = (key, S)
        if best is not None:
            return set(best[1])
    return set(range(V))


@pytest.mark.parametrize("seed", range(12))
def test_top_p_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(2, 9))
    p = rng.dirichlet(np.full(V, 0.7))
    for top_p in (0.05, 0.3, 0.5, 0.9, 0.97):
        mask, _ = nucleus_mask(p, top_p)
        assert set(np.nonzero(mask)[0]) == brute_force_nucleus(p, top_p)


def test_top_p_ties_by_lower_id_and_full_keep():
    p = np.full(4, 0.25)
    mask, _ = nucleus_mask(p, 0.5)
    assert mask.tolist() == [True, True, False, False]
    mask, m = nucleus_mask(p, 1.0)
    assert mask.all() and not m.uncertain
    mask, _ = nucleus_mask(np.array([0.1, 0.6, 0.3]), 0.6)   # exactly reaching
    assert mask.tolist() == [False, True, False]


def test_top_p_uncertain_tokens():
    """Target rows: a near-tied cut puts the tied tokens in the uncertain set;
    a cut that barely reaches top_p makes the last kept token uncertain; a
    clear cut has none."""
    p = np.array([0.5, 0.2, 0.2 * (1 - 1e-7), 0.1 - 0.2 * (1 - 1e-7) + 0.2])
    p = p / p.sum()
    mask, info = nucleus_mask(p, 0.6, logp_tol=1e-5)   # cut between tokens 1 and 2
    assert mask.tolist() == [True, True, False, False]
    assert info.uncertain == {1, 2} and info.mass > 0
    mask, info = nucleus_mask(p, 0.6, logp_tol=0.0)
    assert not info.uncertain
    mask, info = nucleus_mask(np.array([0.5, 0.3, 0.2]), 0.6, logp_tol=1e-5)
    assert not info.uncertain
    mask, info = nucleus_mask(np.array([0.5, 0.3, 0.2]), 0.8 - 1e-7)   # 0.5 + 0.3 barely reaches
    assert mask.tolist() == [True, True, False] and info.uncertain == {2}
    mask, info = nucleus_mask(np.array([0.5, 0.3, 0.2]), 0.5 + 1e-7)   # 0.5 barely misses
    assert info.uncertain == {1}


def test_uncertain_token_ratio_test_is_a_knife_edge():
    ell = np.log(np.array([0.5, 0.2, 0.2 * (1 - 1e-9), 0.1]))
    p, cut = warp_logits(ell, 1.0, 0.6)
    assert not cut.uncertain              # same logits on both sides: the order is exact
    p, cut = warp_logits(ell, 1.0, 0.6, logit_err=1e-6)
    assert cut.uncertain == {1, 2}
    q = np.full(4, 0.25)
    _, _, mg = verify_row([p, p], [q], [2], [(0.1, 0.5), (0.5, 0.5)], p_cuts=[cut, cut])
    assert mg[0].kind == "accept" and mg[0].flagged and mg[0].slack == np.inf
    _, _, mg = verify_row([p, p], [q], [0], [(0.999, 0.5), (0.5, 0.5)], p_cuts=[cut, cut])
    # a certain token's ratio test widens its slack by ratio x uncertain mass
    assert mg[0].margin == abs(0.999 - p[0] / 0.25)
    assert mg[0].slack >= oracle.MARGIN + p[0] / 0.25 * cut.mass


def test_warp_logits_is_library_softmax():
    rng = np.random.default_rng(3)
    ell = rng.standard_normal(50) * 3
    for T in (1.0, 0.7, 2.5, 0.05):
        p, _ = warp_logits(ell, T, 1.0)
        assert np.allclose(p, softmax(ell / T), rtol=1e-12, atol=1e-300)


def test_warp_probs_is_tempered_draft():
    rng = np.random.default_rng(4)
    q = softmax(rng.standard_normal(40))
    q1, _ = warp_probs(q, 1.0, 1.0)
    assert np.allclose(q1, q / q.sum(), rtol=1e-14)
    for T in (0.7, 1.6):
        qt, _ = warp_probs(q, T, 1.0)
        assert np.allclose(qt, softmax(np.log(q) / T), rtol=1e-12)
    qz = q.copy(); qz[5] = 0.0
    qt, _ = warp_probs(qz, 0.7, 1.0)
    assert qt[5] == 0.0 and abs(qt.sum() - 1) < 1e-14


def test_top_p_then_renormalise():
    ell = np.log(np.array([0.5, 0.3, 0.15, 0.05]))
    p, _ = warp_logits(ell, 1.0, 0.75)
    assert np.allclose(p, [0.5 / 0.8, 0.3 / 0.8, 0, 0], atol=1e-14)


# ---------------------------------------------------------------- ratio test

def test_ratio_test_edges():
    assert accept_test(0.2, 0.1, 0.999)[0]            # p >= q always accepts
    assert not accept_test(0.0, 0.3, 0.0)[0]          # p = 0 never accepts
    assert accept_test(1e-30, 0.0, 0.9)[0]            # q' = 0 accepts iff p' > 0
    assert not accept_test(0.0, 0.0, 0.0)[0]
    assert not accept_test(0.25, 0.5, 0.5)[0]         # r equal to p/q rejects (strict)
    assert accept_test(0.25, 0.5, 0.5 - 2 ** -24)[0]


def test_inverse_cdf_convention():
    w = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert inverse_cdf(w, 0.0)[0] == 1                # zero-mass ids never chosen
    assert inverse_cdf(w, 0.25 - 2 ** -24)[0] == 1
    assert inverse_cdf(w, 0.25)[0] == 3               # strict '>' at a boundary
    assert inverse_cdf(w, 0.75)[0] == 4
    assert inverse_cdf(w, 1 - 2 ** -24)[0] == 4
    assert inverse_cdf(w * 1e-3, 0.6)[0] == np.searchsorted(np.cumsum(w), 0.6, side="right")


def test_residual_zero_falls_back_to_p():
    p = np.array([0.5, 0.5, 0.0])
    n, tok, _ = verify_row([p, p], [p.copy()], [2], [(0.0, 0.7), (0.0, 0.0)])
    assert n == 0 and tok == 1                          # sampled from p, u = 0.7


# ---------------------------------------------------------------- emission law by quadrature

def quadrature_law(p, q, N=2000):
    """P(emit t at position 0) and P(accept) for gamma = 1, integrating the
    oracle's decisions over midpoint grids of r and u (drafts weighted by q)."""
    V = len(p)
    grid = (np.arange(N) + 0.5) / N
    law = np.zeros(V)
    p_acc = 0.0
    for x in range(V):
        if q[x] == 0:
            continue
        acc = np.array([verify_row([p, p], [q], [x], [(r, 0.5), (0.5, 0.5)])[0] == 1
                        for r in grid])
        pa = acc.mean()
        p_acc += q[x] * pa
        law[x] += q[x] * pa
        if pa < 1:
            r_rej = grid[np.argmin(acc)]
            toks = [verify_row([p, p], [q], [x], [(r_rej, u), (0.5, 0.5)])[1] for u in grid]
            law += q[x] * (1 - pa) * np.bincount(toks, minlength=V) / N
    return law, p_acc


@pytest.mark.parametrize("case", range(4))
def test_emission_law_equals_target_by_quadrature(case):
    rng = np.random.default_rng(100 + case)
    V = 5
    p = rng.dirichlet(np.ones(V))
    q = rng.dirichlet(np.ones(V))
    if case == 3:                        # warped distributions (T and top-p on both)
        p, _ = warp_logits(np.log(p), 0.7, 0.9)
        q, _ = warp_probs(q, 0.7, 0.9)
    law, p_acc = quadrature_law(p, q)
    assert np.allclose(law, p, atol=3e-3)
    # alpha = sum min(p, q) = 1 - TV(p, q)
    alpha = np.minimum(p, q).sum()
    assert abs(alpha - (1 - 0.5 * np.abs(p - q).sum())) < 1e-14
    assert abs(p_acc - alpha) < 2e-3


def test_quadrature_detects_a_planted_residual_mistake(monkeypatch):
    """Plant 'resample from p instead of the residual' in the oracle: the
    emission law must move away from p."""
    rng = np.random.default_rng(7)
    p, q = rng.dirichlet(np.ones(5)), rng.dirichlet(np.ones(5))
    monkeypatch.setattr(oracle.rule, "residual", lambda p_, q_: p_)
    law, _ = quadrature_law(p, q, N=500)
    assert np.abs(law - p).max() > 0.02


# ---------------------------------------------------------------- greedy branch

def test_greedy_is_the_zero_temperature_limit():
    rng = np.random.default_rng(9)
    B, gamma, V = 40, 4, 30
    # logits on a 0.1-spaced grid, so at T = 1e-3 every runner-up is e^-100 down
    ell = np.stack([np.stack([rng.permutation(V) * 0.1 for _ in range(gamma + 1)])
                    for _ in range(B)])
    # the draft agrees with the target's top token about half the time
    qlog = np.where(rng.random((B, gamma, 1)) < 0.5, ell[:, :gamma],
                    np.stack([np.stack([rng.permutation(V) * 0.1 for _ in range(gamma)])
                              for _ in range(B)]))
    q = np.exp(qlog - qlog.max(-1, keepdims=True)); q /= q.sum(-1, keepdims=True)
    draft = q.argmax(-1)                       # a greedy draft proposes argmax q
    g = spec_verify_from_logits(ell, draft, q, 0.0, 1.0, seed=1)
    s = spec_verify_from_logits(ell, draft, q, 1e-3, 1.0, seed=1)
    assert np.array_equal(g.n_accepted, s.n_accepted)
    assert np.array_equal(g.emitted, s.emitted)
    assert 0 < np.mean(g.n_accepted) < gamma   # both accepts and rejects occur


def test_greedy_ties_take_lowest_index():
    ell = np.array([[1.0, 3.0, 3.0], [0.0, 0.0, 0.0]])
    n, tok, m = verify_row_greedy(ell, [2])
    assert (n, tok) == (0, 1) and m[0].margin == 0.0
    # reading the same logits, an exact tie is no knife edge: both sides
    # take the lowest index
    assert not m[0].flagged
    n, tok, m = verify_row_greedy(ell, [2], logit_err=1e-3)
    assert m[0].flagged and m[0].band == {1, 2}


def test_bad_token_row_is_rejected_whole():
    ell = np.zeros((2, 3, 6))
    q = np.full((2, 2, 6), 1 / 6)
    r = spec_verify_from_logits(ell, [[1, 6], [0, 1]], q, 1.0, 1.0, seed=0)
    assert r.n_accepted[0] == -1 and (r.emitted[0] == -1).all()
    assert r.n_accepted[1] >= 0
    r = spec_verify_from_logits(ell, [[-1, 0], [0, 1]], None, 0.0, 1.0, seed=0)
    assert r.n_accepted[0] == -1


def test_gamma_zero_is_a_plain_sample():
    ell = np.log(np.array([[[0.1, 0.2, 0.7]]]))
    r = spec_verify_from_logits(ell, np.zeros((1, 0), dtype=int), np.zeros((1, 0, 3)),
                                1.0, 1.0, seed=0)
    u = oracle.row_uniforms(0, 0, 0)[1]
    assert r.n_accepted[0] == 0
    assert r.emitted[0, 0] == np.searchsorted(np.cumsum([0.1, 0.2, 0.7]), u * 1.0, side="right")


def test_scalar_validation():
    ell = np.zeros((1, 2, 3)); q = np.full((1, 1, 3), 1 / 3)
    for T, tp in ((-1.0, 1.0), (1.0, 0.0), (1.0, 1.5), (float("nan"), 1.0)):
        with pytest.raises(ValueError):
            spec_verify_from_logits(ell, [[0]], q, T, tp, seed=0)
