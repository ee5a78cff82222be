"""Statistical pins for the oracle's full verify path (Philox uniforms included).

* E[tokens per pass] = (1 - alpha^(gamma+1)) / (1 - alpha) when every position
  has the same (p, q): Monte Carlo mean within 4 standard errors, the variance
  taken from the exact truncated-geometric law.
* Emitted tokens at each emitted position are distributed as the target's
  warped distribution p' (chi-square goodness of fit on a tiny vocabulary).
* A planted mistake (the ratio test uses an untempered q while the drafts
  came from the tempered q') fails the chi-square test.
"""

import json
import os

import numpy as np
import pytest
from scipy.stats import chisquare

import oracle
from oracle import spec_verify_from_logits, warp_logits, warp_probs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def expected_tokens(alpha, gamma):
    return (1 - alpha ** (gamma + 1)) / (1 - alpha)


def test_closed_form_reproduces_page_values():
    with open(os.path.join(GOLDEN, "expected_tokens.json")) as f:
        g = json.load(f)
    for v in g["values"]:
        assert abs(expected_tokens(v["alpha"], v["gamma"]) - v["value"]) <= v["tol"], v
    for v in g["excluded_page_values"]:
        assert abs(expected_tokens(v["alpha"], v["gamma"]) - v["formula"]) < 0.005, v


def sample_drafts(qprime, rng):
    """Harness-side draft sampling from q' (any generator will do; the verify
    step's own uniforms come from Philox purpose 0)."""
    B, gamma, V = qprime.shape
    c = np.cumsum(qprime, axis=-1)
    u = rng.random((B, gamma, 1))
    return np.minimum((c <= u * c[..., -1:]).sum(-1), V - 1)


def make_case(B, gamma, V, T, top_p, seed, same_every_position=False):
    rng = np.random.default_rng(seed)
    shape = (1, 1, V) if same_every_position else (1, gamma + 1, V)
    ell = np.broadcast_to(rng.standard_normal(shape) * 1.5, (B, gamma + 1, V)).copy()
    qlog = ell[:, :gamma] + rng.standard_normal((1, gamma, V)) * 0.8
    if same_every_position:
        qlog = np.broadcast_to(qlog[:, :1], (B, gamma, V))
    qlog = np.broadcast_to(qlog, (B, gamma, V))
    q = np.exp(qlog - qlog.max(-1, keepdims=True))
    q = q / q.sum(-1, keepdims=True)
    qprime = np.stack([warp_probs(q[0, i], T, top_p)[0] for i in range(gamma)])
    drafts = sample_drafts(np.broadcast_to(qprime, (B, gamma, V)), rng)
    pprime = np.stack([warp_logits(ell[0, i], T, top_p)[0] for i in range(gamma + 1)])
    return ell, q, drafts, pprime, qprime


@pytest.mark.parametrize("alpha_case,gamma", [(0, 4), (1, 2), (2, 6)])
def test_mc_expected_tokens_per_pass(alpha_case, gamma):
    B, V = 6000, 8
    ell, q, drafts, pprime, qprime = make_case(B, gamma, V, 1.0, 1.0, 40 + alpha_case,
                                               same_every_position=True)
    alpha = np.minimum(pprime[0], qprime[0]).sum()
    res = spec_verify_from_logits(ell, drafts, q, 1.0, 1.0, seed=1000 + alpha_case)
    n = res.n_accepted.astype(np.float64) + 1
    # exact law of n_accepted: alpha^k (1 - alpha) for k < gamma, alpha^gamma at gamma
    k = np.arange(gamma + 1)
    pmf = np.where(k < gamma, alpha ** k * (1 - alpha), alpha ** gamma)
    mean = (pmf * (k + 1)).sum()
    var = (pmf * (k + 1) ** 2).sum() - mean ** 2
    assert abs(mean - expected_tokens(alpha, gamma)) < 1e-12
    assert abs(n.mean() - mean) < 4 * np.sqrt(var / B), (n.mean(), mean, alpha)
    # acceptance frequency at the first position estimates alpha
    acc0 = (res.n_accepted >= 1).mean()
    assert abs(acc0 - alpha) < 4 * np.sqrt(alpha * (1 - alpha) / B)


def chi2_per_position(res, pprime, gamma, V, min_expected=5.0):
    """p-values of the emitted tokens at each position against p'_position."""
    pvals = []
    for pos in range(gamma + 1):
        rows = res.n_accepted >= pos          # token at pos was emitted
        toks = res.emitted[rows, pos]
        if toks.size < 200:
            continue
        expct = pprime[pos] * toks.size
        keep = expct >= min_expected
        obs = np.bincount(toks, minlength=V)
        o = np.append(obs[keep], obs[~keep].sum())
        e = np.append(expct[keep], expct[~keep].sum())
        if e[-1] == 0:
            o, e = o[:-1], e[:-1]
        pvals.append(chisquare(o, e).pvalue)
    return pvals


@pytest.mark.parametrize("T,top_p", [(1.0, 1.0), (0.7, 0.9), (1.3, 0.6)])
def test_chi_square_emitted_tokens_follow_target(T, top_p):
    B, gamma, V = 8000, 3, 8
    ell, q, drafts, pprime, _ = make_case(B, gamma, V, T, top_p, 7)
    res = spec_verify_from_logits(ell, drafts, q, T, top_p, seed=77)
    pvals = chi2_per_position(res, pprime, gamma, V)
    assert len(pvals) >= 2
    assert min(pvals) > 1e-4, pvals


def test_chi_square_detects_temperature_on_p_only(monkeypatch):
    """Plant in the oracle: the ratio test uses the untempered draft q while
    the drafts were sampled from the tempered q' (the draft ran at T, the
    verifier forgot to temper q)."""
    B, gamma, V, T = 8000, 2, 8, 0.5
    ell, q, drafts, pprime, _ = make_case(B, gamma, V, T, 1.0, 8)
    res_ok = spec_verify_from_logits(ell, drafts, q, T, 1.0, seed=5)
    assert min(chi2_per_position(res_ok, pprime, gamma, V)) > 1e-4
    real = oracle.verify.warp_probs
    monkeypatch.setattr(oracle.verify, "warp_probs", lambda qq, TT, tp: real(qq, 1.0, tp))
    res = spec_verify_from_logits(ell, drafts, q, T, 1.0, seed=5)
    pvals = chi2_per_position(res, pprime, gamma, V)
    assert min(pvals) < 1e-6, pvals
