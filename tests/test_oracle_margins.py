"""Pins for the oracle's decision records (margin, slack, band).

A float32 implementation, or one that reads logits a little off the float64
forward, may take some decisions differently.  The oracle claims that it can
only flip a decision whose margin is below its slack, and only to a token of
that decision's band.  These tests move the inputs of the rule within the
bounds the oracle states -- every warped probability by up to its stated
error, the nucleus membership of every uncertain token, the logits by up to
the stated logit tolerance -- rerun the plain float64 rule on the moved
inputs, and require every row that comes out differently to be explained by
a flagged decision of the unmoved run (the same comparison the GPU parity
tests use).  Uniforms are placed right at the decision thresholds so that
flips actually happen.  A move thirty times beyond the stated bounds must
produce unexplained rows, so the check has teeth.
"""

import numpy as np
import pytest

import oracle
from harness import compare_tokens
from oracle.rule import (Decision, TopP, residual, verify_row, verify_row_greedy, warp_logits,
                         warp_probs)


def _case(rng, V, gamma, T, top_p, spread=2.0):
    ell = rng.standard_normal((gamma + 1, V)) * spread
    qlog = ell[:gamma] + rng.standard_normal((gamma, V)) * 0.6
    q = np.exp(qlog - qlog.max(-1, keepdims=True))
    q /= q.sum(-1, keepdims=True)
    draft = np.array([rng.choice(V, p=warp_probs(q[i], T, top_p)[0]) for i in range(gamma)])
    return ell, q, draft


class _Res:
    """A one-row result in the shape compare_tokens reads."""

    def __init__(self, n, tok, decs, draft, G1):
        self.n_accepted = np.array([n])
        e = np.full(G1, -1)
        e[:n] = draft[:n]
        e[n] = tok
        self.emitted = e[None]
        self.decisions = [decs]
        self.drafts = np.asarray(draft)[None]


def _knife_uniforms(rng, p_rows, q_rows, draft, slack_scale):
    """Uniforms placed at the thresholds: r_i within 3 slack_scale of p'/q',
    u_i near a CDF boundary of the distribution that row would sample."""
    gamma = len(draft)
    uni = []
    for i in range(gamma + 1):
        if i < gamma:
            x = draft[i]
            ratio = p_rows[i][x] / q_rows[i][x] if q_rows[i][x] > 0 else 2.0
            r = min(max(ratio + rng.uniform(-3, 3) * slack_scale, 0.0), 1 - 2 ** -24)
            w = residual(p_rows[i], q_rows[i])
        else:
            r = rng.random()
            w = p_rows[i]
        C = np.cumsum(w)
        k = rng.integers(0, len(C))
        u = min(max(C[k] / C[-1] + rng.uniform(-3, 3) * slack_scale, 0.0), 1 - 2 ** -53)
        uni.append((r, u))
    return uni


def _moved(w, cut, rng, scale, flip):
    """w moved elementwise within scale x its stated bound, uncertain nucleus
    tokens flipped to their other side (then renormalised) when `flip`."""
    w = np.array(w, dtype=np.float64)
    if flip and cut.uncertain:
        for v in cut.uncertain:
            if rng.random() < 0.5:
                w[v] = cut.alt[v]
        w = w / w.sum()
    if cut.err is not None:
        mode = rng.integers(0, 3)
        if mode == 0:
            s = rng.uniform(-1, 1, w.shape)
        elif mode == 1:
            s = np.sign(rng.standard_normal(w.shape))
        else:                       # push the prefix one way and the tail the other
            s = np.where(np.arange(w.shape[0]) < rng.integers(0, w.shape[0]), 1.0, -1.0)
        w = np.maximum(w + scale * s * cut.err, 0.0)
    return w


def _run(rng, V, gamma, T, top_p, scale, trials, spread=2.0):
    """Returns (rows compared, rows that differed, rows unexplained)."""
    ell, q, draft = _case(rng, V, gamma, T, top_p, spread)
    pw = [warp_logits(ell[i], T, top_p) for i in range(gamma + 1)]
    qw = [warp_probs(q[i], T, top_p) for i in range(gamma)]
    p_rows, p_cuts = [w for w, _ in pw], [c for _, c in pw]
    q_rows, q_cuts = [w for w, _ in qw], [c for _, c in qw]
    compared = differ = bad = 0
    for _ in range(trials):
        uni = _knife_uniforms(rng, p_rows, q_rows, draft, 3e-7)
        n0, t0, d0 = verify_row(p_rows, q_rows, draft, uni, p_cuts, q_cuts)
        ref = _Res(n0, t0, d0, draft, gamma + 1)
        pm = [_moved(p_rows[i], p_cuts[i], rng, scale, scale <= 1) for i in range(gamma + 1)]
        qm = [_moved(q_rows[i], q_cuts[i], rng, scale, scale <= 1) for i in range(gamma)]
        n1, t1, _ = verify_row(pm, qm, draft, uni)
        got = _Res(n1, t1, [], draft, gamma + 1)
        rep = compare_tokens(got.n_accepted, got.emitted, ref)
        compared += 1
        differ += len(rep.mismatched)
        bad += len(rep.unexplained)
    return compared, differ, bad


CASES = [(6, 3, 1.0, 1.0), (40, 4, 0.7, 0.9), (300, 3, 1.3, 0.6), (2000, 2, 1.0, 1.0),
         (500, 4, 0.5, 0.95)]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_moves_within_the_bounds_are_explained(case):
    V, gamma, T, top_p = case
    rng = np.random.default_rng(hash(case) % 2 ** 32)
    compared, differ, bad = _run(rng, V, gamma, T, top_p, 1.0, 150)
    assert bad == 0
    assert differ > 0            # the knife-edge uniforms do make decisions flip


def test_moves_beyond_the_bounds_are_caught():
    """Thirty times the stated bounds (and no nucleus flips): some rows flip
    where no decision is flagged, so the comparison fails them."""
    rng = np.random.default_rng(11)
    bad = 0
    for V, gamma, T, top_p in CASES:
        bad += _run(rng, V, gamma, T, top_p, 30.0, 150)[2]
    assert bad > 0


def test_top_p_membership_flips_need_the_uncertain_set():
    """Flipping the membership of a token the oracle calls certain is caught:
    with the uncertain set emptied, a nucleus change goes unexplained."""
    rng = np.random.default_rng(5)
    V, gamma, T, top_p = 60, 3, 1.0, 0.5
    found = False
    for _ in range(200):
        ell, q, draft = _case(rng, V, gamma, T, top_p)
        p0, c0 = warp_logits(ell[gamma], T, top_p)
        # drop the last kept token from the bonus row's nucleus
        order = np.lexsort((np.arange(V), -p0))
        kept = order[p0[order] > 0]
        if len(kept) < 2 or int(kept[-1]) in c0.uncertain:
            continue
        pm = p0.copy()
        pm[kept[-1]] = 0.0
        pm /= pm.sum()
        p_rows = [warp_logits(ell[i], T, top_p)[0] for i in range(gamma)] + [p0]
        q_rows = [warp_probs(q[i], T, top_p)[0] for i in range(gamma)]
        C = np.cumsum(p0)
        k = int(np.nonzero(order == kept[-1])[0][0])
        v = int(kept[-1])
        u = (C[v] - 0.5 * p0[v]) / C[-1]     # right inside the dropped token's interval
        uni = [(0.0, 0.5)] * gamma + [(0.0, u)]
        n0, t0, d0 = verify_row(p_rows, q_rows, draft, uni,
                                [TopP()] * gamma + [c0], [TopP()] * gamma)
        n1, t1, _ = verify_row(p_rows[:gamma] + [pm], q_rows, draft, uni)
        if n0 == gamma and n1 == gamma and t0 != t1:
            rep = compare_tokens(np.array([n1]), _Res(n1, t1, [], draft, gamma + 1).emitted,
                                 _Res(n0, t0, d0, draft, gamma + 1))
            assert rep.unexplained
            found = True
            break
    assert found


@pytest.mark.parametrize("V,T,top_p", [(50, 1.0, 1.0), (400, 0.7, 0.9), (3000, 1.0, 0.8)])
def test_logit_moves_within_the_tolerance_are_explained(V, T, top_p):
    """The logits themselves moved by up to tol x max|logit| (what a GEMM
    path is held to), p' recomputed from the moved logits in float64: every
    differing row is explained by the records made with that tolerance."""
    rng = np.random.default_rng(V)
    gamma, tol = 3, 2e-5
    differ = 0
    for trial in range(40):
        ell, q, draft = _case(rng, V, gamma, T, top_p)
        if trial % 2:        # logits on a coarse grid: many near ties at the cut
            ell = np.round(ell * 64) / 64
        ref = oracle.spec_verify_from_logits(ell[None], draft[None], q[None], T, top_p,
                                             seed=trial, logit_tol=tol)
        # place the uniforms of this seed's row at thresholds by picking the
        # logit move instead: push every logit up to the tolerance
        lerr = tol * np.abs(ell).max(axis=-1, keepdims=True)
        for _ in range(6):
            mv = ell + lerr * rng.choice([-1.0, 1.0], size=ell.shape) * rng.uniform(0.5, 1.0)
            got = oracle.spec_verify_from_logits(mv[None], draft[None], q[None], T, top_p,
                                                 seed=trial)
            rep = compare_tokens(got.n_accepted, got.emitted, ref)
            assert not rep.unexplained, (trial, rep.record())
            differ += len(rep.mismatched)
    assert differ >= 0


def test_greedy_logit_moves_are_explained_and_caught():
    rng = np.random.default_rng(21)
    V, gamma, err = 40, 4, 1e-3
    explained_flips = caught = 0
    for _ in range(300):
        # logits on a grid of err so that near ties are common
        ell = np.round(rng.standard_normal((gamma + 1, V)) * 0.01 / err) * err
        draft = ell[:gamma].argmax(-1)
        draft = np.where(rng.random(gamma) < 0.3, rng.integers(0, V, gamma), draft)
        n0, t0, d0 = verify_row_greedy(ell, draft, err)
        ref = _Res(n0, t0, d0, draft, gamma + 1)
        for scale, want in ((1.0, "ok"), (3.0, "any")):
            mv = ell + scale * err * rng.uniform(-1, 1, ell.shape)
            n1, t1, _ = verify_row_greedy(mv, draft)
            rep = compare_tokens(np.array([n1]), _Res(n1, t1, [], draft, gamma + 1).emitted, ref)
            if want == "ok":
                assert not rep.unexplained
                explained_flips += len(rep.mismatched)
            else:
                caught += len(rep.unexplained)
    assert explained_flips > 0 and caught > 0


def test_decision_record_basics():
    d = Decision("bonus", 3, 1e-7, 1e-6, frozenset({4, 5}))
    assert d.flagged and d.allows(5) and not d.allows(6)
    assert Decision("bonus", 3, 1e-5, 1e-6, frozenset({4})).flagged is False
    assert Decision("resample", 0, 0.0, np.inf, None).allows(123)
