"""The acceptance rule over the vocabulary, in float64, with decision margins.

Steps, in the pages' order:

1. Sampling transforms, applied identically to the target distribution p and
   the draft distribution q before the ratio test ([PIG] "When it breaks",
   last item; [SSD] "Quality, Evaluation, and Guardrails", item 1):
   temperature T first, then top-p.
     p' from target logits:  softmax(ell / T)
     q' from the draft's T = 1 probability vector:  q^(1/T) / sum q^(1/T)
        (the same as tempering the draft's logits; 0 stays 0)
   Top-p keeps, for each distribution separately, the shortest prefix of the
   tokens sorted by probability (descending, ties by lower token id) whose
   mass reaches top_p, then renormalises.  top_p >= 1 keeps everything.

2. Ratio test for draft token x at position i ([LAT] acceptance rule: accept
   when r < min(1, p(x)/q(x)) with r uniform in [0, 1); [PIG] "How it works",
   step 3; [SSD] "The Accept/Reject Mechanism").  Written in the multiply form
   r * q'(x) < p'(x), which equals the min form for q'(x) > 0 because r < 1,
   and accepts exactly when p'(x) > 0 if q'(x) = 0.  The epsilons the pages'
   sketches add to q are division guards and are not part of the rule.

3. First rejection at position j: sample a replacement from the residual
   norm(max(0, p'_j - q'_j)) and drop the later drafts ([LAT] acceptance rule
   and worked example; [PIG] step 4).  If the residual mass is exactly zero,
   sample p'_j instead ([SSD] "The Accept/Reject Mechanism", the numerical
   edge-case fallback).

4. No rejection: one bonus sample from p'_gamma ([PIG] step 5; [LAT]
   reference implementation, the for-else branch).

5. Temperature 0: accept while the draft token equals the target's argmax
   (lowest index on ties); the replacement or bonus is the argmax ([LAT]
   acceptance rule, greedy remark; [SSD] FAQ on beam search).  No uniforms
   are used and q is not read.

Sampling a distribution w with a uniform u is the inverse CDF in token-index
order: the smallest v whose inclusive prefix sum C(v) exceeds u * C(V-1).

Margins.  Every decision also returns how far it was from flipping, so a
float32 implementation may be compared decision by decision:
  ratio test       |r - p'(x)/q'(x)|            (p'(x) when q'(x) = 0)
  inverse CDF      distance of u*R to the nearest of C(v-1), C(v), over R
                   (and R itself when R < 1e-6)
  top-p cut        tokens whose nucleus membership is uncertain: the next
                   token when the kept mass exceeds top_p by less than MARGIN,
                   the last kept token when the mass before it falls short of
                   top_p by less than MARGIN, and (target rows only) every
                   token in a near-tied band at the cut, i.e. within
                   MARGIN * max|logit| of the last kept or first dropped logit.
                   A ratio test on an uncertain token has margin 0; other
                   ratio tests lose ratio * (uncertain mass of p' and q') of
                   margin; the inverse CDF loses twice that mass over R
  greedy argmax    gap between the two largest logits over max |logit|
A decision whose margin is below MARGIN is a knife-edge event.  The draft
distribution needs no order band: both sides sort the same float32 q.

Pinned by: the [LAT] worked example (tests/golden/worked_example.json); the
two-case identity and the emission law P(emit t) = p'(t) by quadrature over
(r, u) and by a chi-square test; alpha = sum min(p, q) = 1 - TV(p, q) by
Monte Carlo; a brute-force top-p over all subsets of a tiny vocabulary;
scipy.special.softmax for the temperature step; the T -> 0 limit of the
sampling branch for the greedy branch (tests/test_oracle_rule.py).
"""

import numpy as np

MARGIN = 1e-5


class TopP:
    """Knife-edge information of one nucleus cut (see the module docstring)."""

    def __init__(self, uncertain=(), mass=0.0):
        self.uncertain = set(int(v) for v in uncertain)   # may change sides
        self.mass = float(mass)    # their mass in the renormalised distribution


def nucleus_mask(probs, top_p, logp_tol=0.0):
    """Boolean mask of the top-p nucleus of a probability vector, and its
    knife-edge information.

    logp_tol: log-probability tolerance within which two tokens may swap
    order on the other side of the comparison (0: the order is exact).
    Returns (mask, TopP).  top_p >= 1 keeps every token.
    """
    probs = np.asarray(probs, dtype=np.float64)
    V = probs.shape[0]
    if top_p >= 1.0:
        return np.ones(V, dtype=bool), TopP()
    order = np.lexsort((np.arange(V), -probs))   # prob descending, id ascending
    s = probs[order]
    c = np.cumsum(s)
    hit = np.nonzero(c >= top_p)[0]
    k = int(hit[0]) if hit.size else V - 1
    mask = np.zeros(V, dtype=bool)
    mask[order[:k + 1]] = True
    unc = set()
    if k + 1 < V and c[k] - top_p < MARGIN:
        unc.add(int(order[k + 1]))                 # could join
    if k > 0 and top_p - c[k - 1] < MARGIN:
        unc.add(int(order[k]))                     # could drop out
    if logp_tol > 0 and k + 1 < V and s[k + 1] > 0:
        lo, hi = np.log(s[k + 1]), np.log(s[k])
        if hi - lo < logp_tol:
            with np.errstate(divide="ignore"):
                lp = np.log(probs)
            unc.update(int(v) for v in np.nonzero((lp >= lo - logp_tol) & (lp <= hi + logp_tol))[0])
    mass = probs[sorted(unc)].sum() / c[k] if unc else 0.0
    return mask, TopP(unc, mass)


def _apply_top_p(w, top_p, logp_tol=0.0):
    mask, info = nucleus_mask(w, top_p, logp_tol)
    if top_p < 1.0:
        w = np.where(mask, w, 0.0)
        w = w / w.sum()
    return w, info


def warp_logits(ell, T, top_p):
    """p' = top_p(softmax(ell / T)) for T > 0; returns (p', TopP)."""
    ell = np.asarray(ell, dtype=np.float64)
    e = np.exp((ell - ell.max()) / T)
    scale = np.abs(ell).max()
    return _apply_top_p(e / e.sum(), top_p, MARGIN * (scale if scale > 0 else 1.0) / T)


def warp_probs(q, T, top_p):
    """q' = top_p(q^(1/T) / sum q^(1/T)) for T > 0; returns (q', TopP)."""
    q = np.asarray(q, dtype=np.float64)
    # q^(1/T) scaled by qmax^(-1/T) so small T cannot underflow every entry
    pos = q > 0
    w = np.zeros_like(q)
    with np.errstate(divide="ignore"):
        w[pos] = np.exp((np.log(q[pos]) - np.log(q.max())) / T)
    return _apply_top_p(w / w.sum(), top_p)


def accept_test(p_x, q_x, r):
    """(accepted, margin) for one drafted token."""
    accepted = r * q_x < p_x
    if q_x > 0:
        margin = abs(r - p_x / q_x)
    else:
        # accept iff p'(x) > 0: a knife edge only if p'(x) is tiny but nonzero
        margin = p_x if p_x > 0 else np.inf
    return bool(accepted), float(margin)


def inverse_cdf(w, u):
    """Smallest v with C(v) > u*R, C the inclusive prefix sum, R = C(V-1)."""
    C = np.cumsum(np.asarray(w, dtype=np.float64))
    R = C[-1]
    assert R > 0
    t = u * R
    v = int(np.searchsorted(C, t, side="right"))
    lo = C[v - 1] if v > 0 else 0.0
    margin = min(C[v] - t, t - lo) / R
    if R < 1e-6:
        margin = min(margin, R)
    return v, float(margin)


def residual(p, q):
    """norm-free residual max(0, p - q); p itself when that is all zero."""
    res = np.maximum(0.0, p - q)
    return res if np.cumsum(res)[-1] > 0 else p


def verify_row(p_rows, q_rows, draft, uniforms, p_cuts=None, q_cuts=None):
    """Sampling branch (T > 0) for one batch row.

    p_rows   : gamma+1 warped target distributions p'_0 .. p'_gamma
    q_rows   : gamma warped draft distributions q'_0 .. q'_{gamma-1}
    draft    : gamma token ids, already checked to lie in [0, V)
    uniforms : gamma+1 pairs (r_i, u_i)
    p_cuts, q_cuts : optional TopP per row (top-p knife edges)
    Returns (n_accepted, token, margins) with margins a list of
    (kind, position, value) for the decisions actually taken.
    """
    gamma = len(draft)
    margins = []
    none = TopP()
    pc = (lambda i: p_cuts[i]) if p_cuts is not None else (lambda i: none)
    qc = (lambda i: q_cuts[i]) if q_cuts is not None else (lambda i: none)
    for i in range(gamma):
        x = int(draft[i])
        r, u = uniforms[i]
        ok, m = accept_test(p_rows[i][x], q_rows[i][x], r)
        unc_mass = pc(i).mass + qc(i).mass
        if x in pc(i).uncertain or x in qc(i).uncertain:
            m = 0.0
        elif unc_mass and q_rows[i][x] > 0:
            m -= p_rows[i][x] / q_rows[i][x] * unc_mass
        margins.append(("accept", i, m))
        if ok:
            continue
        w = residual(p_rows[i], q_rows[i])
        tok, m = inverse_cdf(w, u)
        if unc_mass:
            m -= 2.0 * unc_mass / np.cumsum(w)[-1]
        margins.append(("resample", i, m))
        return i, tok, margins
    tok, m = inverse_cdf(p_rows[gamma], uniforms[gamma][1])
    m -= 2.0 * pc(gamma).mass
    margins.append(("bonus", gamma, m))
    return gamma, tok, margins


def _argmax_margin(ell):
    ell = np.asarray(ell, dtype=np.float64)
    a = int(np.argmax(ell))                      # first index on ties
    rest = np.delete(ell, a)
    gap = ell[a] - rest.max() if rest.size else np.inf
    scale = np.abs(ell).max()
    return a, float(gap / (scale if scale > 0 else 1.0))


def verify_row_greedy(ell_rows, draft):
    """Greedy branch (T == 0) for one batch row; same returns as verify_row."""
    gamma = len(draft)
    margins = []
    for i in range(gamma):
        a, m = _argmax_margin(ell_rows[i])
        margins.append(("argmax", i, m))
        if int(draft[i]) != a:
            return i, a, margins
    a, m = _argmax_margin(ell_rows[gamma])
    margins.append(("argmax", gamma, m))
    return gamma, a, margins
