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

Decision records.  The rule is exact in float64; an implementation in float32
(with logits that may themselves differ from these by up to `logit_err`) can
only flip a decision whose margin is smaller than what its arithmetic may
move.  Every decision therefore carries
  margin  the distance of its decision variable to the threshold
  slack   the largest change of that variable the other implementation's
          arithmetic may cause (a flip is explained when margin < slack)
  band    token decisions only: every token the other side may emit
          (None: any token)
with
  ratio test    margin |r - p'(x)/q'(x)| (p'(x) when q'(x) = 0);
                slack MARGIN + the bound on |delta(p'/q')| from the
                per-token bounds below and the masses of uncertain nucleus
                tokens; infinite when x itself is an uncertain token
  inverse CDF   margin the distance of t = u R to the nearest of C(v-1),
                C(v); slack delta = sum_v |delta w(v)| bound, because
                C(v) - u R moves by at most max(u, 1-u) sum |delta w|; the
                band holds every v whose [C(v-1) - delta, C(v) + delta)
                contains t; a row whose residual mass R is within delta of
                zero may fall back to p' on either side (band None)
  greedy argmax margin the gap between the two largest logits; slack
                2 logit_err; the band is every token within 2 logit_err of
                the maximum
Per-token bounds, float32 unit roundoff e = 2^-24, x = (l - max l) / T.  A
float32 p'(v) = exp(fl((l - m) * fl(1/T))) * (1/Z) [* (1/Z_nucleus)] carries
  own      e (6 + 3 |x_v|)      the argument's three roundings (difference,
                                1/T, product: |delta x| <= 3 e |x|), exp to
                                two units, the products with the normalisers
  common   e (10 + log2 V + 3 E_p'|x|)   the normalising sums (V terms, each
                                with its own error, summed in a tree of depth
                                log2 V) and the reciprocals
  logits   2 logit_err / T      a logit error moves exp(l / T) by at most
                                logit_err / T, and the normaliser as much
and q'(v) (y = ln q / T - max) the same with |x| replaced by
|y_v| + |ln q_v| / T (the log adds its own rounding); at T = 1, q' = q / Z
carries e (1 + 4 + log2 V).
Top-p membership: the cut is uncertain when the kept mass exceeds top_p by
less than MARGIN + the mass bound (the next token may join), or the mass
before the last kept token falls short by less than that (it may drop out),
and, when logits differ, every token whose log-probability lies within
2 logit_err / T of the cut's two neighbours may change order.

MARGIN = 1e-5 is the knife-edge width the ratio test is held to.

Pinned by: the [LAT] worked example (tests/golden/worked_example.json); the
two-case identity and the emission law P(emit t) = p'(t) by quadrature over
(r, u) and by a chi-square test; alpha = sum min(p, q) = 1 - TV(p, q) by
Monte Carlo; a brute-force top-p over all subsets of a tiny vocabulary;
scipy.special.softmax for the temperature step; the T -> 0 limit of the
sampling branch for the greedy branch; and the decision records by
perturbation: p', q' and logits moved within the stated bounds, and nucleus
memberships of uncertain tokens flipped, change only flagged decisions, and
only to tokens in their bands (tests/test_oracle_rule.py,
tests/test_oracle_margins.py).
"""

import math

import numpy as np

MARGIN = 1e-5
EPS32 = 2.0 ** -24


class TopP:
    """Result of one warp: knife-edge information of the nucleus cut and the
    per-token error bound of the warped distribution (see the module
    docstring)."""

    def __init__(self, uncertain=(), mass=0.0, err=None, alt=None):
        self.uncertain = set(int(v) for v in uncertain)   # may change sides
        self.mass = float(mass)    # their mass in the renormalised distribution
        self.err = err             # per-token absolute bound on |delta w'| (kept tokens)
        self.alt = dict(alt or {})  # uncertain token -> its w' had it been on the other side


class Decision:
    """One decision of the rule: kind ('accept', 'resample', 'bonus',
    'argmax'), position, margin, slack and band (see the module docstring).
    `raw` is the ratio test's |r - p'/q'|, whose near-zero draws are counted
    as knife edges."""

    __slots__ = ("kind", "pos", "margin", "slack", "band", "raw")

    def __init__(self, kind, pos, margin, slack=0.0, band=(), raw=None):
        self.kind, self.pos = kind, int(pos)
        self.margin, self.slack = float(margin), float(slack)
        self.band = band
        self.raw = raw

    @property
    def flagged(self):
        return self.margin < self.slack

    def allows(self, token):
        """Whether the other implementation may emit `token` here."""
        return self.band is None or int(token) in self.band

    def __repr__(self):
        return (f"Decision({self.kind}, pos={self.pos}, margin={self.margin:.3g}, "
                f"slack={self.slack:.3g}, flagged={self.flagged})")


def _rel_bound(a, w, V):
    """Per-token relative bound of a float32 warp whose exp argument has
    magnitude a (see the module docstring), w the warped distribution."""
    return EPS32 * ((6.0 + 3.0 * a) + (10.0 + math.log2(max(V, 2)) + 3.0 * float(np.dot(w, a))))


def nucleus_mask(probs, top_p, logp_tol=0.0, mass_tol=MARGIN):
    """Boolean mask of the top-p nucleus of a probability vector, and its
    knife-edge information.

    logp_tol: log-probability tolerance within which two tokens may swap
    order on the other side of the comparison (0: the order is exact).
    mass_tol: how far the other side's cumulative masses may be off.
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
    if k + 1 < V and c[k] - top_p < mass_tol:
        unc.add(int(order[k + 1]))                 # could join
    if k > 0 and top_p - c[k - 1] < mass_tol:
        unc.add(int(order[k]))                     # could drop out
    if logp_tol > 0 and k + 1 < V and s[k + 1] > 0:
        lo, hi = np.log(s[k + 1]), np.log(s[k])
        if hi - lo < logp_tol:
            with np.errstate(divide="ignore"):
                lp = np.log(probs)
            unc.update(int(v) for v in np.nonzero((lp >= lo - logp_tol) & (lp <= hi + logp_tol))[0])
    mass = probs[sorted(unc)].sum() / c[k] if unc else 0.0
    return mask, TopP(unc, mass)


def _apply_top_p(w, rel, top_p, logp_tol=0.0):
    """Nucleus of w (with per-token relative bound rel), renormalised."""
    err_mass = float(np.dot(w, rel))
    mask, info = nucleus_mask(w, top_p, logp_tol, MARGIN + err_mass)
    if top_p < 1.0:
        kept = w[mask].sum()
        info.alt = {v: (0.0 if mask[v] else w[v] / kept) for v in info.uncertain}
        w = np.where(mask, w, 0.0) / kept
    info.err = w * rel
    return w, info


def warp_logits(ell, T, top_p, logit_err=0.0):
    """p' = top_p(softmax(ell / T)) for T > 0; returns (p', TopP).

    logit_err: absolute bound on how far the other implementation's logits
    of this row may lie from ell (0 when both read the same float32 logits).
    """
    ell = np.asarray(ell, dtype=np.float64)
    x = (ell - ell.max()) / T
    e = np.exp(x)
    p = e / e.sum()
    rel = _rel_bound(np.abs(x), p, ell.shape[0]) + 2.0 * logit_err / T
    return _apply_top_p(p, rel, top_p, 2.0 * logit_err / T)


def warp_probs(q, T, top_p):
    """q' = top_p(q^(1/T) / sum q^(1/T)) for T > 0; returns (q', TopP)."""
    q = np.asarray(q, dtype=np.float64)
    V = q.shape[0]
    # q^(1/T) scaled by qmax^(-1/T) so small T cannot underflow every entry
    pos = q > 0
    y = np.zeros_like(q)
    lq = np.zeros_like(q)
    w = np.zeros_like(q)
    with np.errstate(divide="ignore"):
        lq[pos] = np.abs(np.log(q[pos])) / T
        y[pos] = (np.log(q[pos]) - np.log(q.max())) / T
        w[pos] = np.exp(y[pos])
    w = w / w.sum()
    if T == 1.0:
        rel = np.full(V, EPS32 * (5.0 + math.log2(max(V, 2))))
    else:
        rel = _rel_bound(np.abs(y) + lq, w, V)
    return _apply_top_p(w, rel, top_p)


def accept_test(p_x, q_x, r):
    """(accepted, |r - p'/q'|) for one drafted token (p'(x) when q'(x) = 0)."""
    accepted = r * q_x < p_x
    if q_x > 0:
        margin = abs(r - p_x / q_x)
    else:
        # accept iff p'(x) > 0: a knife edge only if p'(x) is tiny but nonzero
        margin = p_x if p_x > 0 else np.inf
    return bool(accepted), float(margin)


def inverse_cdf(w, u):
    """(v, margin): the smallest v with C(v) > u*R, C the inclusive prefix
    sum, R = C(V-1); margin = distance of u*R to the nearest of C(v-1), C(v)."""
    C = np.cumsum(np.asarray(w, dtype=np.float64))
    R = C[-1]
    assert R > 0
    t = u * R
    v = int(np.searchsorted(C, t, side="right"))
    lo = C[v - 1] if v > 0 else 0.0
    return v, float(min(C[v] - t, t - lo))


def cdf_band(w, t, delta):
    """Every token v whose [C(v-1) - delta, C(v) + delta) contains t."""
    C = np.cumsum(np.asarray(w, dtype=np.float64))
    lo = np.concatenate(([0.0], C[:-1]))
    return frozenset(int(v) for v in np.nonzero((lo - delta <= t) & (t < C + delta))[0])


def residual(p, q):
    """norm-free residual max(0, p - q); p itself when that is all zero."""
    res = np.maximum(0.0, p - q)
    return res if np.cumsum(res)[-1] > 0 else p


def _sample_decision(kind, pos, w, u, delta):
    """Inverse-CDF decision on w with the other side's sum |delta w| <= delta."""
    tok, margin = inverse_cdf(w, u)
    R = np.cumsum(w)[-1]
    t = u * R
    delta = delta + 4.0 * w.shape[0] * 2.0 ** -53 * R   # float64 prefix sums
    return tok, Decision(kind, pos, margin, delta, cdf_band(w, t, delta))


def verify_row(p_rows, q_rows, draft, uniforms, p_cuts=None, q_cuts=None):
    """Sampling branch (T > 0) for one batch row.

    p_rows   : gamma+1 warped target distributions p'_0 .. p'_gamma
    q_rows   : gamma warped draft distributions q'_0 .. q'_{gamma-1}
    draft    : gamma token ids, already checked to lie in [0, V)
    uniforms : gamma+1 pairs (r_i, u_i)
    p_cuts, q_cuts : optional TopP per row (nucleus knife edges, error bounds)
    Returns (n_accepted, token, decisions): the Decision of every test and
    sample actually taken, in order.
    """
    gamma = len(draft)
    decisions = []
    none = TopP()
    pc = (lambda i: p_cuts[i]) if p_cuts is not None else (lambda i: none)
    qc = (lambda i: q_cuts[i]) if q_cuts is not None else (lambda i: none)

    def err(cut, i, x):
        return 0.0 if cut.err is None else float(cut.err[x])

    def l1(cut, w):
        return 0.0 if cut.err is None else float(cut.err.sum())

    for i in range(gamma):
        x = int(draft[i])
        r, u = uniforms[i]
        p_x, q_x = p_rows[i][x], q_rows[i][x]
        ok, raw = accept_test(p_x, q_x, r)
        cp, cq = pc(i), qc(i)
        unc_mass = cp.mass + cq.mass
        if x in cp.uncertain or x in cq.uncertain:
            slack = np.inf
        elif q_x > 0:
            ratio = p_x / q_x
            slack = MARGIN + (err(cp, i, x) + ratio * err(cq, i, x)) / q_x + ratio * unc_mass
        else:
            slack = MARGIN + err(cp, i, x)
        decisions.append(Decision("accept", i, raw, slack, raw=raw))
        if ok:
            continue
        w = residual(p_rows[i], q_rows[i])
        delta = l1(cp, w) + l1(cq, w) + 2.0 * unc_mass
        if np.cumsum(np.maximum(0.0, p_rows[i] - q_rows[i]))[-1] <= delta:
            # the residual may be zero on either side: p' or the residual
            tok, _ = inverse_cdf(w, u)
            decisions.append(Decision("resample", i, 0.0, np.inf, None))
        else:
            tok, d = _sample_decision("resample", i, w, u, delta)
            decisions.append(d)
        return i, tok, decisions
    cg = pc(gamma)
    tok, d = _sample_decision("bonus", gamma, p_rows[gamma], uniforms[gamma][1],
                              l1(cg, p_rows[gamma]) + 2.0 * cg.mass)
    decisions.append(d)
    return gamma, tok, decisions


def _argmax_decision(ell, pos, logit_err):
    ell = np.asarray(ell, dtype=np.float64)
    a = int(np.argmax(ell))                      # first index on ties
    rest = np.delete(ell, a)
    gap = ell[a] - rest.max() if rest.size else np.inf
    slack = 2.0 * logit_err
    band = frozenset(int(v) for v in np.nonzero(ell >= ell[a] - slack)[0])
    return a, Decision("argmax", pos, gap, slack, band)


def verify_row_greedy(ell_rows, draft, logit_err=0.0):
    """Greedy branch (T == 0) for one batch row; same returns as verify_row.
    logit_err: absolute bound on the other side's logit error per row (a
    sequence, or one value for every row)."""
    gamma = len(draft)
    errs = np.broadcast_to(np.asarray(logit_err, dtype=np.float64), (gamma + 1,))
    decisions = []
    for i in range(gamma):
        a, d = _argmax_decision(ell_rows[i], i, errs[i])
        decisions.append(d)
        if int(draft[i]) != a:
            return i, a, decisions
    a, d = _argmax_decision(ell_rows[gamma], gamma, errs[gamma])
    decisions.append(d)
    return gamma, a, decisions
