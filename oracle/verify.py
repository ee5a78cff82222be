"""spec_verify over a batch: target pass, then the rule per batch row.

Interface shape follows the verification call the pages describe: the drafted
token ids, the draft's distributions [gamma, V] and the target's scores at
gamma + 1 positions in, the number accepted and the accepted tokens plus one
correction or bonus token out ([SSD] "The Accept/Reject Mechanism",
SpeculationResult and speculative_accept_reject; [PIG] "How it works").

Batch rows are independent ([SSD] "Batch-Level Speculation": rows accept
different counts); row b draws its uniforms from counter (i, b, 0, 0).

Outputs per row b:
  n_accepted[b]  in 0..gamma, or -1 when a draft token id lies outside [0, V)
  emitted[b]     drafts[0 .. n) followed by the correction / bonus token at
                 index n, then -1 padding; all -1 for a rejected row
"""

from dataclasses import dataclass, field

import numpy as np

from .model import as_f64, forward
from .philox import row_uniforms
from .rule import verify_row, verify_row_greedy, warp_logits, warp_probs


@dataclass
class VerifyResult:
    n_accepted: np.ndarray
    emitted: np.ndarray
    decisions: list = field(default_factory=list)  # per row: [rule.Decision]
    logits: np.ndarray = None
    cuts: list = field(default_factory=list)      # per row: (p TopPs, q TopPs) at T > 0
    drafts: np.ndarray = None                     # the draft tokens the rule read

    def nucleus_uncertain(self, b):
        """(p rows, q rows) of row b whose top-p membership is uncertain."""
        if not self.cuts or self.cuts[b] is None:
            return set(), set()
        pc, qc = self.cuts[b]
        return ({i for i, c in enumerate(pc) if c.uncertain},
                {i for i, c in enumerate(qc) if c.uncertain})

    def row_flagged(self, b):
        """Whether any decision of row b could flip on the other side."""
        return any(d.flagged for d in self.decisions[b])

    def n_decisions(self):
        return sum(len(d) for d in self.decisions)

    def n_flagged_decisions(self):
        return sum(1 for row in self.decisions for d in row if d.flagged)


def _check_scalars(temperature, top_p):
    if not (temperature >= 0.0) or not np.isfinite(temperature):
        raise ValueError("temperature must be finite and >= 0")
    if not (0.0 < top_p <= 1.0):
        raise ValueError("top_p must lie in (0, 1]")


def spec_verify_from_logits(logits, draft_tokens, q, temperature, top_p, seed,
                            batch_ids=None, logit_tol=0.0):
    """Acceptance rule for a batch given target logits [B, gamma+1, V].

    q is [B, gamma, V] (the draft's T = 1 probabilities); it is not read and
    may be None when temperature == 0.  batch_ids gives the batch index b of
    each row for its uniforms (default 0..B-1), so a few sequences of a larger
    batch can be checked on their own.  logit_tol only shapes the decision
    records: the other implementation's logits of a row may differ from these
    by up to logit_tol * max |logit| of the row (0: it reads the same logits).
    """
    _check_scalars(temperature, top_p)
    ell = as_f64(logits)
    draft = np.asarray(draft_tokens, dtype=np.int64)
    B, G1, V = ell.shape
    gamma = G1 - 1
    if draft.shape != (B, gamma):
        raise ValueError("draft_tokens must be [B, gamma]")
    if not np.all(np.isfinite(ell)):
        raise ValueError("non-finite logits")
    greedy = temperature == 0.0
    if not greedy:
        qq = as_f64(q)
        if qq.shape != (B, gamma, V):
            raise ValueError("q must be [B, gamma, V]")
        if not np.all(np.isfinite(qq)) or np.any(qq < 0):
            raise ValueError("q must be finite and non-negative")

    bids = np.arange(B) if batch_ids is None else np.asarray(batch_ids, dtype=np.int64)
    if bids.shape != (B,):
        raise ValueError("batch_ids must have one entry per row")
    n_acc = np.full(B, -1, dtype=np.int32)
    emitted = np.full((B, G1), -1, dtype=np.int32)
    decisions, cuts = [], []
    for b in range(B):
        xs = draft[b]
        if np.any(xs < 0) or np.any(xs >= V):
            decisions.append([])
            cuts.append(None)
            continue
        lerr = logit_tol * np.abs(ell[b]).max(axis=-1)
        if greedy:
            j, tok, mg = verify_row_greedy(ell[b], xs, lerr)
            cuts.append(None)
        else:
            p_rows, p_mg = zip(*[warp_logits(ell[b, i], temperature, top_p, lerr[i])
                                 for i in range(G1)])
            q_rows, q_mg = zip(*[warp_probs(qq[b, i], temperature, top_p)
                                 for i in range(gamma)]) if gamma else ((), ())
            uni = [row_uniforms(seed, int(bids[b]), i) for i in range(G1)]
            j, tok, mg = verify_row(p_rows, q_rows, xs, uni, p_cuts=p_mg, q_cuts=q_mg)
            cuts.append((list(p_mg), list(q_mg)))
        n_acc[b] = j
        emitted[b, :j] = xs[:j]
        emitted[b, j] = tok
        decisions.append(mg)
    return VerifyResult(n_acc, emitted, decisions, ell, cuts, draft)


def spec_verify(hidden, weights, draft_tokens, q, temperature, top_p, seed):
    """Full verification step: target pass over [B, gamma+1, d], then the rule.

    weights: dict with "blocks" (list of {w_up, w_down, gain}), "lm_head" and
    optionally "eps" (default 1e-6).
    """
    logits = forward(hidden, weights["blocks"], weights["lm_head"],
                     weights.get("eps", 1e-6))
    return spec_verify_from_logits(logits, draft_tokens, q, temperature,
                                   top_p, seed)
