"""Host policy around the verification step: the speculation-depth (gamma)
controller and the repacking of a batch whose rows accepted different
counts.  Plain Python.

Gamma controller ("Build a Speculative Decoding Engine to Cut LLM Latency by
3x", scalablesystem.dev, "Dynamic Gamma Controller" and "Speculation Depth
Tuning and Tree Drafting"):
  * every verification step records (n_accepted, n_rejected) of a sequence,
    n_rejected = gamma - n_accepted as that article's SpeculationResult
    defines it; the last WINDOW = 20 steps are kept;
  * the rolling acceptance rate is sum(accepted) / sum(accepted + rejected)
    over the window (0.80 before any step);
  * from 5 recorded steps on, each step sets gamma to the value in
    [gamma_min, gamma_max] that maximises expected tokens per unit time,
        E(gamma) / (gamma * t_draft + t_target(gamma)),
        E(gamma) = (1 - alpha^(gamma + 1)) / (1 - alpha),
    the first (smallest) gamma on ties.
Readings where the article leaves a step open:
  * t_target(gamma): the article calibrates one constant target time per
    pass; here it may instead be a table of measured verification times per
    gamma (a verify pass of gamma + 1 rows costs more as gamma grows); a
    constant table reproduces the article.
  * alpha = 1: the article's code counts gamma tokens there, against its
    own formula, whose limit is gamma + 1 (every draft plus the bonus); the
    formula's limit is taken.
  * a row the verification step refused (n_accepted = -1) records nothing.

Ragged repacking ("Build a Speculative Decoding Engine...", "Batch-Level
Speculation"): after a step, sequence b emitted n_accepted[b] + 1 tokens
and its committed length grows by that much, so the rows are ragged.  The
repack gives both remedies the article names:
  * padding (one batch, padded to the longest row): the row offsets of the
    emitted tokens packed end to end, each sequence's new committed length,
    the padded width max(n_accepted) + 1 and the padding waste;
  * binning (micro-batches by accepted count): the sequences ordered by
    emitted count, stably, and the offsets of each bin.
A refused row (n_accepted = -1) emits nothing and sorts into bin 0.

Pinned by: the E(gamma) formula's page values (tests/golden/
expected_tokens.json); limiting cases (alpha = 0 picks the cheapest gamma,
free drafts with a constant target time pick gamma_max); the decision is
non-decreasing in alpha for a fixed cost model; brute-force enumeration of
tokens per second over every gamma on a grid of alphas; the window and
warm-up rules step by step; the repack against a hand-worked batch and
invariants (a permutation, sorted stably, offsets that sum, tokens that
round-trip) (tests/test_oracle_control.py).
"""

WINDOW = 20
MIN_STEPS = 5
DEFAULT_ALPHA = 0.80


def expected_tokens(alpha, gamma):
    """(1 - alpha^(gamma+1)) / (1 - alpha), with its limit gamma + 1 at 1."""
    if alpha >= 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


class GammaController:
    """Rolling-window gamma choice of one sequence."""

    def __init__(self, gamma_min=2, gamma_max=8, gamma_init=4, draft_ms_per_token=2.0,
                 target_ms=20.0):
        """target_ms: one number (every gamma) or a sequence indexed by gamma
        (entries gamma_min .. gamma_max are read)."""
        if not (0 <= gamma_min <= gamma_init <= gamma_max):
            raise ValueError("need 0 <= gamma_min <= gamma_init <= gamma_max")
        self.gamma = gamma_init
        self.gamma_min, self.gamma_max = gamma_min, gamma_max
        self.draft_ms = float(draft_ms_per_token)
        if isinstance(target_ms, (int, float)):
            self.target_ms = [float(target_ms)] * (gamma_max + 1)
        else:
            self.target_ms = [float(x) for x in target_ms]
            if len(self.target_ms) <= gamma_max:
                raise ValueError("target_ms needs an entry for every gamma up to gamma_max")
        self.window = []

    def rolling_alpha(self):
        if not self.window:
            return DEFAULT_ALPHA
        acc = sum(a for a, _ in self.window)
        tot = sum(a + r for a, r in self.window)
        return acc / max(tot, 1)

    def tokens_per_ms(self, alpha, gamma):
        return expected_tokens(alpha, gamma) / (gamma * self.draft_ms + self.target_ms[gamma])

    def optimal_gamma(self, alpha):
        best, best_rate = self.gamma_min, -1.0
        for g in range(self.gamma_min, self.gamma_max + 1):
            rate = self.tokens_per_ms(alpha, g)
            if rate > best_rate:
                best, best_rate = g, rate
        return best

    def step(self, n_accepted, n_rejected):
        if n_accepted < 0:
            return self.gamma
        self.window.append((int(n_accepted), int(n_rejected)))
        if len(self.window) > WINDOW:
            self.window.pop(0)
        if len(self.window) >= MIN_STEPS:
            self.gamma = self.optimal_gamma(self.rolling_alpha())
        return self.gamma


def repack(n_accepted, emitted, committed):
    """Ragged repacking after one verification step of a batch.

    n_accepted : [B] ints (-1 for a refused row)
    emitted    : [B][gamma + 1] tokens (-1 padding)
    committed  : [B] committed lengths before the step
    Returns a dict with
      tokens      the emitted tokens of every row, end to end
      offsets     [B + 1] row offsets into tokens
      committed   [B] new committed lengths (old + emitted count)
      order       [B] sequence ids sorted by emitted count, stably
      bin_offsets [gamma + 3] start of each emitted-count bin 0 .. gamma + 1
                  in `order`, then B
      width       max emitted count (the padded width of one batch)
      waste       padded slots that hold no token, B * width - sum counts
    """
    B = len(n_accepted)
    G1 = len(emitted[0]) if B else 1
    counts = [int(n) + 1 if int(n) >= 0 else 0 for n in n_accepted]
    offsets = [0]
    tokens = []
    for b in range(B):
        tokens.extend(int(t) for t in emitted[b][:counts[b]])
        offsets.append(offsets[-1] + counts[b])
    new_committed = [int(committed[b]) + counts[b] for b in range(B)]
    order = sorted(range(B), key=lambda b: (counts[b], b))
    bin_offsets = []
    for c in range(G1 + 1):
        bin_offsets.append(sum(1 for b in range(B) if counts[b] < c))
    bin_offsets.append(B)
    width = max(counts) if B else 0
    return {"tokens": tokens, "offsets": offsets, "committed": new_committed, "order": order,
            "bin_offsets": bin_offsets, "width": width, "waste": B * width - sum(counts)}
