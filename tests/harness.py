"""Shared helpers for parity tests: workload construction and comparison.

Inputs are built with synth (random draws) and the oracle (target logits,
softmax), never with the HIP path.  Comparison follows the margin rule: a
GPU row must equal the oracle row unless the oracle made a knife-edge
decision (margin < oracle.MARGIN) in that row.
"""

import collections
import json
import os

import numpy as np

import oracle
import synth


# ---------------------------------------------------------------- workload construction

def softmax_rows(x):
    """softmax over the last axis via the oracle's T = 1 warper."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1, x.shape[-1])
    if flat.shape[0] == 0:
        return np.zeros(x.shape)
    out = np.stack([oracle.warp_logits(r, 1.0, 1.0)[0] for r in flat])
    return out.reshape(x.shape)


def draft_q(ell, noise):
    """q = softmax(target logits + noise) for the gamma draft rows, fp32."""
    gamma = noise.shape[1]
    return softmax_rows(ell[:, :gamma] + noise).astype(np.float32)


def sample_drafts(q, T, top_p, key):
    """Drafts ~ q' (the draft's own sampling, harness side)."""
    gen = synth.generator(*key, synth.T_DRAFT)
    B, gamma, V = q.shape
    out = np.zeros((B, gamma), dtype=np.int32)
    for b in range(B):
        for i in range(gamma):
            w = oracle.warp_probs(q[b, i], T, top_p)[0] if T > 0 else q[b, i] / q[b, i].sum()
            c = np.cumsum(w)
            out[b, i] = min(int(np.searchsorted(c, gen.random() * c[-1], side="right")), V - 1)
    return out


def mean_alpha(ell, q, T=1.0, top_p=1.0):
    B, gamma = q.shape[:2]
    a = [np.minimum(oracle.warp_logits(ell[b, i], T, top_p)[0],
                    oracle.warp_probs(q[b, i], T, top_p)[0]).sum()
         for b in range(B) for i in range(gamma)]
    return float(np.mean(a))


def calibrate_sigma(ell, z, target, lo=0.01, hi=4.0, iters=18):
    """Bisection on sigma so that q = softmax(ell + sigma z) has mean alpha ~ target."""
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if mean_alpha(ell, draft_q(ell, mid * z)) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def greedy_drafts(ell, key, agree=0.75):
    """Draft = argmax of the target with probability `agree`, else a uniform other id."""
    gen = synth.generator(*key, synth.T_DRAFT)
    B, G1, V = ell.shape
    gamma = G1 - 1
    out = np.zeros((B, gamma), dtype=np.int32)
    for b in range(B):
        for i in range(gamma):
            a = int(np.argmax(ell[b, i]))
            if gen.random() < agree:
                out[b, i] = a
            else:
                o = int(gen.integers(0, V - 1))
                out[b, i] = o + (o >= a)
    return out


# ---------------------------------------------------------------- comparison

def logits_rel_err(gpu, ref):
    """Per row max |gpu - ref| / max |ref|."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.abs(gpu - ref).max(axis=-1) / np.maximum(np.abs(ref).max(axis=-1), 1e-30)


def compare_tokens(n_gpu, emit_gpu, ref, rows=None):
    """Returns (mismatched rows, unexplained rows, flagged decisions by kind,
    decisions by kind)."""
    rows = range(len(ref.n_accepted)) if rows is None else rows
    mism, unexplained = [], []
    for j, b in enumerate(rows):
        same = int(n_gpu[j]) == int(ref.n_accepted[b]) and \
            np.array_equal(np.asarray(emit_gpu[j]), ref.emitted[b])
        if not same:
            mism.append(b)
            if ref.row_min_margin(b) >= oracle.MARGIN:
                unexplained.append(b)
    flagged, total = collections.Counter(), collections.Counter()
    for b in rows:
        for kind, _, m in ref.margins[b]:
            total[kind] += 1
            if m < oracle.MARGIN:
                flagged[kind] += 1
    return mism, unexplained, flagged, total


def log_measurement(record):
    """Append a JSON line to $SV_PARITY_LOG when set (for reading rates)."""
    path = os.environ.get("SV_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps(record) + "\n")


def assert_tokens_match(n_gpu, emit_gpu, ref, rows=None, what=""):
    """Rows must match unless the oracle made a knife-edge decision in them;
    knife-edge ratio tests (|r - p'/q'| < 1e-5) must stay under 0.1% of the
    ratio tests; the other knife-edge kinds are counted and reported."""
    mism, unexplained, flagged, total = compare_tokens(n_gpu, emit_gpu, ref, rows)
    log_measurement({"what": what, "rows": len(ref.n_accepted) if rows is None else len(rows),
                     "mismatched_rows": len(mism), "flagged": dict(flagged),
                     "decisions": dict(total)})
    assert not unexplained, f"{what}: rows differ without a knife-edge decision: {unexplained[:10]}"
    assert flagged["accept"] <= max(1, 0.001 * total["accept"]), \
        f"{what}: {flagged['accept']} knife-edge ratio tests of {total['accept']}"
    return mism, sum(flagged.values()), sum(total.values())


def ref_probs(ell, q, T, top_p):
    """Oracle p' [B][gamma+1][V] and q' [B][gamma][V] (float64)."""
    B, G1, V = ell.shape
    p = np.stack([[oracle.warp_logits(ell[b, i], T, top_p)[0] for i in range(G1)] for b in range(B)])
    qq = np.stack([[oracle.warp_probs(q[b, i], T, top_p)[0] for i in range(G1 - 1)]
                   for b in range(B)]) if G1 > 1 else np.zeros((B, 0, V))
    return p, qq


def compare_probs(p_gpu, q_gpu, ref, ell, q, T, top_p, rows, what):
    """p' and q' within 1e-5 absolute, on every row whose nucleus is certain
    (a knife-edge cut renormalises the whole row by one token's mass)."""
    pr, qr = ref_probs(ell, q, T, top_p)
    worst = 0.0
    for b in rows:
        if ref.n_accepted[b] < 0:
            continue
        up, uq = ref.nucleus_uncertain(b)
        for i in range(pr.shape[1]):
            if i not in up:
                worst = max(worst, float(np.abs(p_gpu[b, i] - pr[b, i]).max()))
        for i in range(qr.shape[1]):
            if i not in uq:
                worst = max(worst, float(np.abs(q_gpu[b, i] - qr[b, i]).max()))
    log_measurement({"what": f"{what} probs", "abs_err_max": worst})
    assert worst <= 1e-5, f"{what}: p'/q' abs err {worst:.2e}"
