"""The synthetic target network, in float64.

What it computes: one target pass scores every drafted position plus the
bonus slot at once ([LAT] reference implementation, the single target call
over k+1 positions; [PIG] "How it works", step 2).  The synthetic target is a
stack of MLP blocks, each

    n = h / sqrt(mean(h^2) + eps) * g        (RMSNorm, gain g)
    a = SiLU(n @ W_up)                       (SiLU(x) = x / (1 + e^-x))
    h = h + a @ W_down                       (residual)

followed by the LM head  logits = h @ W_lm.  Weights are row-major
[in][out].  There is no final norm before the LM head.  Rows are independent.

Weights may be float32 arrays or bfloat16 bit patterns held in uint16 arrays;
both widen exactly to float64 (a bfloat16 is the top half of a float32).

Pinned by: closed forms and invariants of RMSNorm and SiLU, the W_down = 0
special case (output equals h @ W_lm), row-permutation equivariance, and an
exact small integer example (tests/test_oracle_model.py).
"""

import numpy as np


def bf16_to_f64(bits):
    """Widen bfloat16 bit patterns (uint16) exactly to float64."""
    bits = np.asarray(bits)
    assert bits.dtype == np.uint16
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def as_f64(x):
    """float32 / float64 arrays, or bf16 bits in uint16, as float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    return np.asarray(x, dtype=np.float64)       # no copy when already float64


def rmsnorm(h, g, eps):
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * g


def silu(x):
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def forward(hidden, blocks, lm_head, eps=1e-6):
    """Logits [..., V] in float64.

    hidden  : [..., d] float array
    blocks  : list of dicts with keys w_up [d][ffn], w_down [ffn][d] and an
              optional gain [d] (None means all ones)
    lm_head : [d][V]
    """
    h = as_f64(hidden)
    for blk in blocks:
        g = blk.get("gain")
        g = np.ones(h.shape[-1]) if g is None else as_f64(g)
        n = rmsnorm(h, g, eps)
        a = silu(n @ as_f64(blk["w_up"]))
        h = h + a @ as_f64(blk["w_down"])
    return h @ as_f64(lm_head)
