"""Pins for the oracle's synthetic target network (RMSNorm / SiLU MLP / LM head)."""

import numpy as np
import pytest
from scipy.special import expit

from oracle import bf16_to_f64, forward, rmsnorm, silu
from synth import f32_to_bf16_bits, model_np, hidden_np


def test_bf16_known_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3FC0, 0x0000, 0x8000, 0x7F7F, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.5, 0.0, -0.0, 3.3895313892515355e38, 3.140625]
    got = bf16_to_f64(bits)
    assert got.tolist() == want


def test_bf16_rounding_of_generator_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -3.0 - 2 ** -7],
                 dtype=np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7 -> even (1); 1+3*2^-8 ties up to 1+2^-6
    assert bf16_to_f64(f32_to_bf16_bits(x)).tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -3.0]


def test_silu_against_library_logistic():
    x = np.linspace(-30, 30, 601)
    assert np.allclose(silu(x), x * expit(x), rtol=1e-14, atol=1e-300)
    assert silu(np.array([0.0]))[0] == 0.0
    assert silu(np.array([-1000.0]))[0] == 0.0


def test_rmsnorm_invariants():
    rng = np.random.default_rng(0)
    h = rng.standard_normal((4, 37))
    g = np.ones(37)
    n = rmsnorm(h, g, 0.0)
    assert np.allclose(np.sqrt(np.mean(n * n, axis=-1)), 1.0, rtol=1e-14)
    assert np.allclose(rmsnorm(7.5 * h, g, 0.0), n, rtol=1e-13)            # scale invariant
    gain = rng.standard_normal(37)
    assert np.allclose(rmsnorm(h, gain, 0.0), n * gain, rtol=1e-13)
    c = np.full((1, 5), 0.01)
    eps = 1e-4                                                         # eps inside the root
    assert np.allclose(rmsnorm(c, np.ones(5), eps), 0.01 / np.sqrt(1e-4 + eps), rtol=1e-14)


def test_forward_exact_small_example():
    """Hand-worked 2 -> 3 -> 2 block with a 2-token head (all matrices
    non-symmetric so a transposed operand changes the answer)."""
    h = np.array([[1.0, -1.0]])                 # mean(h^2) = 1, so n = h
    blk = {"w_up": np.array([[1.0, 0.0, 2.0], [1.0, -1.0, 0.0]]),
           "w_down": np.array([[1.0, 0.0], [0.0, 1.0], [1.0, -1.0]]),
           "gain": None}
    lm = np.array([[1.0, 0.0], [1.0, 1.0]])
    # n @ W_up = [0, 1, 2]; a = [0, e1, 2 e2]; a @ W_down = [2 e2, e1 - 2 e2]
    e1, e2 = expit(1.0), expit(2.0)
    h1 = np.array([1.0 + 2 * e2, -1.0 + e1 - 2 * e2])
    want = np.array([h1[0] + h1[1], h1[1]])
    got = forward(h, [blk], lm, eps=0.0)[0]
    assert np.allclose(got, want, rtol=1e-15, atol=1e-15)


def test_zero_down_projection_passes_hidden_through():
    m = model_np((99,), 16, 24, 2, 10, "f32")
    for blk in m["blocks"]:
        blk["w_down"] = np.zeros_like(blk["w_down"])
    h = hidden_np((99,), 2, 3, 16)
    got = forward(h, m["blocks"], m["lm_head"])
    want = h.astype(np.float64) @ m["lm_head"].astype(np.float64)
    assert np.allclose(got, want, rtol=1e-13, atol=1e-13)


def test_rows_are_independent_and_permutation_equivariant():
    m = model_np((98,), 16, 24, 2, 10, "bf16", random_gain=True)
    h = hidden_np((98,), 3, 2, 16).reshape(9, 16)
    full = forward(h, m["blocks"], m["lm_head"])
    perm = np.random.default_rng(1).permutation(9)
    assert np.allclose(forward(h[perm], m["blocks"], m["lm_head"]), full[perm], rtol=1e-13, atol=1e-13)
    one = forward(h[4:5], m["blocks"], m["lm_head"])
    assert np.allclose(one, full[4:5], rtol=1e-13, atol=1e-13)


def test_gain_enters_as_elementwise_scale():
    m = model_np((97,), 8, 12, 1, 6, "f32")
    h = hidden_np((97,), 1, 1, 8)[0]
    base = forward(h, m["blocks"], m["lm_head"])
    # a gain of 2 on every feature equals doubling W_up
    m2 = {"blocks": [dict(m["blocks"][0], gain=np.full(8, 2.0, dtype=np.float32))],
          "lm_head": m["lm_head"]}
    m3 = {"blocks": [dict(m["blocks"][0], w_up=2.0 * m["blocks"][0]["w_up"].astype(np.float64))],
          "lm_head": m["lm_head"]}
    assert np.allclose(forward(h, m2["blocks"], m2["lm_head"]),
                       forward(h, m3["blocks"], m3["lm_head"]), rtol=1e-13)
    assert not np.allclose(base, forward(h, m2["blocks"], m2["lm_head"]))
