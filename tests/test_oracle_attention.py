"""Pins for the oracle's decode attention and KV commit (oracle/attention.py)."""

import numpy as np
import pytest
import torch

from oracle import attention, tree


def rand_case(rng, B=2, n_new=5, H=8, Hkv=2, hd=16, max_seq=64):
    q = rng.standard_normal((B, n_new, H, hd))
    k = rng.standard_normal((B, Hkv, max_seq, hd))
    v = rng.standard_normal((B, Hkv, max_seq, hd))
    L = rng.integers(0, max_seq - n_new + 1, B)
    return q, k, v, L


def test_chain_mask_is_causal_and_tree_mask_matches_the_tree_module():
    assert (attention.visible_new([-1, 0, 1, 2]) == np.tril(np.ones((4, 4), dtype=bool))).all()
    # the page's nodes A, B, A1, A2, B1, B2 under a root row 0
    parent_nodes = [-1, -1, 0, 0, 1, 1]
    rows = [-1] + [p + 1 for p in parent_nodes]        # root first, then the nodes
    vis = attention.visible_new(rows)
    assert (vis[1:, 1:].astype(int) == tree.tree_mask(parent_nodes)).all()
    assert vis[:, 0].all()                              # every node sees the root


def test_single_visible_position_returns_its_value():
    rng = np.random.default_rng(1)
    q, k, v, _ = rand_case(rng, B=1, n_new=1, max_seq=8)
    out = attention.decode_attention(q, k, v, [0])      # empty prefix: the root sees itself
    H, Hkv = q.shape[2], k.shape[1]
    for h in range(H):
        assert np.allclose(out[0, 0, h], v[0, h // (H // Hkv), 0], rtol=0, atol=1e-15)


def test_equal_scores_average_the_visible_values():
    rng = np.random.default_rng(2)
    q, k, v, _ = rand_case(rng, B=1, n_new=3)
    q[:] = 0.0
    L = [10]
    out = attention.decode_attention(q, k, v, L)
    H, Hkv = q.shape[2], k.shape[1]
    for i in range(3):
        for h in range(H):
            kv = h // (H // Hkv)
            want = v[0, kv, :L[0] + i + 1].mean(axis=0)    # prefix plus rows 0..i
            assert np.allclose(out[0, i, h], want, atol=1e-14)


@pytest.mark.parametrize("seed", range(4))
def test_matches_torch_sdpa_with_an_explicit_mask(seed):
    rng = np.random.default_rng(10 + seed)
    q, k, v, L = rand_case(rng)
    B, n_new, H, hd = q.shape
    Hkv = k.shape[1]
    parent = np.array([[-1] + [int(rng.integers(-1, i)) for i in range(1, n_new)] for _ in range(B)])
    out = attention.decode_attention(q, k, v, L, parent)
    for b in range(B):
        T = L[b] + n_new
        mask = np.zeros((n_new, T), dtype=bool)
        mask[:, :L[b]] = True
        mask[:, L[b]:] = attention.visible_new(parent[b])
        kk = torch.from_numpy(k[b, :, :T]).repeat_interleave(H // Hkv, 0)      # [H][T][hd]
        vv = torch.from_numpy(v[b, :, :T]).repeat_interleave(H // Hkv, 0)
        qq = torch.from_numpy(q[b].transpose(1, 0, 2).copy())                  # [H][n_new][hd]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=torch.from_numpy(mask)).numpy().transpose(1, 0, 2)
        assert np.allclose(out[b], ref, rtol=1e-12, atol=1e-12)


def test_commit_chain_moves_only_the_pointer_and_tree_gathers_the_path():
    rng = np.random.default_rng(3)
    B, Hkv, S, hd, n_new = 2, 2, 20, 4, 6
    k = rng.standard_normal((B, Hkv, S, hd))
    v = rng.standard_normal((B, Hkv, S, hd))
    k0, v0 = k.copy(), v.copy()
    L = [5, 9]
    new = attention.kv_commit(k, v, L, [2, -1])
    assert new.tolist() == [8, 9] and (k == k0).all() and (v == v0).all()
    path = np.array([[1, 3, -1, -1, -1], [0, -1, -1, -1, -1]])      # nodes; node j is row j + 1
    new = attention.kv_commit(k, v, L, [2, 1], path)
    assert new.tolist() == [8, 11]
    assert (k[0, :, 5] == k0[0, :, 5]).all()                        # the root stays
    assert (k[0, :, 6] == k0[0, :, 5 + 1 + 1]).all() and (k[0, :, 7] == k0[0, :, 5 + 1 + 3]).all()
    assert (v[1, :, 10] == v0[1, :, 10]).all()                      # path [0]: already in place
