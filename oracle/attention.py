"""Attention of the verification pass's new rows over a KV-cached prefix, and
the commit of the accepted rows' keys and values, in float64.

What it computes:
  * A verification pass feeds the target n_new new rows at once: the last
    committed token (the root) and the drafted tokens, in chain or tree
    order.  Row i attends to every cached position of its sequence and,
    among the new rows, to itself and its ancestors: the chain's causal
    mask, or the tree mask of "Speculative Decoding: Speeding Sequential
    Generation" (aicomputerinstitute.com, Constructing the Tree Attention
    Mask in Code), with position ids by depth applied by the caller before
    the keys are written.
  * Grouped-query attention: H query heads share Hkv key/value heads
    (query head h reads kv head h // (H / Hkv)), as the KV layout of "Build a
    Speculative Decoding Engine to Cut LLM Latency by 3x" (scalablesystem.dev,
    KV Cache Management for Dual Models: 8 KV heads of 128 dimensions).
  * out[b, i, h] = sum_t softmax_t(scale * q[b, i, h] . k[b, t]) v[b, t] over
    the visible positions t.
  * Commit after the step (same article, KV Cache Management for Dual
    Models and Rollback Protocol): the committed length is a pointer; a
    rejection is a pointer that does not move past the accepted rows.  With
    a tree, the accepted path's rows are first gathered to sit right after
    the root, in path order, so the cache stays a contiguous prefix; with a
    chain they already do.

Cache layout (a choice of this library, so that one key's or value's head
dimension is contiguous): k_cache, v_cache [B][Hkv][max_seq][hd]; sequence
b's committed positions are 0 .. L_b - 1 and the new rows' keys and values
sit at L_b .. L_b + n_new - 1.

Readings where the pages leave a step open:
  * The new rows' keys and values are in the cache before the attention
    call (written by the caller's projection), as the article's single
    forward pass over the prompt plus drafts implies.
  * parent[i] is the new row i's parent among the new rows (-1: none, it
    sees only the cached prefix, as the root does); parents precede
    children.  A chain is parent[i] = i - 1.
  * The commit keeps the root and the accepted drafts: L_b grows by
    n_accepted + 1 (the correction or bonus token has no key yet; it is the
    next pass's root).

Pinned by: closed forms (one visible position returns its value row;
equal scores return the mean of the visible values), the chain mask equal
to a causal mask, agreement with torch's float64 scaled-dot-product
attention under an explicit boolean mask (a library routine), a tree mask
taken from oracle/tree.py (itself pinned to the page's printed mask), and
the commit against a hand-built example (tests/test_oracle_attention.py).
"""

import numpy as np

from .model import as_f64


def visible_new(parent):
    """[n][n] bool: new row i sees new row j (itself or an ancestor)."""
    parent = [int(p) for p in parent]
    n = len(parent)
    vis = np.zeros((n, n), dtype=bool)
    for i in range(n):
        if not (-1 <= parent[i] < i):
            raise ValueError(f"row {i}: parent {parent[i]} must lie in [-1, {i})")
        vis[i, i] = True
        if parent[i] >= 0:
            vis[i] |= vis[parent[i]]
    return vis


def decode_attention(q, k_cache, v_cache, cache_len, parent=None, scale=None):
    """q [B][n_new][H][hd], caches [B][Hkv][max_seq][hd] (bf16 bits or
    floats), cache_len [B], parent [B][n_new] or None (chain).
    Returns out [B][n_new][H][hd] float64."""
    q = as_f64(q)
    K, Vc = as_f64(k_cache), as_f64(v_cache)
    B, n_new, H, hd = q.shape
    Hkv = K.shape[1]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    G = H // Hkv
    scale = 1.0 / np.sqrt(hd) if scale is None else float(scale)
    out = np.zeros((B, n_new, H, hd))
    for b in range(B):
        L = int(cache_len[b])
        par = list(range(-1, n_new - 1)) if parent is None else [int(x) for x in parent[b]]
        vis = visible_new(par)
        for h in range(H):
            kv = h // G
            keys = K[b, kv, :L + n_new]
            vals = Vc[b, kv, :L + n_new]
            for i in range(n_new):
                s = scale * (keys @ q[b, i, h])
                mask = np.concatenate([np.ones(L, dtype=bool), vis[i]])
                s = np.where(mask, s, -np.inf)
                w = np.exp(s - s[mask].max())
                out[b, i, h] = (w / w.sum()) @ vals
    return out


def kv_commit(k_cache, v_cache, cache_len, n_accepted, path=None):
    """Commit one step in place: the accepted rows' keys and values move to
    follow the root (tree: path[b][:n] gives the accepted nodes, node j
    being new row j + 1), and cache_len[b] grows by n_accepted[b] + 1.  A
    refused row (n_accepted < 0) commits nothing.  Returns the new lengths."""
    B = k_cache.shape[0]
    new_len = np.array(cache_len, dtype=np.int64).copy()
    for b in range(B):
        n = int(n_accepted[b])
        if n < 0:
            continue
        L = int(cache_len[b])
        if path is not None:
            rows = [L + 1 + int(path[b][k]) for k in range(n)]
            kk = k_cache[b][:, rows].copy()
            vv = v_cache[b][:, rows].copy()
            k_cache[b][:, L + 1:L + 1 + n] = kk
            v_cache[b][:, L + 1:L + 1 + n] = vv
        new_len[b] = L + n + 1
    return new_len
