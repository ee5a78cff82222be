"""Pins for the oracle's greedy tree verification (oracle/tree.py)."""

import json
import os

import numpy as np
import pytest

from oracle import tree
from oracle.rule import verify_row_greedy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden():
    with open(os.path.join(GOLDEN, "tree_mask.json")) as f:
        return json.load(f)


def test_mask_and_depths_match_the_printed_example():
    g = golden()
    assert tree.tree_mask(g["parent"]).tolist() == g["mask"]
    assert tree.tree_depths(g["parent"]) == g["depths"]


def test_chain_mask_is_causal():
    """A tree with one child per node is a chain; its mask is the causal
    (lower-triangular) one."""
    n = 7
    parent = [-1] + list(range(n - 1))
    assert (tree.tree_mask(parent) == np.tril(np.ones((n, n), dtype=int))).all()
    assert tree.tree_depths(parent) == list(range(1, n + 1))


def test_bad_parents_are_refused():
    for parent in ([0], [-1, 1], [-2], [-1, 5]):
        with pytest.raises(ValueError):
            tree.tree_mask(parent)


@pytest.mark.parametrize("seed", range(6))
def test_chain_reduces_to_the_chain_rule(seed):
    rng = np.random.default_rng(seed)
    n, V = 6, 40
    ell = rng.standard_normal((n + 1, V))
    am = ell.argmax(-1)
    tokens = np.where(rng.random(n) < 0.7, am[:n], rng.integers(0, V, n))
    parent = [-1] + list(range(n - 1))
    k, em, path, _ = tree.verify_tree_greedy(ell, parent, tokens)
    k2, tok2, _ = verify_row_greedy(ell, tokens)
    assert k == k2 and em[:k] == [int(t) for t in tokens[:k]] and em[k] == tok2
    assert path == list(range(k))


def random_tree(rng, n, V, distinct=True):
    parent = [-1] + [int(rng.integers(-1, j)) for j in range(1, n)]
    tokens = np.zeros(n, dtype=int)
    used = {}
    for j, pj in enumerate(parent):
        while True:
            t = int(rng.integers(0, V))
            if not distinct or t not in used.setdefault(pj, set()):
                break
        used.setdefault(pj, set()).add(t)
        tokens[j] = t
    return parent, tokens


@pytest.mark.parametrize("seed", range(30))
def test_walk_is_the_deepest_passing_path(seed):
    """Siblings carry distinct tokens, so at most one child of a node passes:
    the accepted path is the deepest node whose whole root path passes."""
    rng = np.random.default_rng(100 + seed)
    n, V = int(rng.integers(1, 14)), 6
    parent, tokens = random_tree(rng, n, V)
    ell = rng.standard_normal((n + 1, V))
    am = ell.argmax(-1)
    # bias the draft toward passing so deep paths occur
    for j in range(n):
        if rng.random() < 0.6:
            sib = {int(tokens[s]) for s in range(n) if parent[s] == parent[j] and s != j}
            if int(am[parent[j] + 1]) not in sib:
                tokens[j] = am[parent[j] + 1]
    passes = [int(tokens[j]) == int(am[parent[j] + 1]) for j in range(n)]
    best = []
    for j in range(n):
        chain = [j] + tree.ancestors(parent, j)
        if all(passes[c] for c in chain) and len(chain) > len(best):
            best = chain[::-1]
    k, em, path, decs = tree.verify_tree_greedy(ell, parent, tokens)
    assert path == best and k == len(best)
    last = best[-1] if best else -1
    assert em == [int(tokens[c]) for c in best] + [int(am[last + 1])]
    assert len(decs) >= 1 and all(d.kind == "argmax" for d in decs)


def test_duplicate_sibling_tokens_take_the_lower_index():
    ell = np.array([[0.0, 5.0, 1.0], [0.0, 0.0, 9.0], [9.0, 0.0, 0.0]])
    k, em, path, _ = tree.verify_tree_greedy(ell, [-1, -1], [1, 1])
    assert path == [0] and em == [1, 2]


@pytest.mark.parametrize("case", golden()["expected_tokens"]["values"], ids=lambda c: f"p={c['p']}")
def test_expected_depth_of_a_full_binary_tree(case):
    """The page's model: every node passes independently with probability p;
    the walk reaches depth d with probability q^d, q = 1 - (1 - p)^b."""
    p, b, D = case["p"], case["b"], case["D"]
    q = 1 - (1 - p) ** b
    assert abs(q - case["q"]) < 1e-12
    assert abs(sum(q ** d for d in range(1, D + 1)) - case["expected_depth"]) <= case["tol"]
    assert abs(1 + case["expected_depth"] - case["tokens_per_round"]) < 1e-12
    parent = [-1, -1]
    for lvl in range(1, D):
        first = len(parent) - b ** lvl
        for node in range(first, first + b ** lvl):
            parent += [node] * b
    assert len(parent) == sum(b ** d for d in range(1, D + 1))
    rng = np.random.default_rng(int(p * 100))
    N = 60000
    depths = np.array([len(tree.tree_walk(parent, lambda j, a=rng.random(len(parent)): a[j] < p))
                       for _ in range(N)])
    mean = sum(q ** d for d in range(1, D + 1))
    probs = [q ** d - q ** (d + 1) for d in range(D)] + [q ** D]
    var = sum(pr * d * d for d, pr in enumerate(probs)) - mean ** 2
    assert abs(depths.mean() - mean) < 4 * np.sqrt(var / N)


def test_batch_form_rejects_bad_rows():
    rng = np.random.default_rng(3)
    ell = rng.standard_normal((3, 4, 10))
    parent = np.array([[-1, 0, 0], [-1, 1, 0], [-1, -1, 1]])     # row 1: parent 1 of node 1
    tokens = np.array([[1, 2, 3], [1, 2, 3], [1, 2, 10]])        # row 2: token out of range
    n, em, path, _ = tree.spec_verify_tree_greedy(ell, parent, tokens)
    assert n[0] >= 0 and n[1] == -1 and n[2] == -1
    assert (em[1] == -1).all() and (path[2] == -1).all()
