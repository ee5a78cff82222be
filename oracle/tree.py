"""Greedy verification of a draft tree, in float64.

What it computes ("Speculative Decoding: Speeding Sequential Generation",
aicomputerinstitute.com, sections "Tree-Based Drafting: Testing More Than One
Guess", "Constructing the Tree Attention Mask in Code" and "Expected Tokens
per Verification Round: Chain vs. Tree"; "Build a Speculative Decoding
Engine to Cut LLM Latency by 3x", scalablesystem.dev, "Speculation Depth
Tuning and Tree Drafting"):

  * The draft is a tree of candidate tokens.  Node j has a token and a
    parent (-1: a child of the root, the last committed position).  Parents
    are listed before their children (parent[j] < j), so the nodes can be
    scored in one pass.
  * Node i may see node j iff j is i itself or one of i's ancestors (the
    tree attention mask); its position id is its depth (level-1 nodes sit at
    depth 1), not its offset in the flattened node list.
  * One target pass scores the root row and every node row: the root's row
    predicts the level-1 token, a node's row predicts its children's token.
  * The same test as for a chain is applied per node; a branch survives if
    one of its children passes, and the walk descends through it.  At
    temperature 0 a node passes when its token equals the argmax of its
    parent's row.  The walk stops at the first row none of whose children
    passes and emits that row's argmax (the correction, or the bonus at a
    leaf), so a round yields the accepted path plus one token.

Readings where the pages leave a step open:
  * Only the greedy rule is built: the pages do not fix a stochastic rule for
    several candidate children of one node.
  * Two children of one node carrying the same token: the lower node index is
    taken (either gives the same emitted tokens; the path records which).
  * Argmax ties: the lowest token id, as for a chain.

Pinned by: the page's printed 6 x 6 mask and depths for nodes A, B, A1, A2,
B1, B2 (tests/golden/tree_mask.json); a chain (every parent the previous
node) reduces to the chain's greedy rule; brute force over every
root-to-node path on small random trees; the page's expected depth
q + q^2 + q^3 with q = 1 - (1 - p)^b for a full binary tree whose nodes pass
independently, by Monte Carlo (tests/test_oracle_tree.py).
"""

import numpy as np

from .model import as_f64
from .rule import Decision, _argmax_decision


def check_parents(parent):
    parent = [int(x) for x in parent]
    for j, pj in enumerate(parent):
        if not (-1 <= pj < j):
            raise ValueError(f"node {j}: parent {pj} must lie in [-1, {j})")
    return parent


def ancestors(parent, j):
    """Ancestors of node j, nearest first (the root itself is not a node)."""
    out = []
    cur = parent[j]
    while cur != -1:
        out.append(cur)
        cur = parent[cur]
    return out


def tree_mask(parent):
    """[n][n] 0/1 mask: node i sees node j iff j == i or j is an ancestor of i."""
    parent = check_parents(parent)
    n = len(parent)
    mask = np.zeros((n, n), dtype=int)
    for i in range(n):
        mask[i, i] = 1
        for j in ancestors(parent, i):
            mask[i, j] = 1
    return mask


def tree_depths(parent):
    """Depth of every node: 1 for children of the root."""
    parent = check_parents(parent)
    return [1 + len(ancestors(parent, j)) for j in range(len(parent))]


def tree_walk(parent, passes):
    """The accepted path: from the root, repeatedly descend to the
    lowest-index child that passes (passes(node) -> bool), until none does.
    Returns the node indices of the path, root excluded."""
    parent = check_parents(parent)
    children = {}
    for j, pj in enumerate(parent):
        children.setdefault(pj, []).append(j)
    path, cur = [], -1
    while True:
        nxt = next((j for j in children.get(cur, []) if passes(j)), None)
        if nxt is None:
            return path
        path.append(nxt)
        cur = nxt


def verify_tree_greedy(ell_rows, parent, tokens, logit_err=0.0):
    """Greedy tree verification of one sequence.

    ell_rows : [n + 1][V] logits, row 0 the root, row 1 + j node j
    parent   : n parents (-1 for children of the root), parent[j] < j
    tokens   : n draft tokens in [0, V)
    logit_err: absolute bound on the other implementation's logit error
               per row (shapes the decision records only)
    Returns (n_accepted, emitted, path, decisions): the accepted depth,
    the accepted tokens followed by the row's argmax, the accepted node
    indices, and the argmax Decision of every row the walk read.
    """
    ell = as_f64(ell_rows)
    parent = check_parents(parent)
    n = len(parent)
    if ell.shape[0] != n + 1:
        raise ValueError("need one logits row for the root and one per node")
    errs = np.broadcast_to(np.asarray(logit_err, dtype=np.float64), (n + 1,))
    decisions = []
    memo = {}

    def argmax_of(node):          # row of a node (-1: the root)
        if node not in memo:
            a, d = _argmax_decision(ell[node + 1], len(decisions), errs[node + 1])
            decisions.append(d)
            memo[node] = a
        return memo[node]

    path = tree_walk(parent, lambda j: int(tokens[j]) == argmax_of(parent[j]))
    last = path[-1] if path else -1
    emitted = [int(tokens[j]) for j in path] + [argmax_of(last)]
    return len(path), emitted, path, decisions


def spec_verify_tree_greedy(logits, parent, tokens, logit_tol=0.0):
    """Batch form: logits [B][n+1][V], parent and tokens [B][n].  Returns
    (n_accepted [B], emitted [B][n+1], path [B][n], decisions per row);
    a sequence with a bad parent or token gets n_accepted = -1 and all -1
    rows.  logit_tol: relative logit tolerance of the other side (per row,
    times max |logit| of the row)."""
    ell = as_f64(logits)
    parent = np.asarray(parent, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    B, G1, V = ell.shape
    n = G1 - 1
    if parent.shape != (B, n) or tokens.shape != (B, n):
        raise ValueError("parent and tokens must be [B][n]")
    n_acc = np.full(B, -1, dtype=np.int32)
    emitted = np.full((B, n + 1), -1, dtype=np.int32)
    paths = np.full((B, n), -1, dtype=np.int32)
    decisions = []
    for b in range(B):
        ok = all(-1 <= int(parent[b, j]) < j for j in range(n)) and \
            bool(np.all((tokens[b] >= 0) & (tokens[b] < V)))
        if not ok:
            decisions.append([])
            continue
        lerr = logit_tol * np.abs(ell[b]).max(axis=-1)
        k, em, path, decs = verify_tree_greedy(ell[b], parent[b], tokens[b], lerr)
        n_acc[b] = k
        emitted[b, :k + 1] = em
        paths[b, :k] = path
        decisions.append(decs)
    return n_acc, emitted, paths, decisions
