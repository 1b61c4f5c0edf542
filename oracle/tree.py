"""DDTree: a draft tree under a node budget, and its greedy verification -- oracle.

Test infrastructure: see the package header for who may import this.

Follows [Spec-decoding tutorial, section 6]:
* 6.1: the root is the last committed token; every block position offers its
  top-K candidates, and the tree branches over them;
* 6.3: a path's joint probability is the product of the per-position
  marginals (the drafter's positions are independent); the tree is grown
  best first: all children of the root go into a heap, the most probable
  leaf is popped and its children (the next position's top-K) are pushed,
  until the tree holds B nodes;
* 6.4: a node sees only its ancestors (the ancestor-only mask of the
  target's parallel verification);
* 6.5: greedy walk -- from the root, step to the child the target accepts,
  stop at the first rejection; the accepted path is committed and the
  target's prediction at the last accepted node is the bonus.

Readings where the pages leave a step open (also in the design doc):
* the candidates of a position are its K most probable tokens under
  softmax(row / T), ties to the lower token id (equal logits, equal
  probabilities); a node's score is its joint log-probability;
* heap order: higher score first; equal scores pop in the order of the
  parents' pops (the root first), then by sibling rank; so a parent always
  precedes its children and the result is unique;
* a candidate of probability zero (a logit of -inf) is never a node, so a
  tree can stop short of the budget before the full K-ary tree is spent;
* nodes are numbered in pop order; parent -1 means the root; depth d means
  block position d (1-based), drawn from draft row d - 1;
* greedy acceptance of a child: its token equals the target's argmax at its
  parent (row 0 for the root, row 1 + j for node j; ties to the lower id);
  siblings carry distinct tokens, so at most one child is accepted.
"""
import heapq
from dataclasses import dataclass

import numpy as np

from .numerics import widen


def topk_logprobs(draft_logits, dtype, K, temperature=1.0):
    """Per row of draft_logits [B, n, V]: the K most probable tokens (ties to
    the lower id) and their log-probabilities log softmax(row / T).
    Returns (tokens int64 [B, n, K], logp float64 [B, n, K])."""
    d = widen(draft_logits, dtype) / temperature
    B, n, V = d.shape
    tok = np.zeros((B, n, K), dtype=np.int64)
    lp = np.zeros((B, n, K))
    for b in range(B):
        for i in range(n):
            row = d[b, i]
            m = row.max()
            lse = m + np.log(np.exp(row - m).sum())
            order = np.lexsort((np.arange(V), -row))[:K]   # value descending, then id
            tok[b, i] = order
            lp[b, i] = row[order] - lse
    return tok, lp


@dataclass
class Tree:
    token: np.ndarray    # [n_nodes] int64
    parent: np.ndarray   # [n_nodes] int64, -1 = the root
    depth: np.ndarray    # [n_nodes] int64, 1-based block position
    score: np.ndarray    # [n_nodes] joint log-probability
    rank: np.ndarray     # [n_nodes] sibling rank within its position's top-K


def build_tree(tokens, logp, budget):
    """Best-first tree of one request from its per-position top-K lists
    (tokens, logp: [n, K]).  Returns a Tree with min(budget, all) nodes in pop
    order."""
    n, K = logp.shape
    heap = [(-float(logp[0, r]), -1, r, 1) for r in range(K)   # (-score, parent pop, rank, depth)
            if logp[0, r] > -np.inf]
    heapq.heapify(heap)
    tok, par, dep, sc, rk = [], [], [], [], []
    while heap and len(tok) < budget:
        neg, p, r, dpt = heapq.heappop(heap)
        i = len(tok)
        tok.append(int(tokens[dpt - 1, r]))
        par.append(p)
        dep.append(dpt)
        sc.append(-neg)
        rk.append(r)
        if dpt < n:
            for r2 in range(K):
                if logp[dpt, r2] > -np.inf:
                    heapq.heappush(heap, (neg - float(logp[dpt, r2]), i, r2, dpt + 1))
    return Tree(np.array(tok, dtype=np.int64), np.array(par, dtype=np.int64),
                np.array(dep, dtype=np.int64), np.array(sc), np.array(rk, dtype=np.int64))


def ancestor_mask(parent):
    """[N, N] bool: node i sees node j iff j is i or one of its ancestors."""
    N = len(parent)
    m = np.zeros((N, N), dtype=bool)
    for i in range(N):
        j = i
        while j >= 0:
            m[i, j] = True
            j = int(parent[j])
    return m


@dataclass
class TreeWalk:
    accept_len: int
    bonus: int
    path: list          # accepted node indices, root side first


def walk_greedy(tree_token, tree_parent, target_predict):
    """Greedy walk of one request's tree.  target_predict[0] is the target's
    argmax after the root, target_predict[1 + j] after node j."""
    cur, path = -1, []
    while True:
        want = int(target_predict[cur + 1])
        nxt = [j for j in range(len(tree_token)) if tree_parent[j] == cur and tree_token[j] == want]
        if not nxt:
            return TreeWalk(len(path), want, path)
        cur = nxt[0]
        path.append(cur)


def target_argmax(target_logits, dtype):
    """Row argmax of [B, R, V] logits, ties to the lower id."""
    t = widen(target_logits, dtype)
    B, R, _ = t.shape
    out = np.zeros((B, R), dtype=np.int64)
    for b in range(B):
        for r in range(R):
            row = t[b, r]
            out[b, r] = int(np.flatnonzero(row == row.max())[0])
    return out
