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
  target's parallel verification): ``ancestor_mask``, and ``tree_attention``,
  the target's attention over the flattened tree under that mask;
* 6.5: greedy walk -- from the root, step to the child the target accepts,
  stop at the first rejection; the accepted path is committed and the
  target's prediction at the last accepted node is the bonus;
* 6.6: only the accepted path's KV is appended to the cache
  (``commit_tree_kv``).

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
  siblings carry distinct tokens, so at most one child is accepted;
* the tree pass of the target: the root is not in the cache yet, so the
  flattened rows are the root (row 0) and the nodes (row 1 + j), each seeing
  the committed context, the root and its own ancestors; Q and K arrive
  position-encoded (a node's position is the context length plus its depth);
  rows past the tree see the context and the root;
* KV recycling commits the root and the accepted nodes, in path order, at the
  positions that follow the committed prefix; the bonus token is the next
  round's root and is not committed.
"""
import heapq
from dataclasses import dataclass

import numpy as np

from .materialize import slots
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


def walk_greedy(tree_token, tree_parent, target_predict, max_depth=None):
    """Greedy walk of one request's tree.  target_predict[0] is the target's
    argmax after the root, target_predict[1 + j] after node j.

    With ``max_depth`` the walk stops after that many accepted nodes (the
    caller keeps room for only that many); the bonus is then the target's
    argmax at the last node kept, so the commit (accepted + 1) never exceeds
    max_depth + 1 and every committed row has a tree row behind it."""
    cur, path = -1, []
    while True:
        want = int(target_predict[cur + 1])
        if max_depth is not None and len(path) >= max_depth:
            return TreeWalk(len(path), want, path)
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


def _root_path(parent, x):
    """Node x and its ancestors, root side first."""
    p = []
    while x >= 0:
        p.append(x)
        x = int(parent[x])
    return p[::-1]


def tree_attention(q, k_tree, v_tree, cache_k, cache_v, block_table, ctx_lens, node_parent,
                   n_nodes, dtype, scale=None, rows=None):
    """The target's attention over the flattened tree ([Spec-decoding tutorial] 6.4).

    Rows of a request: row 0 is the root (the last committed token, not yet in
    the cache), row 1 + j is node j.  Every row attends to the committed
    context (logical positions [0, ctx_lens[b]) of the paged cache) and to the
    tree rows on its own root path: the root, the node's ancestors and the node
    itself -- never to siblings or cousins.  A row past the tree (node index
    >= n_nodes[b]) sees the context and the root.

    q [B, R, Hq, D], k_tree / v_tree [B, R, Hkv, D] with R = 1 + budget;
    node_parent [B, budget] (-1: a child of the root).  Returns
    (out [B, R, Hq, D], lse [B, Hq, R]); with ``rows`` (a list of row
    indices) only those rows are computed, the others are left zero."""
    q, kt, vt = widen(q, dtype), widen(k_tree, dtype), widen(v_tree, dtype)
    ck, cv = widen(cache_k, dtype), widen(cache_v, dtype)
    B, R, Hq, D = q.shape
    Hkv = kt.shape[2]
    G = Hq // Hkv
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, R, Hq, D))
    lse = np.zeros((B, Hq, R))
    for b in range(B):
        C = int(ctx_lens[b])
        pos = np.arange(C)
        pages = block_table[b, pos // 16]
        ctx_k, ctx_v = slots(ck)[pages, pos % 16], slots(cv)[pages, pos % 16]
        n = int(n_nodes[b])
        for r in (range(R) if rows is None else rows):
            seen = [0] if r == 0 or r - 1 >= n else [0] + [1 + y for y in _root_path(node_parent[b], r - 1)]
            keys = np.concatenate([ctx_k, kt[b, seen]], axis=0)
            vals = np.concatenate([ctx_v, vt[b, seen]], axis=0)
            for h in range(Hq):
                s = scale * (keys[:, h // G, :] @ q[b, r, h])
                m = s.max()
                e = np.exp(s - m)
                out[b, r, h] = (e @ vals[:, h // G, :]) / e.sum()
                lse[b, h, r] = m + np.log(e.sum())
    return out, lse


def commit_tree_kv(k_tree, v_tree, accepted_nodes, accept_len, prefix_lens, cache_k, cache_v,
                   block_table):
    """KV recycling ([Spec-decoding tutorial] 6.6): after the walk only the
    accepted path's rows join the request's cache; the rest are never stored.

    The rows committed for request b are the root (tree row 0) and its
    accepted nodes in path order (tree rows 1 + accepted_nodes[b, t]), at the
    logical positions prefix_lens[b] + 0, 1, ...; a request whose accept_len
    is negative (the walk's in-band error) commits nothing.  Writes in place
    (rows on unmapped pages are skipped, as in ``paged_write``) and returns the
    bool [num_pages, 16] of slots written, for K (V is written alike)."""
    from .materialize import paged_write
    B, R = k_tree.shape[:2]
    width = accepted_nodes.shape[1] + 1
    src = np.zeros(B * width, dtype=np.int64)
    commit = np.zeros(B, dtype=np.int64)
    for b in range(B):
        a = int(accept_len[b])
        if a < 0:
            continue
        path = [0] + [1 + int(j) for j in accepted_nodes[b, :a]]
        commit[b] = len(path)
        src[b * width: b * width + len(path)] = path
    rows_k = np.asarray(k_tree)[np.repeat(np.arange(B), width), src]
    rows_v = np.asarray(v_tree)[np.repeat(np.arange(B), width), src]
    written = paged_write(cache_k, rows_k, block_table, width, prefix_lens, commit)
    paged_write(cache_v, rows_v, block_table, width, prefix_lens, commit)
    return written
