"""Pins for the DDTree oracle: top-K against a brute-force selection and a
library log-softmax, the best-first tree against a hand example and against
exhaustive search for the best ancestor-closed node set, the ancestor mask
against a path walk, and the greedy walk against the pages' example and
against the chain verify it reduces to when the tree is one path."""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth


def test_topk_matches_brute_force_selection_and_log_softmax():
    rng = np.random.default_rng(60)
    x = (rng.standard_normal((2, 3, 200)) * 2).astype(np.float32)
    x[0, 0, 7] = x[0, 0, 50] = x[0, 0, 120] = 9.0       # a three-way tie at the top
    x[1, 2, 3] = x[1, 2, 4] = -9.0                       # ties far below: irrelevant
    tok, lp = oracle.topk_logprobs(x, "f32", K=5, temperature=0.7)
    ref_lp = scipy.special.log_softmax(x.astype(np.float64) / 0.7, axis=-1)
    for b in range(2):
        for i in range(3):
            row = x[b, i].astype(np.float64)
            taken, picks = np.zeros(200, dtype=bool), []
            for _ in range(5):                           # repeated maximum, lowest index first
                best = max(v for v, t in zip(row, taken) if not t)
                j = next(j for j in range(200) if not taken[j] and row[j] == best)
                taken[j] = True
                picks.append(j)
            assert tok[b, i].tolist() == picks
            np.testing.assert_allclose(lp[b, i], ref_lp[b, i, picks], rtol=0, atol=1e-12)
    assert tok[0, 0, :3].tolist() == [7, 50, 120]


def _lists(probs):
    """Per-position top-K as (tokens, logp) from explicit probability lists."""
    tokens = np.array([[t for t, _ in pos] for pos in probs])
    logp = np.log(np.array([[p for _, p in pos] for pos in probs]))
    return tokens, logp


def test_best_first_hand_example():
    """Positions 1-3 offer (cat .7, dog .2), (sat .6, lay .3), (on .65, in .2);
    K = 2, budget 5.  By hand the pops are cat .70, cat>sat .42,
    cat>sat>on .273, cat>lay .21, dog .20 (cat>sat>in .084 and dog>sat .12 stay
    in the heap)."""
    CAT, DOG, SAT, LAY, ON, IN = 10, 11, 20, 21, 30, 31
    tokens, logp = _lists([[(CAT, .7), (DOG, .2)], [(SAT, .6), (LAY, .3)], [(ON, .65), (IN, .2)]])
    t = oracle.build_tree(tokens, logp, budget=5)
    assert t.token.tolist() == [CAT, SAT, ON, LAY, DOG]
    assert t.parent.tolist() == [-1, 0, 1, 0, -1]
    assert t.depth.tolist() == [1, 2, 3, 2, 1]
    np.testing.assert_allclose(np.exp(t.score), [.7, .42, .273, .21, .2], rtol=1e-12)
    # one more node: dog>sat (.12) beats cat>lay>on (.1365)? no: .1365 > .12
    t6 = oracle.build_tree(tokens, logp, budget=6)
    assert t6.token[5] == ON and t6.parent[5] == 3


def _all_nodes(K, n):
    return [p for d in range(1, n + 1) for p in itertools.product(range(K), repeat=d)]


@pytest.mark.parametrize("K,n,bmax,seed", [(2, 3, 7, 61), (3, 2, 7, 62), (2, 4, 7, 63),
                                            (3, 3, 5, 64)])
def test_best_first_is_optimal_among_ancestor_closed_sets(K, n, bmax, seed):
    """The best-first tree of B nodes has the largest total node probability
    (the expected number of accepted tokens under independent positions)
    among all node sets of size B that contain every member's ancestors."""
    rng = np.random.default_rng(seed)
    logp = np.log(np.sort(rng.dirichlet(np.ones(K + 2), size=n)[:, :K], axis=1)[:, ::-1])
    tokens = np.arange(n * K).reshape(n, K)
    nodes = _all_nodes(K, n)
    score = {p: sum(logp[d, r] for d, r in enumerate(p)) for p in nodes}
    for B in range(1, min(len(nodes), bmax) + 1):
        best = -1.0
        for subset in itertools.combinations(nodes, B):
            s = set(subset)
            if all(p[:-1] in s for p in subset if len(p) > 1):
                best = max(best, sum(math.exp(score[p]) for p in subset))
        t = oracle.build_tree(tokens, logp, budget=B)
        assert abs(np.exp(t.score).sum() - best) < 1e-12


def test_zero_probability_candidates_are_no_nodes():
    """Position 2 has only two tokens of nonzero probability (the rest have
    logit -inf): with K = 3 over two positions the whole tree is the 3 roots'
    children plus 3 x 2 grandchildren, so a budget of 20 stops at 9 nodes, and
    no node carries a zero-probability token."""
    x = np.full((1, 2, 6), -np.inf)
    x[0, 0] = [0.5, 1.0, -1.0, 2.0, 0.0, -0.5]
    x[0, 1, [1, 4]] = [0.3, -0.2]
    tok, lp = oracle.topk_logprobs(x, "f64", K=3)
    assert tok[0, 1, :2].tolist() == [1, 4] and lp[0, 1, 2] == -np.inf
    t = oracle.build_tree(tok[0], lp[0], budget=20)
    assert len(t.token) == 9
    assert np.all(np.isfinite(t.score))
    assert sorted(t.token[t.depth == 2].tolist()) == [1, 1, 1, 4, 4, 4]


def test_tree_order_properties_on_synthetic_draft():
    """Parents precede children, scores never increase along the pop order,
    children scores are the parent's plus their position's log-probability,
    and siblings carry distinct tokens."""
    x = synth.tree_case(65, dtype="f32", B=2, n_pos=7, V=500, std=2.0).draft_logits
    tok, lp = oracle.topk_logprobs(x, "f32", K=4)
    for b in range(2):
        t = oracle.build_tree(tok[b], lp[b], budget=60)
        assert len(t.token) == 60
        assert all(t.parent[i] < i for i in range(60))
        assert np.all(np.diff(t.score) <= 1e-15)
        for i in range(60):
            base = 0.0 if t.parent[i] < 0 else t.score[t.parent[i]]
            assert abs(t.score[i] - (base + lp[b, t.depth[i] - 1, t.rank[i]])) < 1e-12
            if t.parent[i] >= 0:
                assert t.depth[i] == t.depth[t.parent[i]] + 1
        kids = {}
        for i in range(60):
            kids.setdefault(int(t.parent[i]), []).append(int(t.token[i]))
        assert all(len(v) == len(set(v)) for v in kids.values())


def test_ancestor_mask_matches_path_walk():
    parent = np.array([-1, 0, 1, 0, -1, 4, 2, 6])
    m = oracle.ancestor_mask(parent)
    for i in range(len(parent)):
        anc = {i}
        j = parent[i]
        while j >= 0:
            anc.add(int(j))
            j = parent[j]
        assert set(np.flatnonzero(m[i]).tolist()) == anc
        assert (m[i] == (m[parent[i]] | (np.arange(len(parent)) == i))).all() if parent[i] >= 0 \
            else m[i].sum() == 1


def test_walk_pages_example():
    """[Spec-decoding tutorial, section 6.5]: root -> cat (accepted) -> sat
    (accepted) -> on (rejected); dog is rejected at the root.  Two tokens are
    committed and the bonus is the target's prediction after sat."""
    CAT, DOG, SAT, LAY, ON, THE = 1, 2, 3, 4, 5, 6
    token = np.array([CAT, DOG, SAT, LAY, ON])
    parent = np.array([-1, -1, 0, 0, 2])
    tp = np.array([CAT, SAT, 9, THE, 9, 9])   # after root, after node 0 (cat), 1 (dog), 2 (sat), ...
    w = oracle.walk_greedy(token, parent, tp)
    assert (w.accept_len, w.bonus, w.path) == (2, THE, [0, 2])
    w = oracle.walk_greedy(token, parent, np.array([7, SAT, 9, THE, 9, 9]))
    assert (w.accept_len, w.bonus, w.path) == (0, 7, [])
    w = oracle.walk_greedy(token, parent, np.array([CAT, SAT, 9, ON, 9, 8]))
    assert (w.accept_len, w.bonus, w.path) == (3, 8, [0, 2, 4])   # a leaf: bonus after it


def test_walk_stops_at_max_depth():
    """A caller with room for max_depth accepted nodes: the walk of the page's
    example (cat, sat, on all accepted) stops after max_depth nodes and the
    bonus is the target's prediction at the last node kept, so commit =
    accepted + 1 rows all have a tree row behind them."""
    CAT, DOG, SAT, LAY, ON = 1, 2, 3, 4, 5
    token = np.array([CAT, DOG, SAT, LAY, ON])
    parent = np.array([-1, -1, 0, 0, 2])
    tp = np.array([CAT, SAT, 9, ON, 9, 8])
    for md, want in [(1, (1, SAT, [0])), (2, (2, ON, [0, 2])), (3, (3, 8, [0, 2, 4])),
                     (9, (3, 8, [0, 2, 4]))]:
        w = oracle.walk_greedy(token, parent, tp, max_depth=md)
        assert (w.accept_len, w.bonus, w.path) == want


def test_walk_on_a_single_path_is_the_chain_verify():
    """With K = 1 the tree is one path: the walk equals greedy chain
    verification of those drafts."""
    c = synth.greedy_case(66, dtype="f32", B=6, L=7, V=300, plant=True)
    ref = oracle.verify_greedy(c.target_logits, "f32", draft_tokens=c.draft_tokens)
    tp = oracle.target_argmax(c.target_logits, "f32")
    for b in range(6):
        parent = np.arange(-1, 6)
        w = oracle.walk_greedy(c.draft_tokens[b], parent, tp[b])
        assert w.accept_len == ref.accept_len[b] and w.bonus == ref.bonus[b]


# ------------------------------------------------------------ tree attention

def _chain_parents(n):
    return np.arange(n) - 1


def test_tree_attention_of_a_chain_is_causal_block_attention():
    """A tree that is one path (node j's parent is node j - 1) is a block of
    n + 1 rows in which row i sees rows 0..i: the causal block mask."""
    R = 7
    c = synth.attention_case(71, dtype="f32", B=2, k=R, n_q_heads=4, n_kv_heads=2, head_dim=16,
                             ctx_lens=[20, 0])
    par = np.stack([_chain_parents(R - 1)] * 2)
    out, lse = oracle.tree_attention(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v, c.block_table,
                                     c.ctx_lens, par, [R - 1, R - 1], "f32")
    ref, rlse = oracle.block_attention(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v, c.block_table,
                                       c.ctx_lens, "f32", causal=True)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-12)


def test_tree_attention_row_is_its_root_path_prefilled_alone():
    """6.4: verifying the tree in one pass gives each node what prefilling its
    own root path alone would: node x's row equals the last row of causal
    block attention over [root, ancestors of x, x]."""
    x = synth.tree_case(72, dtype="f32", B=1, n_pos=4, V=50, std=1.0).draft_logits
    tok, lp = oracle.topk_logprobs(x, "f32", K=3)
    t = oracle.build_tree(tok[0], lp[0], budget=20)
    R = 21
    c = synth.attention_case(73, dtype="f32", B=1, k=R, n_q_heads=4, n_kv_heads=1, head_dim=16,
                             ctx_lens=[33])
    out, _ = oracle.tree_attention(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v, c.block_table,
                                   c.ctx_lens, t.parent[None], [20], "f32")
    for node in (0, 5, 11, 19):
        path, y = [], node
        while y >= 0:
            path.append(1 + y)
            y = int(t.parent[y])
        rows = [0] + path[::-1]
        ref, _ = oracle.block_attention(c.q[:, rows], c.k_blk[:, rows], c.v_blk[:, rows],
                                        c.cache_k, c.cache_v, c.block_table, c.ctx_lens, "f32",
                                        causal=True)
        np.testing.assert_allclose(out[0, 1 + node], ref[0, -1], rtol=0, atol=1e-12)


def test_tree_attention_star_and_rows_past_the_tree():
    """Children of the root see the context, the root and themselves; rows
    past n_nodes see the context and the root only."""
    R = 6
    c = synth.attention_case(74, dtype="f32", B=1, k=R, n_q_heads=2, n_kv_heads=2, head_dim=8,
                             ctx_lens=[5])
    par = np.full((1, R - 1), -1)
    out, _ = oracle.tree_attention(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v, c.block_table,
                                   c.ctx_lens, par, [3], "f32")
    for r in range(R):
        rows = [0, r] if 1 <= r <= 3 else [0]
        q = c.q[:, [r]]
        # one query row against the context and the rows it sees (bidirectional block)
        ref, _ = oracle.block_attention(np.repeat(q, len(rows), axis=1), c.k_blk[:, rows],
                                        c.v_blk[:, rows], c.cache_k, c.cache_v, c.block_table,
                                        c.ctx_lens, "f32")
        np.testing.assert_allclose(out[0, r], ref[0, 0], rtol=0, atol=1e-12)


# ------------------------------------------------------------ KV recycling

def test_commit_tree_kv_hand_example():
    """Tree of 5 nodes, the walk accepted nodes 1 then 3 (accept_len 2): the
    root and tree rows 2 and 4 land at positions prefix .. prefix + 2, in that
    order; nothing else is written; a request with accept_len -1 commits
    nothing; an unmapped page is skipped."""
    Hkv, D, R = 1, 2, 6
    kt = np.zeros((2, R, Hkv, D), dtype=np.float32)
    for r in range(R):
        kt[:, r] = 10 * np.arange(2)[:, None, None] + r
    vt = -kt
    ck = np.full((4, Hkv, 16, D), 7e3, dtype=np.float32)     # head-major pages
    cv = ck.copy()
    bt = np.array([[2, 0], [1, -1]], dtype=np.int32)       # request 1's second page unmapped
    acc_nodes = np.array([[1, 3, -1], [0, 1, 2]])
    written = oracle.commit_tree_kv(kt, vt, acc_nodes, [2, -1], [14, 3], ck, cv, bt)
    # request 0: positions 14, 15 on page 2, position 16 on page 0 slot 0
    assert ck[2, 0, 14, 0] == 0 and ck[2, 0, 15, 0] == 2 and ck[0, 0, 0, 0] == 4
    assert cv[0, 0, 0, 0] == -4
    assert written.sum() == 3
    assert np.all(ck[1] == 7e3) and np.all(ck[3] == 7e3)
