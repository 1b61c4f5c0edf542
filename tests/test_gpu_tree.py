"""GPU parity: DDTree construction and greedy tree verification through the
C ABI, against the CPU oracle on the same seeded inputs.

* Top-K: tokens bit-exact (both sides select on the stored logits, ties to
  the lower id); log-probabilities within 1e-4 absolute (fp32 log-sum-exp).
* Tree: the kernel accumulates joint log-probabilities in fp32, the oracle in
  fp64, so two candidates whose scores differ by less than the accumulated
  rounding may pop in either order.  The checks therefore are: the node count;
  every node's (parent, token, depth) is a valid tree over the oracle's top-K
  lists; its score equals the oracle's path score within TOL_SCORE; the pop
  order never rises by more than TOL_TIE; no candidate left outside the tree
  beats a node inside it by more than TOL_TIE (the best-first optimality
  condition); and where no two of the oracle's candidate scores lie within
  TOL_TIE of each other the arrays must equal the oracle's exactly.
* Ancestor mask: bit-exact against a walk of the kernel's own parents, and
  against the oracle's mask where the tree is exact.
* Greedy walk: bit-exact against the oracle's walk on the same tree (the
  oracle's tree, uploaded), with the target's argmax taken by the oracle.
"""
import numpy as np
import pytest

import block_diffusion_draft_ctx_amd as dfl
import oracle
import synth
from tests.gpu_util import down, log, up

pytestmark = pytest.mark.gpu

V_QWEN = 151936
TOL_LP = 1e-4
TOL_SCORE = 2e-4
TOL_TIE = 2e-4


def _candidate_scores(tree, lp, K):
    """Scores of every popped node and of every candidate the heap still
    holds (children of popped nodes not popped, root children not popped)."""
    n_pos = lp.shape[0]
    popped = {(int(tree.parent[i]), int(tree.rank[i])) for i in range(len(tree.token))}
    s = list(tree.score)
    for r in range(K):
        if (-1, r) not in popped and lp[0, r] > -np.inf:
            s.append(lp[0, r])
    for i in range(len(tree.token)):
        d = int(tree.depth[i])
        if d >= n_pos:
            continue
        for r in range(K):
            if (i, r) not in popped and lp[d, r] > -np.inf:
                s.append(tree.score[i] + lp[d, r])
    return np.sort(np.array(s))


def _near_tie(tree, lp, K):
    """Two candidate scores closer than TOL_TIE, equal ones included: an fp64
    tie between paths through different logits (frequent with bf16 logits on
    a coarse grid, e.g. 8.5 + 7.25 = 8.25 + 7.5) is not a tie in fp32."""
    g = np.diff(_candidate_scores(tree, lp, K))
    return bool(np.any(g < TOL_TIE))


def _unpack_mask(words, budget):
    w = words.astype(np.int64) & 0xFFFFFFFF
    bits = (w[:, :, None] >> np.arange(32)) & 1
    return bits.reshape(words.shape[0], -1)[:, :budget].astype(bool)


def _check_request(b, r, tok_o, lp_o, tree_o, budget, n_pos, K, want_mask=True):
    """Returns True if the kernel's tree equals the oracle's exactly."""
    n = int(down(r["n_nodes"])[b])
    assert n == len(tree_o.token), (b, n, len(tree_o.token))
    kt = down(r["node_token"])[b]
    kp = down(r["node_parent"])[b]
    kd = down(r["node_depth"])[b]
    kl = down(r["node_logp"])[b]
    assert np.all(kt[n:] == -1) and np.all(kp[n:] == -2) and np.all(kd[n:] == 0)
    assert np.all(kl[n:] == -np.inf)
    kt, kp, kd, kl = kt[:n], kp[:n], kd[:n], kl[:n]
    osc = np.zeros(n)
    inside = set()
    for i in range(n):
        p = int(kp[i])
        assert -1 <= p < i, (b, i, p)
        d = int(kd[i])
        assert d == (1 if p < 0 else int(kd[p]) + 1) and 1 <= d <= n_pos
        hit = np.flatnonzero(tok_o[d - 1] == kt[i])
        assert len(hit) == 1, (b, i, int(kt[i]))
        osc[i] = (0.0 if p < 0 else osc[p]) + lp_o[d - 1, hit[0]]
        assert (p, int(hit[0])) not in inside      # siblings carry distinct tokens
        inside.add((p, int(hit[0])))
    assert np.abs(kl - osc).max(initial=0.0) <= TOL_SCORE
    assert np.all(np.diff(osc) <= TOL_TIE)
    # best-first optimality: nothing left out beats a node inside
    out_best = -np.inf
    for r_ in range(K):
        if (-1, r_) not in inside:
            out_best = max(out_best, lp_o[0, r_])
    for i in range(n):
        d = int(kd[i])
        if d < n_pos:
            for r_ in range(K):
                if (i, r_) not in inside:
                    out_best = max(out_best, osc[i] + lp_o[d, r_])
    if n:
        assert out_best <= osc.min() + TOL_TIE, (b, out_best, osc.min())
    exact = (np.array_equal(kt, tree_o.token) and np.array_equal(kp, tree_o.parent)
             and np.array_equal(kd, tree_o.depth))
    if not _near_tie(tree_o, lp_o, K):
        assert exact, f"request {b}: no near-tie, yet the tree differs from the oracle's"
        np.testing.assert_allclose(kl, tree_o.score, rtol=0, atol=TOL_SCORE)
    if want_mask:
        m = _unpack_mask(down(r["ancestor_mask"])[b], budget)
        want = np.zeros((budget, budget), dtype=bool)
        for i in range(n):
            j = i
            while j >= 0:
                want[i, j] = True
                j = int(kp[j])
        np.testing.assert_array_equal(m, want)
        if exact:
            np.testing.assert_array_equal(m[:n, :n], oracle.ancestor_mask(tree_o.parent))
    return exact


def _topk_check(r, tok_o, lp_o, rows=None):
    kt = down(r["topk_tokens"])
    kl = down(r["topk_logp"])
    if rows is not None:
        kt, kl = kt[rows], kl[rows]
    np.testing.assert_array_equal(kt, tok_o)
    np.testing.assert_allclose(kl, lp_o, rtol=0, atol=TOL_LP)


@pytest.mark.parametrize("dtype,B,n_pos,V,K,budget,T,peaked,seed", [
    ("f32", 2, 5, 1000, 4, 40, 1.0, 0.0, 3101),          # small: one chunk per row
    ("f32", 3, 4, 5003, 3, 64, 0.7, 4.0, 3102),          # ragged vocabulary tail
    ("bf16", 3, 7, 50257, 8, 128, 1.0, 6.0, 3103),       # several chunks per row
    ("bf16", 2, 15, V_QWEN, 16, 512, 1.0, 8.0, 3104),    # Qwen3 vocabulary, K and budget of the bench
    ("bf16", 2, 2, 4099, 3, 64, 1.0, 0.0, 3105),         # whole tree (3 + 9) below the budget
    ("bf16", 1, 3, 37, 16, 100, 1.0, 0.0, 3106),         # tiny vocabulary, scalar tail only
    ("f32", 2, 6, 16, 16, 1, 1.3, 0.0, 3107),            # K = V, budget 1
    ("bf16", 1, 64, 3000, 2, 1024, 1.0, 5.0, 3108),      # deepest block, largest budget
])
def test_tree_build_parity(dtype, B, n_pos, V, K, budget, T, peaked, seed):
    log(f"tree_build dtype={dtype} B={B} n_pos={n_pos} V={V} K={K} budget={budget} T={T} seed={seed}")
    c = synth.tree_case(seed, dtype=dtype, B=B, n_pos=n_pos, V=V, peaked=peaked)
    r = dfl.tree_build(up(c.draft_logits, dtype), K, budget, temperature=T)
    tok_o, lp_o = oracle.topk_logprobs(c.draft_logits, dtype, K, T)
    _topk_check(r, tok_o, lp_o)
    n_exact = 0
    for b in range(B):
        tree_o = oracle.build_tree(tok_o[b], lp_o[b], budget)
        n_exact += _check_request(b, r, tok_o[b], lp_o[b], tree_o, budget, n_pos, K)
    log(f"  trees equal to the oracle's: {n_exact}/{B}")


def test_tree_build_ties_and_zero_probability():
    """Equal logits (ties to the lower token id, exact in both) and tokens of
    probability zero (never nodes) on fp32 rows."""
    x = np.full((2, 3, 300), -np.inf, dtype=np.float32)
    x[:, :, :40] = np.round(synth.tree_case(3111, dtype="f32", B=2, n_pos=3, V=40).draft_logits)
    x[1, 1, 2:] = -np.inf                                   # position 2: two live tokens
    r = dfl.tree_build(up(x, "f32"), 6, 200)
    tok_o, lp_o = oracle.topk_logprobs(x, "f32", 6)
    _topk_check(r, tok_o, lp_o)
    for b in range(2):
        tree_o = oracle.build_tree(tok_o[b], lp_o[b], 200)
        _check_request(b, r, tok_o[b], lp_o[b], tree_o, 200, 3, 6)


@pytest.mark.parametrize("K,n_pos,budget,flat", [
    (2, 8, 64, 2),       # every path of a depth ties; the budget cuts a tie group
    (16, 4, 1024, 16),   # 16 equal candidates per position: the frontier outgrows the
                         # parallel build's buffers and the serial loop builds the tree
])
def test_tree_build_exact_ties(K, n_pos, budget, flat):
    """Rows whose top `flat` logits are equal (the rest of the top-K a half
    apart, everything else -inf): whole depths of the tree tie exactly, in
    fp32 as in fp64, and the pops must follow the page's order for equal
    scores (the parents' pop order, then rank) exactly as the oracle does."""
    x = np.full((2, n_pos, 64), -np.inf, dtype=np.float32)
    x[:, :, :K] = -0.5 * np.arange(K, dtype=np.float32)
    x[:, :, :flat] = 0.0
    log(f"tree_build exact ties K={K} n_pos={n_pos} budget={budget}")
    r = dfl.tree_build(up(x, "f32"), K, budget)
    tok_o, lp_o = oracle.topk_logprobs(x, "f32", K)
    for b in range(2):
        tree_o = oracle.build_tree(tok_o[b], lp_o[b], budget)
        n = int(down(r["n_nodes"])[b])
        assert n == len(tree_o.token)
        np.testing.assert_array_equal(down(r["node_parent"])[b, :n], tree_o.parent)
        np.testing.assert_array_equal(down(r["node_token"])[b, :n], tree_o.token)
        np.testing.assert_array_equal(down(r["node_depth"])[b, :n], tree_o.depth)
        np.testing.assert_allclose(down(r["node_logp"])[b, :n], tree_o.score, rtol=0, atol=TOL_SCORE)
        _check_request(b, r, tok_o[b], lp_o[b], tree_o, budget, n_pos, K)


def test_tree_build_full_size_sampled():
    """The bench's launch configuration: 64 requests, 15 block positions,
    the Qwen3 vocabulary, K = 8, budget 512; requests checked one by one on a
    sample, the rest by the structural checks that hold at any size."""
    B, n_pos, V, K, budget = 64, 15, V_QWEN, 8, 512
    log(f"tree_build full B={B} n_pos={n_pos} V={V} K={K} budget={budget}")
    c = synth.tree_case(3121, dtype="bf16", B=B, n_pos=n_pos, V=V, peaked=7.0)
    r = dfl.tree_build(up(c.draft_logits, "bf16"), K, budget)
    sample = [0, 17, 40, 63]
    tok_o, lp_o = oracle.topk_logprobs(c.draft_logits[sample], "bf16", K)
    _topk_check(r, tok_o, lp_o, rows=sample)
    for j, b in enumerate(sample):
        tree_o = oracle.build_tree(tok_o[j], lp_o[j], budget)
        _check_request(b, r, tok_o[j], lp_o[j], tree_o, budget, n_pos, K)
    # every request: a full budget, parents first, scores non-increasing
    nn = down(r["n_nodes"])
    assert np.all(nn == budget)
    par = down(r["node_parent"])
    sc = down(r["node_logp"])
    assert np.all(par < np.arange(budget)[None, :])
    assert np.all(np.diff(sc, axis=1) <= TOL_TIE)


# --------------------------------------------------------------- greedy walk

class _LazyPredict:
    """target_predict for oracle.walk_greedy, one row at a time."""

    def __init__(self, logits_b, dtype):
        self.t, self.dtype = logits_b, dtype

    def __getitem__(self, r):
        return int(oracle.target_argmax(self.t[None, r:r + 1], self.dtype)[0, 0])


def _padded(tree, budget):
    tok = np.full(budget, -1, dtype=np.int64)
    par = np.full(budget, -2, dtype=np.int64)
    n = len(tree.token)
    tok[:n], par[:n] = tree.token, tree.parent
    return tok, par


def _deepest_path(tree):
    leaf = int(np.argmax(tree.depth))
    p = []
    while leaf >= 0:
        p.append(leaf)
        leaf = int(tree.parent[leaf])
    return p[::-1]


def _walk_case(seed, dtype, B, n_pos, V, K, budget, stop_at=None):
    """Oracle trees of B requests and target logits in which request b's
    target follows the deepest path of its tree for stop_at[b] steps (all of
    it if None), so that the accepted lengths span the range."""
    c = synth.tree_case(seed, dtype=dtype, B=B, n_pos=n_pos, V=V, peaked=6.0)
    tok_o, lp_o = oracle.topk_logprobs(c.draft_logits, dtype, K)
    trees = [oracle.build_tree(tok_o[b], lp_o[b], budget) for b in range(B)]
    follow = []
    for b, t in enumerate(trees):
        path = _deepest_path(t)
        steps = len(path) if stop_at is None else min(stop_at[b], len(path))
        pairs = [(0 if j == 0 else 1 + path[j - 1], int(t.token[path[j]])) for j in range(steps)]
        follow.append(pairs)
    tl = synth.tree_target_logits(seed + 1, dtype=dtype, B=B, n_rows=budget + 1, V=V,
                                  follow=follow)
    return trees, tl


def _walk_check(r, trees, tl, dtype, max_depth, n_nodes=None, prefix=None):
    acc = down(r["accept_len"])
    bon = down(r["bonus"])
    com = down(r["commit_lens"])
    path = down(r["accepted_nodes"])
    for b, t in enumerate(trees):
        n = len(t.token) if n_nodes is None else int(n_nodes[b])
        if n < 0 or n > tl.shape[1] - 1:
            assert (acc[b], bon[b], com[b]) == (-1, -1, 0)
            continue
        w = oracle.walk_greedy(t.token[:n], t.parent[:n], _LazyPredict(tl[b], dtype),
                               max_depth=max_depth)
        assert acc[b] == w.accept_len and bon[b] == w.bonus and com[b] == w.accept_len + 1, b
        want = (w.path + [-1] * max_depth)[:max_depth]
        np.testing.assert_array_equal(path[b], want)
        if prefix is not None:
            assert down(r["new_seq_lens"])[b] == prefix[b] + w.accept_len + 1


@pytest.mark.parametrize("dtype,B,n_pos,V,K,budget,seed", [
    ("f32", 4, 5, 1000, 3, 30, 3201),
    ("bf16", 6, 7, 50257, 4, 64, 3202),
    ("bf16", 3, 15, V_QWEN, 8, 512, 3203),
    ("bf16", 2, 3, 777, 2, 5, 3204),       # ragged tail, scalar loads
])
def test_tree_verify_parity(dtype, B, n_pos, V, K, budget, seed):
    log(f"tree_verify dtype={dtype} B={B} n_pos={n_pos} V={V} K={K} budget={budget} seed={seed}")
    stop = [b % (n_pos + 1) for b in range(B)]          # 0 .. n_pos followed steps
    trees, tl = _walk_case(seed, dtype, B, n_pos, V, K, budget, stop_at=stop)
    toks = np.stack([_padded(t, budget)[0] for t in trees])
    pars = np.stack([_padded(t, budget)[1] for t in trees])
    nn = np.array([len(t.token) for t in trees])
    prefix = np.arange(B) * 7 + 3
    max_depth = n_pos
    r = dfl.tree_verify_greedy(up(tl, dtype), up(toks, "i32"), up(pars, "i32"), up(nn, "i32"),
                               max_depth, prefix_lens=up(prefix, "i32"))
    _walk_check(r, trees, tl, dtype, max_depth, prefix=prefix)
    log(f"  accept_len {down(r['accept_len']).tolist()}")


def test_tree_verify_edge_cases():
    """An empty tree (bonus only), node counts out of range (in-band error),
    and a tree whose accepted path is longer than max_depth (the walk stops
    after max_depth nodes; the bonus is the prediction at the last node
    kept)."""
    B, n_pos, V, K, budget = 4, 6, 2000, 3, 40
    trees, tl = _walk_case(3211, "bf16", B, n_pos, V, K, budget)
    toks = np.stack([_padded(t, budget)[0] for t in trees])
    pars = np.stack([_padded(t, budget)[1] for t in trees])
    nn = np.array([0, budget + 1, -3, len(trees[3].token)])
    max_depth = len(_deepest_path(trees[3])) - 1       # request 3 follows its deepest path
    assert max_depth >= 1
    r = dfl.tree_verify_greedy(up(tl, "bf16"), up(toks, "i32"), up(pars, "i32"), up(nn, "i32"),
                               max_depth)
    _walk_check(r, trees, tl, "bf16", max_depth, n_nodes=nn)
    assert down(r["accept_len"])[3] == max_depth
    assert (down(r["accepted_nodes"])[3] >= 0).all()


def test_build_then_verify_on_device():
    """The kernel's own tree feeds the kernel's walk; where the tree equals
    the oracle's, the walk must equal the oracle's walk."""
    dtype, B, n_pos, V, K, budget = "bf16", 4, 7, 32000, 4, 96
    c = synth.tree_case(3221, dtype=dtype, B=B, n_pos=n_pos, V=V, peaked=8.0)
    rb = dfl.tree_build(up(c.draft_logits, dtype), K, budget)
    tok_o, lp_o = oracle.topk_logprobs(c.draft_logits, dtype, K)
    trees = [oracle.build_tree(tok_o[b], lp_o[b], budget) for b in range(B)]
    exact = [_check_request(b, rb, tok_o[b], lp_o[b], trees[b], budget, n_pos, K)
             for b in range(B)]
    follow = []
    for t in trees:
        path = _deepest_path(t)[:5]
        follow.append([(0 if j == 0 else 1 + path[j - 1], int(t.token[path[j]]))
                       for j in range(len(path))])
    tl = synth.tree_target_logits(3222, dtype=dtype, B=B, n_rows=budget + 1, V=V, follow=follow)
    rv = dfl.tree_verify_greedy(up(tl, dtype), rb["node_token"], rb["node_parent"], rb["n_nodes"],
                                n_pos)
    keep = [b for b in range(B) if exact[b]]
    assert keep, "no request's tree came out exact"
    sub = {k: v[keep] for k, v in rv.items()}
    _walk_check(sub, [trees[b] for b in keep], tl[keep], dtype, n_pos)


# ------------------------------------------------------------ tree attention

def _pack_mask(m, budget):
    """bool [n, n] ancestor matrix of an n-node tree -> int32 bit rows
    [budget, ceil(budget / 32)] (bit j of row i: node j is i or an ancestor),
    rows past n all zero: the layout dflash_tree_build writes."""
    W = (budget + 31) // 32
    out = np.zeros((budget, W), dtype=np.uint32)
    n = m.shape[0]
    for i in range(n):
        for j in np.flatnonzero(m[i]):
            out[i, j >> 5] |= np.uint32(1) << np.uint32(j & 31)
    return out.view(np.int32)


def _oracle_trees(seed, B, n_pos, K, budget, V=64, peaked=3.0):
    c = synth.tree_case(seed, dtype="f32", B=B, n_pos=n_pos, V=V, peaked=peaked)
    tok, lp = oracle.topk_logprobs(c.draft_logits, "f32", K)
    trees = [oracle.build_tree(tok[b], lp[b], budget) for b in range(B)]
    par = np.full((B, budget), -2, dtype=np.int64)
    nn = np.zeros(B, dtype=np.int64)
    masks = np.zeros((B, budget, (budget + 31) // 32), dtype=np.int32)
    for b, t in enumerate(trees):
        n = len(t.token)
        nn[b] = n
        par[b, :n] = t.parent
        masks[b] = _pack_mask(oracle.ancestor_mask(t.parent), budget)
    return trees, par, nn, masks


def _tree_attn_check(c, par, nn, masks, out, lse, sel=None, rows=None):
    import torch
    from tests.test_gpu_attention import _subset
    if sel is not None:
        c = _subset(c, sel)
        out, lse = out[sel], lse[sel]
        par, nn = par[sel], nn[sel]
    o_ref, l_ref = oracle.tree_attention(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v,
                                         c.block_table, c.ctx_lens, par, nn, c.dtype, rows=rows)
    o_k, l_k = down(out), down(lse)
    if rows is not None:
        o_ref, o_k = o_ref[:, rows], o_k[:, rows]
        l_ref, l_k = l_ref[:, :, rows], l_k[:, :, rows]
    rms = np.sqrt(np.mean(o_ref ** 2))
    diff = np.abs(o_k - o_ref)
    if out.dtype == torch.bfloat16:
        diff = np.maximum(diff - 2.0 ** -8 * np.abs(o_ref), 0.0)   # storage rounding
    e = float(diff.max() / rms)
    el = float(np.abs(l_k - l_ref).max() / np.sqrt(np.mean(l_ref ** 2)))
    log(f"  tree attention out({out.dtype}) err {e:.2e}, lse err {el:.2e}")
    tol = {"bf16": 2e-2, "f32": 1e-4}[c.dtype]
    assert e <= tol and el <= tol


def _tree_attn_run(c, masks, out_dtype=None):
    import torch
    kind = c.dtype
    q = up(c.q, kind)
    lse = torch.empty((c.B, c.n_q_heads, c.k), dtype=torch.float32, device=q.device)
    od = {"f32": torch.float32, "bf16": torch.bfloat16, None: None}[out_dtype]
    return dfl.tree_attention(q, up(c.k_blk, kind), up(c.v_blk, kind), up(c.cache_k, kind),
                              up(c.cache_v, kind), up(c.block_table, "i32"), up(c.ctx_lens, "i32"),
                              up(masks, "i32"), lse=lse, out_dtype=od)


@pytest.mark.parametrize("dtype,B,n_pos,K,budget,Hq,Hkv,D,ctx,out_dtype,seed", [
    ("f32", 2, 5, 3, 20, 4, 2, 64, [37, 0], None, 3301),          # tiny fp32
    ("bf16", 2, 6, 4, 63, 32, 8, 128, [100, 1000], "f32", 3302),  # 64 tree rows
    ("bf16", 2, 6, 4, 63, 32, 8, 128, [100, 1000], "bf16", 3302),
    ("bf16", 1, 15, 8, 512, 32, 8, 128, [2048], "f32", 3303),     # the page's budget
    ("bf16", 2, 2, 3, 100, 16, 4, 64, [333, 17], "f32", 3304),    # 12-node trees in 100 rows
    ("bf16", 1, 64, 2, 1024, 8, 8, 64, [64], "f32", 3305),        # largest budget, deepest block
])
def test_tree_attention_parity(dtype, B, n_pos, K, budget, Hq, Hkv, D, ctx, out_dtype, seed):
    log(f"tree_attention dtype={dtype} B={B} budget={budget} heads={Hq}/{Hkv}x{D} ctx={ctx}")
    trees, par, nn, masks = _oracle_trees(seed, B, n_pos, K, budget)
    c = synth.attention_case(seed + 1, dtype=dtype, B=B, k=budget + 1, n_q_heads=Hq,
                             n_kv_heads=Hkv, head_dim=D, ctx_lens=ctx)
    out, lse = _tree_attn_run(c, masks, out_dtype)
    _tree_attn_check(c, par, nn, masks, out, lse)


def test_tree_attention_full_size_sampled():
    """64 requests, ctx 8192, 32 Q / 8 KV heads x 128, budget 512 (the
    bench's launch): sampled rows of sampled requests against the oracle,
    every output finite."""
    B, C, budget = 64, 8192, 512
    log(f"tree_attention full B={B} ctx={C} budget={budget}")
    trees, par, nn, masks = _oracle_trees(3311, B, 15, 8, budget)
    c = synth.attention_case(3312, dtype="bf16", B=B, k=budget + 1, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[C] * B)
    out, lse = _tree_attn_run(c, masks, "bf16")
    assert np.isfinite(down(out)).all()
    rows = [0, 1, 2, 3, 64, 200, 389, 511, 512]
    _tree_attn_check(c, par, nn, masks, out, lse, sel=[0, 37, 63], rows=rows)


def test_tree_attention_of_a_chain_equals_causal_block_attention_on_device():
    """The kernel's two mask modes agree where the page's definitions do: a
    one-path tree of 31 nodes is the causal block of 32 rows."""
    import torch
    R = 32
    c = synth.attention_case(3321, dtype="bf16", B=3, k=R, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[500, 0, 77])
    par = np.arange(R - 1) - 1
    m = _pack_mask(oracle.ancestor_mask(par), R - 1)
    masks = np.stack([m] * 3)
    out_t, _ = _tree_attn_run(c, masks, "f32")
    out_c, _ = dfl.block_attention(up(c.q, "bf16"), up(c.k_blk, "bf16"), up(c.v_blk, "bf16"),
                                   up(c.cache_k, "bf16"), up(c.cache_v, "bf16"),
                                   up(c.block_table, "i32"), up(c.ctx_lens, "i32"),
                                   out_dtype=torch.float32, causal=True)
    np.testing.assert_array_equal(down(out_t), down(out_c))


# ------------------------------------------------------------ KV recycling

@pytest.mark.parametrize("dtype,seed", [("bf16", 3401), ("f32", 3402)])
def test_tree_commit_kv_parity(dtype, seed):
    """The accepted paths of oracle walks (lengths 0 .. depth, one in-band
    error) committed into three layers' caches: every slot bit-exact against
    the oracle's commit, including the untouched sentinel slots and a request
    whose next page is unmapped."""
    import torch
    B, n_pos, K, budget, Hkv, D, Ld = 5, 6, 3, 40, 2, 64, 3
    trees, tl = _walk_case(seed, "f32", B, n_pos, 500, K, budget, stop_at=[0, 1, 3, 6, 6])
    walks = [oracle.walk_greedy(t.token, t.parent, _LazyPredict(tl[b], "f32"))
             for b, t in enumerate(trees)]
    md = n_pos
    acc = np.array([w.accept_len for w in walks])
    acc[4] = -1                                            # the walk's in-band error
    path = np.full((B, md), -1, dtype=np.int64)
    for b, w in enumerate(walks):
        path[b, :len(w.path)] = w.path[:md]
    rng = np.random.default_rng(seed)
    prefix = np.array([0, 14, 31, 60, 5])
    max_pages = 8
    n_pages = 40
    bt = rng.permutation(n_pages)[:B * max_pages].reshape(B, max_pages).astype(np.int32)
    bt[3, 4] = -1                                          # positions 64.. of request 3 unmapped
    kts, vts, cks, cvs, refs = [], [], [], [], []
    for l in range(Ld):
        ktree = synth.attention_case(seed + 10 + l, dtype=dtype, B=B, k=budget + 1, n_q_heads=Hkv,
                                     n_kv_heads=Hkv, head_dim=D, ctx_lens=[0] * B)
        sent = np.full((n_pages, Hkv, 16, D), 0x7FA1 if dtype == "bf16" else np.nan,
                       dtype=np.uint16 if dtype == "bf16" else np.float32)
        rk, rv = sent.copy(), sent.copy()
        oracle.commit_tree_kv(ktree.k_blk, ktree.v_blk, path, acc, prefix, rk, rv, bt)
        refs.append((rk, rv))
        kts.append(up(ktree.k_blk, dtype))
        vts.append(up(ktree.v_blk, dtype))
        cks.append(up(sent, dtype))
        cvs.append(up(sent, dtype))
    dfl.tree_commit_kv(kts, vts, cks, cvs, up(bt, "i32"), up(path, "i32"), up(acc, "i32"),
                       up(prefix, "i32"))
    from tests.gpu_util import bits
    for l in range(Ld):
        want_k = refs[l][0].view(np.uint16 if dtype == "bf16" else np.uint32)
        want_v = refs[l][1].view(np.uint16 if dtype == "bf16" else np.uint32)
        np.testing.assert_array_equal(bits(cks[l]), want_k)
        np.testing.assert_array_equal(bits(cvs[l]), want_v)
    log(f"  committed rows per request: {[int(a) + 1 if a >= 0 else 0 for a in acc]}")
