"""Pins for the block-attention oracle: brute force with explicit masks, a
library routine (torch CPU float64 scaled-dot-product attention), closed forms
and invariances."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _case(seed, B=3, k=4, Hq=4, Hkv=2, D=8, ctx=(0, 5, 19), dtype="f32", **kw):
    return synth.attention_case(seed, dtype=dtype, B=B, k=k, n_q_heads=Hq, n_kv_heads=Hkv,
                                head_dim=D, ctx_lens=list(ctx), **kw)


def _run(c, fn=oracle.block_attention, scale=None):
    return fn(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v, c.block_table, c.ctx_lens, c.dtype,
              scale=scale)


@pytest.mark.parametrize("seed,ctx", [(1, (0, 5, 19)), (2, (8, 1, 33)), (3, (16, 16, 0))])
def test_gather_form_equals_explicit_mask_brute_force(seed, ctx):
    c = _case(seed, ctx=ctx)
    o1, l1 = _run(c)
    o2, l2 = _run(c, oracle.block_attention_masked)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_bf16_gather_equals_brute_force():
    c = _case(4, B=2, k=8, Hq=4, Hkv=2, D=16, ctx=(7, 40), dtype="bf16", q_scale=3.0)
    o1, l1 = _run(c)
    o2, l2 = _run(c, oracle.block_attention_masked)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_float64_with_bool_mask():
    """Library routine: torch CPU float64 SDPA over each request's keys with
    an explicit bool mask (all True: the block is non-causal)."""
    c = _case(5, B=2, k=4, Hq=6, Hkv=2, D=16, ctx=(9, 23))
    out, lse = _run(c)
    q = oracle.widen(c.q, "f32")
    for b in range(c.B):
        C = int(c.ctx_lens[b])
        keys = np.concatenate([oracle.gather_paged(oracle.widen(c.cache_k, "f32"),
                                                   c.block_table[b], C),
                               oracle.widen(c.k_blk, "f32")[b]])
        vals = np.concatenate([oracle.gather_paged(oracle.widen(c.cache_v, "f32"),
                                                   c.block_table[b], C),
                               oracle.widen(c.v_blk, "f32")[b]])
        G = c.n_q_heads // c.n_kv_heads
        for h in range(c.n_q_heads):
            qt = torch.from_numpy(q[b, :, h, :])[None, None]
            kt = torch.from_numpy(keys[:, h // G, :])[None, None]
            vt = torch.from_numpy(vals[:, h // G, :])[None, None]
            mask = torch.ones(c.k, C + c.k, dtype=torch.bool)
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
            np.testing.assert_allclose(out[b, :, h, :], ref[0, 0].numpy(), atol=1e-12)


def test_closed_form_single_key_returns_value():
    """C = 0 and k = 1: the only visible key is the query's own, so o = v."""
    c = _case(6, B=2, k=1, ctx=(0, 0))
    out, lse = _run(c)
    v = oracle.widen(c.v_blk, "f32")
    G = c.n_q_heads // c.n_kv_heads
    for h in range(c.n_q_heads):
        np.testing.assert_allclose(out[:, 0, h], v[:, 0, h // G], atol=1e-15)


def test_closed_form_zero_query_is_mean_of_values():
    c = _case(7, ctx=(3, 0, 21))
    c.q[:] = 0
    out, lse = _run(c)
    v = oracle.widen(c.v_blk, "f32"); cv = oracle.widen(c.cache_v, "f32")
    G = c.n_q_heads // c.n_kv_heads
    for b in range(c.B):
        C = int(c.ctx_lens[b])
        vals = np.concatenate([oracle.gather_paged(cv, c.block_table[b], C), v[b]])
        for h in range(c.n_q_heads):
            np.testing.assert_allclose(out[b, :, h], np.broadcast_to(vals[:, h // G].mean(0),
                                                                     (c.k, c.head_dim)),
                                       atol=1e-14)
            np.testing.assert_allclose(lse[b, h], np.log(C + c.k), atol=1e-14)


def test_identical_keys_give_mean_of_values():
    c = _case(8, ctx=(5, 12, 2))
    key = oracle.slots(c.cache_k)[0, 0].copy()        # [Hkv, D]: page 0, position 0
    c.cache_k[:] = key[None, :, None, :]               # every position of every page
    c.k_blk[:] = key[None, None]
    out, _ = _run(c)
    v = oracle.widen(c.v_blk, "f32"); cv = oracle.widen(c.cache_v, "f32")
    G = c.n_q_heads // c.n_kv_heads
    for b in range(c.B):
        vals = np.concatenate([oracle.gather_paged(cv, c.block_table[b], int(c.ctx_lens[b])),
                               v[b]])
        for h in range(c.n_q_heads):
            np.testing.assert_allclose(out[b, :, h], np.broadcast_to(vals[:, h // G].mean(0),
                                                                     (c.k, c.head_dim)),
                                       atol=1e-12)


def test_invariant_to_physical_page_order():
    a = _case(9, ctx=(40, 17, 33), shuffle=False)
    b = _case(9, ctx=(40, 17, 33), shuffle=True)
    # same logical contents, different physical placement
    for bb in range(a.B):
        for lp in range(a.block_table.shape[1]):
            pa, pb = a.block_table[bb, lp], b.block_table[bb, lp]
            if pa >= 0:
                b.cache_k[pb] = a.cache_k[pa]
                b.cache_v[pb] = a.cache_v[pa]
    oa, la = _run(a)
    ob, lb = _run(b)
    np.testing.assert_allclose(oa, ob, atol=1e-14)
    np.testing.assert_allclose(la, lb, atol=1e-14)


def test_scale_argument():
    c = _case(10)
    o1, l1 = _run(c, scale=0.25)
    o2, l2 = _run(c, oracle.block_attention_masked, scale=0.25)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    o3, _ = _run(c, scale=0.0)
    o4, _ = _run(c)
    np.testing.assert_allclose(o3, o4, atol=0)


def test_packed_training_mask_equals_dense_sequence_mask():
    """[DFlash overview] 随机锚点采样: blocks packed into one training sequence
    see the injected context of target positions before their anchor, all of
    their own positions, and nothing of the other blocks.  Written here as one
    dense mask over [context positions ; all block positions]."""
    seq, k, Hq, Hkv, D = 96, 4, 2, 1, 8
    c, P = synth.packed_attention_case(77, dtype="f32", seq_len=seq, k=k, n_q_heads=Hq,
                                       n_kv_heads=Hkv, head_dim=D, max_anchors=9,
                                       prompt_range=(20, 30))
    nb = c.B
    out, _ = _run(c)
    q = oracle.widen(c.q, "f32"); kb = oracle.widen(c.k_blk, "f32"); vb = oracle.widen(c.v_blk, "f32")
    ck = oracle.gather_paged(oracle.widen(c.cache_k, "f32"), c.block_table[0], seq)
    cv = oracle.gather_paged(oracle.widen(c.cache_v, "f32"), c.block_table[0], seq)
    keys = np.concatenate([ck, kb.reshape(nb * k, Hkv, D)])
    vals = np.concatenate([cv, vb.reshape(nb * k, Hkv, D)])
    mask = np.zeros((nb * k, seq + nb * k), dtype=bool)
    for i, a in enumerate(c.ctx_lens):
        mask[i * k:(i + 1) * k, :a] = True                               # context before anchor
        mask[i * k:(i + 1) * k, seq + i * k: seq + (i + 1) * k] = True    # own block
    for h in range(Hq):
        qq = torch.from_numpy(q[:, :, h, :].reshape(nb * k, D))[None, None]
        kk = torch.from_numpy(keys[:, 0, :])[None, None]
        vv = torch.from_numpy(vals[:, 0, :])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=torch.from_numpy(mask)[None, None])
        np.testing.assert_allclose(out[:, :, h, :].reshape(nb * k, D), ref[0, 0].numpy(),
                                   atol=1e-12)
    # anchors are disjoint blocks in the loss region
    a = np.sort(c.ctx_lens)
    assert (np.diff(a) >= k).all() and a[0] >= P and a[-1] + k <= seq


# --- causal block (block position i sees block positions 0..i) -------------

@pytest.mark.parametrize("seed,ctx", [(21, (0, 5, 19)), (22, (8, 1, 33)), (23, (16, 0, 3))])
def test_causal_gather_form_equals_explicit_mask_brute_force(seed, ctx):
    c = _case(seed, ctx=ctx)
    o1, l1 = _run_causal(c)
    o2, l2 = _run_causal(c, oracle.block_attention_masked)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def _run_causal(c, fn=oracle.block_attention):
    return fn(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v, c.block_table, c.ctx_lens, c.dtype,
              causal=True)


def test_causal_matches_torch_sdpa_float64():
    """Library routine: torch CPU float64 SDPA -- is_causal=True over the block
    alone when C = 0, and an explicit [context | lower-triangular] bool mask
    when C > 0."""
    c = _case(24, B=2, k=6, Hq=4, Hkv=2, D=16, ctx=(0, 13))
    out, lse = _run_causal(c)
    q = oracle.widen(c.q, "f32")
    G = c.n_q_heads // c.n_kv_heads
    for b in range(c.B):
        C = int(c.ctx_lens[b])
        keys = np.concatenate([oracle.gather_paged(oracle.widen(c.cache_k, "f32"),
                                                   c.block_table[b], C),
                               oracle.widen(c.k_blk, "f32")[b]])
        vals = np.concatenate([oracle.gather_paged(oracle.widen(c.cache_v, "f32"),
                                                   c.block_table[b], C),
                               oracle.widen(c.v_blk, "f32")[b]])
        for h in range(c.n_q_heads):
            qt = torch.from_numpy(q[b, :, h, :])[None, None]
            kt = torch.from_numpy(keys[:, h // G, :])[None, None]
            vt = torch.from_numpy(vals[:, h // G, :])[None, None]
            if C == 0:
                ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
            else:
                mask = torch.cat([torch.ones(c.k, C, dtype=torch.bool),
                                  torch.tril(torch.ones(c.k, c.k, dtype=torch.bool))], dim=1)
                ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
            np.testing.assert_allclose(out[b, :, h, :], ref[0, 0].numpy(), atol=1e-12)


def test_causal_closed_forms():
    """With no context, block position 0 sees only its own key: o = v_blk[0]
    exactly.  The last block position sees the whole block, so its row equals
    the bidirectional result; with k = 1 the two modes coincide."""
    c = _case(25, B=2, k=5, Hq=4, Hkv=2, D=8, ctx=(0, 0))
    out, _ = _run_causal(c)
    vb = oracle.widen(c.v_blk, "f32")
    for h in range(c.n_q_heads):
        np.testing.assert_array_equal(out[:, 0, h, :], vb[:, 0, h // 2, :])
    c = _case(26, B=3, k=5, Hq=4, Hkv=2, D=8, ctx=(0, 7, 21))
    oc, lc = _run_causal(c)
    ob, lb = _run(c)
    np.testing.assert_allclose(oc[:, -1], ob[:, -1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lc[:, :, -1], lb[:, :, -1], rtol=0, atol=1e-12)
    c = _case(27, B=2, k=1, Hq=2, Hkv=1, D=8, ctx=(3, 9))
    np.testing.assert_allclose(_run_causal(c)[0], _run(c)[0], rtol=0, atol=1e-12)


# --- split-context merge and logical-position permutation -------------------

def test_split_context_lse_merge_equals_unsplit():
    """Splitting the keys into parts and merging the parts' outputs by their
    log-sum-exp reproduces the unsplit attention: with S(A) = exp(lse_A) and
    N(A) = O_A * S(A), S and N are additive over disjoint key sets.  The
    three runs below see A = ctx[0, 16) + block, B = ctx[16, C) + block and
    the block alone, so S(all) = S(A) + S(B) - S(block) and likewise N.  This
    checks the exported lse as well as the output."""
    c = _case(31, B=2, k=4, Hq=4, Hkv=2, D=8, ctx=(40, 37))
    full_o, full_l = _run(c)

    def with_ctx(lens, table):
        return oracle.block_attention(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v, table,
                                      np.asarray(lens), c.dtype)

    oA, lA = with_ctx([16, 16], c.block_table)
    shifted = np.full_like(c.block_table, -1)
    shifted[:, :-1] = c.block_table[:, 1:]                 # logical page p+1 becomes page p
    oB, lB = with_ctx(c.ctx_lens - 16, shifted)
    o0, l0 = with_ctx([0, 0], c.block_table)
    sA, sB, s0 = (np.exp(l)[..., None] for l in (lA, lB, l0))          # [B, Hq, k, 1]
    to_bhk = lambda o: np.transpose(o, (0, 2, 1, 3))                  # [B, Hq, k, D]
    S = sA + sB - s0
    N = to_bhk(oA) * sA + to_bhk(oB) * sB - to_bhk(o0) * s0
    np.testing.assert_allclose(np.log(S[..., 0]), full_l, rtol=0, atol=1e-12)
    np.testing.assert_allclose(N / S, to_bhk(full_o), rtol=0, atol=1e-12)


def test_invariant_to_permutation_of_context_positions():
    """Attention without positions inside is a set function of the visible
    (key, value) pairs: permuting which logical context position holds which
    pair leaves every output unchanged (only the summation order moves)."""
    c = _case(32, B=3, k=4, Hq=4, Hkv=2, D=8, ctx=(40, 17, 33))
    o1, l1 = _run(c)
    rng = np.random.default_rng(33)
    ck, cv = oracle.slots(c.cache_k.copy()), oracle.slots(c.cache_v.copy())
    new_k, new_v = c.cache_k.copy(), c.cache_v.copy()
    nk, nv = oracle.slots(new_k), oracle.slots(new_v)
    for b in range(c.B):
        C = int(c.ctx_lens[b])
        perm = rng.permutation(C)
        for dst, src in enumerate(perm):
            pd, ps = c.block_table[b, dst // 16], c.block_table[b, src // 16]
            nk[pd, dst % 16] = ck[ps, src % 16]
            nv[pd, dst % 16] = cv[ps, src % 16]
    o2, l2 = oracle.block_attention(c.q, c.k_blk, c.v_blk, new_k, new_v, c.block_table,
                                    c.ctx_lens, c.dtype)
    assert not np.array_equal(new_k, c.cache_k)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-13)


# --- BD3-LM block-causal mask ([Spec tutorial] 5.3) --------------------------

def block_causal_case(seed, dtype="f32", n_blocks=3, k=3, Hq=4, Hkv=2, D=8):
    """The page's block-causal figure as block attention: block j is one
    request whose context is the K/V of blocks 0..j-1, stored in a paged cache
    at logical positions 0..3j-1 (one page table shared by all blocks), and
    whose own k rows are its block.  Returns (case, dense q/k/v [n*k, H, D] in
    float64 for the explicit-mask reference)."""
    rng = synth.make_rng(seed)
    n = n_blocks * k
    q = synth._draw(rng, (n_blocks, k, Hq, D), 1.0, dtype)
    kk = synth._draw(rng, (n_blocks, k, Hkv, D), 1.0, dtype)
    vv = synth._draw(rng, (n_blocks, k, Hkv, D), 1.0, dtype)
    num_pages = 3
    perm = rng.permutation(num_pages).astype(np.int32)
    table = np.tile(perm, (n_blocks, 1))
    ck = synth.empty_cache(num_pages, Hkv, D, dtype)
    cv = synth.empty_cache(num_pages, Hkv, D, dtype)
    sk, sv = oracle.slots(ck), oracle.slots(cv)
    for pos in range(n):
        sk[perm[pos // 16], pos % 16] = kk.reshape(n, Hkv, D)[pos]
        sv[perm[pos // 16], pos % 16] = vv.reshape(n, Hkv, D)[pos]
    ctx = (np.arange(n_blocks) * k).astype(np.int32)
    c = synth.AttentionCase(dtype, n_blocks, k, Hq, Hkv, D, q, kk, vv, ck, cv, table, ctx)
    dense = [oracle.widen(a, dtype).reshape(n, -1, D) for a in (q, kk, vv)]
    return c, dense


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_block_causal_figure_equals_context_plus_bidirectional_block(dtype):
    """Each row of the page's 3-block figure, evaluated by torch CPU float64
    SDPA with the figure's boolean mask over the nine positions, equals the
    bidirectional block attention of that row's block over a context holding
    the earlier blocks."""
    from tests.golden.load import block_causal_mask
    mask = torch.tensor(block_causal_mask(), dtype=torch.bool)
    assert mask.shape == (9, 9)
    c, (q, kk, vv) = block_causal_case(51, dtype)
    out, _ = _run(c)
    G = c.n_q_heads // c.n_kv_heads
    for h in range(c.n_q_heads):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h])[None, None], torch.from_numpy(kk[:, h // G])[None, None],
            torch.from_numpy(vv[:, h // G])[None, None], attn_mask=mask[None, None])[0, 0]
        np.testing.assert_allclose(out[:, :, h].reshape(9, -1), ref.numpy(), rtol=0, atol=1e-12)
    # the mask is the figure's: not causal inside a block, causal across blocks
    assert mask[0, 2] and not mask[2, 3] and mask[8, 0] and not mask[5, 6]
