"""Pins of the drafter-layer oracle (oracle/draft.py) to facts fixed by the
mathematics: RMSNorm and SiLU closed forms, the residual identity, what a
block of one row with no context must attend to, the head through an
identity projection, and the causal mask's first row."""
import math

import numpy as np

import oracle
import synth
from oracle import draft


def test_rms_norm_closed_form_and_scale_invariance():
    x = np.array([[3.0, 4.0]])
    y = draft.rms_norm(x, np.array([1.0, 2.0]), 0.0)
    r = np.sqrt(12.5)
    np.testing.assert_allclose(y, [[3 / r, 8 / r]], rtol=1e-15)
    z = np.random.default_rng(1).standard_normal((5, 64))
    np.testing.assert_allclose(draft.rms_norm(7.5 * z, 1.0, 0.0), draft.rms_norm(z, 1.0, 0.0), rtol=1e-13)
    # unit RMS
    np.testing.assert_allclose(np.sqrt(np.mean(draft.rms_norm(z, 1.0, 0.0) ** 2, axis=-1)), 1.0, rtol=1e-13)


def test_silu_closed_forms():
    x = np.linspace(-8, 8, 33)
    np.testing.assert_allclose(draft.silu(x) - draft.silu(-x), x, atol=1e-14)
    assert draft.silu(0.0) == 0.0
    np.testing.assert_allclose(draft.silu(np.array([40.0])), [40.0], rtol=1e-15)


def _layer_case(seed, d=32, Hq=4, Hkv=2, D=8, I=16, B=2, k=3, ctx=(5, 0)):
    rng = np.random.default_rng(seed)
    f = lambda *s, sd=0.3: rng.standard_normal(s) * sd
    w = {"ln1": 1 + f(d, sd=0.1), "qkv": f((Hq + 2 * Hkv) * D, d), "q_norm": 1 + f(D, sd=0.1),
         "k_norm": 1 + f(D, sd=0.1), "o": f(d, Hq * D), "ln2": 1 + f(d, sd=0.1),
         "gate_up": f(2 * I, d), "down": f(d, I)}
    c = synth.attention_case(seed, dtype="f32", B=B, k=k, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                             ctx_lens=list(ctx))
    x = f(B * k, d, sd=1.0)
    return x, w, c


def _run(x, w, c, k, **kw):
    return draft.draft_layer(x, w, c.cache_k.astype(np.float64), c.cache_v.astype(np.float64),
                             c.block_table, c.ctx_lens, k=k, n_q_heads=c.n_q_heads,
                             n_kv_heads=c.n_kv_heads, head_dim=c.head_dim, dtype="f64", **kw)


def test_zero_output_projections_leave_the_residual_stream():
    x, w, c = _layer_case(11)
    w["o"] = np.zeros_like(w["o"])
    w["down"] = np.zeros_like(w["down"])
    np.testing.assert_array_equal(_run(x, w, c, 3), x)


def test_a_lone_row_without_context_attends_to_itself_only():
    """k = 1, no context: the softmax has one key, so the attention output is
    the row's own v whatever q and k are: changing W_q, W_k and their norms
    changes nothing, changing W_v does."""
    x, w, c = _layer_case(12, B=2, k=1, ctx=(0, 0))
    base = _run(x, w, c, 1)
    w2 = dict(w)
    qkv = w["qkv"].copy()
    qkv[:(4 + 2) * 8] = np.random.default_rng(5).standard_normal(((4 + 2) * 8, 32))   # q and k rows
    w2["qkv"], w2["q_norm"], w2["k_norm"] = qkv, w["q_norm"] * 3, None
    np.testing.assert_allclose(_run(x, w2, c, 1), base, rtol=0, atol=1e-12)
    w3 = dict(w)
    qkv = w["qkv"].copy()
    qkv[(4 + 2) * 8:] *= 2.0                                                       # v rows
    w3["qkv"] = qkv
    assert np.abs(_run(x, w3, c, 1) - base).max() > 1e-3


def test_causal_first_row_sees_only_itself_and_the_context():
    """Under the causal block mask row 0 of a 3-row block equals the same row
    run as a block of one."""
    x, w, c = _layer_case(13, B=1, k=3, ctx=(6,))
    full = _run(x, w, c, 3, causal=True)
    c1 = synth.AttentionCase(c.dtype, 1, 1, c.n_q_heads, c.n_kv_heads, c.head_dim, c.q[:, :1],
                             c.k_blk[:, :1], c.v_blk[:, :1], c.cache_k, c.cache_v, c.block_table,
                             c.ctx_lens)
    one = _run(x[:1], w, c1, 1)
    np.testing.assert_allclose(full[0], one[0], rtol=0, atol=1e-12)


def test_head_through_an_identity_projection_is_the_final_norm():
    x = np.random.default_rng(14).standard_normal((6, 16))
    wn = 1 + 0.1 * np.random.default_rng(15).standard_normal(16)
    got = draft.draft_head(x, wn, np.eye(16), "f64")
    np.testing.assert_allclose(got, draft.rms_norm(x, wn, 1e-6), rtol=1e-14)


def test_embed_gathers_rows():
    table = np.arange(40, dtype=np.float32).reshape(10, 4)
    out = draft.embed(table, np.array([[3, 9], [0, 3]]), "f32")
    np.testing.assert_array_equal(out, table[[3, 9, 0, 3]])


def _tiny_cache(n_pages=1, D=2, keys=(), values=()):
    """A float64 paged cache of one kv-head with the given keys/values at
    logical positions 0.. (page i of the table is physical page i)."""
    ck = np.zeros((n_pages, 1, 16, D)); cv = np.zeros((n_pages, 1, 16, D))
    for pos, (kk, vv) in enumerate(zip(keys, values)):
        ck[pos // 16, 0, pos % 16] = kk
        cv[pos // 16, 0, pos % 16] = vv
    return ck, cv


def test_hand_computed_layer_mlp_order_and_second_norm():
    """One row, no context (the attention output is the row's own v), d = 4,
    one head of D = 2, d_ff = 2, no q/k norms, no rotation, eps = 0; every
    value below is worked out by hand from the layer's definition:
      x  = (1, -1, 1, -1), ln1 = 1          -> n1 = x (unit RMS)
      v  = (n1_0, n1_1) = (1, -1)            -> x1 = x + O v = (2, -2, 2, -2)
      ln2 = (1, 2, 1, 1)                    -> n2 = x1 / 2 * ln2 = (1, -2, 1, -1)
      gate = (n2_0, n2_1) = (1, -2), up = (n2_2, n2_3) = (1, -1)
      h  = silu(gate) * up = (1 / (1 + e^-1), 2 / (1 + e^2))
      x2 = x1 + (h_0, h_1, h_0 + h_1, 0)
    Planted mistakes that this fails on (each checked by hand): gate and up
    rows swapped, or SiLU applied to up instead of gate (h_1 becomes
    2 / (1 + e)); ln2 left out, applied before the RMS division, or ln1 used
    in its place; the second residual add dropped."""
    x = np.array([[1.0, -1.0, 1.0, -1.0]])
    I4 = np.eye(4)
    w = {"ln1": np.ones(4),
         "qkv": np.vstack([np.zeros((4, 4)), I4[:2]]),          # q, k rows zero; v = n1[:2]
         "q_norm": None, "k_norm": None,
         "o": np.array([[1.0, 0], [0, 1], [1, 0], [0, 1]]),
         "ln2": np.array([1.0, 2.0, 1.0, 1.0]),
         "gate_up": I4.copy(),                                   # gate rows first, then up rows
         "down": np.array([[1.0, 0], [0, 1], [1, 1], [0, 0]])}
    ck, cv = _tiny_cache()
    got = draft.draft_layer(x, w, ck, cv, np.zeros((1, 1), np.int32), np.array([0]), k=1,
                            n_q_heads=1, n_kv_heads=1, head_dim=2, dtype="f64", eps=0.0,
                            rope_theta=0.0)
    h0 = 1.0 / (1.0 + math.exp(-1.0))
    h1 = 2.0 / (1.0 + math.exp(2.0))
    want = [2.0 + h0, -2.0 + h1, 2.0 + h0 + h1, -2.0]
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-15)


def test_block_rows_sit_after_the_context_positions():
    """Rotary positions of the block: with a context of one key at position 0,
    block row i must be rotated to position 1 + i (ctx_len + i).  D = 2 has a
    single rotation pair turning by the position itself (radians), so q_i =
    2 (cos t_i, sin t_i), k_i = (cos t_i, sin t_i) with t_i = 1 + i, and the
    context key (1, 0) is given already positioned.  The context value is
    (1, 0) and the block values are zero, so the attention output's first
    entry is the context key's softmax weight, written out here:
      row 0: e^{r cos 1} / (2 e^{r cos 1} + e^{r}),
      row 1: e^{r cos 2} / (e^{r cos 2} + e^{r cos 1} + e^{r}),   r = 2 / sqrt(2).
    Taking positions i (no context offset) or ctx_len for every row fails."""
    x = np.array([[1.0, -1.0, 1.0, -1.0], [1.0, -1.0, 1.0, -1.0]])
    qkv = np.zeros((6, 4)); qkv[0, 0] = 2.0; qkv[2, 0] = 1.0     # q = (2, 0), k = (1, 0), v = 0
    w = {"ln1": np.ones(4), "qkv": qkv, "q_norm": None, "k_norm": None,
         "o": np.array([[1.0, 0], [0, 0], [0, 0], [0, 0]]), "ln2": np.ones(4),
         "gate_up": np.zeros((4, 4)), "down": np.zeros((4, 2))}
    ck, cv = _tiny_cache(keys=[(1.0, 0.0)], values=[(1.0, 0.0)])
    got = draft.draft_layer(x, w, ck, cv, np.zeros((1, 1), np.int32), np.array([1]), k=2,
                            n_q_heads=1, n_kv_heads=1, head_dim=2, dtype="f64", eps=0.0,
                            rope_theta=10000.0)
    r = math.sqrt(2.0)
    e = lambda a: math.exp(r * math.cos(a))
    a0 = e(1) / (2 * e(1) + math.exp(r))
    a1 = e(2) / (e(2) + e(1) + math.exp(r))
    np.testing.assert_allclose(got[:, 0], [1.0 + a0, 1.0 + a1], rtol=0, atol=1e-14)
    np.testing.assert_allclose(got[:, 1:], x[:, 1:], rtol=0, atol=0)


def test_unrounded_layer_is_the_rounded_one_in_float64():
    """With dtype f64 the storage points round nothing, so the layer with
    and without storage rounding agree exactly; in bf16 they differ by the
    rounding only (a few bf16 units relative to the output's RMS)."""
    x, w, c = _layer_case(16)
    a = _run(x, w, c, 3)
    b = draft.draft_layer(x, w, c.cache_k.astype(np.float64), c.cache_v.astype(np.float64),
                          c.block_table, c.ctx_lens, k=3, n_q_heads=c.n_q_heads,
                          n_kv_heads=c.n_kv_heads, head_dim=c.head_dim, dtype="f64",
                          storage_rounding=False)
    np.testing.assert_array_equal(a, b)
