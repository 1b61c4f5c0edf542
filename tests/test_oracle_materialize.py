"""Pins for the materialisation oracle: special cases with exact answers,
linearity in the bias, a hand example, the paged commit-masked write, and
the bf16 rounding routine against the hardware float32 round trip."""
import numpy as np
import pytest

import oracle
import synth


def test_round_to_bf16_matches_float32_bit_truncation_rule():
    """bf16 rounding of values that are exact float32 numbers equals the
    round-to-nearest-even of the float32's upper 16 bits (independent
    integer route)."""
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10 ** rng.uniform(-3, 3, 100000)).astype(np.float32)
    # include exact halfway points with both parities
    x[:4] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2.0 + 2 ** -7],
                     dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    hi = u >> 16
    up = (lower > 0x8000) | ((lower == 0x8000) & ((hi & 1) == 1))
    ref = ((hi + up) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = oracle.round_to_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    assert got[0] == 1.0 and got[1] == 1 + 2 ** -6 and got[2] == -1.0


def test_identity_weights_reproduce_hidden():
    """m = 1, W_f = I, b_f = 0, W_K = [I], W_V = 2 I: K = H and V = 2 H exactly."""
    T, d = 12, 8
    H = np.random.default_rng(1).standard_normal((T, d)).astype(np.float32)
    res = oracle.materialize([H], np.eye(d, dtype=np.float32), None, [np.eye(d, dtype=np.float32)],
                             [2 * np.eye(d, dtype=np.float32)], n_kv_heads=2, head_dim=4,
                             dtype="f32")
    np.testing.assert_array_equal(res["K"][0].reshape(T, d), H.astype(np.float64))
    np.testing.assert_array_equal(res["V"][0].reshape(T, d), 2 * H.astype(np.float64))


def test_selector_weights_pick_a_layer_in_concat_order():
    """W_f that selects the j-th hidden's block returns hidden j: the concat
    order is the order the hiddens are supplied in."""
    rng = np.random.default_rng(2)
    T, d, m = 5, 4, 3
    hs = [rng.standard_normal((T, d)) for _ in range(m)]
    for j in range(m):
        W = np.zeros((d, m * d)); W[:, j * d:(j + 1) * d] = np.eye(d)
        np.testing.assert_array_equal(oracle.fuse_hiddens(hs, W), hs[j])


def test_hand_example():
    h1 = np.array([[1.0, 2.0]]); h2 = np.array([[3.0, 4.0]])
    W_f = np.array([[1.0, 0, 0, 0], [0, 0, 0, 1.0]])
    b_f = np.array([0.5, -1.0])
    res = oracle.materialize([h1, h2], W_f, b_f, [np.array([[1.0, 1.0]])],
                             [np.array([[2.0, -1.0]])], n_kv_heads=1, head_dim=1, dtype="f64")
    assert res["h_ctx"].tolist() == [[1.5, 3.0]]
    assert res["K"][0].ravel().tolist() == [4.5]
    assert res["V"][0].ravel().tolist() == [0.0]


def test_bias_linearity_and_zero_hidden():
    c = synth.materialize_case(5, dtype="f32", m=3, d_model=16, n_layers=2, n_kv_heads=2,
                               head_dim=4, n_seq=2, rows_per_seq=3)
    hid = [oracle.widen(h, "f32") for h in c.hiddens]
    Wf, bf = oracle.widen(c.W_f, "f32"), oracle.widen(c.b_f, "f32")
    Wk = oracle.widen(c.W_K[1], "f32")
    with_b = oracle.project_kv(oracle.fuse_hiddens(hid, Wf, bf), Wk, 2, 4)
    no_b = oracle.project_kv(oracle.fuse_hiddens(hid, Wf, None), Wk, 2, 4)
    np.testing.assert_allclose(with_b - no_b, np.broadcast_to((bf @ Wk.T).reshape(2, 4),
                                                              with_b.shape), atol=1e-13)
    zero = oracle.project_kv(oracle.fuse_hiddens([0 * h for h in hid], Wf, bf), Wk, 2, 4)
    np.testing.assert_allclose(zero, np.broadcast_to((bf @ Wk.T).reshape(2, 4), zero.shape),
                               atol=1e-15)


def test_bf16_outputs_lie_on_grid():
    c = synth.materialize_case(6, dtype="bf16", m=2, d_model=32, n_layers=1, n_kv_heads=1,
                               head_dim=8, n_seq=1, rows_per_seq=4)
    res = oracle.materialize(c.hiddens, c.W_f, c.b_f, c.W_K, c.W_V, 1, 8, "bf16")
    for a in (res["h_ctx"], res["K"][0], res["V"][0]):
        np.testing.assert_array_equal(oracle.round_to_bf16(a), a)


def test_paged_commit_masked_write_and_gather():
    c = synth.materialize_case(7, dtype="f32", m=2, d_model=8, n_layers=1, n_kv_heads=2,
                               head_dim=4, n_seq=3, rows_per_seq=5, start_pos=[0, 14, 30],
                               commit=[5, 2, 0])
    res = oracle.materialize(c.hiddens, c.W_f, c.b_f, c.W_K, c.W_V, 2, 4, "f32")
    cache = oracle.widen(c.cache_k[0], "f32")
    before = oracle.slots(c.cache_k[0].view(np.uint32).copy())
    written = oracle.paged_write(cache, res["K"][0], c.block_table, 5, c.seq_start_pos,
                                 c.commit_lens)
    assert written.sum() == 5 + 2 + 0
    # committed rows read back at their logical positions
    for s, n in enumerate([5, 2, 0]):
        start = int(c.seq_start_pos[s])
        got = oracle.gather_paged(cache, c.block_table[s], start + n)[start:]
        np.testing.assert_array_equal(got, res["K"][0][s * 5: s * 5 + n])
    # untouched slots keep the sentinel bits
    after = oracle.slots(cache.astype(np.float32).view(np.uint32))
    np.testing.assert_array_equal(after[~written], before[~written])


def test_unmapped_page_is_skipped():
    c = synth.materialize_case(8, dtype="f32", m=1, d_model=4, n_layers=1, n_kv_heads=1,
                               head_dim=4, n_seq=1, rows_per_seq=20, start_pos=[0])
    bt = c.block_table.copy(); bt[0, 1] = -1     # positions 16..19 unmapped
    res = oracle.materialize(c.hiddens, c.W_f, c.b_f, c.W_K, c.W_V, 1, 4, "f32")
    cache = oracle.widen(c.cache_k[0], "f32")
    w = oracle.paged_write(cache, res["K"][0], bt, 20, c.seq_start_pos, None)
    assert w.sum() == 16


# --- K epilogue: per-head RMSNorm, then the rotary embedding ----------------

def test_k_epilogue_hand_example():
    """One head, D = 4, k = (3, 4, 0, 0), w = (1, 2, 3, 4), eps = 0, position
    1, theta = 10000.  By hand: mean(k^2) = 25/4, so the norm divides by 2.5
    and scales by w: (1.2, 3.2, 0, 0).  Pairs are (0, 2) at frequency
    10000^0 = 1 and (1, 3) at 10000^(-1/2) = 0.01; at position 1 the angles are
    1 and 0.01 rad, and (x, 0) rotates to (x cos a, x sin a)."""
    import math
    k = np.array([[[3.0, 4.0, 0.0, 0.0]]])
    out = oracle.rope_half_split(oracle.k_norm(k, np.array([1.0, 2.0, 3.0, 4.0]), 0.0),
                                 np.array([1]), 10000.0)
    want = [1.2 * math.cos(1.0), 3.2 * math.cos(0.01), 1.2 * math.sin(1.0), 3.2 * math.sin(0.01)]
    np.testing.assert_allclose(out[0, 0], want, rtol=0, atol=1e-15)


def test_k_norm_unit_weight_gives_unit_rms():
    """With w = 1 and eps = 0 every head has mean square exactly 1; eps > 0
    gives ms / (ms + eps)."""
    rng = np.random.default_rng(40)
    K = rng.standard_normal((7, 3, 16)) * rng.uniform(0.1, 10, (7, 3, 1))
    out = oracle.k_norm(K, np.ones(16), 0.0)
    np.testing.assert_allclose(np.mean(out ** 2, axis=-1), 1.0, rtol=0, atol=1e-14)
    ms = np.mean(K ** 2, axis=-1)
    out = oracle.k_norm(K, np.ones(16), 0.5)
    np.testing.assert_allclose(np.mean(out ** 2, axis=-1), ms / (ms + 0.5), rtol=1e-13)


def test_rope_identity_at_zero_norm_preserving_and_relative():
    """Position 0 is the identity; every (i, i + D/2) pair keeps its length;
    the dot product of two rotated vectors depends only on the difference
    of their positions (shifting both positions by s changes nothing)."""
    rng = np.random.default_rng(41)
    D = 32
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    np.testing.assert_array_equal(oracle.rope_half_split(k, np.array([0]), 1e4), k)
    r = oracle.rope_half_split(k, np.array([777]), 1e4)
    np.testing.assert_allclose(r[..., :D // 2] ** 2 + r[..., D // 2:] ** 2,
                               k[..., :D // 2] ** 2 + k[..., D // 2:] ** 2, rtol=1e-13)
    for m, n, sft in [(5, 2, 11), (100, 3000, 257), (0, 31, 1000)]:
        a = np.sum(oracle.rope_half_split(q, np.array([m]), 1e4) *
                   oracle.rope_half_split(k, np.array([n]), 1e4))
        b = np.sum(oracle.rope_half_split(q, np.array([m + sft]), 1e4) *
                   oracle.rope_half_split(k, np.array([n + sft]), 1e4))
        assert abs(a - b) < 1e-11 * max(1.0, abs(a))


def test_k_epilogue_in_the_chain():
    """In materialize: the epilogue changes K only (V and h_ctx as without
    it), acts at each row's logical position, and theta = 0 with no weight
    is the plain chain."""
    rng = np.random.default_rng(42)
    T, d, m, Hkv, D = 8, 16, 2, 2, 8
    hs = [rng.standard_normal((T, d)).astype(np.float32) for _ in range(m)]
    Wf = (rng.standard_normal((d, m * d)) * 0.2).astype(np.float32)
    WK = [(rng.standard_normal((Hkv * D, d)) * 0.2).astype(np.float32)]
    WV = [(rng.standard_normal((Hkv * D, d)) * 0.2).astype(np.float32)]
    w = [rng.uniform(0.5, 1.5, D).astype(np.float32)]
    plain = oracle.materialize(hs, Wf, None, WK, WV, Hkv, D, "f32")
    same = oracle.materialize(hs, Wf, None, WK, WV, Hkv, D, "f32", rope_theta=0.0,
                              rows_per_seq=4, seq_start_pos=[0, 0])
    np.testing.assert_array_equal(plain["K"][0], same["K"][0])
    epi = oracle.materialize(hs, Wf, None, WK, WV, Hkv, D, "f32", k_norm_weight=w,
                             k_norm_eps=1e-6, rope_theta=1e4, rows_per_seq=4,
                             seq_start_pos=[10, 500])
    np.testing.assert_array_equal(plain["V"][0], epi["V"][0])
    np.testing.assert_array_equal(plain["h_ctx"], epi["h_ctx"])
    pos = np.array([10, 11, 12, 13, 500, 501, 502, 503])
    np.testing.assert_array_equal(oracle.row_positions(T, 4, [10, 500]), pos)
    want = oracle.round_to_f32(oracle.rope_half_split(
        oracle.k_norm(plain["K"][0], w[0].astype(np.float64), 1e-6), pos, 1e4))
    np.testing.assert_array_equal(epi["K"][0], want)


def test_brute_force_exact_sums_on_a_tiny_case():
    """A second path for the whole chain on a tiny bf16 case: every h_ctx,
    K and V element is an explicit sum over the concatenated features,
    accumulated exactly by math.fsum and rounded once, with the
    concatenation indexed by hand (feature j of X is feature j mod d of hidden
    j // d).  No matrix product is involved; the oracle must agree to the last
    bit except where the two sums straddle a bf16 rounding boundary, which an
    exact sum and a float64 matmul may do on a near-halfway value."""
    import math
    c = synth.materialize_case(61, dtype="bf16", m=3, d_model=8, n_layers=2, n_kv_heads=2,
                               head_dim=4, n_seq=1, rows_per_seq=5, commit=[5])
    res = oracle.materialize(c.hiddens, c.W_f, c.b_f, c.W_K, c.W_V, 2, 4, "bf16")
    H = [oracle.widen(h, "bf16") for h in c.hiddens]
    Wf, bf = oracle.widen(c.W_f, "bf16"), oracle.widen(c.b_f, "bf16")
    T, d, m = 5, 8, 3
    h = np.zeros((T, d))
    for r in range(T):
        for o in range(d):
            h[r, o] = math.fsum([H[j // d][r, j % d] * Wf[o, j] for j in range(m * d)] + [bf[o]])
    h = oracle.round_to_bf16(h)
    off = 0
    for name, Ws in (("K", c.W_K), ("V", c.W_V)):
        for l, W in enumerate(Ws):
            W = oracle.widen(W, "bf16")
            want = np.array([[math.fsum(h[r, j] * W[o, j] for j in range(d)) for o in range(8)]
                             for r in range(T)])
            want = oracle.round_to_bf16(want).reshape(T, 2, 4)
            got = res[name][l]
            ulp = 2.0 ** (np.floor(np.log2(np.abs(want) + 1e-300)) - 7)
            assert (np.abs(got - want) <= ulp).all()
            off += int((got != want).sum())
    off += int((res["h_ctx"] != h).sum())
    hulp = 2.0 ** (np.floor(np.log2(np.abs(h) + 1e-300)) - 7)
    assert (np.abs(res["h_ctx"] - h) <= hulp).all()
    assert off <= 2     # at most a rare near-halfway disagreement
