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
    before = c.cache_k[0].view(np.uint32).copy()
    written = oracle.paged_write(cache, res["K"][0], c.block_table, 5, c.seq_start_pos,
                                 c.commit_lens)
    assert written.sum() == 5 + 2 + 0
    # committed rows read back at their logical positions
    for s, n in enumerate([5, 2, 0]):
        start = int(c.seq_start_pos[s])
        got = oracle.gather_paged(cache, c.block_table[s], start + n)[start:]
        np.testing.assert_array_equal(got, res["K"][0][s * 5: s * 5 + n])
    # untouched slots keep the sentinel bits
    after = cache.astype(np.float32).view(np.uint32)
    np.testing.assert_array_equal(after[~written], before[~written])


def test_unmapped_page_is_skipped():
    c = synth.materialize_case(8, dtype="f32", m=1, d_model=4, n_layers=1, n_kv_heads=1,
                               head_dim=4, n_seq=1, rows_per_seq=20, start_pos=[0])
    bt = c.block_table.copy(); bt[0, 1] = -1     # positions 16..19 unmapped
    res = oracle.materialize(c.hiddens, c.W_f, c.b_f, c.W_K, c.W_V, 1, 4, "f32")
    cache = oracle.widen(c.cache_k[0], "f32")
    w = oracle.paged_write(cache, res["K"][0], bt, 20, c.seq_start_pos, None)
    assert w.sum() == 16
