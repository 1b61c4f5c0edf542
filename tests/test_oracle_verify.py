"""Pins for the verification oracle (greedy, sampled, gate).

Each test checks the oracle against something other than itself: numbers the
pages print (tests/golden/worked_pq_example.txt), planted answers known by
construction, closed forms, a library routine, or a statistical test of the
lossless property.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import synth
from tests.golden.load import worked_pq_example

# ----------------------------------------------------------------------------
# worked p/q example ([Spec-decoding tutorial], section 3)
# ----------------------------------------------------------------------------


def _worked_inputs(u, u2, row1=None):
    toks, cols, _ = worked_pq_example()
    p = np.array(cols["p"])
    q = np.array(cols["q"])
    V = len(p)
    t = np.zeros((1, 2, V))
    t[0, 0] = np.log(p)
    t[0, 1] = np.log(row1 if row1 is not None else np.full(V, 1.0 / V))
    d = np.log(q)[None, None, :]
    x = np.array([[toks.index("cat")]], dtype=np.int32)
    return t, d, x, np.array([[u]]), np.array([u2])


def test_worked_example_ratio_and_beta():
    toks, cols, scal = worked_pq_example()
    t, d, x, u, u2 = _worked_inputs(0.99, 0.3)
    r = oracle.verify_sample(t, d, x, u, u2, "f64")
    assert r.ratio[0, 0] == pytest.approx(scal["accept_prob_cat"], abs=1e-12)
    assert r.rejected[0]
    assert r.beta[0] == pytest.approx(scal["beta"], abs=1e-12)
    assert 1 - r.beta[0] == pytest.approx(scal["one_minus_beta"], abs=1e-12)


@pytest.mark.parametrize("u,acc", [(0.71, 1), (0.714, 1), (0.715, 0), (0.72, 0), (0.0, 1)])
def test_worked_example_accept_threshold(u, acc):
    t, d, x, uu, u2 = _worked_inputs(u, 0.5)
    r = oracle.verify_sample(t, d, x, uu, u2, "f64")
    assert r.accept_len[0] == acc
    assert r.commit_lens[0] == acc + 1


@pytest.mark.parametrize("u2,tok", [(0.0, "dog"), (0.49, "dog"), (0.4999, "dog"),
                                     (0.5001, "sat"), (0.51, "sat"), (0.999, "sat")])
def test_worked_example_residual_draw(u2, tok):
    toks, _, _ = worked_pq_example()
    t, d, x, u, uu2 = _worked_inputs(0.9, u2)
    r = oracle.verify_sample(t, d, x, u, uu2, "f64")
    assert r.accept_len[0] == 0
    assert toks[r.bonus[0]] == tok


def test_worked_example_residual_distribution_not_naive():
    """Sweeping u' over a fine grid reproduces the printed residual column:
    dog and sat 0.5 each, and 'on' never (the naive renormalisation would
    give it 0.20)."""
    toks, cols, scal = worked_pq_example()
    grid = (np.arange(4000) + 0.5) / 4000
    counts = np.zeros(5)
    for g in grid:
        t, d, x, u, u2 = _worked_inputs(0.9, g)
        counts[oracle.verify_sample(t, d, x, u, u2, "f64").bonus[0]] += 1
    freq = counts / len(grid)
    np.testing.assert_allclose(freq, cols["res"], atol=1e-3)
    assert freq[toks.index("on")] == 0.0
    assert scal["naive_renorm_on"] > 0.1  # the printed counter-example differs


def test_worked_example_all_accepted_bonus_from_next_row():
    """When the draft is accepted, the bonus is drawn from the target's next
    row ([DFlash overview] pseudocode, all-accepted branch)."""
    row1 = np.array([0.0, 0.0, 0.0, 1.0, 0.0]) + 1e-300
    row1 = row1 / row1.sum()
    t, d, x, u, u2 = _worked_inputs(0.1, 0.7, row1=row1)
    r = oracle.verify_sample(t, d, x, u, u2, "f64")
    assert r.accept_len[0] == 1 and not r.rejected[0]
    assert r.bonus[0] == 3 and r.bonus_row[0] == 1


# ----------------------------------------------------------------------------
# identities and special cases
# ----------------------------------------------------------------------------


def test_beta_matches_acceptance_probability_closed_form():
    """P(accept) = sum_x q(x) min(1, p(x)/q(x)) = sum_x min(p, q) = beta: the
    oracle's ratios, averaged under q in closed form, equal its own beta."""
    rng = np.random.default_rng(7)
    V = 64
    t = rng.normal(0, 2, (1, 2, V))
    d = t[:, :1] + rng.normal(0, 1, (1, 1, V))
    p = scipy.special.softmax(t[0, 0])
    q = scipy.special.softmax(d[0, 0])
    acc_prob = 0.0
    beta = None
    for x in range(V):
        r = oracle.verify_sample(t, d, np.array([[x]]), np.array([[0.999999]]),
                                 np.array([0.5]), "f64")
        acc_prob += q[x] * min(1.0, r.ratio[0, 0])
        if r.rejected[0]:
            beta = r.beta[0]
    assert beta is not None
    assert acc_prob == pytest.approx(beta, abs=1e-12)
    assert beta == pytest.approx(np.minimum(p, q).sum(), abs=1e-12)


def test_q_equals_p_always_accepts():
    """q == p gives beta = 1: every draft is accepted ([Spec-decoding
    tutorial], section 4)."""
    rng = np.random.default_rng(3)
    B, L, V = 8, 6, 50
    t = rng.normal(0, 2, (B, L + 1, V))
    d = t[:, :L].copy()
    x = rng.integers(0, V, (B, L)).astype(np.int32)
    u = np.full((B, L), 1 - 2.0 ** -24)
    r = oracle.verify_sample(t, d, x, u, np.full(B, 0.3), "f64")
    assert (r.accept_len == L).all()
    np.testing.assert_allclose(r.ratio, 1.0, atol=1e-12)


def test_disjoint_support_always_rejects():
    """q and p with disjoint support: beta = 0, every draft is rejected and
    the bonus comes from p."""
    V = 10
    t = np.full((1, 2, V), -np.inf); t[0, :, :5] = 0.0
    d = np.full((1, 1, V), -np.inf); d[0, 0, 5:] = 0.0
    for x in range(5, 10):
        r = oracle.verify_sample(t, d, np.array([[x]]), np.array([[0.0]]),
                                 np.array([0.5]), "f64")
        assert r.accept_len[0] == 0
        assert r.beta[0] == 0.0
        assert 0 <= r.bonus[0] < 5


def _chi2_marginal(t_row, d_row, n, seed, temperature=1.0):
    """Run n single-draft trials (x ~ q, fresh u, u'); return the histogram of
    the emitted token and the expected p."""
    rng = np.random.default_rng(seed)
    V = t_row.shape[0]
    q = scipy.special.softmax(d_row / temperature)
    p = scipy.special.softmax(t_row / temperature)
    cq = np.cumsum(q)
    hist = np.zeros(V)
    chunk = 2000
    t = np.broadcast_to(t_row, (chunk, 2, V))
    d = np.broadcast_to(d_row, (chunk, 1, V))
    for s in range(0, n, chunk):
        xs = np.minimum(np.searchsorted(cq, rng.random(chunk) * cq[-1], side="right"), V - 1)
        u = rng.random((chunk, 1))
        u2 = rng.random(chunk)
        r = oracle.verify_sample(t, d, xs[:, None].astype(np.int32), u, u2, "f64",
                                 temperature=temperature)
        out = np.where(r.accept_len == 1, xs, r.bonus)
        np.add.at(hist, out, 1)
    return hist, p


def _chi2_pvalue(hist, p):
    n = hist.sum()
    exp = p * n
    order = np.argsort(exp)
    h, e = hist[order], exp[order]
    # pool the small-expectation bins into one until it holds >= 5
    cut = np.searchsorted(np.cumsum(e), 5.0) + 1
    hp = np.concatenate([[h[:cut].sum()], h[cut:]])
    ep = np.concatenate([[e[:cut].sum()], e[cut:]])
    keep = ep >= 5
    hp = np.concatenate([hp[keep], [hp[~keep].sum()]]) if (~keep).any() else hp
    ep = np.concatenate([ep[keep], [ep[~keep].sum()]]) if (~keep).any() else ep
    return scipy.stats.chisquare(hp, ep * hp.sum() / ep.sum()).pvalue


def test_lossless_chi_square_worked_example():
    """The emitted token's marginal equals p ([Spec-decoding tutorial],
    section 3: min(p,q) + max(0, p-q) = p)."""
    _, cols, _ = worked_pq_example()
    hist, p = _chi2_marginal(np.log(cols["p"]), np.log(cols["q"]), 200_000, seed=11)
    assert _chi2_pvalue(hist, p) > 1e-3
    np.testing.assert_allclose(hist / hist.sum(), cols["p"], atol=4e-3)


@pytest.mark.slow
def test_lossless_chi_square_random_vocab():
    rng = np.random.default_rng(5)
    V = 1024
    t = rng.normal(0, 2, V)
    d = t + rng.normal(0, 1.5, V)
    hist, p = _chi2_marginal(t, d, 100_000, seed=12)
    assert _chi2_pvalue(hist, p) > 1e-3


def test_chi_square_detects_a_planted_mistake():
    """Sanity of the statistical pin: a sampler that draws the bonus from the
    naive renormalisation (p without the rejected token) fails it."""
    _, cols, _ = worked_pq_example()
    p = np.array(cols["p"]); q = np.array(cols["q"])
    rng = np.random.default_rng(13)
    n = 200_000
    xs = np.searchsorted(np.cumsum(q), rng.random(n), side="right")
    acc = rng.random(n) < np.minimum(1, p[xs] / q[xs])
    out = xs.copy()
    for i in np.flatnonzero(~acc):
        w = p.copy(); w[xs[i]] = 0; w /= w.sum()
        out[i] = np.searchsorted(np.cumsum(w), rng.random(), side="right")
    hist = np.bincount(out, minlength=5).astype(float)
    assert _chi2_pvalue(hist, p) < 1e-6


def test_chain_equals_stage_by_stage():
    """[DLoop], 验证与无损性: verifying S stages as one chain gives what
    verifying them one after another gives, for the same uniforms."""
    rng = np.random.default_rng(21)
    B, k, S, V = 12, 4, 3, 40
    L = S * k
    t = rng.normal(0, 1.0, (B, L + 1, V))
    d = t[:, :L] + rng.normal(0, 0.8, (B, L, V))
    x = np.zeros((B, L), dtype=np.int32)
    for b in range(B):
        for i in range(L):
            x[b, i] = rng.choice(V, p=scipy.special.softmax(d[b, i]))
    u = rng.random((B, L)) * 0.8   # bias towards acceptance so chains get long
    u2 = rng.random(B)
    chain = oracle.verify_sample(t, d, x, u, u2, "f64")
    for b in range(B):
        base = 0
        while True:
            lo = base
            r = oracle.verify_sample(t[b:b + 1, lo:lo + k + 1], d[b:b + 1, lo:lo + k],
                                     x[b:b + 1, lo:lo + k], u[b:b + 1, lo:lo + k],
                                     u2[b:b + 1], "f64")
            if r.accept_len[0] < k or lo + k == L:
                assert chain.accept_len[b] == lo + r.accept_len[0]
                assert chain.bonus[b] == r.bonus[0]
                break
            base += k
    assert len(set(chain.accept_len.tolist())) > 2


def test_sample_chain_lens_and_invalid_tokens():
    rng = np.random.default_rng(2)
    B, L, V = 4, 5, 30
    t = rng.normal(0, 1, (B, L + 1, V))
    d = t[:, :L].copy()
    x = rng.integers(0, V, (B, L)).astype(np.int32)
    x[2, 1] = V      # out of range inside the chain -> in-band error
    x[3, 4] = -5     # out of range past the chain  -> ignored
    cl = np.array([5, 0, 3, 2], dtype=np.int32)
    u = np.full((B, L), 0.5)
    r = oracle.verify_sample(t, d, x, u, np.full(B, 0.5), "f64", chain_lens=cl,
                             prefix_lens=np.array([10, 20, 30, 40]))
    assert r.accept_len.tolist() == [5, 0, -1, 2]
    assert r.commit_lens.tolist() == [6, 1, 0, 3]
    assert r.new_seq_lens.tolist() == [16, 21, 30, 43]


def test_temperature_divides_logits():
    rng = np.random.default_rng(4)
    V = 20
    t = rng.normal(0, 2, (1, 2, V)); d = t[:, :1] + rng.normal(0, 1, (1, 1, V))
    x = np.array([[3]], dtype=np.int32)
    T = 0.7
    r1 = oracle.verify_sample(t, d, x, np.array([[0.2]]), np.array([0.4]), "f64", temperature=T)
    p = scipy.special.softmax(t[0, 0] / T); q = scipy.special.softmax(d[0, 0] / T)
    assert r1.ratio[0, 0] == pytest.approx(p[3] / q[3], rel=1e-12)


# ----------------------------------------------------------------------------
# greedy ([SGLang DFlash], section 3)
# ----------------------------------------------------------------------------


def _cumprod_form(drafts, tp):
    """The page's vectorised statement: leading matches via a cumulative
    product of the match indicators."""
    matches = (drafts == tp[:, :-1]).astype(np.int32)
    acc = np.cumprod(matches, axis=1).sum(axis=1)
    return acc, tp[np.arange(len(acc)), acc]


def test_greedy_planted_acceptance():
    c = synth.greedy_case(101, dtype="bf16", B=16, L=15, V=4096, plant=True)
    r = oracle.verify_greedy(c.target_logits, "bf16", draft_tokens=c.draft_tokens,
                             prefix_lens=c.prefix_lens)
    assert (r.accept_len == c.planted_accept).all()
    assert (r.commit_lens == c.planted_accept + 1).all()
    assert (r.new_seq_lens == c.prefix_lens + c.planted_accept + 1).all()
    acc, bonus = _cumprod_form(c.draft_tokens, r.target_predict)
    assert (acc == r.accept_len).all() and (bonus == r.bonus).all()


def test_greedy_hand_cases():
    V = 6
    t = np.zeros((2, 4, V))
    tops = [[1, 2, 3, 4], [5, 0, 1, 2]]
    for b in range(2):
        for i in range(4):
            t[b, i, tops[b][i]] = 1.0
    drafts = np.array([[1, 2, 3], [4, 0, 1]], dtype=np.int32)
    r = oracle.verify_greedy(t, "f64", draft_tokens=drafts)
    assert r.accept_len.tolist() == [3, 0]       # all match / first mismatches
    assert r.bonus.tolist() == [4, 5]


def test_greedy_ties_lowest_index_and_neg_inf():
    V = 8
    t = np.zeros((1, 3, V))
    t[0, 0, [5, 2, 7]] = 3.0          # tie: 2 wins
    t[0, 1, :] = -np.inf              # all -inf: 0
    t[0, 2, [6, 4]] = 1.0
    r = oracle.verify_greedy(t, "f64", draft_tokens=np.array([[2, 0]], dtype=np.int32))
    assert r.target_predict[0].tolist() == [2, 0, 4]
    assert r.accept_len[0] == 2 and r.bonus[0] == 4


def test_greedy_planted_bf16_ties():
    c = synth.greedy_case(102, dtype="bf16", B=8, L=7, V=1000, ties=20)
    r = oracle.verify_greedy(c.target_logits, "bf16", draft_tokens=c.draft_tokens)
    t = oracle.widen(c.target_logits, "bf16")
    for b in range(8):
        for i in range(8):
            row = t[b, i]
            assert r.target_predict[b, i] == np.flatnonzero(row == row.max()).min()


def test_greedy_draft_argmax_fused():
    c = synth.greedy_case(103, dtype="bf16", B=6, L=9, V=777, with_draft_logits=True)
    r = oracle.verify_greedy(c.target_logits, "bf16", draft_logits=c.draft_logits)
    assert (r.draft_tokens == c.draft_tokens).all()
    assert (r.accept_len == c.planted_accept).all()


def test_greedy_chain_lens_and_invalid():
    c = synth.greedy_case(104, dtype="bf16", B=5, L=6, V=300)
    dr = c.draft_tokens.copy()
    dr[1, 0] = 300
    cl = np.array([6, 3, 0, 2, 6], dtype=np.int32)
    r = oracle.verify_greedy(c.target_logits, "bf16", draft_tokens=dr, chain_lens=cl)
    assert r.accept_len[1] == -1 and r.bonus[1] == -1 and r.commit_lens[1] == 0
    assert r.accept_len[2] == 0
    for b in (0, 3, 4):
        assert r.accept_len[b] == min(c.planted_accept[b], cl[b])
    assert (r.target_predict[3, 3:] == -1).all()


# ----------------------------------------------------------------------------
# gate ([DLoop], 机制一)
# ----------------------------------------------------------------------------


def test_gate_uniform_logits_closed_form():
    B, n, V = 3, 8, 1000
    d = np.zeros((B, n, V))
    x = np.zeros((B, n), dtype=np.int32)
    r = oracle.gate(d, x, "f64", g=-0.5)
    np.testing.assert_allclose(r.c, -n * math.log(V), rtol=0, atol=1e-10)
    assert not r.go.any()


def test_gate_one_hot_margin_near_zero_and_nonpositive():
    B, n, V = 2, 8, 500
    d = np.zeros((B, n, V))
    x = np.tile(np.arange(n, dtype=np.int32), (B, 1))
    d[:, np.arange(n), np.arange(n)] = 40.0
    r = oracle.gate(d, x, "f64", g=-0.5)
    assert (r.c <= 0).all()
    np.testing.assert_allclose(r.c, -n * np.log1p((V - 1) * np.exp(-40.0)), rtol=0, atol=1e-13)
    assert r.go.all()


def test_gate_library_logsumexp_and_threshold_flip():
    c = synth.gate_case(301, dtype="bf16", B=6, n=8, V=2048, temperature=0.8,
                        boost=[0, 10, 14, 16, 20, 30])
    r = oracle.gate(c.draft_logits, c.draft_tokens, "bf16", temperature=0.8)
    d = oracle.widen(c.draft_logits, "bf16") / 0.8
    for b in range(6):
        lse = scipy.special.logsumexp(d[b], axis=-1)
        ref = sum(d[b, i, c.draft_tokens[b, i]] - lse[i] for i in range(8))
        assert r.c[b] == pytest.approx(ref, abs=1e-9)
        assert (r.c[b] <= 0)
        np.testing.assert_allclose(r.row_lse[b], lse, atol=1e-12)
        hi = oracle.gate(c.draft_logits[b:b + 1], c.draft_tokens[b:b + 1], "bf16", 0.8,
                         g=r.c[b] + 1e-3)
        lo = oracle.gate(c.draft_logits[b:b + 1], c.draft_tokens[b:b + 1], "bf16", 0.8,
                         g=r.c[b] - 1e-3)
        eq = oracle.gate(c.draft_logits[b:b + 1], c.draft_tokens[b:b + 1], "bf16", 0.8,
                         g=r.c[b])
        assert not hi.go[0] and lo.go[0] and eq.go[0]


def test_gate_valid_lens():
    c = synth.gate_case(302, dtype="f32", B=4, n=6, V=100, valid=[6, 0, 3, 1])
    full = oracle.gate(c.draft_logits, c.draft_tokens, "f32")
    part = oracle.gate(c.draft_logits, c.draft_tokens, "f32", valid_lens=c.valid_lens)
    ls = oracle.widen(c.draft_logits, "f32")
    for b, vl in enumerate([6, 0, 3, 1]):
        per = [ls[b, i, c.draft_tokens[b, i]] - full.row_lse[b, i] for i in range(vl)]
        assert part.c[b] == pytest.approx(sum(per), abs=1e-12)


# ----------------------------------------------------------------------------
# the residual identity and the acceptance probability
# ----------------------------------------------------------------------------


def _identity_rows():
    """The worked example's (p, q) as logits, then random rows at two
    temperatures and a row pair with disjoint and -inf entries."""
    _, cols, _ = worked_pq_example()
    rows = [(np.log(cols["p"]), np.log(cols["q"]))]
    rng = np.random.default_rng(41)
    for T in (1.0, 0.6):
        t = rng.normal(0, 3, 1024)
        rows.append((t / T, (t + rng.normal(0, 1, 1024)) / T))
    t = np.full(8, -np.inf); t[:5] = rng.normal(0, 1, 5)
    d = np.full(8, -np.inf); d[3:] = rng.normal(0, 1, 5)
    rows.append((t, d))
    return rows


def test_overlap_plus_residual_is_p_elementwise():
    """[Spec-decoding tutorial] section 3: min(p, q) + max(0, p - q) = p for
    every token (accepted mass plus resampled mass), sum min = beta and the
    residual sums to 1 - beta.  A residual with the operands swapped
    (max(0, q - p)) or an overlap of max(p, q) fails it (checked below)."""
    for t, d in _identity_rows():
        p, q, overlap, res = oracle.residual(t, d)
        np.testing.assert_allclose(overlap + res, p, rtol=0, atol=1e-15)
        assert np.all(res >= 0) and np.all(overlap <= q + 1e-300)
        assert abs(res.sum() - (1.0 - overlap.sum())) <= 1e-12
        np.testing.assert_allclose(p.sum(), 1.0, atol=1e-12)
        np.testing.assert_allclose(q.sum(), 1.0, atol=1e-12)
    # the identity is not vacuous: the swapped residual breaks it
    t, d = _identity_rows()[0]
    p, q, overlap, _ = oracle.residual(t, d)
    assert np.abs(overlap + np.maximum(0.0, q - p) - p).max() > 0.1
    assert np.abs(np.maximum(p, q) + np.maximum(0.0, p - q) - p).max() > 0.1


def test_verify_sample_beta_is_the_overlap_of_the_rejected_row():
    """The beta that verify_sample reports equals sum min(p, q) of the rejected
    row, and on the worked example that is the printed 0.80."""
    _, cols, scal = worked_pq_example()
    t, d, x, u, u2 = _worked_inputs(0.9, 0.3)
    r = oracle.verify_sample(t, d, x, u, u2, "f64")
    _, _, overlap, res = oracle.residual(t[0, 0], d[0, 0])
    assert r.beta[0] == overlap.sum() == pytest.approx(scal["beta"], abs=1e-12)
    np.testing.assert_allclose(res / res.sum(), cols["res"], atol=1e-12)


def test_binomial_acceptance_rate_equals_beta():
    """Monte Carlo: draft x ~ q and u ~ U[0, 1) fresh per trial, run the
    oracle's acceptance test; the number of accepts is Binomial(n, beta)
    ([Spec-decoding tutorial] section 3: P(accept) = sum min(p, q)).  A
    two-sided exact binomial test must not reject (p-value > 1e-3)."""
    _, cols, scal = worked_pq_example()
    p, q = np.array(cols["p"]), np.array(cols["q"])
    rng = np.random.default_rng(43)
    n, chunk = 100_000, 5000
    t = np.broadcast_to(np.stack([np.log(p), np.log(np.full(5, 0.2))]), (chunk, 2, 5))
    d = np.broadcast_to(np.log(q), (chunk, 1, 5))
    accepts = 0
    for _ in range(n // chunk):
        xs = np.minimum(np.searchsorted(np.cumsum(q), rng.random(chunk) * q.sum(), side="right"), 4)
        u = synth.uniforms(rng, (chunk, 1))
        r = oracle.verify_sample(t, d, xs[:, None].astype(np.int32), u, synth.uniforms(rng, (chunk,)),
                                 "f64")
        accepts += int((r.accept_len == 1).sum())
    pv = scipy.stats.binomtest(accepts, n, scal["beta"]).pvalue
    assert pv > 1e-3, (accepts / n, pv)
    # the test has power: a rate of 0.79 would be rejected at this n
    assert scipy.stats.binomtest(int(0.79 * n), n, scal["beta"]).pvalue < 1e-6


def test_zero_draft_probability_accepts():
    """A drafted token the drafter gave probability zero (logit -inf) is
    accepted whatever its target probability (ratio taken as +inf), also when
    the target gives it probability zero too."""
    V = 6
    t = np.zeros((2, 2, V)); t[1, 0, 2] = -np.inf
    d = np.zeros((2, 1, V)); d[:, 0, 2] = -np.inf
    x = np.array([[2], [2]], dtype=np.int32)
    r = oracle.verify_sample(t, d, x, np.full((2, 1), 1 - 2.0 ** -24), np.array([0.5, 0.5]), "f64")
    assert r.accept_len.tolist() == [1, 1]
    assert np.isinf(r.ratio).all()
