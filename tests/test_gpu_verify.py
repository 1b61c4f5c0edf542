"""GPU parity: greedy verification, sampled verification and the gate,
through the C ABI, against the CPU oracle on the same seeded inputs.

Integer outputs (accept_len, bonus, commit, predictions) must be bit-exact;
for sampled verification a mismatch is allowed only where the oracle reports
a near-tie (|u - p/q| < 1e-5 at the deciding row, or the bonus draw within
1e-5 of a CDF boundary), and the near-tie count is printed.  Floating outputs
must agree within max-abs / RMS <= 1e-4 (they are fp32 arithmetic in both
dtypes)."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import block_diffusion_draft_ctx_amd as dfl
import oracle
import synth
from tests.golden.load import worked_pq_example
from tests.gpu_util import down, log, rel_err, report, up

pytestmark = pytest.mark.gpu

V_LLAMA = 128256
V_QWEN = 151936


def _greedy_check(c, r, ref):
    B, L = c.B, c.L
    n = np.full(B, L) if c.chain_lens is None else c.chain_lens
    np.testing.assert_array_equal(down(r["accept_len"]), ref.accept_len)
    np.testing.assert_array_equal(down(r["bonus"]), ref.bonus)
    np.testing.assert_array_equal(down(r["commit_lens"]), ref.commit_lens)
    if "new_seq_lens" in r:
        np.testing.assert_array_equal(down(r["new_seq_lens"]), ref.new_seq_lens)
    if "target_predict" in r:
        np.testing.assert_array_equal(down(r["target_predict"]), ref.target_predict)
    if c.draft_logits is not None:
        dt = down(r["draft_tokens"])
        for b in range(B):
            np.testing.assert_array_equal(dt[b, :n[b]], ref.draft_tokens[b, :n[b]])


@pytest.mark.parametrize("dtype,B,L,V,dl,plant,ties,chain,seed", [
    ("f32", 1, 7, 1024, False, True, 0, None, 1001),     # tiny fp32 workload
    ("f32", 1, 7, 1024, True, False, 0, None, 1002),
    ("f32", 5, 7, 1024, False, True, 3, "random", 1003),
    ("bf16", 1, 15, V_LLAMA, False, True, 0, None, 2001),  # Llama-3.1-8B-shaped decode
    ("bf16", 8, 15, V_LLAMA, True, True, 4, None, 2002),
    ("bf16", 32, 15, V_LLAMA, False, False, 0, None, 2003),
    ("bf16", 64, 15, V_LLAMA, False, True, 8, "random", 2004),
    ("bf16", 3, 5, 1001, True, True, 2, None, 2005),      # ragged tail, scalar path
    ("bf16", 4, 0, 777, False, True, 0, None, 2006),      # no drafts: bonus only
])
def test_greedy_parity(dtype, B, L, V, dl, plant, ties, chain, seed):
    log(f"greedy dtype={dtype} B={B} L={L} V={V} draft_logits={dl} seed={seed}")
    c = synth.greedy_case(seed, dtype=dtype, B=B, L=L, V=V, plant=plant, ties=ties,
                          with_draft_logits=dl, chain=chain)
    kind = dtype
    r = dfl.verify_greedy(up(c.target_logits, kind),
                          draft_tokens=None if dl else up(c.draft_tokens, "i32"),
                          draft_logits=up(c.draft_logits, kind) if dl else None,
                          chain_lens=None if c.chain_lens is None else up(c.chain_lens, "i32"),
                          prefix_lens=up(c.prefix_lens, "i32"))
    ref = oracle.verify_greedy(c.target_logits, dtype, draft_tokens=None if dl else c.draft_tokens,
                               draft_logits=c.draft_logits, chain_lens=c.chain_lens,
                               prefix_lens=c.prefix_lens)
    _greedy_check(c, r, ref)
    if plant and not ties and chain is None and not dl:
        np.testing.assert_array_equal(down(r["accept_len"]), c.planted_accept)


def test_greedy_unaligned_rows_and_wide_buffer():
    """Rows V elements long inside a wider buffer (row stride V+3, odd):
    the kernel falls back to element loads and must agree exactly."""
    import torch
    c = synth.greedy_case(2011, dtype="bf16", B=6, L=7, V=3001, ties=2)
    wide = np.zeros((6, 8, 3004), dtype=np.uint16)
    wide[:, :, :3001] = c.target_logits
    t = up(wide, "bf16")[:, :, :3001]
    r = dfl.verify_greedy(t, draft_tokens=up(c.draft_tokens, "i32"))
    ref = oracle.verify_greedy(c.target_logits, "bf16", draft_tokens=c.draft_tokens)
    np.testing.assert_array_equal(down(r["accept_len"]), ref.accept_len)
    np.testing.assert_array_equal(down(r["target_predict"]), ref.target_predict)


def test_greedy_in_band_errors_and_neg_inf_rows():
    c = synth.greedy_case(2012, dtype="f32", B=4, L=5, V=999)
    t = c.target_logits.copy()
    t[2, 0, :] = -np.inf                       # all -inf row: argmax 0
    d = c.draft_tokens.copy()
    d[1, 2] = 999                              # out of range inside the chain
    d[3, 4] = -7                               # out of range past the chain
    cl = np.array([5, 5, 5, 3], dtype=np.int32)
    r = dfl.verify_greedy(up(t, "f32"), draft_tokens=up(d, "i32"), chain_lens=up(cl, "i32"),
                          prefix_lens=up(c.prefix_lens, "i32"))
    ref = oracle.verify_greedy(t, "f32", draft_tokens=d, chain_lens=cl, prefix_lens=c.prefix_lens)
    assert ref.accept_len[1] == -1 and ref.target_predict[2, 0] == 0
    np.testing.assert_array_equal(down(r["accept_len"]), ref.accept_len)
    np.testing.assert_array_equal(down(r["bonus"]), ref.bonus)
    np.testing.assert_array_equal(down(r["commit_lens"]), ref.commit_lens)
    np.testing.assert_array_equal(down(r["new_seq_lens"]), ref.new_seq_lens)


def test_greedy_bad_chain_length_is_in_band_error():
    c = synth.greedy_case(2013, dtype="f32", B=3, L=4, V=100)
    cl = np.array([4, 9, -1], dtype=np.int32)
    r = dfl.verify_greedy(up(c.target_logits, "f32"), draft_tokens=up(c.draft_tokens, "i32"),
                          chain_lens=up(cl, "i32"))
    acc = down(r["accept_len"])
    assert acc[1] == -1 and acc[2] == -1 and acc[0] >= 0
    assert (down(r["commit_lens"])[1:] == 0).all()


# ----------------------------------------------------------------------------
# sampled verification
# ----------------------------------------------------------------------------

def _sample_compare(c, r, ref, what):
    """Bit-exact accept/bonus except at oracle near-ties; returns #near-ties."""
    B = c.B
    acc, bon = down(r["accept_len"]), down(r["bonus"])
    mism = np.flatnonzero((acc != ref.accept_len) | (bon != ref.bonus))
    near = []
    for b in mism:
        # the deciding uniform: the row where the two sides disagree first
        j = int(min(acc[b], ref.accept_len[b])) if acc[b] >= 0 else 0
        ru = abs(float(c.u_accept[b, j]) - ref.ratio[b, j]) if j < c.L and not np.isnan(ref.ratio[b, j]) else np.inf
        if ru < 1e-5 or (acc[b] == ref.accept_len[b] and ref.cdf_gap[b] < 1e-5):
            near.append(b)
        else:
            raise AssertionError(f"{what}: request {b}: gpu (acc={acc[b]}, bonus={bon[b]}) vs "
                                 f"oracle (acc={ref.accept_len[b]}, bonus={ref.bonus[b]}); "
                                 f"ratio gap {ru}, cdf gap {ref.cdf_gap[b]}")
    np.testing.assert_array_equal(down(r["commit_lens"])[acc == ref.accept_len],
                                  ref.commit_lens[acc == ref.accept_len])
    # audit outputs: ratio on every tested row, beta where a row was rejected
    rg = down(r["ratio"])
    tested = ~np.isnan(ref.ratio)
    finite = tested & np.isfinite(ref.ratio)
    if finite.any():
        assert rel_err(rg[finite], ref.ratio[finite]) <= 1e-4
    bg = down(r["beta"])
    rej = ref.rejected & (acc == ref.accept_len)
    if rej.any():
        assert np.abs(bg[rej] - ref.beta[rej]).max() <= 1e-4
    assert np.isnan(bg[~ref.rejected & (acc == ref.accept_len)]).all()
    ties_ratio = int((ref.ratio_gap < 1e-5).sum())
    ties_cdf = int((ref.cdf_gap < 1e-5).sum())
    report(f"{what}: {len(near)} near-tie mismatches; near-ties in the inputs "
           f"(|u - p/q| < 1e-5): ratio {ties_ratio}, cdf {ties_cdf}; accept_len histogram "
           f"{np.bincount(ref.accept_len[ref.accept_len >= 0]).tolist()}")
    return len(near)


@pytest.mark.parametrize("dtype,B,L,V,sigma,chain,T,seed", [
    ("f32", 1, 7, 1024, 1.0, None, 1.0, 1101),           # tiny fp32 workload
    ("f32", 16, 7, 1024, 0.5, "random", 0.7, 1102),
    ("bf16", 16, 8, V_QWEN, 0.5, None, 1.0, 3001),        # Qwen3-4B-shaped, S = 1
    ("bf16", 16, 16, V_QWEN, 1.0, "random", 1.0, 3002),   # S = 2, ragged chains
    ("bf16", 16, 24, V_QWEN, 2.0, None, 1.0, 3003),       # S = 3
    ("bf16", 16, 32, V_QWEN, 0.5, "random", 1.0, 3004),   # S = 4
    ("bf16", 5, 9, 4099, 0.1, None, 1.3, 3005),           # ragged V, long accepts
])
def test_sample_parity(dtype, B, L, V, sigma, chain, T, seed):
    log(f"sample dtype={dtype} B={B} L={L} V={V} sigma={sigma} T={T} seed={seed}")
    c = synth.sample_case(seed, dtype=dtype, B=B, L=L, V=V, sigma=sigma, temperature=T,
                          chain=chain)
    r = dfl.verify_sample(up(c.target_logits, dtype), up(c.draft_logits, dtype),
                          up(c.draft_tokens, "i32"), up(c.u_accept, "f32"), up(c.u_bonus, "f32"),
                          temperature=T,
                          chain_lens=None if c.chain_lens is None else up(c.chain_lens, "i32"),
                          prefix_lens=up(c.prefix_lens, "i32"))
    ref = oracle.verify_sample(c.target_logits, c.draft_logits, c.draft_tokens, c.u_accept,
                               c.u_bonus, dtype, temperature=T, chain_lens=c.chain_lens,
                               prefix_lens=c.prefix_lens)
    _sample_compare(c, r, ref, f"sample seed {seed}")


def test_sample_planted_confident_stages():
    """DLoop-style chains: boosted stages accept long prefixes (chains of
    several stages verified at once)."""
    B, L, V = 16, 32, V_QWEN
    rng = np.random.default_rng(7)
    stages = [list(range(int(s))) for s in rng.integers(0, 5, size=B)]
    c = synth.sample_case(3010, dtype="bf16", B=B, L=L, V=V, sigma=1.0, boost_stages=stages,
                          stage=8, boost=20.0)
    r = dfl.verify_sample(up(c.target_logits, "bf16"), up(c.draft_logits, "bf16"),
                          up(c.draft_tokens, "i32"), up(c.u_accept, "f32"), up(c.u_bonus, "f32"))
    ref = oracle.verify_sample(c.target_logits, c.draft_logits, c.draft_tokens, c.u_accept,
                               c.u_bonus, "bf16")
    assert ref.accept_len.max() >= 16
    _sample_compare(c, r, ref, "planted stages")


def _worked_gpu(u, u2, B=1):
    _, cols, _ = worked_pq_example()
    p, q = np.array(cols["p"]), np.array(cols["q"])
    t = np.zeros((B, 2, 5), dtype=np.float32)
    t[:, 0] = np.log(p)
    t[:, 1] = np.log(np.full(5, 0.2))
    d = np.broadcast_to(np.log(q).astype(np.float32), (B, 1, 5)).copy()
    return t, d


def test_worked_example_on_gpu():
    toks, cols, scal = worked_pq_example()
    t, d = _worked_gpu(0, 0, B=4)
    x = np.zeros((4, 1), dtype=np.int32)          # the drafted token is "cat"
    u = np.array([[0.71], [0.72], [0.72], [0.9]], dtype=np.float32)
    u2 = np.array([0.3, 0.49, 0.51, 0.99], dtype=np.float32)
    r = dfl.verify_sample(up(t, "f32"), up(d, "f32"), up(x, "i32"), up(u, "f32"), up(u2, "f32"))
    acc, bon = down(r["accept_len"]), down(r["bonus"])
    assert acc.tolist() == [1, 0, 0, 0]
    assert [toks[i] for i in bon[1:]] == ["dog", "sat", "sat"]
    assert abs(down(r["ratio"])[0, 0] - scal["accept_prob_cat"]) < 1e-6
    assert np.allclose(down(r["beta"])[1:], scal["beta"], atol=1e-6)


def test_lossless_chi_square_through_gpu():
    """10^5 single-draft trials of the worked example through the kernels:
    the emitted token follows p."""
    _, cols, _ = worked_pq_example()
    p, q = np.array(cols["p"]), np.array(cols["q"])
    n = 100_000
    rng = np.random.default_rng(31)
    t, d = _worked_gpu(0, 0, B=n)
    x = np.searchsorted(np.cumsum(q), rng.random(n) * q.sum(), side="right").astype(np.int32)
    x = np.minimum(x, 4)[:, None]
    u = synth.uniforms(rng, (n, 1))
    u2 = synth.uniforms(rng, (n,))
    r = dfl.verify_sample(up(t, "f32"), up(d, "f32"), up(x, "i32"), up(u, "f32"), up(u2, "f32"),
                          audit=False)
    acc, bon = down(r["accept_len"]), down(r["bonus"])
    out = np.where(acc == 1, x[:, 0], bon)
    hist = np.bincount(out, minlength=5)
    pv = scipy.stats.chisquare(hist, p * n).pvalue
    log(f"chi-square over {n} GPU trials: p-value {pv:.3g}, freq {hist / n}")
    assert pv > 1e-3


# ----------------------------------------------------------------------------
# gate
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,B,n,V,T,valid,seed", [
    ("f32", 4, 7, 1024, 1.0, None, 1201),
    ("bf16", 16, 8, V_QWEN, 1.0, None, 3101),
    ("bf16", 16, 8, V_QWEN, 0.8, "random", 3102),
    ("bf16", 3, 5, 2001, 1.5, None, 3103),
])
def test_gate_parity(dtype, B, n, V, T, valid, seed):
    log(f"gate dtype={dtype} B={B} n={n} V={V} T={T} seed={seed}")
    boost = np.linspace(0, 30, B)
    c = synth.gate_case(seed, dtype=dtype, B=B, n=n, V=V, temperature=T, boost=boost, valid=valid)
    r = dfl.gate(up(c.draft_logits, dtype), up(c.draft_tokens, "i32"), temperature=T, g=-0.5,
                 valid_lens=None if c.valid_lens is None else up(c.valid_lens, "i32"))
    ref = oracle.gate(c.draft_logits, c.draft_tokens, dtype, temperature=T, g=-0.5,
                      valid_lens=c.valid_lens)
    cg = down(r["c"])
    assert rel_err(cg, ref.c) <= 1e-4
    assert rel_err(down(r["row_lse"]), ref.row_lse) <= 1e-4
    assert rel_err(down(r["row_max"]), ref.row_max) <= 1e-4
    go = down(r["go"])
    decided = np.abs(ref.c - (-0.5)) >= 1e-4
    np.testing.assert_array_equal(go[decided], ref.go[decided].astype(np.int64))
    report(f"gate seed {seed}: near-ties |c - g| < 1e-4: {int((~decided).sum())} of {B}")


def test_gate_invalid_token_gives_nan():
    c = synth.gate_case(3104, dtype="f32", B=3, n=4, V=50)
    x = c.draft_tokens.copy()
    x[1, 2] = 50
    r = dfl.gate(up(c.draft_logits, "f32"), up(x, "i32"))
    cg = down(r["c"])
    assert np.isnan(cg[1]) and down(r["go"])[1] == 0 and np.isfinite(cg[[0, 2]]).all()


# --- draft normalisers reused from the gate --------------------------------

@pytest.mark.parametrize("source", ["oracle", "gpu"])
def test_sample_reuses_gate_row_lse(source):
    """DLoop: the gate computes every draft row's log-sum-exp while drafting;
    the chain verify given those (draft_row_lse) reduces only the target rows
    and must match the oracle as the full pass does (Qwen-shaped, 4 stages)."""
    import torch
    B, L, V, T = 16, 32, V_QWEN, 1.0
    c = synth.sample_case(3020, dtype="bf16", B=B, L=L, V=V, sigma=1.0, temperature=T)
    dl = up(c.draft_logits, "bf16")
    toks = up(c.draft_tokens, "i32")
    if source == "oracle":
        lse = oracle.gate(c.draft_logits, c.draft_tokens, "bf16", temperature=T).row_lse
        lse_t = torch.from_numpy(lse.astype(np.float32)).to(dl.device)
    else:
        # one gate per stage of 8 drafts, as the drafter runs it, each writing
        # its columns of the chain's [B, L] statistics
        lse_t = torch.full((B, L), float("nan"), dtype=torch.float32, device=dl.device)
        mx = torch.empty_like(lse_t)
        for s in range(0, L, 8):
            dfl.gate(dl[:, s:s + 8].contiguous(), toks[:, s:s + 8].contiguous(), temperature=T,
                     out={"row_lse": lse_t[:, s:s + 8], "row_max": mx[:, s:s + 8]})
        assert torch.isfinite(lse_t).all()
    r = dfl.verify_sample(up(c.target_logits, "bf16"), dl, toks, up(c.u_accept, "f32"),
                          up(c.u_bonus, "f32"), temperature=T, draft_row_lse=lse_t.contiguous())
    ref = oracle.verify_sample(c.target_logits, c.draft_logits, c.draft_tokens, c.u_accept,
                               c.u_bonus, "bf16", temperature=T)
    _sample_compare(c, r, ref, f"gate lse from {source}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sample_zero_draft_probability_accepts(dtype):
    """A drafted token with draft logit -inf (q(x) = 0) is accepted, as the
    oracle reads it (ratio +inf), both with a finite target logit and with the
    target logit -inf too (0/0); u is the largest uniform, so nothing else
    would accept.  Other requests and rows keep the ordinary rule."""
    B, L, V = 5, 4, 3001
    c = synth.sample_case(3040, dtype=dtype, B=B, L=L, V=V, sigma=1.0)
    t, d, x = c.target_logits.copy(), c.draft_logits.copy(), c.draft_tokens.copy()
    u = c.u_accept.copy()
    ninf = np.uint16(0xFF80) if dtype == "bf16" else np.float32(-np.inf)
    top = np.float32(1 - 2.0 ** -24)
    d[0, 0, x[0, 0]] = ninf; u[0, 0] = top                            # target finite
    d[1, 0, x[1, 0]] = ninf; t[1, 0, x[1, 0]] = ninf; u[1, 0] = top   # both -inf
    for i in range(L):                                                 # a whole chain at q = 0
        d[2, i, x[2, i]] = ninf; u[2, i] = top
    d[3, 2, x[3, 2]] = ninf; t[3, 2, x[3, 2]] = ninf; u[3, :3] = 0.0   # accepted up to it
    r = dfl.verify_sample(up(t, dtype), up(d, dtype), up(x, "i32"), up(u, "f32"),
                          up(c.u_bonus, "f32"))
    ref = oracle.verify_sample(t, d, x, u, c.u_bonus, dtype)
    assert ref.accept_len[0] >= 1 and ref.accept_len[1] >= 1 and ref.accept_len[2] == L
    assert ref.accept_len[3] >= 3
    rg = down(r["ratio"])
    assert np.isinf(rg[[0, 1, 2, 3], [0, 0, 0, 2]]).all() and (rg[[0, 1, 2, 3], [0, 0, 0, 2]] > 0).all()
    c2 = synth.SampleCase(**{**c.__dict__, "u_accept": u})
    _sample_compare(c2, r, ref, f"q(x) = 0 drafts ({dtype})")
