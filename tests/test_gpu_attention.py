"""GPU parity: block attention through the C ABI against the CPU oracle.

Tolerance: max-abs / RMS <= 2e-2 (bf16 inputs) or 1e-4 (fp32), for the
output and the log-sum-exp.  The bar applies to the computed output: the
kernels are run with an fp32 output, and with a bf16 output whose elements
may in addition differ by the storage rounding, half a bf16 unit in the last
place (at most 2^-8 of the value)."""
import numpy as np
import pytest

import block_diffusion_draft_ctx_amd as dfl
import oracle
import synth
from tests.gpu_util import TOL, bits, down, log, rel_err, up

pytestmark = pytest.mark.gpu


def _run(c, lse=True, out_dtype=None, causal=False):
    import torch
    kind = c.dtype
    q = up(c.q, kind)
    lse_t = torch.empty((c.B, c.n_q_heads, c.k), dtype=torch.float32, device=q.device) if lse else None
    od = {"f32": torch.float32, "bf16": torch.bfloat16, None: None}[out_dtype]
    out, lse_t = dfl.block_attention(q, up(c.k_blk, kind), up(c.v_blk, kind), up(c.cache_k, kind),
                                     up(c.cache_v, kind), up(c.block_table, "i32"),
                                     up(c.ctx_lens, "i32"), lse=lse_t, out_dtype=od, causal=causal)
    return out, lse_t


def _check(c, out, lse, sel=None, causal=False):
    """Compare (optionally only the requests in sel) with the oracle."""
    import torch
    if sel is not None:
        c = _subset(c, sel)
        out = out[sel]
        lse = lse[sel] if lse is not None else None
    o_ref, l_ref = oracle.block_attention(c.q, c.k_blk, c.v_blk, c.cache_k, c.cache_v,
                                          c.block_table, c.ctx_lens, c.dtype, causal=causal)
    rms = np.sqrt(np.mean(o_ref ** 2))
    diff = np.abs(down(out) - o_ref)
    if out.dtype == torch.bfloat16:
        diff = np.maximum(diff - 2.0 ** -8 * np.abs(o_ref), 0.0)   # storage rounding
    e = float(diff.max() / rms)
    el = rel_err(down(lse), l_ref) if lse is not None else 0.0
    log(f"  out({out.dtype}) err {e:.2e}, lse err {el:.2e}")
    assert e <= TOL[c.dtype]
    assert el <= TOL[c.dtype]


def _subset(c, sel):
    """The listed requests with a compacted cache holding only their pages
    (same logical contents), so the oracle widens little memory."""
    sel = list(sel)
    pages = sorted({int(p) for b in sel for p in c.block_table[b] if p >= 0})
    remap = {p: i for i, p in enumerate(pages)}
    bt = np.full((len(sel), c.block_table.shape[1]), -1, dtype=np.int32)
    for i, b in enumerate(sel):
        for j, p in enumerate(c.block_table[b]):
            if p >= 0:
                bt[i, j] = remap[int(p)]
    idx = np.array(pages, dtype=np.int64)
    return synth.AttentionCase(c.dtype, len(sel), c.k, c.n_q_heads, c.n_kv_heads, c.head_dim,
                               c.q[sel], c.k_blk[sel], c.v_blk[sel], c.cache_k[idx],
                               c.cache_v[idx], bt, c.ctx_lens[sel])


@pytest.mark.parametrize("dtype,B,k,Hq,Hkv,D,ctx,qs,seed", [
    ("f32", 1, 8, 4, 2, 64, [64], 1.0, 1301),              # tiny fp32 workload
    ("f32", 1, 8, 4, 2, 64, [64], 10.0, 1302),             # peaked attention
    ("f32", 3, 4, 6, 2, 128, [0, 17, 40], 1.0, 1303),
    ("bf16", 3, 16, 32, 8, 128, [0, 45, 1000], 1.0, 2301),  # GQA 4, several tiles, ragged
    ("bf16", 2, 16, 32, 8, 128, [1024, 777], 4.0, 2302),
    ("bf16", 2, 8, 16, 4, 64, [33, 300], 1.0, 2303),        # D = 64, 2 waves
    ("bf16", 2, 1, 8, 8, 128, [0, 5], 1.0, 2304),           # k = 1, G = 1
    ("bf16", 2, 16, 64, 8, 128, [100, 513], 1.0, 2305),     # G = 8: 8 waves
    ("bf16", 1, 64, 16, 4, 64, [95], 1.0, 2306),            # k = 64: two 128-row chunks
    ("bf16", 2, 16, 40, 4, 128, [70, 300], 1.0, 2308),      # 160 rows: a partial second chunk
    ("bf16", 2, 5, 12, 3, 128, [31, 32], 2.0, 2307),        # rows not a multiple of 16
    ("bf16", 2, 64, 32, 8, 128, [100, 1000], 1.0, 2309),    # 256 rows, splits of one tile
])
def test_attention_parity(dtype, B, k, Hq, Hkv, D, ctx, qs, seed):
    log(f"attention dtype={dtype} B={B} k={k} Hq={Hq} Hkv={Hkv} D={D} ctx={ctx} seed={seed}")
    c = synth.attention_case(seed, dtype=dtype, B=B, k=k, n_q_heads=Hq, n_kv_heads=Hkv,
                             head_dim=D, ctx_lens=ctx, q_scale=qs)
    for od in (["f32"] if dtype == "f32" else ["f32", "bf16"]):
        out, lse = _run(c, out_dtype=od)
        _check(c, out, lse)


@pytest.mark.parametrize("B,C,seed", [(1, 8192, 2311), (8, 4096, 2312), (1, 1024, 2313)])
def test_attention_split_context(B, C, seed):
    """Few requests: the context is split across workgroups and merged by LSE."""
    log(f"attention split B={B} C={C}")
    assert dfl.lib().dflash_attention_workspace_size(B, 16, 32, 8, 128, (C + 15) // 16, dfl.BF16) > 0
    c = synth.attention_case(seed, dtype="bf16", B=B, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[C - 3 * b for b in range(B)])
    for od in ("f32", "bf16"):
        out, lse = _run(c, out_dtype=od)
        _check(c, out, lse)


def test_attention_llama_decode_full_size_sampled():
    """The timed launch: Llama-3.1-8B-shaped decode, B = 64, ctx 8192, k = 16,
    32 Q / 8 KV heads, D = 128.  Sampled requests are checked against the
    oracle; every output must be finite."""
    B, C = 64, 8192
    log(f"attention full size B={B} C={C}")
    c = synth.attention_case(2320, dtype="bf16", B=B, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[C] * B)
    out, lse = _run(c)
    assert np.isfinite(down(out)).all()
    _check(c, out, lse, sel=[0, 21, 63])


def test_attention_ragged_contexts():
    rng = np.random.default_rng(5)
    ctx = rng.integers(1024, 8193, size=12)
    c = synth.attention_case(2321, dtype="bf16", B=12, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=ctx)
    out, lse = _run(c)
    _check(c, out, lse, sel=[0, 5, 11])


def test_attention_packed_training_mask_sampled():
    """Packed training blocks: every block's table lists the same sequence's
    pages, ctx = anchor; checked on sampled blocks."""
    c, P = synth.packed_attention_case(2330, dtype="bf16", seq_len=8192, k=16, n_q_heads=32,
                                       n_kv_heads=8, head_dim=128, max_anchors=512)
    log(f"packed: {c.B} blocks, prompt {P}")
    sel = [0, c.B // 3, c.B // 2, c.B - 1]
    for od in ("f32", "bf16"):
        out, lse = _run(c, out_dtype=od)
        assert np.isfinite(down(out)).all()
        _check(c, out, lse, sel=sel)


def test_attention_determinism_and_page_order_invariance():
    """Two runs are bitwise equal; moving the same logical pages to other
    physical pages changes nothing."""
    a = synth.attention_case(2340, dtype="bf16", B=4, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[300, 2000, 17, 900], shuffle=False)
    b = synth.attention_case(2340, dtype="bf16", B=4, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[300, 2000, 17, 900], shuffle=True)
    for bb in range(4):
        for lp in range(a.block_table.shape[1]):
            pa, pb = a.block_table[bb, lp], b.block_table[bb, lp]
            if pa >= 0:
                b.cache_k[pb] = a.cache_k[pa]
                b.cache_v[pb] = a.cache_v[pa]
    o1, l1 = _run(a)
    o2, l2 = _run(a)
    o3, l3 = _run(b)
    np.testing.assert_array_equal(bits(o1), bits(o2))
    np.testing.assert_array_equal(bits(o1), bits(o3))
    np.testing.assert_array_equal(bits(l1), bits(l3))


def test_attention_in_band_errors():
    """A ctx length beyond the table's capacity or an out-of-range page entry
    poisons only that request's outputs (NaN)."""
    c = synth.attention_case(2350, dtype="bf16", B=3, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[40, 40, 40])
    ctx = c.ctx_lens.copy()
    ctx[0] = c.block_table.shape[1] * 16 + 1
    bt = c.block_table.copy()
    bt[2, 1] = c.cache_k.shape[0] + 5
    import torch
    kind = "bf16"
    lse = torch.empty((3, 32, 16), dtype=torch.float32, device="cuda:0")
    out, lse = dfl.block_attention(up(c.q, kind), up(c.k_blk, kind), up(c.v_blk, kind),
                                   up(c.cache_k, kind), up(c.cache_v, kind), up(bt, "i32"),
                                   up(ctx, "i32"), lse=lse)
    o = down(out)
    assert np.isnan(o[0]).all() and np.isnan(o[2]).all() and np.isfinite(o[1]).all()
    assert np.isnan(down(lse)[0]).all() and np.isfinite(down(lse)[1]).all()


def _run_shared(c, out_dtype=None, causal=False):
    """The same case through a one-row block table (every request reads row 0)."""
    import torch
    kind = c.dtype
    assert (c.block_table == c.block_table[:1]).all()
    q = up(c.q, kind)
    lse = torch.empty((c.B, c.n_q_heads, c.k), dtype=torch.float32, device=q.device)
    od = {"f32": torch.float32, "bf16": torch.bfloat16, None: None}[out_dtype]
    return dfl.block_attention(q, up(c.k_blk, kind), up(c.v_blk, kind), up(c.cache_k, kind),
                               up(c.cache_v, kind), up(c.block_table[:1], "i32"),
                               up(c.ctx_lens, "i32"), lse=lse, out_dtype=od, causal=causal)


def _shared_case(seed, B, ctx, Hq=32, Hkv=8, D=128, k=16):
    """A case whose block-table rows all list the same sequence's pages."""
    c = synth.attention_case(seed, dtype="bf16", B=B, k=k, n_q_heads=Hq, n_kv_heads=Hkv,
                             head_dim=D, ctx_lens=[max(ctx)] * B)
    c.block_table[:] = c.block_table[:1]
    c.ctx_lens[:] = np.asarray(ctx, dtype=np.int32)
    return c


@pytest.mark.parametrize("B,ctx,Hq,Hkv,D,seed", [
    (5, [100, 37, 0, 260, 64], 32, 8, 128, 2360),       # unsorted, ragged, a zero context
    (4, [1000, 1003, 17, 500], 32, 8, 128, 2361),
    (3, [64, 65, 130], 16, 4, 64, 2362),                 # D = 64
    (2, [300, 301], 64, 8, 128, 2363),                   # G = 8: too many rows to pair
    (2, [8000, 5003], 32, 8, 128, 2365),                 # one pair, context split across workgroups
    (3, [4100, 0, 3000], 32, 8, 128, 2366),              # split, and a last request without a partner
])
def test_attention_shared_table(B, ctx, Hq, Hkv, D, seed):
    """One block-table row shared by every request (table_rows = 1): each
    request must match the oracle on its own context length."""
    log(f"attention shared table B={B} ctx={ctx} Hq={Hq} Hkv={Hkv} D={D}")
    c = _shared_case(seed, B, ctx, Hq, Hkv, D)
    for od in ("f32", "bf16"):
        out, lse = _run_shared(c, out_dtype=od)
        _check(c, out, lse)


def test_attention_packed_training_mask_shared_table_sampled():
    """The packed training sequence through one shared table row (blocks in
    anchor order); sampled blocks at both ends and in the middle."""
    c, P = synth.packed_attention_case(2330, dtype="bf16", seq_len=8192, k=16, n_q_heads=32,
                                       n_kv_heads=8, head_dim=128, max_anchors=512)
    log(f"packed shared table: {c.B} blocks, prompt {P}")
    sel = [0, 1, c.B // 2 - 1, c.B // 2, c.B - 2, c.B - 1]
    out, lse = _run_shared(c, out_dtype="f32")
    assert np.isfinite(down(out)).all()
    _check(c, out, lse, sel=sel)


def test_attention_shared_table_bad_page_poisons_only_its_readers():
    """A bad entry in the shared row poisons the requests whose context
    reaches it and no other."""
    c = _shared_case(2364, 4, [40, 200, 20, 200])
    bt = c.block_table[:1].copy()
    bt[0, 5] = c.cache_k.shape[0] + 3          # positions 80..95: read by requests 1 and 3
    import torch
    lse = torch.empty((4, 32, 16), dtype=torch.float32, device="cuda:0")
    out, lse = dfl.block_attention(up(c.q, "bf16"), up(c.k_blk, "bf16"), up(c.v_blk, "bf16"),
                                   up(c.cache_k, "bf16"), up(c.cache_v, "bf16"), up(bt, "i32"),
                                   up(c.ctx_lens, "i32"), lse=lse, out_dtype=torch.float32)
    o = down(out)
    assert np.isnan(o[1]).all() and np.isnan(o[3]).all()
    assert np.isfinite(o[0]).all() and np.isfinite(o[2]).all()
    _check(c, out, lse, sel=[0, 2])


# --- causal block mask: block position i sees block keys 0..i ---------------

@pytest.mark.parametrize("dtype,B,k,Hq,Hkv,D,ctx,seed", [
    ("f32", 1, 8, 4, 2, 64, [64], 1401),
    ("f32", 3, 4, 6, 2, 128, [0, 17, 40], 1402),
    ("bf16", 3, 16, 32, 8, 128, [0, 45, 1000], 2401),     # several tiles, ragged, no context
    ("bf16", 2, 8, 16, 4, 64, [33, 300], 2402),           # D = 64
    ("bf16", 1, 64, 16, 4, 64, [95], 2403),               # k = 64: block spans two key tiles
    ("bf16", 2, 5, 12, 3, 128, [31, 32], 2404),           # rows not a multiple of 16
    ("bf16", 2, 16, 64, 8, 128, [100, 513], 2405),        # G = 8
    ("bf16", 2, 64, 32, 8, 128, [100, 1000], 2406),       # 256 rows, splits of one tile
    ("bf16", 2, 16, 40, 4, 128, [70, 300], 2407),         # 160 rows: a partial chunk
])
def test_attention_causal_parity(dtype, B, k, Hq, Hkv, D, ctx, seed):
    log(f"attention causal dtype={dtype} B={B} k={k} Hq={Hq} Hkv={Hkv} D={D} ctx={ctx}")
    c = synth.attention_case(seed, dtype=dtype, B=B, k=k, n_q_heads=Hq, n_kv_heads=Hkv,
                             head_dim=D, ctx_lens=ctx)
    for od in (["f32"] if dtype == "f32" else ["f32", "bf16"]):
        out, lse = _run(c, out_dtype=od, causal=True)
        _check(c, out, lse, causal=True)


def test_attention_causal_split_context():
    """One request: the context is split across workgroups; the masked block
    keys sit in the last split only."""
    c = synth.attention_case(2410, dtype="bf16", B=1, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[6000])
    out, lse = _run(c, out_dtype="f32", causal=True)
    _check(c, out, lse, causal=True)


def test_attention_causal_shared_table_pairs():
    """Causal blocks on one shared table row (two requests per workgroup)."""
    c = _shared_case(2411, 5, [100, 37, 0, 260, 64])
    for od in ("f32", "bf16"):
        out, lse = _run_shared(c, out_dtype=od, causal=True)
        _check(c, out, lse, causal=True)


def test_attention_causal_packed_training_sampled():
    """Packed training with the causal-within-block mask (one shared row)."""
    c, P = synth.packed_attention_case(2330, dtype="bf16", seq_len=8192, k=16, n_q_heads=32,
                                       n_kv_heads=8, head_dim=128, max_anchors=512)
    log(f"packed causal: {c.B} blocks")
    out, lse = _run_shared(c, out_dtype="f32", causal=True)
    assert np.isfinite(down(out)).all()
    _check(c, out, lse, sel=[0, c.B // 2, c.B - 1], causal=True)


def test_attention_causal_first_position_and_last_row():
    """Closed forms through the kernel: with no context, block position 0
    returns v_blk[0] (fp32 path exactly up to the division by l = 1); the
    last block position equals the bidirectional result (to 1e-5 of its size)."""
    c = synth.attention_case(2412, dtype="f32", B=2, k=6, n_q_heads=4, n_kv_heads=2,
                             head_dim=64, ctx_lens=[0, 0])
    out, _ = _run(c, causal=True)
    o = down(out)
    for h in range(4):
        np.testing.assert_allclose(o[:, 0, h], c.v_blk[:, 0, h // 2], rtol=0, atol=1e-6)
    c = synth.attention_case(2413, dtype="bf16", B=2, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[300, 1000])
    oc, lc = _run(c, out_dtype="f32", causal=True)
    ob, lb = _run(c, out_dtype="f32")
    e = float(np.abs(down(oc)[:, -1] - down(ob)[:, -1]).max())
    assert e <= 1e-5 * float(np.abs(down(ob)[:, -1]).max()), e


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_block_causal_figure_through_the_kernel(dtype, D):
    """[Spec tutorial] 5.3, the BD3-LM block-causal figure (three blocks of
    three positions): block j is one request of the bidirectional kernel with
    the earlier blocks as its context (one shared page table).  Compared with
    torch CPU float64 SDPA under the figure's 9 x 9 boolean mask."""
    import torch
    from tests.golden.load import block_causal_mask
    from tests.test_oracle_attention import block_causal_case
    log(f"block-causal figure dtype={dtype} D={D}")
    mask = torch.tensor(block_causal_mask(), dtype=torch.bool)
    c, (q, kk, vv) = block_causal_case(52, dtype, Hq=8, Hkv=2, D=D)
    out, lse = _run(c, out_dtype="f32")
    got = down(out).reshape(9, c.n_q_heads, D)
    G = c.n_q_heads // c.n_kv_heads
    ref = np.stack([torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[:, h])[None, None], torch.from_numpy(kk[:, h // G])[None, None],
        torch.from_numpy(vv[:, h // G])[None, None], attn_mask=mask[None, None])[0, 0].numpy()
        for h in range(c.n_q_heads)], axis=1)
    e = rel_err(got, ref)
    log(f"  err {e:.2e}")
    assert e <= TOL[dtype]
    _check(c, out, lse)
