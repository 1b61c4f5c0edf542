"""GPU parity: target-context KV materialisation through the C ABI against
the CPU oracle.  Cache slots that are written must match within max-abs / RMS
<= 2e-2 (bf16) or 1e-4 (fp32); every other slot must keep its sentinel bits."""
import numpy as np
import pytest

import block_diffusion_draft_ctx_amd as dfl
import oracle
import synth
from tests.gpu_util import TOL, bits, down, log, rel_err, rel_err_chained, up

pytestmark = pytest.mark.gpu


def _run(c, want_h=True, epi=None):
    """epi: None, or dict(w=per-layer norm weights or None, eps=..., theta=...)."""
    import torch
    kind = c.dtype
    ck = [up(x, kind) for x in c.cache_k]
    cv = [up(x, kind) for x in c.cache_v]
    hid = [up(h, kind) for h in c.hiddens]
    h_out = None
    if want_h:
        h_out = torch.empty((c.T, c.d_model), dtype=hid[0].dtype, device=hid[0].device)
    kw = {}
    if epi is not None:
        kw = dict(k_norm_weight=None if epi["w"] is None else [up(w, kind) for w in epi["w"]],
                  k_norm_eps=epi["eps"], rope_theta=epi["theta"])
    dfl.materialize_ctx_kv(hid, up(c.W_f, kind), None if c.b_f is None else up(c.b_f, kind),
                           [up(w, kind) for w in c.W_K], [up(w, kind) for w in c.W_V], ck, cv,
                           up(c.block_table, "i32"), c.rows_per_seq, up(c.seq_start_pos, "i32"),
                           None if c.commit_lens is None else up(c.commit_lens, "i32"),
                           h_ctx_out=h_out, **kw)
    return ck, cv, h_out


def _check(c, ck, cv, h_out, rows=None, epi=None):
    """Compare written slots (all rows, or the listed rows) with the oracle and
    the untouched slots with the sentinel."""
    T = c.T
    rows = np.arange(T) if rows is None else np.asarray(rows)
    kw = {}
    if epi is not None:
        # the oracle's rows are the listed ones: give each its own position
        pos = oracle.row_positions(T, c.rows_per_seq, c.seq_start_pos)[rows]
        kw = dict(k_norm_weight=epi["w"], k_norm_eps=epi["eps"], rope_theta=epi["theta"],
                  rows_per_seq=1, seq_start_pos=pos)
    ref = oracle.materialize([h[rows] for h in c.hiddens], c.W_f, c.b_f, c.W_K, c.W_V,
                             c.n_kv_heads, c.head_dim, c.dtype, **kw)
    if h_out is not None:
        e = rel_err(down(h_out)[rows], ref["h_ctx"])
        log(f"  h_ctx err {e:.2e}")
        assert e <= TOL[c.dtype]
    sentinel = c.cache_k[0].reshape(-1).view(np.uint16 if c.dtype == "bf16" else np.uint32)[0]
    for l in range(c.n_layers):
        for name, gpu, rv in (("K", ck[l], ref["K"][l]), ("V", cv[l], ref["V"][l])):
            g = oracle.slots(down(gpu))       # [num_pages, 16, Hkv, D] by page position
            gb = oracle.slots(bits(gpu))
            written = np.zeros(g.shape[:2], dtype=bool)
            got, want = [], []
            for i, r in enumerate(rows):
                s, j = divmod(int(r), c.rows_per_seq)
                if c.commit_lens is not None and j >= c.commit_lens[s]:
                    continue
                pos = int(c.seq_start_pos[s]) + j
                page = int(c.block_table[s, pos // 16])
                if page < 0 or page >= c.num_pages:
                    continue
                written[page, pos % 16] = True
                got.append(g[page, pos % 16])
                want.append(rv[i])
            if got:
                if epi is not None and name == "K":   # two storage points in the chain
                    e = rel_err_chained(np.array(got), np.array(want), c.dtype,
                                        what=f"K epilogue, layer {l}, {len(got)} rows")
                else:
                    e = rel_err(np.array(got), np.array(want))
                assert e <= TOL[c.dtype], f"layer {l} {name}: err {e}"
            if len(rows) == T:   # every row checked: untouched slots keep the sentinel
                untouched = gb[~written]
                assert (untouched == sentinel).all(), f"layer {l} {name}: stray writes"
        log(f"  layer {l} ok")


@pytest.mark.parametrize("dtype,m,d,Ld,Hkv,D,n_seq,rps,start,commit,seed", [
    ("f32", 5, 256, 1, 2, 64, 1, 64, [0], None, 1401),          # tiny fp32: 64-position prefill
    ("f32", 5, 256, 1, 2, 64, 1, 8, [64], "random", 1402),      # then an 8-row decode commit
    ("f32", 3, 96, 2, 1, 64, 3, 5, [0, 14, 30], [5, 2, 0], 1403),
    ("bf16", 5, 256, 2, 2, 64, 3, 16, None, "random", 2401),
    ("bf16", 2, 384, 3, 1, 128, 2, 40, [3, 0], [40, 17], 2402),  # rows straddle pages
    ("bf16", 5, 4096, 5, 8, 128, 8, 16, None, "random", 2403),   # Llama-shaped decode, B = 8
    ("bf16", 5, 4096, 5, 8, 128, 1, 16, [8192], "random", 2404),  # B = 1: the 32-row tile plan
    ("bf16", 5, 4096, 5, 8, 128, 2, 16, [1000, 77], [16, 3], 2405),  # B = 2: 32 rows, split-K
    # Hkv*D = 128: no tile may straddle a layer's K and V blocks (256-wide tiles are not allowed)
    ("bf16", 5, 256, 5, 2, 64, 4, 2048, None, None, 2406),       # prefill-sized T = 8192
    ("bf16", 2, 128, 17, 2, 64, 2, 16, [0, 40], "random", 2407),  # 17 layers: two layer groups
    ("bf16", 5, 512, 2, 8, 128, 16, 16, None, "random", 2408),    # T = 256: two 128-row tiles
])
def test_materialize_parity(dtype, m, d, Ld, Hkv, D, n_seq, rps, start, commit, seed):
    log(f"materialise dtype={dtype} m={m} d={d} layers={Ld} Hkv={Hkv} D={D} rows={n_seq}x{rps}")
    c = synth.materialize_case(seed, dtype=dtype, m=m, d_model=d, n_layers=Ld, n_kv_heads=Hkv,
                               head_dim=D, n_seq=n_seq, rows_per_seq=rps, start_pos=start,
                               commit=commit)
    ck, cv, h = _run(c)
    _check(c, ck, cv, h)


def test_materialize_decode_launch_config_sampled():
    """The timed launch: 64 requests x 16 committed-row candidates (T = 1024)
    of the Llama-3.1-8B-shaped draft (d 4096, 5 hiddens, 5 layers, 8 KV heads
    x 128); sampled rows against the oracle."""
    c = synth.materialize_case(2410, dtype="bf16", m=5, d_model=4096, n_layers=5, n_kv_heads=8,
                               head_dim=128, n_seq=64, rows_per_seq=16, commit="random")
    ck, cv, h = _run(c)
    rows = np.random.default_rng(0).choice(c.T, size=48, replace=False)
    _check(c, ck, cv, h, rows=np.sort(rows))


@pytest.mark.parametrize("n_seq,rps,seed", [(125, 8, 2415), (65, 16, 2416)])
def test_materialize_ragged_rows_on_large_tiles(n_seq, rps, seed):
    """Row counts that are not a multiple of the row tile (T = 1000 and 1040)
    at full width: the fusion GEMM splits its contraction over 256 x 256 tiles
    and the K/V GEMM runs 192 x 256 tiles whole (240 tiles fill the CUs where
    256-row ones would leave some idle), both with a partial last row tile;
    rows at the tile edges of both tilings are checked."""
    c = synth.materialize_case(seed, dtype="bf16", m=5, d_model=4096, n_layers=5, n_kv_heads=8,
                               head_dim=128, n_seq=n_seq, rows_per_seq=rps, commit="random")
    T = c.T
    log(f"materialise ragged T={T}")
    ck, cv, h = _run(c)
    rng = np.random.default_rng(seed)
    rows = sorted({0, 191, 192, 255, 256, 767, 768, 959, 960, T - 2, T - 1, *rng.choice(T, size=16, replace=False).tolist()})
    _check(c, ck, cv, h, rows=np.asarray(rows))


def test_materialize_prefill_shape_sampled():
    """Prefill-shaped materialisation (whole sequences, 16-token pages, every
    row committed) at T = 8192; sampled rows against the oracle."""
    c = synth.materialize_case(2420, dtype="bf16", m=5, d_model=4096, n_layers=5, n_kv_heads=8,
                               head_dim=128, n_seq=2, rows_per_seq=4096, start_pos=[0, 0])
    ck, cv, h = _run(c, want_h=False)
    rows = np.sort(np.random.default_rng(1).choice(c.T, size=32, replace=False))
    _check(c, ck, cv, None, rows=rows)


def test_materialize_unmapped_and_out_of_range_pages_are_skipped():
    c = synth.materialize_case(2430, dtype="bf16", m=2, d_model=256, n_layers=1, n_kv_heads=2,
                               head_dim=64, n_seq=2, rows_per_seq=32, start_pos=[0, 0])
    c.block_table[0, 1] = -1
    c.block_table[1, 0] = 10_000
    ck, cv, h = _run(c)
    _check(c, ck, cv, h, rows=list(range(0, 16)) + list(range(48, 64)))
    # rows 16..31 of seq 0 (unmapped) and 0..15 of seq 1 (out of range): nothing written anywhere
    gb = bits(ck[0])
    sentinel = c.cache_k[0].reshape(-1)[0]
    written = 32  # 16 rows of seq 0 + 16 rows of seq 1
    assert oracle.slots(gb != sentinel).any(axis=(2, 3)).sum() == written


def test_materialize_is_deterministic():
    c = synth.materialize_case(2440, dtype="bf16", m=5, d_model=512, n_layers=2, n_kv_heads=4,
                               head_dim=128, n_seq=4, rows_per_seq=16)
    a = _run(c)
    b = _run(c)
    for x, y in zip(a[0] + a[1] + [a[2]], b[0] + b[1] + [b[2]]):
        np.testing.assert_array_equal(bits(x), bits(y))


def test_materialize_prefill_full_size_sampled():
    """The prefill launch at full size: 4 sequences x 32768 rows (T = 131072),
    five hiddens of 4096, W_f [4096, 20480] + b_f, five draft layers of 8 KV
    heads x 128, 16-token pages in shuffled order, every row committed.  The
    inputs are seeded normals drawn on the device by torch (too large to draw
    on the host); the sampled rows and the weights are copied back bit for bit
    for the oracle, and those rows' cache slots are compared."""
    import torch
    n_seq, rps, d, m, Ld, Hkv, D = 4, 32768, 4096, 5, 5, 8, 128
    T = n_seq * rps
    log(f"materialise full prefill T={T}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(2450)
    bf = torch.bfloat16

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device=dev) * std).to(bf)

    hid = [randn(T, d) for _ in range(m)]
    Wf, bfv = randn(d, m * d, std=0.02), randn(d, std=0.02)
    WK = [randn(Hkv * D, d, std=0.02) for _ in range(Ld)]
    WV = [randn(Hkv * D, d, std=0.02) for _ in range(Ld)]
    maxp = rps // 16
    bt = torch.randperm(n_seq * maxp, generator=g, device=dev).to(torch.int32).view(n_seq, maxp)
    ck = [torch.zeros(n_seq * maxp, Hkv, 16, D, dtype=bf, device=dev) for _ in range(Ld)]
    cv = [torch.zeros(n_seq * maxp, Hkv, 16, D, dtype=bf, device=dev) for _ in range(Ld)]
    start = torch.zeros(n_seq, dtype=torch.int32, device=dev)
    dfl.materialize_ctx_kv(hid, Wf, bfv, WK, WV, ck, cv, bt.contiguous(), rps, start, None)
    torch.cuda.synchronize()
    # sampled rows: each sequence's first and last row, a page boundary, random rows
    rng = np.random.default_rng(2450)
    rows = sorted({0, rps - 1, rps, 2 * rps + 15, 2 * rps + 16, T - 1,
                   *rng.choice(T, size=18, replace=False).tolist()})
    ridx = torch.tensor(rows, dtype=torch.int64, device=dev)
    ref = oracle.materialize([bits(h.index_select(0, ridx)) for h in hid], bits(Wf), bits(bfv),
                             [bits(w) for w in WK], [bits(w) for w in WV], Hkv, D, "bf16")
    btn = bt.cpu().numpy()
    sidx = torch.tensor([int(btn[r // rps, (r % rps) // 16]) * 16 + r % 16 for r in rows],
                        dtype=torch.int64, device=dev)
    for l in range(Ld):
        for name, cache, rv in (("K", ck[l], ref["K"][l]), ("V", cv[l], ref["V"][l])):
            by_slot = cache.transpose(1, 2).reshape(-1, Hkv, D)   # head-major -> slot order
            got = down(by_slot.index_select(0, sidx))
            e = rel_err(got, rv)
            assert e <= TOL["bf16"], (l, name, e)
    log(f"  {len(rows)} rows x {Ld} layers x K/V within {TOL['bf16']}")



def test_materialize_past_32bit_operand_offsets_sampled():
    """Rows enough that a hidden-state buffer exceeds 4 GiB (T = 528384 rows of
    4096 bf16 per hidden, two hiddens, one draft layer): both GEMMs then load
    their operands with 64-bit addresses instead of 32-bit buffer offsets.
    Device-drawn seeded normals as in the full-size prefill test; sampled rows
    (including rows whose operand bytes lie past 4 GiB) are compared."""
    import torch
    n_seq, rps, d, m, Ld, Hkv, D = 1, 528384, 4096, 2, 1, 8, 128
    T = n_seq * rps
    assert T * d * 2 > 2 ** 32
    log(f"materialise past 32-bit offsets T={T}")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(2460)
    bf = torch.bfloat16

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device=dev) * std).to(bf)

    hid = [randn(T, d) for _ in range(m)]
    Wf, bfv = randn(d, m * d, std=0.02), randn(d, std=0.02)
    WK = [randn(Hkv * D, d, std=0.02) for _ in range(Ld)]
    WV = [randn(Hkv * D, d, std=0.02) for _ in range(Ld)]
    maxp = rps // 16
    bt = torch.randperm(n_seq * maxp, generator=g, device=dev).to(torch.int32).view(n_seq, maxp)
    ck = [torch.zeros(n_seq * maxp, Hkv, 16, D, dtype=bf, device=dev) for _ in range(Ld)]
    cv = [torch.zeros(n_seq * maxp, Hkv, 16, D, dtype=bf, device=dev) for _ in range(Ld)]
    start = torch.zeros(n_seq, dtype=torch.int32, device=dev)
    dfl.materialize_ctx_kv(hid, Wf, bfv, WK, WV, ck, cv, bt.contiguous(), rps, start, None)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2460)
    past = 2 ** 32 // (d * 2)   # first row whose bytes start past 4 GiB
    rows = sorted({0, 255, past - 1, past, past + 255, T - 256, T - 1,
                   *rng.choice(T, size=12, replace=False).tolist()})
    ridx = torch.tensor(rows, dtype=torch.int64, device=dev)
    ref = oracle.materialize([bits(h.index_select(0, ridx)) for h in hid], bits(Wf), bits(bfv),
                             [bits(w) for w in WK], [bits(w) for w in WV], Hkv, D, "bf16")
    btn = bt.cpu().numpy()
    sidx = torch.tensor([int(btn[r // rps, (r % rps) // 16]) * 16 + r % 16 for r in rows],
                        dtype=torch.int64, device=dev)
    for l in range(Ld):
        for name, cache, rv in (("K", ck[l], ref["K"][l]), ("V", cv[l], ref["V"][l])):
            by_slot = cache.transpose(1, 2).reshape(-1, Hkv, D)
            got = down(by_slot.index_select(0, sidx))
            e = rel_err(got, rv)
            assert e <= TOL["bf16"], (l, name, e)
    log(f"  {len(rows)} rows x {Ld} layer x K/V within {TOL['bf16']}")
    del hid, ck, cv
    torch.cuda.empty_cache()

# --- K epilogue: per-head RMSNorm, then the rotary embedding at each row's position

def _epi(seed, c, norm=True, theta=1e6, eps=1e-6):
    w = synth.k_norm_weights(seed, n_layers=c.n_layers, head_dim=c.head_dim, dtype=c.dtype) \
        if norm else None
    return dict(w=w, eps=eps, theta=theta)


@pytest.mark.parametrize("dtype,m,d,Ld,Hkv,D,n_seq,rps,start,commit,norm,theta,seed", [
    ("f32", 5, 256, 1, 2, 64, 1, 64, [0], None, True, 1e4, 1501),          # tiny prefill
    ("f32", 5, 256, 1, 2, 64, 1, 8, [64], "random", True, 1e4, 1502),      # then a decode commit
    ("f32", 3, 96, 2, 1, 128, 3, 5, [0, 14, 30], [5, 2, 0], False, 1e6, 1503),   # rotary only
    ("bf16", 5, 256, 2, 2, 64, 3, 16, None, "random", True, 0.0, 2501),    # norm only
    ("bf16", 2, 384, 3, 1, 128, 2, 40, [3, 0], [40, 17], True, 1e6, 2502),
    ("bf16", 5, 4096, 5, 8, 128, 8, 16, [8192, 100, 5000, 0, 77, 8000, 31, 4096], "random",
     True, 1e6, 2503),                                                       # Llama-shaped decode
    ("bf16", 2, 256, 1, 2, 128, 2, 16, [60000, 131000], None, True, 1e6, 2504),   # long positions
])
def test_materialize_k_epilogue_parity(dtype, m, d, Ld, Hkv, D, n_seq, rps, start, commit, norm,
                                       theta, seed):
    log(f"materialise + K epilogue dtype={dtype} layers={Ld} Hkv={Hkv} D={D} rows={n_seq}x{rps} "
        f"norm={norm} theta={theta}")
    c = synth.materialize_case(seed, dtype=dtype, m=m, d_model=d, n_layers=Ld, n_kv_heads=Hkv,
                               head_dim=D, n_seq=n_seq, rows_per_seq=rps, start_pos=start,
                               commit=commit)
    epi = _epi(seed + 7, c, norm=norm, theta=theta)
    ck, cv, h = _run(c, epi=epi)
    _check(c, ck, cv, h, epi=epi)


def test_materialize_k_epilogue_decode_launch_sampled():
    """The decode launch (T = 1024, Llama-shaped, 5 layers) with the K
    epilogue, rows at positions past 8192; sampled rows."""
    c = synth.materialize_case(2510, dtype="bf16", m=5, d_model=4096, n_layers=5, n_kv_heads=8,
                               head_dim=128, n_seq=64, rows_per_seq=16, start_pos=8192,
                               commit="random")
    epi = _epi(2511, c)
    ck, cv, h = _run(c, epi=epi)
    rows = np.sort(np.random.default_rng(3).choice(c.T, size=48, replace=False))
    _check(c, ck, cv, h, rows=rows, epi=epi)


def test_materialize_k_epilogue_prefill_sampled():
    """Prefill shape (2 x 4096 rows, positions 0..4095, every row committed)
    with the K epilogue; sampled rows."""
    c = synth.materialize_case(2520, dtype="bf16", m=5, d_model=4096, n_layers=5, n_kv_heads=8,
                               head_dim=128, n_seq=2, rows_per_seq=4096, start_pos=[0, 0])
    epi = _epi(2521, c)
    ck, cv, h = _run(c, want_h=False, epi=epi)
    rows = np.sort(np.random.default_rng(4).choice(c.T, size=32, replace=False))
    _check(c, ck, cv, None, rows=rows, epi=epi)
