"""GPU parity: the drafter's decoder layer, head and embedding gather through
the C ABI, against the CPU oracle (oracle/draft.py) on the same seeded
inputs.  Floating outputs: max-abs / RMS <= 2e-2 (bf16 storage: every stored
intermediate of a layer is rounded, and a value may land on either side of
a rounding boundary, so one bf16 unit of the output is allowed on top) or
1e-4 (fp32); the embedding gather is bit-exact."""
import numpy as np
import pytest

import block_diffusion_draft_ctx_amd as dfl
import oracle
import synth
from tests.gpu_util import bits, down, log, rel_err, rel_err_chained, report, up

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _case(seed, dtype, B, k, d, Hq, Hkv, D, I, ctx, qk_norm=True):
    c = synth.attention_case(seed, dtype=dtype, B=B, k=k, n_q_heads=Hq, n_kv_heads=Hkv,
                             head_dim=D, ctx_lens=ctx)
    w = synth.draft_layer_weights(seed + 1, dtype=dtype, d_model=d, n_q_heads=Hq, n_kv_heads=Hkv,
                                  head_dim=D, d_ff=I, qk_norm=qk_norm)
    rng = synth.make_rng(seed + 2)
    x = rng.standard_normal((B * k, d), dtype=np.float32)
    x = synth.bf16_bits(x) if dtype == "bf16" else x
    return c, w, x


def _gpu_layer(c, w, x, k, Hq, rope_theta, causal):
    xt = up(x, c.dtype)
    wt = {n: (None if v is None else up(v, c.dtype)) for n, v in w.items()}
    dfl.draft_layer(xt, wt, up(c.cache_k, c.dtype), up(c.cache_v, c.dtype),
                    up(c.block_table, "i32"), up(c.ctx_lens, "i32"), k, Hq,
                    rope_theta=rope_theta, causal=causal)
    return down(xt)


def _oracle_layer(c, w, x, k, Hq, rope_theta, causal, rows=None, storage_rounding=True):
    if rows is not None:
        from tests.test_gpu_attention import _subset
        sel = sorted({r // k for r in rows})
        c = _subset(c, sel)
        x = np.concatenate([x[b * k:(b + 1) * k] for b in sel])
    out = oracle.draft_layer(x, w, c.cache_k, c.cache_v, c.block_table, c.ctx_lens, k=k,
                             n_q_heads=Hq, n_kv_heads=c.n_kv_heads, head_dim=c.head_dim,
                             dtype=c.dtype, rope_theta=rope_theta, causal=causal,
                             storage_rounding=storage_rounding)
    return out


@pytest.mark.parametrize("dtype,B,k,d,Hq,Hkv,D,I,ctx,theta,causal,qkn,seed", [
    ("f32", 2, 4, 128, 4, 2, 64, 256, [37, 0], 1e4, False, True, 5101),
    ("f32", 2, 4, 128, 4, 2, 64, 256, [37, 0], 0.0, True, False, 5102),
    ("bf16", 3, 16, 256, 4, 2, 64, 384, [100, 0, 33], 1e6, False, True, 5103),
    ("bf16", 2, 16, 256, 4, 2, 64, 384, [500, 17], 1e6, True, True, 5104),
    ("bf16", 2, 16, 4096, 32, 8, 128, 12288, [300, 1000], 1e6, False, True, 5105),  # Qwen3-8B-shaped
    # 64 and 128 block rows: the few-row GEMM tiles with the residual epilogue
    ("bf16", 4, 16, 512, 8, 4, 64, 1536, [64, 0, 200, 31], 1e6, False, True, 5106),
    ("bf16", 8, 16, 512, 8, 4, 64, 1536, [16 * i + 5 for i in range(8)], 1e6, True, True, 5107),
    ("bf16", 12, 16, 512, 8, 4, 64, 1536, [40 * i for i in range(12)], 1e6, False, True, 5108),  # 192 rows
])
def test_draft_layer_parity(dtype, B, k, d, Hq, Hkv, D, I, ctx, theta, causal, qkn, seed):
    log(f"draft_layer dtype={dtype} B={B} k={k} d={d} heads={Hq}/{Hkv}x{D} I={I} ctx={ctx} "
        f"theta={theta} causal={causal}")
    c, w, x = _case(seed, dtype, B, k, d, Hq, Hkv, D, I, ctx, qkn)
    got = _gpu_layer(c, w, x, k, Hq, theta, causal)
    ref = _oracle_layer(c, w, x, k, Hq, theta, causal)
    e = rel_err_chained(got, ref, dtype, what=f"draft layer {seed}") if dtype == "bf16" \
        else rel_err(got, ref)
    log(f"  layer out err {e:.2e} (plain {rel_err(got, ref):.2e})")
    assert e <= TOL[dtype]
    # the layer's exact value (no intermediate rounding, float64 throughout):
    # the stored output is allowed only its own final rounding (bf16: half a
    # unit, 2^-8 |ref|), so the kernel's storage plan is not assumed
    exact = _oracle_layer(c, w, x, k, Hq, theta, causal, storage_rounding=False)
    rms = np.sqrt(np.mean(exact ** 2))
    half_unit = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
    e_exact = np.maximum(np.abs(got - exact) - half_unit * np.abs(exact), 0.0).max() / rms
    report(f"draft layer {seed}: against the unrounded float64 layer {e_exact:.3g} "
           f"(after the output's own half-unit storage allowance)")
    assert e_exact <= TOL[dtype]


def test_draft_layer_full_size_sampled():
    """The bench's launch: 64 requests, block 16, ctx 8192, Qwen3-8B-shaped
    layer; sampled requests against the oracle, every output finite."""
    B, k, C = 64, 16, 8192
    log(f"draft_layer full B={B} k={k} ctx={C}")
    c, w, x = _case(5111, "bf16", B, k, 4096, 32, 8, 128, 12288, [C] * B)
    got = _gpu_layer(c, w, x, k, 32, 1e6, False)
    assert np.isfinite(got).all()
    sel = [0, 41, 63]
    rows = [b * k + i for b in sel for i in range(k)]
    ref = _oracle_layer(c, w, x, k, 32, 1e6, False, rows=rows)
    e = rel_err_chained(got[rows], ref, "bf16", what="draft layer, 64-request launch")
    log(f"  sampled layer out err {e:.2e}")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("dtype,M,d,V,seed", [
    ("f32", 8, 128, 384, 5201), ("bf16", 32, 4096, 151936, 5202), ("bf16", 5, 256, 1024, 5203),
])
def test_draft_head_parity(dtype, M, d, V, seed):
    log(f"draft_head dtype={dtype} M={M} d={d} V={V}")
    rng = synth.make_rng(seed)
    x = rng.standard_normal((M, d), dtype=np.float32)
    wn = 1 + 0.1 * rng.standard_normal(d, dtype=np.float32)
    wl = 0.02 * rng.standard_normal((V, d), dtype=np.float32)
    if dtype == "bf16":
        x, wn, wl = synth.bf16_bits(x), synth.bf16_bits(wn), synth.bf16_bits(wl)
    got = down(dfl.draft_head(up(x, dtype), up(wn, dtype), up(wl, dtype)))
    ref = oracle.draft_head(x, wn, wl, dtype)
    e = rel_err_chained(got, ref, dtype, what=f"draft head {seed}") if dtype == "bf16" \
        else rel_err(got, ref)
    log(f"  logits err {e:.2e}")
    assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_embed_bit_exact_and_invalid_token(dtype):
    rng = synth.make_rng(5301)
    table = rng.standard_normal((1000, 256), dtype=np.float32)
    if dtype == "bf16":
        table = synth.bf16_bits(table)
    tok = np.array([[5, 999, 0, 5], [7, 1000, -1, 3]])
    out = dfl.embed(up(table, dtype), up(tok, "i32"))
    got = bits(out)
    ok = np.array([5, 999, 0, 5, 7, 3])
    rows = [0, 1, 2, 3, 4, 7]
    ref = oracle.embed(table, tok.reshape(-1)[rows], dtype)
    np.testing.assert_array_equal(down(out)[rows], ref)
    assert np.isnan(down(out)[[5, 6]]).all()
