"""The rest of the draft model around block attention -- oracle.

Test infrastructure: see the package header for who may import this.

Follows [DFlash overview], section "草稿模型架构": the drafter is a small
Qwen3-style decoder-only transformer that shares the target's embedding table
and output projection (lm_head); its input block is the anchor followed by
mask tokens (section "块扩散"), and each layer's attention sees the injected
target context ("KV 注入", computed by ``materialize``) and the block itself
(``block_attention``).

One layer, for the block rows x [B*k, d] (request-major, k rows each):
    n1  = rms_norm(x, w_ln1)
    q, kb, vb = split(n1 @ W_qkv^T)              (Hq, Hkv, Hkv heads of D)
    q  = rope(rms_norm_head(q, w_qn), pos);  kb = rope(rms_norm_head(kb, w_kn), pos)
    a  = block_attention(q, kb, vb, ctx cache)   (the context and the whole block)
    x1 = x + a @ W_o^T
    n2 = rms_norm(x1, w_ln2)
    g, u = split(n2 @ W_gu^T)                    (gate rows first, then up)
    x2 = x1 + (silu(g) * u) @ W_down^T
and the head: logits = rms_norm(x, w_final) @ W_lm^T.

Readings where the pages leave a step open (also in the design doc):
* the Qwen3 layer layout: pre-norm RMSNorm (x / sqrt(mean(x^2) + eps) * w),
  per-head RMSNorm of q and k before the rotary embedding (the same k_norm
  the K epilogue of materialisation applies to the context keys), half-split
  rotary embedding, SwiGLU MLP, residual adds, no biases;
* positions: block position i of request b sits at ctx_lens[b] + i (the
  context holds positions [0, ctx_lens[b]));
* storage: every intermediate that a kernel stores is rounded to the storage
  type there (the normed rows, the q/k/v projection, q and k after their norm
  and rotation, the attention output, each projection's product before its
  residual add, the sum after it, the gated product, the logits); the oracle
  rounds at exactly those points and computes in float64 between them.
"""
import numpy as np

from .attention import block_attention
from .materialize import k_norm, rope_half_split
from .numerics import round_to, widen


def rms_norm(x, w, eps):
    """x [..., d] float64 / sqrt(mean(x^2) + eps) * w."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def silu(g):
    return g / (1.0 + np.exp(-g))


def embed(table, tokens, dtype):
    """Rows of the shared embedding table [V, d] for tokens [B, k] -> [B*k, d]."""
    t = widen(table, dtype)
    return t[np.asarray(tokens).reshape(-1)]


def draft_layer(x, w, cache_k, cache_v, block_table, ctx_lens, *, k, n_q_heads, n_kv_heads,
                head_dim, dtype, eps=1e-6, rope_theta=1e6, causal=False, storage_rounding=True):
    """One drafter layer on the stored block rows x [B*k, d].  ``w`` holds the
    stored weights: ln1 [d], qkv [(Hq + 2 Hkv) D, d], q_norm / k_norm [D] or
    None, o [d, Hq D], ln2 [d], gate_up [2 I, d], down [d, I].  cache_k/v are
    this layer's injected context.  Returns x2 [B*k, d], on the storage grid
    when ``storage_rounding`` (the default); with it off, every step after
    widening the inputs stays in float64 (the layer's exact value for the
    stored inputs, which the rounded form approximates)."""
    if storage_rounding:
        round_to_storage = lambda v: round_to(v, dtype)
    else:
        round_to_storage = lambda v: v
    X = widen(x, dtype)
    M, d = X.shape
    B = M // k
    Hq, Hkv, D = n_q_heads, n_kv_heads, head_dim
    W = {name: (None if v is None else widen(v, dtype)) for name, v in w.items()}
    n1 = round_to_storage(rms_norm(X, W["ln1"], eps))
    qkv = round_to_storage(n1 @ W["qkv"].T)
    q = qkv[:, :Hq * D].reshape(M, Hq, D)
    kb = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D)
    vb = qkv[:, (Hq + Hkv) * D:].reshape(M, Hkv, D)
    pos = (np.asarray(ctx_lens, dtype=np.int64)[:, None] + np.arange(k)[None, :]).reshape(-1)
    if W["q_norm"] is not None:
        q = k_norm(q, W["q_norm"], eps)
    if W["k_norm"] is not None:
        kb = k_norm(kb, W["k_norm"], eps)
    if rope_theta > 0:
        q = rope_half_split(q, pos, rope_theta)
        kb = rope_half_split(kb, pos, rope_theta)
    q, kb = round_to_storage(q), round_to_storage(kb)
    # block_attention widens its inputs from storage: hand it the float64
    # values (on the storage grid when rounding), declared as float64
    a, _ = block_attention(q.reshape(B, k, Hq, D), kb.reshape(B, k, Hkv, D), vb.reshape(B, k, Hkv, D),
                           widen(cache_k, dtype), widen(cache_v, dtype), block_table, ctx_lens,
                           "f64", causal=causal)
    a = round_to_storage(a.reshape(M, Hq * D))
    x1 = round_to_storage(X + round_to_storage(a @ W["o"].T))
    n2 = round_to_storage(rms_norm(x1, W["ln2"], eps))
    gu = round_to_storage(n2 @ W["gate_up"].T)
    I = gu.shape[1] // 2
    h = round_to_storage(silu(gu[:, :I]) * gu[:, I:])
    return round_to_storage(x1 + round_to_storage(h @ W["down"].T))


def draft_head(x, w_norm, w_lm, dtype, eps=1e-6):
    """logits [M, V] = rms_norm(x, w_norm) @ W_lm^T, on the storage grid."""
    n = round_to(rms_norm(widen(x, dtype), widen(w_norm, dtype), eps), dtype)
    return round_to(n @ widen(w_lm, dtype).T, dtype)
