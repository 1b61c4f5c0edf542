"""Non-causal block attention over injected context K/V -- oracle.

Test infrastructure: see the package header for who may import this.

Follows [DFlash overview, section "KV 注入", step 3 and its Attention
formula]: a draft query attends to the concatenation of the injected context
keys/values and the block's own keys/values; [DFlash overview, section
"块扩散"]: attention inside the block is bidirectional (no causal mask); and
[DFlash overview, section "随机锚点采样"]: in packed training every block sees
the injected target context, sees all of its own positions, and none of the
other blocks.

For request b, q-head h, block position i, with G = Hq / Hkv and g = h // G:
    keys   = [K_ctx[b, 0:C_b, g]; K_blk[b, 0:k, g]]
    values = [V_ctx[b, 0:C_b, g]; V_blk[b, 0:k, g]]
    s      = scale * keys @ q[b, i, h],   scale = 1/sqrt(D) unless given
    o      = softmax(s) @ values,         lse = log(sum(exp(s)))

Causal variant (``causal=True``), following [DFlash overview, section
"块扩散的双向注意力问题"] (the JetSpec change): inside the block, position i
sees only the block positions 0..i; the injected context stays fully visible.
The block-causal mask of [Spec tutorial, section 5.3] (a block sees every
earlier block and all of itself) is the default mode applied to a context that
holds the earlier blocks.

Readings (also in the design doc): GQA groups are contiguous (q-head h reads kv-head
h // G); the visible context of a request is its logical positions [0, C_b),
strictly before the anchor; C_b = 0 is allowed; Q and K arrive already
position-encoded (no RoPE inside); the block's own K/V are an input and are
not written to the cache.
"""
import numpy as np

from .materialize import slots
from .numerics import widen

PAGE = 16


def _softmax_rows(s):
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, (m + np.log(l))[..., 0]


def block_attention(q, k_blk, v_blk, cache_k, cache_v, block_table, ctx_lens, dtype,
                    scale=None, causal=False):
    """Per-request gather form.  Returns (out [B, k, Hq, D], lse [B, Hq, k]).
    With ``causal`` the score of block key j for block position i is removed
    when j > i."""
    q, kb, vb = widen(q, dtype), widen(k_blk, dtype), widen(v_blk, dtype)
    ck, cv = widen(cache_k, dtype), widen(cache_v, dtype)
    B, k, Hq, D = q.shape
    Hkv = kb.shape[2]
    G = Hq // Hkv
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, k, Hq, D))
    lse = np.zeros((B, Hq, k))
    for b in range(B):
        C = int(ctx_lens[b])
        pos = np.arange(C)
        pages = block_table[b, pos // PAGE]
        keys = np.concatenate([slots(ck)[pages, pos % PAGE], kb[b]], axis=0)   # [C+k, Hkv, D]
        vals = np.concatenate([slots(cv)[pages, pos % PAGE], vb[b]], axis=0)
        for h in range(Hq):
            g = h // G
            s = scale * (q[b, :, h, :] @ keys[:, g, :].T)               # [k, C+k]
            if causal:
                s[:, C:] = np.where(np.tril(np.ones((k, k), dtype=bool)), s[:, C:], -np.inf)
            p, l = _softmax_rows(s)
            out[b, :, h, :] = p @ vals[:, g, :]
            lse[b, h, :] = l
    return out, lse


def block_attention_masked(q, k_blk, v_blk, cache_k, cache_v, block_table, ctx_lens, dtype,
                           scale=None, causal=False):
    """Brute force with an explicit boolean mask over *every* key that exists:
    all physical cache slots followed by every request's block keys.  A query
    of request b may see slot (page, j) iff that slot holds one of b's logical
    positions < C_b, and may see block key (b', i') iff b' == b (and, with
    ``causal``, i' <= its own block position).  Exponentials of masked scores
    are dropped explicitly.  Same outputs as ``block_attention``; used to pin
    it."""
    q, kb, vb = widen(q, dtype), widen(k_blk, dtype), widen(v_blk, dtype)
    ck, cv = slots(widen(cache_k, dtype)), slots(widen(cache_v, dtype))   # [P, PAGE, Hkv, D]
    B, k, Hq, D = q.shape
    P, _, Hkv, _ = ck.shape
    G = Hq // Hkv
    if scale is None or scale == 0.0:
        scale = 1.0 / np.sqrt(D)
    n_slots = P * PAGE
    keys = np.concatenate([ck.reshape(n_slots, Hkv, D), kb.reshape(B * k, Hkv, D)], axis=0)
    vals = np.concatenate([cv.reshape(n_slots, Hkv, D), vb.reshape(B * k, Hkv, D)], axis=0)
    mask = np.zeros((B, n_slots + B * k), dtype=bool)
    for b in range(B):
        for pos in range(int(ctx_lens[b])):
            mask[b, block_table[b, pos // PAGE] * PAGE + pos % PAGE] = True
        mask[b, n_slots + b * k: n_slots + (b + 1) * k] = True
    out = np.zeros((B, k, Hq, D))
    lse = np.zeros((B, Hq, k))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(k):
                vis = mask[b].copy()
                if causal:
                    vis[n_slots + b * k + i + 1: n_slots + (b + 1) * k] = False
                s = scale * (keys[:, g, :] @ q[b, i, h, :])
                m = s[vis].max()
                e = np.where(vis, np.exp(s - m), 0.0)
                out[b, i, h] = (e @ vals[:, g, :]) / e.sum()
                lse[b, h, i] = m + np.log(e.sum())
    return out, lse
