"""Seeded synthetic inputs for the DFlash draft-and-verify step.

This module only *draws* inputs: hidden states, weights, logits, uniforms,
page tables and anchor lists.  It holds none of the step's arithmetic (no
fusion, projection, attention, softmax or acceptance), so both the CPU oracle
tests and the GPU path can take their inputs from here without sharing any
computation.

Conventions
-----------
* One ``numpy.random.default_rng(seed)`` (PCG64) per case; callers use
  ``seed = 1000 * workload_id + case``.
* Floating tensors are drawn in float32.  bf16 tensors are returned as
  ``uint16`` arrays holding the bf16 bit patterns, obtained from the float32
  draw by round-to-nearest-even on the upper 16 bits.  fp32 tensors are
  returned as ``float32`` arrays.
* Uniforms are ``int * 2**-24`` with ``int`` in ``[0, 2**24)``, so every value
  is exactly representable in float32 and lies in ``[0, 1)``.
* Paged KV caches use pages of 16 token slots, shape
  ``[num_pages, n_kv_heads, 16, head_dim]`` (head-major); the physical page order is a
  seeded random permutation, and ``block_table[seq, logical_page]`` maps a
  sequence's logical page to a physical page (``-1`` = unmapped).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

PAGE = 16
BF16 = "bf16"
F32 = "f32"
CACHE_SENTINEL_BF16 = np.uint16(0x7FA1)  # a NaN pattern: any stray read shows up
CACHE_SENTINEL_F32_BITS = np.uint32(0x7FC0DEAD)


def make_rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    return ((u + bias) >> 16).astype(np.uint16)


def _draw(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x) if dtype == BF16 else x


def uniforms(rng, shape) -> np.ndarray:
    return (rng.integers(0, 1 << 24, size=shape, dtype=np.int64).astype(np.float64)
            * 2.0 ** -24).astype(np.float32)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Input view as float64 (bf16 bits widened exactly).  Used by the
    generators themselves (e.g. to draw drafts from q); tests hand the raw
    arrays to both sides."""
    if dtype == BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# paged layout
# ----------------------------------------------------------------------------

def page_table(rng, n_positions: Sequence[int], max_pages: Optional[int] = None,
               spare_pages: int = 0, shuffle: bool = True):
    """Pages covering positions [0, n) of each sequence.

    Returns (block_table int32 [n_seq, max_pages], num_pages)."""
    need = [int(math.ceil(n / PAGE)) for n in n_positions]
    if max_pages is None:
        max_pages = max(1, max(need) if need else 1)
    total = sum(need) + spare_pages
    phys = rng.permutation(total) if shuffle else np.arange(total)
    bt = np.full((len(need), max_pages), -1, dtype=np.int32)
    at = 0
    for s, n in enumerate(need):
        assert n <= max_pages
        bt[s, :n] = phys[at:at + n]
        at += n
    return bt, max(total, 1)


def empty_cache(num_pages, n_kv_heads, head_dim, dtype):
    shape = (num_pages, n_kv_heads, PAGE, head_dim)
    if dtype == BF16:
        return np.full(shape, CACHE_SENTINEL_BF16, dtype=np.uint16)
    return np.full(shape, CACHE_SENTINEL_F32_BITS, dtype=np.uint32).view(np.float32)


# ----------------------------------------------------------------------------
# materialisation
# ----------------------------------------------------------------------------

@dataclass
class MaterializeCase:
    dtype: str
    m: int
    d_model: int
    n_layers: int
    n_kv_heads: int
    head_dim: int
    n_seq: int
    rows_per_seq: int
    hiddens: List[np.ndarray]          # m x [T, d]
    W_f: np.ndarray                    # [d, m*d]
    b_f: Optional[np.ndarray]          # [d]
    W_K: List[np.ndarray]              # n_layers x [Hkv*D, d]
    W_V: List[np.ndarray]
    seq_start_pos: np.ndarray          # [n_seq] int32
    commit_lens: Optional[np.ndarray]  # [n_seq] int32 or None
    block_table: np.ndarray            # [n_seq, max_pages] int32
    num_pages: int
    cache_k: List[np.ndarray] = field(default_factory=list)  # per layer, sentinel-filled
    cache_v: List[np.ndarray] = field(default_factory=list)

    @property
    def T(self):
        return self.n_seq * self.rows_per_seq


def materialize_case(seed, *, dtype, m, d_model, n_layers, n_kv_heads, head_dim,
                     n_seq, rows_per_seq, start_pos=None, commit=None,
                     bias=True, w_std=0.02, h_std=1.0, spare_pages=1,
                     max_pages=None) -> MaterializeCase:
    """Draw order: hiddens, W_f, b_f, W_K (all layers), W_V (all layers),
    start positions, commit lengths, page permutation."""
    rng = make_rng(seed)
    T = n_seq * rows_per_seq
    hid = [_draw(rng, (T, d_model), h_std, dtype) for _ in range(m)]
    W_f = _draw(rng, (d_model, m * d_model), w_std, dtype)
    b_f = _draw(rng, (d_model,), 0.02, dtype) if bias else None
    W_K = [_draw(rng, (n_kv_heads * head_dim, d_model), w_std, dtype) for _ in range(n_layers)]
    W_V = [_draw(rng, (n_kv_heads * head_dim, d_model), w_std, dtype) for _ in range(n_layers)]
    if start_pos is None:
        start_pos = rng.integers(0, 64, size=n_seq)
    elif np.isscalar(start_pos):
        start_pos = np.full(n_seq, int(start_pos))
    start_pos = np.asarray(start_pos, dtype=np.int32)
    if isinstance(commit, str) and commit == "random":
        commit_lens = rng.integers(1, rows_per_seq + 1, size=n_seq).astype(np.int32)
    elif commit is None:
        commit_lens = None
    else:
        commit_lens = np.asarray(commit, dtype=np.int32)
    ends = [int(start_pos[s]) + rows_per_seq for s in range(n_seq)]
    bt, num_pages = page_table(rng, ends, max_pages=max_pages, spare_pages=spare_pages)
    ck = [empty_cache(num_pages, n_kv_heads, head_dim, dtype) for _ in range(n_layers)]
    cv = [empty_cache(num_pages, n_kv_heads, head_dim, dtype) for _ in range(n_layers)]
    return MaterializeCase(dtype, m, d_model, n_layers, n_kv_heads, head_dim, n_seq,
                           rows_per_seq, hid, W_f, b_f, W_K, W_V, start_pos, commit_lens,
                           bt, num_pages, ck, cv)


def k_norm_weights(seed, *, n_layers, head_dim, dtype):
    """Per-layer norm weights [head_dim], uniform on [0.5, 1.5), stored in
    the given dtype (a trained norm weight's scale, drawn at random)."""
    rng = make_rng(seed)
    out = []
    for _ in range(n_layers):
        x = rng.uniform(0.5, 1.5, size=head_dim).astype(np.float32)
        out.append(bf16_bits(x) if dtype == BF16 else x)
    return out


# ----------------------------------------------------------------------------
# block attention
# ----------------------------------------------------------------------------

@dataclass
class AttentionCase:
    dtype: str
    B: int
    k: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    q: np.ndarray            # [B, k, Hq, D]
    k_blk: np.ndarray        # [B, k, Hkv, D]
    v_blk: np.ndarray
    cache_k: np.ndarray      # [num_pages, Hkv, 16, D]
    cache_v: np.ndarray
    block_table: np.ndarray  # [B, max_pages] int32
    ctx_lens: np.ndarray     # [B] int32


def attention_case(seed, *, dtype, B, k, n_q_heads, n_kv_heads, head_dim, ctx_lens,
                   q_scale=1.0, kv_std=1.0, max_pages=None, shuffle=True) -> AttentionCase:
    """Draw order: Q, K_blk, V_blk, page permutation, cache K, cache V."""
    rng = make_rng(seed)
    ctx_lens = np.asarray(ctx_lens, dtype=np.int32)
    assert ctx_lens.shape == (B,)
    q = _draw(rng, (B, k, n_q_heads, head_dim), q_scale, dtype)
    kb = _draw(rng, (B, k, n_kv_heads, head_dim), kv_std, dtype)
    vb = _draw(rng, (B, k, n_kv_heads, head_dim), kv_std, dtype)
    bt, num_pages = page_table(rng, [int(c) for c in ctx_lens], max_pages=max_pages,
                               shuffle=shuffle)
    ck = _draw(rng, (num_pages, n_kv_heads, PAGE, head_dim), kv_std, dtype)
    cv = _draw(rng, (num_pages, n_kv_heads, PAGE, head_dim), kv_std, dtype)
    return AttentionCase(dtype, B, k, n_q_heads, n_kv_heads, head_dim, q, kb, vb, ck, cv,
                         bt, ctx_lens)


def packed_anchors(rng, seq_len, k, max_anchors=512, prompt_range=(256, 2048)):
    """Training-style anchors: a prompt prefix P ~ U{lo..hi} has loss_mask 0,
    the rest 1; candidate anchors are positions a whose whole block
    [a, a+k) lies in the loss region; a shuffled candidate list is accepted
    greedily when it does not overlap an accepted block, up to max_anchors.
    Returns (sorted anchors int32, P)."""
    P = int(rng.integers(prompt_range[0], prompt_range[1] + 1))
    cand = np.arange(P, seq_len - k + 1)
    rng.shuffle(cand)
    taken = np.zeros(seq_len, dtype=bool)
    out = []
    for a in cand:
        if len(out) >= max_anchors:
            break
        if not taken[a:a + k].any():
            taken[a:a + k] = True
            out.append(int(a))
    return np.array(sorted(out), dtype=np.int32), P


def packed_attention_case(seed, *, dtype=BF16, seq_len=8192, k=16, n_q_heads=32,
                          n_kv_heads=8, head_dim=128, max_anchors=512,
                          prompt_range=(256, 2048), kv_std=1.0):
    """One packed training sequence mapped onto block attention: every block
    row of the page table points at the same sequence's pages and its ctx
    length is its anchor, so a block sees exactly the target positions before
    its anchor plus its own k positions.
    Draw order: prompt length and anchors, Q, K_blk, V_blk, page permutation,
    cache K, cache V."""
    rng = make_rng(seed)
    anchors, P = packed_anchors(rng, seq_len, k, max_anchors, prompt_range)
    nb = len(anchors)
    q = _draw(rng, (nb, k, n_q_heads, head_dim), 1.0, dtype)
    kb = _draw(rng, (nb, k, n_kv_heads, head_dim), kv_std, dtype)
    vb = _draw(rng, (nb, k, n_kv_heads, head_dim), kv_std, dtype)
    bt1, num_pages = page_table(rng, [seq_len])
    bt = np.repeat(bt1, nb, axis=0)
    ck = _draw(rng, (num_pages, n_kv_heads, PAGE, head_dim), kv_std, dtype)
    cv = _draw(rng, (num_pages, n_kv_heads, PAGE, head_dim), kv_std, dtype)
    case = AttentionCase(dtype, nb, k, n_q_heads, n_kv_heads, head_dim, q, kb, vb, ck, cv,
                         np.ascontiguousarray(bt), anchors.copy())
    return case, P


# ----------------------------------------------------------------------------
# verification
# ----------------------------------------------------------------------------

@dataclass
class GreedyCase:
    dtype: str
    B: int
    L: int
    V: int
    target_logits: np.ndarray           # [B, L+1, V]
    draft_logits: Optional[np.ndarray]  # [B, L, V] or None
    draft_tokens: np.ndarray            # [B, L] int32 (input when draft_logits is None)
    chain_lens: Optional[np.ndarray]
    prefix_lens: np.ndarray             # [B] int32
    planted_accept: Optional[np.ndarray]


def greedy_case(seed, *, dtype, B, L, V, std=3.0, plant=True, with_draft_logits=False,
                ties=0, chain=None, boost=30.0) -> GreedyCase:
    """Target logits ~ N(0, std).  With ``plant``, a chosen token per row is
    raised to ``boost`` (far above any N(0, std) draw) so the row's top token
    is known by construction, and the drafts copy it for the first a_b rows
    (a_b ~ U{0..L}) and differ at row a_b.  ``ties`` rows get a second token
    set to the same boosted value (a planted exact tie).
    Draw order: target logits, planted tokens, planted lengths, tie rows,
    draft logits / tokens, chain lengths, prefix lengths."""
    rng = make_rng(seed)
    t = rng.standard_normal(size=(B, L + 1, V), dtype=np.float32) * np.float32(std)
    top = rng.integers(0, V, size=(B, L + 1))
    acc = rng.integers(0, L + 1, size=B) if plant else None
    tie_rows = []
    if plant:
        t[np.arange(B)[:, None], np.arange(L + 1)[None, :], top] = boost
        for _ in range(ties):
            b = int(rng.integers(0, B)); i = int(rng.integers(0, L + 1))
            other = int(rng.integers(0, V))
            t[b, i, other] = boost
            tie_rows.append((b, i, other))
    drafts = rng.integers(0, V, size=(B, L)).astype(np.int64)
    if plant:
        for b in range(B):
            drafts[b, :acc[b]] = top[b, :acc[b]]
            if acc[b] < L:
                # a token that is certainly not the planted top (ties aside)
                drafts[b, acc[b]] = (top[b, acc[b]] + 1 + rng.integers(0, V - 1)) % V
    dl = None
    if with_draft_logits:
        dl = rng.standard_normal(size=(B, L, V), dtype=np.float32) * np.float32(std)
        dl[np.arange(B)[:, None], np.arange(L)[None, :], drafts] = boost
    if chain is None:
        chain_lens = None
    elif isinstance(chain, str) and chain == "random":
        chain_lens = rng.integers(0, L + 1, size=B).astype(np.int32)
    else:
        chain_lens = np.asarray(chain, dtype=np.int32)
    prefix = rng.integers(1, 4096, size=B).astype(np.int32)
    conv = bf16_bits if dtype == BF16 else (lambda a: a)
    return GreedyCase(dtype, B, L, V, conv(t), None if dl is None else conv(dl),
                      drafts.astype(np.int32), chain_lens, prefix, acc)


@dataclass
class SampleCase:
    dtype: str
    B: int
    L: int
    V: int
    temperature: float
    target_logits: np.ndarray   # [B, L+1, V]
    draft_logits: np.ndarray    # [B, L, V]
    draft_tokens: np.ndarray    # [B, L] int32, drawn from q
    chain_lens: Optional[np.ndarray]
    u_accept: np.ndarray        # [B, L] float32
    u_bonus: np.ndarray         # [B] float32
    prefix_lens: np.ndarray


def _gumbel_pick(rng, logits64, temperature):
    """One draw from softmax(logits / T) per row by the Gumbel-max trick."""
    g = -np.log(-np.log(rng.random(size=logits64.shape)))
    return np.argmax(logits64 / temperature + g, axis=-1)


def sample_case(seed, *, dtype, B, L, V, std=3.0, sigma=1.0, temperature=1.0,
                chain=None, boost_stages=None, stage=8, boost=0.0) -> SampleCase:
    """Target logits ~ N(0, std), draft = target + N(0, sigma) (both rounded
    to the storage type), drafts drawn from q = softmax(draft / T).  With
    ``boost`` > 0, for the listed stages (blocks of ``stage`` drafts) the drawn
    draft token is raised by ``boost`` on both the target row and the draft
    row, which plants high-confidence stages.
    Draw order: target noise, draft noise, draft tokens (Gumbel), chain
    lengths, u, u', prefix lengths."""
    rng = make_rng(seed)
    t = rng.standard_normal(size=(B, L + 1, V), dtype=np.float32) * np.float32(std)
    d = t[:, :L, :] + rng.standard_normal(size=(B, L, V), dtype=np.float32) * np.float32(sigma)
    conv = bf16_bits if dtype == BF16 else (lambda a: np.ascontiguousarray(a))
    tb, db = conv(t), conv(d)
    toks = _gumbel_pick(rng, widen(db, dtype), temperature).astype(np.int64)
    if boost and boost_stages is not None:
        t2 = widen(tb, dtype).astype(np.float32)
        d2 = widen(db, dtype).astype(np.float32)
        for b in range(B):
            for s in boost_stages[b]:
                for i in range(s * stage, min((s + 1) * stage, L)):
                    x = toks[b, i]
                    t2[b, i, x] += boost
                    d2[b, i, x] += boost
        tb, db = conv(t2), conv(d2)
    if chain is None:
        chain_lens = None
    elif isinstance(chain, str) and chain == "random":
        chain_lens = rng.integers(0, L + 1, size=B).astype(np.int32)
    else:
        chain_lens = np.asarray(chain, dtype=np.int32)
    u = uniforms(rng, (B, L))
    u2 = uniforms(rng, (B,))
    prefix = rng.integers(1, 4096, size=B).astype(np.int32)
    return SampleCase(dtype, B, L, V, float(temperature), tb, db, toks.astype(np.int32),
                      chain_lens, u, u2, prefix)


@dataclass
class GateCase:
    dtype: str
    B: int
    n: int
    V: int
    temperature: float
    g: float
    draft_logits: np.ndarray   # [B, n, V]
    draft_tokens: np.ndarray   # [B, n]
    valid_lens: Optional[np.ndarray]


def gate_case(seed, *, dtype, B, n, V, std=3.0, temperature=1.0, g=-0.5, boost=None,
              valid=None) -> GateCase:
    """Draft logits ~ N(0, std), tokens drawn from softmax(logits / T);
    with ``boost`` (array [B]) the drawn tokens of request b are raised by
    boost[b], so the block confidence straddles the threshold.
    Draw order: logits, tokens (Gumbel), valid lengths."""
    rng = make_rng(seed)
    d = rng.standard_normal(size=(B, n, V), dtype=np.float32) * np.float32(std)
    conv = bf16_bits if dtype == BF16 else (lambda a: a)
    db = conv(d)
    toks = _gumbel_pick(rng, widen(db, dtype), temperature)
    if boost is not None:
        d2 = widen(db, dtype).astype(np.float32)
        for b in range(B):
            d2[b, np.arange(n), toks[b]] += np.float32(boost[b])
        db = conv(d2)
    if valid is None:
        vl = None
    elif isinstance(valid, str) and valid == "random":
        vl = rng.integers(0, n + 1, size=B).astype(np.int32)
    else:
        vl = np.asarray(valid, dtype=np.int32)
    return GateCase(dtype, B, n, V, float(temperature), float(g), db, toks.astype(np.int32), vl)


# ----------------------------------------------------------------------------
# DDTree draft trees
# ----------------------------------------------------------------------------

@dataclass
class TreeCase:
    dtype: str
    B: int
    n_pos: int
    V: int
    draft_logits: np.ndarray    # [B, n_pos, V]: row d is block position d + 1


def tree_case(seed, *, dtype, B, n_pos, V, std=2.0, peaked=0.0) -> TreeCase:
    """Draft logits ~ N(0, std) per block position; with ``peaked`` > 0 a
    random token per row is raised by that amount (a confident drafter, so
    that the best-first tree grows deep along likely paths)."""
    rng = make_rng(seed)
    x = rng.standard_normal(size=(B, n_pos, V), dtype=np.float32) * np.float32(std)
    if peaked > 0:
        top = rng.integers(0, V, size=(B, n_pos))
        for b in range(B):
            for i in range(n_pos):
                x[b, i, top[b, i]] += np.float32(peaked)
    return TreeCase(dtype, B, n_pos, V, bf16_bits(x) if dtype == BF16 else x)


def tree_target_logits(seed, *, dtype, B, n_rows, V, std=3.0, follow=None, boost=30.0):
    """Target logits [B, n_rows, V] ~ N(0, std).  ``follow``: per request a
    list of (row, token) pairs whose token is raised by ``boost``, so the
    target's prediction at that row is known by construction."""
    rng = make_rng(seed)
    x = rng.standard_normal(size=(B, n_rows, V), dtype=np.float32) * np.float32(std)
    if follow is not None:
        for b, pairs in enumerate(follow):
            for r, t in pairs:
                x[b, r, t] += np.float32(boost)
    return bf16_bits(x) if dtype == BF16 else x


def draft_layer_weights(seed, *, dtype, d_model, n_q_heads, n_kv_heads, head_dim, d_ff,
                        qk_norm=True, std=0.02):
    """One drafter layer's weights (row-major [out, in]): projections ~N(0,
    std), norm weights 1 + N(0, 0.1).  Draw order: ln1, qkv, q_norm, k_norm,
    o, ln2, gate_up, down."""
    rng = make_rng(seed)
    D = head_dim
    w = {"ln1": 1.0 + rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.1),
         "qkv": rng.standard_normal(((n_q_heads + 2 * n_kv_heads) * D, d_model), dtype=np.float32) * np.float32(std),
         "q_norm": 1.0 + rng.standard_normal(D, dtype=np.float32) * np.float32(0.1),
         "k_norm": 1.0 + rng.standard_normal(D, dtype=np.float32) * np.float32(0.1),
         "o": rng.standard_normal((d_model, n_q_heads * D), dtype=np.float32) * np.float32(std),
         "ln2": 1.0 + rng.standard_normal(d_model, dtype=np.float32) * np.float32(0.1),
         "gate_up": rng.standard_normal((2 * d_ff, d_model), dtype=np.float32) * np.float32(std),
         "down": rng.standard_normal((d_model, d_ff), dtype=np.float32) * np.float32(std)}
    if not qk_norm:
        w["q_norm"] = w["k_norm"] = None
    return {k: (None if v is None else (bf16_bits(v.astype(np.float32)) if dtype == BF16
                                        else v.astype(np.float32))) for k, v in w.items()}
