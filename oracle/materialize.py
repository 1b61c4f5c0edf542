"""Target-context KV injection ("materialisation") -- oracle.

Test infrastructure: see the package header for who may import this.

Follows [DFlash overview, section "KV 注入", steps 2-3]: the m captured target
hidden states are concatenated along the feature axis and fused by one linear
layer, h_ctx = W_f [h_l1; ...; h_lm] + b_f with W_f of shape d x (m d); every
draft layer l then projects h_ctx with its own W_K^(l) and W_V^(l) and the
results are stored in that layer's KV cache.  [SGLang DFlash, section 4.1]
gives the same chain (fuse, per-layer K/V projection, write only the first
commit_lens rows of each request into its paged slots).

Readings where the pages are silent (listed in the design doc as well):
* concatenation order = the order the hiddens are supplied in;
* weights are stored [out, in] as the page writes W_f (d rows, m d columns),
  so h_ctx = X @ W_f.T and K = h_ctx @ W_K.T;
* h_ctx is rounded to the storage type before the K/V projections (the point
  where a kernel hands it from one GEMM to the next), and K/V are rounded to
  the storage type when written;
* no normalisation of h_ctx (the page's formula has none);
* the per-layer context transform named in section 4.1 has no body on the
  page and is taken as the identity.

Optional K epilogue ([SGLang DFlash, section 4.1]: kv_proj_only, then
apply_k_norm, then apply_k_rope(positions, k), then the prefix-valid write).
The page names the two steps without their bodies; the readings are:
* k_norm: RMSNorm of each head's K over head_dim with the layer's weight w
  [D]:  k / sqrt(mean(k^2) + eps) * w;
* rope: the rotary position embedding, half-split layout -- dims i and
  i + D/2 (i < D/2) form a pair rotated by the angle pos * theta^(-2i/D):
  (x, y) -> (x cos a - y sin a, y cos a + x sin a);
* pos is the row's logical position (seq_start_pos[s] + r mod rows_per_seq,
  the position that also chooses its cache slot);
* the epilogue acts on the stored K projection (rounded to the storage type,
  as the projection hands it over) and its result is rounded once when
  stored; V is untouched.
"""
import numpy as np

from .numerics import widen, round_to

PAGE = 16


def slots(cache):
    """The paged cache is stored head-major, [num_pages, Hkv, PAGE, D] (a
    page's positions of one kv-head lie together).  This returns the
    [num_pages, PAGE, Hkv, D] view of it by page position; it is a view, so
    writes through it land in ``cache``."""
    return np.swapaxes(cache, 1, 2)


def fuse_hiddens(hiddens, W_f, b_f=None):
    """h_ctx = [h_1; ...; h_m] W_f^T + b_f in float64 (no rounding)."""
    X = np.concatenate(list(hiddens), axis=1)
    h = X @ W_f.T
    if b_f is not None:
        h = h + b_f[None, :]
    return h


def project_kv(h_ctx, W, n_kv_heads, head_dim):
    """[T, d] @ W^T -> [T, Hkv, D] in float64."""
    out = h_ctx @ W.T
    return out.reshape(h_ctx.shape[0], n_kv_heads, head_dim)


def k_norm(K, weight, eps):
    """Per-head RMSNorm over head_dim: K [T, Hkv, D] float64, weight [D]."""
    ms = np.mean(K * K, axis=-1, keepdims=True)
    return K / np.sqrt(ms + eps) * weight


def rope_half_split(K, positions, theta):
    """Rotary embedding of K [T, Hkv, D] at positions [T] (float64): dims i
    and i + D/2 rotate by positions * theta^(-2i/D)."""
    D = K.shape[-1]
    half = D // 2
    inv_freq = theta ** (-2.0 * np.arange(half) / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]   # [T, D/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x, y = K[..., :half], K[..., half:]
    return np.concatenate([x * c - y * s, y * c + x * s], axis=-1)


def row_positions(T, rows_per_seq, seq_start_pos):
    """Logical position of every row: seq_start_pos[r // rows_per_seq] + r mod rows_per_seq."""
    r = np.arange(T)
    return np.asarray(seq_start_pos, dtype=np.int64)[r // rows_per_seq] + r % rows_per_seq


def materialize(hiddens, W_f, b_f, W_K, W_V, n_kv_heads, head_dim, dtype, k_norm_weight=None,
                k_norm_eps=1e-6, rope_theta=0.0, rows_per_seq=None, seq_start_pos=None):
    """Full chain on stored inputs.  Returns dict with the stored-precision
    h_ctx [T, d] and per-layer K, V [T, Hkv, D] (float64 arrays whose values
    lie on the storage grid).  With k_norm_weight (per layer [D]) and/or
    rope_theta > 0, K goes through the epilogue (norm, then rotary embedding
    at each row's logical position, which needs rows_per_seq and
    seq_start_pos) before it is stored."""
    hid = [widen(h, dtype) for h in hiddens]
    Wf = widen(W_f, dtype)
    bf = None if b_f is None else widen(b_f, dtype)
    h = round_to(fuse_hiddens(hid, Wf, bf), dtype)
    K = [round_to(project_kv(h, widen(w, dtype), n_kv_heads, head_dim), dtype) for w in W_K]
    V = [round_to(project_kv(h, widen(w, dtype), n_kv_heads, head_dim), dtype) for w in W_V]
    if k_norm_weight is not None or rope_theta > 0:
        pos = row_positions(h.shape[0], rows_per_seq, seq_start_pos) if rope_theta > 0 else None
        for l in range(len(K)):
            k = K[l]
            if k_norm_weight is not None:
                k = k_norm(k, widen(k_norm_weight[l], dtype), k_norm_eps)
            if rope_theta > 0:
                k = rope_half_split(k, pos, rope_theta)
            K[l] = round_to(k, dtype)
    return {"h_ctx": h, "K": K, "V": V}


def paged_write(cache, rows, block_table, rows_per_seq, seq_start_pos, commit_lens=None):
    """Write ``rows`` [T, Hkv, D] into ``cache`` [num_pages, Hkv, 16, D] in place.

    Row r belongs to request s = r // rows_per_seq at logical position
    seq_start_pos[s] + (r mod rows_per_seq).  It is written only if its index
    within the request is below commit_lens[s] (when given) and its logical
    page is mapped (block_table entry >= 0).  Returns a bool [num_pages, 16]
    marking the slots written."""
    sv = slots(cache)
    written = np.zeros(sv.shape[:2], dtype=bool)
    T = rows.shape[0]
    for r in range(T):
        s, i = divmod(r, rows_per_seq)
        if commit_lens is not None and i >= commit_lens[s]:
            continue
        pos = int(seq_start_pos[s]) + i
        page = int(block_table[s, pos // PAGE])
        if page < 0:
            continue
        sv[page, pos % PAGE] = rows[r]
        written[page, pos % PAGE] = True
    return written


def gather_paged(cache, block_table_row, n):
    """Logical positions [0, n) of one request -> [n, Hkv, D]."""
    pos = np.arange(n)
    pages = block_table_row[pos // PAGE]
    return slots(cache)[pages, pos % PAGE]
