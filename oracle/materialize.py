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
* no normalisation, K-norm or RoPE is applied (the page's formula has none);
* the per-layer context transform named in section 4.1 has no body on the
  page and is taken as the identity.
"""
import numpy as np

from .numerics import widen, round_to

PAGE = 16


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


def materialize(hiddens, W_f, b_f, W_K, W_V, n_kv_heads, head_dim, dtype):
    """Full chain on stored inputs.  Returns dict with the stored-precision
    h_ctx [T, d] and per-layer K, V [T, Hkv, D] (float64 arrays whose values
    lie on the storage grid)."""
    hid = [widen(h, dtype) for h in hiddens]
    Wf = widen(W_f, dtype)
    bf = None if b_f is None else widen(b_f, dtype)
    h = round_to(fuse_hiddens(hid, Wf, bf), dtype)
    K = [round_to(project_kv(h, widen(w, dtype), n_kv_heads, head_dim), dtype) for w in W_K]
    V = [round_to(project_kv(h, widen(w, dtype), n_kv_heads, head_dim), dtype) for w in W_V]
    return {"h_ctx": h, "K": K, "V": V}


def paged_write(cache, rows, block_table, rows_per_seq, seq_start_pos, commit_lens=None):
    """Write ``rows`` [T, Hkv, D] into ``cache`` [num_pages, 16, Hkv, D] in place.

    Row r belongs to request s = r // rows_per_seq at logical position
    seq_start_pos[s] + (r mod rows_per_seq).  It is written only if its index
    within the request is below commit_lens[s] (when given) and its logical
    page is mapped (block_table entry >= 0).  Returns a bool [num_pages, 16]
    marking the slots written."""
    written = np.zeros(cache.shape[:2], dtype=bool)
    T = rows.shape[0]
    for r in range(T):
        s, i = divmod(r, rows_per_seq)
        if commit_lens is not None and i >= commit_lens[s]:
            continue
        pos = int(seq_start_pos[s]) + i
        page = int(block_table[s, pos // PAGE])
        if page < 0:
            continue
        cache[page, pos % PAGE] = rows[r]
        written[page, pos % PAGE] = True
    return written


def gather_paged(cache, block_table_row, n):
    """Logical positions [0, n) of one request -> [n, Hkv, D]."""
    pos = np.arange(n)
    pages = block_table_row[pos // PAGE]
    return cache[pages, pos % PAGE]
