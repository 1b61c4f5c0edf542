"""Python binding of the DFlash step library (libdflash.so, C ABI in include/dflash.h).

Argument marshalling only: tensors are PyTorch device tensors (PyTorch is
used for device memory and streams); every step of the computation runs in
the HIP kernels behind the C ABI.  There is no fallback: if the library is
missing this module raises on first use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIBRARY names another build of the same library (the AddressSanitizer
# build of the ABI tests); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("DFLASH_LIBRARY") or os.path.join(HERE, "libdflash.so")

OK, E_ARG, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_TOO_LARGE = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
MASK_BIDIRECTIONAL, MASK_CAUSAL = 0, 1

EXPORTS = (
    "dflash_status_string", "dflash_version",
    "dflash_materialize_workspace_size", "dflash_materialize_ctx_kv",
    "dflash_attention_workspace_size", "dflash_block_attention",
    "dflash_verify_greedy_noalloc", "dflash_noalloc_scratch_bytes",
    "dflash_verify_workspace_size", "dflash_verify_greedy", "dflash_verify_sample",
    "dflash_gate_workspace_size", "dflash_gate",
    "dflash_tree_workspace_size", "dflash_tree_verify_workspace_size", "dflash_tree_build",
    "dflash_tree_verify_greedy", "dflash_tree_attention_workspace_size", "dflash_tree_attention",
    "dflash_tree_commit_kv", "dflash_draft_layer_workspace_size", "dflash_draft_layer",
    "dflash_draft_head_workspace_size", "dflash_draft_head", "dflash_embed",
)


class KVLayer(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32)]


class KEpilogue(ctypes.Structure):
    _fields_ = [("k_norm_weight", ctypes.POINTER(ctypes.c_void_p)), ("k_norm_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float)]


class DraftLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ln1", "qkv", "q_norm", "k_norm", "o", "ln2",
                                                "gate_up", "down")]


class DFlashError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int
I64 = ctypes.c_int64
SZ = ctypes.c_size_t
F = ctypes.c_float
PP = ctypes.POINTER(ctypes.c_void_p)


def _declare(lib):
    lib.dflash_status_string.restype = ctypes.c_char_p
    lib.dflash_status_string.argtypes = [I32]
    lib.dflash_version.restype = I32
    lib.dflash_version.argtypes = []
    lib.dflash_materialize_workspace_size.restype = SZ
    lib.dflash_materialize_workspace_size.argtypes = [I64, I32, I32, I32, I32, I32, I32]
    lib.dflash_materialize_ctx_kv.restype = I32
    lib.dflash_materialize_ctx_kv.argtypes = [
        I64, I32, I32, PP, P, P, I32, I32, I32, PP, PP, ctypes.POINTER(KVLayer), P, I32, I32,
        P, P, ctypes.POINTER(KEpilogue), P, I32, P, SZ, P]
    lib.dflash_attention_workspace_size.restype = SZ
    lib.dflash_attention_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.dflash_block_attention.restype = I32
    lib.dflash_block_attention.argtypes = [
        I32, I32, I32, I32, I32, P, P, P, P, P, I32, I32, P, I32, I32, P, F, I32, P, P, I32, I32, P,
        SZ, P]
    lib.dflash_verify_workspace_size.restype = SZ
    lib.dflash_verify_workspace_size.argtypes = [I32, I32, I32]
    lib.dflash_verify_greedy.restype = I32
    lib.dflash_verify_greedy.argtypes = [
        I32, I32, I32, P, I64, P, I64, P, P, P, P, P, P, P, P, I32, P, SZ, P]
    lib.dflash_verify_greedy_noalloc.restype = I32
    lib.dflash_verify_greedy_noalloc.argtypes = [
        I32, I32, I32, P, I64, P, I64, P, P, P, P, P, P, P, P, I32, P]
    lib.dflash_noalloc_scratch_bytes.restype = SZ
    lib.dflash_noalloc_scratch_bytes.argtypes = []
    lib.dflash_verify_sample.restype = I32
    lib.dflash_verify_sample.argtypes = [
        I32, I32, I32, P, I64, P, I64, P, P, P, P, F, P, P, P, P, P, P, P, P, P, I32, P, SZ, P]
    lib.dflash_gate_workspace_size.restype = SZ
    lib.dflash_gate_workspace_size.argtypes = [I32, I32, I32]
    lib.dflash_gate.restype = I32
    lib.dflash_gate.argtypes = [I32, I32, I32, P, I64, P, P, F, F, P, P, P, P, I32, I32, P, SZ, P]
    lib.dflash_tree_workspace_size.restype = SZ
    lib.dflash_tree_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.dflash_tree_verify_workspace_size.restype = SZ
    lib.dflash_tree_verify_workspace_size.argtypes = [I32, I32, I32]
    lib.dflash_tree_build.restype = I32
    lib.dflash_tree_build.argtypes = [
        I32, I32, I32, P, I64, F, I32, I32, P, P, P, P, P, P, P, P, I32, P, SZ, P]
    lib.dflash_tree_verify_greedy.restype = I32
    lib.dflash_tree_verify_greedy.argtypes = [
        I32, I32, I32, P, I64, P, P, P, I32, P, P, P, P, P, P, I32, P, SZ, P]
    lib.dflash_tree_attention_workspace_size.restype = SZ
    lib.dflash_tree_attention_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.dflash_tree_attention.restype = I32
    lib.dflash_tree_attention.argtypes = [
        I32, I32, I32, I32, I32, P, P, P, P, P, I32, I32, P, I32, P, P, F, P, P, I32, I32, P, SZ, P]
    lib.dflash_draft_layer_workspace_size.restype = SZ
    lib.dflash_draft_layer_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, I32]
    lib.dflash_draft_layer.restype = I32
    lib.dflash_draft_layer.argtypes = [
        I32, I32, I32, I32, I32, I32, I32, P, ctypes.POINTER(DraftLayerWeights), F, F, P, P, I32, I32,
        P, I32, P, I32, I32, P, SZ, P]
    lib.dflash_draft_head_workspace_size.restype = SZ
    lib.dflash_draft_head_workspace_size.argtypes = [I32, I32, I32, I32]
    lib.dflash_draft_head.restype = I32
    lib.dflash_draft_head.argtypes = [I32, I32, I32, P, P, P, F, P, I32, P, SZ, P]
    lib.dflash_embed.restype = I32
    lib.dflash_embed.argtypes = [I32, I32, I32, P, P, P, I32, P]
    lib.dflash_tree_commit_kv.restype = I32
    lib.dflash_tree_commit_kv.argtypes = [
        I32, I32, I32, I32, I32, PP, PP, ctypes.POINTER(KVLayer), P, I32, P, I32, P, P, I32, P]


def lib():
    """The loaded C library (loads on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_diffusion_draft_ctx_amd.build` first")
        handle = ctypes.CDLL(LIB_PATH)
        _declare(handle)
        _lib = handle
    return _lib


def status_string(s: int) -> str:
    return lib().dflash_status_string(s).decode()


def _check(s: int, what: str):
    if s != OK:
        raise DFlashError(s, f"{what}: {status_string(s)}")


# ----------------------------------------------------------------------------
# tensor marshalling
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _cache_pair(ck, cv, Hkv, D):
    """One layer's K and V caches, each [num_pages, Hkv, page_size, D]
    (head-major) on the device with the same shape; returns (num_pages,
    page_size)."""
    for name, t in (("cache_k", ck), ("cache_v", cv)):
        if t.dim() != 4 or t.shape[1] != Hkv or t.shape[3] != D:
            raise ValueError(f"{name} must be [num_pages, {Hkv}, page_size, {D}] (head-major), "
                             f"got {tuple(t.shape)}")
    if ck.shape != cv.shape:
        raise ValueError(f"cache_k {tuple(ck.shape)} and cache_v {tuple(cv.shape)} differ")
    _dev(ck, "cache_k")
    _dev(cv, "cache_v")
    return ck.shape[0], ck.shape[2]


def _i32(t, name):
    torch = _torch()
    if t is None:
        return None
    _dev(t, name)
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return t


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _workspace(nbytes, device, ws):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws, ws.numel() * ws.element_size()
    buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return buf, nbytes


def _pp(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return ctypes.cast(arr, PP), arr


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------

def materialize_ctx_kv(hiddens: Sequence, W_f, b_f, W_K: Sequence, W_V: Sequence,
                       cache_k: Sequence, cache_v: Sequence, block_table, rows_per_seq: int,
                       seq_start_pos, commit_lens=None, h_ctx_out=None, workspace=None,
                       stream=None, k_norm_weight: Optional[Sequence] = None,
                       k_norm_eps: float = 1e-6, rope_theta: float = 0.0):
    """dflash_materialize_ctx_kv.  hiddens: m tensors [T, d]; W_f [d, m*d];
    b_f [d] or None; W_K/W_V: per-layer [Hkv*D, d]; cache_k/cache_v: per-layer
    [num_pages, Hkv, 16, D]; block_table [n_seq, max_pages] int32.  K
    epilogue: k_norm_weight (per-layer [D] tensors, or None) and rope_theta
    (0: none)."""
    L = lib()
    m = len(hiddens)
    T, d = hiddens[0].shape
    for i, h in enumerate(hiddens):
        _dev(h, f"hiddens[{i}]")
    dt = _dtype_code(hiddens[0])
    n_layers = len(W_K)
    _, Hkv, _, D = cache_k[0].shape
    _i32(block_table, "block_table")
    _i32(seq_start_pos, "seq_start_pos")
    _i32(commit_lens, "commit_lens")
    caches = (KVLayer * n_layers)(*[KVLayer(_ptr(k), _ptr(v), *_cache_pair(k, v, Hkv, D))
                                    for k, v in zip(cache_k, cache_v)])
    need = L.dflash_materialize_workspace_size(T, m, d, n_layers, Hkv, D, dt)
    ws, nws = _workspace(need, hiddens[0].device, workspace)
    hp, _h = _pp([_ptr(h) for h in hiddens])
    kp, _k = _pp([_ptr(_dev(w, "W_K")) for w in W_K])
    vp, _v = _pp([_ptr(_dev(w, "W_V")) for w in W_V])
    epi, _w = None, None
    if k_norm_weight is not None or rope_theta:
        if k_norm_weight is not None:
            if len(k_norm_weight) != n_layers:
                raise ValueError("k_norm_weight needs one tensor per layer")
            for w in k_norm_weight:
                _dev(w, "k_norm_weight")
                if _dtype_code(w) != dt or w.numel() != D:
                    raise ValueError("k_norm_weight tensors are [head_dim] in the storage dtype")
            wp, _w = _pp([_ptr(w) for w in k_norm_weight])
        else:
            wp = None
        epi = ctypes.pointer(KEpilogue(wp, float(k_norm_eps), float(rope_theta)))
    s = L.dflash_materialize_ctx_kv(
        T, m, d, hp, _ptr(_dev(W_f, "W_f")), _ptr(b_f), n_layers, Hkv, D, kp, vp, caches,
        _ptr(block_table), block_table.shape[1], rows_per_seq, _ptr(seq_start_pos),
        _ptr(commit_lens), epi, _ptr(h_ctx_out), dt, _ptr(ws), nws, _stream(stream))
    _check(s, "dflash_materialize_ctx_kv")
    return h_ctx_out


def block_attention(q, k_blk, v_blk, cache_k, cache_v, block_table, ctx_lens, scale=0.0,
                    out=None, lse=None, workspace=None, stream=None, out_dtype=None,
                    causal=False):
    """dflash_block_attention.  q [B,k,Hq,D]; k_blk/v_blk [B,k,Hkv,D]; caches
    [num_pages,16,Hkv,D]; block_table [B,max_pages], or [1,max_pages] when
    every request reads the same (packed) sequence; ctx_lens [B].  ``causal``
    lets block position i see block keys 0..i only (the context stays
    visible).  The output takes the dtype of ``out`` (or ``out_dtype``,
    default: q's dtype).  Returns (out, lse) where lse is the tensor given (or
    None)."""
    torch = _torch()
    L = lib()
    B, k, Hq, D = q.shape
    Hkv = k_blk.shape[2]
    dt = _dtype_code(q)
    for n, t in (("q", q), ("k_blk", k_blk), ("v_blk", v_blk)):
        _dev(t, n)
    npg, psz = _cache_pair(cache_k, cache_v, Hkv, D)
    _i32(block_table, "block_table")
    _i32(ctx_lens, "ctx_lens")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _dev(out, "out")
    odt = _dtype_code(out)
    need = L.dflash_attention_workspace_size(B, k, Hq, Hkv, D, block_table.shape[1], dt)
    ws, nws = _workspace(need, q.device, workspace)
    s = L.dflash_block_attention(
        B, k, Hq, Hkv, D, _ptr(q), _ptr(k_blk), _ptr(v_blk), _ptr(cache_k), _ptr(cache_v),
        npg, psz, _ptr(block_table), block_table.shape[1],
        block_table.shape[0], _ptr(ctx_lens), float(scale), MASK_CAUSAL if causal else MASK_BIDIRECTIONAL,
        _ptr(out), _ptr(lse), dt, odt,
        _ptr(ws), nws,
        _stream(stream))
    _check(s, "dflash_block_attention")
    return out, lse


def _logit_rows(t, name):
    """Row stride (elements) of a [B, R, V] logits view whose rows are evenly
    spaced (contiguous, or a slice of a wider row buffer)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    B, R, V = t.shape
    if t.stride(2) != 1 or (B > 1 and t.stride(0) != R * t.stride(1)) or t.stride(1) < V:
        raise ValueError(f"{name}: rows must be evenly spaced with unit element stride")
    return t.stride(1)


def _row_stride(t):
    return _logit_rows(t, "logits")


def verify_greedy(target_logits, draft_tokens=None, draft_logits=None, chain_lens=None,
                  prefix_lens=None, want_target_predict=True, out=None, workspace=None,
                  stream=None):
    """dflash_verify_greedy.  target_logits [B, L+1, V]; draft_logits [B, L, V]
    or None (then draft_tokens [B, L] int32 is the input).  Returns a dict of
    device tensors: accept_len, bonus, commit_lens, new_seq_lens (if
    prefix_lens), target_predict (if wanted), draft_tokens."""
    torch = _torch()
    L_ = lib()
    _logit_rows(target_logits, "target_logits")
    B, Lp1, V = target_logits.shape
    L = Lp1 - 1
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    o = dict(out or {})
    if draft_logits is not None:
        _logit_rows(draft_logits, "draft_logits")
        if draft_tokens is None:
            draft_tokens = torch.empty((B, L), dtype=torch.int32, device=dev)
    _i32(draft_tokens, "draft_tokens")
    _i32(chain_lens, "chain_lens")
    _i32(prefix_lens, "prefix_lens")
    for name in ("accept_len", "bonus", "commit_lens"):
        o.setdefault(name, torch.empty(B, dtype=torch.int32, device=dev))
    if prefix_lens is not None:
        o.setdefault("new_seq_lens", torch.empty(B, dtype=torch.int32, device=dev))
    if want_target_predict:
        o.setdefault("target_predict", torch.empty((B, L + 1), dtype=torch.int32, device=dev))
    need = L_.dflash_verify_workspace_size(B, L, V)
    ws, nws = _workspace(need, dev, workspace)
    s = L_.dflash_verify_greedy(
        B, L, V, _ptr(target_logits), _row_stride(target_logits), _ptr(draft_logits),
        _row_stride(draft_logits) if draft_logits is not None else 0, _ptr(draft_tokens),
        _ptr(chain_lens), _ptr(o.get("target_predict")), _ptr(o["accept_len"]), _ptr(o["bonus"]),
        _ptr(o["commit_lens"]), _ptr(prefix_lens), _ptr(o.get("new_seq_lens")), dt, _ptr(ws),
        nws, _stream(stream))
    _check(s, "dflash_verify_greedy")
    o["draft_tokens"] = draft_tokens
    return o


def verify_greedy_noalloc(target_logits, draft_tokens=None, draft_logits=None, chain_lens=None,
                          prefix_lens=None, want_target_predict=True, out=None, stream=None):
    """dflash_verify_greedy_noalloc: verify_greedy without a workspace (the
    library's static per-GPU scratch holds the partials).  Same arguments and
    results as verify_greedy; the caller still provides the outputs (``out``)
    or lets this allocate them here, outside the library call."""
    torch = _torch()
    L_ = lib()
    _logit_rows(target_logits, "target_logits")
    B, Lp1, V = target_logits.shape
    L = Lp1 - 1
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    o = dict(out or {})
    if draft_logits is not None:
        _logit_rows(draft_logits, "draft_logits")
        if draft_tokens is None:
            draft_tokens = torch.empty((B, L), dtype=torch.int32, device=dev)
    _i32(draft_tokens, "draft_tokens")
    _i32(chain_lens, "chain_lens")
    _i32(prefix_lens, "prefix_lens")
    for name in ("accept_len", "bonus", "commit_lens"):
        o.setdefault(name, torch.empty(B, dtype=torch.int32, device=dev))
    if prefix_lens is not None:
        o.setdefault("new_seq_lens", torch.empty(B, dtype=torch.int32, device=dev))
    if want_target_predict:
        o.setdefault("target_predict", torch.empty((B, L + 1), dtype=torch.int32, device=dev))
    s = L_.dflash_verify_greedy_noalloc(
        B, L, V, _ptr(target_logits), _row_stride(target_logits), _ptr(draft_logits),
        _row_stride(draft_logits) if draft_logits is not None else 0, _ptr(draft_tokens),
        _ptr(chain_lens), _ptr(o.get("target_predict")), _ptr(o["accept_len"]), _ptr(o["bonus"]),
        _ptr(o["commit_lens"]), _ptr(prefix_lens), _ptr(o.get("new_seq_lens")), dt,
        _stream(stream))
    _check(s, "dflash_verify_greedy_noalloc")
    o["draft_tokens"] = draft_tokens
    return o


def verify_sample(target_logits, draft_logits, draft_tokens, u_accept, u_bonus, temperature=1.0,
                  chain_lens=None, prefix_lens=None, audit=True, out=None, workspace=None,
                  stream=None, draft_row_lse=None):
    """dflash_verify_sample.  Returns a dict with accept_len, bonus,
    commit_lens, new_seq_lens (if prefix_lens) and, with ``audit``, ratio
    [B, L], beta [B] and cdf_gap [B].  draft_row_lse [B, L] float32: the
    draft rows' log-sum-exp as ``gate`` returns it (row_lse), to skip
    reducing the draft rows again."""
    torch = _torch()
    L_ = lib()
    _logit_rows(target_logits, "target_logits")
    B, Lp1, V = target_logits.shape
    L = Lp1 - 1
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    if draft_logits is not None:
        _logit_rows(draft_logits, "draft_logits")
    _i32(draft_tokens, "draft_tokens")
    _i32(chain_lens, "chain_lens")
    _i32(prefix_lens, "prefix_lens")
    for n, t in (("u_accept", u_accept), ("u_bonus", u_bonus), ("draft_row_lse", draft_row_lse)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{n} must be float32")
        if t is not None:
            _dev(t, n)
    o = dict(out or {})
    for name in ("accept_len", "bonus", "commit_lens"):
        o.setdefault(name, torch.empty(B, dtype=torch.int32, device=dev))
    if prefix_lens is not None:
        o.setdefault("new_seq_lens", torch.empty(B, dtype=torch.int32, device=dev))
    if audit:
        o.setdefault("ratio", torch.empty((B, L), dtype=torch.float32, device=dev))
        o.setdefault("beta", torch.empty(B, dtype=torch.float32, device=dev))
        o.setdefault("cdf_gap", torch.empty(B, dtype=torch.float32, device=dev))
    need = L_.dflash_verify_workspace_size(B, L, V)
    ws, nws = _workspace(need, dev, workspace)
    s = L_.dflash_verify_sample(
        B, L, V, _ptr(target_logits), _row_stride(target_logits), _ptr(draft_logits),
        _row_stride(draft_logits) if draft_logits is not None else 0, _ptr(draft_tokens),
        _ptr(chain_lens), _ptr(u_accept), _ptr(u_bonus), float(temperature), _ptr(draft_row_lse),
        _ptr(o["accept_len"]), _ptr(o["bonus"]), _ptr(o["commit_lens"]), _ptr(prefix_lens),
        _ptr(o.get("new_seq_lens")), _ptr(o.get("ratio")), _ptr(o.get("beta")),
        _ptr(o.get("cdf_gap")), dt, _ptr(ws), nws, _stream(stream))
    _check(s, "dflash_verify_sample")
    return o


def gate(draft_logits, draft_tokens, temperature=1.0, g=-0.5, valid_lens=None, row_stats=True,
         out=None, workspace=None, stream=None):
    """dflash_gate.  Returns a dict with c [B], go [B] and, with row_stats,
    row_max and row_lse [B, n]."""
    torch = _torch()
    L_ = lib()
    _logit_rows(draft_logits, "draft_logits")
    B, n, V = draft_logits.shape
    dt = _dtype_code(draft_logits)
    dev = draft_logits.device
    _i32(draft_tokens, "draft_tokens")
    _i32(valid_lens, "valid_lens")
    o = dict(out or {})
    o.setdefault("c", torch.empty(B, dtype=torch.float32, device=dev))
    o.setdefault("go", torch.empty(B, dtype=torch.int32, device=dev))
    if row_stats:
        o.setdefault("row_max", torch.empty((B, n), dtype=torch.float32, device=dev))
        o.setdefault("row_lse", torch.empty((B, n), dtype=torch.float32, device=dev))
    # row statistics may be column slices [B, n] of a wider [B, ld] array
    # (a DLoop stage writing its columns of the chain's array)
    ld = 0
    for name in ("row_max", "row_lse"):
        t = o.get(name)
        if t is None:
            continue
        if not t.is_cuda or t.dtype != torch.float32 or tuple(t.shape) != (B, n) or t.stride(1) != 1:
            raise ValueError(f"{name}: [B, n] float32 device tensor with unit column stride")
        if ld and t.stride(0) != ld:
            raise ValueError("row_max and row_lse need the same row stride")
        ld = t.stride(0)
    need = L_.dflash_gate_workspace_size(B, n, V)
    ws, nws = _workspace(need, dev, workspace)
    s = L_.dflash_gate(B, n, V, _ptr(draft_logits), _row_stride(draft_logits), _ptr(draft_tokens),
                       _ptr(valid_lens), float(temperature), float(g), _ptr(o["c"]), _ptr(o["go"]),
                       _ptr(o.get("row_max")), _ptr(o.get("row_lse")), ld if B > 1 else 0, dt,
                       _ptr(ws), nws, _stream(stream))
    _check(s, "dflash_gate")
    return o


def tree_build(draft_logits, topk, budget, temperature=1.0, want_mask=True, out=None,
               workspace=None, stream=None):
    """dflash_tree_build.  draft_logits [B, n_pos, V] (row d: block position
    d + 1).  Returns a dict of device tensors: topk_tokens, topk_logp
    [B, n_pos, topk]; node_token, node_parent, node_depth, node_logp
    [B, budget]; n_nodes [B]; ancestor_mask [B, budget, ceil(budget / 32)]
    int32 bit rows (if wanted)."""
    torch = _torch()
    L_ = lib()
    _logit_rows(draft_logits, "draft_logits")
    B, n_pos, V = draft_logits.shape
    dt = _dtype_code(draft_logits)
    dev = draft_logits.device
    o = dict(out or {})
    o.setdefault("topk_tokens", torch.empty((B, n_pos, topk), dtype=torch.int32, device=dev))
    o.setdefault("topk_logp", torch.empty((B, n_pos, topk), dtype=torch.float32, device=dev))
    for name, dtp in (("node_token", torch.int32), ("node_parent", torch.int32),
                      ("node_depth", torch.int32), ("node_logp", torch.float32)):
        o.setdefault(name, torch.empty((B, budget), dtype=dtp, device=dev))
    o.setdefault("n_nodes", torch.empty(B, dtype=torch.int32, device=dev))
    if want_mask:
        o.setdefault("ancestor_mask",
                     torch.empty((B, budget, (budget + 31) // 32), dtype=torch.int32, device=dev))
    need = L_.dflash_tree_workspace_size(B, n_pos, V, topk)
    ws, nws = _workspace(need, dev, workspace)
    s = L_.dflash_tree_build(
        B, n_pos, V, _ptr(draft_logits), _row_stride(draft_logits), float(temperature), int(topk),
        int(budget), _ptr(o["topk_tokens"]), _ptr(o["topk_logp"]), _ptr(o["node_token"]),
        _ptr(o["node_parent"]), _ptr(o["node_depth"]), _ptr(o["node_logp"]), _ptr(o["n_nodes"]),
        _ptr(o.get("ancestor_mask")), dt, _ptr(ws), nws, _stream(stream))
    _check(s, "dflash_tree_build")
    return o


def tree_verify_greedy(target_logits, node_token, node_parent, n_nodes, max_depth,
                       prefix_lens=None, out=None, workspace=None, stream=None):
    """dflash_tree_verify_greedy.  target_logits [B, budget + 1, V] (row 0:
    after the root, row 1 + j: after node j); node_token, node_parent
    [B, budget] and n_nodes [B] int32.  Returns a dict with accept_len,
    bonus, commit_lens [B], accepted_nodes [B, max_depth] and new_seq_lens
    (if prefix_lens)."""
    torch = _torch()
    L_ = lib()
    _logit_rows(target_logits, "target_logits")
    B, R, V = target_logits.shape
    budget = R - 1
    dt = _dtype_code(target_logits)
    dev = target_logits.device
    for name, t in (("node_token", node_token), ("node_parent", node_parent)):
        _i32(t, name)
        if tuple(t.shape) != (B, budget):
            raise ValueError(f"{name} must be [B, budget] = [{B}, {budget}]")
    _i32(n_nodes, "n_nodes")
    _i32(prefix_lens, "prefix_lens")
    o = dict(out or {})
    for name in ("accept_len", "bonus", "commit_lens"):
        o.setdefault(name, torch.empty(B, dtype=torch.int32, device=dev))
    o.setdefault("accepted_nodes", torch.empty((B, max_depth), dtype=torch.int32, device=dev))
    if prefix_lens is not None:
        o.setdefault("new_seq_lens", torch.empty(B, dtype=torch.int32, device=dev))
    need = L_.dflash_tree_verify_workspace_size(B, budget, V)
    ws, nws = _workspace(need, dev, workspace)
    s = L_.dflash_tree_verify_greedy(
        B, budget, V, _ptr(target_logits), _row_stride(target_logits), _ptr(node_token),
        _ptr(node_parent), _ptr(n_nodes), int(max_depth), _ptr(o["accept_len"]), _ptr(o["bonus"]),
        _ptr(o["accepted_nodes"]), _ptr(o["commit_lens"]), _ptr(prefix_lens),
        _ptr(o.get("new_seq_lens")), dt, _ptr(ws), nws, _stream(stream))
    _check(s, "dflash_tree_verify_greedy")
    return o


def tree_attention(q, k_tree, v_tree, cache_k, cache_v, block_table, ctx_lens, ancestor_mask,
                   scale=0.0, out=None, lse=None, workspace=None, stream=None, out_dtype=None):
    """dflash_tree_attention.  q [B, R, Hq, D], k_tree / v_tree [B, R, Hkv, D]
    with R = 1 + budget (row 0 the root, row 1 + j node j); caches
    [num_pages, Hkv, 16, D]; block_table [B, max_pages]; ctx_lens [B];
    ancestor_mask [B, R - 1, ceil((R - 1) / 32)] int32 bit rows as
    ``tree_build`` returns them.  Returns (out, lse)."""
    torch = _torch()
    L = lib()
    B, R, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    dt = _dtype_code(q)
    for n, t in (("q", q), ("k_tree", k_tree), ("v_tree", v_tree)):
        _dev(t, n)
    npg, psz = _cache_pair(cache_k, cache_v, Hkv, D)
    _i32(block_table, "block_table")
    _i32(ctx_lens, "ctx_lens")
    if ancestor_mask is not None:
        _i32(ancestor_mask, "ancestor_mask")
        if tuple(ancestor_mask.shape) != (B, R - 1, (R + 30) // 32):
            raise ValueError("ancestor_mask must be [B, R - 1, ceil((R - 1) / 32)]")
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    _dev(out, "out")
    odt = _dtype_code(out)
    need = L.dflash_tree_attention_workspace_size(B, R, Hq, Hkv, D, block_table.shape[1], dt)
    ws, nws = _workspace(need, q.device, workspace)
    s = L.dflash_tree_attention(
        B, R, Hq, Hkv, D, _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(cache_k), _ptr(cache_v),
        npg, psz, _ptr(block_table), block_table.shape[1],
        _ptr(ctx_lens), _ptr(ancestor_mask), float(scale), _ptr(out), _ptr(lse), dt, odt,
        _ptr(ws), nws, _stream(stream))
    _check(s, "dflash_tree_attention")
    return out, lse


def tree_commit_kv(k_tree: Sequence, v_tree: Sequence, cache_k: Sequence, cache_v: Sequence,
                   block_table, accepted_nodes, accept_len, prefix_lens, stream=None):
    """dflash_tree_commit_kv.  Per layer l: k_tree[l] / v_tree[l]
    [B, R, Hkv, D], cache_k[l] / cache_v[l] [num_pages, Hkv, 16, D];
    block_table [B, max_pages]; accepted_nodes [B, max_depth], accept_len and
    prefix_lens [B] int32 (tree_verify_greedy's outputs and its prefix)."""
    L = lib()
    n_layers = len(k_tree)
    B, R, Hkv, D = k_tree[0].shape
    dt = _dtype_code(k_tree[0])
    for t in (accepted_nodes, accept_len, prefix_lens, block_table):
        _i32(t, "int32 argument")
    kp, kpa = _pp([_ptr(_dev(t, "k_tree")) for t in k_tree])
    vp, vpa = _pp([_ptr(_dev(t, "v_tree")) for t in v_tree])
    caches = (KVLayer * n_layers)(*[KVLayer(_ptr(k), _ptr(v), *_cache_pair(k, v, Hkv, D))
                                    for k, v in zip(cache_k, cache_v)])
    s = L.dflash_tree_commit_kv(
        B, R, n_layers, Hkv, D, kp, vp, caches, _ptr(block_table), block_table.shape[1],
        _ptr(accepted_nodes), accepted_nodes.shape[1], _ptr(accept_len), _ptr(prefix_lens), dt,
        _stream(stream))
    _check(s, "dflash_tree_commit_kv")


_DRAFT_KEYS = ("ln1", "qkv", "q_norm", "k_norm", "o", "ln2", "gate_up", "down")


def draft_layer(x, weights, cache_k, cache_v, block_table, ctx_lens, k, n_q_heads, eps=1e-6,
                rope_theta=1e6, causal=False, workspace=None, stream=None):
    """dflash_draft_layer: one drafter layer on x [B*k, d] (updated in place).
    weights: dict of device tensors ln1 [d], qkv [(Hq + 2 Hkv) D, d], q_norm /
    k_norm [D] or None, o [d, Hq D], ln2 [d], gate_up [2 I, d], down [d, I].
    cache_k / cache_v [num_pages, Hkv, 16, D] (this layer's context),
    block_table [B, max_pages], ctx_lens [B].  Returns x."""
    L = lib()
    M, d = x.shape
    B = M // k
    Hkv, D = cache_k.shape[1], cache_k.shape[3]
    npg, psz = _cache_pair(cache_k, cache_v, Hkv, D)
    I = weights["down"].shape[1]
    dt = _dtype_code(x)
    _dev(x, "x")
    for n in _DRAFT_KEYS:
        if weights.get(n) is not None:
            _dev(weights[n], n)
    _i32(block_table, "block_table")
    _i32(ctx_lens, "ctx_lens")
    wst = DraftLayerWeights(*[_ptr(weights.get(n)) for n in _DRAFT_KEYS])
    need = L.dflash_draft_layer_workspace_size(B, k, d, n_q_heads, Hkv, D, I, block_table.shape[1], dt)
    ws, nws = _workspace(need, x.device, workspace)
    s = L.dflash_draft_layer(B, k, d, n_q_heads, Hkv, D, I, _ptr(x), ctypes.byref(wst), float(eps),
                             float(rope_theta), _ptr(cache_k), _ptr(cache_v), npg, psz,
                             _ptr(block_table), block_table.shape[1], _ptr(ctx_lens),
                             MASK_CAUSAL if causal else MASK_BIDIRECTIONAL, dt, _ptr(ws), nws,
                             _stream(stream))
    _check(s, "dflash_draft_layer")
    return x


def draft_head(x, norm_weight, lm_head, eps=1e-6, out=None, workspace=None, stream=None):
    """dflash_draft_head: logits [M, V] = rmsnorm(x) * norm_weight . lm_head^T."""
    torch = _torch()
    L = lib()
    M, d = x.shape
    V = lm_head.shape[0]
    dt = _dtype_code(x)
    for n, t in (("x", x), ("norm_weight", norm_weight), ("lm_head", lm_head)):
        _dev(t, n)
    if out is None:
        out = torch.empty((M, V), dtype=x.dtype, device=x.device)
    _dev(out, "out")
    need = L.dflash_draft_head_workspace_size(M, d, V, dt)
    ws, nws = _workspace(need, x.device, workspace)
    s = L.dflash_draft_head(M, d, V, _ptr(x), _ptr(norm_weight), _ptr(lm_head), float(eps),
                            _ptr(out), dt, _ptr(ws), nws, _stream(stream))
    _check(s, "dflash_draft_head")
    return out


def embed(table, tokens, out=None, stream=None):
    """dflash_embed: rows of table [V, d] for tokens [M] (or [B, k]) -> [M, d]."""
    torch = _torch()
    L = lib()
    V, d = table.shape
    _dev(table, "table")
    _i32(tokens, "tokens")
    M = tokens.numel()
    if out is None:
        out = torch.empty((M, d), dtype=table.dtype, device=table.device)
    _dev(out, "out")
    s = L.dflash_embed(M, d, V, _ptr(table), _ptr(tokens), _ptr(out), _dtype_code(table),
                       _stream(stream))
    _check(s, "dflash_embed")
    return out
