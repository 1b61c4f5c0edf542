"""Boundary tests that need no GPU: the library loads, exports every symbol
the header declares, sizes workspaces, and rejects bad arguments before it
touches the device (fake pointers are only passed where validation must
fail first; the calls that would get past validation are never made)."""
import ctypes
import os
import re

import pytest

import block_diffusion_draft_ctx_amd as dfl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")

# Calls with fake addresses are kept off machines with a GPU driver, where a
# validation bug would turn into a device access.
no_gpu = pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="fake-pointer tests run on CPU hosts")

FAKE = 0x10000  # 16-byte aligned, never dereferenced
WS = 0x100000   # 256-byte aligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dflash_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dfl.LIB_PATH):
        from block_diffusion_draft_ctx_amd import build
        build.build()
    return dfl.lib()


def test_header_lists_the_exports():
    assert declared_functions() == sorted(dfl.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for s in range(6):
        assert dfl.status_string(s).startswith("DFLASH_")
    assert "UNKNOWN" in dfl.status_string(99)
    assert lib.dflash_version() >= 100


def test_workspace_queries(lib):
    # greedy/sample partials grow with rows; degenerate sizes need nothing
    a = lib.dflash_verify_workspace_size(64, 15, 128256)
    b = lib.dflash_verify_workspace_size(1, 15, 128256)
    assert a > b > 0 and a % 256 == 0
    assert lib.dflash_verify_workspace_size(0, 15, 100) == 0
    assert lib.dflash_verify_workspace_size(4, 65, 100) == 0
    assert lib.dflash_gate_workspace_size(16, 8, 151936) > 0
    # attention: large batches need no split, small ones do
    assert lib.dflash_attention_workspace_size(256, 16, 32, 8, 128, 512, dfl.BF16) == 0
    assert lib.dflash_attention_workspace_size(1, 16, 32, 8, 128, 512, dfl.BF16) > 0
    assert lib.dflash_attention_workspace_size(1, 16, 32, 8, 128, 512, dfl.F32) == 0
    # materialise: h_ctx staging, plus split-K partials for few rows
    big = lib.dflash_materialize_workspace_size(131072, 5, 4096, 5, 8, 128, dfl.BF16)
    assert big >= 131072 * 4096 * 2
    small = lib.dflash_materialize_workspace_size(16, 5, 4096, 5, 8, 128, dfl.BF16)
    assert small > 16 * 4096 * 2


@no_gpu
def test_zero_batch_is_a_noop(lib):
    assert lib.dflash_verify_greedy(0, 15, 100, None, 100, None, 0, None, None, None, None, None,
                                    None, None, None, dfl.BF16, None, 0, None) == dfl.OK
    assert lib.dflash_block_attention(0, 16, 32, 8, 128, None, None, None, None, None, 1, 16,
                                      None, 1, 0, None, 0.0, dfl.MASK_BIDIRECTIONAL, None, None,
                                      dfl.BF16, dfl.BF16, None, 0, None) == dfl.OK
    assert lib.dflash_gate(0, 8, 100, None, 100, None, None, 1.0, -0.5, None, None, None, None,
                           0, dfl.BF16, None, 0, None) == dfl.OK
    assert lib.dflash_verify_sample(0, 8, 100, None, 100, None, 100, None, None, None, None, 1.0,
                                    None, None, None, None, None, None, None, None, None,
                                    dfl.BF16, None, 0, None) == dfl.OK


def _greedy(lib, **kw):
    a = dict(B=2, L=3, V=100, tl=FAKE, ts=100, dl=None, ds=0, dt=FAKE, cl=None, tp=None,
             acc=FAKE, bo=FAKE, cm=FAKE, pre=None, new=None, dtype=dfl.BF16, ws=WS, nws=1 << 20)
    a.update(kw)
    return lib.dflash_verify_greedy(a["B"], a["L"], a["V"], a["tl"], a["ts"], a["dl"], a["ds"],
                                    a["dt"], a["cl"], a["tp"], a["acc"], a["bo"], a["cm"],
                                    a["pre"], a["new"], a["dtype"], a["ws"], a["nws"], None)


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), dfl.E_ARG), (dict(V=0), dfl.E_ARG), (dict(L=65), dfl.E_UNSUPPORTED),
    (dict(tl=None), dfl.E_ARG), (dict(ts=99), dfl.E_ARG), (dict(dl=FAKE, ds=10), dfl.E_ARG),
    (dict(acc=None), dfl.E_ARG), (dict(dt=None), dfl.E_ARG), (dict(pre=FAKE), dfl.E_ARG),
    (dict(ws=None), dfl.E_WORKSPACE), (dict(nws=16), dfl.E_WORKSPACE),
    (dict(ws=WS + 8), dfl.E_WORKSPACE), (dict(dtype=7), dfl.E_ARG),
])
def test_greedy_argument_errors(lib, kw, code):
    assert _greedy(lib, **kw) == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(T=0.0), dfl.E_ARG), (dict(T=float("nan")), dfl.E_ARG), (dict(dl=None), dfl.E_ARG),
    (dict(u=None), dfl.E_ARG), (dict(u2=None), dfl.E_ARG), (dict(nws=0), dfl.E_WORKSPACE),
])
def test_sample_argument_errors(lib, kw, code):
    a = dict(T=1.0, dl=FAKE, u=FAKE, u2=FAKE, nws=1 << 24)
    a.update(kw)
    s = lib.dflash_verify_sample(2, 3, 100, FAKE, 100, a["dl"], 100, FAKE, None, a["u"], a["u2"],
                                 a["T"], None, FAKE, FAKE, FAKE, None, None, None, None, None,
                                 dfl.BF16, WS, a["nws"], None)
    assert s == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(n=0), dfl.E_ARG), (dict(n=65), dfl.E_UNSUPPORTED), (dict(T=-1.0), dfl.E_ARG),
    (dict(g=float("nan")), dfl.E_ARG), (dict(rs=5), dfl.E_ARG), (dict(c=None), dfl.E_ARG),
    (dict(nws=0), dfl.E_WORKSPACE), (dict(ld=7), dfl.E_ARG), (dict(ld=-1), dfl.E_ARG),
])
def test_gate_argument_errors(lib, kw, code):
    a = dict(n=8, T=1.0, g=-0.5, rs=100, c=FAKE, nws=1 << 20, ld=32)
    a.update(kw)
    s = lib.dflash_gate(2, a["n"], 100, FAKE, a["rs"], FAKE, None, a["T"], a["g"], a["c"], FAKE,
                        None, None, a["ld"], dfl.BF16, WS, a["nws"], None)
    assert s == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(D=96), dfl.E_UNSUPPORTED), (dict(Hq=30), dfl.E_ARG), (dict(k=65), dfl.E_UNSUPPORTED),
    (dict(Hq=64, Hkv=2, k=16), dfl.E_UNSUPPORTED), (dict(ps=32), dfl.E_UNSUPPORTED),
    (dict(scale=-1.0), dfl.E_ARG), (dict(q=None), dfl.E_ARG), (dict(q=FAKE + 2), dfl.E_UNSUPPORTED),
    (dict(np_=0), dfl.E_ARG), (dict(nws=0, B=1, rows=1), dfl.E_WORKSPACE),
    (dict(dt=dfl.F32, odt=dfl.BF16), dfl.E_UNSUPPORTED), (dict(odt=5), dfl.E_ARG),
    (dict(rows=2), dfl.E_ARG), (dict(rows=0), dfl.E_ARG), (dict(rows=5), dfl.E_ARG),
    (dict(mask=2), dfl.E_ARG), (dict(mask=-1), dfl.E_ARG),
])
def test_attention_argument_errors(lib, kw, code):
    a = dict(B=4, k=16, Hq=32, Hkv=8, D=128, q=FAKE, ps=16, scale=0.0, np_=10, nws=1 << 26,
             dt=dfl.BF16, odt=dfl.BF16, rows=4, mask=dfl.MASK_CAUSAL)
    a.update(kw)
    s = lib.dflash_block_attention(a["B"], a["k"], a["Hq"], a["Hkv"], a["D"], a["q"], FAKE, FAKE,
                                   FAKE, FAKE, a["np_"], a["ps"], FAKE, 64, a["rows"], FAKE,
                                   a["scale"], a["mask"], FAKE, None, a["dt"], a["odt"], WS,
                                   a["nws"], None)
    assert s == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(m=9), dfl.E_UNSUPPORTED), (dict(D=80), dfl.E_UNSUPPORTED), (dict(d=200), dfl.E_UNSUPPORTED),
    (dict(rps=5), dfl.E_ARG), (dict(T=-2), dfl.E_ARG), (dict(page=32), dfl.E_UNSUPPORTED),
    (dict(hid0=None), dfl.E_ARG), (dict(wf=None), dfl.E_ARG), (dict(nws=0), dfl.E_WORKSPACE),
    (dict(ck=FAKE + 2), dfl.E_UNSUPPORTED),    # bf16 caches take 16-byte stores
    (dict(eps=-1.0), dfl.E_ARG), (dict(eps=float("nan")), dfl.E_ARG),
    (dict(theta=0.5), dfl.E_ARG), (dict(theta=float("inf")), dfl.E_ARG),
    (dict(theta=-2.0), dfl.E_ARG), (dict(knw=0), dfl.E_ARG), (dict(knw=FAKE + 4), dfl.E_UNSUPPORTED),
])
def test_materialize_argument_errors(lib, kw, code):
    a = dict(T=32, m=2, d=256, D=128, rps=16, page=16, hid0=FAKE, wf=FAKE, nws=1 << 26, ck=FAKE,
             eps=1e-6, theta=1e4, knw=FAKE)
    a.update(kw)
    knw = (ctypes.c_void_p * 1)(a["knw"] or None)
    epi = dfl.KEpilogue(ctypes.cast(knw, dfl.PP), a["eps"], a["theta"])
    m = a["m"]
    hid = (ctypes.c_void_p * max(m, 1))(*([a["hid0"]] + [FAKE] * (m - 1)))
    wk = (ctypes.c_void_p * 1)(FAKE)
    wv = (ctypes.c_void_p * 1)(FAKE)
    caches = (dfl.KVLayer * 1)(dfl.KVLayer(a["ck"], FAKE, 8, a["page"]))
    s = lib.dflash_materialize_ctx_kv(a["T"], m, a["d"], ctypes.cast(hid, dfl.PP), a["wf"], None,
                                      1, 1, a["D"], ctypes.cast(wk, dfl.PP), ctypes.cast(wv, dfl.PP),
                                      caches, FAKE, 4, a["rps"], FAKE, None, ctypes.byref(epi),
                                      None, dfl.BF16, WS, a["nws"], None)
    assert s == code


def test_tree_workspace_queries(lib):
    a = lib.dflash_tree_workspace_size(8, 16, 151936, 8)
    assert a > 0 and a % 256 == 0
    assert lib.dflash_tree_workspace_size(8, 16, 151936, 17) == 0
    assert lib.dflash_tree_workspace_size(0, 16, 151936, 8) == 0
    v = lib.dflash_tree_verify_workspace_size(8, 256, 151936)
    assert v > 0 and v % 256 == 0
    assert lib.dflash_tree_verify_workspace_size(8, 1025, 151936) == 0


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(K=0), dfl.E_ARG), (dict(K=17), dfl.E_UNSUPPORTED), (dict(K=8, V=7), dfl.E_UNSUPPORTED),
    (dict(budget=0), dfl.E_ARG), (dict(budget=1025), dfl.E_UNSUPPORTED),
    (dict(n=0), dfl.E_ARG), (dict(n=65), dfl.E_UNSUPPORTED), (dict(T=0.0), dfl.E_ARG),
    (dict(T=float("inf")), dfl.E_ARG), (dict(T=float("nan")), dfl.E_ARG),
    (dict(rs=50), dfl.E_ARG), (dict(dl=None), dfl.E_ARG), (dict(nn=None), dfl.E_ARG),
    (dict(nws=0), dfl.E_WORKSPACE), (dict(dtype=3), dfl.E_ARG),
])
def test_tree_build_argument_errors(lib, kw, code):
    a = dict(B=2, n=8, V=100, dl=FAKE, rs=100, T=1.0, K=4, budget=64, nn=FAKE, nws=1 << 24,
             dtype=dfl.BF16)
    a.update(kw)
    s = lib.dflash_tree_build(a["B"], a["n"], a["V"], a["dl"], a["rs"], a["T"], a["K"],
                              a["budget"], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["nn"], None,
                              a["dtype"], WS, a["nws"], None)
    assert s == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(budget=0), dfl.E_ARG), (dict(budget=1025), dfl.E_UNSUPPORTED), (dict(md=0), dfl.E_ARG),
    (dict(tl=None), dfl.E_ARG), (dict(rs=99), dfl.E_ARG), (dict(path=None), dfl.E_ARG),
    (dict(pre=FAKE), dfl.E_ARG), (dict(nws=0), dfl.E_WORKSPACE), (dict(V=0), dfl.E_ARG),
])
def test_tree_verify_argument_errors(lib, kw, code):
    a = dict(B=2, budget=64, V=100, tl=FAKE, rs=100, md=8, path=FAKE, pre=None, nws=1 << 24)
    a.update(kw)
    s = lib.dflash_tree_verify_greedy(a["B"], a["budget"], a["V"], a["tl"], a["rs"], FAKE, FAKE,
                                      FAKE, a["md"], FAKE, FAKE, a["path"], FAKE, a["pre"], None,
                                      dfl.BF16, WS, a["nws"], None)
    assert s == code


@no_gpu
def test_tree_zero_batch_is_a_noop(lib):
    assert lib.dflash_tree_build(0, 8, 100, None, 100, 1.0, 4, 64, None, None, None, None, None,
                                 None, None, None, dfl.BF16, None, 0, None) == dfl.OK
    assert lib.dflash_tree_verify_greedy(0, 64, 100, None, 100, None, None, None, 8, None, None,
                                         None, None, None, None, dfl.BF16, None, 0, None) == dfl.OK


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(R=0), dfl.E_ARG), (dict(R=1026), dfl.E_UNSUPPORTED), (dict(D=96), dfl.E_UNSUPPORTED),
    (dict(Hq=30), dfl.E_ARG), (dict(mask=None), dfl.E_ARG), (dict(q=None), dfl.E_ARG),
    (dict(q=FAKE + 2), dfl.E_UNSUPPORTED), (dict(ps=32), dfl.E_UNSUPPORTED),
    (dict(nws=0, B=1), dfl.E_WORKSPACE), (dict(dt=dfl.F32, odt=dfl.BF16), dfl.E_UNSUPPORTED),
    (dict(scale=-1.0), dfl.E_ARG),
])
def test_tree_attention_argument_errors(lib, kw, code):
    a = dict(B=4, R=513, Hq=32, Hkv=8, D=128, q=FAKE, ps=16, scale=0.0, nws=1 << 28,
             dt=dfl.BF16, odt=dfl.BF16, mask=FAKE)
    a.update(kw)
    s = lib.dflash_tree_attention(a["B"], a["R"], a["Hq"], a["Hkv"], a["D"], a["q"], FAKE, FAKE,
                                  FAKE, FAKE, 10, a["ps"], FAKE, 64, FAKE, a["mask"], a["scale"],
                                  FAKE, None, a["dt"], a["odt"], WS, a["nws"], None)
    assert s == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(L=0), dfl.E_ARG), (dict(L=65), dfl.E_UNSUPPORTED), (dict(md=0), dfl.E_ARG),
    (dict(acc=None), dfl.E_ARG), (dict(ps=32), dfl.E_UNSUPPORTED), (dict(kt=FAKE + 4), dfl.E_UNSUPPORTED),
    (dict(kt=0), dfl.E_ARG), (dict(D=3, Hkv=1), dfl.E_UNSUPPORTED),
])
def test_tree_commit_argument_errors(lib, kw, code):
    a = dict(L=1, md=8, acc=FAKE, ps=16, kt=FAKE, D=128, Hkv=8)
    a.update(kw)
    n = max(a["L"], 1)
    kt = (ctypes.c_void_p * n)(*([a["kt"] or None] * n))
    vt = (ctypes.c_void_p * n)(*([FAKE] * n))
    caches = (dfl.KVLayer * n)(*([dfl.KVLayer(FAKE, FAKE, 8, a["ps"])] * n))
    s = lib.dflash_tree_commit_kv(2, 9, a["L"], a["Hkv"], a["D"], ctypes.cast(kt, dfl.PP),
                                  ctypes.cast(vt, dfl.PP), caches, FAKE, 4, FAKE, a["md"], a["acc"],
                                  FAKE, dfl.BF16, None)
    assert s == code


@no_gpu
@pytest.mark.parametrize("kw,code", [
    (dict(D=96), dfl.E_UNSUPPORTED), (dict(k=65), dfl.E_UNSUPPORTED), (dict(d=200), dfl.E_UNSUPPORTED),
    (dict(I=100), dfl.E_UNSUPPORTED), (dict(Hq=30), dfl.E_ARG), (dict(eps=-1.0), dfl.E_ARG),
    (dict(theta=0.5), dfl.E_ARG), (dict(mask=3), dfl.E_ARG), (dict(ps=32), dfl.E_UNSUPPORTED),
    (dict(x=None), dfl.E_ARG), (dict(x=FAKE + 2), dfl.E_UNSUPPORTED), (dict(nws=0), dfl.E_WORKSPACE),
    (dict(ln1=None), dfl.E_ARG),
])
def test_draft_layer_argument_errors(lib, kw, code):
    a = dict(D=128, k=16, d=4096, I=12288, Hq=32, eps=1e-6, theta=1e6, mask=0, ps=16, x=FAKE,
             nws=1 << 30, ln1=FAKE)
    a.update(kw)
    w = dfl.DraftLayerWeights(a["ln1"], FAKE, None, None, FAKE, FAKE, FAKE, FAKE)
    s = lib.dflash_draft_layer(4, a["k"], a["d"], a["Hq"], 8, a["D"], a["I"], a["x"], ctypes.byref(w),
                               a["eps"], a["theta"], FAKE, FAKE, 100, a["ps"], FAKE, 64, FAKE,
                               a["mask"], dfl.BF16, WS, a["nws"], None)
    assert s == code


@no_gpu
def test_draft_head_and_embed_argument_errors(lib):
    assert lib.dflash_draft_head(16, 4096, 1000, FAKE, FAKE, FAKE, 1e-6, FAKE, dfl.BF16, WS, 1 << 30,
                                 None) == dfl.E_UNSUPPORTED            # V % 128
    assert lib.dflash_draft_head(16, 4096, 1024, FAKE, FAKE, None, 1e-6, FAKE, dfl.BF16, WS, 1 << 30,
                                 None) == dfl.E_ARG
    assert lib.dflash_draft_head(16, 4096, 1024, FAKE, FAKE, FAKE, 1e-6, FAKE, dfl.BF16, WS, 0,
                                 None) == dfl.E_WORKSPACE
    assert lib.dflash_embed(4, 100, 10, FAKE, FAKE, FAKE, dfl.BF16, None) == dfl.E_UNSUPPORTED
    assert lib.dflash_embed(4, 128, 10, None, FAKE, FAKE, dfl.BF16, None) == dfl.E_ARG
    assert lib.dflash_embed(0, 128, 10, None, None, None, dfl.BF16, None) == dfl.OK


def test_binding_rejects_caches_not_in_head_major_layout():
    """The paged cache is [num_pages, Hkv, 16, D]; the binding checks each
    cache against the call's Hkv and D (and K against V) before any pointer
    crosses the ABI.  Shape checks come first, so CPU tensors reach them."""
    import torch
    Hkv, D = 8, 128
    good = torch.empty(4, Hkv, 16, D, dtype=torch.bfloat16)
    pos_major = torch.empty(4, 16, Hkv, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="head-major"):
        dfl._cache_pair(pos_major, pos_major, Hkv, D)
    with pytest.raises(ValueError, match="differ"):
        dfl._cache_pair(good, torch.empty(5, Hkv, 16, D, dtype=torch.bfloat16), Hkv, D)
    with pytest.raises(ValueError, match="device tensor"):
        dfl._cache_pair(good, good, Hkv, D)   # right shape, but host memory


@no_gpu
def test_noalloc_rejects_more_than_its_static_scratch(lib):
    """dflash_verify_greedy_noalloc: the chunk partials of B*(2L+1) rows fit
    the 1 MiB static scratch up to 131072 rows; one more row is rejected with
    DFLASH_E_TOO_LARGE before anything touches the device; argument errors
    come first, as in dflash_verify_greedy."""
    assert lib.dflash_noalloc_scratch_bytes() == 1 << 20

    def call(B, L, V=128256, **kw):
        a = dict(tl=FAKE, acc=FAKE, dtype=dfl.BF16)
        a.update(kw)
        return lib.dflash_verify_greedy_noalloc(B, L, V, a["tl"], V, None, 0, FAKE, None, None,
                                                a["acc"], FAKE, FAKE, None, None, a["dtype"], None)
    assert call(131073, 0) == dfl.E_TOO_LARGE            # 131073 rows of one target row each
    assert call(4033, 16) == dfl.E_TOO_LARGE             # 4033 * 33 = 133089 rows
    assert call(2, 65) == dfl.E_UNSUPPORTED
    assert call(131073, 0, acc=None) == dfl.E_ARG
    assert call(131073, 0, dtype=9) == dfl.E_ARG
    assert call(0, 15) == dfl.OK
