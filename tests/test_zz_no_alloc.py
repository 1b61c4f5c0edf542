"""GPU: dflash_verify_greedy_noalloc (the allocation-free greedy verify for
callers that cannot allocate) against dflash_verify_greedy with a caller
workspace, through the C ABI, on two calls in a row -- the second smaller --
so that the static scratch's leftovers from the first call cannot leak into
the second.  Integer outputs must be bit-identical, and also equal the
oracle's."""
import numpy as np
import pytest

import block_diffusion_draft_ctx_amd as dfl
import oracle
import synth
from tests.gpu_util import down, log, up

pytestmark = pytest.mark.gpu

FIELDS = ("accept_len", "bonus", "commit_lens", "new_seq_lens", "target_predict", "draft_tokens")


def _inputs(seed, dtype, B, L, V, dl):
    c = synth.greedy_case(seed, dtype=dtype, B=B, L=L, V=V, plant=True, ties=3,
                          with_draft_logits=dl, chain="random")
    args = dict(draft_tokens=None if dl else up(c.draft_tokens, "i32"),
                draft_logits=up(c.draft_logits, dtype) if dl else None,
                chain_lens=up(c.chain_lens, "i32"), prefix_lens=up(c.prefix_lens, "i32"))
    ref = oracle.verify_greedy(c.target_logits, dtype, draft_tokens=None if dl else c.draft_tokens,
                               draft_logits=c.draft_logits, chain_lens=c.chain_lens,
                               prefix_lens=c.prefix_lens)
    return c, up(c.target_logits, dtype), args, ref


def _compare(c, a, b, ref):
    n = c.chain_lens
    for f in FIELDS:
        x, y = down(a[f]), down(b[f])
        if f == "draft_tokens":      # rows past a request's chain are not written
            for r in range(c.B):
                np.testing.assert_array_equal(x[r, :n[r]], y[r, :n[r]])
        else:
            np.testing.assert_array_equal(x, y, err_msg=f)
    np.testing.assert_array_equal(down(b["accept_len"]), ref.accept_len)
    np.testing.assert_array_equal(down(b["bonus"]), ref.bonus)
    np.testing.assert_array_equal(down(b["target_predict"]), ref.target_predict)


def test_noalloc_matches_the_workspace_entry_point_twice():
    import torch
    for seed, dtype, B, L, V, dl in [(4101, "bf16", 64, 15, 128256, True),    # decode launch
                                     (4102, "f32", 3, 5, 1001, False)]:      # then a smaller one
        log(f"noalloc greedy dtype={dtype} B={B} L={L} V={V} draft_logits={dl} seed={seed}")
        c, tl, args, ref = _inputs(seed, dtype, B, L, V, dl)
        ws_out = dfl.verify_greedy(tl, **args)
        na = dict(args)
        if dl:   # its own draft-token output buffer
            na["draft_tokens"] = torch.full((B, L), -7, dtype=torch.int32, device=tl.device)
        na_out = dfl.verify_greedy_noalloc(tl, **na)
        torch.cuda.synchronize()
        _compare(c, ws_out, na_out, ref)
        log(f"  ok: accept_len {down(na_out['accept_len'])[:8].tolist()}")
