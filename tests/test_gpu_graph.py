"""HIP-graph capture of whole steps: every entry point launches on the
caller's stream and neither allocates nor clears memory, so a step can be
captured once and replayed.  Each replay (with eager work of the same calls
between replays) must reproduce the eager outputs bit for bit."""
import numpy as np
import pytest

import block_diffusion_draft_ctx_amd as dfl
import synth
from tests.gpu_util import bits, log, up

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match_eager(fn, outputs, partial=(), n=3):
    """outputs: tensors every call rewrites entirely (poisoned before each
    replay); partial: tensors a call writes only in part (paged caches:
    restored to their initial contents before each replay)."""
    import torch
    init = [t.clone() for t in partial]
    fn()
    torch.cuda.synchronize()
    eager = [bits(t).copy() for t in list(outputs) + list(partial)]
    g = _capture(fn)
    for r in range(n):
        for t in outputs:           # poison so that a replay must rewrite them
            t.view(torch.uint8).fill_(0xA5)
        for t, t0 in zip(partial, init):
            t.copy_(t0)
        g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(list(outputs) + list(partial), eager)):
            np.testing.assert_array_equal(bits(t), e, err_msg=f"replay {r}, output {i}")
        fn()                        # eager work between the replays
        torch.cuda.synchronize()
        log(f"  replay {r} matches eager")


def test_graph_replay_decode_step():
    """materialise + two layers of block attention (one split over the
    context) + greedy verify with the fused draft argmax."""
    import torch
    c = synth.materialize_case(2600, dtype="bf16", m=5, d_model=512, n_layers=2, n_kv_heads=8,
                               head_dim=128, n_seq=4, rows_per_seq=16, commit="random")
    ck = [up(x, "bf16") for x in c.cache_k]
    cv = [up(x, "bf16") for x in c.cache_v]
    hid = [up(h, "bf16") for h in c.hiddens]
    Wf, bf = up(c.W_f, "bf16"), up(c.b_f, "bf16")
    WK = [up(w, "bf16") for w in c.W_K]
    WV = [up(w, "bf16") for w in c.W_V]
    bt, start = up(c.block_table, "i32"), up(c.seq_start_pos, "i32")
    commit = up(c.commit_lens, "i32")
    h_out = torch.empty(c.T, 512, dtype=torch.bfloat16, device="cuda:0")
    wsm = torch.empty(max(256, dfl.lib().dflash_materialize_workspace_size(c.T, 5, 512, 2, 8, 128,
                                                                          dfl.BF16)),
                      dtype=torch.uint8, device="cuda:0")
    a = synth.attention_case(2601, dtype="bf16", B=2, k=16, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ctx_lens=[3000, 700])
    att_in = [up(x, "bf16") for x in (a.q, a.k_blk, a.v_blk, a.cache_k, a.cache_v)]
    abt, actx = up(a.block_table, "i32"), up(a.ctx_lens, "i32")
    att_out = torch.empty(a.q.shape, dtype=torch.bfloat16, device="cuda:0")
    att_lse = torch.empty((2, 32, 16), dtype=torch.float32, device="cuda:0")
    wsa = torch.empty(max(256, dfl.lib().dflash_attention_workspace_size(
        2, 16, 32, 8, 128, a.block_table.shape[1], dfl.BF16)), dtype=torch.uint8, device="cuda:0")
    v = synth.greedy_case(2602, dtype="bf16", B=4, L=15, V=32000, plant=False,
                          with_draft_logits=True)
    tl, dl = up(v.target_logits, "bf16"), up(v.draft_logits, "bf16")
    vo = {n: torch.empty(4, dtype=torch.int32, device="cuda:0")
          for n in ("accept_len", "bonus", "commit_lens")}
    vo["target_predict"] = torch.empty(4, 16, dtype=torch.int32, device="cuda:0")
    dtoks = torch.empty(4, 15, dtype=torch.int32, device="cuda:0")
    wsv = torch.empty(max(256, dfl.lib().dflash_verify_workspace_size(4, 15, 32000)),
                      dtype=torch.uint8, device="cuda:0")

    def step():
        dfl.materialize_ctx_kv(hid, Wf, bf, WK, WV, ck, cv, bt, 16, start, commit,
                               h_ctx_out=h_out, workspace=wsm)
        for causal in (False, True):
            dfl.block_attention(*att_in, abt, actx, out=att_out, lse=att_lse, workspace=wsa,
                                causal=causal)
        dfl.verify_greedy(tl, draft_tokens=dtoks, draft_logits=dl, out=vo, workspace=wsv)

    _replays_match_eager(step, [h_out, att_out, att_lse, dtoks, vo["accept_len"], vo["bonus"],
                                vo["target_predict"]], partial=[ck[0], ck[1], cv[0], cv[1]])


def test_graph_replay_dloop_gates_and_sampled_verify():
    """Four gates writing their columns of the chain's row statistics, then
    the sampled chain verify reusing them."""
    import torch
    B, L, V, kk = 8, 32, 50000, 8
    c = synth.sample_case(2603, dtype="bf16", B=B, L=L, V=V, sigma=1.0)
    tl, dl = up(c.target_logits, "bf16"), up(c.draft_logits, "bf16")
    toks = up(c.draft_tokens, "i32")
    u, u2 = up(c.u_accept, "f32"), up(c.u_bonus, "f32")
    stages = [(dl[:, s:s + kk].contiguous(), toks[:, s:s + kk].contiguous())
              for s in range(0, L, kk)]
    lse = torch.empty(B, L, dtype=torch.float32, device="cuda:0")
    mx = torch.empty(B, L, dtype=torch.float32, device="cuda:0")
    gouts = [{"c": torch.empty(B, dtype=torch.float32, device="cuda:0"),
              "go": torch.empty(B, dtype=torch.int32, device="cuda:0"),
              "row_lse": lse[:, s * kk:(s + 1) * kk], "row_max": mx[:, s * kk:(s + 1) * kk]}
             for s in range(L // kk)]
    wsg = torch.empty(max(256, dfl.lib().dflash_gate_workspace_size(B, kk, V)),
                      dtype=torch.uint8, device="cuda:0")
    wsv = torch.empty(max(256, dfl.lib().dflash_verify_workspace_size(B, L, V)),
                      dtype=torch.uint8, device="cuda:0")
    vo = {n: torch.empty(B, dtype=torch.int32, device="cuda:0")
          for n in ("accept_len", "bonus", "commit_lens")}
    vo["ratio"] = torch.empty(B, L, dtype=torch.float32, device="cuda:0")
    vo["beta"] = torch.empty(B, dtype=torch.float32, device="cuda:0")
    vo["cdf_gap"] = torch.empty(B, dtype=torch.float32, device="cuda:0")

    def step():
        for (d, t), o in zip(stages, gouts):
            dfl.gate(d, t, out=o, workspace=wsg)
        dfl.verify_sample(tl, dl, toks, u, u2, out=vo, workspace=wsv, draft_row_lse=lse)

    _replays_match_eager(step, [lse, mx, gouts[0]["c"], gouts[3]["go"], vo["accept_len"],
                                vo["bonus"], vo["ratio"], vo["beta"]])
