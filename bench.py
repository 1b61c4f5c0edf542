#!/usr/bin/env python3
"""Throughput of the DFlash draft-and-verify step on one MI355X.

One step = ctx-KV materialisation of the rows committed by the previous
verify (B requests x k rows, all five captured hiddens fused, K/V for every
draft layer written to the paged caches) + block attention for each draft
layer + greedy verification over the full vocabulary (target argmax, fused
draft argmax, acceptance, bonus).  Workload: the Llama-3.1-8B-shaped decode
step -- d_model 4096, 5 captured hiddens, 5 draft layers with 32 Q / 8 KV
heads of 128, block k = 16, ctx 8192 per request, vocab 128256, batch 64,
random weights ~N(0, 0.02), logits ~N(0, 3), caches ~N(0, 1), all bf16 and
resident in HBM before timing starts.

Prints one JSON line (rank 0) with blocks/s, the roofline of the dominant
kernel (block attention) measured live with HIP events, every part of the
step against its roofline (median of 50 launches after 10 warm-ups) with the
step-level fraction, and the CPU oracle timed on a bounded sample of the same
step.  Unless --headline-only, the line also carries one object per other
workload of the measurement plan -- the Qwen3-4B-shaped sampled chain verify
with DLoop gates (with the oracle's near-tie counts and its parity on the
bench's own inputs), the 4 x 32768-row prefill materialisation, and the
packed training mask -- each with its own roofline and oracle baseline.
"""
import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
# The attention kernel's measured HBM traffic (two rocprofv3 counter passes,
# scaled by a copy kernel of known size) is recorded with a hash of the
# sources it was measured on; it is reported only while they still match.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_b64_ctx8192_hbm_traffic.md")
ATTN_SOURCES = [os.path.join(ROOT, "block_diffusion_draft_ctx_amd", "csrc", f)
                for f in ("attention.hip", "common.h")]
BF16_PEAK = 2.5e15         # dense bf16 MFMA flop/s
METRIC = "draft-step blocks/sec (inject+block attn+verify); % HBM / MFMA peak"


def source_hash(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic():
    """Bytes per attention launch from the committed counter summary, or None
    when the summary is missing or the kernel sources changed since."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^\s*(\w+) = (\S+)\s*$", text, re.M))
    if vals.get("attention_sources_sha256") != source_hash(ATTN_SOURCES):
        return None
    try:
        return float(vals["attention_traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--ctx", type=int, default=8192)
    ap.add_argument("--block", type=int, default=16)
    ap.add_argument("--vocab", type=int, default=128256)
    ap.add_argument("--layers", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=32, help="requests in the oracle sample")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="prefill: rows in the oracle sample")
    ap.add_argument("--cpu-blocks", type=int, default=96,
                    help="packed: blocks in the oracle sample")
    ap.add_argument("--headline-only", action="store_true",
                    help="decode: skip the sub-objects of the other workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (HBM counter calibration)")
    ap.add_argument("--breakdown", action="store_true", help="per-part timings to stderr")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "sample-gate", "prefill", "packed", "tree", "tree-attn",
                             "draft"],
                    help="decode: the greedy decode step (default); sample-gate: Qwen3-4B-shaped "
                         "stochastic chain verify with DLoop gates; prefill: 4 x 32768-row "
                         "ctx-KV materialisation; packed: training-style packed block mask; "
                         "tree: DDTree build (top-K, best-first tree, ancestor mask) + greedy "
                         "tree verify; tree-attn: the target's attention over the flattened tree "
                         "(ancestor-only mask), one layer; draft: the drafter's forward (embedding, "
                         "5 Qwen3-8B-shaped layers over injected context, head)")
    ap.add_argument("--topk", type=int, default=8, help="tree: candidates per block position")
    ap.add_argument("--budget", type=int, default=512, help="tree: node budget")
    ap.add_argument("--sigma", type=float, default=1.0, help="sample-gate: draft = target + N(0, sigma)")
    ap.add_argument("--stages", type=int, default=4, help="sample-gate: DLoop stages of 8")
    ap.add_argument("--no-gate-lse", action="store_true",
                    help="sample-gate: the verify reduces the draft rows itself instead of reusing "
                         "the normalisers the gates computed")
    ap.add_argument("--k-epilogue", action="store_true",
                    help="decode and prefill: K goes through the per-head RMSNorm and the rotary "
                         "embedding (base 1e6) before it is stored")
    ap.add_argument("--causal", action="store_true",
                    help="decode and packed: causal mask inside the block (position i sees "
                         "block keys 0..i) instead of the bidirectional one")
    return ap.parse_args()


class Step:
    """Device-resident inputs, outputs and workspaces of one draft step."""

    def __init__(self, B, C, k, V, Ld, d=4096, m=5, Hq=32, Hkv=8, D=128, seed=0, causal=False,
                 k_epilogue=False):
        import torch
        import block_diffusion_draft_ctx_amd as dfl
        self.dfl = dfl
        self.causal = causal
        self.B, self.C, self.k, self.V, self.Ld = B, C, k, V, Ld
        self.d, self.m, self.Hq, self.Hkv, self.D = d, m, Hq, Hkv, D
        dev = torch.device("cuda:0")
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        bf = torch.bfloat16

        def randn(*shape, std=1.0):
            return (torch.randn(*shape, generator=g, device=dev, dtype=torch.float32) * std).to(bf)

        T = B * k
        self.T = T
        self.hiddens = [randn(T, d) for _ in range(m)]
        self.W_f = randn(d, m * d, std=0.02)
        self.b_f = randn(d, std=0.02)
        self.W_K = [randn(Hkv * D, d, std=0.02) for _ in range(Ld)]
        self.W_V = [randn(Hkv * D, d, std=0.02) for _ in range(Ld)]
        # K epilogue: per-layer norm weights around 1, rotary base 1e6
        self.k_epi = {}
        if k_epilogue:
            self.k_epi = dict(k_norm_weight=[(torch.rand(D, generator=g, device=dev) + 0.5).to(bf)
                                             for _ in range(Ld)],
                              k_norm_eps=1e-6, rope_theta=1e6)
        # pages for positions [0, C + k) of every request, physically shuffled
        self.max_pages = (C + k + 15) // 16
        num_pages = B * self.max_pages
        perm = torch.randperm(num_pages, generator=g, device=dev).to(torch.int32)
        self.block_table = perm.view(B, self.max_pages).contiguous()
        self.num_pages = num_pages
        self.cache_k = [randn(num_pages, Hkv, 16, D) for _ in range(Ld)]
        self.cache_v = [randn(num_pages, Hkv, 16, D) for _ in range(Ld)]
        self.q = [randn(B, k, Hq, D) for _ in range(Ld)]
        self.k_blk = [randn(B, k, Hkv, D) for _ in range(Ld)]
        self.v_blk = [randn(B, k, Hkv, D) for _ in range(Ld)]
        self.attn_out = [torch.empty(B, k, Hq, D, dtype=bf, device=dev) for _ in range(Ld)]
        self.ctx_lens = torch.full((B,), C, dtype=torch.int32, device=dev)
        # the rows committed last round sit right after the visible context
        self.seq_start = torch.full((B,), C, dtype=torch.int32, device=dev)
        self.commit = torch.full((B,), k, dtype=torch.int32, device=dev)
        self.target_logits = randn(B, k, V, std=3.0)
        self.draft_logits = randn(B, k - 1, V, std=3.0)
        self.draft_tokens = torch.empty(B, k - 1, dtype=torch.int32, device=dev)
        self.prefix = torch.full((B,), C, dtype=torch.int32, device=dev)
        L = dfl.lib()
        self.ws_mat = torch.empty(max(256, L.dflash_materialize_workspace_size(
            T, m, d, Ld, Hkv, D, dfl.BF16)), dtype=torch.uint8, device=dev)
        self.ws_att = torch.empty(max(256, L.dflash_attention_workspace_size(
            B, k, Hq, Hkv, D, self.max_pages, dfl.BF16)), dtype=torch.uint8, device=dev)
        self.ws_ver = torch.empty(max(256, L.dflash_verify_workspace_size(B, k - 1, V)),
                                  dtype=torch.uint8, device=dev)
        self.ver_out = {n: torch.empty(B, dtype=torch.int32, device=dev)
                        for n in ("accept_len", "bonus", "commit_lens", "new_seq_lens")}
        self.ver_out["target_predict"] = torch.empty(B, k, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    def materialize(self):
        self.dfl.materialize_ctx_kv(self.hiddens, self.W_f, self.b_f, self.W_K, self.W_V,
                                    self.cache_k, self.cache_v, self.block_table, self.k,
                                    self.seq_start, self.commit, workspace=self.ws_mat,
                                    **self.k_epi)

    def attention(self, l):
        self.dfl.block_attention(self.q[l], self.k_blk[l], self.v_blk[l], self.cache_k[l],
                                 self.cache_v[l], self.block_table, self.ctx_lens,
                                 out=self.attn_out[l], workspace=self.ws_att, causal=self.causal)

    def verify(self):
        self.dfl.verify_greedy(self.target_logits, draft_tokens=self.draft_tokens,
                               draft_logits=self.draft_logits, prefix_lens=self.prefix,
                               out=self.ver_out, workspace=self.ws_ver)

    # algorithmic work per launch
    def attn_bytes(self):
        B, C, k, Hq, Hkv, D = self.B, self.C, self.k, self.Hq, self.Hkv, self.D
        return B * C * Hkv * D * 2 * 2 + B * k * (2 * Hq + 2 * Hkv) * D * 2

    def attn_flops(self):
        blk = (self.k + 1) / 2 if self.causal else self.k   # block keys a query row sees, on average
        return 4.0 * self.B * self.k * self.Hq * self.D * (self.C + blk)

    def verify_bytes(self):
        return self.B * (2 * self.k - 1) * self.V * 2

    def mat_flops(self):
        return 2.0 * self.T * (self.m * self.d ** 2 + 2 * self.Ld * self.Hkv * self.D * self.d)

    def mat_bytes(self):
        d, m, T = self.d, self.m, self.T
        w = 2 * (m * d * d + d + 2 * self.Ld * self.Hkv * self.D * d)
        return T * m * d * 2 + w + T * 2 * self.Ld * self.Hkv * self.D * 2


def time_steps(st, steps, warmup):
    """Run warmup steps, then time `steps` whole steps; HIP events on the
    launch stream bracket every attention call inside the timed region."""
    import torch
    for _ in range(warmup):
        st.materialize()
        for l in range(st.Ld):
            st.attention(l)
        st.verify()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps * st.Ld)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    i = 0
    for _ in range(steps):
        st.materialize()
        for l in range(st.Ld):
            ev[i][0].record()
            st.attention(l)
            ev[i][1].record()
            i += 1
        st.verify()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    return total_ms / steps, sum(attn_ms) / len(attn_ms), wall


def time_part(fn, reps):
    import torch
    fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def cpu_baseline(st, n_req):
    """The oracle, as it stands, on n_req requests of the same step: their
    materialisation rows, their block attention for every layer, and their
    greedy verification.  Returns blocks/s on the host and the thread count."""
    import numpy as np
    import torch
    import oracle

    def host(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    k, C = st.k, st.C
    rows = slice(0, n_req * k)
    hid = [host(h[rows]) for h in st.hiddens]
    Wf, bf = host(st.W_f), host(st.b_f)
    WK = [host(w) for w in st.W_K]
    WV = [host(w) for w in st.W_V]
    bt = host(st.block_table[:n_req])
    pages = np.unique(bt[bt >= 0])
    remap = np.full(st.num_pages, -1, dtype=np.int64)
    remap[pages] = np.arange(len(pages))
    bt_c = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
    idx = torch.from_numpy(pages).to(st.block_table.device)
    ck = [host(c.index_select(0, idx)) for c in st.cache_k]
    cv = [host(c.index_select(0, idx)) for c in st.cache_v]
    q = [host(x[:n_req]) for x in st.q]
    kb = [host(x[:n_req]) for x in st.k_blk]
    vb = [host(x[:n_req]) for x in st.v_blk]
    tl = host(st.target_logits[:n_req])
    dl = host(st.draft_logits[:n_req])
    ctx = np.full(n_req, C, dtype=np.int32)
    t0 = time.perf_counter()
    epi = {}
    if st.k_epi:
        epi = dict(k_norm_weight=[host(w) for w in st.k_epi["k_norm_weight"]],
                   k_norm_eps=st.k_epi["k_norm_eps"], rope_theta=st.k_epi["rope_theta"],
                   rows_per_seq=k, seq_start_pos=np.full(n_req, C))
    res = oracle.materialize(hid, Wf, bf, WK, WV, st.Hkv, st.D, "bf16", **epi)
    for l in range(st.Ld):
        kc = oracle.widen(ck[l], "bf16")
        oracle.paged_write(kc, res["K"][l], bt_c, k, np.full(n_req, C), np.full(n_req, k))
        oracle.block_attention(q[l], kb[l], vb[l], ck[l], cv[l], bt_c, ctx, "bf16",
                               causal=st.causal)
    oracle.verify_greedy(tl, "bf16", draft_logits=dl, prefix_lens=np.full(n_req, C))
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return n_req / dt, dt, cores


def _events_ms(fn, steps, warmup):
    """Average milliseconds of fn() over `steps` calls after `warmup`, from HIP
    events recorded on the stream the library launches on."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _median_us(fn, n=50, warmup=10):
    """Median microseconds of fn() over n calls after `warmup` calls, each call
    bracketed by HIP events on the stream the library launches on (the timing
    protocol of the measurement plan: 10 warm-ups, then the median of 50)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return t[n // 2] if n % 2 else 0.5 * (t[n // 2 - 1] + t[n // 2])


def _host(t):
    """Device tensor -> numpy in storage form (bf16 as uint16 bits)."""
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def _graph_ms(fn, steps, warmup):
    """Average milliseconds of fn() replayed from a HIP graph: the calls are
    captured once (all outputs and workspaces allocated beforehand, no
    allocation or memset inside), then the graph is replayed `steps` times,
    so no host launch overhead sits between the kernels."""
    import torch
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(1, warmup)):
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def _base_line(args, metric, value, unit, ms, workload, higher=True, **cfg):
    return {"metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": higher,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": dict(workload=workload, **cfg)}


def bench_sample_gate(args):
    """Qwen3-4B-shaped stochastic verify with DLoop gating: batch 16, vocab
    151936, S stages of 8 drafts chained into one verify of 8S candidates
    (+ bonus).  One step = S gates (one per stage's draft rows) + one sampled
    chain verify; every request verifies the whole chain (the longest case)."""
    import torch
    import block_diffusion_draft_ctx_amd as dfl
    B, V, kk, S = 16, 151936, 8, args.stages
    L = kk * S
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(3000 + S)
    tl32 = torch.randn(B, L + 1, V, generator=g, device=dev) * 3.0
    dl32 = tl32[:, :L] + torch.randn(B, L, V, generator=g, device=dev) * args.sigma
    gumbel = -torch.log(-torch.log(torch.rand(B, L, V, generator=g, device=dev).clamp_min(1e-20)))
    drafts = torch.argmax(dl32 + gumbel, dim=-1).to(torch.int32)
    del gumbel
    tl = tl32.to(torch.bfloat16)
    dl = dl32.to(torch.bfloat16)
    del tl32, dl32
    # each stage's draft rows as the draft model emits them (one tensor per
    # stage, gated on its own); the chain verify reads all stages as one
    dstage = [dl[:, s_ * kk:(s_ + 1) * kk].contiguous() for s_ in range(S)]
    tstage = [drafts[:, s_ * kk:(s_ + 1) * kk].contiguous() for s_ in range(S)]
    u = (torch.randint(0, 1 << 24, (B, L), generator=g, device=dev).float() * 2.0 ** -24)
    u2 = (torch.randint(0, 1 << 24, (B,), generator=g, device=dev).float() * 2.0 ** -24)
    ws = torch.empty(max(256, dfl.lib().dflash_verify_workspace_size(B, L, V)), dtype=torch.uint8,
                     device=dev)
    wsg = torch.empty(max(256, dfl.lib().dflash_gate_workspace_size(B, kk, V)), dtype=torch.uint8,
                      device=dev)
    out = {}
    reuse = not args.no_gate_lse
    # each stage's gate writes its columns of the chain's [B, L] row statistics
    lse = torch.empty(B, L, dtype=torch.float32, device=dev)
    rmax = torch.empty(B, L, dtype=torch.float32, device=dev)
    gouts = [{"c": torch.empty(B, dtype=torch.float32, device=dev),
              "go": torch.empty(B, dtype=torch.int32, device=dev),
              "row_lse": lse[:, s_ * kk:(s_ + 1) * kk], "row_max": rmax[:, s_ * kk:(s_ + 1) * kk]}
             for s_ in range(S)]

    def gates():
        for s_ in range(S):
            dfl.gate(dstage[s_], tstage[s_], g=-0.5, out=gouts[s_], workspace=wsg)

    def verify():
        out.update(dfl.verify_sample(tl, dl, drafts, u, u2, audit=False, out=out or None,
                                     workspace=ws, draft_row_lse=lse if reuse else None))

    def step():
        gates()
        verify()

    ms = _events_ms(step, args.steps, args.warmup)
    vms = _events_ms(verify, args.steps, args.warmup)
    gms = _events_ms(gates, args.steps, args.warmup) / S
    # the verify's algorithmic bytes: every target row, and the draft rows
    # unless the gates already reduced them (then they count once, there)
    vbytes = B * ((L + 1) + (0 if reuse else L)) * V * 2
    gbytes = B * kk * V * 2
    step_bytes = B * (2 * L + 1) * V * 2    # each logit row once per step
    line = _base_line(args, "Qwen3-4B-shaped stochastic chain verify + DLoop gates, blocks/sec",
                      round(B / (ms * 1e-3), 1), "blocks/s", ms,
                      f"stochastic verify of a {S}-stage DLoop chain ({L} drafts + bonus) over vocab "
                      f"{V}, batch {B}, draft = target + N(0, {args.sigma}), T = 1, plus {S} gates "
                      f"(c >= -0.5) on the stages' draft rows" +
                      ("; the verify reuses the gates' draft-row normalisers" if reuse else ""),
                      batch=B, vocab=V, stages=S, chain=L, sigma=args.sigma,
                      gate_normalisers_reused=reuse)
    line["step_hbm_frac"] = round(step_bytes / (ms * 1e-3) / HBM_PEAK, 4)
    gms_step = _graph_ms(step, args.steps, args.warmup)
    line["graph_replay"] = {"ms_per_step": round(gms_step, 4),
                            "value": round(B / (gms_step * 1e-3), 1),
                            "step_hbm_frac": round(step_bytes / (gms_step * 1e-3) / HBM_PEAK, 4)}
    line["roofline"] = {"kernel": "verify_sample (all its launches)", "bound": "hbm",
                        "achieved": round(vbytes / (vms * 1e-3) / 1e9, 1), "peak": HBM_PEAK / 1e9,
                        "unit": "GB/s", "frac": round(vbytes / (vms * 1e-3) / HBM_PEAK, 4),
                        "traffic": None, "algorithmic_bytes": vbytes,
                        "avg_launch_us": round(vms * 1e3, 2)}
    line["gate"] = {"avg_us": round(gms * 1e3, 2), "algorithmic_bytes": gbytes,
                    "hbm_frac": round(gbytes / (gms * 1e-3) / HBM_PEAK, 4),
                    "go_fraction": round(float(torch.cat([o["go"] for o in gouts]).float().mean()), 4)}
    line["accept_len_mean"] = round(float(out["accept_len"].float().mean()), 3)
    vmed = _median_us(verify)
    gmed = _median_us(lambda: dfl.gate(dstage[0], tstage[0], g=-0.5, out=gouts[0], workspace=wsg))
    line["roofline"]["median_us"] = round(vmed, 2)
    line["roofline"]["frac_at_median"] = round(vbytes / (vmed * 1e-6) / HBM_PEAK, 4)
    line["gate"]["median_us"] = round(gmed, 2)
    # What bounds the call: its row pass streams the target rows once (a
    # library reduction over the same rows is the reference for the rate a
    # pass of this size reaches), then two dependent per-request launches
    # follow (acceptance scan + residual sums, bonus selection), each at
    # least one dependent launch of a trivial kernel.
    # (with the gates' normalisers reused the pass reads the target rows
    # alone; otherwise the draft rows too)
    rows2d = tl.view(-1, V) if reuse else torch.cat([tl.view(-1, V), dl.view(-1, V)])
    ref_us = _median_us(lambda: torch.sum(rows2d, dim=1, dtype=torch.float32))
    tiny = torch.zeros(16, device=dev)

    def ten_launches():
        for _ in range(10):
            tiny.add_(1.0)
    launch_us = _median_us(ten_launches) / 10
    line["bounds"] = {
        "row_pass_reference": {"what": f"torch.sum (fp32 accumulation) over the same "
                                       f"{rows2d.shape[0]} x {V} bf16 logit rows",
                               "median_us": round(ref_us, 2),
                               "hbm_frac": round(vbytes / (ref_us * 1e-6) / HBM_PEAK, 4)},
        "dependent_launch_us": round(launch_us, 2),
        "tail_launches": 2,
        "floor_us": round(ref_us + 2 * launch_us, 2),
        "frac_at_floor": round(vbytes / ((ref_us + 2 * launch_us) * 1e-6) / HBM_PEAK, 4)}
    if not getattr(args, "no_cpu_baseline", False):
        import numpy as np
        import oracle
        tlh, dlh, xh = _host(tl), _host(dl), _host(drafts)
        uh, u2h = _host(u), _host(u2)
        t0 = time.perf_counter()
        ref = oracle.verify_sample(tlh, dlh, xh, uh, u2h, "bf16")
        for s_ in range(S):
            oracle.gate(dlh[:, s_ * kk:(s_ + 1) * kk], xh[:, s_ * kk:(s_ + 1) * kk], "bf16", g=-0.5)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": round(B / dt, 3), "unit": "blocks/s", "cores": _cores(), "kind": "oracle",
            "sample": f"all {B} requests of the same step: the {S} gates and the sampled chain "
                      f"verify; {dt:.1f} s of CPU work"}
        acc, bon = _host(out["accept_len"]).astype(np.int64), _host(out["bonus"]).astype(np.int64)
        mism = np.flatnonzero((acc != ref.accept_len) | (bon != ref.bonus))
        near = [b for b in mism if ref.ratio_gap[b] < 1e-5 or ref.cdf_gap[b] < 1e-5]
        line["near_ties"] = {"ratio_lt_1e-5": int((ref.ratio_gap < 1e-5).sum()),
                             "cdf_lt_1e-5": int((ref.cdf_gap < 1e-5).sum()), "requests": B}
        line["oracle_parity"] = {"accept_len_or_bonus_mismatches": int(len(mism)),
                                 "of_which_near_ties": int(len(near))}
    return line


def bench_prefill(args):
    """Prefill ctx-KV materialisation: 4 sequences x 32768 positions, five
    captured hiddens fused by W_f [4096, 20480] + b_f, then K and V for five
    draft layers (8 KV heads x 128) into 16-token paged caches."""
    import torch
    import block_diffusion_draft_ctx_amd as dfl
    n_seq, rps, d, m, Ld, Hkv, D = 4, 32768, 4096, 5, 5, 8, 128
    T = n_seq * rps
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(4000)
    bf = torch.bfloat16

    def randn(*shape, std=1.0):
        return (torch.randn(*shape, generator=g, device=dev) * std).to(bf)

    hid = [randn(T, d) for _ in range(m)]
    Wf, bfv = randn(d, m * d, std=0.02), randn(d, std=0.02)
    WK = [randn(Hkv * D, d, std=0.02) for _ in range(Ld)]
    WV = [randn(Hkv * D, d, std=0.02) for _ in range(Ld)]
    maxp = rps // 16
    npg = n_seq * maxp
    bt = torch.randperm(npg, generator=g, device=dev).to(torch.int32).view(n_seq, maxp).contiguous()
    ck = [torch.empty(npg, Hkv, 16, D, dtype=bf, device=dev) for _ in range(Ld)]
    cv = [torch.empty(npg, Hkv, 16, D, dtype=bf, device=dev) for _ in range(Ld)]
    start = torch.zeros(n_seq, dtype=torch.int32, device=dev)
    ws = torch.empty(dfl.lib().dflash_materialize_workspace_size(T, m, d, Ld, Hkv, D, dfl.BF16),
                     dtype=torch.uint8, device=dev)
    epi = {}
    if args.k_epilogue:
        epi = dict(k_norm_weight=[(torch.rand(D, generator=g, device=dev) + 0.5).to(bf)
                                  for _ in range(Ld)], k_norm_eps=1e-6, rope_theta=1e6)

    def step():
        dfl.materialize_ctx_kv(hid, Wf, bfv, WK, WV, ck, cv, bt, rps, start, None, workspace=ws,
                               **epi)

    ms = _events_ms(step, args.steps, args.warmup)
    flops = 2.0 * T * (m * d * d + 2 * Ld * Hkv * D * d)
    line = _base_line(args, "prefill ctx-KV materialisation, rows/sec", round(T / (ms * 1e-3), 1),
                      "rows/s", ms, f"prefill ctx-KV materialisation: {n_seq} x {rps} rows, 5 "
                      f"hiddens of 4096 fused by W_f [4096, 20480] + b_f, K and V of {Ld} draft "
                      f"layers (8 KV heads x 128) written to 16-token paged caches, K epilogue: "
                      f"{_epi_name(args)}", rows=T, d_model=d, draft_layers=Ld,
                      k_epilogue=_epi_name(args))
    line["roofline"] = {"kernel": "materialize (both GEMMs)", "bound": "mfma",
                        "achieved": round(flops / (ms * 1e-3) / 1e12, 1), "peak": BF16_PEAK / 1e12,
                        "unit": "TFLOP/s", "frac": round(flops / (ms * 1e-3) / BF16_PEAK, 4),
                        "traffic": None, "algorithmic_flops": flops,
                        "avg_launch_us": round(ms * 1e3, 2)}
    med = _median_us(step)
    line["roofline"]["median_us"] = round(med, 1)
    line["roofline"]["frac_at_median"] = round(flops / (med * 1e-6) / BF16_PEAK, 4)
    if not getattr(args, "no_cpu_baseline", False):
        import numpy as np
        import oracle
        n = min(args.cpu_rows, rps)
        hh = [_host(h[:n]) for h in hid]
        Wfh, bfh = _host(Wf), _host(bfv)
        WKh, WVh = [_host(w) for w in WK], [_host(w) for w in WV]
        pages = _host(bt[0, :(n + 15) // 16]).astype(np.int64)
        table = np.arange(len(pages), dtype=np.int32)[None, :]   # the rows' pages, compacted
        epi_h = {}
        if args.k_epilogue:
            epi_h = dict(k_norm_weight=[_host(w) for w in epi["k_norm_weight"]], k_norm_eps=1e-6,
                         rope_theta=1e6, rows_per_seq=n, seq_start_pos=np.zeros(1, np.int64))
        t0 = time.perf_counter()
        res = oracle.materialize(hh, Wfh, bfh, WKh, WVh, Hkv, D, "bf16", **epi_h)
        for l in range(Ld):
            for rows in (res["K"][l], res["V"][l]):
                cache = np.zeros((len(pages), Hkv, 16, D))
                oracle.paged_write(cache, rows, table, n, np.zeros(1, np.int64))
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": round(n / dt, 1), "unit": "rows/s", "cores": _cores(), "kind": "oracle",
            "sample": f"the first {n} of the {T} rows (sequence 0, positions 0..{n - 1}): fused, "
                      f"projected for all {Ld} layers and written to a compact copy of their "
                      f"pages; {dt:.1f} s of CPU work, scaled to rows/s (rows are independent, "
                      f"so the rate extrapolates linearly in T)"}
    return line


def _mask_name(args):
    return "causal" if args.causal else "bidirectional"


def _epi_name(args):
    return "k_norm + rope (base 1e6)" if args.k_epilogue else "none"


def bench_packed(args):
    """Training-style packed block mask, forward only: one 8192-token
    sequence, up to 512 non-overlapping anchors in the loss region, block 16;
    each block attends to the target positions before its anchor and to its
    own block (32 Q / 8 KV heads x 128, one layer)."""
    import numpy as np
    import torch
    import block_diffusion_draft_ctx_amd as dfl
    import synth
    seq, kk, Hq, Hkv, D = 8192, 16, 32, 8, 128
    rng = synth.make_rng(5000)
    anchors, P = synth.packed_anchors(rng, seq, kk, 512)
    nb = len(anchors)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(5000)
    bf = torch.bfloat16
    npg = seq // 16
    perm = torch.randperm(npg, generator=g, device=dev).to(torch.int32)
    bt = perm.view(1, npg).contiguous()   # one shared row: every block reads the sequence
    ck = torch.randn(npg, Hkv, 16, D, generator=g, device=dev).to(bf)
    cv = torch.randn(npg, Hkv, 16, D, generator=g, device=dev).to(bf)
    q = torch.randn(nb, kk, Hq, D, generator=g, device=dev).to(bf)
    kb = torch.randn(nb, kk, Hkv, D, generator=g, device=dev).to(bf)
    vb = torch.randn(nb, kk, Hkv, D, generator=g, device=dev).to(bf)
    ctx = torch.from_numpy(anchors.astype(np.int32)).to(dev)
    out = torch.empty(nb, kk, Hq, D, dtype=bf, device=dev)
    ws = torch.empty(max(256, dfl.lib().dflash_attention_workspace_size(nb, kk, Hq, Hkv, D, npg,
                                                                        dfl.BF16)),
                     dtype=torch.uint8, device=dev)

    def step():
        dfl.block_attention(q, kb, vb, ck, cv, bt, ctx, out=out, workspace=ws, causal=args.causal)

    ms = _events_ms(step, args.steps, args.warmup)
    # keys seen summed over query rows: kk rows per block see its context and
    # kk block keys (or, causal, 1..kk of them)
    row_keys = kk * int(anchors.astype(np.int64).sum()) + nb * (kk * (kk + 1) // 2 if args.causal
                                                                 else kk * kk)
    flops = 4.0 * Hq * D * row_keys
    stream = float(anchors.astype(np.int64).sum()) * Hkv * D * 2 * 2
    line = _base_line(args, "packed block-mask attention, blocks/sec", round(nb / (ms * 1e-3), 1),
                      "blocks/s", ms, f"training-style packed block mask, forward: sequence {seq}, "
                      f"prompt {P}, {nb} anchors, block {kk} ({_mask_name(args)} inside the "
                      f"block), 32 Q / 8 KV heads x 128, one layer",
                      blocks=nb, seq_len=seq, prompt=P, mean_anchor=round(float(anchors.mean()), 1),
                      block_mask=_mask_name(args))
    line["roofline"] = {"kernel": "block_attention (packed)", "bound": "mfma",
                        "achieved": round(flops / (ms * 1e-3) / 1e12, 1), "peak": BF16_PEAK / 1e12,
                        "unit": "TFLOP/s", "frac": round(flops / (ms * 1e-3) / BF16_PEAK, 4),
                        "traffic": None, "algorithmic_flops": flops,
                        "avg_launch_us": round(ms * 1e3, 2),
                        "ctx_stream_GBps": round(stream / (ms * 1e-3) / 1e9, 1)}
    med = _median_us(step)
    line["roofline"]["median_us"] = round(med, 1)
    line["roofline"]["frac_at_median"] = round(flops / (med * 1e-6) / BF16_PEAK, 4)
    if not getattr(args, "no_cpu_baseline", False):
        import oracle
        sel = np.linspace(0, nb - 1, min(args.cpu_blocks, nb)).round().astype(np.int64)
        qh, kbh, vbh = _host(q)[sel], _host(kb)[sel], _host(vb)[sel]
        ckh, cvh = _host(ck), _host(cv)
        bth = np.repeat(_host(bt), len(sel), axis=0)
        t0 = time.perf_counter()
        oracle.block_attention(qh, kbh, vbh, ckh, cvh, bth, anchors[sel], "bf16",
                               causal=args.causal)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": round(len(sel) / dt, 3), "unit": "blocks/s", "cores": _cores(),
            "kind": "oracle",
            "sample": f"{len(sel)} of the {nb} blocks, evenly spaced in anchor order (mean anchor "
                      f"{float(anchors[sel].mean()):.0f}), all 32 heads; {dt:.1f} s of CPU work"}
    return line


def bench_tree(args):
    """DDTree on a Qwen3-8B-shaped drafter: 64 requests, a block of 16 (15
    drafted positions), vocab 151936, top-8 candidates per position, node
    budget 512.  One step = the tree build (top-K over every draft row, the
    best-first tree, the ancestor mask) + the greedy tree verify (argmax of
    the target row of the root and of every node, then the walk)."""
    import numpy as np
    import torch
    import block_diffusion_draft_ctx_amd as dfl
    B, n_pos, V, K, N = args.batch, args.block - 1, 151936, args.topk, args.budget
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(4000)
    # a confident drafter: one token per row raised well above the noise
    dl32 = torch.randn(B, n_pos, V, generator=g, device=dev) * 2.0
    peak = torch.randint(0, V, (B, n_pos), generator=g, device=dev)
    dl32.scatter_add_(2, peak[..., None], torch.full((B, n_pos, 1), 14.0, device=dev))
    dl = dl32.to(torch.bfloat16)
    del dl32
    tl = torch.empty(B, N + 1, V, dtype=torch.bfloat16, device=dev)
    for b in range(B):
        tl[b] = (torch.randn(N + 1, V, generator=g, device=dev) * 3.0).to(torch.bfloat16)
    wsb = torch.empty(max(256, dfl.lib().dflash_tree_workspace_size(B, n_pos, V, K)),
                      dtype=torch.uint8, device=dev)
    wsv = torch.empty(max(256, dfl.lib().dflash_tree_verify_workspace_size(B, N, V)),
                      dtype=torch.uint8, device=dev)
    tb, tv = {}, {}

    def build():
        tb.update(dfl.tree_build(dl, K, N, out=tb or None, workspace=wsb))

    def verify():
        tv.update(dfl.tree_verify_greedy(tl, tb["node_token"], tb["node_parent"], tb["n_nodes"],
                                         n_pos, out=tv or None, workspace=wsv))

    def step():
        build()
        verify()

    build()
    ms = _events_ms(step, args.steps, args.warmup)
    bms = _events_ms(build, args.steps, args.warmup)
    vms = _events_ms(verify, args.steps, args.warmup)
    gms = _graph_ms(step, args.steps, args.warmup)
    # algorithmic bytes: the verify reads every target row it needs once (the
    # root's and each built node's), the build every draft row once
    n_nodes = int(tb["n_nodes"].sum().item())
    vbytes = (B + n_nodes) * V * 2
    bbytes = B * n_pos * V * 2
    line = _base_line(args, "DDTree draft tree + greedy tree verify, blocks/sec",
                      round(B / (ms * 1e-3), 1), "blocks/s", ms,
                      f"Qwen3-8B-shaped DDTree step: batch {B}, {n_pos} drafted positions, vocab "
                      f"{V}, top-{K} per position, node budget {N}; build (top-K, best-first tree, "
                      f"ancestor mask) + greedy tree verify over {N + 1} target rows per request",
                      batch=B, positions=n_pos, vocab=V, topk=K, budget=N)
    line["roofline"] = {"kernel": "tree verify (target argmax over every node's row)",
                        "bound": "hbm", "achieved": round(vbytes / (vms * 1e-3) / 1e9, 1),
                        "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                        "frac": round(vbytes / (vms * 1e-3) / HBM_PEAK, 4), "traffic": None,
                        "algorithmic_bytes": vbytes, "avg_launch_us": round(vms * 1e3, 2)}
    line["breakdown"] = {"build_us": round(bms * 1e3, 1),
                         "build_topk_hbm_bytes": bbytes,
                         "verify_us": round(vms * 1e3, 1),
                         "mean_accept_len": round(float(tv["accept_len"].float().mean().item()), 3)}
    line["graph_replay"] = {"ms_per_step": round(gms, 4), "value": round(B / (gms * 1e-3), 1)}
    if not args.no_cpu_baseline:
        import time
        import oracle
        n_req = min(args.cpu_sample, B)

        def host(t):
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

        dt = 0.0
        for b in range(n_req):
            dh, th = host(dl[b:b + 1]), host(tl[b:b + 1])     # copies outside the timed part
            t0 = time.perf_counter()
            tok, lp = oracle.topk_logprobs(dh, "bf16", K)
            tree = oracle.build_tree(tok[0], lp[0], N)
            oracle.ancestor_mask(tree.parent)
            pred = oracle.target_argmax(th[:, :len(tree.token) + 1], "bf16")[0]
            oracle.walk_greedy(tree.token, tree.parent, pred)
            dt += time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": round(n_req / dt, 3), "unit": "blocks/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n_req} of the {B} requests: their top-K, tree, mask, target argmax over "
                      f"the root's and every node's row, and the walk; {dt:.1f} s of CPU work"}
    return line


def bench_tree_attn(args):
    """The target's attention over the flattened DDTree, one layer
    (Llama-3.1-8B-shaped target: 32 Q / 8 KV heads x 128): 64 requests, ctx
    8192, node budget 512 (513 rows: the root and the nodes), the ancestor-only
    mask of trees built by dflash_tree_build from a confident drafter's rows
    (15 positions, top-8)."""
    import numpy as np
    import torch
    import block_diffusion_draft_ctx_amd as dfl
    B, C, N, Hq, Hkv, D = args.batch, args.ctx, args.budget, 32, 8, 128
    R = N + 1
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(6000)
    bf = torch.bfloat16
    # tree shapes from a confident drafter (the vocabulary only sets the shape)
    dl = torch.randn(B, args.block - 1, 4096, generator=g, device=dev) * 2.0
    peak = torch.randint(0, 4096, (B, args.block - 1), generator=g, device=dev)
    dl.scatter_add_(2, peak[..., None], torch.full((B, args.block - 1, 1), 8.0, device=dev))
    tb = dfl.tree_build(dl.to(bf), args.topk, N)
    mask = tb["ancestor_mask"]
    npg = B * C // 16
    bt = torch.randperm(npg, generator=g, device=dev).to(torch.int32).view(B, C // 16).contiguous()
    ck = torch.randn(npg, Hkv, 16, D, generator=g, device=dev).to(bf)
    cv = torch.randn(npg, Hkv, 16, D, generator=g, device=dev).to(bf)
    q = torch.randn(B, R, Hq, D, generator=g, device=dev).to(bf)
    kt = torch.randn(B, R, Hkv, D, generator=g, device=dev).to(bf)
    vt = torch.randn(B, R, Hkv, D, generator=g, device=dev).to(bf)
    ctx = torch.full((B,), C, dtype=torch.int32, device=dev)
    out = torch.empty(B, R, Hq, D, dtype=bf, device=dev)
    ws = torch.empty(max(256, dfl.lib().dflash_tree_attention_workspace_size(B, R, Hq, Hkv, D,
                                                                             C // 16, dfl.BF16)),
                     dtype=torch.uint8, device=dev)

    def step():
        dfl.tree_attention(q, kt, vt, ck, cv, bt, ctx, mask, out=out, workspace=ws)

    ms = _events_ms(step, args.steps, args.warmup)
    # keys each row sees: the context, the root, and (node rows) its ancestors
    # and itself -- the bits of its mask row
    m = mask.cpu().numpy().view(np.uint32)
    node_bits = int(np.unpackbits(m.view(np.uint8)).sum())
    row_keys = B * R * (C + 1) + node_bits
    flops = 4.0 * Hq * D * row_keys
    line = _base_line(args, "DDTree tree attention (one target layer), blocks/sec",
                      round(B / (ms * 1e-3), 1), "blocks/s", ms,
                      f"the target's attention over the flattened DDTree, one layer: batch {B}, ctx "
                      f"{C}, node budget {N} ({R} rows: root + nodes), ancestor-only mask of trees "
                      f"built from 15 drafted positions (top-{args.topk}), 32 Q / 8 KV heads x 128",
                      batch=B, ctx=C, budget=N, topk=args.topk)
    line["roofline"] = {"kernel": "tree_attention (k_attn_wide, tree mask)", "bound": "mfma",
                        "achieved": round(flops / (ms * 1e-3) / 1e12, 1), "peak": BF16_PEAK / 1e12,
                        "unit": "TFLOP/s", "frac": round(flops / (ms * 1e-3) / BF16_PEAK, 4),
                        "traffic": None, "algorithmic_flops": flops,
                        "avg_launch_us": round(ms * 1e3, 2),
                        "mean_tree_keys_per_node_row": round(node_bits / (B * N), 2)}
    if not args.no_cpu_baseline:
        import time
        import oracle

        def host(t):
            t = t.detach().cpu().contiguous()
            return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == bf else t.numpy()

        # one request, all its rows, its own pages compacted
        pages = bt[0].long()
        par = host(tb["node_parent"][:1]).astype(np.int64)
        nn = host(tb["n_nodes"][:1])
        args_h = (host(q[:1]), host(kt[:1]), host(vt[:1]), host(ck[pages]), host(cv[pages]),
                  np.arange(C // 16, dtype=np.int32)[None], np.array([C], dtype=np.int32))
        rows = list(range(0, R, 2))
        t0 = time.perf_counter()
        oracle.tree_attention(*args_h, par, nn, "bf16", rows=rows)
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": round(len(rows) / R / dt, 5), "unit": "blocks/s", "cores": 1, "kind": "oracle",
            "sample": f"every 2nd row ({len(rows)} of {R}) of 1 of the {B} requests, all {Hq} "
                      f"heads at ctx {C}, scaled to a whole request; {dt:.1f} s of CPU work"}
    return line


def bench_draft(args):
    """The drafter's forward for one block per request, Qwen3-8B-shaped:
    embedding gather of [anchor, mask x 15], five decoder layers (d 4096, 32 Q
    / 8 KV heads x 128, d_ff 12288, q/k head norms, rotary base 1e6) each
    attending to its injected context (ctx 8192) and the block, then the
    final norm and the shared lm_head over vocab 151936 -> the draft logits."""
    import numpy as np
    import torch
    import block_diffusion_draft_ctx_amd as dfl
    B, k, C, Ld = args.batch, args.block, args.ctx, args.layers
    d, Hq, Hkv, D, I, V = 4096, 32, 8, 128, 12288, 151936
    M = B * k
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(7000)
    bf = torch.bfloat16

    def rnd(*shape, std=1.0, mean=0.0):
        return (torch.randn(*shape, generator=g, device=dev) * std + mean).to(bf)

    layers = []
    npg = B * C // 16
    for _ in range(Ld):
        w = {"ln1": rnd(d, std=0.1, mean=1.0), "qkv": rnd((Hq + 2 * Hkv) * D, d, std=0.02),
             "q_norm": rnd(D, std=0.1, mean=1.0), "k_norm": rnd(D, std=0.1, mean=1.0),
             "o": rnd(d, Hq * D, std=0.02), "ln2": rnd(d, std=0.1, mean=1.0),
             "gate_up": rnd(2 * I, d, std=0.02), "down": rnd(d, I, std=0.02)}
        layers.append((w, rnd(npg, Hkv, 16, D), rnd(npg, Hkv, 16, D)))
    bt = torch.randperm(npg, generator=g, device=dev).to(torch.int32).view(B, C // 16).contiguous()
    ctx = torch.full((B,), C, dtype=torch.int32, device=dev)
    table = rnd(V, d, std=0.02)
    lm = rnd(V, d, std=0.02)
    fnorm = rnd(d, std=0.1, mean=1.0)
    toks = torch.randint(0, V, (B, k), generator=g, device=dev).to(torch.int32)
    toks[:, 1:] = V - 1                                   # the mask token after each anchor
    x = torch.empty(M, d, dtype=bf, device=dev)
    logits = torch.empty(M, V, dtype=bf, device=dev)
    wsl = torch.empty(dfl.lib().dflash_draft_layer_workspace_size(B, k, d, Hq, Hkv, D, I, C // 16,
                                                                  dfl.BF16), dtype=torch.uint8, device=dev)
    wsh = torch.empty(dfl.lib().dflash_draft_head_workspace_size(M, d, V, dfl.BF16), dtype=torch.uint8,
                      device=dev)

    def step():
        dfl.embed(table, toks, out=x)
        for w, ck, cv in layers:
            dfl.draft_layer(x, w, ck, cv, bt, ctx, k, Hq, workspace=wsl)
        dfl.draft_head(x, fnorm, lm, out=logits, workspace=wsh)

    ms = _events_ms(step, args.steps, args.warmup)
    hms = _events_ms(lambda: dfl.draft_head(x, fnorm, lm, out=logits, workspace=wsh), args.steps,
                     args.warmup)
    lms = _events_ms(lambda: dfl.draft_layer(x, layers[0][0], layers[0][1], layers[0][2], bt, ctx, k,
                                             Hq, workspace=wsl), args.steps, args.warmup)
    gms = _graph_ms(step, args.steps, args.warmup)
    layer_params = (Hq + 2 * Hkv) * D * d + d * Hq * D + 2 * I * d + d * I
    gemm_flops = 2.0 * M * (Ld * layer_params + V * d)
    attn_flops = Ld * 4.0 * M * Hq * D * (C + k)
    head_flops = 2.0 * M * V * d
    line = _base_line(args, "drafter forward (embedding + layers + head), blocks/sec",
                      round(B / (ms * 1e-3), 1), "blocks/s", ms,
                      f"Qwen3-8B-shaped DFlash drafter forward: batch {B}, block {k}, {Ld} layers "
                      f"(d 4096, 32 Q / 8 KV heads x 128, d_ff 12288, q/k head norms, rotary 1e6) over "
                      f"injected context {C}, final norm and shared lm_head over vocab {V}",
                      batch=B, block=k, ctx=C, layers=Ld, d_model=d, d_ff=I, vocab=V)
    line["roofline"] = {"kernel": "lm_head GEMM (draft head)", "bound": "mfma",
                        "achieved": round(head_flops / (hms * 1e-3) / 1e12, 1),
                        "peak": BF16_PEAK / 1e12, "unit": "TFLOP/s",
                        "frac": round(head_flops / (hms * 1e-3) / BF16_PEAK, 4), "traffic": None,
                        "algorithmic_flops": head_flops, "avg_launch_us": round(hms * 1e3, 2)}
    line["breakdown"] = {"layer_us": round(lms * 1e3, 1), "head_us": round(hms * 1e3, 1),
                         "step_gemm_tflop": round(gemm_flops / 1e12, 3),
                         "step_attention_tflop": round(attn_flops / 1e12, 3),
                         "step_mfma_frac": round((gemm_flops + attn_flops) / (ms * 1e-3) / BF16_PEAK, 4)}
    line["graph_replay"] = {"ms_per_step": round(gms, 4), "value": round(B / (gms * 1e-3), 1)}
    if not args.no_cpu_baseline:
        import time
        import oracle

        def host(t):
            return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

        # one request: its 16 rows through every layer and the head
        pages = bt[0].long()
        hw = [({n: host(v) for n, v in w.items()}, host(ck[pages]), host(cv[pages])) for w, ck, cv in layers]
        th, tk = host(table), toks[:1].cpu().numpy()
        bth = np.arange(C // 16, dtype=np.int32)[None]
        ch = np.array([C], dtype=np.int32)
        fh, lh = host(fnorm), host(lm)
        t0 = time.perf_counter()
        xb = oracle.embed(th, tk, "bf16")          # float64 values on the bf16 grid
        for w, ck, cv in hw:
            xb = oracle.draft_layer(_f64_to_bf16_bits(xb), w, ck, cv, bth, ch, k=k, n_q_heads=Hq,
                                    n_kv_heads=Hkv, head_dim=D, dtype="bf16")
        oracle.draft_head(_f64_to_bf16_bits(xb), fh, lh, "bf16")
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {
            "value": round(1 / dt, 4), "unit": "blocks/s", "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"1 of the {B} requests: its {k} rows through the embedding, {Ld} layers "
                      f"(ctx {C}) and the head; {dt:.1f} s of CPU work"}
    return line


def _f64_to_bf16_bits(x):
    """float64 values already on the bf16 grid -> their bf16 bit patterns."""
    import numpy as np
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the step is "
              "data parallel by request (no collective), so one GPU's throughput at its share "
              "of the batch is the figure.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload != "decode":
        fn = {"sample-gate": bench_sample_gate, "prefill": bench_prefill,
              "packed": bench_packed, "tree": bench_tree,
              "tree-attn": bench_tree_attn, "draft": bench_draft}[args.workload]
        print(json.dumps(fn(args)), flush=True)
        return
    st = Step(args.batch, args.ctx, args.block, args.vocab, args.layers, causal=args.causal,
              k_epilogue=args.k_epilogue)
    print(f"[bench] inputs ready: B={st.B} ctx={st.C} k={st.k} V={st.V} layers={st.Ld}",
          file=sys.stderr, flush=True)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    ms, attn_ms, wall = time_steps(st, args.steps, args.warmup)
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    value = st.B / (ms * 1e-3)
    ab = st.attn_bytes()
    achieved = ab / (attn_ms * 1e-3)
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "blocks/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"Llama-3.1-8B-shaped DFlash decode step: batch {st.B}, ctx "
                                f"{st.C}, block {st.k} ({_mask_name(args)} inside the block), "
                                f"{st.Ld} draft layers (32 Q / 8 KV heads x 128), d_model 4096 "
                                f"with 5 captured hiddens, greedy verify over vocab {st.V} with "
                                f"fused draft argmax"),
                   "batch": st.B, "ctx": st.C, "block": st.k, "draft_layers": st.Ld,
                   "vocab": st.V, "d_model": st.d, "committed_rows": st.T,
                   "block_mask": _mask_name(args), "k_epilogue": _epi_name(args)},
        "roofline": {"kernel": "block_attention (per layer)", "bound": "hbm",
                     "achieved": round(achieved / 1e9, 1), "peak": HBM_PEAK / 1e9,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK, 4),
                     "traffic": recorded_traffic(), "algorithmic_bytes": ab,
                     "avg_launch_us": round(attn_ms * 1e3, 2)},
    }
    def whole_step():
        st.materialize()
        for l in range(st.Ld):
            st.attention(l)
        st.verify()

    gms = _graph_ms(whole_step, args.steps, args.warmup)
    out["graph_replay"] = {"ms_per_step": round(gms, 4), "value": round(st.B / (gms * 1e-3), 1)}
    # every part of the step: median of 50 launches after 10 warm-ups, against
    # its roofline time max(bytes / 8 TB/s, flops / 2.5 PF)
    parts = {}
    for name, fn, nbytes, flops, count in (
            ("inject", st.materialize, st.mat_bytes(), st.mat_flops(), 1),
            ("attention", lambda: st.attention(0), st.attn_bytes(), st.attn_flops(), st.Ld),
            ("verify", st.verify, st.verify_bytes(), 0.0, 1)):
        med = _median_us(fn)
        roof = max(nbytes / HBM_PEAK, flops / BF16_PEAK) * 1e6
        parts[name] = {"median_us": round(med, 2), "launches_per_step": count,
                       "roofline_us": round(roof, 2),
                       "bound": "hbm" if nbytes / HBM_PEAK >= flops / BF16_PEAK else "mfma",
                       "frac": round(roof / med, 4)}
    out["parts"] = parts
    out["step_roofline_frac"] = round(
        sum(p["roofline_us"] * p["launches_per_step"] for p in parts.values()) /
        sum(p["median_us"] * p["launches_per_step"] for p in parts.values()), 4)
    print(f"[bench] parts {json.dumps(parts)}", file=sys.stderr, flush=True)
    if args.breakdown:
        tm = time_part(st.materialize, 10)
        tv = time_part(st.verify, 10)
        br = {"materialize_us": round(tm * 1e3, 1),
              "materialize_mfma_frac": round(st.mat_flops() / (tm * 1e-3) / BF16_PEAK, 4),
              "attention_us_per_layer": round(attn_ms * 1e3, 1),
              "attention_hbm_frac": round(achieved / HBM_PEAK, 4),
              "verify_us": round(tv * 1e3, 1),
              "verify_hbm_frac": round(st.verify_bytes() / (tv * 1e-3) / HBM_PEAK, 4)}
        out["breakdown"] = br
        print(f"[bench] breakdown {json.dumps(br)}", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        v, dt, cores = cpu_baseline(st, args.cpu_sample)
        out["cpu_baseline"] = {
            "value": round(v, 3), "unit": "blocks/s", "cores": cores, "kind": "oracle",
            "sample": (f"{args.cpu_sample} of the {st.B} requests of the same step: their "
                       f"{args.cpu_sample * st.k} committed rows materialised, their block "
                       f"attention for all {st.Ld} layers at ctx {st.C}, their greedy verify "
                       f"({st.k} target + {st.k - 1} draft rows each); {dt:.1f} s of CPU work")}
    if not args.headline_only:
        # the other workloads of the measurement plan, each with its own
        # roofline and oracle baseline (defaults: 4 DLoop stages, sigma 1,
        # bidirectional block, no K epilogue)
        del st
        torch.cuda.empty_cache()
        sub = argparse.Namespace(**vars(args))
        sub.stages, sub.sigma, sub.no_gate_lse = 4, 1.0, False
        sub.causal, sub.k_epilogue = False, False
        out["configs"] = {}
        for key, fn in (("qwen3_4b_sampled_verify_dloop", bench_sample_gate),
                        ("prefill_materialize_t131072", bench_prefill),
                        ("packed_training_mask", bench_packed)):
            line = fn(sub)
            for k in ("n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline",
                      "dtype", "data"):
                line.pop(k, None)
            out["configs"][key] = line
            torch.cuda.empty_cache()
            print(f"[bench] {key}: {line['value']} {line['unit']}, roofline frac "
                  f"{line['roofline']['frac']}", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
