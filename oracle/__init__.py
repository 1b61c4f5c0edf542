"""CPU oracle for the DFlash draft-and-verify step -- TEST INFRASTRUCTURE.

Plain, slow, float64 NumPy statements of what the step computes.  Only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package; the product path (the HIP library and
its Python binding) never does, and this package never imports the product.

The pages this follows (cited by short title and section throughout):

* [DFlash overview] "DFlash 块扩散解码：以并行扩散替代自回归草稿，实现无损 6 倍推理加速"
  (pinghaoyang.com.cn/aigc/posts/dflash/) -- sections "块扩散", "KV 注入",
  "训练策略 / 随机锚点采样", "验证流程", "关键伪代码", and "草稿模型架构" (the
  drafter's decoder layers and shared head, followed by ``draft.py``).
* [SGLang DFlash] "详解SGlang 最新DFlash投机解码算法的工程实现、overlap策略和改进点"
  (10100.com/article/149138197) -- sections 3 (decode) and 4.1 (KV materialisation).
* [Spec-decoding tutorial] "让大模型快 8 倍：从投机解码到 DDTree 的完整原理"
  (liyongzhi.xyz/posts/2026/04/speculative-decoding/) -- sections 2, 3 (the
  acceptance rule, the residual distribution and the worked cat/dog example), 4,
  and 6 (DDTree: the draft tree, its best-first growth under a node budget, the
  ancestor-only mask and the target's attention under it, the greedy walk, and
  the commit of the accepted path's KV; followed by ``tree.py``).
* [DLoop] "DLoop 完全拆解：让一次验证覆盖多个草稿阶段的循环投机解码"
  (pinghaoyang.com.cn/aigc/posts/dloop-looped-speculative-decoding/) --
  "机制一：置信度门控" and "验证与无损性".

Inputs arrive as the raw storage arrays (bf16 as uint16 bit patterns, fp32
as float32); every function widens them exactly to float64 first.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
facts fixed by the pages or by mathematics (the worked example, closed forms,
identities, brute force with explicit masks, library routines on special
cases, a chi-square test of losslessness).  No function is "parity unpinned".
"""
from .numerics import widen, round_to_bf16, round_to_f32
from .materialize import (fuse_hiddens, project_kv, materialize, paged_write, gather_paged, slots,
                          k_norm, rope_half_split, row_positions)
from .attention import block_attention, block_attention_masked
from .verify import (verify_greedy, verify_sample, gate, row_log_softmax, residual, GreedyResult,
                     SampleResult, GateResult)
from .tree import (topk_logprobs, build_tree, ancestor_mask, walk_greedy, target_argmax, Tree,
                   TreeWalk, tree_attention, commit_tree_kv)
from .draft import rms_norm, silu, embed, draft_layer, draft_head

__all__ = [
    "widen", "round_to_bf16", "round_to_f32", "fuse_hiddens", "project_kv", "materialize",
    "paged_write", "gather_paged", "slots", "k_norm", "rope_half_split", "row_positions", "block_attention", "block_attention_masked",
    "verify_greedy", "verify_sample", "gate", "row_log_softmax", "residual", "GreedyResult",
    "SampleResult", "GateResult", "topk_logprobs", "build_tree", "ancestor_mask", "walk_greedy",
    "target_argmax", "Tree", "TreeWalk", "tree_attention", "commit_tree_kv", "rms_norm", "silu",
    "embed", "draft_layer", "draft_head",
]
