/*
 * dflash.h -- C ABI of the DFlash draft-and-verify step on AMD MI355X (gfx950).
 *
 * Twelve operations.  The five of the draft-and-verify step:
 *   dflash_materialize_ctx_kv  target-context KV injection
 *   dflash_block_attention     non-causal block attention over [ctx; block]
 *   dflash_verify_greedy       greedy acceptance over the full vocabulary
 *   dflash_verify_sample       lossless rejection sampling over the full vocabulary
 *   dflash_gate                DLoop block-confidence gate
 * and seven around them:
 *   dflash_tree_build          DDTree: top-K per position, best-first tree, ancestor mask
 *   dflash_tree_verify_greedy  DDTree: target argmax per node and the greedy walk
 *   dflash_tree_attention      DDTree: the target's attention under the ancestor-only mask
 *   dflash_tree_commit_kv      DDTree: the accepted path's KV into the paged cache
 *   dflash_draft_layer         the drafter's decoder layer around block attention
 *   dflash_draft_head          the drafter's final norm and shared lm_head
 *   dflash_embed               the shared embedding gather
 * plus one workspace-size query per operation that needs scratch memory,
 * dflash_status_string and dflash_version, and dflash_verify_greedy_noalloc
 * (the greedy verify on a static scratch buffer, for callers that cannot
 * allocate) with its dflash_noalloc_scratch_bytes.
 *
 * Pages these follow (cited by short title):
 *   [DFlash overview]  "DFlash 块扩散解码：以并行扩散替代自回归草稿，实现无损 6 倍推理加速"
 *                      pinghaoyang.com.cn/aigc/posts/dflash/
 *   [SGLang DFlash]    "详解SGlang 最新DFlash投机解码算法的工程实现、overlap策略和改进点"
 *                      www.10100.com/article/149138197
 *   [Spec tutorial]    "让大模型快 8 倍：从投机解码到 DDTree 的完整原理"
 *                      liyongzhi.xyz/posts/2026/04/speculative-decoding/
 *   [DLoop]            "DLoop 完全拆解：让一次验证覆盖多个草稿阶段的循环投机解码"
 *                      pinghaoyang.com.cn/aigc/posts/dloop-looped-speculative-decoding/
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership   Every tensor pointer is a device pointer owned by the caller,
 *             except where a parameter is documented as a host array.  The
 *             library never allocates, frees or keeps a pointer after the
 *             call returns.  Scratch memory comes from the caller's workspace
 *             `ws` of at least the size reported by the matching
 *             dflash_*_workspace_size() query (ws may be NULL when that size
 *             is 0).  The workspace must be 256-byte aligned and must not be
 *             shared by calls that may run concurrently.
 * Async       Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *             stream) and the call returns without waiting.  No entry point
 *             synchronises or copies to the host.
 * Layout      Row-major and contiguous unless a stride is given.  Strides
 *             are in elements.
 * Dtypes      DFLASH_BF16: bf16 storage for hiddens, weights, logits, Q/K/V
 *             and caches; all accumulation, softmax, ratio and CDF arithmetic
 *             is fp32.  DFLASH_F32: fp32 storage and arithmetic throughout.
 * Paged cache One tensor each for K and V, shape [num_pages, n_kv_heads,
 *             page_size, head_dim] (head-major: a page's positions of one
 *             kv-head are contiguous); page_size must be 16.  A block table
 *             [n_seq, max_pages_per_seq] of int32 maps a request's logical
 *             page (position / 16) to a physical page; -1 = unmapped.
 * Errors      A call returns DFLASH_OK or an error code.  Every argument error
 *             that the host can see is reported before anything is enqueued,
 *             and then nothing is enqueued.  DFLASH_E_HIP reports a failed
 *             launch.  Errors in device-resident data (a token id outside
 *             [0, V), a chain length outside [0, L], a page-table entry
 *             outside [0, num_pages)) are reported in band, as described at
 *             each entry point.  No exception crosses the ABI; the library
 *             never prints.
 * Threads     Calls from several host threads are safe.  The only global
 *             state is the static scratch of dflash_verify_greedy_noalloc
 *             (one buffer per GPU) and the per-device lookup of its address.
 */
#ifndef DFLASH_H_
#define DFLASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFLASH_OK = 0,
  DFLASH_E_ARG = 1,          /* a NULL pointer, a negative or inconsistent size */
  DFLASH_E_UNSUPPORTED = 2,  /* a valid request outside what is implemented (e.g. head_dim) */
  DFLASH_E_WORKSPACE = 3,    /* ws too small or misaligned */
  DFLASH_E_HIP = 4,          /* a HIP launch failed */
  DFLASH_E_TOO_LARGE = 5     /* more scratch than the allocation-free entry point's static
                                buffer holds (dflash_verify_greedy_noalloc) */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* What a block position sees of its own block (dflash_block_attention). */
typedef enum { DFLASH_MASK_BIDIRECTIONAL = 0, DFLASH_MASK_CAUSAL = 1 } dflash_block_mask;

/* One draft layer's paged KV cache (device pointers). */
typedef struct {
  void* k;           /* [num_pages, n_kv_heads, page_size, head_dim] */
  void* v;           /* same shape as k */
  int32_t num_pages;
  int32_t page_size; /* must be 16 */
} dflash_kv_layer;

typedef void* dflash_stream_t; /* a hipStream_t */

/* Human-readable name of a status code (static storage). */
const char* dflash_status_string(dflash_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int dflash_version(void);

/* ---------------------------------------------------------------------------
 * Target-context KV injection.
 *
 * [DFlash overview], section "KV 注入", steps 2-3: the m captured target
 * hidden states are concatenated along features and fused,
 *     h_ctx = [h_1; ...; h_m] W_f^T + b_f            (W_f: [d, m*d], b_f: [d])
 * and every draft layer l projects h_ctx into its own cache,
 *     K^(l) = h_ctx W_K^(l)^T,  V^(l) = h_ctx W_V^(l)^T  (W: [Hkv*D, d]).
 * [SGLang DFlash], section 4.1: only the committed rows of each request are
 * written, at the physical slots of their logical positions.
 *
 * T            rows to materialise (T = n_seq * rows_per_seq; T = 0 is a no-op)
 * m, d_model   number of captured hiddens and their width
 * hiddens      HOST array of m device pointers, each [T, d_model]; they are
 *              read as one virtual [T, m*d_model] matrix, hidden 0 first
 * W_f, b_f     [d_model, m*d_model] and [d_model] (b_f may be NULL: no bias)
 * n_layers, n_kv_heads, head_dim   draft layers and their KV geometry
 * W_K, W_V     HOST arrays of n_layers device pointers, each [Hkv*D, d_model]
 * caches       HOST array of n_layers dflash_kv_layer
 * block_table  [n_seq, max_pages_per_seq] int32
 * rows_per_seq row r belongs to request s = r / rows_per_seq and sits at
 *              logical position seq_start_pos[s] + r % rows_per_seq
 * commit_lens  [n_seq] int32 or NULL; when given, only rows with
 *              r % rows_per_seq < commit_lens[s] are written (the prefix-valid
 *              write of the SGLang page)
 * h_ctx_out    [T, d_model] in the storage dtype, or NULL
 * k_epilogue   NULL, or the K epilogue below
 * Rows whose page-table entry is outside [0, num_pages) are not written.
 * h_ctx is rounded to the storage dtype before the K/V projections; cache
 * entries are rounded to the storage dtype (bf16: round to nearest even).
 * Rows that map to one cache slot (aliased pages) leave that slot undefined.
 *
 * K epilogue ([SGLang DFlash], section 4.1: kv_proj_only, then k_norm, then
 * the rotary embedding at the token positions, then the prefix-valid write).
 * The page names the steps without their bodies; this library computes, per
 * row and kv-head, on the stored K projection and in fp32:
 *   k_norm   k <- k / sqrt(mean(k^2) + eps) * w      (w: the layer's [head_dim])
 *   rope     dims i and i + D/2 (i < D/2) rotate by a = pos * theta^(-2i/D):
 *            (x, y) <- (x cos a - y sin a, y cos a + x sin a)
 * with pos the row's logical position (the one that picks its cache slot),
 * then rounds once to the storage dtype.  V is untouched.
 *   k_norm_weight  HOST array of n_layers device pointers, each [head_dim] in
 *                  the storage dtype and 16-byte aligned; NULL: no k_norm
 *   k_norm_eps     >= 0 (finite)
 *   rope_theta     rotary base > 1 (finite); 0: no rotary embedding
 * Shape limits: bf16 needs d_model % 128 == 0, (n_kv_heads*head_dim) % 128
 * == 0 and 16-byte aligned tensors; m <= 8; n_layers <= 64; head_dim in
 * {64, 128}.
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* const* k_norm_weight;
  float k_norm_eps;
  float rope_theta;
} dflash_k_epilogue;

size_t dflash_materialize_workspace_size(int64_t T, int m, int d_model, int n_layers,
                                         int n_kv_heads, int head_dim, dflash_dtype dtype);

dflash_status dflash_materialize_ctx_kv(
    int64_t T, int m, int d_model, const void* const* hiddens,
    const void* W_f, const void* b_f,
    int n_layers, int n_kv_heads, int head_dim,
    const void* const* W_K, const void* const* W_V,
    const dflash_kv_layer* caches,
    const int32_t* block_table, int max_pages_per_seq,
    int rows_per_seq, const int32_t* seq_start_pos, const int32_t* commit_lens,
    const dflash_k_epilogue* k_epilogue, void* h_ctx_out,
    dflash_dtype dtype, void* ws, size_t ws_bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * Non-causal block attention.
 *
 * [DFlash overview], section "KV 注入" (the Attention formula) and section
 * "块扩散": each of the k positions of a request's block attends, with no
 * causal mask, to [K_ctx; K_blk] and [V_ctx; V_blk]; section "随机锚点采样":
 * in packed training each block sees the injected context of positions before
 * its anchor and only its own block (map each block to one request whose
 * ctx_len is its anchor, all requests reading the one sequence's block-table
 * row: table_rows = 1).
 *
 * For request b, q-head h (kv-head h / (Hq/Hkv)), block position i:
 *   keys   = cache K at logical positions [0, ctx_lens[b]) ++ k_blk[b, 0:k]
 *   out    = softmax(scale * q . keys) @ values,  lse = natural log-sum-exp
 *
 * block_mask selects what a block position sees of its own block:
 *   DFLASH_MASK_BIDIRECTIONAL  all k block keys (DFlash, as above);
 *   DFLASH_MASK_CAUSAL         block keys 0..i only ([DFlash overview], section
 *                              "块扩散的双向注意力问题": the JetSpec change);
 * the context part is fully visible in both modes.  The block-causal mask of
 * [Spec tutorial], section 5.3 (a block sees every earlier block and all of
 * itself) is the bidirectional mode over a context that holds the earlier
 * blocks.  Any other value is DFLASH_E_ARG.
 *
 * q            [B, k, Hq, D]      k_blk, v_blk  [B, k, Hkv, D]
 * cache_k/v    [num_pages, Hkv, 16, D]
 * block_table  [table_rows, max_pages_per_seq] int32;  ctx_lens [B] int32 (0 allowed)
 * table_rows   B (request b reads row b) or 1 (every request reads row 0:
 *              the blocks of one packed sequence)
 * scale        softmax scale; 0 means 1/sqrt(D)
 * out          [B, k, Hq, D] in out_dtype (DFLASH_BF16 needs bf16 inputs;
 *              DFLASH_F32 keeps the fp32 result unrounded);
 * lse_out      [B, Hq, k] fp32 or NULL
 * In band: if ctx_lens[b] is negative or exceeds max_pages_per_seq*16, or a
 * page entry it needs is outside [0, num_pages), request b's outputs are NaN.
 * Shape limits: head_dim in {64, 128}; Hq % Hkv == 0; 1 <= k <= 64;
 * (Hq/Hkv)*k <= 256; bf16 tensors 16-byte aligned.  The fp32 path needs no
 * workspace.
 * ------------------------------------------------------------------------- */
size_t dflash_attention_workspace_size(int B, int k, int n_q_heads, int n_kv_heads,
                                       int head_dim, int max_pages_per_seq, dflash_dtype dtype);

dflash_status dflash_block_attention(
    int B, int k, int n_q_heads, int n_kv_heads, int head_dim,
    const void* q, const void* k_blk, const void* v_blk,
    const void* cache_k, const void* cache_v, int num_pages, int page_size,
    const int32_t* block_table, int max_pages_per_seq, int table_rows,
    const int32_t* ctx_lens, float scale, dflash_block_mask block_mask, void* out,
    float* lse_out, dflash_dtype dtype, dflash_dtype out_dtype, void* ws, size_t ws_bytes,
    dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * Greedy verification.
 *
 * [SGLang DFlash], section 3: the target's prediction at row i is the argmax
 * of its logits; draft i is accepted while it equals the target prediction at
 * row i (leading run of matches); bonus = target prediction at row
 * accept_len; commit = accept_len + 1; new_seq_len = prefix_len + commit.
 * Argmax ties go to the lowest token id.
 *
 * target_logits  rows b*(L+1)+i, i = 0..L, each of V elements, t_row_stride
 *                elements apart
 * draft_logits   rows b*L+i (d_row_stride apart) or NULL.  When given, the
 *                drafts are their argmax and are written to draft_tokens
 *                (rows i < chain length); when NULL, draft_tokens is input.
 * draft_tokens   [B, L] int32
 * chain_lens     [B] int32 in [0, L], or NULL (= L): rows past the chain are
 *                not read
 * target_predict [B, L+1] int32 or NULL; -1 past the chain
 * accept_len, bonus, commit_lens  [B] int32 outputs
 * prefix_lens, new_seq_lens       [B] int32, both NULL or both given
 * In band: a chain length outside [0, L] or a draft token outside [0, V)
 * within the chain gives accept_len = bonus = -1, commit = 0,
 * new_seq_len = prefix_len.
 * Limits: 0 <= L <= 64; V >= 1.
 * ------------------------------------------------------------------------- */
size_t dflash_verify_workspace_size(int B, int L, int V);

dflash_status dflash_verify_greedy(
    int B, int L, int V,
    const void* target_logits, int64_t t_row_stride,
    const void* draft_logits, int64_t d_row_stride,
    int32_t* draft_tokens, const int32_t* chain_lens,
    int32_t* target_predict, int32_t* accept_len, int32_t* bonus, int32_t* commit_lens,
    const int32_t* prefix_lens, int32_t* new_seq_lens,
    dflash_dtype dtype, void* ws, size_t ws_bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * dflash_verify_greedy_noalloc -- for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): dflash_verify_greedy without a workspace.  Arguments,
 * results, layouts and in-band errors are those of dflash_verify_greedy, and
 * the results are bit-identical to it.
 *
 * Scratch   The chunk partials live in a static device buffer of
 *           DFLASH_NOALLOC_SCRATCH_BYTES (1 MiB) that each GPU holds from the
 *           first call on it until the process ends.  That holds every call
 *           with B * (2L + 1) <= 131072 rows; a larger call returns
 *           DFLASH_E_TOO_LARGE before anything is enqueued.  The call
 *           allocates nothing (no hipMalloc, hipFree or allocating library
 *           routine); its first call on a device looks up the buffer's
 *           address there (hipGetSymbolAddress).
 * Sharing   Every call on one GPU uses the same buffer, and every word a call
 *           reads it wrote first, so no state carries between calls.  Calls
 *           that can overlap on one GPU (concurrent streams, or several host
 *           threads on one device) race on it: serialise them, or use
 *           dflash_verify_greedy with a workspace each.
 * ------------------------------------------------------------------------- */
#define DFLASH_NOALLOC_SCRATCH_BYTES ((size_t)1 << 20)

dflash_status dflash_verify_greedy_noalloc(
    int B, int L, int V,
    const void* target_logits, int64_t t_row_stride,
    const void* draft_logits, int64_t d_row_stride,
    int32_t* draft_tokens, const int32_t* chain_lens,
    int32_t* target_predict, int32_t* accept_len, int32_t* bonus, int32_t* commit_lens,
    const int32_t* prefix_lens, int32_t* new_seq_lens,
    dflash_dtype dtype, dflash_stream_t stream);

/* The static scratch size the library was built with (bytes). */
size_t dflash_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------------------
 * Lossless rejection-sampling verification.
 *
 * [Spec tutorial], section 3: with p = softmax(target/T) and q =
 * softmax(draft/T) at a row, draft x is kept with probability min(1, p(x)/q(x));
 * at the first rejection the bonus is drawn from max(0, p - q) / (1 - beta),
 * beta = sum min(p, q); section 4: later drafts are discarded.  [DFlash
 * overview], pseudocode: if all drafts are kept the bonus is drawn from p of
 * the row after the last draft.  [DLoop], "验证与无损性": several stages are
 * verified as one chain of chain_lens[b] drafts.
 *
 * Randomness is supplied: row i is accepted iff u_accept[b,i] < p(x)/q(x);
 * the bonus is the smallest token x whose cumulative weight (ascending token
 * id) exceeds u_bonus[b] times the total weight, where the weight is the
 * residual max(0, p-q) (or p when that residual sums to 0) at a rejection and
 * p of row chain_len when all drafts are kept.
 *
 * target_logits [B, L+1, V] rows (t_row_stride apart); draft_logits [B, L, V]
 * rows (d_row_stride apart); draft_tokens [B, L]; chain_lens [B] or NULL;
 * u_accept [B, L] and u_bonus [B] in [0, 1); temperature > 0.
 * draft_row_lse [B, L] fp32 or NULL: logsumexp(draft row / T) of every draft
 *   row, as dflash_gate's row_lse_out gives it for the stages of a DLoop
 *   chain ([DLoop], "机制一：置信度门控" computes these normalisers during
 *   drafting).  When given, the draft rows are not reduced again: the verify
 *   reads the target rows, the drafted tokens' draft logits and the one
 *   rejected draft row.  It must come from the same draft_logits and
 *   temperature.
 * Outputs accept_len, bonus, commit_lens [B]; new_seq_lens as for greedy.
 * Audit outputs (each may be NULL):
 *   ratio_out [B, L]  p/q of every draft within the chain (NaN past it)
 *   beta_out  [B]     sum min(p, q) of the rejected row (NaN if none)
 *   u_cdf_gap_out [B] distance of u'*Z to the nearer CDF boundary of the
 *                     chosen token, divided by the total weight Z
 * In band: as for greedy.
 * Limits: 0 <= L <= 64; V >= 1.
 * ------------------------------------------------------------------------- */
dflash_status dflash_verify_sample(
    int B, int L, int V,
    const void* target_logits, int64_t t_row_stride,
    const void* draft_logits, int64_t d_row_stride,
    const int32_t* draft_tokens, const int32_t* chain_lens,
    const float* u_accept, const float* u_bonus, float temperature,
    const float* draft_row_lse,
    int32_t* accept_len, int32_t* bonus, int32_t* commit_lens,
    const int32_t* prefix_lens, int32_t* new_seq_lens,
    float* ratio_out, float* beta_out, float* u_cdf_gap_out,
    dflash_dtype dtype, void* ws, size_t ws_bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * DLoop confidence gate.
 *
 * [DLoop], "机制一：置信度门控": c = sum over the stage's drafted tokens of
 * the drafter's log-probability of that token; drafting continues iff c >= g.
 *   c[b]  = sum_{i < n_b} ( x_i-th logit / T - logsumexp(row / T) )
 *   go[b] = c[b] >= g
 * draft_logits [B, n, V] rows (row_stride apart); draft_tokens [B, n];
 * valid_lens [B] in [0, n] or NULL (= n); temperature > 0.
 * c_out [B] fp32, go_out [B] int32 (1/0); row_max_out, row_lse_out fp32
 * (max and logsumexp of row / T) or NULL: row i of request b goes to
 * element b * stats_ld + i (stats_ld >= n, or 0 for n), so the stages of a
 * DLoop chain can write their columns of one [B, chain] array, the layout
 * dflash_verify_sample's draft_row_lse reads.
 * In band: a token outside [0, V) or a valid length outside [0, n] gives
 * c = NaN and go = 0.
 * Limits: 1 <= n <= 64.
 * ------------------------------------------------------------------------- */
size_t dflash_gate_workspace_size(int B, int n, int V);

dflash_status dflash_gate(
    int B, int n, int V, const void* draft_logits, int64_t row_stride,
    const int32_t* draft_tokens, const int32_t* valid_lens,
    float temperature, float g, float* c_out, int32_t* go_out,
    float* row_max_out, float* row_lse_out, int stats_ld,
    dflash_dtype dtype, void* ws, size_t ws_bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * DDTree: a draft tree under a node budget, and its greedy verification.
 *
 * [Spec tutorial], section 6.  6.1: the root is the last committed token and
 * each block position offers its top-K candidates; 6.3: a path's joint
 * probability is the product of the per-position marginals and the tree is
 * grown best first (pop the most probable leaf, push its children) until it
 * holds `budget` nodes; 6.4: a node sees only its ancestors; 6.5: greedy
 * walk -- from the root step to the child whose token is the target's
 * prediction, stop at the first node without one; the path is committed and
 * the target's prediction there is the bonus.
 *
 * dflash_tree_build
 *   draft_logits [B, n_pos, V] rows (row_stride apart): row d is block
 *     position d + 1; temperature > 0; 1 <= topk <= 16, topk <= V;
 *     1 <= budget <= 1024; 1 <= n_pos <= 64
 *   topk_tokens, topk_logp  [B, n_pos, topk] outputs: each position's topk
 *     most probable tokens (ties to the lower id) and log softmax(row / T)
 *   node_token, node_parent, node_depth, node_logp  [B, budget] outputs, in
 *     pop order: the token, the parent node (-1: the root), the block
 *     position (1-based) and the joint log-probability; slots past n_nodes
 *     hold token -1, parent -2, depth 0, logp -inf
 *   n_nodes [B] output: nodes built (budget, or fewer if the whole tree of
 *     topk^1 + ... + topk^n_pos nodes is smaller)
 *   ancestor_mask [B, budget, (budget + 31) / 32] uint32 or NULL: bit j of
 *     row i is set iff node j is node i or one of its ancestors (the target's
 *     attention mask over the flattened tree); rows past n_nodes are zero
 *   Order of equal joint probabilities: the parent popped earlier first
 *   (the root's children first), then the lower sibling rank; so every
 *   parent precedes its children and the tree is unique.
 *
 * dflash_tree_verify_greedy
 *   target_logits [B, budget + 1, V] rows (row_stride apart): row 0 is the
 *     target's output after the root, row 1 + j its output after node j
 *     (rows past n_nodes[b] are not read); the prediction of a row is its
 *     argmax (ties to the lower id)
 *   node_token, node_parent, n_nodes  the tree, as dflash_tree_build gives it
 *   accept_len, bonus, commit_lens [B] outputs; accepted_nodes [B, max_depth]
 *     output: the accepted path's node indices, -1 past it.  The walk stops
 *     after max_depth accepted nodes: accept_len <= max_depth, the bonus is
 *     the target's prediction at the last node kept, and every committed row
 *     (commit = accept_len + 1) is the root or a listed node, so
 *     dflash_tree_commit_kv writes exactly commit_lens rows
 *   prefix_lens, new_seq_lens [B] or both NULL: new = prefix + commit
 *   In band: n_nodes[b] outside [0, budget] gives accept_len = bonus = -1,
 *   commit = 0.
 * ------------------------------------------------------------------------- */
size_t dflash_tree_workspace_size(int B, int n_pos, int V, int topk);
size_t dflash_tree_verify_workspace_size(int B, int budget, int V);

dflash_status dflash_tree_build(
    int B, int n_pos, int V, const void* draft_logits, int64_t row_stride,
    float temperature, int topk, int budget,
    int32_t* topk_tokens, float* topk_logp,
    int32_t* node_token, int32_t* node_parent, int32_t* node_depth, float* node_logp,
    int32_t* n_nodes, uint32_t* ancestor_mask,
    dflash_dtype dtype, void* ws, size_t ws_bytes, dflash_stream_t stream);

dflash_status dflash_tree_verify_greedy(
    int B, int budget, int V, const void* target_logits, int64_t row_stride,
    const int32_t* node_token, const int32_t* node_parent, const int32_t* n_nodes,
    int max_depth, int32_t* accept_len, int32_t* bonus, int32_t* accepted_nodes,
    int32_t* commit_lens, const int32_t* prefix_lens, int32_t* new_seq_lens,
    dflash_dtype dtype, void* ws, size_t ws_bytes, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * DDTree: the target's attention over the flattened tree, and the KV commit
 * of the accepted path.
 *
 * dflash_tree_attention -- [Spec tutorial], section 6.4: the target verifies
 * the whole tree in one pass.  The rows of request b are the root (row 0, the
 * last committed token, not yet in the cache) and the nodes (row 1 + j, node j
 * of dflash_tree_build).  Every row attends to the committed context (cache
 * positions [0, ctx_lens[b])) and to the tree rows on its own root path: row 0
 * sees itself; row 1 + j sees row 0 and the rows 1 + y of every node y whose
 * bit is set in node j's ancestor row (node j itself and its ancestors) --
 * never siblings or cousins, as if each path were prefilled alone.  A node
 * row whose ancestor row is all zero (past the tree) sees the context and the
 * root.  Key tiles with no visible key are skipped (the sparse blocks of the
 * mask).
 *
 * q            [B, n_rows, Hq, D]     k_tree, v_tree  [B, n_rows, Hkv, D]
 *              (position-encoded by the caller: a node's position is the
 *              context length plus its depth)
 * cache_k/v, num_pages, page_size, block_table [B, max_pages_per_seq],
 *   ctx_lens   as dflash_block_attention (one table row per request)
 * ancestor_mask [B, n_rows - 1, (n_rows + 30) / 32] uint32, as
 *              dflash_tree_build writes it for budget = n_rows - 1
 *              (NULL allowed only when n_rows = 1)
 * 1 <= n_rows <= 1025; head_dim 64 or 128; bf16 pointers 16-byte aligned
 * out, lse_out, scale, dtype, out_dtype, ws: as dflash_block_attention, with
 *   the workspace sized by dflash_tree_attention_workspace_size
 * In band: a page-table entry outside [0, num_pages) or ctx_len outside
 *   [0, 16 * max_pages_per_seq] makes that request's outputs NaN.
 *
 * dflash_tree_commit_kv -- [Spec tutorial], section 6.6: after the walk only
 * the accepted path's KV joins the cache; rejected rows are never stored.
 * For every layer l and request b with accept_len[b] >= 0, the rows
 *   t = 0 (the root) and t = 1 .. min(accept_len[b], max_depth) (tree row
 *   1 + accepted_nodes[b, t - 1])
 * of k_tree[l] / v_tree[l] ([B, n_rows, Hkv, D]) are copied to the cache slot
 * of logical position prefix_lens[b] + t (block_table [B, max_pages_per_seq],
 * 16-token pages of caches[l]).  A row on an unmapped or out-of-range page,
 * or whose node index is outside [0, n_rows - 1), is skipped.  accepted_nodes,
 * accept_len and the prefix are dflash_tree_verify_greedy's accepted_nodes,
 * accept_len and prefix_lens (the commit length is accept_len + 1).
 * n_layers <= 64; Hkv * D * element size a multiple of 16; every pointer
 * 16-byte aligned.  No workspace.
 * ------------------------------------------------------------------------- */
size_t dflash_tree_attention_workspace_size(int B, int n_rows, int n_q_heads, int n_kv_heads,
                                            int head_dim, int max_pages_per_seq,
                                            dflash_dtype dtype);

dflash_status dflash_tree_attention(
    int B, int n_rows, int n_q_heads, int n_kv_heads, int head_dim,
    const void* q, const void* k_tree, const void* v_tree,
    const void* cache_k, const void* cache_v, int num_pages, int page_size,
    const int32_t* block_table, int max_pages_per_seq, const int32_t* ctx_lens,
    const uint32_t* ancestor_mask, float scale, void* out, float* lse_out,
    dflash_dtype dtype, dflash_dtype out_dtype, void* ws, size_t ws_bytes,
    dflash_stream_t stream);

dflash_status dflash_tree_commit_kv(
    int B, int n_rows, int n_layers, int n_kv_heads, int head_dim,
    const void* const* k_tree, const void* const* v_tree, const dflash_kv_layer* caches,
    const int32_t* block_table, int max_pages_per_seq,
    const int32_t* accepted_nodes, int max_depth, const int32_t* accept_len,
    const int32_t* prefix_lens, dflash_dtype dtype, dflash_stream_t stream);

/* ---------------------------------------------------------------------------
 * The drafter around block attention.
 *
 * [DFlash overview], section "草稿模型架构": the drafter is a small
 * Qwen3-style decoder that shares the target's embedding table and lm_head;
 * its block is the anchor followed by mask tokens (section "块扩散"), and
 * every layer's attention sees that layer's injected context ("KV 注入",
 * written by dflash_materialize_ctx_kv) and the whole block.
 *
 * dflash_draft_layer: one decoder layer on the block rows x [B*k, d_model]
 * (request-major, updated in place):
 *   n1 = rmsnorm(x) * ln1;  [q | k | v] = n1 . qkv^T  (Hq, Hkv, Hkv heads of D)
 *   q = rope(rmsnorm_head(q) * q_norm), k = rope(rmsnorm_head(k) * k_norm)
 *       (a NULL norm weight skips that norm; rope_theta 0 skips the rotary
 *       embedding; half-split rotation; block position i of request b sits
 *       at ctx_lens[b] + i)
 *   a  = dflash_block_attention(q, k, v, the layer's cache, block_mask)
 *   x += a . o^T;  n2 = rmsnorm(x) * ln2
 *   [g | u] = n2 . gate_up^T;  x += (silu(g) * u) . down^T
 * rmsnorm(x) = x / sqrt(mean(x^2) + eps).  Weights are row-major [out, in];
 * no biases.  Every intermediate is stored (rounded) in the workspace; each
 * projection's product is rounded before its residual add.
 * bf16: d_model, (Hq + 2 Hkv) * D, Hq * D and d_ff multiples of 128, every
 * pointer 16-byte aligned; head_dim 64 or 128; k <= 64 and (Hq/Hkv) * k <=
 * 256 (dflash_block_attention's limits).  The cache arguments are those of
 * dflash_block_attention (one table row per request).
 *
 * dflash_draft_head: logits [M, V] = (rmsnorm(x) * norm_w) . lm_head^T.
 * dflash_embed: out [M, d_model] = table[tokens] (the shared embedding
 *   table [V, d_model]); a token outside [0, V) gives a NaN row (in band).
 * ------------------------------------------------------------------------- */
typedef struct {
  const void* ln1;        /* [d_model] */
  const void* qkv;        /* [(Hq + 2 Hkv) * D, d_model] */
  const void* q_norm;     /* [D] or NULL */
  const void* k_norm;     /* [D] or NULL */
  const void* o;          /* [d_model, Hq * D] */
  const void* ln2;        /* [d_model] */
  const void* gate_up;    /* [2 * d_ff, d_model]: gate rows, then up rows */
  const void* down;       /* [d_model, d_ff] */
} dflash_draft_layer_weights;

size_t dflash_draft_layer_workspace_size(int B, int k, int d_model, int n_q_heads, int n_kv_heads,
                                         int head_dim, int d_ff, int max_pages_per_seq,
                                         dflash_dtype dtype);

dflash_status dflash_draft_layer(
    int B, int k, int d_model, int n_q_heads, int n_kv_heads, int head_dim, int d_ff,
    void* x, const dflash_draft_layer_weights* weights, float eps, float rope_theta,
    const void* cache_k, const void* cache_v, int num_pages, int page_size,
    const int32_t* block_table, int max_pages_per_seq, const int32_t* ctx_lens,
    dflash_block_mask block_mask, dflash_dtype dtype, void* ws, size_t ws_bytes,
    dflash_stream_t stream);

size_t dflash_draft_head_workspace_size(int M, int d_model, int V, dflash_dtype dtype);

dflash_status dflash_draft_head(int M, int d_model, int V, const void* x, const void* norm_weight,
                                const void* lm_head, float eps, void* logits, dflash_dtype dtype,
                                void* ws, size_t ws_bytes, dflash_stream_t stream);

dflash_status dflash_embed(int M, int d_model, int V, const void* table, const int32_t* tokens,
                           void* out, dflash_dtype dtype, dflash_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DFLASH_H_ */
