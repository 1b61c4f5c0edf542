// C ABI of the DFlash step: argument validation, workspace sizing, dispatch.
// Every host-visible argument error is reported before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/dflash.h"
#include "launch.h"

using namespace dflash;

namespace {

constexpr int kMaxL = 64;
constexpr size_t kWsAlign = 256;

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool bad_dtype(dflash_dtype d) { return d != DFLASH_F32 && d != DFLASH_BF16; }

dflash_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return DFLASH_OK;
  if (!ws || have < need) return DFLASH_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kWsAlign) return DFLASH_E_WORKSPACE;
  return DFLASH_OK;
}

dflash_status hip_status(hipError_t e) { return e == hipSuccess ? DFLASH_OK : DFLASH_E_HIP; }

// Shared checks of the verify entry points.
dflash_status check_verify_common(int B, int L, int V, const void* tl, int64_t ts,
                                  const void* dl, int64_t ds, bool need_dl) {
  if (B < 0 || L < 0 || V < 1) return DFLASH_E_ARG;
  if (L > kMaxL) return DFLASH_E_UNSUPPORTED;
  if (B == 0) return DFLASH_OK;
  if (!tl || ts < V) return DFLASH_E_ARG;
  if ((need_dl && !dl) || (dl && ds < V)) return DFLASH_E_ARG;
  return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "DFLASH_OK";
    case DFLASH_E_ARG: return "DFLASH_E_ARG: invalid argument";
    case DFLASH_E_UNSUPPORTED: return "DFLASH_E_UNSUPPORTED: shape or dtype not implemented";
    case DFLASH_E_WORKSPACE: return "DFLASH_E_WORKSPACE: workspace missing, too small or misaligned";
    case DFLASH_E_HIP: return "DFLASH_E_HIP: kernel launch failed";
    case DFLASH_E_TOO_LARGE:
      return "DFLASH_E_TOO_LARGE: the problem needs more scratch than the allocation-free "
             "entry point's static buffer holds";
  }
  return "DFLASH_E_UNKNOWN";
}

int dflash_version(void) { return 100; }

// ------------------------------------------------------------ materialise
size_t dflash_materialize_workspace_size(int64_t T, int m, int d_model, int n_layers,
                                         int n_kv_heads, int head_dim, dflash_dtype dtype) {
  if (T <= 0 || m <= 0 || d_model <= 0 || n_layers <= 0 || n_kv_heads <= 0 || head_dim <= 0)
    return 0;
  return materialize_ws_bytes(T, m, d_model, n_layers, n_kv_heads, head_dim, dtype == DFLASH_BF16);
}

dflash_status dflash_materialize_ctx_kv(
    int64_t T, int m, int d_model, const void* const* hiddens, const void* W_f, const void* b_f,
    int n_layers, int n_kv_heads, int head_dim, const void* const* W_K, const void* const* W_V,
    const dflash_kv_layer* caches, const int32_t* block_table, int max_pages_per_seq,
    int rows_per_seq, const int32_t* seq_start_pos, const int32_t* commit_lens,
    const dflash_k_epilogue* k_epilogue, void* h_ctx_out,
    dflash_dtype dtype, void* ws, size_t ws_bytes, dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (T < 0 || m < 1 || d_model < 1 || n_layers < 1 || n_kv_heads < 1 || head_dim < 1)
    return DFLASH_E_ARG;
  if (m > 8 || n_layers > kMaxLayers) return DFLASH_E_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return DFLASH_E_UNSUPPORTED;
  if (T == 0) return DFLASH_OK;
  if (T > INT32_MAX || (int64_t)m * d_model > INT32_MAX) return DFLASH_E_UNSUPPORTED;
  if (rows_per_seq < 1 || T % rows_per_seq != 0 || max_pages_per_seq < 1) return DFLASH_E_ARG;
  if (!hiddens || !W_f || !W_K || !W_V || !caches || !block_table || !seq_start_pos)
    return DFLASH_E_ARG;
  const bool bf16 = dtype == DFLASH_BF16;
  const int HD = n_kv_heads * head_dim;
  if (bf16 && (d_model % 128 != 0 || HD % 128 != 0)) return DFLASH_E_UNSUPPORTED;
  MatArgs a{};
  a.T = T; a.m = m; a.d = d_model;
  for (int s = 0; s < m; ++s) {
    if (!hiddens[s]) return DFLASH_E_ARG;
    if (bf16 && !al16(hiddens[s])) return DFLASH_E_UNSUPPORTED;
    a.hiddens[s] = hiddens[s];
  }
  if (bf16 && (!al16(W_f) || (h_ctx_out && !al16(h_ctx_out)))) return DFLASH_E_UNSUPPORTED;
  a.W_f = W_f; a.b_f = b_f;
  a.n_layers = n_layers; a.Hkv = n_kv_heads; a.D = head_dim;
  for (int l = 0; l < n_layers; ++l) {
    if (!W_K[l] || !W_V[l] || !caches[l].k || !caches[l].v) return DFLASH_E_ARG;
    if (caches[l].page_size != 16) return DFLASH_E_UNSUPPORTED;
    if (caches[l].num_pages < 1) return DFLASH_E_ARG;
    if (bf16 && (!al16(W_K[l]) || !al16(W_V[l]) || !al16(caches[l].k) || !al16(caches[l].v)))
      return DFLASH_E_UNSUPPORTED;
    a.W_K[l] = W_K[l]; a.W_V[l] = W_V[l];
    a.cache_k[l] = caches[l].k; a.cache_v[l] = caches[l].v;
    a.num_pages[l] = caches[l].num_pages;
  }
  a.block_table = block_table; a.max_pages = max_pages_per_seq;
  a.rows_per_seq = rows_per_seq; a.seq_start = seq_start_pos; a.commit_lens = commit_lens;
  a.h_out = h_ctx_out;
  if (k_epilogue) {
    const float eps = k_epilogue->k_norm_eps, theta = k_epilogue->rope_theta;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return DFLASH_E_ARG;
    if (!std::isfinite(theta) || !(theta == 0.f || theta > 1.f)) return DFLASH_E_ARG;
    if (k_epilogue->k_norm_weight) {
      for (int l = 0; l < n_layers; ++l) {
        const void* w = k_epilogue->k_norm_weight[l];
        if (!w) return DFLASH_E_ARG;
        if (!al16(w)) return DFLASH_E_UNSUPPORTED;
        a.k_norm_w[l] = w;
      }
      a.k_norm_on = true;
    }
    a.k_norm_eps = eps;
    a.rope_theta = theta;
  }
  const size_t need = materialize_ws_bytes(T, m, d_model, n_layers, n_kv_heads, head_dim, bf16);
  if (dflash_status s = check_ws(ws, ws_bytes, need)) return s;
  return hip_status(launch_materialize(bf16, a, ws, ws_bytes, static_cast<hipStream_t>(stream)));
}

// --------------------------------------------------------------- attention
size_t dflash_attention_workspace_size(int B, int k, int n_q_heads, int n_kv_heads, int head_dim,
                                       int max_pages_per_seq, dflash_dtype dtype) {
  if (B <= 0 || k <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      max_pages_per_seq <= 0 || n_q_heads % n_kv_heads)
    return 0;
  if (dtype != DFLASH_BF16) return 0;
  return attention_ws_bytes(B, k, n_q_heads, n_kv_heads, head_dim, max_pages_per_seq, true);
}

dflash_status dflash_block_attention(int B, int k, int n_q_heads, int n_kv_heads, int head_dim,
                                     const void* q, const void* k_blk, const void* v_blk,
                                     const void* cache_k, const void* cache_v, int num_pages,
                                     int page_size, const int32_t* block_table,
                                     int max_pages_per_seq, int table_rows,
                                     const int32_t* ctx_lens, float scale,
                                     dflash_block_mask block_mask, void* out, float* lse_out,
                                     dflash_dtype dtype,
                                     dflash_dtype out_dtype, void* ws, size_t ws_bytes,
                                     dflash_stream_t stream) {
  if (bad_dtype(dtype) || bad_dtype(out_dtype)) return DFLASH_E_ARG;
  if (dtype == DFLASH_F32 && out_dtype != DFLASH_F32) return DFLASH_E_UNSUPPORTED;
  if (B < 0 || k < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return DFLASH_E_ARG;
  if (n_q_heads % n_kv_heads) return DFLASH_E_ARG;
  if (head_dim != 64 && head_dim != 128) return DFLASH_E_UNSUPPORTED;
  if (k > 64 || (n_q_heads / n_kv_heads) * k > 256) return DFLASH_E_UNSUPPORTED;
  if (page_size != 16) return DFLASH_E_UNSUPPORTED;
  if (!(scale >= 0.f)) return DFLASH_E_ARG;
  if (block_mask != DFLASH_MASK_BIDIRECTIONAL && block_mask != DFLASH_MASK_CAUSAL) return DFLASH_E_ARG;
  if (B == 0) return DFLASH_OK;
  if (num_pages < 1 || max_pages_per_seq < 1) return DFLASH_E_ARG;
  if (table_rows != B && table_rows != 1) return DFLASH_E_ARG;
  if (!q || !k_blk || !v_blk || !cache_k || !cache_v || !block_table || !ctx_lens || !out)
    return DFLASH_E_ARG;
  const bool bf16 = dtype == DFLASH_BF16;
  if (bf16 && !(al16(q) && al16(k_blk) && al16(v_blk) && al16(cache_k) && al16(cache_v) && al16(out)))
    return DFLASH_E_UNSUPPORTED;
  const size_t need = bf16 ? attention_ws_bytes(B, k, n_q_heads, n_kv_heads, head_dim,
                                                max_pages_per_seq, true)
                           : 0;
  if (dflash_status s = check_ws(ws, ws_bytes, need)) return s;
  AttnArgs a{B, k, n_q_heads, n_kv_heads, head_dim, q, k_blk, v_blk, cache_k, cache_v, num_pages,
             block_table, max_pages_per_seq, table_rows == 1, ctx_lens, scale,
             block_mask == DFLASH_MASK_CAUSAL ? kMaskCausal : kMaskBidir, nullptr, out, lse_out,
             out_dtype == DFLASH_F32};
  return hip_status(launch_attention(bf16, a, ws, static_cast<hipStream_t>(stream)));
}

size_t dflash_tree_attention_workspace_size(int B, int n_rows, int n_q_heads, int n_kv_heads,
                                            int head_dim, int max_pages_per_seq,
                                            dflash_dtype dtype) {
  if (B <= 0 || n_rows <= 0 || n_rows > kTreeBudgetMax + 1 || n_q_heads <= 0 || n_kv_heads <= 0 ||
      head_dim <= 0 || max_pages_per_seq <= 0 || n_q_heads % n_kv_heads)
    return 0;
  if (dtype != DFLASH_BF16) return 0;
  return attention_ws_bytes(B, n_rows, n_q_heads, n_kv_heads, head_dim, max_pages_per_seq, true);
}

dflash_status dflash_tree_attention(int B, int n_rows, int n_q_heads, int n_kv_heads, int head_dim,
                                    const void* q, const void* k_tree, const void* v_tree,
                                    const void* cache_k, const void* cache_v, int num_pages,
                                    int page_size, const int32_t* block_table,
                                    int max_pages_per_seq, const int32_t* ctx_lens,
                                    const uint32_t* ancestor_mask, float scale, void* out,
                                    float* lse_out, dflash_dtype dtype, dflash_dtype out_dtype,
                                    void* ws, size_t ws_bytes, dflash_stream_t stream) {
  if (bad_dtype(dtype) || bad_dtype(out_dtype)) return DFLASH_E_ARG;
  if (dtype == DFLASH_F32 && out_dtype != DFLASH_F32) return DFLASH_E_UNSUPPORTED;
  if (B < 0 || n_rows < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return DFLASH_E_ARG;
  if (n_q_heads % n_kv_heads) return DFLASH_E_ARG;
  if (head_dim != 64 && head_dim != 128) return DFLASH_E_UNSUPPORTED;
  if (n_rows > kTreeBudgetMax + 1) return DFLASH_E_UNSUPPORTED;
  if (page_size != 16) return DFLASH_E_UNSUPPORTED;
  if (!(scale >= 0.f)) return DFLASH_E_ARG;
  if (B == 0) return DFLASH_OK;
  if (num_pages < 1 || max_pages_per_seq < 1) return DFLASH_E_ARG;
  if (!q || !k_tree || !v_tree || !cache_k || !cache_v || !block_table || !ctx_lens || !out)
    return DFLASH_E_ARG;
  if (n_rows > 1 && !ancestor_mask) return DFLASH_E_ARG;
  const bool bf16 = dtype == DFLASH_BF16;
  if (bf16 && !(al16(q) && al16(k_tree) && al16(v_tree) && al16(cache_k) && al16(cache_v) && al16(out)))
    return DFLASH_E_UNSUPPORTED;
  const size_t need = bf16 ? attention_ws_bytes(B, n_rows, n_q_heads, n_kv_heads, head_dim,
                                                max_pages_per_seq, true)
                           : 0;
  if (dflash_status s = check_ws(ws, ws_bytes, need)) return s;
  AttnArgs a{B, n_rows, n_q_heads, n_kv_heads, head_dim, q, k_tree, v_tree, cache_k, cache_v,
             num_pages, block_table, max_pages_per_seq, false, ctx_lens, scale, kMaskTree,
             ancestor_mask, out, lse_out, out_dtype == DFLASH_F32};
  return hip_status(launch_attention(bf16, a, ws, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ verify
size_t dflash_verify_workspace_size(int B, int L, int V) {
  if (B <= 0 || L < 0 || L > kMaxL || V < 1) return 0;
  const size_t a = greedy_ws_bytes(B, L, V), b = sample_ws_bytes(B, L, V);
  return a > b ? a : b;
}

dflash_status dflash_verify_greedy(int B, int L, int V, const void* target_logits,
                                   int64_t t_row_stride, const void* draft_logits,
                                   int64_t d_row_stride, int32_t* draft_tokens,
                                   const int32_t* chain_lens, int32_t* target_predict,
                                   int32_t* accept_len, int32_t* bonus, int32_t* commit_lens,
                                   const int32_t* prefix_lens, int32_t* new_seq_lens,
                                   dflash_dtype dtype, void* ws, size_t ws_bytes,
                                   dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (dflash_status s = check_verify_common(B, L, V, target_logits, t_row_stride, draft_logits,
                                            d_row_stride, false))
    return s;
  if (B == 0) return DFLASH_OK;
  if ((L > 0 && !draft_tokens) || !accept_len || !bonus || !commit_lens) return DFLASH_E_ARG;
  if ((prefix_lens == nullptr) != (new_seq_lens == nullptr)) return DFLASH_E_ARG;
  if (dflash_status s = check_ws(ws, ws_bytes, greedy_ws_bytes(B, L, V))) return s;
  return hip_status(launch_verify_greedy(dtype == DFLASH_BF16, B, L, V, target_logits,
                                         t_row_stride, draft_logits, d_row_stride, draft_tokens,
                                         chain_lens, target_predict, accept_len, bonus,
                                         commit_lens, prefix_lens, new_seq_lens, ws,
                                         static_cast<hipStream_t>(stream)));
}

dflash_status dflash_verify_greedy_noalloc(int B, int L, int V, const void* target_logits,
                                           int64_t t_row_stride, const void* draft_logits,
                                           int64_t d_row_stride, int32_t* draft_tokens,
                                           const int32_t* chain_lens, int32_t* target_predict,
                                           int32_t* accept_len, int32_t* bonus,
                                           int32_t* commit_lens, const int32_t* prefix_lens,
                                           int32_t* new_seq_lens, dflash_dtype dtype,
                                           dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (dflash_status s = check_verify_common(B, L, V, target_logits, t_row_stride, draft_logits,
                                            d_row_stride, false))
    return s;
  if (B == 0) return DFLASH_OK;
  if ((L > 0 && !draft_tokens) || !accept_len || !bonus || !commit_lens) return DFLASH_E_ARG;
  if ((prefix_lens == nullptr) != (new_seq_lens == nullptr)) return DFLASH_E_ARG;
  if (greedy_ws_bytes(B, L, V) > kNoallocScratchBytes) return DFLASH_E_TOO_LARGE;
  void* scr = nullptr;
  if (noalloc_scratch(&scr) != hipSuccess) return DFLASH_E_HIP;
  // the kernels write every scratch word they read: nothing needs clearing
  return hip_status(launch_verify_greedy(dtype == DFLASH_BF16, B, L, V, target_logits,
                                         t_row_stride, draft_logits, d_row_stride, draft_tokens,
                                         chain_lens, target_predict, accept_len, bonus,
                                         commit_lens, prefix_lens, new_seq_lens, scr,
                                         static_cast<hipStream_t>(stream)));
}

size_t dflash_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

dflash_status dflash_verify_sample(int B, int L, int V, const void* target_logits,
                                   int64_t t_row_stride, const void* draft_logits,
                                   int64_t d_row_stride, const int32_t* draft_tokens,
                                   const int32_t* chain_lens, const float* u_accept,
                                   const float* u_bonus, float temperature,
                                   const float* draft_row_lse, int32_t* accept_len,
                                   int32_t* bonus, int32_t* commit_lens,
                                   const int32_t* prefix_lens, int32_t* new_seq_lens,
                                   float* ratio_out, float* beta_out, float* u_cdf_gap_out,
                                   dflash_dtype dtype, void* ws, size_t ws_bytes,
                                   dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (!(temperature > 0.f) || temperature == __builtin_huge_valf()) return DFLASH_E_ARG;
  if (dflash_status s = check_verify_common(B, L, V, target_logits, t_row_stride, draft_logits,
                                            d_row_stride, L > 0))
    return s;
  if (B == 0) return DFLASH_OK;
  if ((L > 0 && (!draft_tokens || !u_accept)) || !u_bonus || !accept_len || !bonus ||
      !commit_lens)
    return DFLASH_E_ARG;
  if ((prefix_lens == nullptr) != (new_seq_lens == nullptr)) return DFLASH_E_ARG;
  if (dflash_status s = check_ws(ws, ws_bytes, sample_ws_bytes(B, L, V))) return s;
  return hip_status(launch_verify_sample(
      dtype == DFLASH_BF16, B, L, V, target_logits, t_row_stride,
      draft_logits ? draft_logits : target_logits, draft_logits ? d_row_stride : t_row_stride,
      draft_tokens, chain_lens, u_accept, u_bonus, temperature, accept_len, bonus, commit_lens,
      prefix_lens, new_seq_lens, ratio_out, beta_out, u_cdf_gap_out,
      L > 0 ? draft_row_lse : nullptr, ws, static_cast<hipStream_t>(stream)));
}

// -------------------------------------------------------------------- gate
size_t dflash_gate_workspace_size(int B, int n, int V) {
  if (B <= 0 || n < 1 || n > kMaxL || V < 1) return 0;
  return gate_ws_bytes(B, n, V);
}

dflash_status dflash_gate(int B, int n, int V, const void* draft_logits, int64_t row_stride,
                          const int32_t* draft_tokens, const int32_t* valid_lens,
                          float temperature, float g, float* c_out, int32_t* go_out,
                          float* row_max_out, float* row_lse_out, int stats_ld,
                          dflash_dtype dtype, void* ws, size_t ws_bytes, dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (B < 0 || n < 1 || V < 1) return DFLASH_E_ARG;
  if (n > kMaxL) return DFLASH_E_UNSUPPORTED;
  if (!(temperature > 0.f) || temperature == __builtin_huge_valf() || g != g) return DFLASH_E_ARG;
  if (stats_ld != 0 && stats_ld < n) return DFLASH_E_ARG;
  if (B == 0) return DFLASH_OK;
  if (!draft_logits || row_stride < V || !draft_tokens || !c_out || !go_out) return DFLASH_E_ARG;
  if (dflash_status s = check_ws(ws, ws_bytes, gate_ws_bytes(B, n, V))) return s;
  return hip_status(launch_gate(dtype == DFLASH_BF16, B, n, V, draft_logits, row_stride,
                                draft_tokens, valid_lens, temperature, g, c_out, go_out,
                                row_max_out, row_lse_out, stats_ld ? stats_ld : n, ws,
                                static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ DDTree
size_t dflash_tree_workspace_size(int B, int n_pos, int V, int topk) {
  if (B <= 0 || n_pos <= 0 || V <= 0 || topk <= 0 || topk > kTreeTopkMax) return 0;
  return tree_ws_bytes(B, n_pos, V, topk);
}

size_t dflash_tree_verify_workspace_size(int B, int budget, int V) {
  if (B <= 0 || budget <= 0 || budget > kTreeBudgetMax || V <= 0) return 0;
  return tree_verify_ws_bytes(B, budget, V);
}

dflash_status dflash_tree_build(int B, int n_pos, int V, const void* draft_logits,
                                int64_t row_stride, float temperature, int topk, int budget,
                                int32_t* topk_tokens, float* topk_logp, int32_t* node_token,
                                int32_t* node_parent, int32_t* node_depth, float* node_logp,
                                int32_t* n_nodes, uint32_t* ancestor_mask, dflash_dtype dtype,
                                void* ws, size_t ws_bytes, dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (B < 0 || n_pos < 1 || V < 1 || topk < 1 || budget < 1) return DFLASH_E_ARG;
  if (topk > kTreeTopkMax || topk > V || budget > kTreeBudgetMax || n_pos > kMaxL)
    return DFLASH_E_UNSUPPORTED;
  if (!(temperature > 0.f) || temperature == __builtin_huge_valf()) return DFLASH_E_ARG;
  if (B == 0) return DFLASH_OK;
  if (!draft_logits || row_stride < V || !topk_tokens || !topk_logp || !node_token ||
      !node_parent || !node_depth || !node_logp || !n_nodes)
    return DFLASH_E_ARG;
  if (dflash_status s = check_ws(ws, ws_bytes, tree_ws_bytes(B, n_pos, V, topk))) return s;
  return hip_status(launch_tree_build(dtype == DFLASH_BF16, B, n_pos, V, draft_logits, row_stride,
                                      temperature, topk, budget, topk_tokens, topk_logp,
                                      node_token, node_parent, node_depth, node_logp, n_nodes,
                                      ancestor_mask, ws, static_cast<hipStream_t>(stream)));
}

dflash_status dflash_tree_verify_greedy(int B, int budget, int V, const void* target_logits,
                                        int64_t row_stride, const int32_t* node_token,
                                        const int32_t* node_parent, const int32_t* n_nodes,
                                        int max_depth, int32_t* accept_len, int32_t* bonus,
                                        int32_t* accepted_nodes, int32_t* commit_lens,
                                        const int32_t* prefix_lens, int32_t* new_seq_lens,
                                        dflash_dtype dtype, void* ws, size_t ws_bytes,
                                        dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (B < 0 || budget < 1 || V < 1 || max_depth < 1) return DFLASH_E_ARG;
  if (budget > kTreeBudgetMax) return DFLASH_E_UNSUPPORTED;
  if (B == 0) return DFLASH_OK;
  if (!target_logits || row_stride < V || !node_token || !node_parent || !n_nodes || !accept_len ||
      !bonus || !accepted_nodes || !commit_lens)
    return DFLASH_E_ARG;
  if ((prefix_lens == nullptr) != (new_seq_lens == nullptr)) return DFLASH_E_ARG;
  if (dflash_status s = check_ws(ws, ws_bytes, tree_verify_ws_bytes(B, budget, V))) return s;
  return hip_status(launch_tree_verify(dtype == DFLASH_BF16, B, budget, V, target_logits,
                                       row_stride, node_token, node_parent, n_nodes, max_depth,
                                       accept_len, bonus, accepted_nodes, commit_lens, prefix_lens,
                                       new_seq_lens, ws, static_cast<hipStream_t>(stream)));
}

dflash_status dflash_tree_commit_kv(int B, int n_rows, int n_layers, int n_kv_heads, int head_dim,
                                    const void* const* k_tree, const void* const* v_tree,
                                    const dflash_kv_layer* caches, const int32_t* block_table,
                                    int max_pages_per_seq, const int32_t* accepted_nodes,
                                    int max_depth, const int32_t* accept_len,
                                    const int32_t* prefix_lens, dflash_dtype dtype,
                                    dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (B < 0 || n_rows < 1 || n_layers < 1 || n_kv_heads < 1 || head_dim < 1 || max_depth < 1)
    return DFLASH_E_ARG;
  if (n_layers > kCommitMaxLayers) return DFLASH_E_UNSUPPORTED;
  if (B == 0) return DFLASH_OK;
  if (!k_tree || !v_tree || !caches || !block_table || !accepted_nodes || !accept_len ||
      !prefix_lens || max_pages_per_seq < 1)
    return DFLASH_E_ARG;
  const int es = dtype == DFLASH_BF16 ? 2 : 4;
  if (((int64_t)n_kv_heads * head_dim * es) % 16) return DFLASH_E_UNSUPPORTED;
  CommitArgs a{};
  a.B = B; a.R = n_rows; a.n_layers = n_layers; a.Hkv = n_kv_heads; a.D = head_dim; a.es = es;
  for (int l = 0; l < n_layers; ++l) {
    if (!k_tree[l] || !v_tree[l] || !caches[l].k || !caches[l].v || caches[l].num_pages < 1)
      return DFLASH_E_ARG;
    if (caches[l].page_size != 16) return DFLASH_E_UNSUPPORTED;
    if (!(al16(k_tree[l]) && al16(v_tree[l]) && al16(caches[l].k) && al16(caches[l].v)))
      return DFLASH_E_UNSUPPORTED;
    a.k_tree[l] = k_tree[l]; a.v_tree[l] = v_tree[l];
    a.cache_k[l] = caches[l].k; a.cache_v[l] = caches[l].v; a.num_pages[l] = caches[l].num_pages;
  }
  a.block_table = block_table; a.max_pages = max_pages_per_seq;
  a.path = accepted_nodes; a.max_depth = max_depth; a.accept_len = accept_len;
  a.prefix = prefix_lens;
  return hip_status(launch_tree_commit(a, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ drafter
static dflash_status draft_shape_check(int B, int k, int d, int Hq, int Hkv, int D, int I,
                                       dflash_dtype dtype) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (B < 0 || k < 1 || d < 8 || Hq < 1 || Hkv < 1 || D < 1 || I < 8) return DFLASH_E_ARG;
  if (Hq % Hkv) return DFLASH_E_ARG;
  if (D != 64 && D != 128) return DFLASH_E_UNSUPPORTED;
  if (k > 64 || (Hq / Hkv) * k > 256) return DFLASH_E_UNSUPPORTED;
  if (d % 128 || ((Hq + 2 * Hkv) * D) % 128 || (Hq * D) % 128 || I % 128) return DFLASH_E_UNSUPPORTED;
  return DFLASH_OK;
}

size_t dflash_draft_layer_workspace_size(int B, int k, int d_model, int n_q_heads, int n_kv_heads,
                                         int head_dim, int d_ff, int max_pages_per_seq,
                                         dflash_dtype dtype) {
  if (B <= 0 || max_pages_per_seq < 1 ||
      draft_shape_check(B, k, d_model, n_q_heads, n_kv_heads, head_dim, d_ff, dtype))
    return 0;
  DraftArgs a{};
  a.B = B; a.k = k; a.d = d_model; a.Hq = n_q_heads; a.Hkv = n_kv_heads; a.D = head_dim;
  a.I = d_ff; a.bf16 = dtype == DFLASH_BF16; a.max_pages = max_pages_per_seq;
  return draft_layer_ws_bytes(a);
}

dflash_status dflash_draft_layer(int B, int k, int d_model, int n_q_heads, int n_kv_heads,
                                 int head_dim, int d_ff, void* x,
                                 const dflash_draft_layer_weights* w, float eps, float rope_theta,
                                 const void* cache_k, const void* cache_v, int num_pages,
                                 int page_size, const int32_t* block_table, int max_pages_per_seq,
                                 const int32_t* ctx_lens, dflash_block_mask block_mask,
                                 dflash_dtype dtype, void* ws, size_t ws_bytes,
                                 dflash_stream_t stream) {
  if (dflash_status s = draft_shape_check(B, k, d_model, n_q_heads, n_kv_heads, head_dim, d_ff, dtype))
    return s;
  if (!(eps >= 0.f) || eps == __builtin_huge_valf()) return DFLASH_E_ARG;
  if (!(rope_theta == 0.f || (rope_theta > 1.f && rope_theta < __builtin_huge_valf())))
    return DFLASH_E_ARG;
  if (block_mask != DFLASH_MASK_BIDIRECTIONAL && block_mask != DFLASH_MASK_CAUSAL) return DFLASH_E_ARG;
  if (page_size != 16) return DFLASH_E_UNSUPPORTED;
  if (B == 0) return DFLASH_OK;
  if (!x || !w || !w->ln1 || !w->qkv || !w->o || !w->ln2 || !w->gate_up || !w->down || !cache_k ||
      !cache_v || !block_table || !ctx_lens || num_pages < 1 || max_pages_per_seq < 1)
    return DFLASH_E_ARG;
  const void* ptrs[] = {x, w->ln1, w->qkv, w->q_norm, w->k_norm, w->o, w->ln2, w->gate_up,
                        w->down, cache_k, cache_v};
  for (const void* q : ptrs)
    if (q && !al16(q)) return DFLASH_E_UNSUPPORTED;
  DraftArgs a{};
  a.B = B; a.k = k; a.d = d_model; a.Hq = n_q_heads; a.Hkv = n_kv_heads; a.D = head_dim;
  a.I = d_ff; a.bf16 = dtype == DFLASH_BF16;
  a.x = x; a.ln1 = w->ln1; a.w_qkv = w->qkv; a.q_norm = w->q_norm; a.k_norm = w->k_norm;
  a.w_o = w->o; a.ln2 = w->ln2; a.w_gate_up = w->gate_up; a.w_down = w->down;
  a.eps = eps; a.rope_theta = rope_theta;
  a.cache_k = cache_k; a.cache_v = cache_v; a.num_pages = num_pages;
  a.block_table = block_table; a.max_pages = max_pages_per_seq; a.ctx_lens = ctx_lens;
  a.causal = block_mask == DFLASH_MASK_CAUSAL;
  if (dflash_status s = check_ws(ws, ws_bytes, draft_layer_ws_bytes(a))) return s;
  return hip_status(launch_draft_layer(a, ws, static_cast<hipStream_t>(stream)));
}

size_t dflash_draft_head_workspace_size(int M, int d_model, int V, dflash_dtype dtype) {
  if (M <= 0 || d_model < 8 || V < 1 || bad_dtype(dtype)) return 0;
  return draft_head_ws_bytes(M, d_model, V, dtype == DFLASH_BF16);
}

dflash_status dflash_draft_head(int M, int d_model, int V, const void* x, const void* norm_weight,
                                const void* lm_head, float eps, void* logits, dflash_dtype dtype,
                                void* ws, size_t ws_bytes, dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (M < 0 || d_model < 8 || V < 1) return DFLASH_E_ARG;
  if (d_model % 128 || V % 128) return DFLASH_E_UNSUPPORTED;
  if (!(eps >= 0.f) || eps == __builtin_huge_valf()) return DFLASH_E_ARG;
  if (M == 0) return DFLASH_OK;
  if (!x || !norm_weight || !lm_head || !logits) return DFLASH_E_ARG;
  if (!(al16(x) && al16(norm_weight) && al16(lm_head) && al16(logits))) return DFLASH_E_UNSUPPORTED;
  if (dflash_status s = check_ws(ws, ws_bytes, draft_head_ws_bytes(M, d_model, V, dtype == DFLASH_BF16)))
    return s;
  return hip_status(launch_draft_head(dtype == DFLASH_BF16, M, d_model, V, x, norm_weight, lm_head,
                                      eps, logits, ws, static_cast<hipStream_t>(stream)));
}

dflash_status dflash_embed(int M, int d_model, int V, const void* table, const int32_t* tokens,
                           void* out, dflash_dtype dtype, dflash_stream_t stream) {
  if (bad_dtype(dtype)) return DFLASH_E_ARG;
  if (M < 0 || d_model < 8 || V < 1) return DFLASH_E_ARG;
  if (d_model % 8) return DFLASH_E_UNSUPPORTED;
  if (M == 0) return DFLASH_OK;
  if (!table || !tokens || !out) return DFLASH_E_ARG;
  if (!(al16(table) && al16(out))) return DFLASH_E_UNSUPPORTED;
  return hip_status(launch_embed(dtype == DFLASH_BF16, M, d_model, V, table, tokens, out,
                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"
