// Internal launch interface between the C-ABI layer (api.cpp) and the kernel
// translation units.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash {

// ---------------------------------------------------------------- vocab pass
// Chunking of a vocabulary row: every row is cut into n_chunks pieces of
// `chunk` elements (a multiple of 8) and one workgroup reduces one piece.
struct VocabPlan {
  int chunk;
  int n_chunks;
};
VocabPlan plan_vocab(int64_t n_rows, int V);

struct RowSet {
  const void* base;     // first row
  int64_t stride;       // elements between rows
  int rows_per_req;     // rows of request b are b*rows_per_req + i
  int extra;            // row i is read iff i < n_b + extra
};

size_t greedy_ws_bytes(int B, int L, int V);
size_t sample_ws_bytes(int B, int L, int V);
size_t gate_ws_bytes(int B, int n, int V);

hipError_t launch_verify_greedy(bool bf16, int B, int L, int V, const void* tl, int64_t ts,
                                const void* dl, int64_t ds, int32_t* draft_tokens,
                                const int32_t* chain_lens, int32_t* target_predict,
                                int32_t* accept_len, int32_t* bonus, int32_t* commit_lens,
                                const int32_t* prefix_lens, int32_t* new_seq_lens, void* ws,
                                hipStream_t st);

// Static per-device scratch of the allocation-free greedy verify: its size,
// and its device address on the current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = size_t(1) << 20;
hipError_t noalloc_scratch(void** out);

hipError_t launch_verify_sample(bool bf16, int B, int L, int V, const void* tl, int64_t ts,
                                const void* dl, int64_t ds, const int32_t* draft_tokens,
                                const int32_t* chain_lens, const float* u_accept,
                                const float* u_bonus, float temperature, int32_t* accept_len,
                                int32_t* bonus, int32_t* commit_lens, const int32_t* prefix_lens,
                                int32_t* new_seq_lens, float* ratio_out, float* beta_out,
                                float* gap_out, const float* draft_lse, void* ws, hipStream_t st);

hipError_t launch_gate(bool bf16, int B, int n, int V, const void* dl, int64_t rs,
                       const int32_t* tokens, const int32_t* valid_lens, float temperature,
                       float g, float* c_out, int32_t* go_out, float* row_max, float* row_lse,
                       int stats_ld, void* ws, hipStream_t st);

// ------------------------------------------------------------------- DDTree
constexpr int kTreeTopkMax = 16;
constexpr int kTreeBudgetMax = 1024;
size_t tree_ws_bytes(int B, int n_pos, int V, int K);
size_t tree_build_lds_bytes(int n_pos, int K, int budget);
hipError_t launch_tree_build(bool bf16, int B, int n_pos, int V, const void* dl, int64_t rs,
                             float temperature, int K, int budget, int32_t* topk_tok,
                             float* topk_lp, int32_t* node_token, int32_t* node_parent,
                             int32_t* node_depth, float* node_logp, int32_t* n_nodes,
                             uint32_t* mask, void* ws, hipStream_t st);
size_t tree_verify_ws_bytes(int B, int budget, int V);
// KV commit of the accepted path: per layer, the tree pass's K/V rows and the
// paged cache they join
constexpr int kCommitMaxLayers = 64;
struct CommitArgs {
  int B, R, n_layers, Hkv, D, es;          // es: bytes per element
  const void* k_tree[kCommitMaxLayers];    // [B, R, Hkv, D]
  const void* v_tree[kCommitMaxLayers];
  void* cache_k[kCommitMaxLayers];         // [num_pages, Hkv, 16, D]
  void* cache_v[kCommitMaxLayers];
  int num_pages[kCommitMaxLayers];
  const int32_t* block_table;              // [B, max_pages]
  int max_pages;
  const int32_t* path;                     // [B, max_depth] accepted node indices
  int max_depth;
  const int32_t* accept_len;               // [B]
  const int32_t* prefix;                   // [B]
};
hipError_t launch_tree_commit(const CommitArgs& a, hipStream_t st);
hipError_t launch_tree_verify(bool bf16, int B, int budget, int V, const void* tl, int64_t ts,
                              const int32_t* node_token, const int32_t* node_parent,
                              const int32_t* n_nodes, int max_depth, int32_t* accept_len,
                              int32_t* bonus, int32_t* path, int32_t* commit,
                              const int32_t* prefix, int32_t* new_seq, void* ws, hipStream_t st);

// ----------------------------------------------------------------- attention
struct AttnArgs {
  int B, k, Hq, Hkv, D;
  const void* q;
  const void* k_blk;
  const void* v_blk;
  const void* cache_k;
  const void* cache_v;
  int num_pages;
  const int32_t* block_table;
  int max_pages;
  bool shared_table;  // every request reads block-table row 0
  const int32_t* ctx_lens;
  float scale;
  int mode;           // what a block row sees of the block: kMaskBidir, kMaskCausal, kMaskTree
  const uint32_t* tree_mask;  // kMaskTree: [B, k - 1, (k + 30) / 32] ancestor bit rows of the nodes
  void* out;
  float* lse;
  bool out_f32;  // bf16 inputs with an fp32 output
};
// Block masks: every block row sees all k block rows; row i sees rows 0..i;
// or (a flattened draft tree, row 0 the root, row 1 + j node j) row 0 sees
// itself and row 1 + j sees row 0 and the rows 1 + y of the nodes y whose bit
// is set in node j's ancestor row.
constexpr int kMaskBidir = 0, kMaskCausal = 1, kMaskTree = 2;
int attention_row_chunks(int G, int k);
int attention_splits(int B, int Hkv, int G, int k, int max_pages);
size_t attention_ws_bytes(int B, int k, int Hq, int Hkv, int D, int max_pages, bool bf16);
hipError_t launch_attention(bool bf16, const AttnArgs& a, void* ws, hipStream_t st);

// ------------------------------------------------------------- dense GEMM
// out[M, N] = A[M, K] . B[N, K]^T (+ bias[N]) (+ resid[M, N], added to the
// product rounded to storage); bf16 needs N % 128 == 0 and K % 128 == 0.
size_t dense_gemm_ws_bytes(int64_t M, int64_t N, int64_t K, bool bf16);
hipError_t launch_dense_gemm(bool bf16, int M, int N, int K, const void* A, const void* B,
                             const void* bias, const void* resid, void* out, void* ws,
                             hipStream_t st);
// Whether that product splits its contraction (fp32 partials in ws, then a
// reduction pass).
bool dense_gemm_splits(int M, int N, int K, bool bf16);
// The drafter's gate/up product [M, 2I] (gate columns first) when it splits:
// its reduction writes h[M, I] = silu(gate) * up directly, element-wise as the
// stored product followed by the SiLU kernel would.  Only for split shapes.
hipError_t launch_dense_gemm_silu(bool bf16, int M, int I, int K, const void* A, const void* B, void* h,
                                  void* ws, hipStream_t st);

// ------------------------------------------------------------ drafter layer
struct DraftArgs {
  int B, k, d, Hq, Hkv, D, I;
  bool bf16;
  void* x;                       // [B*k, d] residual stream, updated in place
  const void* ln1;               // [d]
  const void* w_qkv;             // [(Hq + 2 Hkv) D, d]
  const void* q_norm;            // [D] or null
  const void* k_norm;            // [D] or null
  const void* w_o;               // [d, Hq D]
  const void* ln2;               // [d]
  const void* w_gate_up;         // [2 I, d]: gate rows, then up rows
  const void* w_down;            // [d, I]
  float eps, rope_theta;         // rope_theta 0: no rotary embedding
  const void* cache_k;           // this layer's injected context [num_pages, Hkv, 16, D]
  const void* cache_v;
  int num_pages;
  const int32_t* block_table;    // [B, max_pages]
  int max_pages;
  const int32_t* ctx_lens;       // [B]
  bool causal;
};
size_t draft_layer_ws_bytes(const DraftArgs& a);
hipError_t launch_draft_layer(const DraftArgs& a, void* ws, hipStream_t st);
size_t draft_head_ws_bytes(int M, int d, int V, bool bf16);
hipError_t launch_draft_head(bool bf16, int M, int d, int V, const void* x, const void* norm_w,
                             const void* lm_head, float eps, void* logits, void* ws, hipStream_t st);
hipError_t launch_embed(bool bf16, int M, int d, int V, const void* table, const int32_t* tokens,
                        void* out, hipStream_t st);

// ----------------------------------------------------------- materialisation
struct MatArgs {
  int64_t T;
  int m, d;
  const void* hiddens[8];
  const void* W_f;
  const void* b_f;
  int n_layers, Hkv, D;
  const void* W_K[64];
  const void* W_V[64];
  void* cache_k[64];
  void* cache_v[64];
  int num_pages[64];
  const int32_t* block_table;
  int max_pages;
  int rows_per_seq;
  const int32_t* seq_start;
  const int32_t* commit_lens;
  void* h_out;
  // K epilogue (per-head RMSNorm, then the rotary embedding); off when both
  // k_norm_on and rope_theta are zero
  bool k_norm_on;
  const void* k_norm_w[64];
  float k_norm_eps;
  float rope_theta;
};
constexpr int kMaxLayers = 64;
size_t materialize_ws_bytes(int64_t T, int m, int d, int n_layers, int Hkv, int D, bool bf16);
hipError_t launch_materialize(bool bf16, const MatArgs& a, void* ws, size_t ws_bytes,
                              hipStream_t st);

}  // namespace dflash
