// DDTree: the draft tree of [Spec tutorial], section 6.
//
// 6.1 / 6.3: every block position offers its top-K candidates; a path's
// joint probability is the product of the per-position marginals; the tree
// is grown best first under a node budget (pop the most probable leaf, push
// its children).  6.4: each node sees only its ancestors (the ancestor-only
// mask of the target's parallel verification).
//
// Design.
//  * Top-K: one coalesced pass over every draft row, workgroups on row
//    chunks as in the verify passes.  Each thread keeps a sorted list of its
//    16 best (logit, token) pairs -- compared by raw logit, ties to the lower
//    token id, so the selection is exact -- and the chunk's softmax partial
//    (m, sum 2^(z - m)); the lists merge into the chunk's top-K by K rounds
//    of a workgroup argmax.  A second kernel merges the chunk lists and
//    partials of a row into its top-K tokens and natural log-probabilities.
//  * Tree: one wavefront per request runs the best-first loop.  Candidates
//    live in LDS; each lane caches the best of the slots it owns (slot s
//    belongs to lane s % 64), so a pop is a 6-step shuffle argmax plus a
//    rescan by the owner lane.  A pop pushes at most two candidates, the
//    popped node's first child and its next sibling: siblings come sorted,
//    so a sibling can never outrank the one before it and this pops exactly
//    what pushing all K children would.  Order: higher joint log-probability
//    first, then the parent's pop index, then the sibling rank.
#include <climits>

#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kTopkMax = 16;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// (v, i) before (w, j): larger value, then lower index
__device__ __forceinline__ bool before(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

// Insert (v, x) into a thread's sorted list of kTopkMax entries (best first).
__device__ __forceinline__ void list_insert(float (&lv)[kTopkMax], int (&li)[kTopkMax], float v, int x) {
  if (!before(v, x, lv[kTopkMax - 1], li[kTopkMax - 1])) return;
  float cv = v;
  int ci = x;
#pragma unroll
  for (int j = 0; j < kTopkMax; ++j) {
    if (before(cv, ci, lv[j], li[j])) {
      const float tv = lv[j];
      const int ti = li[j];
      lv[j] = cv; li[j] = ci;
      cv = tv; ci = ti;
    }
  }
}

// Workgroup argmax of (v, i) under before(); every thread gets the result.
__device__ __forceinline__ void block_best(float v, int i, float* sv, int* si, float& bv, int& bi) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(i, o, 64);
    if (before(ov, oi, v, i)) { v = ov; i = oi; }
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  bv = sv[0];
  bi = si[0];
  for (int k = 1; k < kThreads / 64; ++k)
    if (before(sv[k], si[k], bv, bi)) { bv = sv[k]; bi = si[k]; }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_row_topk(const T* __restrict__ dl, int64_t rs, int V,
                                                       int K, float a, int chunk, int nc,
                                                       float* __restrict__ cv, int* __restrict__ ci,
                                                       float2* __restrict__ part) {
  const int c = blockIdx.x % nc;
  const int r = blockIdx.x / nc;
  const T* row = dl + (int64_t)r * rs;
  const int x0 = c * chunk;
  const int x1 = min(V, x0 + chunk);
  float lv[kTopkMax];
  int li[kTopkMax];
#pragma unroll
  for (int j = 0; j < kTopkMax; ++j) { lv[j] = neg_inf(); li[j] = INT_MAX; }
  float m = neg_inf(), s = 0.f;
  auto take = [&](float v, int x) {
    const float z = v * a;
    if (z > m) { s *= exp2f(m - z); m = z; }
    if (m != neg_inf()) s += exp2f(z - m);
    list_insert(lv, li, v, x);
  };
  if (VEC) {
    const int nvec = (x1 - x0) >> 3;
    for (int v = threadIdx.x; v < nvec; v += kThreads) {
      float e[8];
      load8(row + x0 + v * 8, e);
#pragma unroll
      for (int j = 0; j < 8; ++j) take(e[j], x0 + v * 8 + j);
    }
    for (int x = x0 + nvec * 8 + threadIdx.x; x < x1; x += kThreads) take(load1(row + x), x);
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kThreads) take(load1(row + x), x);
  }
  // softmax partial of the chunk
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const float os = __shfl_xor(s, o, 64);
    lse2_merge(m, s, om, os);
  }
  __shared__ float sm[kThreads / 64], ss[kThreads / 64];
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  if ((threadIdx.x & 63) == 0) { sm[threadIdx.x >> 6] = m; ss[threadIdx.x >> 6] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = sm[0], s2 = ss[0];
    for (int k = 1; k < kThreads / 64; ++k) lse2_merge(mm, s2, sm[k], ss[k]);
    part[blockIdx.x] = make_float2(mm, s2);
  }
  // the chunk's top-K: K rounds, each taking the best list head
  int head = 0;
  for (int k = 0; k < K; ++k) {
    float hv = neg_inf();
    int hi = INT_MAX;
#pragma unroll
    for (int j = 0; j < kTopkMax; ++j)
      if (j == head) { hv = lv[j]; hi = li[j]; }
    float bv;
    int bi;
    block_best(hv, hi, sv, si, bv, bi);
    if (bi == hi && bv == hv && hi != INT_MAX) ++head;   // tokens are distinct: one owner
    if (threadIdx.x == 0) {
      cv[(int64_t)blockIdx.x * K + k] = bv;
      ci[(int64_t)blockIdx.x * K + k] = bi;
    }
  }
}

// Per row: merge the nc chunk lists (each sorted) into the row's top-K and
// turn them into natural log-probabilities.  One wavefront per row, lane c
// owning chunk c (nc <= 64).
__global__ __launch_bounds__(64) void k_topk_finalize(int K, int nc, float a,
                                                      const float* __restrict__ cv,
                                                      const int* __restrict__ ci,
                                                      const float2* __restrict__ part,
                                                      int32_t* __restrict__ tok_out,
                                                      float* __restrict__ lp_out) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x;
  const float2 pc = lane < nc ? part[(int64_t)r * nc + lane] : make_float2(neg_inf(), 0.f);
  const float M = wave_max(pc.x);
  const float S = wave_sum((M == neg_inf() || pc.x == neg_inf()) ? 0.f : pc.y * exp2f(pc.x - M));
  const float lse2 = M + log2f(S);
  int head = 0;
  for (int k = 0; k < K; ++k) {
    float v = neg_inf();
    int i = INT_MAX;
    if (lane < nc && head < K) {
      v = cv[((int64_t)r * nc + lane) * K + head];
      i = ci[((int64_t)r * nc + lane) * K + head];
    }
    float bv = v;
    int bi = i;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (before(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (bi == i && bv == v && i != INT_MAX) ++head;
    if (lane == 0) {
      tok_out[(int64_t)r * K + k] = bi == INT_MAX ? -1 : bi;
      lp_out[(int64_t)r * K + k] = bi == INT_MAX ? neg_inf() : (bv * a - lse2) * kLn2;
    }
  }
}

// Best-first tree of one request per wavefront.
struct TreeP {
  int n_pos, K, budget, W;         // W: 32-bit words per ancestor-mask row
  const int32_t* tok;              // [B, n_pos, K]
  const float* lp;                 // [B, n_pos, K]
  int32_t* node_token;             // [B, budget]
  int32_t* node_parent;
  int32_t* node_depth;
  float* node_logp;
  int32_t* n_nodes;                // [B]
  uint32_t* mask;                  // [B, budget, W] or null
};

__global__ __launch_bounds__(64) void k_tree_build(TreeP p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int NK = p.n_pos * p.K;
  const int cap = 2 * p.budget + 2;                        // candidates ever appended
  float* e_score = reinterpret_cast<float*>(smem);         // [cap]
  float* e_pscore = e_score + cap;                         // [cap] parent's score
  int* e_par = reinterpret_cast<int*>(e_pscore + cap);     // [cap] parent pop index (-1: root)
  int* e_rd = e_par + cap;                                 // [cap] rank | depth << 8
  float* s_lp = reinterpret_cast<float*>(e_rd + cap);      // [n_pos * K]
  int* s_tok = reinterpret_cast<int*>(s_lp + NK);          // [n_pos * K]
  int* s_par = s_tok + NK;                                 // [budget] node parents
  for (int x = lane; x < NK; x += 64) {
    s_lp[x] = p.lp[(int64_t)b * NK + x];
    s_tok[x] = p.tok[(int64_t)b * NK + x];
  }
  __syncthreads();
  const int K = p.K;
  // candidate key: (score, (parent + 1) * K + rank), larger score first, then smaller key
  auto key2 = [&](int e) { return (e_par[e] + 1) * K + (e_rd[e] & 0xff); };
  // each lane caches the best of its own slots; an empty lane is (-inf, INT_MAX)
  float best_s = neg_inf();
  int best_k = INT_MAX, best_e = -1;
  int n_ent = 0;
  auto append = [&](float sc, float psc, int par, int rank, int depth) {
    if (sc == neg_inf()) return;                  // a token of probability 0 is no candidate
    const int e = n_ent++;                        // uniform: every lane counts
    if ((e & 63) == lane) {
      e_score[e] = sc; e_pscore[e] = psc; e_par[e] = par; e_rd[e] = rank | (depth << 8);
      const int k = (par + 1) * K + rank;
      if (before(sc, k, best_s, best_k)) { best_s = sc; best_k = k; best_e = e; }
    }
  };
  // the root's first child
  append(s_lp[0], 0.f, -1, 0, 1);
  int i = 0;
  for (; i < p.budget; ++i) {
    // wavefront argmax over the lanes' cached bests
    float v = best_s;
    int k = best_k, e = best_e;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int ok = __shfl_xor(k, o, 64);
      const int oe = __shfl_xor(e, o, 64);
      if (before(ov, ok, v, k)) { v = ov; k = ok; e = oe; }   // keys are unique: a strict order
    }
    if (e < 0) break;                              // no candidate left: a full tree
    __syncthreads();
    const float sc = e_score[e], psc = e_pscore[e];
    const int par = e_par[e], rd = e_rd[e];
    const int rank = rd & 0xff, depth = rd >> 8;
    if (lane == 0) {
      const int slot = (depth - 1) * K + rank;
      const int64_t o = (int64_t)b * p.budget + i;
      p.node_token[o] = s_tok[slot];
      p.node_parent[o] = par;
      p.node_depth[o] = depth;
      p.node_logp[o] = sc;
      s_par[i] = par;
    }
    if ((e & 63) == lane) {                        // the owner drops it and rescans its slots
      e_score[e] = neg_inf();
      best_s = neg_inf(); best_k = INT_MAX; best_e = -1;
      for (int x = lane; x < n_ent; x += 64) {
        const float xs = e_score[x];
        if (xs == neg_inf()) continue;
        const int xk = key2(x);
        if (before(xs, xk, best_s, best_k)) { best_s = xs; best_k = xk; best_e = x; }
      }
    }
    if (depth < p.n_pos) append(sc + s_lp[depth * K], sc, i, 0, depth + 1);          // first child
    if (rank + 1 < K) append(psc + s_lp[(depth - 1) * K + rank + 1], psc, par, rank + 1, depth);   // next sibling
    __syncthreads();
  }
  if (lane == 0) p.n_nodes[b] = i;
  for (int x = i + lane; x < p.budget; x += 64) {  // unused node slots
    const int64_t o = (int64_t)b * p.budget + x;
    p.node_token[o] = -1; p.node_parent[o] = -2; p.node_depth[o] = 0; p.node_logp[o] = neg_inf();
  }
  __syncthreads();
  if (p.mask) {
    // node x sees itself and its ancestors; unused rows are all zero
    for (int x = lane; x < p.budget; x += 64) {
      uint32_t* row = p.mask + ((int64_t)b * p.budget + x) * p.W;
      for (int wd = 0; wd < p.W; ++wd) row[wd] = 0u;
      if (x < i) {
        for (int y = x; y >= 0; y = s_par[y]) row[y >> 5] |= 1u << (y & 31);
      }
    }
  }
}

struct TopkPlan {
  VocabPlan pl;
  size_t cand_v, cand_i, part;   // byte offsets in the workspace
  size_t total;
};

TopkPlan topk_plan(int64_t rows, int V, int K) {
  TopkPlan t;
  t.pl = plan_vocab(rows, V);
  const int64_t n = rows * t.pl.n_chunks;
  t.cand_v = 0;
  t.cand_i = align256(sizeof(float) * n * K);
  t.part = t.cand_i + align256(sizeof(int) * n * K);
  t.total = t.part + align256(sizeof(float2) * n);
  return t;
}

size_t tree_lds_bytes(int n_pos, int K, int budget) {
  const size_t cap = 2 * (size_t)budget + 2;
  return cap * 16 + (size_t)n_pos * K * 8 + (size_t)budget * 4;
}

}  // namespace

size_t tree_ws_bytes(int B, int n_pos, int V, int K) {
  return topk_plan((int64_t)B * n_pos, V, K).total;
}

size_t tree_build_lds_bytes(int n_pos, int K, int budget) { return tree_lds_bytes(n_pos, K, budget); }

hipError_t launch_tree_build(bool bf16, int B, int n_pos, int V, const void* dl, int64_t rs,
                             float temperature, int K, int budget, int32_t* topk_tok,
                             float* topk_lp, int32_t* node_token, int32_t* node_parent,
                             int32_t* node_depth, float* node_logp, int32_t* n_nodes,
                             uint32_t* mask, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)B * n_pos;
  const TopkPlan t = topk_plan(rows, V, K);
  char* w = static_cast<char*>(ws);
  float* cv = reinterpret_cast<float*>(w + t.cand_v);
  int* ci = reinterpret_cast<int*>(w + t.cand_i);
  float2* part = reinterpret_cast<float2*>(w + t.part);
  const float a = kLog2e / temperature;
  const int es = bf16 ? 2 : 4;
  const bool vec = (reinterpret_cast<uintptr_t>(dl) % 16 == 0) && ((rs * es) % 16 == 0);
  const dim3 g1((unsigned)(rows * t.pl.n_chunks));
  if (bf16) {
    if (vec) hipLaunchKernelGGL((k_row_topk<uint16_t, true>), g1, dim3(kThreads), 0, st, static_cast<const uint16_t*>(dl), rs, V, K, a, t.pl.chunk, t.pl.n_chunks, cv, ci, part);
    else hipLaunchKernelGGL((k_row_topk<uint16_t, false>), g1, dim3(kThreads), 0, st, static_cast<const uint16_t*>(dl), rs, V, K, a, t.pl.chunk, t.pl.n_chunks, cv, ci, part);
  } else {
    if (vec) hipLaunchKernelGGL((k_row_topk<float, true>), g1, dim3(kThreads), 0, st, static_cast<const float*>(dl), rs, V, K, a, t.pl.chunk, t.pl.n_chunks, cv, ci, part);
    else hipLaunchKernelGGL((k_row_topk<float, false>), g1, dim3(kThreads), 0, st, static_cast<const float*>(dl), rs, V, K, a, t.pl.chunk, t.pl.n_chunks, cv, ci, part);
  }
  hipLaunchKernelGGL(k_topk_finalize, dim3((unsigned)rows), dim3(64), 0, st, K, t.pl.n_chunks, a, cv,
                     ci, part, topk_tok, topk_lp);
  TreeP p{n_pos, K, budget, (budget + 31) / 32, topk_tok, topk_lp, node_token, node_parent,
          node_depth, node_logp, n_nodes, mask};
  hipLaunchKernelGGL(k_tree_build, dim3(B), dim3(64), tree_lds_bytes(n_pos, K, budget), st, p);
  return hipGetLastError();
}

}  // namespace dflash
