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
//    chunks as in the verify passes.  Selection is on the raw logits, ties
//    to the lower token id, so it is exact; each wavefront filters against
//    a threshold (its K-th best so far) and buffers the few elements that
//    beat it, so the pass costs little more than the chunk's softmax
//    partial (m, sum 2^(z - m)) it computes alongside.  A second kernel
//    merges the chunk lists and partials of a row into its top-K tokens
//    and natural log-probabilities.
//  * Tree: one wavefront per request runs the best-first loop.  Candidates
//    live in LDS as 64-bit words whose unsigned order is the pop order;
//    each lane caches the best of the slots it owns (slot s belongs to lane
//    s % 64), so a pop is a DPP wavefront max plus a rescan by the owner
//    lane.  A pop pushes at most two candidates, the popped node's first
//    child and its next sibling: siblings come sorted, so a sibling can
//    never outrank the one before it and this pops exactly what pushing all
//    K children would; the first child takes over the popped slot, so a
//    request uses at most budget + 1 slots.  Order: higher joint
//    log-probability first, then the parent's pop index, then the sibling
//    rank.  The loop stages only the popped words in LDS and touches no
//    global memory; the node outputs are decoded from them at the end.
#include <algorithm>
#include <climits>

#include "common.h"
#include "launch.h"

// 1: the tree is built by the parallel kernel (the serial loop as its
// fallback); 0: by the serial loop, one wavefront per request
#ifndef DFLASH_TREE_PARALLEL
#define DFLASH_TREE_PARALLEL 1
#endif

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

// LDS ordering inside one wavefront: the wave's LDS operations complete in
// issue order, so a fence at wavefront scope (it keeps the compiler from
// moving LDS accesses across it) is all the exchange between lanes needs.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- wave reductions
// Within a row of 16 lanes the butterfly runs on DPP lane permutations (quad
// xor 1 and xor 2, then the half-row and row mirrors), after which every lane
// of a row holds the row's best; the four row bests are then read into scalar
// registers and combined there, so the result is uniform.
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(x, x, CTRL, 0xf, 0xf, false);
}
constexpr int kQuadXor1 = 0xb1, kQuadXor2 = 0x4e, kHalfMirror = 0x141, kMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ void best_step(float& v, int& i) {
  const float ov = __int_as_float(dpp<CTRL>(__float_as_int(v)));
  const int oi = dpp<CTRL>(i);
  if (before(ov, oi, v, i)) { v = ov; i = oi; }
}

// (v, i) best under before() over the wavefront, uniform in every lane.
__device__ __forceinline__ void wave_best(float& v, int& i) {
  best_step<kQuadXor1>(v, i);
  best_step<kQuadXor2>(v, i);
  best_step<kHalfMirror>(v, i);
  best_step<kMirror>(v, i);
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), r));
    const int ri = __builtin_amdgcn_readlane(i, r);
    if (before(rv, ri, bv, bi)) { bv = rv; bi = ri; }
  }
  v = bv;
  i = bi;
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int lanes_below(uint64_t b) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0));
}

#ifndef DFLASH_TOPK_NF
#define DFLASH_TOPK_NF 4
#endif
#ifndef DFLASH_TOPK_PREFETCH
#define DFLASH_TOPK_PREFETCH 1   // top-K pass: next round's loads issued before this round's arithmetic
#endif
#ifndef DFLASH_TOPK_WGS
#define DFLASH_TOPK_WGS 768
#endif
constexpr int kTopkNF = DFLASH_TOPK_NF;   // 16-byte loads in flight per lane
constexpr int kVecBuf = 128;       // buffered vectors of 8 per wavefront

// One workgroup per (row, chunk), four wavefronts, each with its own
// candidates.  A wavefront holds its K best so far in lanes 0..K-1 and a
// threshold, the K-th of them: an element not before the threshold has K
// better ones already, so dropping it is exact.  A lane whose vector of 8
// reaches the threshold appends the whole vector to an LDS buffer (one
// ballot for the wavefront); the buffer is folded into the K best, and the
// threshold raised, when it fills and at the end.  The first round seeds
// the threshold with the K-th largest lane maximum (K lanes hold an element
// at least that large).  A vector below the threshold costs one comparison,
// so the pass is the streaming log-sum-exp plus that test.
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_row_topk(const T* __restrict__ dl, int64_t rs, int V,
                                                       int K, float a, int chunk, int nc,
                                                       float* __restrict__ cv, int* __restrict__ ci,
                                                       float2* __restrict__ part) {
  __shared__ float4 vb_v[kThreads / 64][kVecBuf][2];
  __shared__ int vb_x[kThreads / 64][kVecBuf];     // token of element 0; -1 - token: a single element
  __shared__ float sm[kThreads / 64], ss[kThreads / 64];
  __shared__ float wv[kThreads / 64][kTopkMax];
  __shared__ int wi[kThreads / 64][kTopkMax];
  const int c = blockIdx.x % nc;
  const int r = blockIdx.x / nc;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const T* row = dl + (int64_t)r * rs;
  const int x0 = c * chunk;
  const int x1 = min(V, x0 + chunk);
  int cnt = 0;                                      // buffered vectors (uniform)
  float tv = neg_inf();
  int ti = INT_MAX;                                 // threshold (uniform): nothing dropped yet
  float kv = neg_inf();
  int kx = INT_MAX;                                 // lane k < K: the k-th best so far
  float m = neg_inf(), s = 0.f;

  // fold the buffer into the K best: up to 64 vectors at a time, one per
  // lane, K rounds of wave_best over each lane's best remaining entry (its
  // vector's elements and, in lanes < K, the current k-th best)
  auto fold = [&]() {
    wave_sync();
    while (cnt > 0) {
      const int n = min(cnt, 64);
      float e[8];
      int ex[8];
      const int slot = cnt - n + lane;
      const bool have = lane < n;
      const float4 a0 = vb_v[w][have ? slot : 0][0], a1 = vb_v[w][have ? slot : 0][1];
      const int xb = vb_x[w][have ? slot : 0];
      e[0] = a0.x; e[1] = a0.y; e[2] = a0.z; e[3] = a0.w;
      e[4] = a1.x; e[5] = a1.y; e[6] = a1.z; e[7] = a1.w;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const bool live = have && (xb >= 0 || j == 0);
        ex[j] = live ? (xb >= 0 ? xb + j : -1 - xb) : INT_MAX;
        if (!live) e[j] = neg_inf();
      }
      cnt -= n;
      float nv = neg_inf();
      int ni = INT_MAX;
      for (int k = 0; k < K; ++k) {
        float lb = kv;
        int lx = kx, which = 8;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (before(e[j], ex[j], lb, lx)) { lb = e[j]; lx = ex[j]; which = j; }
        float b1 = lb;
        int b2 = lx;
        wave_best(b1, b2);
        if (b2 == lx && b1 == lb && lx != INT_MAX) {   // this lane holds the winner: retire it
          if (which == 8) { kv = neg_inf(); kx = INT_MAX; }
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j == which) { e[j] = neg_inf(); ex[j] = INT_MAX; }
        }
        if (lane == k) { nv = b1; ni = b2; }
      }
      kv = nv; kx = ni;
    }
    tv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kv), K - 1));
    ti = __builtin_amdgcn_readlane(kx, K - 1);
    wave_sync();
  };
  // buffer the lanes' vectors (x: token of e[0]) that may beat the threshold
  auto push8 = [&](const float (&e)[8], float m8, int x, bool valid) {
    const bool maybe = valid && !(m8 < tv);
    const uint64_t bal = __ballot(maybe);
    if (bal == 0) return;
    if (maybe) {
      const int o = cnt + lanes_below(bal);
      vb_v[w][o][0] = make_float4(e[0], e[1], e[2], e[3]);
      vb_v[w][o][1] = make_float4(e[4], e[5], e[6], e[7]);
      vb_x[w][o] = x;
    }
    cnt += __popcll(bal);
    if (cnt > kVecBuf - 64) fold();
  };
  auto push1 = [&](float e, int x, bool valid) {
    const bool maybe = valid && before(e, x, tv, ti);
    const uint64_t bal = __ballot(maybe);
    if (bal == 0) return;
    if (maybe) {
      const int o = cnt + lanes_below(bal);
      vb_v[w][o][0] = make_float4(e, neg_inf(), neg_inf(), neg_inf());
      vb_v[w][o][1] = make_float4(neg_inf(), neg_inf(), neg_inf(), neg_inf());
      vb_x[w][o] = -1 - x;
    }
    cnt += __popcll(bal);
    if (cnt > kVecBuf - 64) fold();
  };
  // threshold from the first round: the K-th largest lane maximum, ties admitted
  auto seed = [&](float lane_max) {
    float ev = lane_max;
    int ei = lane;
    float b1 = neg_inf();
    for (int k = 0; k < K; ++k) {
      b1 = ev;
      int b2 = ei;
      wave_best(b1, b2);
      if (b2 == lane) { ev = neg_inf(); ei = INT_MAX; }
    }
    tv = b1;
    ti = INT_MAX;
  };
  auto lse1 = [&](float v) {
    const float z = v * a;
    if (z > m) { s *= fexp2(m - z); m = z; }
    if (m != neg_inf()) s += fexp2(z - m);
  };
  if (VEC) {
    const int nvec = (x1 - x0) >> 3;
    constexpr int kStep = kTopkNF * kThreads;
    constexpr int NW = sizeof(T) / 2;   // 16-byte pieces per vector of 8
    // The loads of round base + kStep go out before round base is
    // converted and tested, so they land while this one computes.  They go
    // out unconditionally (past the end they re-read the last vector) so
    // that the registers they fill are never a merge of old and new values,
    // which would make the compiler wait for them at the top of the loop.
    uint4 nx[kTopkNF][NW];
    auto fetch = [&](int base) {
#pragma unroll
      for (int u = 0; u < kTopkNF; ++u) {
        const int v = min(base + lane + u * kThreads, nvec - 1);
        const uint4* q = reinterpret_cast<const uint4*>(row + x0 + (int64_t)v * 8);
#pragma unroll
        for (int i = 0; i < NW; ++i) nx[u][i] = ld_stream16(q + i);
      }
    };
    bool first = true;
    int base = w * 64;
    if (base < nvec) fetch(base);
    for (; base < nvec; base += kStep) {   // uniform per wavefront
      uint4 cur[kTopkNF][NW];
#pragma unroll
      for (int u = 0; u < kTopkNF; ++u)
#pragma unroll
        for (int i = 0; i < NW; ++i) cur[u][i] = nx[u][i];
      if (DFLASH_TOPK_PREFETCH) fetch(base + kStep);
      float e[kTopkNF][8], mx[kTopkNF];
      bool ok[kTopkNF];
#pragma unroll
      for (int u = 0; u < kTopkNF; ++u) {
        ok[u] = base + lane + u * kThreads < nvec;
        if constexpr (NW == 1) {
          const uint4 q = cur[u][0];
          e[u][0] = bf16_lo(q.x); e[u][1] = bf16_hi(q.x);
          e[u][2] = bf16_lo(q.y); e[u][3] = bf16_hi(q.y);
          e[u][4] = bf16_lo(q.z); e[u][5] = bf16_hi(q.z);
          e[u][6] = bf16_lo(q.w); e[u][7] = bf16_hi(q.w);
        } else {
          e[u][0] = __uint_as_float(cur[u][0].x); e[u][1] = __uint_as_float(cur[u][0].y);
          e[u][2] = __uint_as_float(cur[u][0].z); e[u][3] = __uint_as_float(cur[u][0].w);
          e[u][4] = __uint_as_float(cur[u][1].x); e[u][5] = __uint_as_float(cur[u][1].y);
          e[u][6] = __uint_as_float(cur[u][1].z); e[u][7] = __uint_as_float(cur[u][1].w);
        }
      }
      float lm = neg_inf();
#pragma unroll
      for (int u = 0; u < kTopkNF; ++u) {
        float m8 = e[u][0];
#pragma unroll
        for (int j = 1; j < 8; ++j) m8 = fmaxf(m8, e[u][j]);
        mx[u] = m8;
        if (ok[u]) {
          const float gm = m8 * a;
          if (gm > m) { s *= fexp2(m - gm); m = gm; }
          if (m != neg_inf()) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += fexp2(fmaf(e[u][j], a, -m));
            s += acc;
          }
          lm = fmaxf(lm, m8);
        }
      }
      if (first) { seed(lm); first = false; }
#pragma unroll
      for (int u = 0; u < kTopkNF; ++u) push8(e[u], mx[u], x0 + (base + lane + u * kThreads) * 8, ok[u]);
      if (!DFLASH_TOPK_PREFETCH) fetch(base + kStep);
    }
    // the ragged tail (fewer than 8 elements), one per lane of the first wavefront
    if (w == 0) {
      const int x = x0 + nvec * 8 + lane;
      const bool ok = x < x1;
      const float v = ok ? load1(row + x) : neg_inf();
      if (ok) lse1(v);
      push1(v, x, ok);
    }
  } else {
    for (int base = x0 + w * 64; base < x1; base += kThreads) {
      const int x = base + lane;
      const bool ok = x < x1;
      const float v = ok ? load1(row + x) : neg_inf();
      if (ok) lse1(v);
      push1(v, x, ok);
    }
  }
  fold();
  // softmax partial of the chunk
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const float os = __shfl_xor(s, o, 64);
    lse2_merge(m, s, om, os);
  }
  if (lane == 0) { sm[w] = m; ss[w] = s; }
  if (lane < K) { wv[w][lane] = kv; wi[w][lane] = kx; }
  __syncthreads();
  if (w == 0) {
    if (lane == 0) {
      float mm = sm[0], s2 = ss[0];
      for (int k = 1; k < kThreads / 64; ++k) lse2_merge(mm, s2, sm[k], ss[k]);
      part[blockIdx.x] = make_float2(mm, s2);
    }
    // the chunk's K best out of the wavefronts' lists: one entry per lane
    float ev = neg_inf();
    int ei = INT_MAX;
    if (lane < (kThreads / 64) * K) { ev = wv[lane / K][lane % K]; ei = wi[lane / K][lane % K]; }
    for (int k = 0; k < K; ++k) {
      float b1 = ev;
      int b2 = ei;
      wave_best(b1, b2);
      if (b2 == ei && b1 == ev && ei != INT_MAX) { ev = neg_inf(); ei = INT_MAX; }
      if (lane == 0) {
        cv[(int64_t)blockIdx.x * K + k] = b1;
        ci[(int64_t)blockIdx.x * K + k] = b2;
      }
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
    wave_best(bv, bi);
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

// Candidate slots of a request: a pop's first child takes over the popped
// slot and its next sibling a new one, so at most budget + 1 slots are ever
// used; rounded up to whole rounds of 8 slots per lane for the rescan.
__host__ __device__ constexpr int tree_cap(int budget) { return (budget + 1 + 511) / 512 * 512; }

// A candidate is one 64-bit word whose unsigned order is the pop order:
// bits 63..32 the joint log-probability mapped to an order-preserving
// unsigned integer, bits 30..16 (32767 - key) with key = (parent + 1) * 16 +
// rank (smaller key first: the parent popped earlier, then the lower rank;
// rank < K <= 16), bits 6..0 the depth.  Keys are unique, so the depth never
// decides; 0 is below every candidate and marks an empty slot.
__device__ __forceinline__ uint32_t ord_of(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ uint64_t cand(float sc, int key, int depth) {
  return ((uint64_t)ord_of(sc) << 32) | ((uint32_t)(32767 - key) << 16) | (uint32_t)depth;
}

template <int CTRL>
__device__ __forceinline__ uint32_t umax_step(uint32_t x) {
  return max(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xf, 0xf, true));
}

// Largest 32-bit value over the wavefront, uniform (scalar registers).
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = umax_step<kQuadXor1>(x);
  x = umax_step<kQuadXor2>(x);
  x = umax_step<kHalfMirror>(x);
  x = umax_step<kMirror>(x);
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Largest 64-bit value over the wavefront, uniform: the high words first,
// then the low words of the lanes that hold the largest high word.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32);
  const uint32_t H = wave_umax(hi);
  const uint32_t L = wave_umax(hi == H ? (uint32_t)v : 0u);
  return ((uint64_t)H << 32) | L;
}

// The best-first loop of one request by one wavefront (lane = its lane): the
// serial form, used by the parallel build when a request's candidates exceed
// its buffers.  Only wavefront-level synchronisation inside.
__device__ void tree_build_serial(const TreeP& p, unsigned char* smem, int b, int lane) {
  const int K = p.K, NK = p.n_pos * p.K, N = p.budget;
  const int cap = tree_cap(N);
  uint64_t* e_c = reinterpret_cast<uint64_t*>(smem);       // [cap] candidate slots
  uint64_t* n_c = e_c + cap;                               // [budget] the popped words, in order
  float* s_lp = reinterpret_cast<float*>(n_c + N);         // [n_pos * K]
  int* s_tok = reinterpret_cast<int*>(s_lp + NK);          // [n_pos * K]
  int* n_par = s_tok + NK;                                 // [budget] parents, decoded at the end
  for (int x = lane; x < NK; x += 64) {
    s_lp[x] = p.lp[(int64_t)b * NK + x];
    s_tok[x] = p.tok[(int64_t)b * NK + x];
  }
  for (int x = lane; x < cap; x += 64) e_c[x] = 0;
  wave_sync();
  // lane d holds block position d's best log-probability (a first child's term)
  const float lp_first = lane < p.n_pos ? s_lp[lane * K] : neg_inf();
  // each lane caches the best of the slots it owns (slot s: lane s % 64)
  uint64_t best = 0;
  int best_e = -1;
  int n_ent = 1;                                           // uniform: slots in use
  if (lane == 0 && s_lp[0] != neg_inf()) {                 // the root's first child, slot 0
    best = cand(s_lp[0], 0, 1);
    best_e = 0;
    e_c[0] = best;
  }
  int i = 0;
  for (; i < N; ++i) {
    const uint64_t top = wave_max_u64(best);               // uniform
    if (top == 0) break;                                   // no candidate left: a full tree
    const uint32_t thi = (uint32_t)(top >> 32), tlo = (uint32_t)top;
    const float sc = float_of(thi);
    const int key = 32767 - (int)((tlo >> 16) & 0x7fff);
    const int depth = (int)(tlo & 0x7f);
    const int par = (key >> 4) - 1, rank = key & 15;
    const int slot = (depth - 1) * K + rank;
    const uint64_t pword = n_c[max(par, 0)];
    const float lp_sib = s_lp[min(slot + 1, NK - 1)];
    const float lp_fc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lp_first), min(depth, 63)));
    if (lane == 0) n_c[i] = top;
    // the first child takes over the popped slot (an empty slot if none)
    uint64_t c1 = 0;
    if (depth < p.n_pos) {
      const float s1 = sc + lp_fc;
      if (s1 != neg_inf()) c1 = cand(s1, (i + 1) << 4, depth + 1);
    }
    if (best == top) {                                     // the owner refills its slot, rescans
      e_c[best_e] = c1;
      best = 0; best_e = -1;
      // slots past n_ent are zero (cleared at the start, capacity padded to
      // whole rounds of 8 per lane), so each round issues its 8 loads at once
      for (int x = lane; x < n_ent; x += 512) {
        uint64_t cc[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) cc[u] = e_c[x + 64 * u];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (cc[u] > best) { best = cc[u]; best_e = x + 64 * u; }
      }
    }
    // the next sibling takes a new slot
    if (rank + 1 < K) {
      const float psc = par < 0 ? 0.f : float_of((uint32_t)(pword >> 32));
      const float s2 = psc + lp_sib;
      if (s2 != neg_inf()) {
        const int e = n_ent++;
        if ((e & 63) == lane) {
          const uint64_t c2 = cand(s2, ((par + 1) << 4) + rank + 1, depth);
          e_c[e] = c2;
          if (c2 > best) { best = c2; best_e = e; }
        }
      }
    }
    wave_sync();
  }
  wave_sync();
  if (lane == 0) p.n_nodes[b] = i;
  for (int x = lane; x < N; x += 64) {
    const int64_t o = (int64_t)b * N + x;
    if (x < i) {
      const uint64_t c = n_c[x];
      const uint32_t lo = (uint32_t)c;
      const int key = 32767 - (int)((lo >> 16) & 0x7fff);
      const int depth = (int)(lo & 0x7f);
      const int par = (key >> 4) - 1;
      p.node_token[o] = s_tok[(depth - 1) * K + (key & 15)];
      p.node_parent[o] = par;
      p.node_depth[o] = depth;
      p.node_logp[o] = float_of((uint32_t)(c >> 32));
      n_par[x] = par;
    } else {
      p.node_token[o] = -1; p.node_parent[o] = -2; p.node_depth[o] = 0; p.node_logp[o] = neg_inf();
    }
  }
  wave_sync();
  if (p.mask) {
    // row x: bits of x and of its ancestors.  The ancestors come in falling
    // index order, so the row is written word by word from the top, each
    // word once; unused rows are all zero.
    for (int x = lane; x < N; x += 64) {
      uint32_t* row = p.mask + ((int64_t)b * N + x) * p.W;
      int w = p.W - 1;
      if (x < i) {
        const int top_w = x >> 5;
        for (; w > top_w; --w) row[w] = 0u;
        uint32_t acc = 0u;
        for (int y = x; y >= 0; y = n_par[y]) {
          const int yw = y >> 5;
          while (w > yw) { row[w] = acc; acc = 0u; --w; }
          acc |= 1u << (y & 31);
        }
        row[w] = acc;
        --w;
      }
      for (; w >= 0; --w) row[w] = 0u;
    }
  }
}

__global__ __launch_bounds__(64) void k_tree_build(TreeP p) {
  extern __shared__ __align__(16) unsigned char smem[];
  tree_build_serial(p, smem, blockIdx.x, threadIdx.x);
}

// ------------------------------------------------------------ parallel build
// The serial loop pops in the order "higher score first; equal scores by the
// parents' pop order, then by sibling rank".  That order is a fixed total
// order on all nodes in which a parent precedes its children (a child's score
// is its parent's plus a log-probability <= 0), so the tree is its first
// `budget` nodes.  The parallel build finds them without popping one at a
// time:
//  * grow: every frontier candidate is popped at once (a pop pushes its first
//    child and its next sibling, as in the serial loop) until at least
//    `budget` nodes are popped;
//  * finish: while a frontier candidate scores at least the budget-th best
//    popped score, such candidates are popped too.  Every node never pushed
//    is a descendant or a later sibling of a frontier candidate and so comes
//    after it; hence the popped set then holds the first `budget` nodes;
//  * order: the popped nodes scoring at least that score are sorted by the
//    total order (bitonic sort; on equal scores the comparison walks up to
//    the first pair of differing ancestors) and the first `budget` kept.
// A request whose buffers would overflow (huge groups of exactly equal
// scores) is built by the serial loop instead, by its first wavefront.
constexpr int kBT = 256;          // threads of the parallel build
constexpr int kBI = 17;           // frontier items per thread held in registers
constexpr int kSortE = 8;         // sort slots per thread held in registers (up to 2048 slots)

__host__ __device__ constexpr int par_cap(int budget) { return 4 * budget + 64; }
__host__ __device__ constexpr int pow2_at_least(int x) {
  int v = 1;
  while (v < x) v <<= 1;
  return v;
}

__device__ __forceinline__ uint32_t node_meta(int par, int rank, int depth) {
  return ((uint32_t)(par + 1) << 16) | ((uint32_t)rank << 8) | (uint32_t)depth;
}
__device__ __forceinline__ int meta_par(uint32_t m) { return (int)(m >> 16) - 1; }
__device__ __forceinline__ int meta_rank(uint32_t m) { return (int)((m >> 8) & 255u); }
__device__ __forceinline__ int meta_depth(uint32_t m) { return (int)(m & 255u); }

// exclusive prefix sum of v over the workgroup's 256 threads, and the total
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  uint32_t base = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kBT / 64; ++i) {
    const uint32_t t = sh[i];
    if (i < w) base += t;
    total += t;
  }
  __syncthreads();
  return base + x - v;
}

// Does popped node x come before popped node y in the pop order?
__device__ bool pop_before(int x, int y, const float* Ss, const uint32_t* Sm) {
  while (x != y) {
    const float sx = Ss[x], sy = Ss[y];
    if (sx != sy) return sx > sy;
    const int px = meta_par(Sm[x]), py = meta_par(Sm[y]);
    if (px == py) return meta_rank(Sm[x]) < meta_rank(Sm[y]);
    if (px < 0) return true;       // the root's children first
    if (py < 0) return false;
    x = px;
    y = py;
  }
  return false;
}

// Bitonic sort of MS slots (key descending, then index ascending) held in
// registers: a slot is one 64-bit word (key, 0xffff - index) sorted
// descending, thread t holds slots E t + e.  Exchanges inside a thread need
// nothing, inside a wavefront a shuffle, and only the strides that span
// wavefronts go through LDS (xch, MS words).  Every stride is a constant.
template <int MS>
__device__ __forceinline__ void sort_slots(uint32_t* okey, uint16_t* ord, uint64_t* xch) {
  constexpr int E = MS / kBT;
  static_assert(E >= 1 && E <= kSortE && E * kBT == MS, "slots per thread");
  const int tid = threadIdx.x;
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = E * tid + e;
    v[e] = ((uint64_t)okey[i] << 32) | (uint32_t)(0xffffu - ord[i]);
  }
#pragma unroll
  for (int size = 2; size <= MS; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e & stride) continue;
          const int ep = e | stride;
          const bool up = ((E * tid + e) & size) == 0;
          const bool swap = up ? v[e] < v[ep] : v[e] > v[ep];
          if (swap) { const uint64_t tmp = v[e]; v[e] = v[ep]; v[ep] = tmp; }
        }
      } else {
        const int ts = stride / E;             // partner thread: tid ^ ts
        if (ts >= 64) {
          __syncthreads();
#pragma unroll
          for (int e = 0; e < E; ++e) xch[E * tid + e] = v[e];
          __syncthreads();
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = E * tid + e;
          uint64_t o;
          if (ts >= 64) {
            o = xch[i ^ stride];
          } else {
            const uint32_t lo = __shfl_xor((uint32_t)v[e], ts, 64);
            const uint32_t hi = __shfl_xor((uint32_t)(v[e] >> 32), ts, 64);
            o = ((uint64_t)hi << 32) | lo;
          }
          const bool up = (i & size) == 0;
          const bool low = (i & stride) == 0;  // the pair's lower slot
          // descending when up: the lower slot keeps the larger word
          v[e] = (up == low) ? (v[e] > o ? v[e] : o) : (v[e] < o ? v[e] : o);
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    okey[E * tid + e] = (uint32_t)(v[e] >> 32);
    ord[E * tid + e] = (uint16_t)(0xffffu - (uint32_t)v[e]);
  }
  __syncthreads();
}

__global__ __launch_bounds__(kBT) void k_tree_build_par(TreeP p) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int K = p.K, NK = p.n_pos * K, N = p.budget;
  const int CS = par_cap(N), CF = CS + 1, M = pow2_at_least(CS);
  float* s_lp = reinterpret_cast<float*>(smem);                    // [NK]
  int* s_tok = reinterpret_cast<int*>(s_lp + NK);                  // [NK]
  float* Ss = reinterpret_cast<float*>(s_tok + NK);                // [CS] popped scores
  uint32_t* Sm = reinterpret_cast<uint32_t*>(Ss + CS);             // [CS] popped (parent, rank, depth)
  float* Fs = reinterpret_cast<float*>(Sm + CS);                   // [CF] frontier
  uint32_t* Fm = reinterpret_cast<uint32_t*>(Fs + CF);
  uint32_t* okey = Fm + CF;                                        // [M] sort keys
  uint16_t* ord = reinterpret_cast<uint16_t*>(okey + M);           // [M] sort slots
  int16_t* fin = reinterpret_cast<int16_t*>(ord + M);              // [CS] popped -> final index
  int16_t* n_par = fin + CS;                                       // [N] final parents
  __shared__ uint32_t sh_scan[kBT / 64];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel_prefix, sel_k, max_f;
  __shared__ int long_run;

  for (int x = tid; x < NK; x += kBT) {
    s_lp[x] = p.lp[(int64_t)b * NK + x];
    s_tok[x] = p.tok[(int64_t)b * NK + x];
  }
  __syncthreads();
  int nS = 0, nF = 0;
  if (s_lp[0] != neg_inf()) {                                      // the root's first child
    if (tid == 0) { Fs[0] = s_lp[0]; Fm[0] = node_meta(-1, 0, 1); }
    nF = 1;
  }
  __syncthreads();

  // Pops every frontier candidate whose order key is at least th (0: all)
  // and pushes their first children and next siblings; max_f gets the new
  // frontier's largest key.  Returns false on overflow (uniform).
  auto pop_round = [&](uint32_t th) -> bool {
    const int ipt = (nF + kBT - 1) / kBT;
    if (ipt > kBI) return false;
    if (tid == 0) max_f = 0;                   // ordered by the scan's barriers
    const int i0 = tid * ipt;
    float fs[kBI];
    uint32_t fm[kBI];
    uint32_t npop = 0, npush = 0;
#pragma unroll
    for (int j = 0; j < kBI; ++j) {
      const int i = i0 + j;
      const bool have = j < ipt && i < nF;
      fs[j] = have ? Fs[i] : neg_inf();
      fm[j] = have ? Fm[i] : 0u;
      if (have && ord_of(fs[j]) >= th) {
        ++npop;
        const int d = meta_depth(fm[j]), r = meta_rank(fm[j]);
        if (d < p.n_pos && s_lp[d * K] != neg_inf()) ++npush;
        if (r + 1 < K && s_lp[(d - 1) * K + r + 1] != neg_inf()) ++npush;
      }
    }
    uint32_t tot;
    const uint32_t base = block_scan(npop | (npush << 16), sh_scan, tot);
    const int cpop = (int)(tot & 0xffffu), cpush = (int)(tot >> 16);
    const int nrem = nF - cpop;
    if (nS + cpop > CS || nrem + cpush > CF) return false;
    // every thread's items are in registers: the frontier may be rewritten
    uint32_t pp = base & 0xffffu, pu = base >> 16;
    int rp = min(i0, nF) - (int)pp;            // remaining items before this thread's
    uint32_t mk = 0;                           // largest key left in or pushed to the frontier
#pragma unroll
    for (int j = 0; j < kBI; ++j) {
      const int i = i0 + j;
      if (!(j < ipt && i < nF)) continue;
      if (ord_of(fs[j]) >= th) {
        const int g = nS + (int)pp++;
        Ss[g] = fs[j];
        Sm[g] = fm[j];
        const int d = meta_depth(fm[j]), r = meta_rank(fm[j]), par = meta_par(fm[j]);
        if (d < p.n_pos && s_lp[d * K] != neg_inf()) {
          const int o = nrem + (int)pu++;
          const float sc = fs[j] + s_lp[d * K];
          Fs[o] = sc;
          Fm[o] = node_meta(g, 0, d + 1);
          mk = max(mk, ord_of(sc));
        }
        if (r + 1 < K && s_lp[(d - 1) * K + r + 1] != neg_inf()) {
          const float ps = par < 0 ? 0.f : Ss[par];
          const int o = nrem + (int)pu++;
          const float sc = ps + s_lp[(d - 1) * K + r + 1];
          Fs[o] = sc;
          Fm[o] = node_meta(par, r + 1, d);
          mk = max(mk, ord_of(sc));
        }
      } else {
        Fs[rp] = fs[j];
        Fm[rp] = fm[j];
        ++rp;
        mk = max(mk, ord_of(fs[j]));
      }
    }
    mk = wave_umax(mk);
    if (lane == 0) atomicMax(&max_f, mk);
    __syncthreads();
    nS += cpop;
    nF = nrem + cpush;
    return true;
  };

  // the kth largest order key of the popped nodes (radix select, 8 bits a
  // pass); with fewer than 4 passes, the smallest key with the kth's high
  // bytes: a lower bound of it
  auto kth_popped_key = [&](int kth, int passes) -> uint32_t {
    uint32_t prefix = 0, pmask = 0;
    uint32_t krem = (uint32_t)kth;
    for (int pass = 0; pass < passes; ++pass) {
      const int sh = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      // the keys mostly share their high bytes: the lanes of a wavefront
      // whose bin is its first active lane's add together, in one atomic
      for (int g = tid; g < nS; g += kBT) {
        const uint32_t key = ord_of(Ss[g]);
        const bool act = (key & pmask) == prefix;
        const uint32_t bin = (key >> sh) & 255u;
        const uint64_t am = __ballot(act);
        if (am) {
          const int first = __ffsll((unsigned long long)am) - 1;
          const uint32_t b0 = (uint32_t)__shfl((int)bin, first, 64);
          const uint64_t same = __ballot(act && bin == b0);
          if (lane == first) atomicAdd(&hist[b0], (uint32_t)__popcll(same));
          if (act && bin != b0) atomicAdd(&hist[bin], 1u);
        }
      }
      __syncthreads();
      if (w == 0) {
        // lane l holds bins 4l..4l+3; suffix sums from the top bin down
        uint32_t c[4], s4 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { c[q] = hist[4 * lane + q]; s4 += c[q]; }
        uint32_t suf = s4;                        // inclusive suffix over lanes >= lane
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = __shfl_down(suf, o, 64);
          if (lane + o < 64) suf += y;
        }
        const uint32_t above = suf - s4;          // keys in bins of higher lanes
        const bool mine = above < krem && krem <= suf;
        if (mine) {
          uint32_t acc = above;
          int bin = 4 * lane;
#pragma unroll
          for (int q = 3; q >= 0; --q) {
            if (acc + c[q] >= krem) { bin = 4 * lane + q; break; }
            acc += c[q];
          }
          sel_prefix = prefix | ((uint32_t)bin << sh);
          sel_k = krem - acc;
        }
      }
      __syncthreads();
      prefix = sel_prefix;
      krem = sel_k;
      pmask |= 255u << sh;
      __syncthreads();
    }
    return prefix;
  };

  bool ok = true;
  while (ok && nF > 0 && nS < N) ok = pop_round(0u);
  // finish: th is a lower bound of the budget-th best key of the popped
  // nodes (its high 16 bits, from when it was last computed; the key only
  // rises as nodes are popped), which keeps the test below valid (it may pop
  // a few nodes more).  It is recomputed after every budget / 4 new pops.
  uint32_t th = 0;
  int at = -N;
  while (ok && nF > 0) {
    if (nS - at > N / 4) {
      th = kth_popped_key(N, 2);
      at = nS;
    }
    const uint32_t mfv = max_f;                // from the last pop round
    __syncthreads();                           // read by all before the next round resets it
    if (mfv < th) break;
    ok = pop_round(th);
  }
  if (!ok) {
    // overflow: the serial loop, from scratch, in the same memory
    if (w == 0) tree_build_serial(p, smem, b, lane);
    return;
  }
  // the candidates for the first N: popped nodes at or above the budget-th
  // best key (all popped nodes if fewer than N exist)
  if (nS < N) th = 0;
  else th = kth_popped_key(N, 4);
  uint32_t tot;
  {
    // slots in popped order: each thread takes a contiguous range
    const int ipt = (nS + kBT - 1) / kBT;
    const int g0 = tid * ipt, g1 = min(nS, g0 + ipt);
    uint32_t c = 0;
    for (int g = g0; g < g1; ++g) c += ord_of(Ss[g]) >= th;
    uint32_t o = block_scan(c, sh_scan, tot);
    for (int g = g0; g < g1; ++g) {
      const uint32_t key = ord_of(Ss[g]);
      if (key >= th) { okey[o] = key; ord[o++] = (uint16_t)g; }
    }
  }
  const int nc = (int)tot;
  const int Msort = pow2_at_least(max(nc, 2));
  for (int x = nc + tid; x < Msort; x += kBT) { okey[x] = 0u; ord[x] = 0xffffu; }   // sort last
  __syncthreads();
  // bitonic sort of the slots by key descending, then popped index
  // ascending (the pop order wherever the scores differ)
  if (Msort >= kBT && Msort <= kBT * kSortE) {
    uint64_t* xch = reinterpret_cast<uint64_t*>(Fs);    // the frontier's memory, no longer needed
    if (Msort == kBT) sort_slots<kBT>(okey, ord, xch);
    else if (Msort == 2 * kBT) sort_slots<2 * kBT>(okey, ord, xch);
    else if (Msort == 4 * kBT) sort_slots<4 * kBT>(okey, ord, xch);
    else sort_slots<8 * kBT>(okey, ord, xch);
  } else {
    for (int size = 2; size <= Msort; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int x = tid; x < Msort / 2; x += kBT) {
          const int lo = 2 * x - (x & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const uint32_t ka = okey[lo], kb = okey[hi];
          const int a = ord[lo], bb = ord[hi];
          const bool a_after = ka < kb || (ka == kb && a > bb);
          if (a_after == up) {
            okey[lo] = kb; okey[hi] = ka;
            ord[lo] = (uint16_t)bb; ord[hi] = (uint16_t)a;
          }
        }
        __syncthreads();
      }
    }
  }
  // runs of equal scores: put each run in the pop order (its parents' pop
  // order, then rank), by the thread that holds the run's first slot; a run
  // longer than 32 slots sends the whole list through the exact comparison
  if (tid == 0) long_run = 0;
  __syncthreads();
  for (int x = tid; x < nc; x += kBT) {
    if ((x > 0 && okey[x - 1] == okey[x]) || x + 1 >= nc || okey[x + 1] != okey[x]) continue;
    int e = x + 1;
    while (e < nc && okey[e] == okey[x]) ++e;
    if (e - x > 32) {
      long_run = 1;
      continue;
    }
    for (int i = x + 1; i < e; ++i) {            // insertion sort of ord[x, e)
      const int v = ord[i];
      int j = i - 1;
      while (j >= x && pop_before(v, ord[j], Ss, Sm)) {
        ord[j + 1] = ord[j];
        --j;
      }
      ord[j + 1] = (uint16_t)v;
    }
  }
  __syncthreads();
  if (long_run) {
    for (int size = 2; size <= Msort; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int x = tid; x < Msort / 2; x += kBT) {
          const int lo = 2 * x - (x & (stride - 1));
          const int hi = lo + stride;
          const bool up = (lo & size) == 0;
          const int a = ord[lo], bb = ord[hi];
          const bool a_after = a == 0xffff ? bb != 0xffff
                                           : (bb != 0xffff && pop_before(bb, a, Ss, Sm));
          if (a_after == up) { ord[lo] = (uint16_t)bb; ord[hi] = (uint16_t)a; }
        }
        __syncthreads();
      }
    }
  }
  const int n = min(N, nc);
  for (int g = tid; g < nS; g += kBT) fin[g] = -1;
  __syncthreads();
  for (int i = tid; i < n; i += kBT) fin[ord[i]] = (int16_t)i;
  __syncthreads();
  if (tid == 0) p.n_nodes[b] = n;
  for (int x = tid; x < N; x += kBT) {
    const int64_t o = (int64_t)b * N + x;
    if (x < n) {
      const int g = ord[x];
      const uint32_t m = Sm[g];
      const int d = meta_depth(m), par = meta_par(m);
      const int fp = par < 0 ? -1 : fin[par];
      p.node_token[o] = s_tok[(d - 1) * K + meta_rank(m)];
      p.node_parent[o] = fp;
      p.node_depth[o] = d;
      p.node_logp[o] = Ss[g];
      n_par[x] = (int16_t)fp;
    } else {
      p.node_token[o] = -1; p.node_parent[o] = -2; p.node_depth[o] = 0; p.node_logp[o] = neg_inf();
    }
  }
  __syncthreads();
  if (p.mask) {
    // row x: bits of x and of its ancestors, written word by word from the
    // top (the ancestors come in falling index order); unused rows are zero
    for (int x = tid; x < N; x += kBT) {
      uint32_t* row = p.mask + ((int64_t)b * N + x) * p.W;
      int wd = p.W - 1;
      if (x < n) {
        const int top_w = x >> 5;
        for (; wd > top_w; --wd) row[wd] = 0u;
        uint32_t acc = 0u;
        for (int y = x; y >= 0; y = n_par[y]) {
          const int yw = y >> 5;
          while (wd > yw) { row[wd] = acc; acc = 0u; --wd; }
          acc |= 1u << (y & 31);
        }
        row[wd] = acc;
        --wd;
      }
      for (; wd >= 0; --wd) row[wd] = 0u;
    }
  }
}

// KV recycling ([Spec tutorial] 6.6): one workgroup per (layer, request,
// committed row t): row t is the root (t = 0) or the t-th accepted node, and
// it is copied, K and V, to the slot of logical position prefix + t, 16 bytes
// per lane.  Rows past the accepted length, past the path list, or on an
// unmapped or out-of-range page are not written.
__global__ __launch_bounds__(256) void k_tree_commit(CommitArgs a) {
  const int T = a.max_depth + 1;
  const int t = blockIdx.x % T;
  const int b = (blockIdx.x / T) % a.B;
  const int l = blockIdx.x / (T * a.B);
  const int acc = a.accept_len[b];
  if (acc < 0 || t > acc) return;
  const int src = t == 0 ? 0 : 1 + a.path[(int64_t)b * a.max_depth + t - 1];
  if (src < 0 || src >= a.R) return;
  const int pos = a.prefix[b] + t;
  if (pos < 0 || (pos >> 4) >= a.max_pages) return;
  const int page = a.block_table[(int64_t)b * a.max_pages + (pos >> 4)];
  if (page < 0 || page >= a.num_pages[l]) return;
  const int64_t head_bytes = (int64_t)a.D * a.es;
  const int64_t row_bytes = a.Hkv * head_bytes;
  const char* ks = static_cast<const char*>(a.k_tree[l]) + ((int64_t)b * a.R + src) * row_bytes;
  const char* vs = static_cast<const char*>(a.v_tree[l]) + ((int64_t)b * a.R + src) * row_bytes;
  // head-major pages [Hkv, 16, D]: head h of position pos at (h*16 + pos%16) * D
  const int64_t dst0 = (int64_t)page * 16 * row_bytes + (pos & 15) * head_bytes;
  char* kd = static_cast<char*>(a.cache_k[l]) + dst0;
  char* vd = static_cast<char*>(a.cache_v[l]) + dst0;
  for (int64_t c = threadIdx.x; c < row_bytes / 16; c += 256) {
    const int64_t h = 16 * c / head_bytes;
    const int64_t o = h * 16 * head_bytes + (16 * c - h * head_bytes);
    *reinterpret_cast<uint4*>(kd + o) = *reinterpret_cast<const uint4*>(ks + 16 * c);
    *reinterpret_cast<uint4*>(vd + o) = *reinterpret_cast<const uint4*>(vs + 16 * c);
  }
}

struct TopkPlan {
  VocabPlan pl;
  size_t cand_v, cand_i, part;   // byte offsets in the workspace
  size_t total;
};

// Row chunks for the top-K pass: long ones (a wavefront's fixed costs, the
// threshold seed and the folds, are then small next to its stream), split
// only as far as needed for about DFLASH_TOPK_WGS workgroups, at most 64 per
// row.
VocabPlan topk_chunks(int64_t rows, int V) {
  const int64_t want = std::max<int64_t>(1, cdiv(DFLASH_TOPK_WGS, std::max<int64_t>(rows, 1)));
  int64_t n = std::min<int64_t>({want, cdiv(V, 32768), 64});
  n = std::max<int64_t>(n, 1);
  const int64_t chunk = cdiv(cdiv(V, n), 8) * 8;
  return VocabPlan{(int)chunk, (int)cdiv(V, chunk)};
}

TopkPlan topk_plan(int64_t rows, int V, int K) {
  TopkPlan t;
  t.pl = topk_chunks(rows, V);
  const int64_t n = rows * t.pl.n_chunks;
  t.cand_v = 0;
  t.cand_i = align256(sizeof(float) * n * K);
  t.part = t.cand_i + align256(sizeof(int) * n * K);
  t.total = t.part + align256(sizeof(float2) * n);
  return t;
}

size_t tree_lds_bytes(int n_pos, int K, int budget) {
  return (size_t)tree_cap(budget) * 8 + (size_t)budget * 12 + (size_t)n_pos * K * 8;
}

}  // namespace

size_t tree_ws_bytes(int B, int n_pos, int V, int K) {
  return topk_plan((int64_t)B * n_pos, V, K).total;
}

// the parallel build's buffers (or the serial loop's, if larger: its fallback
// runs in the same memory)
size_t par_lds_bytes(int n_pos, int K, int budget) {
  const size_t CS = par_cap(budget), CF = CS + 1, M = pow2_at_least(par_cap(budget));
  const size_t NK = (size_t)n_pos * K;
  const size_t need = NK * 8 + CS * 8 + CF * 8 + M * 6 + CS * 2 + (size_t)budget * 2;
  return std::max(need, tree_lds_bytes(n_pos, K, budget));
}

size_t tree_build_lds_bytes(int n_pos, int K, int budget) {
  return DFLASH_TREE_PARALLEL ? par_lds_bytes(n_pos, K, budget) : tree_lds_bytes(n_pos, K, budget);
}

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
  if (DFLASH_TREE_PARALLEL)
    hipLaunchKernelGGL(k_tree_build_par, dim3(B), dim3(kBT), par_lds_bytes(n_pos, K, budget), st, p);
  else
    hipLaunchKernelGGL(k_tree_build, dim3(B), dim3(64), tree_lds_bytes(n_pos, K, budget), st, p);
  return hipGetLastError();
}

hipError_t launch_tree_commit(const CommitArgs& a, hipStream_t st) {
  const int64_t grid = (int64_t)a.n_layers * a.B * (a.max_depth + 1);
  hipLaunchKernelGGL(k_tree_commit, dim3((unsigned)grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dflash
