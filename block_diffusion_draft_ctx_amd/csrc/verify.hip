// Vocabulary-wide verification and the DLoop gate.
//
// Greedy acceptance: [SGLang DFlash], section 3 (target prediction = row
// argmax; leading matches; bonus = prediction at accept_len).
// Rejection sampling: [Spec tutorial], section 3 (accept with min(1, p/q);
// residual max(0, p - q) renormalised) and section 4 (first rejection ends the
// chain); all-accepted bonus from the next target row ([DFlash overview],
// pseudocode); chains of several stages ([DLoop], "验证与无损性").
// Gate: [DLoop], "机制一：置信度门控" (c = sum of drafted-token log-probs,
// continue iff c >= g).
//
// Design.  Every logit row is read once, coalesced, by workgroups that each
// reduce one chunk of the row (16-byte loads, 4 in flight per lane).  A chunk
// reduces to (max, lowest argmax) for greedy, or to (m, s) with
// m = max(z), s = sum 2^(z - m), z = logit * log2(e) / T for the softmax
// normalisers.  Small per-request kernels merge the chunk partials in a fixed
// order (deterministic), run the sequential acceptance scan, and -- for a
// rejection or the all-accepted bonus -- re-read the one chosen row pair
// (cache-resident) to build the inverse CDF: per-chunk weight sums, then a
// chunk-local scan inside the selected chunk.
#include <algorithm>
#include <climits>
#include <mutex>

#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 64;
// Tuning knobs: workgroups a vocabulary pass aims for, and 16-byte loads in
// flight per lane in the row passes.
#ifndef DFLASH_VOCAB_WGS
#define DFLASH_VOCAB_WGS 2048
#endif
#ifndef DFLASH_VOCAB_INFLIGHT
#define DFLASH_VOCAB_INFLIGHT 8
#endif
constexpr int kNF = DFLASH_VOCAB_INFLIGHT;

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct ReqInfo {
  int row;    // bonus row index within the request (= accept_len)
  int mode;   // 0: residual of a rejected row, 1: bonus from p of the row
  int acc;    // accept_len
  int err;    // in-band error
  float Mt, St, Md, Sd;  // base-2 normalisers of the chosen rows
};

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int chain_of(const int32_t* lens, int b, int L, bool* bad) {
  if (!lens) { if (bad) *bad = false; return L; }
  int v = lens[b];
  bool b_ = (v < 0 || v > L);
  if (bad) *bad = b_;
  return b_ ? L : v;
}

// Map a flat row index of the launch to (set, b, i, row pointer).
template <typename T>
__device__ __forceinline__ bool locate_row(const RowSet& s0, const RowSet& s1, int B, int L,
                                           const int32_t* lens, int r, const T** row) {
  const int rows0 = B * s0.rows_per_req;
  const RowSet& s = (r < rows0) ? s0 : s1;
  const int rl = (r < rows0) ? r : r - rows0;
  const int b = rl / s.rows_per_req;
  const int i = rl - b * s.rows_per_req;
  const int nb = chain_of(lens, b, L, nullptr);
  if (i >= nb + s.extra) return false;
  *row = static_cast<const T*>(s.base) + (int64_t)rl * s.stride;
  return true;
}

// ---------------------------------------------------------------- argmax pass
__device__ __forceinline__ void am_update(const float (&v)[8], int x, float& best, int& bi) {
  float m8 = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                   fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
  if (m8 > best) {
    best = m8;
#pragma unroll
    for (int j = 7; j >= 0; --j)
      if (v[j] == m8) bi = x + j;  // the loop runs downward, so the lowest j wins
  }
}
__device__ __forceinline__ void am_merge(float& best, int& bi, float ob, int oi) {
  if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_row_argmax(RowSet s0, RowSet s1, int B, int L,
                                                         int V, const int32_t* __restrict__ lens,
                                                         int chunk, int n_chunks,
                                                         float* __restrict__ pmax,
                                                         int* __restrict__ pidx) {
  const int c = blockIdx.x % n_chunks;
  const int r = blockIdx.x / n_chunks;
  const T* row;
  if (!locate_row<T>(s0, s1, B, L, lens, r, &row)) return;
  const int x0 = c * chunk;
  const int x1 = min(V, x0 + chunk);
  float best = neg_inf();
  int bi = INT_MAX;
  if (VEC) {
    // full rounds of kNF 16-byte loads in flight per lane, then one last
    // round whose loads are issued together at clamped (always valid)
    // indices, the values past the end being dropped
    const int nvec = (x1 - x0) >> 3;
    int v = threadIdx.x;
    for (; v + (kNF - 1) * kThreads < nvec; v += kNF * kThreads) {
      float a[kNF][8];
#pragma unroll
      for (int u = 0; u < kNF; ++u) load8(row + x0 + (v + u * kThreads) * 8, a[u]);
#pragma unroll
      for (int u = 0; u < kNF; ++u) am_update(a[u], x0 + (v + u * kThreads) * 8, best, bi);
    }
    if (v < nvec) {
      float a[kNF][8];
#pragma unroll
      for (int u = 0; u < kNF; ++u) load8(row + x0 + min(v + u * kThreads, nvec - 1) * 8, a[u]);
#pragma unroll
      for (int u = 0; u < kNF; ++u)
        if (v + u * kThreads < nvec) am_update(a[u], x0 + (v + u * kThreads) * 8, best, bi);
    }
    for (int x = x0 + nvec * 8 + threadIdx.x; x < x1; x += kThreads) {
      float e = load1(row + x);
      if (e > best) { best = e; bi = x; }
    }
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kThreads) {
      float e = load1(row + x);
      if (e > best) { best = e; bi = x; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ob = __shfl_xor(best, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    am_merge(best, bi, ob, oi);
  }
  __shared__ float sb[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sb[w] = best; si[w] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / 64; ++k) am_merge(sb[0], si[0], sb[k], si[k]);
    pmax[blockIdx.x] = sb[0];
    pidx[blockIdx.x] = si[0];
  }
}

// Argmax of one row from its chunk partials, by a group of G lanes (G = 1, 2
// or 4, aligned within the wavefront, nc <= 16 G): lane `sub` of the group
// loads chunks sub, sub + G, ... together, merges them, and the group merges
// its lanes by shuffles.  The merge is a total order (value, then lower
// index; a NaN never wins), so the winner does not depend on the grouping.
// Every lane of the wavefront must call this (the shuffles); lanes with
// valid == false contribute nothing.  An all -inf row: every entry ties and
// the first wins; no entry at all gives 0.
__device__ int group_argmax_row(const float* pmax, const int* pidx, int row, int nc, int G,
                                int sub, bool valid) {
  float best = neg_inf();
  int bi = INT_MAX;
  if (valid) {
    float v[16];
    int ix[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = min(sub + G * j, nc - 1);
      v[j] = pmax[row * nc + c];
      ix[j] = pidx[row * nc + c];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (sub + G * j < nc) am_merge(best, bi, v[j], ix[j]);
  }
  for (int o = 1; o < G; o <<= 1) {
    const float ob = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    am_merge(best, bi, ob, oi);
  }
  return bi == INT_MAX ? 0 : bi;
}

// Greedy acceptance of request b: the argmax of every target row of the
// chain (and, with fused draft logits, of every draft row) from the chunk
// partials, then matches -> cumulative product -> accept_len and the bonus.
// The rows' merges run on groups of lanes, so a request whose rows have many
// chunk partials (small batches) reads them in one round of loads.
__global__ __launch_bounds__(128) void k_greedy_finalize(
    int B, int L, int V, int nc, const float* __restrict__ pmax, const int* __restrict__ pidx,
    int have_dl, int32_t* __restrict__ draft_tokens, const int32_t* __restrict__ lens,
    int32_t* __restrict__ target_predict, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ bonus, int32_t* __restrict__ commit,
    const int32_t* __restrict__ prefix, int32_t* __restrict__ new_seq) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  __shared__ int tp[65];
  __shared__ int dt[64];
  bool bad;
  const int nb = chain_of(lens, b, L, &bad);
  if (t <= L) tp[t] = -1;
  if (t < L) dt[t] = have_dl ? -1 : draft_tokens[b * L + t];
  __syncthreads();
  // rows r <= nb: target row r; rows nb < r <= 2 nb (with draft logits):
  // draft row r - nb - 1
  const int G = nc > 32 ? 4 : (nc > 16 ? 2 : 1);
  const int R = nb + 1 + (have_dl ? nb : 0);
  for (int r0 = 0; r0 < R; r0 += 128 / G) {
    const int r = r0 + t / G;
    const bool valid = r < R;
    const int row = r <= nb ? b * (L + 1) + r : B * (L + 1) + b * L + (r - nb - 1);
    const int v = group_argmax_row(pmax, pidx, valid ? row : 0, nc, G, t % G, valid);
    if (valid && t % G == 0) {
      if (r <= nb) tp[r] = v;
      else dt[r - nb - 1] = v;
    }
  }
  __syncthreads();
  if (t <= L && target_predict) target_predict[b * (L + 1) + t] = tp[t];
  if (have_dl && t < nb) draft_tokens[b * L + t] = dt[t];
  if (t == 0) {
    bool err = bad;
    for (int i = 0; i < nb; ++i) err |= (dt[i] < 0 || dt[i] >= V);
    int a = -1, bo = -1;
    if (!err) {
      a = 0;
      while (a < nb && dt[a] == tp[a]) ++a;
      bo = tp[a];
    }
    const int cm = err ? 0 : a + 1;
    accept_len[b] = a;
    bonus[b] = bo;
    commit[b] = cm;
    if (new_seq) new_seq[b] = prefix[b] + cm;
  }
}

// ------------------------------------------------------------ softmax pass
__device__ __forceinline__ void lse_update(const float (&v)[8], float a, float& m, float& s) {
  float xm = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                   fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
  float gm = xm * a;
  if (gm > m) {
    s *= fexp2(m - gm);
    m = gm;
  }
  if (m != neg_inf()) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += fexp2(fmaf(v[j], a, -m));
    s += acc;
  }
}
__device__ __forceinline__ void lse_update1(float v, float a, float& m, float& s) {
  float z = v * a;
  if (z > m) { s *= fexp2(m - z); m = z; }
  if (m != neg_inf()) s += fexp2(z - m);
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_row_lse(RowSet s0, RowSet s1, int B, int L, int V,
                                                      const int32_t* __restrict__ lens, float a,
                                                      int chunk, int n_chunks,
                                                      float2* __restrict__ part) {
  const int c = blockIdx.x % n_chunks;
  const int r = blockIdx.x / n_chunks;
  const T* row;
  if (!locate_row<T>(s0, s1, B, L, lens, r, &row)) return;
  const int x0 = c * chunk;
  const int x1 = min(V, x0 + chunk);
  float m = neg_inf(), s = 0.f;
  if (VEC) {
    // full rounds of kNF 16-byte loads in flight per lane, then one last
    // round whose loads are issued together at clamped (always valid)
    // indices, the values past the end being dropped
    const int nvec = (x1 - x0) >> 3;
    int v = threadIdx.x;
    for (; v + (kNF - 1) * kThreads < nvec; v += kNF * kThreads) {
      float e[kNF][8];
#pragma unroll
      for (int u = 0; u < kNF; ++u) load8(row + x0 + (v + u * kThreads) * 8, e[u]);
#pragma unroll
      for (int u = 0; u < kNF; ++u) lse_update(e[u], a, m, s);
    }
    if (v < nvec) {
      float e[kNF][8];
#pragma unroll
      for (int u = 0; u < kNF; ++u) load8(row + x0 + min(v + u * kThreads, nvec - 1) * 8, e[u]);
#pragma unroll
      for (int u = 0; u < kNF; ++u)
        if (v + u * kThreads < nvec) lse_update(e[u], a, m, s);
    }
    for (int x = x0 + nvec * 8 + threadIdx.x; x < x1; x += kThreads) lse_update1(load1(row + x), a, m, s);
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kThreads) lse_update1(load1(row + x), a, m, s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float om = __shfl_xor(m, o, 64);
    float os = __shfl_xor(s, o, 64);
    lse2_merge(m, s, om, os);
  }
  __shared__ float sm[kThreads / 64], ss[kThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { sm[w] = m; ss[w] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = sm[0], s2 = ss[0];
    for (int k = 1; k < kThreads / 64; ++k) lse2_merge(mm, s2, sm[k], ss[k]);
    part[blockIdx.x] = make_float2(mm, s2);
  }
}

// Merge a row's chunk partials in chunk order; up to eight are loaded
// together (indices clamped to valid ones) before they are merged.
__device__ void reduce_lse_row(const float2* part, int row, int nc, float& m, float& s) {
  m = neg_inf();
  s = 0.f;
  for (int c0 = 0; c0 < nc; c0 += 8) {
    float2 p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = part[row * nc + min(c0 + j, nc - 1)];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < nc) lse2_merge(m, s, p[j].x, p[j].y);
  }
}

// --------------------------------------------------------- sampled verify
// The acceptance scan of request b, run by a whole workgroup (at least 128
// threads; thread t < 64 owns chain link t): merge each row's chunk partials
// into its base-2 normalisers, form p/q at the drafted token, and find the
// first rejected link by a ballot.  Every thread gets the request's ReqInfo.
// With draft_lse (the draft rows' log-sum-exp at temperature T, as the gate
// exports it) the draft rows have no chunk partials: their base-2
// normaliser is lse * log2(e) with a unit sum.
template <typename T>
__device__ ReqInfo accept_scan(int b, int B, int L, int V, int nc, const float2* __restrict__ part,
                               const T* __restrict__ tl, int64_t ts, const T* __restrict__ dl,
                               int64_t ds, const int32_t* __restrict__ toks,
                               const int32_t* __restrict__ lens, const float* __restrict__ u,
                               float a, float* __restrict__ ratio_out,
                               const float* __restrict__ draft_lse) {
  const int t = threadIdx.x;
  __shared__ float Mt[65], St[65], Md[64], Sd[64], rat[64];
  __shared__ int okx[64];
  __shared__ ReqInfo sI;
  bool bad;
  const int nb = chain_of(lens, b, L, &bad);
  if (t <= nb) reduce_lse_row(part, b * (L + 1) + t, nc, Mt[t], St[t]);
  if (t < nb) {
    if (draft_lse) {
      Md[t] = draft_lse[b * L + t] * kLog2e;
      Sd[t] = 1.f;
    } else {
      reduce_lse_row(part, B * (L + 1) + b * L + t, nc, Md[t], Sd[t]);
    }
    const int x = toks[b * L + t];
    float r = __builtin_nanf("");
    okx[t] = (x >= 0 && x < V);
    if (okx[t]) {
      const float tx = load1(tl + (int64_t)(b * (L + 1) + t) * ts + x);
      const float dx = load1(dl + (int64_t)(b * L + t) * ds + x);
      if (dx == neg_inf()) {
        // q(x) = 0: the ratio is taken as +inf, so the token is accepted
        // whatever p(x) is (0/0 included)
        r = __builtin_inff();
      } else {
        const float e = fmaf(tx, a, -Mt[t]) - fmaf(dx, a, -Md[t]);
        r = exp2f(e) * (Sd[t] / St[t]);
      }
    }
    rat[t] = r;
    if (ratio_out) ratio_out[b * L + t] = r;
  } else if (t < L && ratio_out) {
    ratio_out[b * L + t] = __builtin_nanf("");
  }
  __syncthreads();
  // the first wavefront holds every link (chain <= 64): the first rejected
  // link by a ballot
  const bool in_chain = t < nb;
  const bool rej = in_chain && !(u[b * L + t] < rat[min(t, 63)]);
  const uint64_t rejm = __ballot(rej);
  const uint64_t badm = __ballot(in_chain && !okx[min(t, 63)]);
  if (t == 0) {
    ReqInfo I;
    const bool err = bad || badm != 0;
    I.err = err;
    I.acc = -1; I.row = 0; I.mode = 1;
    I.Mt = I.St = I.Md = I.Sd = 0.f;
    if (!err) {
      const int j = rejm ? __ffsll((unsigned long long)rejm) - 1 : nb;
      I.acc = j;
      I.row = j;
      I.mode = (j < nb) ? 0 : 1;
      I.Mt = Mt[j];
      I.St = St[j];
      if (j < nb) { I.Md = Md[j]; I.Sd = Sd[j]; }
    }
    sI = I;
  }
  __syncthreads();
  return sI;
}

// Weight of token x in the bonus draw: residual max(0, p - q) (kind 0) or the
// unnormalised target exponential 2^(z - Mt) (kind 1).
template <typename T>
struct BonusRow {
  const T* tr;
  const T* dr;
  float a, Mt, invSt, Md, invSd;
  __device__ __forceinline__ float et(float tv) const { return fexp2(fmaf(tv, a, -Mt)); }
  __device__ __forceinline__ float res(float tv, float dv) const {
    float p = et(tv) * invSt;
    float q = fexp2(fmaf(dv, a, -Md)) * invSd;
    return fmaxf(0.f, p - q);
  }
};

// Chunk c's residual weights max(0, p - q) (mode 0), min(p, q) and target
// weights of request b's chosen row pair, summed into rpart.
template <typename T, bool VEC>
__device__ void bonus_chunk_sum(int c, int chunk, int V, const T* __restrict__ tl, int64_t ts,
                                const T* __restrict__ dl, int64_t ds, float a, int b, int L,
                                const ReqInfo I, float4* __restrict__ rpart) {
  BonusRow<T> R{tl + (int64_t)(b * (L + 1) + I.row) * ts,
                I.mode == 0 ? dl + (int64_t)(b * L + I.row) * ds : nullptr,
                a, I.Mt, 1.f / I.St, I.Md, I.mode == 0 ? 1.f / I.Sd : 0.f};
  const int x0 = c * chunk;
  const int x1 = min(V, x0 + chunk);
  float ar = 0.f, amin = 0.f, ap = 0.f;
  auto one = [&](float tv, float dv) {
    float e = R.et(tv);
    ap += e;
    if (I.mode == 0) {
      float p = e * R.invSt;
      float q = fexp2(fmaf(dv, R.a, -R.Md)) * R.invSd;
      ar += fmaxf(0.f, p - q);
      amin += fminf(p, q);
    }
  };
  if (VEC) {
    const int nvec = (x1 - x0) >> 3;
    for (int v = threadIdx.x; v < nvec; v += 2 * kThreads) {
      // two loads per operand row in flight; the second index is clamped
      // (always valid) and its values dropped past the end
      float tv[2][8], dv[2][8] = {};
      const int v1 = min(v + kThreads, nvec - 1);
      load8(R.tr + x0 + v * 8, tv[0]);
      load8(R.tr + x0 + v1 * 8, tv[1]);
      if (I.mode == 0) {
        load8(R.dr + x0 + v * 8, dv[0]);
        load8(R.dr + x0 + v1 * 8, dv[1]);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) one(tv[0][j], dv[0][j]);
      if (v + kThreads < nvec) {
#pragma unroll
        for (int j = 0; j < 8; ++j) one(tv[1][j], dv[1][j]);
      }
    }
    for (int x = x0 + nvec * 8 + threadIdx.x; x < x1; x += kThreads)
      one(load1(R.tr + x), I.mode == 0 ? load1(R.dr + x) : 0.f);
  } else {
    for (int x = x0 + threadIdx.x; x < x1; x += kThreads)
      one(load1(R.tr + x), I.mode == 0 ? load1(R.dr + x) : 0.f);
  }
  ar = wave_sum(ar);
  amin = wave_sum(amin);
  ap = wave_sum(ap);
  __shared__ float s[3][kThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s[0][w] = ar; s[1][w] = amin; s[2][w] = ap; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < kThreads / 64; ++k) { o.x += s[0][k]; o.y += s[1][k]; o.z += s[2][k]; }
    rpart[blockIdx.x] = o;
  }
  __syncthreads();
}

// Bonus draw of request b by one workgroup, once every chunk's residual (or
// target) weight sum of the chosen row pair is in rpart: pick the chunk that
// holds u' * (total weight), then scan inside it.
template <typename T>
__device__ void select_bonus(
    int b, int L, int V, int chunk, int nc, const T* __restrict__ tl, int64_t ts,
    const T* __restrict__ dl, int64_t ds, float a, const ReqInfo I,
    const float4* __restrict__ rpart, const float* __restrict__ u2,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ bonus, int32_t* __restrict__ commit,
    const int32_t* __restrict__ prefix, int32_t* __restrict__ new_seq,
    float* __restrict__ beta_out, float* __restrict__ gap_out) {
  const int t = threadIdx.x;
  if (I.err) {
    if (t == 0) {
      accept_len[b] = -1; bonus[b] = -1; commit[b] = 0;
      if (new_seq) new_seq[b] = prefix[b];
      if (beta_out) beta_out[b] = __builtin_nanf("");
      if (gap_out) gap_out[b] = __builtin_nanf("");
    }
    return;
  }
  __shared__ int sh_kind, sh_cc, sh_x;
  __shared__ float sh_base, sh_thr, sh_Z;
  __shared__ float sh_loc[kThreads / 64];
  __shared__ float sh_gap;
  __shared__ int sh_last;
  // Chunk selection by the first wavefront, lane c holding chunk c (at most
  // 64 chunks): totals by butterfly sums, the running weight by a shuffle
  // scan in chunk order, the chunk by a ballot.
  if (t < 64) {
    const float4 pc = (t < nc) ? rpart[b * nc + t] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float Rs = wave_sum(pc.x), Ms = wave_sum(pc.y), Ps = wave_sum(pc.z);
    const int kind = (I.mode == 0 && Rs > 0.f) ? 0 : 1;
    const float Z = kind == 0 ? Rs : Ps;
    const float thr = u2[b] * Z;
    const float w = kind == 0 ? pc.x : pc.z;
    float incl = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float v = __shfl_up(incl, o, 64);
      if (t >= o) incl += v;
    }
    const uint64_t over = __ballot(t < nc && incl > thr);
    int cc;
    if (over) {
      cc = __ffsll((unsigned long long)over) - 1;
    } else {  // rounding left u'*Z at the very end: the last chunk with mass
      const uint64_t pos = __ballot(t < nc && w > 0.f);
      cc = pos ? 63 - __clzll((long long)pos) : 0;   // no mass at all only with invalid logits
    }
    const float base = __shfl(incl - w, cc, 64);
    if (t == 0) {
      sh_kind = kind; sh_cc = cc; sh_base = base; sh_thr = thr; sh_Z = Z;
      sh_x = INT_MAX; sh_last = -1; sh_gap = 0.f;
      if (beta_out) beta_out[b] = (I.mode == 0) ? Ms : __builtin_nanf("");
    }
  }
  __syncthreads();
  BonusRow<T> R{tl + (int64_t)(b * (L + 1) + I.row) * ts,
                I.mode == 0 ? dl + (int64_t)(b * L + I.row) * ds : nullptr,
                a, I.Mt, 1.f / I.St, I.Md, I.mode == 0 ? 1.f / I.Sd : 0.f};
  const int kind = sh_kind;
  auto wt = [&](int x) -> float {
    float tv = load1(R.tr + x);
    return kind == 0 ? R.res(tv, load1(R.dr + x)) : R.et(tv);
  };
  const int x0 = sh_cc * chunk;
  const int x1 = min(V, x0 + chunk);
  const int seg = (x1 - x0 + kThreads - 1) / kThreads;
  const int xs = min(x1, x0 + t * seg);
  const int xe = min(x1, xs + seg);
  // the thread's segment: up to kSeg weights loaded together and kept in
  // registers (longer segments, for very large vocabularies, are streamed)
  constexpr int kSeg = 16;
  const bool inreg = seg <= kSeg;
  float wv[kSeg];
  float loc = 0.f;
  int lastpos = -1;
  if (inreg) {
    // loads at clamped (always valid) positions, issued together; weights
    // past the segment end are dropped
    const int xl = max(xe - 1, x0);
    float tv[kSeg];
#pragma unroll
    for (int i = 0; i < kSeg; ++i) tv[i] = load1(R.tr + min(xs + i, xl));
    if (kind == 0) {
      float dv[kSeg];
#pragma unroll
      for (int i = 0; i < kSeg; ++i) dv[i] = load1(R.dr + min(xs + i, xl));
#pragma unroll
      for (int i = 0; i < kSeg; ++i) wv[i] = (xs + i < xe) ? R.res(tv[i], dv[i]) : 0.f;
    } else {
#pragma unroll
      for (int i = 0; i < kSeg; ++i) wv[i] = (xs + i < xe) ? R.et(tv[i]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < kSeg; ++i) {
      loc += wv[i];
      if (wv[i] > 0.f) lastpos = xs + i;
    }
  } else {
    for (int x = xs; x < xe; ++x) {
      float w = wt(x);
      loc += w;
      if (w > 0.f) lastpos = x;
    }
  }
  if (lastpos >= 0) atomicMax(&sh_last, lastpos);
  // exclusive prefix of the segment sums in segment order: shuffle scan in
  // each wavefront, then the wavefront totals
  float incl = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_up(incl, o, 64);
    if ((t & 63) >= o) incl += v;
  }
  if ((t & 63) == 63) sh_loc[t >> 6] = incl;
  __syncthreads();
  float wpre = 0.f;
  for (int k = 0; k < (t >> 6); ++k) wpre += sh_loc[k];
  const float thr = sh_thr;
  const float base = sh_base + wpre + (incl - loc);
  if (base <= thr && base + loc > thr) {
    float acc = base;
    int found = -1;
    float lo = 0.f, hi = 0.f;
    if (inreg) {
#pragma unroll
      for (int i = 0; i < kSeg; ++i) {
        if (found < 0 && xs + i < xe) {
          if (acc + wv[i] > thr) { found = xs + i; lo = acc; hi = acc + wv[i]; }
          else acc += wv[i];
        }
      }
    } else {
      for (int x = xs; x < xe; ++x) {
        float w = wt(x);
        if (acc + w > thr) { found = x; lo = acc; hi = acc + w; break; }
        acc += w;
      }
    }
    if (found < 0 && lastpos >= 0) { found = lastpos; lo = hi = thr; }
    if (found >= 0) {
      int prev = atomicMin(&sh_x, found);
      if (found < prev) sh_gap = fminf(thr - lo, hi - thr) / sh_Z;
    }
  }
  __syncthreads();
  if (t == 0) {
    int x = sh_x;
    float gap = sh_gap;
    if (x == INT_MAX) { x = sh_last >= 0 ? sh_last : x0; gap = 0.f; }
    accept_len[b] = I.acc;
    bonus[b] = x;
    commit[b] = I.acc + 1;
    if (new_seq) new_seq[b] = prefix[b] + I.acc + 1;
    if (gap_out) gap_out[b] = gap;
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void k_bonus_partial(
    int B, int L, int V, int chunk, int nc, const T* __restrict__ tl, int64_t ts,
    const T* __restrict__ dl, int64_t ds, float a, int row_nc, const float2* __restrict__ part,
    const int32_t* __restrict__ toks, const int32_t* __restrict__ lens,
    const float* __restrict__ u, float* __restrict__ ratio_out, ReqInfo* __restrict__ info,
    float4* __restrict__ rpart, const float* __restrict__ draft_lse) {
  const int c = blockIdx.x % nc;
  const int b = blockIdx.x / nc;
  // every chunk's workgroup runs the (cheap) acceptance scan itself; chunk 0
  // publishes it for the selection kernel
  const ReqInfo I = accept_scan<T>(b, B, L, V, row_nc, part, tl, ts, dl, ds, toks, lens, u, a,
                                   c == 0 ? ratio_out : nullptr, draft_lse);
  if (c == 0 && threadIdx.x == 0) info[b] = I;
  if (!I.err) bonus_chunk_sum<T, VEC>(c, chunk, V, tl, ts, dl, ds, a, b, L, I, rpart);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_bonus_select(
    int L, int V, int chunk, int nc, const T* __restrict__ tl, int64_t ts,
    const T* __restrict__ dl, int64_t ds, float a, const ReqInfo* __restrict__ info,
    const float4* __restrict__ rpart, const float* __restrict__ u2,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ bonus, int32_t* __restrict__ commit,
    const int32_t* __restrict__ prefix, int32_t* __restrict__ new_seq,
    float* __restrict__ beta_out, float* __restrict__ gap_out) {
  const int b = blockIdx.x;
  select_bonus<T>(b, L, V, chunk, nc, tl, ts, dl, ds, a, info[b], rpart, u2, accept_len, bonus,
                  commit, prefix, new_seq, beta_out, gap_out);
}

// ------------------------------------------------------------- tree walk
// Greedy walk of a DDTree ([Spec tutorial], section 6.5), one wavefront per
// request: the node tables are staged in LDS; from the root, the lanes scan
// the nodes for the child of the current node whose token is the target's
// argmax at that node (row 0: the root, row 1 + j: node j), a ballot picks
// it, and the walk stops at the first node without such a child.
__global__ __launch_bounds__(64) void k_tree_walk(
    int budget, int max_depth, int nc, const float* __restrict__ pmax, const int* __restrict__ pidx,
    const int32_t* __restrict__ node_token, const int32_t* __restrict__ node_parent,
    const int32_t* __restrict__ n_nodes, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ bonus, int32_t* __restrict__ path, int32_t* __restrict__ commit,
    const int32_t* __restrict__ prefix, int32_t* __restrict__ new_seq) {
  extern __shared__ int tw[];
  int* s_tok = tw;             // [budget]
  int* s_par = tw + budget;    // [budget]
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int n = n_nodes[b];
  const bool bad = n < 0 || n > budget;
  const int N = bad ? 0 : n;
  for (int j = lane; j < N; j += 64) {
    s_tok[j] = node_token[(int64_t)b * budget + j];
    s_par[j] = node_parent[(int64_t)b * budget + j];
  }
  __syncthreads();
  // target argmax of row r: the lanes hold its chunks, ties to the lower id
  auto predict = [&](int r) {
    float v = neg_inf();
    int i = INT_MAX;
    if (lane < nc) {
      v = pmax[((int64_t)b * (budget + 1) + r) * nc + lane];
      i = pidx[((int64_t)b * (budget + 1) + r) * nc + lane];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(v, o, 64);
      const int oi = __shfl_xor(i, o, 64);
      am_merge(v, i, ov, oi);
    }
    return i == INT_MAX ? 0 : i;
  };
  int cur = -1, len = 0, want = predict(0);
  // a path holds at most N nodes (this ends the loop on any parent table);
  // the walk also stops once max_depth nodes are accepted
  while (!bad && len < N && len < max_depth) {
    int hit = INT_MAX;
    for (int j0 = 0; j0 < N; j0 += 64) {
      const int j = j0 + lane;
      const bool m = j < N && s_par[j] == cur && s_tok[j] == want;
      const uint64_t bal = __ballot(m);
      if (bal) { hit = j0 + (int)__ffsll((unsigned long long)bal) - 1; break; }
    }
    if (hit == INT_MAX) break;
    if (lane == 0) path[(int64_t)b * max_depth + len] = hit;
    ++len;
    cur = hit;
    want = predict(cur + 1);
  }
  if (lane == 0) {
    for (int d = len; d < max_depth; ++d) path[(int64_t)b * max_depth + d] = -1;
    accept_len[b] = bad ? -1 : len;
    bonus[b] = bad ? -1 : want;
    const int cm = bad ? 0 : len + 1;
    commit[b] = cm;
    if (new_seq) new_seq[b] = prefix[b] + cm;
  }
}

// ------------------------------------------------------------------- gate
// One workgroup per request: each wavefront merges the chunk partials of
// one row at a time (lane c holds chunk c, at most 64 chunks) by butterfly
// max and sum, then the request's terms are summed by the first wavefront.
__global__ __launch_bounds__(256) void k_gate_finalize(
    int B, int n, int V, int nc, const float2* __restrict__ part, const void* __restrict__ dl,
    int64_t rs, int bf16, const int32_t* __restrict__ toks, const int32_t* __restrict__ valid,
    int rows_all, float a, float g, float* __restrict__ c_out, int32_t* __restrict__ go_out,
    float* __restrict__ row_max, float* __restrict__ row_lse, int stats_ld) {
  const int b = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  __shared__ float term[64];
  bool bad;
  const int nv = chain_of(valid, b, n, &bad);
  const int nread = rows_all ? n : nv;
  for (int i = w; i < n; i += 4) {
    float tm = 0.f;
    if (i < nread) {
      const float2 pc = lane < nc ? part[(int64_t)(b * n + i) * nc + lane] : make_float2(neg_inf(), 0.f);
      const float M = wave_max(pc.x);
      const float S = wave_sum((M == neg_inf() || pc.x == neg_inf()) ? 0.f : pc.y * exp2f(pc.x - M));
      const float l2 = M + log2f(S);
      if (lane == 0) {
        if (row_max) row_max[(int64_t)b * stats_ld + i] = M * kLn2;
        if (row_lse) row_lse[(int64_t)b * stats_ld + i] = l2 * kLn2;
        if (i < nv) {
          const int x = toks[b * n + i];
          if (x < 0 || x >= V) {
            tm = __builtin_nanf("");
          } else {
            const int64_t off = (int64_t)(b * n + i) * rs + x;
            const float dx = bf16 ? bf16_to_f32(static_cast<const uint16_t*>(dl)[off])
                                  : static_cast<const float*>(dl)[off];
            tm = (dx * a - l2) * kLn2;
          }
        }
      }
    }
    if (lane == 0) term[i] = tm;
  }
  __syncthreads();
  if (w == 0) {
    float c = wave_sum(lane < nv ? term[lane] : 0.f);
    if (lane == 0) {
      if (bad) c = __builtin_nanf("");
      c_out[b] = c;
      go_out[b] = (c >= g) ? 1 : 0;
    }
  }
}

bool aligned16(const void* p, int64_t stride, int esize) {
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((stride * esize) % 16 == 0);
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <typename T, bool VEC>
void launch_argmax(RowSet s0, RowSet s1, int B, int L, int V, const int32_t* lens, VocabPlan pl,
                   int64_t rows, float* pmax, int* pidx, hipStream_t st) {
  hipLaunchKernelGGL((k_row_argmax<T, VEC>), dim3((unsigned)(rows * pl.n_chunks)), dim3(kThreads),
                     0, st, s0, s1, B, L, V, lens, pl.chunk, pl.n_chunks, pmax, pidx);
}
template <typename T, bool VEC>
void launch_lse(RowSet s0, RowSet s1, int B, int L, int V, const int32_t* lens, float a,
                VocabPlan pl, int64_t rows, float2* part, hipStream_t st) {
  hipLaunchKernelGGL((k_row_lse<T, VEC>), dim3((unsigned)(rows * pl.n_chunks)), dim3(kThreads),
                     0, st, s0, s1, B, L, V, lens, a, pl.chunk, pl.n_chunks, part);
}

template <typename T, bool VEC>
void sample_impl(int B, int L, int V, const void* tl, int64_t ts, const void* dl, int64_t ds,
                 const int32_t* toks, const int32_t* lens, const float* u, const float* u2,
                 float temperature, int32_t* acc, int32_t* bonus, int32_t* commit,
                 const int32_t* prefix, int32_t* new_seq, float* ratio_out, float* beta_out,
                 float* gap_out, const float* draft_lse, void* ws, hipStream_t st) {
  // with draft_lse only the target rows are reduced
  const int64_t rows = (int64_t)B * (draft_lse ? L + 1 : 2 * L + 1);
  const VocabPlan pl = plan_vocab(rows, V);
  const VocabPlan pr = plan_vocab(2 * (int64_t)B, V);
  char* w = static_cast<char*>(ws);
  float2* part = reinterpret_cast<float2*>(w);
  {
    const int64_t ar = (int64_t)B * (2 * L + 1), tr = (int64_t)B * (L + 1);
    w += align256(sizeof(float2) * std::max(ar * plan_vocab(ar, V).n_chunks,
                                            tr * plan_vocab(tr, V).n_chunks));
  }
  ReqInfo* info = reinterpret_cast<ReqInfo*>(w);
  w += align256(sizeof(ReqInfo) * B);
  float4* rpart = reinterpret_cast<float4*>(w);
  const float a = kLog2e / temperature;
  RowSet s0{tl, ts, L + 1, 1}, s1{dl, ds, draft_lse ? 0 : L, 0};
  launch_lse<T, VEC>(s0, s1, B, L, V, lens, a, pl, rows, part, st);
  hipLaunchKernelGGL((k_bonus_partial<T, VEC>), dim3(B * pr.n_chunks), dim3(kThreads), 0, st, B,
                     L, V, pr.chunk, pr.n_chunks, static_cast<const T*>(tl), ts,
                     static_cast<const T*>(dl), ds, a, pl.n_chunks, part, toks, lens, u, ratio_out,
                     info, rpart, draft_lse);
  hipLaunchKernelGGL((k_bonus_select<T>), dim3(B), dim3(kThreads), 0, st, L, V, pr.chunk,
                     pr.n_chunks, static_cast<const T*>(tl), ts, static_cast<const T*>(dl), ds, a,
                     info, rpart, u2, acc, bonus, commit, prefix, new_seq, beta_out, gap_out);
}

}  // namespace

VocabPlan plan_vocab(int64_t n_rows, int V) {
  // About DFLASH_VOCAB_WGS workgroups per launch, chunks of at least 2048 elements, at
  // most kMaxChunks chunks per row; chunk boundaries are multiples of 8 so
  // that 16-byte loads stay aligned.
  const int64_t rows = n_rows > 0 ? n_rows : 1;
  const int64_t want = std::max<int64_t>(1, cdiv(DFLASH_VOCAB_WGS, rows));
  int64_t chunk = std::max<int64_t>(cdiv(V, want), 2048);
  chunk = cdiv(chunk, 8) * 8;
  int64_t n = cdiv(V, chunk);
  if (n > kMaxChunks) {
    chunk = cdiv(cdiv(V, kMaxChunks), 8) * 8;
    n = cdiv(V, chunk);
  }
  return VocabPlan{(int)chunk, (int)std::max<int64_t>(n, 1)};
}

size_t greedy_ws_bytes(int B, int L, int V) {
  const int64_t rows = (int64_t)B * (2 * L + 1);
  const VocabPlan pl = plan_vocab(rows, V);
  return align256(sizeof(float) * rows * pl.n_chunks) + align256(sizeof(int) * rows * pl.n_chunks);
}

size_t sample_ws_bytes(int B, int L, int V) {
  // partials of all 2L+1 rows, or of the L+1 target rows alone (finer chunks)
  const int64_t rows = (int64_t)B * (2 * L + 1), trows = (int64_t)B * (L + 1);
  const int64_t np = std::max(rows * plan_vocab(rows, V).n_chunks,
                              trows * plan_vocab(trows, V).n_chunks);
  const VocabPlan pr = plan_vocab(2 * (int64_t)B, V);
  return align256(sizeof(float2) * np) + align256(sizeof(ReqInfo) * B) +
         align256(sizeof(float4) * B * pr.n_chunks);
}

size_t gate_ws_bytes(int B, int n, int V) {
  const int64_t rows = (int64_t)B * n;
  const VocabPlan pl = plan_vocab(rows, V);
  return align256(sizeof(float2) * rows * pl.n_chunks);
}

hipError_t launch_verify_greedy(bool bf16, int B, int L, int V, const void* tl, int64_t ts,
                                const void* dl, int64_t ds, int32_t* draft_tokens,
                                const int32_t* lens, int32_t* target_predict, int32_t* accept_len,
                                int32_t* bonus, int32_t* commit, const int32_t* prefix,
                                int32_t* new_seq, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)B * ((L + 1) + (dl ? L : 0));
  const VocabPlan pl = plan_vocab((int64_t)B * (2 * L + 1), V);
  float* pmax = static_cast<float*>(ws);
  int* pidx = reinterpret_cast<int*>(static_cast<char*>(ws) +
                                     align256(sizeof(float) * (int64_t)B * (2 * L + 1) * pl.n_chunks));
  const int es = bf16 ? 2 : 4;
  const bool vec = aligned16(tl, ts, es) && (!dl || aligned16(dl, ds, es));
  RowSet s0{tl, ts, L + 1, 1}, s1{dl, ds, dl ? L : 0, 0};
  if (bf16) {
    if (vec) launch_argmax<uint16_t, true>(s0, s1, B, L, V, lens, pl, rows, pmax, pidx, st);
    else launch_argmax<uint16_t, false>(s0, s1, B, L, V, lens, pl, rows, pmax, pidx, st);
  } else {
    if (vec) launch_argmax<float, true>(s0, s1, B, L, V, lens, pl, rows, pmax, pidx, st);
    else launch_argmax<float, false>(s0, s1, B, L, V, lens, pl, rows, pmax, pidx, st);
  }
  hipLaunchKernelGGL(k_greedy_finalize, dim3(B), dim3(128), 0, st, B, L, V, pl.n_chunks, pmax,
                     pidx, dl ? 1 : 0, draft_tokens, lens, target_predict, accept_len, bonus,
                     commit, prefix, new_seq);
  return hipGetLastError();
}

// ---------------------------------------------- static scratch (no allocation)
// The greedy pass's chunk partials for dflash_verify_greedy_noalloc, in place
// of a caller workspace.  Each GPU the library runs on holds its own copy
// until the process ends, and every call on that GPU shares it.  In host code
// `scratch` names a host-side stand-in, never the device memory: its device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in scratch_ptr below; only that address is ever
// handed to a kernel.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_verify_sample(bool bf16, int B, int L, int V, const void* tl, int64_t ts,
                                const void* dl, int64_t ds, const int32_t* toks,
                                const int32_t* lens, const float* u, const float* u2,
                                float temperature, int32_t* acc, int32_t* bonus, int32_t* commit,
                                const int32_t* prefix, int32_t* new_seq, float* ratio_out,
                                float* beta_out, float* gap_out, const float* draft_lse, void* ws,
                                hipStream_t st) {
  const int es = bf16 ? 2 : 4;
  const bool vec = aligned16(tl, ts, es) && aligned16(dl, ds, es);
  if (bf16) {
    if (vec) sample_impl<uint16_t, true>(B, L, V, tl, ts, dl, ds, toks, lens, u, u2, temperature, acc, bonus, commit, prefix, new_seq, ratio_out, beta_out, gap_out, draft_lse, ws, st);
    else sample_impl<uint16_t, false>(B, L, V, tl, ts, dl, ds, toks, lens, u, u2, temperature, acc, bonus, commit, prefix, new_seq, ratio_out, beta_out, gap_out, draft_lse, ws, st);
  } else {
    if (vec) sample_impl<float, true>(B, L, V, tl, ts, dl, ds, toks, lens, u, u2, temperature, acc, bonus, commit, prefix, new_seq, ratio_out, beta_out, gap_out, draft_lse, ws, st);
    else sample_impl<float, false>(B, L, V, tl, ts, dl, ds, toks, lens, u, u2, temperature, acc, bonus, commit, prefix, new_seq, ratio_out, beta_out, gap_out, draft_lse, ws, st);
  }
  return hipGetLastError();
}

size_t tree_verify_ws_bytes(int B, int budget, int V) {
  const int64_t rows = (int64_t)B * (budget + 1);
  const VocabPlan pl = plan_vocab(rows, V);
  return align256(sizeof(float) * rows * pl.n_chunks) + align256(sizeof(int) * rows * pl.n_chunks);
}

hipError_t launch_tree_verify(bool bf16, int B, int budget, int V, const void* tl, int64_t ts,
                              const int32_t* node_token, const int32_t* node_parent,
                              const int32_t* n_nodes, int max_depth, int32_t* accept_len,
                              int32_t* bonus, int32_t* path, int32_t* commit,
                              const int32_t* prefix, int32_t* new_seq, void* ws, hipStream_t st) {
  // rows 0 .. n_nodes[b] of request b: the root and its nodes (the row set's
  // chain lengths are the node counts, one extra row)
  const int64_t rows = (int64_t)B * (budget + 1);
  const VocabPlan pl = plan_vocab(rows, V);
  float* pmax = static_cast<float*>(ws);
  int* pidx = reinterpret_cast<int*>(static_cast<char*>(ws) + align256(sizeof(float) * rows * pl.n_chunks));
  const int es = bf16 ? 2 : 4;
  const bool vec = aligned16(tl, ts, es);
  RowSet s0{tl, ts, budget + 1, 1}, s1{tl, ts, 0, 0};
  if (bf16) {
    if (vec) launch_argmax<uint16_t, true>(s0, s1, B, budget, V, n_nodes, pl, rows, pmax, pidx, st);
    else launch_argmax<uint16_t, false>(s0, s1, B, budget, V, n_nodes, pl, rows, pmax, pidx, st);
  } else {
    if (vec) launch_argmax<float, true>(s0, s1, B, budget, V, n_nodes, pl, rows, pmax, pidx, st);
    else launch_argmax<float, false>(s0, s1, B, budget, V, n_nodes, pl, rows, pmax, pidx, st);
  }
  hipLaunchKernelGGL(k_tree_walk, dim3(B), dim3(64), sizeof(int) * 2 * budget, st, budget,
                     max_depth, pl.n_chunks, pmax, pidx, node_token, node_parent, n_nodes,
                     accept_len, bonus, path, commit, prefix, new_seq);
  return hipGetLastError();
}

hipError_t launch_gate(bool bf16, int B, int n, int V, const void* dl, int64_t rs,
                       const int32_t* toks, const int32_t* valid, float temperature, float g,
                       float* c_out, int32_t* go_out, float* row_max, float* row_lse,
                       int stats_ld, void* ws, hipStream_t st) {
  const int64_t rows = (int64_t)B * n;
  const VocabPlan pl = plan_vocab(rows, V);
  float2* part = static_cast<float2*>(ws);
  const float a = kLog2e / temperature;
  const bool rows_all = (row_max != nullptr) || (row_lse != nullptr);
  const int32_t* lens = rows_all ? nullptr : valid;
  RowSet s0{dl, rs, n, 0}, s1{dl, rs, 0, 0};
  const int es = bf16 ? 2 : 4;
  const bool vec = aligned16(dl, rs, es);
  if (bf16) {
    if (vec) launch_lse<uint16_t, true>(s0, s1, B, n, V, lens, a, pl, rows, part, st);
    else launch_lse<uint16_t, false>(s0, s1, B, n, V, lens, a, pl, rows, part, st);
  } else {
    if (vec) launch_lse<float, true>(s0, s1, B, n, V, lens, a, pl, rows, part, st);
    else launch_lse<float, false>(s0, s1, B, n, V, lens, a, pl, rows, part, st);
  }
  hipLaunchKernelGGL(k_gate_finalize, dim3(B), dim3(256), 0, st, B, n, V, pl.n_chunks, part, dl, rs,
                     bf16 ? 1 : 0, toks, valid, rows_all ? 1 : 0, a, g, c_out, go_out, row_max,
                     row_lse, stats_ld);
  return hipGetLastError();
}

}  // namespace dflash
