// The rest of the drafter around block attention: [DFlash overview], section
// "草稿模型架构" -- a small Qwen3-style decoder that shares the target's
// embedding table and lm_head; its block is the anchor followed by mask
// tokens, and each layer's attention sees the injected target context.
//
// One layer is nine launches on the caller's stream (eight when the gate/up
// product splits its contraction: SiLU then rides on its reduction), every
// intermediate in the caller's workspace:
//   RMSNorm -> QKV GEMM -> q/k head norm + rotary embedding (v copied out)
//   -> block attention over [context; block] -> O GEMM + residual (in place)
//   -> RMSNorm -> gate/up GEMM -> SiLU(gate) * up -> down GEMM + residual.
// The GEMMs are the materialisation GEMM kernel (MFMA, LDS-DMA fed) in its
// dense mode, with the residual added to the rounded product in the store.
// The element-wise kernels are HBM-bound one-pass kernels over 16-byte
// vectors.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

__device__ __forceinline__ void ld8(const uint16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_lo(w[j]); v[2 * j + 1] = bf16_hi(w[j]); }
}
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const f32x4v a = reinterpret_cast<const f32x4v*>(p)[0], b = reinterpret_cast<const f32x4v*>(p)[1];
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
}
__device__ __forceinline__ void st8(uint16_t* p, const float (&v)[8]) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
  *reinterpret_cast<u32x4*>(p) = o;
}
__device__ __forceinline__ void st8(float* p, const float (&v)[8]) {
  reinterpret_cast<f32x4v*>(p)[0] = f32x4v{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4v*>(p)[1] = f32x4v{v[4], v[5], v[6], v[7]};
}

// RMSNorm of rows [M, d]: one wavefront per row, two passes over the row
// (the second from cache): y = x / sqrt(mean(x^2) + eps) * w.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(int M, int d, const T* __restrict__ x,
                                                 const T* __restrict__ w, float eps,
                                                 T* __restrict__ y) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= M) return;
  const T* xr = x + (int64_t)row * d;
  float ss = 0.f;
  for (int c = lane * 8; c < d; c += 512) {
    float v[8];
    ld8(xr + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / d + eps);
  for (int c = lane * 8; c < d; c += 512) {
    float v[8], g[8];
    ld8(xr + c, v);
    ld8(w + c, g);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = v[j] * r * g[j];
    st8(y + (int64_t)row * d + c, v);
  }
}

// The same with one workgroup per row, for rows of at most 2048 * NC
// elements: each lane keeps its NC vectors of 8 in registers between the sum
// of squares (wavefront sums, then the four combined through LDS) and the
// scaling, so the row is read once and every row's loads are in flight at
// once.  Few rows (a small batch) then take one load round, not d / 512.
template <typename T, int NC>
__global__ __launch_bounds__(256) void k_rmsnorm_row(int M, int d, const T* __restrict__ x,
                                                     const T* __restrict__ w, float eps,
                                                     T* __restrict__ y) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  const T* xr = x + (int64_t)row * d;
  float v[NC][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = (threadIdx.x + 256 * c) * 8;
    if (i < d) {
      ld8(xr + i, v[c]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[c][j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss = fmaf(v[c][j], v[c][j], ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  ss = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.f / sqrtf(ss / d + eps);
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int i = (threadIdx.x + 256 * c) * 8;
    if (i < d) {
      float g[8];
      ld8(w + i, g);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[c][j] = v[c][j] * r * g[j];
      st8(y + (int64_t)row * d + i, v[c]);
    }
  }
}

// q / k / v out of the fused projection [M, (Hq + 2 Hkv) D]: per-head RMSNorm
// of q and k (when a weight is given), then the half-split rotary embedding
// at the row's position ctx_lens[row / k] + row % k; v is copied.  A group of
// D/8 lanes owns one (row, head), 8 dims per lane; the rotation partner of
// dim i sits D/16 lanes away.  Angles: revolutions = pos * theta^(-2i/D) /
// (2 pi) reduced in double precision (fractional part kept), then the
// hardware sine and cosine, whose argument is in revolutions.
struct QkvP {
  int M, k, Hq, Hkv, D;
  const void* qkv;
  const void* qn;   // [D] or null
  const void* kn;   // [D] or null
  float eps;
  int rope;
  double l2theta;
  const int32_t* ctx;
  void* q;          // [M, Hq, D]
  void* kb;         // [M, Hkv, D]
  void* vb;         // [M, Hkv, D]
};

template <typename T>
__global__ __launch_bounds__(256) void k_qkv_split(QkvP p) {
  __shared__ double rev_rate[64];
  const int half = p.D / 2;
  for (int i = threadIdx.x; i < half; i += 256)
    rev_rate[i] = exp2(-(2.0 * i / p.D) * p.l2theta) * 0.15915494309189535;
  __syncthreads();
  const int G = p.D / 8;
  const int H = p.Hq + 2 * p.Hkv;
  const int64_t items = (int64_t)p.M * H;
  const int lane = threadIdx.x;
  const int lig = lane % G;
  const bool first = lig < G / 2;
  for (int64_t base = (int64_t)blockIdx.x * (256 / G); base < items; base += (int64_t)gridDim.x * (256 / G)) {
    const int64_t it = base + lane / G;
    const bool live = it < items;
    const int64_t row = live ? it / H : 0;
    const int h = live ? (int)(it - row * H) : 0;
    const int kind = h < p.Hq ? 0 : (h < p.Hq + p.Hkv ? 1 : 2);   // q, k, v
    float v[8];
    ld8(static_cast<const T*>(p.qkv) + (row * H + h) * p.D + 8 * lig, v);
    const void* nw = kind == 0 ? p.qn : (kind == 1 ? p.kn : nullptr);
    if (kind < 2 && nw) {   // uniform per group
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) ss = fmaf(v[j], v[j], ss);
      for (int o = 1; o < G; o <<= 1) ss += __shfl_xor(ss, o, 64);
      const float r = 1.f / sqrtf(ss / p.D + p.eps);
      float g[8];
      ld8(static_cast<const T*>(nw) + 8 * lig, g);
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * r * g[j];
    }
    if (kind < 2 && p.rope) {
      const int pos = p.ctx[row / p.k] + (int)(row % p.k);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pr = __shfl_xor(v[j], G / 2, 64);
        double rev = (double)pos * rev_rate[8 * (lig % (G / 2)) + j];
        rev -= floor(rev);
        const float sn = __builtin_amdgcn_sinf((float)rev), cs = __builtin_amdgcn_cosf((float)rev);
        v[j] = first ? v[j] * cs - pr * sn : v[j] * cs + pr * sn;
      }
    }
    if (live) {
      T* dst;
      if (kind == 0) dst = static_cast<T*>(p.q) + (row * p.Hq + h) * p.D;
      else if (kind == 1) dst = static_cast<T*>(p.kb) + (row * p.Hkv + (h - p.Hq)) * p.D;
      else dst = static_cast<T*>(p.vb) + (row * p.Hkv + (h - p.Hq - p.Hkv)) * p.D;
      st8(dst + 8 * lig, v);
    }
  }
}

// h[M, I] = silu(gu[:, :I]) * gu[:, I:], 8 columns per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_silu_mul(int M, int I, const T* __restrict__ gu,
                                                  T* __restrict__ h) {
  const int i8 = I / 8;
  const int64_t total = (int64_t)M * i8;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t row = e / i8;
    const int c = (int)(e - row * i8) * 8;
    float g[8], u[8];
    ld8(gu + row * 2 * I + c, g);
    ld8(gu + row * 2 * I + I + c, u);
#pragma unroll
    for (int j = 0; j < 8; ++j) g[j] = g[j] / (1.f + __expf(-g[j])) * u[j];
    st8(h + row * I + c, g);
  }
}

// out[r] = table[tokens[r]]; a token outside [0, V) gives a NaN row.
template <typename T>
__global__ __launch_bounds__(256) void k_embed(int M, int d, int V, const T* __restrict__ table,
                                               const int32_t* __restrict__ tok, T* __restrict__ out) {
  const int d8 = d / 8;
  const int64_t total = (int64_t)M * d8;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t row = e / d8;
    const int c = (int)(e - row * d8) * 8;
    const int t = tok[row];
    float v[8];
    if (t >= 0 && t < V) {
      ld8(table + (int64_t)t * d + c, v);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __builtin_nanf("");
    }
    st8(out + row * d + c, v);
  }
}

unsigned grid_for(int64_t threads) {
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(cdiv(threads, 256), 8192));
}

template <typename T>
void rmsnorm(int M, int d, const void* x, const void* w, float eps, void* y, hipStream_t st) {
  const T* xt = static_cast<const T*>(x);
  const T* wt = static_cast<const T*>(w);
  T* yt = static_cast<T*>(y);
  if (M <= 0) return;
  if (d <= 2048)
    hipLaunchKernelGGL((k_rmsnorm_row<T, 1>), dim3((unsigned)M), dim3(256), 0, st, M, d, xt, wt, eps, yt);
  else if (d <= 4096)
    hipLaunchKernelGGL((k_rmsnorm_row<T, 2>), dim3((unsigned)M), dim3(256), 0, st, M, d, xt, wt, eps, yt);
  else if (d <= 8192)
    hipLaunchKernelGGL((k_rmsnorm_row<T, 4>), dim3((unsigned)M), dim3(256), 0, st, M, d, xt, wt, eps, yt);
  else
    hipLaunchKernelGGL(k_rmsnorm<T>, dim3((unsigned)cdiv(M, 4)), dim3(256), 0, st, M, d, xt, wt, eps, yt);
}

struct LayerWs {
  size_t xn, qkv, q, kb, vb, attn, gu, h, gemm, attn_ws, total;
};

LayerWs layer_ws(const DraftArgs& a) {
  const int64_t es = a.bf16 ? 2 : 4;
  const int64_t M = (int64_t)a.B * a.k;
  const int64_t QKV = (int64_t)(a.Hq + 2 * a.Hkv) * a.D;
  LayerWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o += align256(bytes); return at; };
  w.xn = take(M * a.d * es);
  w.qkv = take(M * QKV * es);
  w.q = take(M * a.Hq * a.D * es);
  w.kb = take(M * a.Hkv * a.D * es);
  w.vb = take(M * a.Hkv * a.D * es);
  w.attn = take(M * a.Hq * a.D * es);
  w.gu = take(M * 2 * a.I * es);
  w.h = take(M * a.I * es);
  const size_t g = std::max({dense_gemm_ws_bytes(M, QKV, a.d, a.bf16),
                             dense_gemm_ws_bytes(M, a.d, (int64_t)a.Hq * a.D, a.bf16),
                             dense_gemm_ws_bytes(M, 2LL * a.I, a.d, a.bf16),
                             dense_gemm_ws_bytes(M, a.d, a.I, a.bf16)});
  w.gemm = take(std::max<size_t>(g, 256));
  const size_t aw = a.bf16 ? attention_ws_bytes(a.B, a.k, a.Hq, a.Hkv, a.D, a.max_pages, true) : 0;
  w.attn_ws = take(std::max<size_t>(aw, 256));
  w.total = o;
  return w;
}

template <typename T>
hipError_t layer_impl(const DraftArgs& a, void* ws, hipStream_t st) {
  const LayerWs L = layer_ws(a);
  char* w = static_cast<char*>(ws);
  const int M = a.B * a.k;
  const int QKV = (a.Hq + 2 * a.Hkv) * a.D;
  void* xn = w + L.xn;
  void* qkv = w + L.qkv;
  void* q = w + L.q;
  void* kb = w + L.kb;
  void* vb = w + L.vb;
  void* attn = w + L.attn;
  void* gu = w + L.gu;
  void* h = w + L.h;
  void* gw = w + L.gemm;
  hipError_t e;
  rmsnorm<T>(M, a.d, a.x, a.ln1, a.eps, xn, st);
  if ((e = launch_dense_gemm(a.bf16, M, QKV, a.d, xn, a.w_qkv, nullptr, nullptr, qkv, gw, st))) return e;
  QkvP qp{M, a.k, a.Hq, a.Hkv, a.D, qkv, a.q_norm, a.k_norm, a.eps, a.rope_theta > 0.f ? 1 : 0,
          a.rope_theta > 0.f ? std::log2((double)a.rope_theta) : 0.0, a.ctx_lens, q, kb, vb};
  hipLaunchKernelGGL(k_qkv_split<T>, dim3(grid_for((int64_t)M * (a.Hq + 2 * a.Hkv) * (a.D / 8))),
                     dim3(256), 0, st, qp);
  AttnArgs aa{a.B, a.k, a.Hq, a.Hkv, a.D, q, kb, vb, a.cache_k, a.cache_v, a.num_pages,
              a.block_table, a.max_pages, false, a.ctx_lens, 0.f, a.causal ? kMaskCausal : kMaskBidir,
              nullptr, attn, nullptr, false};
  if ((e = launch_attention(a.bf16, aa, w + L.attn_ws, st))) return e;
  if ((e = launch_dense_gemm(a.bf16, M, a.d, a.Hq * a.D, attn, a.w_o, nullptr, a.x, a.x, gw, st))) return e;
  rmsnorm<T>(M, a.d, a.x, a.ln2, a.eps, xn, st);
  if (dense_gemm_splits(M, 2 * a.I, a.d, a.bf16)) {   // few rows: SiLU in the split reduction
    if ((e = launch_dense_gemm_silu(a.bf16, M, a.I, a.d, xn, a.w_gate_up, h, gw, st))) return e;
  } else {
    if ((e = launch_dense_gemm(a.bf16, M, 2 * a.I, a.d, xn, a.w_gate_up, nullptr, nullptr, gu, gw, st))) return e;
    hipLaunchKernelGGL(k_silu_mul<T>, dim3(grid_for((int64_t)M * a.I / 8)), dim3(256), 0, st, M, a.I,
                       static_cast<const T*>(gu), static_cast<T*>(h));
  }
  if ((e = launch_dense_gemm(a.bf16, M, a.d, a.I, h, a.w_down, nullptr, a.x, a.x, gw, st))) return e;
  return hipGetLastError();
}

}  // namespace

size_t draft_layer_ws_bytes(const DraftArgs& a) { return layer_ws(a).total; }

hipError_t launch_draft_layer(const DraftArgs& a, void* ws, hipStream_t st) {
  return a.bf16 ? layer_impl<uint16_t>(a, ws, st) : layer_impl<float>(a, ws, st);
}

size_t draft_head_ws_bytes(int M, int d, int V, bool bf16) {
  const int64_t es = bf16 ? 2 : 4;
  return align256((size_t)M * d * es) + align256(std::max<size_t>(dense_gemm_ws_bytes(M, V, d, bf16), 256));
}

hipError_t launch_draft_head(bool bf16, int M, int d, int V, const void* x, const void* norm_w,
                             const void* lm_head, float eps, void* logits, void* ws, hipStream_t st) {
  const int64_t es = bf16 ? 2 : 4;
  char* w = static_cast<char*>(ws);
  void* xn = w;
  void* gw = w + align256((size_t)M * d * es);
  if (bf16) rmsnorm<uint16_t>(M, d, x, norm_w, eps, xn, st);
  else rmsnorm<float>(M, d, x, norm_w, eps, xn, st);
  return launch_dense_gemm(bf16, M, V, d, xn, lm_head, nullptr, nullptr, logits, gw, st);
}

hipError_t launch_embed(bool bf16, int M, int d, int V, const void* table, const int32_t* tokens,
                        void* out, hipStream_t st) {
  const unsigned g = grid_for((int64_t)M * d / 8);
  if (bf16)
    hipLaunchKernelGGL(k_embed<uint16_t>, dim3(g), dim3(256), 0, st, M, d, V,
                       static_cast<const uint16_t*>(table), tokens, static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(k_embed<float>, dim3(g), dim3(256), 0, st, M, d, V,
                       static_cast<const float*>(table), tokens, static_cast<float*>(out));
  return hipGetLastError();
}

}  // namespace dflash
