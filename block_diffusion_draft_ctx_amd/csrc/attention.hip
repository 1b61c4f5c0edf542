// Non-causal block attention over injected context K/V.
//
// [DFlash overview], section "KV 注入" (the Attention formula): a draft
// query attends to [K_ctx; K_blk] and [V_ctx; V_blk]; section "块扩散": no
// causal mask inside the block; section "随机锚点采样": packed training blocks
// see the context before their anchor and only their own block (expressed by
// the caller through the block table and ctx_lens).
//
// bf16 design (gfx950, wave64).  One workgroup owns one (request, kv-head,
// ctx-split).  Its G*k query rows (the G q-heads that share the kv-head, times
// the k block positions) are split into 16-row slices, one per wavefront, so
// every K/V byte streamed from HBM is used by all G q-heads.  Keys are
// processed 32 at a time: the tile's K rows and V rows are fetched with
// 16-byte loads (the next tile's loads are issued before the current tile is
// computed), K is stored row-major and V transposed in LDS, and each
// wavefront runs
//   S^T[32 keys x 16 q] = K . Q^T        2 x (D/32) MFMA 16x16x32 bf16
//   online softmax per query column      (4-lane shuffles, exp2 domain)
//   O^T[D x 16 q]      += V^T . P^T      (D/16) MFMA 16x16x32 bf16
// so that a lane's accumulators all belong to one query and rescale with one
// factor.  Small batches split the context across workgroups and a second
// kernel merges the splits by their log-sum-exp.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kKT = 32;  // keys per tile

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

struct AttnP {
  int B, k, Hq, Hkv;
  const uint16_t* q;
  const uint16_t* kb;
  const uint16_t* vb;
  const uint16_t* ck;
  const uint16_t* cv;
  int num_pages;
  const int32_t* bt;
  int max_pages;
  const int32_t* ctx;
  float sl2;  // softmax scale * log2(e)
  void* out;  // bf16 or fp32 (out_f32)
  int out_f32;
  float* lse;
  float* po;    // split partials: O [B*Hkv*S*Mq, D] fp32
  float2* pml;  // split partials: (m, l) [B*Hkv*S*Mq]
  int S;        // ctx splits
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn_bf16(AttnP p) {
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;             // 16-byte chunks per key row
  constexpr int NCH = kKT * CPR;         // chunks per tile
  constexpr int CPT = (NCH + NT - 1) / NT;
  constexpr int KS = D + 8;              // LDS row stride of K (elements)
  constexpr int VS = kKT + 8;            // LDS row stride of V^T
  constexpr int NB = D / 16;
  __shared__ __align__(16) uint16_t Ks[kKT * KS];
  __shared__ __align__(16) uint16_t Vt[D * VS];

  const int split = blockIdx.x % p.S;
  const int g = (blockIdx.x / p.S) % p.Hkv;
  const int b = blockIdx.x / (p.S * p.Hkv);
  const int G = p.Hq / p.Hkv;
  const int k = p.k;
  const int Mq = G * k;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int c16 = lane & 15;   // column (query) of B/C; row of A
  const int grp = lane >> 4;
  const int qrow = w * 16 + c16;
  const bool qvalid = qrow < Mq;
  const int hg = qvalid ? qrow / k : 0;
  const int pos = qvalid ? qrow - hg * k : 0;
  const int h = g * G + hg;

  bf16x8 qf[D / 32];
  {
    const uint16_t* qp = p.q + (((int64_t)b * k + pos) * p.Hq + h) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qp + 32 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = as_bf16x8(v);
    }
  }

  int C = p.ctx[b];
  bool poison = (C < 0 || C > p.max_pages * 16);
  if (poison) C = 0;
  const int total = C + k;
  const int nt = (total + kKT - 1) / kKT;
  const int tps = (nt + p.S - 1) / p.S;
  const int t0 = split * tps;
  const int t1 = min(nt, t0 + tps);
  const int32_t* btr = p.bt + (int64_t)b * p.max_pages;

  uint4 kr[CPT], vr[CPT];
  auto fetch = [&](int tile) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e = threadIdx.x + c * NT;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (e < NCH) {
        const int key = e / CPR;
        const int dc = e - key * CPR;
        const int kp = tile * kKT + key;
        if (kp < C) {
          const int page = btr[kp >> 4];
          if (page < 0 || page >= p.num_pages) {
            poison = true;
          } else {
            const int64_t off = (((int64_t)page * 16 + (kp & 15)) * p.Hkv + g) * D + dc * 8;
            kv = ld_stream16(p.ck + off);
            vv = ld_stream16(p.cv + off);
          }
        } else if (kp < total) {
          const int64_t off = (((int64_t)b * k + (kp - C)) * p.Hkv + g) * D + dc * 8;
          kv = *reinterpret_cast<const uint4*>(p.kb + off);
          vv = *reinterpret_cast<const uint4*>(p.vb + off);
        }
      }
      kr[c] = kv;
      vr[c] = vv;
    }
  };

  float m = neg_inf(), l = 0.f;
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (t0 < t1) fetch(t0);
  for (int tile = t0; tile < t1; ++tile) {
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e = threadIdx.x + c * NT;
      if (e < NCH) {
        const int key = e / CPR;
        const int dc = e - key * CPR;
        *reinterpret_cast<uint4*>(Ks + key * KS + dc * 8) = kr[c];
        const uint32_t vw[4] = {vr[c].x, vr[c].y, vr[c].z, vr[c].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Vt[(dc * 8 + 2 * j) * VS + key] = (uint16_t)(vw[j] & 0xffffu);
          Vt[(dc * 8 + 2 * j + 1) * VS + key] = (uint16_t)(vw[j] >> 16);
        }
      }
    }
    __syncthreads();
    if (tile + 1 < t1) fetch(tile + 1);

    // S^T = K . Q^T for 32 keys (two 16-key blocks)
    f32x4 sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      sacc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        const uint4 a = *reinterpret_cast<const uint4*>(Ks + (16 * mb + c16) * KS + 32 * s + 8 * grp);
        sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), qf[s], sacc[mb], 0, 0, 0);
      }
    }
    // scores of query c16 for keys tile*32 + 16*mb + 4*grp + r
    float sv[8];
    float tmax = neg_inf();
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = tile * kKT + 16 * mb + 4 * grp + r;
        const float v = (kk < total) ? sacc[mb][r] * p.sl2 : neg_inf();
        sv[mb * 4 + r] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mn = fmaxf(m, tmax);
    const float alpha = exp2f(m - mn);
    float ps[8];
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ps[j] = exp2f(sv[j] - mn);
      rs += ps[j];
    }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    l = l * alpha + rs;
    m = mn;
    const uint4 pw = make_uint4(pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3]),
                                pack_bf16x2(ps[4], ps[5]), pack_bf16x2(ps[6], ps[7]));
    const bf16x8 pb = as_bf16x8(pw);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[nb] *= alpha;
      const uint16_t* vrow = Vt + (16 * nb + c16) * VS + 4 * grp;
      const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
      const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
      const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[nb], 0, 0, 0);
    }
  }

  if (p.S == 1) {
    if (qvalid) {
      const float inv = poison ? __builtin_nanf("") : 1.f / l;
      const int64_t o0 = (((int64_t)b * k + pos) * p.Hq + h) * D + 4 * grp;
      if (p.out_f32) {
        float* op = static_cast<float*>(p.out) + o0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          *reinterpret_cast<float4*>(op + 16 * nb) =
              make_float4(acc[nb][0] * inv, acc[nb][1] * inv, acc[nb][2] * inv, acc[nb][3] * inv);
      } else {
        uint16_t* op = static_cast<uint16_t*>(p.out) + o0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          uint2 o;
          o.x = pack_bf16x2(acc[nb][0] * inv, acc[nb][1] * inv);
          o.y = pack_bf16x2(acc[nb][2] * inv, acc[nb][3] * inv);
          *reinterpret_cast<uint2*>(op + 16 * nb) = o;
        }
      }
      if (p.lse && grp == 0)
        p.lse[((int64_t)b * p.Hq + h) * k + pos] = poison ? __builtin_nanf("") : (m + log2f(l)) * kLn2;
    }
  } else {
    const int64_t rowi = (((int64_t)b * p.Hkv + g) * p.S + split) * Mq + qrow;
    if (qvalid) {
      float* op = p.po + rowi * D + 4 * grp;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<float4*>(op + 16 * nb) = make_float4(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3]);
      if (grp == 0) p.pml[rowi] = make_float2(m, poison ? __builtin_nanf("") : l);
    }
  }
}

template <typename OutT>
__global__ __launch_bounds__(256) void k_attn_combine(int B, int k, int Hq, int Hkv, int D, int S,
                                                     const float* __restrict__ po,
                                                     const float2* __restrict__ pml,
                                                     OutT* __restrict__ out, float* __restrict__ lse) {
  const int bg = blockIdx.x;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int G = Hq / Hkv;
  const int Mq = G * k;
  for (int e = threadIdx.x; e < Mq * D; e += blockDim.x) {
    const int qrow = e / D, d = e - qrow * D;
    const int64_t base = (int64_t)bg * S * Mq + qrow;
    float M = neg_inf();
    for (int s = 0; s < S; ++s) M = fmaxf(M, pml[base + (int64_t)s * Mq].x);
    float Ls = 0.f, O = 0.f;
    for (int s = 0; s < S; ++s) {
      const float2 ml = pml[base + (int64_t)s * Mq];
      if (ml.x == neg_inf() && ml.y == 0.f) continue;  // an empty split
      const float wgt = exp2f(ml.x - M);
      Ls += ml.y * wgt;
      O += po[(base + (int64_t)s * Mq) * D + d] * wgt;
    }
    const int hg = qrow / k, pos = qrow - hg * k, h = g * G + hg;
    const float v = O / Ls;
    const int64_t oi = (((int64_t)b * k + pos) * Hq + h) * D + d;
    if constexpr (sizeof(OutT) == 2) out[oi] = f32_to_bf16(v);
    else out[oi] = v;
    if (lse && d == 0) lse[((int64_t)b * Hq + h) * k + pos] = (M + log2f(Ls)) * kLn2;
  }
}

// fp32 path: a plain kernel for small fp32 workloads.  One workgroup of 64
// lanes per (request, q-head, block position); each lane keeps an online
// softmax over its share of the keys, then the 64 partial states are merged
// through LDS.
template <int D>
__global__ __launch_bounds__(64) void k_attn_f32(int B, int k, int Hq, int Hkv, const float* q,
                                                 const float* kb, const float* vb,
                                                 const float* ck, const float* cv, int num_pages,
                                                 const int32_t* bt, int max_pages,
                                                 const int32_t* ctx, float sl2, float* out,
                                                 float* lse, int S, float* po, float2* pml) {
  const int i = blockIdx.x % k;
  const int h = (blockIdx.x / k) % Hq;
  const int b = blockIdx.x / (k * Hq);
  const int G = Hq / Hkv, g = h / G;
  const int t = threadIdx.x;
  __shared__ float qs[D];
  __shared__ float red[64 * (D + 2)];
  for (int d = t; d < D; d += 64) qs[d] = q[(((int64_t)b * k + i) * Hq + h) * D + d];
  __syncthreads();
  int C = ctx[b];
  bool poison = (C < 0 || C > max_pages * 16);
  if (poison) C = 0;
  const int total = C + k;
  float m = neg_inf(), l = 0.f, o[D];
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  for (int j = t; j < total; j += 64) {
    const float* kr;
    const float* vr;
    if (j < C) {
      const int page = bt[(int64_t)b * max_pages + (j >> 4)];
      if (page < 0 || page >= num_pages) { poison = true; continue; }
      const int64_t off = (((int64_t)page * 16 + (j & 15)) * Hkv + g) * D;
      kr = ck + off; vr = cv + off;
    } else {
      const int64_t off = (((int64_t)b * k + (j - C)) * Hkv + g) * D;
      kr = kb + off; vr = vb + off;
    }
    float s = 0.f;
    for (int d = 0; d < D; ++d) s = fmaf(qs[d], kr[d], s);
    s *= sl2;
    const float mn = fmaxf(m, s);
    const float al = exp2f(m - mn), pj = exp2f(s - mn);
    l = l * al + pj;
    for (int d = 0; d < D; ++d) o[d] = o[d] * al + pj * vr[d];
    m = mn;
  }
  red[t * (D + 2)] = m;
  red[t * (D + 2) + 1] = l;
  for (int d = 0; d < D; ++d) red[t * (D + 2) + 2 + d] = o[d];
  __shared__ int any_poison;
  if (t == 0) any_poison = 0;
  __syncthreads();
  if (poison) atomicOr(&any_poison, 1);
  __syncthreads();
  float M = neg_inf();
  for (int u = 0; u < 64; ++u) M = fmaxf(M, red[u * (D + 2)]);
  float Ls = 0.f;
  for (int u = 0; u < 64; ++u) {
    const float mu = red[u * (D + 2)];
    if (mu != neg_inf()) Ls += red[u * (D + 2) + 1] * exp2f(mu - M);
  }
  const bool bad = any_poison != 0;
  for (int d = t; d < D; d += 64) {
    float O = 0.f;
    for (int u = 0; u < 64; ++u) {
      const float mu = red[u * (D + 2)];
      if (mu != neg_inf()) O += red[u * (D + 2) + 2 + d] * exp2f(mu - M);
    }
    out[(((int64_t)b * k + i) * Hq + h) * D + d] = bad ? __builtin_nanf("") : O / Ls;
  }
  if (lse && t == 0) lse[((int64_t)b * Hq + h) * k + i] = bad ? __builtin_nanf("") : (M + log2f(Ls)) * kLn2;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

template <int D, int NW>
void launch_bf16(const AttnArgs& a, AttnP p, hipStream_t st) {
  hipLaunchKernelGGL((k_attn_bf16<D, NW>), dim3((unsigned)(a.B * a.Hkv * p.S)), dim3(NW * 64), 0,
                     st, p);
}

template <int D>
void dispatch_nw(const AttnArgs& a, AttnP p, hipStream_t st) {
  const int nw = (a.Hq / a.Hkv * a.k + 15) / 16;
  if (nw <= 1) launch_bf16<D, 1>(a, p, st);
  else if (nw <= 2) launch_bf16<D, 2>(a, p, st);
  else if (nw <= 4) launch_bf16<D, 4>(a, p, st);
  else if (nw <= 8) launch_bf16<D, 8>(a, p, st);
  else launch_bf16<D, 16>(a, p, st);
}

}  // namespace

int attention_splits(int B, int Hkv, int k, int max_pages) {
  // Enough workgroups to keep every CU streaming (about 1024), but no split
  // shorter than 4 key tiles.
  const int64_t groups = (int64_t)B * Hkv;
  const int64_t tiles = ((int64_t)max_pages * 16 + k + kKT - 1) / kKT;
  int64_t s = (1024 + groups - 1) / std::max<int64_t>(groups, 1);
  s = std::min<int64_t>(s, std::max<int64_t>(1, tiles / 4));
  s = std::min<int64_t>(s, 64);
  return (int)std::max<int64_t>(s, 1);
}

size_t attention_ws_bytes(int B, int k, int Hq, int Hkv, int D, int max_pages, bool bf16) {
  (void)bf16;
  const int S = attention_splits(B, Hkv, k, max_pages);
  if (S == 1) return 0;
  const int64_t rows = (int64_t)B * Hkv * S * (Hq / Hkv) * k;
  return align256(sizeof(float) * rows * D) + align256(sizeof(float2) * rows);
}

hipError_t launch_attention(bool bf16, const AttnArgs& a, void* ws, hipStream_t st) {
  const float scale = a.scale == 0.f ? 1.f / std::sqrt((float)a.D) : a.scale;
  const int S = attention_splits(a.B, a.Hkv, a.k, a.max_pages);
  const int64_t rows = (int64_t)a.B * a.Hkv * S * (a.Hq / a.Hkv) * a.k;
  float* po = static_cast<float*>(ws);
  float2* pml = reinterpret_cast<float2*>(static_cast<char*>(ws) + align256(sizeof(float) * rows * a.D));
  if (bf16) {
    AttnP p{a.B, a.k, a.Hq, a.Hkv,
            static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_blk),
            static_cast<const uint16_t*>(a.v_blk), static_cast<const uint16_t*>(a.cache_k),
            static_cast<const uint16_t*>(a.cache_v), a.num_pages, a.block_table, a.max_pages,
            a.ctx_lens, scale * kLog2e, a.out, a.out_f32 ? 1 : 0, a.lse, po, pml, S};
    if (a.D == 64) dispatch_nw<64>(a, p, st);
    else dispatch_nw<128>(a, p, st);
    if (S > 1) {
      if (a.out_f32)
        hipLaunchKernelGGL((k_attn_combine<float>), dim3(a.B * a.Hkv), dim3(256), 0, st, a.B, a.k,
                           a.Hq, a.Hkv, a.D, S, po, pml, static_cast<float*>(a.out), a.lse);
      else
        hipLaunchKernelGGL((k_attn_combine<uint16_t>), dim3(a.B * a.Hkv), dim3(256), 0, st, a.B,
                           a.k, a.Hq, a.Hkv, a.D, S, po, pml, static_cast<uint16_t*>(a.out), a.lse);
    }
  } else {
    // The fp32 kernel never splits; its workspace is unused.
    const int grid = a.B * a.Hq * a.k;
    if (a.D == 64)
      hipLaunchKernelGGL((k_attn_f32<64>), dim3(grid), dim3(64), 0, st, a.B, a.k, a.Hq, a.Hkv,
                         static_cast<const float*>(a.q), static_cast<const float*>(a.k_blk),
                         static_cast<const float*>(a.v_blk), static_cast<const float*>(a.cache_k),
                         static_cast<const float*>(a.cache_v), a.num_pages, a.block_table,
                         a.max_pages, a.ctx_lens, scale * kLog2e, static_cast<float*>(a.out), a.lse,
                         1, nullptr, nullptr);
    else
      hipLaunchKernelGGL((k_attn_f32<128>), dim3(grid), dim3(64), 0, st, a.B, a.k, a.Hq, a.Hkv,
                         static_cast<const float*>(a.q), static_cast<const float*>(a.k_blk),
                         static_cast<const float*>(a.v_blk), static_cast<const float*>(a.cache_k),
                         static_cast<const float*>(a.cache_v), a.num_pages, a.block_table,
                         a.max_pages, a.ctx_lens, scale * kLog2e, static_cast<float*>(a.out), a.lse,
                         1, nullptr, nullptr);
  }
  return hipGetLastError();
}

}  // namespace dflash
