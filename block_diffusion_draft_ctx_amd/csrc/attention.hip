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
// the k block positions) are cut into 32-row slices; every slice gets two
// wavefronts, one per half of each 64-key tile, so every K/V byte streamed
// from HBM is used by all G q-heads.  The split's physical pages are staged in
// LDS once; tile t+1's K and V rows are fetched with 16-byte loads while tile
// t is computed, then stored to the other LDS stage (one barrier per tile).
// Each wavefront runs, on its 32 keys and 32 query rows,
//   S^T[32 keys x 32 q] = K . Q^T        D/16 MFMA 32x32x16 bf16
//   online softmax per query column      (exp2 domain, lazily moved max)
//   O^T[D x 32 q]      += V^T . P^T      2 * D/32 MFMA 32x32x16 bf16, V read
//                                        from LDS with the transposing read
// so that a lane's accumulators all belong to one query and rescale with one
// factor; the two key halves merge through LDS at the end.  Small batches
// split the context across workgroups and a second kernel merges the splits
// by their log-sum-exp.
//
// The paged context cache is head-major, [num_pages, Hkv, 16, D]: a page's
// 16 keys of one kv-head are one contiguous run (4 KB at D = 128), so a
// 64-key tile is four such runs rather than 64 rows at a stride of Hkv*D.
#include <climits>
#include <cmath>

#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tuning knobs (compile-time): keys per tile, workgroups the split count
// aims for, and whether context K/V loads carry the non-temporal hint.
#ifndef DFLASH_ATTN_KT
#define DFLASH_ATTN_KT 64
#endif
#ifndef DFLASH_ATTN_TARGET_WGS
#define DFLASH_ATTN_TARGET_WGS 512
#endif
#ifndef DFLASH_ATTN_PAIR
#define DFLASH_ATTN_PAIR 1     // two requests per workgroup on a shared table row
#endif
#ifndef DFLASH_ATTN_NT
#define DFLASH_ATTN_NT 1
#endif
#ifndef DFLASH_ATTN_MIN_SPLIT_TILES
#define DFLASH_ATTN_MIN_SPLIT_TILES 4   // shortest context split, in 64-key tiles
#endif
#ifndef DFLASH_ATTN_WIDE
#define DFLASH_ATTN_WIDE 0     // 256-row workgroups (16 wavefronts: they spill at 128 VGPRs)
#endif
#ifndef DFLASH_ATTN_WIDE_LAYOUT
#define DFLASH_ATTN_WIDE_LAYOUT 1   // compute-shaped layouts go to k_attn_wide (head_dim 128)
#endif
#ifndef DFLASH_ATTN_WIDE_NW
#define DFLASH_ATTN_WIDE_NW 8       // k_attn_wide: 8 wavefronts x 32 rows, or 4 x 64
#endif
#ifndef DFLASH_ATTN_KPF
#define DFLASH_ATTN_KPF 4           // k_attn_wide: K fragments read ahead of their MFMA
#endif
#ifndef DFLASH_ATTN_VPF
#define DFLASH_ATTN_VPF 2           // k_attn_wide: V fragments read ahead of their MFMA
#endif
#ifndef DFLASH_ATTN_PINGPONG
#define DFLASH_ATTN_PINGPONG 0      // k_attn_wide: the two wavefronts of a SIMD in opposite orders
#endif
#ifndef DFLASH_ATTN_STEPS
#define DFLASH_ATTN_STEPS 1         // k_attn_wide: steady-state iteration as 32 fenced MFMA steps
#endif
constexpr int kKT = DFLASH_ATTN_KT;  // keys per tile
constexpr int kMaxSplitPages = 1024; // pages one split may span (16384 keys)
constexpr int kWideNW = DFLASH_ATTN_WIDE_NW;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Max and sum of a value and its copy 32 lanes away, by the gfx950 lane swap
// (a VALU instruction: no LDS round trip as with a bpermute).
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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
  int bt_stride;  // elements between block-table rows (0: every request reads row 0)
  const int32_t* ctx;
  float sl2;  // softmax scale * log2(e)
  void* out;  // bf16 or fp32 (out_f32)
  int out_f32;
  float* lse;
  float* po;    // split partials: O [B*Hkv*S*G*k, D] fp32, one row set per request
  float2* pml;  // split partials: (m, l) [B*Hkv*S*G*k]
  int S;        // ctx splits
  int RC;       // query-row chunks per (request, kv-head): more rows than one workgroup holds
  int mode;     // kMaskBidir, kMaskCausal or kMaskTree
  const uint32_t* tm;   // kMaskTree: ancestor bit rows [B, k - 1, tmw]
  int tmw;
};

// Transposing LDS read (gfx950): within each 16-lane group, output lane j
// receives element (j % 4) of the 8 bytes addressed by source lane
// 4*r + j/4, for r = 0..3.  With source lane 4r+q pointing at row key_r,
// columns c0+4q..c0+4q+3 of a row-major [key][d] tile, lane j gets
// (row key_0..key_3, column c0 + j): four keys of one column, which is the
// MFMA operand layout along the key (contraction) axis.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(p));
  return __builtin_bit_cast(uint2, r);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// One workgroup = (request, kv-head, query-row chunk, ctx split); 2*NQ
// wavefronts arranged as NQ query slices of 32 rows x 2 key halves (a
// request with more than 32*NQ rows per kv-head takes several chunks).
// With NB = 2 (requests reading
// one shared block-table row: packed training blocks) a workgroup owns two
// consecutive requests of one kv-head: it streams the context once, up to
// the longer of their ctx lengths, then both blocks' own keys, and every
// query row masks the keys its request does not see; it also keeps two key
// tiles in flight instead of one.  Per 64-key tile, wave
// (wq, wk) computes S^T for keys [32wk, 32wk+32) against its 32 query rows
// and accumulates O^T over the same keys (MFMA 32x32x16 bf16), with its own
// online-softmax state; the two key halves are merged once at the end.
template <int D, int NQ, int NB>
__global__ __launch_bounds__(NQ * 128) __attribute__((amdgpu_waves_per_eu(2)))
void k_attn_bf16(AttnP p) {
  constexpr int NW = 2 * NQ;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;             // 16-byte chunks per key row
  constexpr int NCH = kKT * CPR;         // chunks per tile (each of K and V)
  constexpr int CPT = (NCH + NT - 1) / NT;
  // LDS row strides (elements): K rows are read 16 B per lane down a column
  // (a stride of 4 banks mod 64 keeps 16 lanes conflict-free); V rows are
  // read by the transposing read, four rows x 32 B per half-wave, which is
  // conflict-free with a stride of 16 banks mod 64.
  constexpr int KS = D + 8;
  constexpr int VS = D + 32;
  constexpr int NMB = D / 32;            // 32-row blocks of O^T
  static_assert(kKT == 64, "the 2x2 wave layout assumes 64-key tiles");
  constexpr int STAGE = kKT * KS + kKT * VS;   // one K tile + one V tile
  __shared__ __align__(16) uint16_t smem[2 * STAGE];   // two stages
  __shared__ int pages[kMaxSplitPages];

  // Workgroups that read the same context -- the row chunks of a (request,
  // kv-head), and with a shared table every request's workgroups of one
  // kv-head -- are numbered contiguously, and each XCD takes a contiguous
  // run of numbers (the hardware deals workgroups to the 8 XCDs round
  // robin), so a context streams into one XCD's L2 once instead of eight.
  int id = blockIdx.x;
  const int nwg = (int)gridDim.x;
  const bool shares = p.RC > 1 || p.bt_stride == 0;
  if (shares && (nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int split = id % p.S;
  const int rc = (id / p.S) % p.RC;                   // 32*NQ-row chunk of the query rows
  int g, b0;
  if (p.bt_stride == 0) {                             // shared table: kv-head major
    const int nbg = (p.B + NB - 1) / NB;
    b0 = ((id / (p.S * p.RC)) % nbg) * NB;
    g = id / (p.S * p.RC * nbg);
  } else {
    g = (id / (p.S * p.RC)) % p.Hkv;
    b0 = (id / (p.S * p.RC * p.Hkv)) * NB;            // first request of the workgroup
  }
  const int nbv = min(NB, p.B - b0);                   // requests it owns
  const int G = p.Hq / p.Hkv;
  const int k = p.k;
  const int GK = G * k;                                // query rows per request
  const int Mq = GK * nbv;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int wq = w >> 1, wk = w & 1;
  const int l32 = lane & 31, hh = lane >> 5;
  const int qrow = 32 * NQ * rc + 32 * wq + l32;
  const bool qvalid = qrow < Mq;
  const int jb = (NB == 1 || !qvalid) ? 0 : qrow / GK;   // request of this row within the group
  const int b = b0 + jb;
  const int rr = qrow - jb * GK;
  const int hg = qvalid ? rr / k : 0;
  const int pos = qvalid ? rr - hg * k : 0;
  const int h = g * G + hg;

  // B operand of S^T = K . Q^T: lane (q, hh) holds Q[q][16s + 8hh .. +8]
  bf16x8 qf[D / 16];
  {
    const uint16_t* qp = p.q + (((int64_t)b * k + pos) * p.Hq + h) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint4 v = qvalid ? *reinterpret_cast<const uint4*>(qp + 16 * s) : make_uint4(0, 0, 0, 0);
      qf[s] = as_bf16x8(v);
    }
  }

  // Context lengths: this row's request (Crow), and the longest / shortest
  // of the workgroup's requests (C / Cmin); the key list is the context up
  // to C followed by the nbv blocks' own keys.
  int Crow = p.ctx[b];
  bool poison = (Crow < 0 || Crow > p.max_pages * 16);
  if (poison) Crow = 0;
  int C = Crow, Cmin = Crow;
  if (NB > 1) {
    C = 0;
    Cmin = INT_MAX;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (j < nbv) {
        int cj = p.ctx[b0 + j];
        if (cj < 0 || cj > p.max_pages * 16) cj = 0;
        C = max(C, cj);
        Cmin = min(Cmin, cj);
      }
  }
  const int total = C + k * nbv;
  const int nt = (total + kKT - 1) / kKT;
  const int tps = (nt + p.S - 1) / p.S;
  const int t0 = split * tps;
  const int t1 = min(nt, t0 + tps);

  // Physical pages of this split's context keys, staged in LDS once so that
  // no tile waits on a dependent page-table load.
  const int pg0 = t0 * (kKT / 16);
  const int pg1 = min((t1 * kKT + 15) >> 4, (C + 15) >> 4);
  if (NB == 1) {
    const int32_t* btr = p.bt + (int64_t)b * p.bt_stride;
    bool bad = false;
    for (int i = pg0 + (int)threadIdx.x; i < pg1; i += NT) {
      int pg = btr[i];
      if (pg < 0 || pg >= p.num_pages) { bad = true; pg = 0; }
      pages[i - pg0] = pg;
    }
    poison |= __syncthreads_or(bad) != 0;
  } else {
    // a bad entry poisons only the rows whose context reaches it
    __shared__ int first_bad;
    if (threadIdx.x == 0) first_bad = INT_MAX;
    __syncthreads();
    const int32_t* btr = p.bt + (int64_t)b0 * p.bt_stride;
    for (int i = pg0 + (int)threadIdx.x; i < pg1; i += NT) {
      int pg = btr[i];
      if (pg < 0 || pg >= p.num_pages) { atomicMin(&first_bad, i); pg = 0; }
      pages[i - pg0] = pg;
    }
    __syncthreads();
    poison |= (first_bad != INT_MAX && Crow > first_bad * 16);
  }

  // Per-thread chunk geometry is fixed for the whole loop: chunk c of every
  // tile is key kc[c] of the tile, 16-byte column dcc[c].
  int kc[CPT];
  int64_t coff[CPT];   // offset of (head g, slot kc%16, column) inside a head-major page
  int64_t boff[CPT];   // offset of (head g, column) inside a block row
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e = min((int)threadIdx.x + c * NT, NCH - 1);
    kc[c] = e / CPR;
    const int dc = e - kc[c] * CPR;
    coff[c] = ((int64_t)g * 16 + (kc[c] & 15)) * D + dc * 8;
    boff[c] = (int64_t)g * D + dc * 8;
  }
  const int64_t page_elems = (int64_t)16 * p.Hkv * D;
  // the group's block keys are consecutive rows of k_blk / v_blk
  const uint16_t* kblk = p.kb + (int64_t)b0 * k * p.Hkv * D;
  const uint16_t* vblk = p.vb + (int64_t)b0 * k * p.Hkv * D;

  // Branch-free tile fetch: every chunk issues the same two 16-byte loads
  // (context slot, block key, or -- past the last key -- a clamped block key
  // whose score is masked), so no load waits on another.
  u32x4 kr[CPT], vr[CPT];
  auto fetch = [&](int tile, u32x4 (&kr_)[CPT], u32x4 (&vr_)[CPT]) __attribute__((always_inline)) {
    const int pbase = (tile - t0) * (kKT / 16);
    if (tile * kKT + kKT <= C) {     // the whole tile is context (uniform)
      // a context read by one workgroup streams past the caches; the layouts
      // whose contexts other workgroups read too (row chunks, shared tables)
      // keep it in L2
      if (DFLASH_ATTN_NT && NQ <= 2 && NB == 1) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int64_t off = (int64_t)pages[pbase + (kc[c] >> 4)] * page_elems + coff[c];
          kr_[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.ck + off));
          vr_[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.cv + off));
        }
      } else {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          const int64_t off = (int64_t)pages[pbase + (kc[c] >> 4)] * page_elems + coff[c];
          kr_[c] = *reinterpret_cast<const u32x4*>(p.ck + off);
          vr_[c] = *reinterpret_cast<const u32x4*>(p.cv + off);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        const int kp = tile * kKT + kc[c];
        const int64_t off_c = (int64_t)pages[pbase + (kc[c] >> 4)] * page_elems + coff[c];
        const int64_t off_b = (int64_t)min(max(kp - C, 0), k * nbv - 1) * p.Hkv * D + boff[c];
        const bool in_ctx = kp < C;
        const uint16_t* pk = in_ctx ? p.ck + off_c : kblk + off_b;
        const uint16_t* pv = in_ctx ? p.cv + off_c : vblk + off_b;
        kr_[c] = *reinterpret_cast<const u32x4*>(pk);
        vr_[c] = *reinterpret_cast<const u32x4*>(pv);
      }
    }
  };

  // Online softmax in the exp2 domain with a lazily moved reference: m only
  // moves when a score exceeds it by more than 2^kLazy, so the accumulator
  // rescale is skipped on almost every tile (terms stay below 2^kLazy, safe
  // in fp32 and bf16); the result is exactly normalised by l at the end.
  constexpr float kLazy = 8.f;
  float m = neg_inf(), l = 0.f;
  f32x16 acc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[mb][j] = 0.f;

  // Transposing-read source lane (4r + q) within a 16-lane group
  const int tr_r = (lane & 15) >> 2, tr_q = lane & 3;
  const int grp16 = lane >> 4;             // 16-lane group: d offset 16*(grp16&1), key half hh

  auto stage = [&](uint16_t* Kd, const u32x4 (&kr_)[CPT], const u32x4 (&vr_)[CPT]) __attribute__((always_inline)) {
    uint16_t* Vd = Kd + kKT * KS;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e = threadIdx.x + c * NT;
      if (NCH % NT == 0 || e < NCH) {
        const int dc = e - kc[c] * CPR;
        *reinterpret_cast<u32x4*>(Kd + kc[c] * KS + dc * 8) = kr_[c];
        *reinterpret_cast<u32x4*>(Vd + kc[c] * VS + dc * 8) = vr_[c];
      }
    }
  };

  // One 64-key tile from the LDS stage at Ks: scores, online softmax, and the
  // P.V accumulation for this wave's query slice and key half.
  auto compute = [&](const uint16_t* Ks, int tile) __attribute__((always_inline)) {
    const uint16_t* Vs = Ks + kKT * KS;
    // no masked key in the tile (uniform): all context, or -- with the
    // bidirectional mask -- all keys of a single request's list
    const bool dense = tile * kKT + kKT <= (NB == 1 && p.mode == kMaskBidir ? total : Cmin);
    // visibility of this lane's 16 keys; key j of the lane is key
    // 32wk + 8*(j/4) + 4*hh + j%4 of the tile (the S^T accumulator order)
    uint32_t vis = 0xffffu;
    if (!dense) {
      uint64_t win = 0;       // tree: ancestor bits of this row for nodes [ybase, ybase + 64)
      int ybase = 0;
      if (p.mode == kMaskTree) {
        const int y0 = tile * kKT + 32 * wk - C - 1;   // node of the wave half's first key
        ybase = y0 >= 0 ? (y0 & ~31) : -32;
        if (qvalid && pos >= 1) {
          const uint32_t* mrow = p.tm + ((int64_t)b * (k - 1) + (pos - 1)) * p.tmw;
          const int w0 = ybase >> 5;
          const uint32_t lo = (w0 >= 0 && w0 < p.tmw) ? mrow[w0] : 0u;
          const uint32_t hi = (w0 + 1 >= 0 && w0 + 1 < p.tmw) ? mrow[w0 + 1] : 0u;
          win = ((uint64_t)hi << 32) | lo;
        }
      }
      vis = 0u;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int kk = tile * kKT + 32 * wk + 8 * (j >> 2) + 4 * hh + (j & 3);
        bool v = kk < total;
        if (NB > 1) v = kk < C ? kk < Crow : (v && (kk - C) / k == jb);
        if (p.mode == kMaskCausal && kk >= C) v = v && (kk - C) % k <= pos;
        if (p.mode == kMaskTree && kk >= C) {
          const int y = kk - C - 1;                     // -1: the root
          v = v && (y < 0 || ((win >> (y - ybase)) & 1));
        }
        vis |= (v ? 1u : 0u) << j;
      }
      // a wave half with no visible key in the tile skips it (the sparse
      // blocks of a tree mask); its softmax state is unchanged
      if (p.mode == kMaskTree && !__any(vis != 0u)) return;
    }
    // S^T[32 keys x 32 q] for this wave's key half
    f32x16 sacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
    const uint16_t* krow = Ks + (32 * wk + l32) * KS + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint4 a = *reinterpret_cast<const uint4*>(krow + 16 * s);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[s], sacc, 0, 0, 0);
    }
    // sacc[j]: key 32wk + 8*(j/4) + 4*hh + j%4 of the tile, query l32
    float sv[16];
    float tmax = neg_inf();
    if (dense) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sv[j] = sacc[j] * p.sl2;
        tmax = fmaxf(tmax, sv[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        sv[j] = ((vis >> j) & 1u) ? sacc[j] * p.sl2 : neg_inf();
        tmax = fmaxf(tmax, sv[j]);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    if (__any(tmax > m + kLazy)) {     // move the reference (rare after the first tile)
      const float mn = (tmax > m + kLazy) ? tmax : m;
      const float alpha = (mn == neg_inf()) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) acc[mb] *= alpha;
      m = mn;
    }
    const float mref = (m == neg_inf()) ? 0.f : m;   // a key half with no key yet
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      sv[j] = __builtin_amdgcn_exp2f(sv[j] - mref);
      rs += sv[j];
    }
    rs += __shfl_xor(rs, 32, 64);
    l += rs;
    // O^T[d x 32 q] += V^T . P^T over this wave's 32 keys, 16 per MFMA.  In
    // both operands contraction index 8*hh + e is key 16*kk2 + 8*(e/4) +
    // 4*hh + e%4 (the order the S^T accumulators already hold).
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const float* ps = sv + 8 * kk2;
      const bf16x8 pb = as_bf16x8(make_uint4(pack_bf16x2(ps[0], ps[1]), pack_bf16x2(ps[2], ps[3]),
                                             pack_bf16x2(ps[4], ps[5]), pack_bf16x2(ps[6], ps[7])));
      const uint16_t* v0 = Vs + (32 * wk + 16 * kk2 + 4 * (grp16 >> 1) + tr_r) * VS +
                           16 * (grp16 & 1) + 4 * tr_q;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const uint2 lo = lds_read_tr16(v0 + 32 * mb);
        const uint2 hi = lds_read_tr16(v0 + 8 * VS + 32 * mb);
        const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        acc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[mb], 0, 0, 0);
      }
    }
  };

  // Pipeline, one barrier per tile: compute tile t from one LDS stage while
  // tile t+1 (fetched one step earlier) waits in registers; then stage it
  // into the other LDS stage and fetch tile t+2.  With NB = 2 a second
  // register set keeps tile t+2 in flight as well (tile t+3 is fetched).
  if (NB == 1) {
    if (t0 < t1) {
      fetch(t0, kr, vr);
      stage(smem, kr, vr);
      if (t0 + 1 < t1) fetch(t0 + 1, kr, vr);
    }
    __syncthreads();
    for (int tile = t0; tile < t1; ++tile) {
      const int cur = (tile - t0) & 1;
      compute(smem + cur * STAGE, tile);
      if (tile + 1 < t1) {
        stage(smem + (cur ^ 1) * STAGE, kr, vr);
        if (tile + 2 < t1) fetch(tile + 2, kr, vr);
      }
      __syncthreads();
    }
  } else {
    u32x4 kr2[CPT], vr2[CPT];
    if (t0 < t1) {
      fetch(t0, kr, vr);
      stage(smem, kr, vr);
      if (t0 + 1 < t1) fetch(t0 + 1, kr, vr);
      if (t0 + 2 < t1) fetch(t0 + 2, kr2, vr2);
    }
    __syncthreads();
    // two tiles per trip so each register set has a fixed role: tile t
    // (even offset) sits in LDS stage 0, t+1 in stage 1
    for (int tile = t0; tile < t1; tile += 2) {
      compute(smem, tile);
      if (tile + 1 < t1) {
        stage(smem + STAGE, kr, vr);
        if (tile + 3 < t1) fetch(tile + 3, kr, vr);
      }
      __syncthreads();
      if (tile + 1 >= t1) break;
      compute(smem + STAGE, tile + 1);
      if (tile + 2 < t1) {
        stage(smem, kr2, vr2);
        if (tile + 4 < t1) fetch(tile + 4, kr2, vr2);
      }
      __syncthreads();
    }
  }
  // Merge the two key halves: wave (wq, 1) hands its state to wave (wq, 0)
  // through LDS, one query slice at a time.
  float* xo = reinterpret_cast<float*>(smem);          // [64 lanes][D/2] partial O
  float* xm = xo + 64 * (D / 2);                        // [32] m, [32] l
  for (int sl = 0; sl < NQ; ++sl) {
    if (sl) __syncthreads();
    if (wq == sl && wk == 1) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) xo[(mb * 16 + j) * 64 + lane] = acc[mb][j];
      if (hh == 0) { xm[l32] = m; xm[32 + l32] = l; }
    }
    __syncthreads();
    if (wq == sl && wk == 0) {
      const float m1 = xm[l32], l1 = xm[32 + l32];
      const float M = fmaxf(m, m1);
      const float Mr = (M == neg_inf()) ? 0.f : M;
      const float w0 = exp2f(m - Mr), w1 = exp2f(m1 - Mr);
      l = l * w0 + l1 * w1;
      m = M;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mb][j] = acc[mb][j] * w0 + xo[(mb * 16 + j) * 64 + lane] * w1;
    }
  }
  if (wk != 0 || !qvalid) return;

  // lane (q, hh) holds O^T[d][q] for d = 32mb + 8*(j/4) + 4*hh + j%4
  if (p.S == 1) {
    const float inv = poison ? __builtin_nanf("") : 1.f / l;
    const int64_t o0 = (((int64_t)b * k + pos) * p.Hq + h) * D + 4 * hh;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d0 = 32 * mb + 8 * jq;
        if (p.out_f32) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o0 + d0) =
              make_float4(acc[mb][4 * jq] * inv, acc[mb][4 * jq + 1] * inv,
                          acc[mb][4 * jq + 2] * inv, acc[mb][4 * jq + 3] * inv);
        } else {
          uint2 o;
          o.x = pack_bf16x2(acc[mb][4 * jq] * inv, acc[mb][4 * jq + 1] * inv);
          o.y = pack_bf16x2(acc[mb][4 * jq + 2] * inv, acc[mb][4 * jq + 3] * inv);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o0 + d0) = o;
        }
      }
    if (p.lse && hh == 0)
      p.lse[((int64_t)b * p.Hq + h) * k + pos] = poison ? __builtin_nanf("") : (m + log2f(l)) * kLn2;
  } else {
    const int64_t rowi = (((int64_t)b * p.Hkv + g) * p.S + split) * GK + rr;
    float* op = p.po + rowi * D + 4 * hh;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq)
        *reinterpret_cast<float4*>(op + 32 * mb + 8 * jq) =
            make_float4(acc[mb][4 * jq], acc[mb][4 * jq + 1], acc[mb][4 * jq + 2], acc[mb][4 * jq + 3]);
    if (hh == 0) p.pml[rowi] = make_float2(m, poison ? __builtin_nanf("") : l);
  }
}

// Compute-shaped layout (D = 128): many query rows share one context -- the
// packed training mask (consecutive blocks on one shared block-table row)
// and long row lists of one request (tree attention, large blocks).  Here the
// work is MFMA-bound, so each context tile is read from L2 once for 256 query
// rows:
//  * one workgroup = NWV wavefronts x 32 JQ query rows = up to 256 rows on
//    one kv-head (8 x 32 by default: two wavefronts per SIMD; 4 x 64 lets
//    each K and V fragment feed two MFMAs but does not fit the registers);
//    every wavefront covers whole 64-key tiles;
//  * iteration t issues the P.V products of tile t-1 and the scores of tile
//    t+1 on the matrix cores and runs the softmax of tile t on the vector
//    ALU (the three are independent); the reference max moves lazily (by
//    more than 2^8), and the rare accumulator rescale runs at the end of the
//    iteration, after the products that used the old reference;
//  * four LDS stages of K and V: tile t-1's V, tile t's V, tile t+1's K and V
//    and tile t+2 (stored from registers, fetched one iteration earlier) are
//    resident together; one barrier per tile.
// nbw > 0: nbw consecutive requests on a shared table row per workgroup;
// nbw == 0: chunks of rows_wg rows of one request (p.RC chunks).
template <int D, int NWV, int JQ, bool TREE, bool OFF32>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(NWV / 4, NWV / 4)))
void k_attn_wide(AttnP p, int nbw, int rows_wg) {
  static_assert(D == 128, "the wide layout is built for head_dim 128");
  static_assert(NWV * JQ == 8 && NWV % 4 == 0, "256 query rows per workgroup");
  constexpr int NT = 64 * NWV;
  constexpr int CPR = D / 8;
  constexpr int NCH = kKT * CPR;
  constexpr int CPT = NCH / NT;
  constexpr int KS = D + 8;
  constexpr int VS = D + 32;
  constexpr int NMB = D / 32;
  constexpr int NSTG = 4;
  static_assert(kKT == 64 && NCH % NT == 0, "tile geometry");
  constexpr int STAGE = kKT * KS + kKT * VS;
  __shared__ __align__(16) uint16_t smem[NSTG * STAGE];
  __shared__ int pages[kMaxSplitPages];
  __shared__ int first_bad;

  const int G = p.Hq / p.Hkv;
  const int k = p.k;
  const int GK = G * k;
  const int id = blockIdx.x;
  const int split = id % p.S;
  const int rest = id / p.S;
  int g, b0, nb, r0, Mq;
  if (nbw > 0) {
    // kv-head fastest: with 8 kv-heads each XCD streams one head's context;
    // groups are taken from the end (later anchors, longer contexts, first)
    const int ngrp = (p.B + nbw - 1) / nbw;
    g = rest % p.Hkv;
    const int grp = ngrp - 1 - rest / p.Hkv;
    b0 = grp * nbw;
    nb = min(nbw, p.B - b0);
    r0 = 0;
    Mq = nb * GK;
  } else {
    // the chunks of one (request, kv-head) are numbered so that they land on
    // one XCD back to back (workgroups are dealt to the 8 XCDs round robin)
    const int npair = p.B * p.Hkv;
    int pair, c;
    if ((npair & 7) == 0) {
      const int x = rest & 7, r2 = rest >> 3;
      c = r2 % p.RC;
      pair = (r2 / p.RC) * 8 + x;
    } else {
      c = rest % p.RC;
      pair = rest / p.RC;
    }
    b0 = pair / p.Hkv;
    g = pair - b0 * p.Hkv;
    nb = 1;
    r0 = c * rows_wg;
    Mq = min(GK - r0, rows_wg);
  }
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // the lane's two query rows (q-blocks jq = 0, 1 of its wavefront)
  bool qv[JQ];
  int bq[JQ], pos[JQ], hq[JQ], jr[JQ], rr_[JQ];
#pragma unroll
  for (int jq = 0; jq < JQ; ++jq) {
    const int r = 32 * JQ * w + 32 * jq + l32;
    qv[jq] = r < Mq;
    const int rg = r0 + (qv[jq] ? r : 0);
    jr[jq] = rg / GK;
    rr_[jq] = rg - jr[jq] * GK;
    const int hg = rr_[jq] / k;
    pos[jq] = rr_[jq] - hg * k;
    bq[jq] = b0 + jr[jq];
    hq[jq] = g * G + hg;
  }
  bf16x8 qf[JQ][D / 16];
#pragma unroll
  for (int jq = 0; jq < JQ; ++jq) {
    const uint16_t* qp = p.q + (((int64_t)bq[jq] * k + pos[jq]) * p.Hq + hq[jq]) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      uint4 v = qv[jq] ? *reinterpret_cast<const uint4*>(qp + 16 * s) : make_uint4(0, 0, 0, 0);
      qf[jq][s] = as_bf16x8(v);
    }
  }

  // context lengths: each row's own (Crow), the longest and shortest of the
  // workgroup's requests (C, Cmin); the key list is the context up to C,
  // then the nb requests' own keys
  bool poison[JQ];
  int Crow[JQ];
#pragma unroll
  for (int jq = 0; jq < JQ; ++jq) {
    Crow[jq] = p.ctx[bq[jq]];
    poison[jq] = Crow[jq] < 0 || Crow[jq] > p.max_pages * 16;
    if (poison[jq]) Crow[jq] = 0;
  }
  int C = 0, Cmin = INT_MAX;
  for (int j = 0; j < nb; ++j) {
    int cj = p.ctx[b0 + j];
    if (cj < 0 || cj > p.max_pages * 16) cj = 0;
    C = max(C, cj);
    Cmin = min(Cmin, cj);
  }
  // The block keys start at the first tile boundary at or after the
  // context (Cb), so that a tile holds context keys only (and past C, pad
  // keys nobody sees) or block keys only: the tile's kind is uniform, and so
  // are the base pointers of its loads.
  const int Cb = (C + kKT - 1) / kKT * kKT;
  const int total = Cb + k * nb;
  const int nt = (total + kKT - 1) / kKT;
  const int tps = (nt + p.S - 1) / p.S;
  const int t0 = split * tps;
  const int t1 = min(nt, t0 + tps);

  // the split's physical pages, staged once; a bad entry poisons only the
  // rows whose context reaches it
  const int pg0 = t0 * (kKT / 16);
  const int pg1 = min((t1 * kKT + 15) >> 4, (C + 15) >> 4);
  if (threadIdx.x == 0) first_bad = INT_MAX;
  __syncthreads();
  {
    const int32_t* btr = p.bt + (int64_t)b0 * p.bt_stride;
    for (int i = pg0 + (int)threadIdx.x; i < min(pg1, pg0 + kMaxSplitPages); i += NT) {
      int pg = btr[i];
      if (pg < 0 || pg >= p.num_pages) { atomicMin(&first_bad, i); pg = 0; }
      pages[i - pg0] = pg;
    }
  }
  __syncthreads();
#pragma unroll
  for (int jq = 0; jq < JQ; ++jq) poison[jq] |= (first_bad != INT_MAX && Crow[jq] > first_bad * 16);

  // tile fetch geometry (as in k_attn_bf16): chunk c of every tile is key
  // kc[c], 16-byte column dcc
  // byte offsets: of chunk c inside its page (slot kc & 15, and slot 0 for
  // pad keys), and inside one block key row
  int kc[CPT], coff[CPT], coff0[CPT], boff[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int e = (int)threadIdx.x + c * NT;
    kc[c] = e / CPR;
    const int dc = e - kc[c] * CPR;
    coff[c] = 2 * ((g * 16 + (kc[c] & 15)) * D + dc * 8);
    coff0[c] = 2 * (g * 16 * D + dc * 8);
    boff[c] = 2 * (g * D + dc * 8);
  }
  const int64_t page_bytes = (int64_t)32 * p.Hkv * D;
  const int row_bytes = 2 * p.Hkv * D;
  const char* kblk = reinterpret_cast<const char*>(p.kb + (int64_t)b0 * k * p.Hkv * D);
  const char* vblk = reinterpret_cast<const char*>(p.vb + (int64_t)b0 * k * p.Hkv * D);
  u32x4 kr[CPT], vr[CPT];
  // Tiles past the split's end are fetched as its last tile (their products
  // are never used).  The fetch is branch-free, so it shares a basic block
  // with the products.  A pad key (a context tile's key at or past C) reads
  // the tile's first key: a context key, so finite (its score is masked, and
  // P = 0 times a finite V adds nothing).  With OFF32 every byte offset from
  // the uniform base fits 32 bits (checked by the launcher), which gives
  // loads with a scalar base and a 32-bit lane offset.
  auto fetch = [&](int tile) __attribute__((always_inline)) {
    tile = min(tile, t1 - 1);
    const int t0k = tile * kKT;
    const bool ctx_tile = t0k < C;
    const int pbase = (tile - t0) * (kKT / 16);
    const char* bk = ctx_tile ? reinterpret_cast<const char*>(p.ck) : kblk;
    const char* bv = ctx_tile ? reinterpret_cast<const char*>(p.cv) : vblk;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const bool pad = t0k + kc[c] >= C;
      const int pi = min(pbase + (pad ? 0 : kc[c] >> 4), kMaxSplitPages - 1);
      const int co = pad ? coff0[c] : coff[c];
      const int bo = min(t0k - Cb + kc[c], k * nb - 1) * row_bytes + boff[c];
      if constexpr (OFF32) {
        const uint32_t oc = (uint32_t)pages[pi] * (uint32_t)page_bytes + (uint32_t)co;
        const uint32_t off = ctx_tile ? oc : (uint32_t)bo;
        kr[c] = *reinterpret_cast<const u32x4*>(bk + off);
        vr[c] = *reinterpret_cast<const u32x4*>(bv + off);
      } else {
        const int64_t oc = (int64_t)pages[pi] * page_bytes + co;
        const int64_t off = ctx_tile ? oc : (int64_t)bo;
        kr[c] = *reinterpret_cast<const u32x4*>(bk + off);
        vr[c] = *reinterpret_cast<const u32x4*>(bv + off);
      }
    }
  };
  auto stage = [&](int st) __attribute__((always_inline)) {
    uint16_t* Kd = smem + st * STAGE;
    uint16_t* Vd = Kd + kKT * KS;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int e = threadIdx.x + c * NT;
      const int dc = e - kc[c] * CPR;
      *reinterpret_cast<u32x4*>(Kd + kc[c] * KS + dc * 8) = kr[c];
      *reinterpret_cast<u32x4*>(Vd + kc[c] * VS + dc * 8) = vr[c];
    }
  };

  constexpr float kLazy = 8.f;
  float m[JQ], l[JQ];
  f32x16 acc[JQ][NMB];
#pragma unroll
  for (int jq = 0; jq < JQ; ++jq) {
    m[jq] = neg_inf();
    l[jq] = 0.f;
  }
#pragma unroll
  for (int jq = 0; jq < JQ; ++jq)
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[jq][mb][j] = 0.f;
  const int tr_r = (lane & 15) >> 2, tr_q = lane & 3;
  const int grp16 = lane >> 4;

  // S^T[64 keys x 64 q] of the tile in stage st: sc[kb][jq][j] is the score
  // of key 32kb + 8(j/4) + 4hh + j%4 against query row 32jq + l32
  auto scores = [&](int st, f32x16 (&sc)[2][JQ]) __attribute__((always_inline)) {
    const uint16_t* Ks = smem + st * STAGE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jq = 0; jq < JQ; ++jq)
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[kb][jq][j] = 0.f;
    // K fragments f = 2s + kb go through a ring of KPF registers: fragment
    // f + KPF is read while the MFMAs of fragment f run, so an LDS read is
    // never consumed by the instruction right after it
    constexpr int NF = 2 * (D / 16);
    constexpr int KPF = DFLASH_ATTN_KPF;
    auto kaddr = [&](int f) __attribute__((always_inline)) {
      return reinterpret_cast<const uint4*>(Ks + (32 * (f & 1) + l32) * KS + 16 * (f >> 1) + 8 * hh);
    };
    uint4 ring[KPF];
#pragma unroll
    for (int f = 0; f < KPF; ++f) ring[f] = *kaddr(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint4 a = ring[f % KPF];
      if (f + KPF < NF) ring[f % KPF] = *kaddr(f + KPF);
      const int kb = f & 1, s = f >> 1;
#pragma unroll
      for (int jq = 0; jq < JQ; ++jq)
        sc[kb][jq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[jq][s], sc[kb][jq], 0, 0, 0);
    }
  };
  // masked scores of tile `tile` set to -inf (tiles not wholly visible to
  // every row only); kept apart from the softmax so that the softmax stays in
  // one basic block with the products it overlaps
  auto mask = [&](f32x16 (&sc)[2][JQ], int tile) __attribute__((always_inline)) {
    const int tk = tile * kKT;
    const bool dense = tk + kKT <= Cmin ||
                       (nb == 1 && !TREE && p.mode == kMaskBidir && tk >= Cb && tk + kKT <= total);
    if (dense) return;
    // A row sees the context keys [0, Crow) and, of the block keys (from
    // Cb), its own block's [lo, hi) -- or, with the tree mask, the root (key
    // Cb) and the rows of its ancestors (bits of its mask row).  The tests
    // are bitwise, without short-circuit branches, so the scores never pass
    // through divergent code.
    const int kbase = tk + 4 * hh;
#pragma unroll
    for (int jq = 0; jq < JQ; ++jq) {
      if constexpr (!TREE) {
        const int lo = Cb + (nbw > 0 ? jr[jq] * k : 0);
        const int hi = lo + (p.mode == kMaskCausal ? pos[jq] + 1 : k);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int kk = kbase + 32 * kb + 8 * (j >> 2) + (j & 3);
            const unsigned v = (unsigned)(kk < Crow[jq]) | ((unsigned)(kk >= lo) & (unsigned)(kk < hi));
            sc[kb][jq][j] = v ? sc[kb][jq][j] : neg_inf();
          }
      } else {
        // Branch-free on purpose: the mask words load at clamped (valid)
        // indices and are zeroed by selects, the shift is clamped, and the
        // visibility is bitwise arithmetic, so the scores never pass through
        // divergent branches.  (With short-circuit tests and a guarded shift
        // the compiler split every element into branches, and the code it
        // made overwrote kept scores.)  The launcher sends k > 1 only, so
        // the mask array has rows.
        const bool has_row = qv[jq] && pos[jq] >= 1;
        const uint32_t* mrow = p.tm + ((int64_t)bq[jq] * (k - 1) + max(pos[jq] - 1, 0)) * p.tmw;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          // ancestor bits of this row for nodes [ybase, ybase + 64)
          const int y0 = tk + 32 * kb - Cb - 1;
          const int ybase = y0 >= 0 ? (y0 & ~31) : -32;
          const int w0 = ybase >> 5;
          const uint32_t wlo = mrow[min(max(w0, 0), p.tmw - 1)];
          const uint32_t whi = mrow[min(max(w0 + 1, 0), p.tmw - 1)];
          const bool okl = has_row && w0 >= 0 && w0 < p.tmw;
          const bool okh = has_row && w0 + 1 >= 0 && w0 + 1 < p.tmw;
          const uint64_t win = ((uint64_t)(okh ? whi : 0u) << 32) | (okl ? wlo : 0u);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int kk = kbase + 32 * kb + 8 * (j >> 2) + (j & 3);
            const int y = kk - Cb - 1;                      // -1: the root
            const unsigned bit = (unsigned)(win >> min(max(y - ybase, 0), 63)) & 1u;
            const unsigned v = (unsigned)(kk < Crow[jq]) |
                               ((unsigned)(kk >= Cb) & (unsigned)(kk < total) & ((unsigned)(y < 0) | bit));
            sc[kb][jq][j] = v ? sc[kb][jq][j] : neg_inf();
          }
        }
      }
    }
  };
  // softmax of a (masked) tile: the exponentials relative to the lazily
  // moved reference, in place (pack turns them into P, bf16, in the P^T
  // operand order: contraction index 8hh + e of k-step (kb, kk2) is key
  // 32kb + 16kk2 + 8(e/4) + 4hh + e%4), and the factor alpha by which the
  // accumulators and the row sum must be rescaled
  auto softmax = [&](f32x16 (&sc)[2][JQ], float (&alpha)[JQ]) __attribute__((always_inline)) {
#pragma unroll
    for (int jq = 0; jq < JQ; ++jq) {
      float tmax = neg_inf();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, sc[kb][jq][j]);
      tmax *= p.sl2;
      tmax = xor32_max(tmax);
      const float mn = (tmax > m[jq] + kLazy) ? tmax : m[jq];
      alpha[jq] = (mn == m[jq]) ? 1.f : __builtin_amdgcn_exp2f(m[jq] - mn);
      m[jq] = mn;
      const float mref = (mn == neg_inf()) ? 0.f : mn;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          sc[kb][jq][j] = __builtin_amdgcn_exp2f(fmaf(sc[kb][jq][j], p.sl2, -mref));
    }
  };
  // The exponentials, in place in the score registers, to P (bf16), and the
  // row sum of P as the products use it (the bf16 values, summed in fp32 two
  // at a time by dot products with (1, 1)): the normaliser then matches the
  // weights exactly.
  auto pack = [&](const f32x16 (&sc)[2][JQ], uint4 (&pb)[2][2][JQ], const float (&alpha)[JQ])
      __attribute__((always_inline)) {
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int jq = 0; jq < JQ; ++jq) {
      float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const int o = 8 * kk2;
          pb[kb][kk2][jq] = make_uint4(pack_bf16x2(sc[kb][jq][o], sc[kb][jq][o + 1]),
                                       pack_bf16x2(sc[kb][jq][o + 2], sc[kb][jq][o + 3]),
                                       pack_bf16x2(sc[kb][jq][o + 4], sc[kb][jq][o + 5]),
                                       pack_bf16x2(sc[kb][jq][o + 6], sc[kb][jq][o + 7]));
          const uint4 w = pb[kb][kk2][jq];
          rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), ones, rs0, false);
          rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), ones, rs1, false);
          rs0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), ones, rs0, false);
          rs1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), ones, rs1, false);
        }
      float rs = rs0 + rs1;
      rs = xor32_sum(rs);
      l[jq] = l[jq] * alpha[jq] + rs;
    }
  };
  // O^T[d x 64 q] += V^T . P^T over the tile in stage st
  // V fragments f = 4(2kb + kk2) + mb go through a ring of VPF register
  // pairs like the K fragments: fragment f + VPF is read while the MFMAs of
  // fragment f run (read just before its MFMA, each fragment's latency would
  // stall the matrix pipe once per MFMA)
  auto pv = [&](int st, const uint4 (&pb)[2][2][JQ]) __attribute__((always_inline)) {
    const uint16_t* Vs = smem + st * STAGE + kKT * KS;
    const uint16_t* vbase = Vs + (4 * (grp16 >> 1) + tr_r) * VS + 16 * (grp16 & 1) + 4 * tr_q;
    constexpr int NF = 4 * NMB;
    constexpr int VPF = DFLASH_ATTN_VPF;
    auto vaddr = [&](int f) __attribute__((always_inline)) {
      const int kb = f / (2 * NMB), kk2 = (f / NMB) & 1, mb = f % NMB;
      return vbase + (32 * kb + 16 * kk2) * VS + 32 * mb;
    };
    uint2 rlo[VPF], rhi[VPF];
#pragma unroll
    for (int f = 0; f < VPF; ++f) {
      rlo[f] = lds_read_tr16(vaddr(f));
      rhi[f] = lds_read_tr16(vaddr(f) + 8 * VS);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint2 lo = rlo[f % VPF], hi = rhi[f % VPF];
      if (f + VPF < NF) {
        rlo[f % VPF] = lds_read_tr16(vaddr(f + VPF));
        rhi[f % VPF] = lds_read_tr16(vaddr(f + VPF) + 8 * VS);
      }
      const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
      const int kb = f / (2 * NMB), kk2 = (f / NMB) & 1, mb = f % NMB;
#pragma unroll
      for (int jq = 0; jq < JQ; ++jq)
        acc[jq][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pb[kb][kk2][jq]),
                                                               acc[jq][mb], 0, 0, 0);
    }
  };
  auto rescale = [&](const float (&alpha)[JQ]) __attribute__((always_inline)) {
    bool move = false;
#pragma unroll
    for (int jq = 0; jq < JQ; ++jq) move = move || alpha[jq] != 1.f;
    if (__any(move)) {
#pragma unroll
      for (int jq = 0; jq < JQ; ++jq)
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) acc[jq][mb] *= alpha[jq];
    }
  };

  // The steady-state iteration as 32 steps, each one MFMA -- the 16
  // products of the tile in stage spv (P = pb), then the 16 scores of the
  // tile in stage ssc (into so) -- with a slice of the softmax of si on the
  // vector ALU, and a scheduling barrier closing every step, so that the
  // vector instructions of a step can issue while its MFMA runs.  (Left to
  // itself the compiler issues the 32 MFMAs back to back and the softmax
  // after them.)  Slices: row max (steps 0-3), the reference (4), the
  // exponentials, two per step (5-20), P packed to bf16 with its row sum
  // (21-28), the normaliser (29); the tile in registers goes to stage sst
  // at step 8 and the loads of tile tf go out at step 10.  The products read
  // P of the previous tile before step 21 packs the new one into pb.
  auto steps = [&](int spv, int ssc, f32x16 (&si)[2][JQ], f32x16 (&so)[2][JQ], uint4 (&pb)[2][2][JQ],
                   float (&alpha)[JQ], int sst, int tf) __attribute__((always_inline)) {
    const uint16_t* Vs = smem + spv * STAGE + kKT * KS;
    const uint16_t* vbase = Vs + (4 * (grp16 >> 1) + tr_r) * VS + 16 * (grp16 & 1) + 4 * tr_q;
    const uint16_t* Ks = smem + ssc * STAGE;
    constexpr int NFV = 4 * NMB;
    constexpr int NFK = 2 * (D / 16);
    constexpr int VPF = DFLASH_ATTN_VPF;
    constexpr int KPF = DFLASH_ATTN_KPF;
    static_assert(NFV == 16 && NFK == 16, "step slices assume 16 + 16 MFMA steps");
    auto vaddr = [&](int f) __attribute__((always_inline)) {
      const int kb = f / (2 * NMB), kk2 = (f / NMB) & 1, mb = f % NMB;
      return vbase + (32 * kb + 16 * kk2) * VS + 32 * mb;
    };
    auto kaddr = [&](int f) __attribute__((always_inline)) {
      return reinterpret_cast<const uint4*>(Ks + (32 * (f & 1) + l32) * KS + 16 * (f >> 1) + 8 * hh);
    };
    uint2 rlo[VPF], rhi[VPF];
    uint4 kring[KPF];
#pragma unroll
    for (int f = 0; f < VPF; ++f) {
      rlo[f] = lds_read_tr16(vaddr(f));
      rhi[f] = lds_read_tr16(vaddr(f) + 8 * VS);
    }
    float tmax[JQ], mref[JQ], rs0[JQ], rs1[JQ];
#pragma unroll
    for (int jq = 0; jq < JQ; ++jq) {
      tmax[jq] = neg_inf();
      mref[jq] = 0.f;
      rs0[jq] = 0.f;
      rs1[jq] = 0.f;
    }
    const bf16x2_t ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
    for (int s = 0; s < NFV + NFK; ++s) {
      if (s < NFV) {
        const int f = s;
        const uint2 lo = rlo[f % VPF], hi = rhi[f % VPF];
        if (f + VPF < NFV) {
          rlo[f % VPF] = lds_read_tr16(vaddr(f + VPF));
          rhi[f % VPF] = lds_read_tr16(vaddr(f + VPF) + 8 * VS);
        }
        const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        const int kb = f / (2 * NMB), kk2 = (f / NMB) & 1, mb = f % NMB;
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq)
          acc[jq][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, as_bf16x8(pb[kb][kk2][jq]), acc[jq][mb], 0, 0, 0);
        // the K ring fills during the last products
        if (s >= NFV - KPF) kring[s - (NFV - KPF)] = *kaddr(s - (NFV - KPF));
      } else {
        const int f = s - NFV;
        if (f == 0) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int jq = 0; jq < JQ; ++jq)
#pragma unroll
              for (int j = 0; j < 16; ++j) so[kb][jq][j] = 0.f;
        }
        const uint4 a = kring[f % KPF];
        if (f + KPF < NFK) kring[f % KPF] = *kaddr(f + KPF);
        const int kb = f & 1, ks = f >> 1;
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq)
          so[kb][jq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), qf[jq][ks], so[kb][jq], 0, 0, 0);
      }
      // softmax slices (as softmax() and pack(), spread over the steps)
      if (s < 4) {
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int e = 8 * s + i;
            tmax[jq] = fmaxf(tmax[jq], si[e >> 4][jq][e & 15]);
          }
      } else if (s == 4) {
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq) {
          const float tm = xor32_max(tmax[jq] * p.sl2);
          const float mn = (tm > m[jq] + kLazy) ? tm : m[jq];
          alpha[jq] = (mn == m[jq]) ? 1.f : __builtin_amdgcn_exp2f(m[jq] - mn);
          m[jq] = mn;
          mref[jq] = (mn == neg_inf()) ? 0.f : mn;
        }
      } else if (s < 21) {
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int e = 2 * (s - 5) + i;
            si[e >> 4][jq][e & 15] = __builtin_amdgcn_exp2f(fmaf(si[e >> 4][jq][e & 15], p.sl2, -mref[jq]));
          }
      } else if (s < 29) {
        const int q = s - 21, kb = q >> 2, kk2 = (q >> 1) & 1, half = q & 1;
        const int o = 8 * kk2 + 4 * half;
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq) {
          const uint32_t w0 = pack_bf16x2(si[kb][jq][o], si[kb][jq][o + 1]);
          const uint32_t w1 = pack_bf16x2(si[kb][jq][o + 2], si[kb][jq][o + 3]);
          if (half == 0) {
            pb[kb][kk2][jq].x = w0;
            pb[kb][kk2][jq].y = w1;
          } else {
            pb[kb][kk2][jq].z = w0;
            pb[kb][kk2][jq].w = w1;
          }
          rs0[jq] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w0), ones, rs0[jq], false);
          rs1[jq] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w1), ones, rs1[jq], false);
        }
      } else if (s == 29) {
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq) l[jq] = l[jq] * alpha[jq] + xor32_sum(rs0[jq] + rs1[jq]);
      }
      if (s == 8) stage(sst);
      if (s == 10) fetch(tf);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (t0 < t1) {
    f32x16 sa[2][JQ], sb[2][JQ];
    uint4 pa[2][2][JQ];   // P of the tile whose products come next
    float al[JQ];
    // tile x lives in LDS stage (x - t0) mod 4
    auto sg = [&](int x) __attribute__((always_inline)) { return (x - t0) & (NSTG - 1); };
    // The products, the scores and the softmax of an iteration are
    // independent.  The two wavefronts that share a SIMD (w and w + NWV/2)
    // take them in opposite orders -- matrix work first, or the softmax
    // first -- so that while one keeps the matrix core busy the other runs
    // on the vector ALU, instead of both meeting at every tile's barrier
    // in the same phase.
    const bool mfma_first = !DFLASH_ATTN_PINGPONG || w < NWV / 2;
    // prologue: tiles t0, t0+1 in LDS, t0+2 in registers, scores of t0
    fetch(t0);
    stage(0);
    fetch(t0 + 1);
    stage(1);
    fetch(t0 + 2);
    __syncthreads();
    scores(0, sa);
    // iteration t0: softmax of t0, scores of t0+1 (no product yet)
    mask(sa, t0);
    scores(1, sb);
    softmax(sa, al);
    pack(sa, pa, al);
    stage(2);
    fetch(t0 + 3);
    __syncthreads();
    // iteration t (t0 < t < t1): products of t-1 (their P is read before the
    // softmax of t overwrites it), scores of t+1, softmax of t, tile t+2 into
    // the stage tile t-2 left; live stages hold V(t-1), V(t), K and V(t+1)
    // and tile t+2.  The roles of the two score sets alternate, two tiles per
    // trip.
    int t = t0 + 1;
    for (; t + 1 < t1; t += 2) {
      mask(sb, t);
      if constexpr (DFLASH_ATTN_STEPS) {
        steps(sg(t - 1), sg(t + 1), sb, sa, pa, al, sg(t + 2), t + 3);
      } else {
        if (mfma_first) {
          pv(sg(t - 1), pa);
          scores(sg(t + 1), sa);
          softmax(sb, al);
        } else {
          softmax(sb, al);
          pv(sg(t - 1), pa);
          scores(sg(t + 1), sa);
        }
        pack(sb, pa, al);          // after the products of t-1 have read pa
        stage(sg(t + 2));
        fetch(t + 3);
      }
      rescale(al);
      __syncthreads();
      mask(sa, t + 1);
      if constexpr (DFLASH_ATTN_STEPS) {
        steps(sg(t), sg(t + 2), sa, sb, pa, al, sg(t + 3), t + 4);
      } else {
        if (mfma_first) {
          pv(sg(t), pa);
          scores(sg(t + 2), sb);
          softmax(sa, al);
        } else {
          softmax(sa, al);
          pv(sg(t), pa);
          scores(sg(t + 2), sb);
        }
        pack(sa, pa, al);
        stage(sg(t + 3));
        fetch(t + 4);
      }
      rescale(al);
      __syncthreads();
    }
    if (t < t1) {            // one tile left: t = t1 - 1 (its scores are in sb)
      mask(sb, t);
      pv(sg(t - 1), pa);
      softmax(sb, al);
      pack(sb, pa, al);
      rescale(al);
      pv(sg(t), pa);
    } else {                 // the last tile (t1 - 1) has its P in pa
      pv(sg(t - 1), pa);
    }
  }

  // lane (q, hh) holds O^T[d][q] of q-block jq for d = 32mb + 8(j/4) + 4hh + j%4
#pragma unroll
  for (int jq = 0; jq < JQ; ++jq) {
    if (!qv[jq]) continue;
    const int b = bq[jq], h = hq[jq];
    if (p.S == 1) {
      const float inv = poison[jq] ? __builtin_nanf("") : 1.f / l[jq];
      const int64_t o0 = (((int64_t)b * k + pos[jq]) * p.Hq + h) * D + 4 * hh;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int d0 = 32 * mb + 8 * jj;
          if (p.out_f32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o0 + d0) =
                make_float4(acc[jq][mb][4 * jj] * inv, acc[jq][mb][4 * jj + 1] * inv,
                            acc[jq][mb][4 * jj + 2] * inv, acc[jq][mb][4 * jj + 3] * inv);
          } else {
            uint2 o;
            o.x = pack_bf16x2(acc[jq][mb][4 * jj] * inv, acc[jq][mb][4 * jj + 1] * inv);
            o.y = pack_bf16x2(acc[jq][mb][4 * jj + 2] * inv, acc[jq][mb][4 * jj + 3] * inv);
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o0 + d0) = o;
          }
        }
      if (p.lse && hh == 0)
        p.lse[((int64_t)b * p.Hq + h) * k + pos[jq]] =
            poison[jq] ? __builtin_nanf("") : (m[jq] + log2f(l[jq])) * kLn2;
    } else {
      const int64_t rowi = (((int64_t)b * p.Hkv + g) * p.S + split) * GK + rr_[jq];
      float* op = p.po + rowi * D + 4 * hh;
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<float4*>(op + 32 * mb + 8 * jj) =
              make_float4(acc[jq][mb][4 * jj], acc[jq][mb][4 * jj + 1], acc[jq][mb][4 * jj + 2],
                          acc[jq][mb][4 * jj + 3]);
      if (hh == 0) p.pml[rowi] = make_float2(m[jq], poison[jq] ? __builtin_nanf("") : l[jq]);
    }
  }
}

template <typename OutT>
__global__ __launch_bounds__(128) void k_attn_combine(int B, int k, int Hq, int Hkv, int D, int S,
                                                     const float* __restrict__ po,
                                                     const float2* __restrict__ pml,
                                                     OutT* __restrict__ out, float* __restrict__ lse) {
  // one workgroup per (request, kv-head, query row); lanes over head_dim
  const int G = Hq / Hkv;
  const int Mq = G * k;
  const int qrow = blockIdx.x % Mq;
  const int bg = blockIdx.x / Mq;
  const int b = bg / Hkv, g = bg - b * Hkv;
  const int64_t base = (int64_t)bg * S * Mq + qrow;
  // the splits' partials load 8 at a time at clamped (valid) indices, so each
  // group's loads are in flight together; they merge in split order
  constexpr int SB = 8;
  float M = neg_inf();
  for (int s0 = 0; s0 < S; s0 += SB) {
    float mx[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) mx[j] = pml[base + (int64_t)min(s0 + j, S - 1) * Mq].x;
#pragma unroll
    for (int j = 0; j < SB; ++j)
      if (s0 + j < S) M = fmaxf(M, mx[j]);
  }
  const int hg = qrow / k, pos = qrow - hg * k, h = g * G + hg;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float Ls = 0.f, O = 0.f;
    for (int s0 = 0; s0 < S; s0 += SB) {
      float2 ml[SB];
      float ov[SB];
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int64_t r = base + (int64_t)min(s0 + j, S - 1) * Mq;
        ml[j] = pml[r];
        ov[j] = po[r * D + d];
      }
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        if (s0 + j >= S || (ml[j].x == neg_inf() && ml[j].y == 0.f)) continue;  // past S, or an empty split
        const float wgt = exp2f(ml[j].x - M);
        Ls += ml[j].y * wgt;
        O += ov[j] * wgt;
      }
    }
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
                                                 const int32_t* bt, int max_pages, int bt_stride,
                                                 const int32_t* ctx, float sl2, int mode,
                                                 const uint32_t* tm, int tmw,
                                                 float* out, float* lse, int S, float* po,
                                                 float2* pml) {
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
  const int total = C + (mode == kMaskCausal ? i + 1 : k);   // causal: block keys 0..i
  const uint32_t* mrow = (mode == kMaskTree && i >= 1) ? tm + ((int64_t)b * (k - 1) + (i - 1)) * tmw : nullptr;
  float m = neg_inf(), l = 0.f, o[D];
  for (int d = 0; d < D; ++d) o[d] = 0.f;
  for (int j = t; j < total; j += 64) {
    const float* kr;
    const float* vr;
    if (j < C) {
      const int page = bt[(int64_t)b * bt_stride + (j >> 4)];
      if (page < 0 || page >= num_pages) { poison = true; continue; }
      const int64_t off = (((int64_t)page * Hkv + g) * 16 + (j & 15)) * D;
      kr = ck + off; vr = cv + off;
    } else {
      if (mode == kMaskTree && j > C) {           // node y = j - C - 1: an ancestor (or itself)?
        const int y = j - C - 1;
        if (!mrow || !((mrow[y >> 5] >> (y & 31)) & 1u)) continue;
      }
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
// 32-bit words of a tree mask row for a block of k rows (k - 1 nodes)
inline int tree_words(int k) { return k > 1 ? (k - 1 + 31) / 32 : 1; }

template <int D, int NQ, int NB>
void launch_bf16(const AttnArgs& a, AttnP p, hipStream_t st) {
  const int groups = (a.B + NB - 1) / NB;
  hipLaunchKernelGGL((k_attn_bf16<D, NQ, NB>), dim3((unsigned)(groups * a.Hkv * p.RC * p.S)),
                     dim3(NQ * 128), 0, st, p);
}

// Compute-shaped layouts (head_dim 128): several requests on one shared
// table row (nbw of them per workgroup, up to 256 rows), or the rows of one
// request cut into chunks of at most 256.
template <int D, bool TREE>
void launch_wide_k(const AttnArgs& a, AttnP p, dim3 grid, int nbw, int rows_wg, hipStream_t st) {
  // every byte offset from a load's base fits 32 bits: the context cache, and
  // the nbw requests' block rows
  const bool off32 = (int64_t)a.num_pages * 32 * a.Hkv * D <= (int64_t)UINT32_MAX &&
                     (int64_t)a.k * std::max(nbw, 1) * 2 * a.Hkv * D <= (int64_t)UINT32_MAX;
  if (off32)
    hipLaunchKernelGGL((k_attn_wide<D, kWideNW, 8 / kWideNW, TREE, true>), grid, dim3(64 * kWideNW), 0,
                       st, p, nbw, rows_wg);
  else
    hipLaunchKernelGGL((k_attn_wide<D, kWideNW, 8 / kWideNW, TREE, false>), grid, dim3(64 * kWideNW), 0,
                       st, p, nbw, rows_wg);
}

// Compute-shaped layouts (head_dim 128): several requests on one shared
// table row (nbw of them per workgroup, up to 256 rows), or the rows of one
// request cut into chunks of at most 256.
template <int D>
bool launch_wide(const AttnArgs& a, AttnP p, hipStream_t st) {
  if constexpr (D != 128) {
    return false;
  } else {
    if (!DFLASH_ATTN_WIDE_LAYOUT) return false;
    const int rows = a.Hq / a.Hkv * a.k;
    // a split's context pages must fit the kernel's page list: at most
    // kMaxSplitPages / 4 tiles per split, for the longest key list (the
    // context rounded up to a tile, then up to 256 block keys or one
    // request's k)
    const int64_t nt_max = ((int64_t)a.max_pages * 16 + kKT - 1) / kKT +
                           (std::max<int64_t>(256, a.k) + kKT - 1) / kKT;
    if ((nt_max + p.S - 1) / p.S * (kKT / 16) > kMaxSplitPages) return false;
    if (a.shared_table && a.mode != kMaskTree && a.B > 1 && rows <= 128) {
      const int nbw = 256 / rows;
      const int groups = (a.B + nbw - 1) / nbw;
      launch_wide_k<D, false>(a, p, dim3((unsigned)(groups * a.Hkv * p.S)), nbw, 0, st);
      return true;
    }
    if (rows > 128 && (a.mode != kMaskTree || a.k > 1)) {
      p.RC = (rows + 255) / 256;
      const int rows_wg = (rows + p.RC - 1) / p.RC;
      const dim3 grid((unsigned)(a.B * a.Hkv * p.RC * p.S));
      if (a.mode == kMaskTree) launch_wide_k<D, true>(a, p, grid, 0, rows_wg, st);
      else launch_wide_k<D, false>(a, p, grid, 0, rows_wg, st);
      return true;
    }
    return false;
  }
}

template <int D>
void dispatch_nw(const AttnArgs& a, AttnP p, hipStream_t st) {
  if (launch_wide<D>(a, p, st)) return;
  const int rows = a.Hq / a.Hkv * a.k;            // query rows per request and kv-head
  // Requests on one shared table row go two (or four) to a workgroup when
  // their rows fit its 32-row slices: the shared context is then read once
  // per group.  Where the work is MFMA-bound the context comes from L2 and
  // the infinity cache, and rows per workgroup is what divides that traffic.
  if (DFLASH_ATTN_PAIR && a.shared_table && a.mode != kMaskTree && a.B > 1 && 2 * rows <= 128) {
    // (the sixteen-wavefront variants are compiled only when enabled: at
    // the 128 VGPRs they allow they spill)
    if constexpr (DFLASH_ATTN_WIDE != 0) {
      if (a.B > 2 && 4 * rows <= 256 && 2 * rows > 64) { launch_bf16<D, 8, 4>(a, p, st); return; }
    }
    if (2 * rows <= 64) launch_bf16<D, 2, 2>(a, p, st);
    else launch_bf16<D, 4, 2>(a, p, st);
    return;
  }
  // Otherwise one request per workgroup, at most 128 query rows each, or 256
  // for long row lists (more rows take several workgroups, each streaming
  // the context from L2).
  const int nq = (rows + 31) / 32;                 // 32-row query slices
  if (nq <= 1) launch_bf16<D, 1, 1>(a, p, st);
  else if (nq <= 2) launch_bf16<D, 2, 1>(a, p, st);
  else {
    p.RC = attention_row_chunks(a.Hq / a.Hkv, a.k);
    if constexpr (DFLASH_ATTN_WIDE != 0) {
      if (nq > 8) { launch_bf16<D, 8, 1>(a, p, st); return; }
    }
    launch_bf16<D, 4, 1>(a, p, st);
  }
}

}  // namespace

int attention_row_chunks(int G, int k) {
  // query-row chunks of one (request, kv-head): one workgroup up to 64 rows,
  // chunks of 128 rows (four 32-row slices) up to 256, of 256 rows beyond
  const int nq = (G * k + 31) / 32;
  if (nq <= 2) return 1;
  if (DFLASH_ATTN_WIDE && nq > 8) return (nq + 7) / 8;
  return (nq + 3) / 4;
}

int attention_splits(int B, int Hkv, int G, int k, int max_pages) {
  // About two workgroups per CU so every CU keeps several tiles in flight,
  // but no split shorter than DFLASH_ATTN_MIN_SPLIT_TILES key tiles; a split
  // never spans more pages than its LDS page list holds.  Row chunks already multiply the
  // workgroups.
  const int64_t groups = (int64_t)B * Hkv * attention_row_chunks(G, k);
  // (sized for the longest key list of either workgroup shape: a pair of
  // requests on one shared table row adds 2k block keys)
  const int64_t tiles = ((int64_t)max_pages * 16 + 2 * k + kKT - 1) / kKT;
  int64_t s = (DFLASH_ATTN_TARGET_WGS + groups - 1) / std::max<int64_t>(groups, 1);
  s = std::min<int64_t>(s, std::max<int64_t>(1, tiles / DFLASH_ATTN_MIN_SPLIT_TILES));
  s = std::min<int64_t>(s, 64);
  const int64_t tiles_cap = kMaxSplitPages * 16 / kKT;
  s = std::max<int64_t>(s, (tiles + tiles_cap - 1) / tiles_cap);
  return (int)std::max<int64_t>(s, 1);
}

size_t attention_ws_bytes(int B, int k, int Hq, int Hkv, int D, int max_pages, bool bf16) {
  (void)bf16;
  const int S = attention_splits(B, Hkv, Hq / Hkv, k, max_pages);
  if (S == 1) return 0;
  const int64_t rows = (int64_t)B * Hkv * S * (Hq / Hkv) * k;
  return align256(sizeof(float) * rows * D) + align256(sizeof(float2) * rows);
}

hipError_t launch_attention(bool bf16, const AttnArgs& a, void* ws, hipStream_t st) {
  const float scale = a.scale == 0.f ? 1.f / std::sqrt((float)a.D) : a.scale;
  const int S = bf16 ? attention_splits(a.B, a.Hkv, a.Hq / a.Hkv, a.k, a.max_pages) : 1;
  const int64_t rows = (int64_t)a.B * a.Hkv * S * (a.Hq / a.Hkv) * a.k;
  float* po = static_cast<float*>(ws);
  float2* pml = reinterpret_cast<float2*>(static_cast<char*>(ws) + align256(sizeof(float) * rows * a.D));
  if (bf16) {
    AttnP p{a.B, a.k, a.Hq, a.Hkv,
            static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_blk),
            static_cast<const uint16_t*>(a.v_blk), static_cast<const uint16_t*>(a.cache_k),
            static_cast<const uint16_t*>(a.cache_v), a.num_pages, a.block_table, a.max_pages,
            a.shared_table ? 0 : a.max_pages, a.ctx_lens, scale * kLog2e, a.out,
            a.out_f32 ? 1 : 0, a.lse, po, pml, S, 1, a.mode, a.tree_mask, tree_words(a.k)};
    if (a.D == 64) dispatch_nw<64>(a, p, st);
    else dispatch_nw<128>(a, p, st);
    if (S > 1) {
      const unsigned rows = (unsigned)(a.B * a.Hkv * (a.Hq / a.Hkv) * a.k);
      if (a.out_f32)
        hipLaunchKernelGGL((k_attn_combine<float>), dim3(rows), dim3(128), 0, st, a.B, a.k,
                           a.Hq, a.Hkv, a.D, S, po, pml, static_cast<float*>(a.out), a.lse);
      else
        hipLaunchKernelGGL((k_attn_combine<uint16_t>), dim3(rows), dim3(128), 0, st, a.B,
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
                         a.max_pages, a.shared_table ? 0 : a.max_pages, a.ctx_lens,
                         scale * kLog2e, a.mode, a.tree_mask, tree_words(a.k),
                         static_cast<float*>(a.out), a.lse, 1, nullptr, nullptr);
    else
      hipLaunchKernelGGL((k_attn_f32<128>), dim3(grid), dim3(64), 0, st, a.B, a.k, a.Hq, a.Hkv,
                         static_cast<const float*>(a.q), static_cast<const float*>(a.k_blk),
                         static_cast<const float*>(a.v_blk), static_cast<const float*>(a.cache_k),
                         static_cast<const float*>(a.cache_v), a.num_pages, a.block_table,
                         a.max_pages, a.shared_table ? 0 : a.max_pages, a.ctx_lens,
                         scale * kLog2e, a.mode, a.tree_mask, tree_words(a.k),
                         static_cast<float*>(a.out), a.lse, 1, nullptr, nullptr);
  }
  return hipGetLastError();
}

}  // namespace dflash
