// Target-context KV injection: two GEMMs.
//
// [DFlash overview], section "KV 注入", steps 2-3: h_ctx = [h_1;...;h_m] W_f^T
// + b_f, then K^(l) = h_ctx W_K^(l)^T and V^(l) = h_ctx W_V^(l)^T for every
// draft layer l.  [SGLang DFlash], section 4.1: only the committed rows of a
// request go into its paged draft KV cache.
//
// Design.  Both products are "NT" GEMMs (every operand row is contiguous
// along the contraction), run on the gfx950 MFMA 32x32x16 bf16 instruction
// with 128x128x64 workgroup tiles (four wavefronts, 64x64 each).
//  * GEMM 1 reads A as a virtual concatenation: the contraction index picks
//    one of the m hidden-state buffers, so the [T, m*d] matrix never exists.
//  * GEMM 2 fuses all layers' K and V projections horizontally: output column
//    n belongs to layer n / (2*Hkv*D), to K or V by (n / (Hkv*D)) mod 2, and
//    a 128-wide column tile never straddles two weight matrices.
//  * The GEMM 2 epilogue turns each output row into its physical cache slot
//    (request, logical position, block table) and drops rows past the
//    request's committed length, so K/V go straight from accumulators to the
//    paged cache.
//  * When rows are few (decode), the contraction is split across workgroups
//    (fp32 partials in the workspace, then a reduction kernel that applies
//    the same epilogue) so that enough workgroups stream the weights.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kML = 16;  // layers a single launch can address
constexpr int BK = 64;   // granularity of split-K chunks (a multiple of the pipeline step)

// Tuning knobs: the block-tile height used below 256 x 256 (128 or 256, with
// 128 columns), and the workgroup count split-K aims for.
#ifndef DFLASH_GEMM_SMALL_BM
#define DFLASH_GEMM_SMALL_BM 128
#endif
#ifndef DFLASH_GEMM_WGS
#define DFLASH_GEMM_WGS 512
#endif

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

enum { EPI_DENSE = 0, EPI_PAGED = 1, EPI_PARTIAL = 2 };

struct GemmP {
  int M, N, K;
  const void* a[8];  // A sources; source s covers contraction [s*a_seg, (s+1)*a_seg)
  int a_seg;         // also the row stride of every source
  const void* b;     // plain B: row n at b + n*ldb
  int64_t ldb;
  int b_layered;     // B rows from per-layer K/V weights (row stride K)
  const void* wk[kML];
  const void* wv[kML];
  int HD;            // Hkv * D
  int ksplit, kchunk;
  float* part;       // [ksplit, M, N]
  const void* bias;  // [N] or null (dense epilogue)
  void* out;         // dense epilogue output [M, N]
  void* ck[kML];
  void* cv[kML];
  int np[kML];
  const int32_t* bt;
  int max_pages;
  int rows_per_seq;
  const int32_t* seq_start;
  const int32_t* commit;
};

// Uniform selection from a kernel-argument array without dynamic indexing
// (which would copy the array to scratch memory).
template <typename T, int N>
__device__ __forceinline__ T pick(const T (&arr)[N], int i) {
  T r = arr[0];
#pragma unroll
  for (int j = 1; j < N; ++j)
    if (i == j) r = arr[j];
  return r;
}

// Physical slot of output row r in layer l's cache, or -1 when the row is not
// written (past the committed length, or an unmapped / out-of-range page).
__device__ __forceinline__ int64_t row_slot(const GemmP& p, int r, int l) {
  const int s = r / p.rows_per_seq;
  const int i = r - s * p.rows_per_seq;
  if (p.commit && i >= p.commit[s]) return -1;
  const int pos = p.seq_start[s] + i;
  if (pos < 0 || (pos >> 4) >= p.max_pages) return -1;
  const int page = p.bt[(int64_t)s * p.max_pages + (pos >> 4)];
  if (page < 0 || page >= pick(p.np, l)) return -1;
  return (int64_t)page * 16 + (pos & 15);
}

template <typename T>
__device__ __forceinline__ void store_val(T* base, int64_t i, float v);
template <>
__device__ __forceinline__ void store_val<uint16_t>(uint16_t* base, int64_t i, float v) { base[i] = f32_to_bf16(v); }
template <>
__device__ __forceinline__ void store_val<float>(float* base, int64_t i, float v) { base[i] = v; }

// Final epilogue for one output element (dense with bias, or paged scatter).
template <typename T, int EPI>
__device__ __forceinline__ void emit(const GemmP& p, int row, int col, float v, int64_t slot) {
  if (EPI == EPI_DENSE) {
    if (p.bias) v += static_cast<float>(load1(static_cast<const T*>(p.bias) + col));
    store_val<T>(static_cast<T*>(p.out), (int64_t)row * p.N + col, v);
  } else {
    if (slot < 0) return;
    const int l = col / (2 * p.HD);
    const int kv = (col / p.HD) & 1;
    const int hd = col - (col / p.HD) * p.HD;
    T* cache = static_cast<T*>(kv ? pick(p.cv, l) : pick(p.ck, l));
    store_val<T>(cache, slot * p.HD + hd, v);
  }
}

// bf16 MFMA GEMM, C[M x N] = A[M x K] . B[N x K]^T, one BM x BN tile per
// workgroup of four wavefronts (2 x 2, each BM/2 x BN/2 built from MFMA
// 32x32x16 blocks).  Operands stream into LDS with direct global->LDS loads
// (no staging registers, no LDS store instructions) through NSTG stages of
// 32 contraction columns: step k is computed while steps k+1..k+NSTG-1 are in
// flight.  Each 64-byte LDS row holds its four 16-byte chunks in XOR-swizzled
// order (chunk c of row r at slot c ^ ((r/4) mod 4)), which keeps the MFMA
// operand reads free of bank conflicts.
constexpr int KB = 32;          // contraction columns per pipeline step
constexpr int NSTG = 4;         // pipeline stages
constexpr int ROWB = KB * 2;    // bytes per operand row per stage

#define GPTR(p) ((const void __attribute__((address_space(1)))*)(p))
#define LPTR(p) ((void __attribute__((address_space(3)))*)(p))

template <int BM_, int BN_>
constexpr size_t gemm_lds_bytes() {
  return std::max<size_t>((size_t)NSTG * (BM_ + BN_) * ROWB, (size_t)BM_ * (BN_ + 8) * 2);
}

template <int BM_, int BN_, int EPI>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmP p) {
  constexpr int MI = BM_ / 64, NJ = BN_ / 64;     // 32x32 blocks per wave (rows, cols)
  constexpr int STG = (BM_ + BN_) * ROWB;         // bytes per stage
  constexpr int AI = BM_ / 16 / 4, BI = BN_ / 16 / 4;   // DMA instructions per wave per step
  constexpr int DMA_PER_STEP = AI + BI;
  extern __shared__ __align__(16) uint16_t lds[];
  uint8_t* lb = reinterpret_cast<uint8_t*>(lds);
  const int tid = threadIdx.x;
  const int n_nt = p.N / BN_;
  const int tiles = (int)gridDim.x;
  int id = blockIdx.x;
  // Consecutive workgroups land on different XCDs; renumber so that each XCD
  // owns a contiguous run of tiles, then walk the tiles in groups of GM
  // row-tiles so that the B columns of a group stay in that XCD's L2.
  if ((tiles & 7) == 0) id = (id & 7) * (tiles >> 3) + (id >> 3);
  constexpr int GM = 8;
  const int n_mt = (p.M + BM_ - 1) / BM_;
  const int group = id / (GM * n_nt);
  const int first_m = group * GM;
  const int gsz = min(GM, n_mt - first_m);
  const int mt = first_m + (id % (GM * n_nt)) % gsz;
  const int nt = (id % (GM * n_nt)) / gsz;
  const int m0 = mt * BM_, n0 = nt * BN_;
  const int split = blockIdx.y;
  const int kbeg = split * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int nk = (kend - kbeg) / KB;

  const uint16_t* bbase;
  int64_t ldb;
  if (p.b_layered) {
    const int l = n0 / (2 * p.HD);
    const int kv = (n0 / p.HD) & 1;
    const int hd0 = n0 - (n0 / p.HD) * p.HD;
    bbase = static_cast<const uint16_t*>(kv ? pick(p.wv, l) : pick(p.wk, l)) + (int64_t)hd0 * p.K;
    ldb = p.K;
  } else {
    bbase = static_cast<const uint16_t*>(p.b) + (int64_t)n0 * p.ldb;
    ldb = p.ldb;
  }

  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  // DMA geometry: one instruction fills 16 rows x 64 B; lane L writes slot
  // L%4 of row L/4, which holds logical chunk (L%4) ^ ((row/4) mod 4).
  const int drow = lane >> 2;
  int64_t aoff[AI], boff[BI];
  int achk[AI], bchk[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (w * AI + i) * 16 + drow;
    achk[i] = 8 * ((lane & 3) ^ ((row >> 2) & 3));
    aoff[i] = (int64_t)min(m0 + row, p.M - 1) * p.a_seg;   // rows past M load a valid row
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = (w * BI + i) * 16 + drow;
    bchk[i] = 8 * ((lane & 3) ^ ((row >> 2) & 3));
    boff[i] = (int64_t)row * ldb;
  }
  auto issue = [&](int st, int k0) __attribute__((always_inline)) {
    uint8_t* base = lb + st * STG;
    const int src = k0 / p.a_seg;
    const uint16_t* asrc = static_cast<const uint16_t*>(pick(p.a, src)) + (k0 - src * p.a_seg);
#pragma unroll
    for (int i = 0; i < AI; ++i)
      __builtin_amdgcn_global_load_lds(GPTR(asrc + aoff[i] + achk[i]),
                                       LPTR(base + (w * AI + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < BI; ++i)
      __builtin_amdgcn_global_load_lds(GPTR(bbase + boff[i] + k0 + bchk[i]),
                                       LPTR(base + BM_ * ROWB + (w * BI + i) * 1024), 16, 0, 0);
  };

  const int r32 = lane & 31, hh = lane >> 5;
  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // operand read offsets within a stage (row, swizzled chunk), per sub-step
  int aro[MI][2], bro[NJ][2];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int row = BM_ / 2 * wm + 32 * i + r32;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) aro[i][ss] = row * ROWB + 16 * ((2 * ss + hh) ^ ((row >> 2) & 3));
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = BN_ / 2 * wn + 32 * j + r32;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
      bro[j][ss] = BM_ * ROWB + row * ROWB + 16 * ((2 * ss + hh) ^ ((row >> 2) & 3));
  }

  for (int s = 0; s < NSTG - 1 && s < nk; ++s) issue(s, kbeg + s * KB);
  for (int kt = 0; kt < nk; ++kt) {
    // wait for this step's DMA (later steps may stay in flight), then make
    // every wave's part visible
    const int ahead = min(NSTG - 2, nk - 1 - kt);
    if (ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DMA_PER_STEP) : "memory");
    else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(DMA_PER_STEP) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + NSTG - 1 < nk) issue((kt + NSTG - 1) % NSTG, kbeg + (kt + NSTG - 1) * KB);
    const uint8_t* sb = lb + (kt % NSTG) * STG;
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      bf16x8 a[MI], b[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + aro[i][ss]));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + bro[j][ss]));
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  __syncthreads();   // every wave is done with the stages before they are reused

  // C layout of the 32x32 MFMA: lane holds column (lane % 32); accumulator q
  // holds row 8*(q/4) + 4*(lane/32) + q%4.
  if (EPI == EPI_PARTIAL) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = m0 + BM_ / 2 * wm + 32 * i + 8 * (q >> 2) + 4 * hh + (q & 3);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          p.part[((int64_t)split * p.M + row) * p.N + n0 + BN_ / 2 * wn + 32 * j + r32] = acc[i][j][q];
      }
    return;
  }
  // Final epilogue: bias, bf16 rounding, then the tile goes through LDS so
  // that every output row leaves as contiguous 16-byte stores (a row of a
  // column tile is contiguous in h_ctx and in one layer's K or V cache slot).
  constexpr int OS = BN_ + 8;   // LDS row stride of the output tile
  uint16_t* ot = lds;           // [BM][OS] bf16 (reuses the operand stages)
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int cl = BN_ / 2 * wn + 32 * j + r32;
    const float bias = (EPI == EPI_DENSE && p.bias)
                           ? bf16_to_f32(static_cast<const uint16_t*>(p.bias)[n0 + cl]) : 0.f;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rl = BM_ / 2 * wm + 32 * i + 8 * (q >> 2) + 4 * hh + (q & 3);
        ot[rl * OS + cl] = f32_to_bf16(acc[i][j][q] + bias);
      }
  }
  __syncthreads();
  uint16_t* dst_base;
  int64_t row_stride;
  int hd0 = 0, layer = 0;
  if (EPI == EPI_DENSE) {
    dst_base = static_cast<uint16_t*>(p.out) + n0;
    row_stride = p.N;
  } else {
    layer = n0 / (2 * p.HD);
    const int kv = (n0 / p.HD) & 1;
    hd0 = n0 - (n0 / p.HD) * p.HD;
    dst_base = static_cast<uint16_t*>(kv ? pick(p.cv, layer) : pick(p.ck, layer)) + hd0;
    row_stride = p.HD;
  }
  constexpr int CPRW = BN_ / 8;            // 16-byte chunks per output row
  for (int e = tid; e < BM_ * CPRW; e += 256) {
    const int rl = e / CPRW, c = e - rl * CPRW;
    const int row = m0 + rl;
    if (row >= p.M) continue;
    int64_t dst;
    if (EPI == EPI_DENSE) {
      dst = (int64_t)row * row_stride;
    } else {
      const int64_t slot = row_slot(p, row, layer);
      if (slot < 0) continue;
      dst = slot * row_stride;
    }
    *reinterpret_cast<u32x4*>(dst_base + dst + 8 * c) =
        *reinterpret_cast<const u32x4*>(ot + rl * OS + 8 * c);
  }
}

// fp32 GEMM for fp32 storage: 64x64 tiles, 256 threads with 4x4 outputs each.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmP p) {
  constexpr int TM = 64, TN = 64, TK = 16;
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][TN + 1];
  const int tid = threadIdx.x;
  const int n_nt = (p.N + TN - 1) / TN;
  const int mt = blockIdx.x / n_nt, nt = blockIdx.x - mt * n_nt;
  const int m0 = mt * TM, n0 = nt * TN;
  const int split = blockIdx.y;
  const int kbeg = split * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += TK) {
    for (int e = tid; e < TK * TM; e += 256) {
      const int kk = e % TK, r = e / TK;
      const int gk = k0 + kk, gr = m0 + r;
      float v = 0.f;
      if (gk < kend && gr < p.M) {
        const int src = gk / p.a_seg;
        v = static_cast<const float*>(pick(p.a, src))[(int64_t)gr * p.a_seg + (gk - src * p.a_seg)];
      }
      As[kk][r] = v;
    }
    for (int e = tid; e < TK * TN; e += 256) {
      const int kk = e % TK, c = e / TK;
      const int gk = k0 + kk, gc = n0 + c;
      float v = 0.f;
      if (gk < kend && gc < p.N) {
        if (p.b_layered) {
          const int l = gc / (2 * p.HD), kv = (gc / p.HD) & 1, hd = gc - (gc / p.HD) * p.HD;
          v = static_cast<const float*>(kv ? pick(p.wv, l) : pick(p.wk, l))[(int64_t)hd * p.K + gk];
        } else {
          v = static_cast<const float*>(p.b)[(int64_t)gc * p.ldb + gk];
        }
      }
      Bs[kk][c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= p.M) continue;
    int64_t slot = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= p.N) continue;
      if (EPI == EPI_PARTIAL) {
        p.part[((int64_t)split * p.M + row) * p.N + col] = acc[i][j];
      } else {
        if (EPI == EPI_PAGED) slot = row_slot(p, row, col / (2 * p.HD));
        emit<float, EPI>(p, row, col, acc[i][j], slot);
      }
    }
  }
}

// Sum the split-K partials in split order, then the final epilogue.
template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_splitk_reduce(GemmP p) {
  const int64_t total = (int64_t)p.M * p.N;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int row = (int)(e / p.N);
    const int col = (int)(e - (int64_t)row * p.N);
    float v = 0.f;
    for (int s = 0; s < p.ksplit; ++s) v += p.part[(int64_t)s * total + e];
    int64_t slot = -1;
    if (EPI == EPI_PAGED) slot = row_slot(p, row, col / (2 * p.HD));
    emit<T, EPI>(p, row, col, v, slot);
  }
}

struct Plan {
  int bm, bn;          // block tile (bf16)
  int ksplit, kchunk;
};

Plan plan_gemm(int64_t M, int64_t N, int64_t K, bool bf16) {
  if (!bf16) {
    const int64_t tiles = cdiv(M, 64) * cdiv(N, 64);
    int64_t ks = 1;
    if (tiles < 512) ks = std::min<int64_t>(cdiv(1024, tiles), std::max<int64_t>(1, K / 64));
    int64_t kchunk = cdiv(cdiv(K, ks), 16) * 16;
    return Plan{64, 64, (int)cdiv(K, kchunk), (int)kchunk};
  }
  // 256 x 256 tiles when they alone give every CU a workgroup; else the
  // smaller tile, and split the contraction until about DFLASH_GEMM_WGS
  // workgroups exist.
  int bm = 256, bn = 256;
  if (N % 256 != 0 || cdiv(M, 256) * (N / 256) < 256) {
    bm = DFLASH_GEMM_SMALL_BM;
    bn = 128;
  }
  const int64_t tiles = cdiv(M, bm) * (N / bn);
  int64_t ks = 1;
  if (tiles < DFLASH_GEMM_WGS)
    ks = std::min<int64_t>(cdiv(DFLASH_GEMM_WGS, tiles), std::max<int64_t>(1, K / (4 * BK)));
  const int64_t kchunk = cdiv(cdiv(K, ks), BK) * BK;
  ks = cdiv(K, kchunk);
  return Plan{bm, bn, (int)ks, (int)kchunk};
}

template <int BM_, int BN_>
void launch_bf16_gemm(GemmP p, int epi, dim3 grid, hipStream_t st) {
  const size_t lds = gemm_lds_bytes<BM_, BN_>();
  if (epi == EPI_DENSE) hipLaunchKernelGGL((k_gemm_bf16<BM_, BN_, EPI_DENSE>), grid, dim3(256), lds, st, p);
  else if (epi == EPI_PAGED) hipLaunchKernelGGL((k_gemm_bf16<BM_, BN_, EPI_PAGED>), grid, dim3(256), lds, st, p);
  else hipLaunchKernelGGL((k_gemm_bf16<BM_, BN_, EPI_PARTIAL>), grid, dim3(256), lds, st, p);
}

void run_gemm(bool bf16, GemmP p, int epi_final, hipStream_t st) {
  const Plan pl = plan_gemm(p.M, p.N, p.K, bf16);
  p.ksplit = pl.ksplit;
  p.kchunk = pl.kchunk;
  const int epi = pl.ksplit > 1 ? EPI_PARTIAL : epi_final;
  if (bf16) {
    const dim3 grid((unsigned)(cdiv(p.M, pl.bm) * (p.N / pl.bn)), (unsigned)pl.ksplit);
    if (pl.bm == 256 && pl.bn == 256) launch_bf16_gemm<256, 256>(p, epi, grid, st);
    else if (pl.bm == 256) launch_bf16_gemm<256, 128>(p, epi, grid, st);
    else launch_bf16_gemm<128, 128>(p, epi, grid, st);
  } else {
    const dim3 grid((unsigned)(cdiv(p.M, 64) * cdiv(p.N, 64)), (unsigned)pl.ksplit);
    if (epi == EPI_DENSE) hipLaunchKernelGGL(k_gemm_f32<EPI_DENSE>, grid, dim3(256), 0, st, p);
    else if (epi == EPI_PAGED) hipLaunchKernelGGL(k_gemm_f32<EPI_PAGED>, grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_gemm_f32<EPI_PARTIAL>, grid, dim3(256), 0, st, p);
  }
  if (pl.ksplit > 1) {
    const int64_t total = (int64_t)p.M * p.N;
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(total, 256), 8192);
    if (bf16) {
      if (epi_final == EPI_DENSE) hipLaunchKernelGGL((k_splitk_reduce<uint16_t, EPI_DENSE>), dim3(blocks), dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_splitk_reduce<uint16_t, EPI_PAGED>), dim3(blocks), dim3(256), 0, st, p);
    } else {
      if (epi_final == EPI_DENSE) hipLaunchKernelGGL((k_splitk_reduce<float, EPI_DENSE>), dim3(blocks), dim3(256), 0, st, p);
      else hipLaunchKernelGGL((k_splitk_reduce<float, EPI_PAGED>), dim3(blocks), dim3(256), 0, st, p);
    }
  }
}

size_t partial_bytes(int64_t M, int64_t N, int64_t K, bool bf16) {
  const Plan pl = plan_gemm(M, N, K, bf16);
  return pl.ksplit > 1 ? align256(sizeof(float) * pl.ksplit * M * N) : 0;
}

}  // namespace

size_t materialize_ws_bytes(int64_t T, int m, int d, int n_layers, int Hkv, int D, bool bf16) {
  const int64_t es = bf16 ? 2 : 4;
  const size_t h = align256((size_t)(T * d * es));
  const size_t p1 = partial_bytes(T, d, (int64_t)m * d, bf16);
  const size_t p2 = partial_bytes(T, 2LL * std::min(n_layers, kML) * Hkv * D, d, bf16);
  return h + std::max(p1, p2);
}

hipError_t launch_materialize(bool bf16, const MatArgs& a, void* ws, size_t ws_bytes,
                              hipStream_t st) {
  (void)ws_bytes;
  const int64_t es = bf16 ? 2 : 4;
  char* w = static_cast<char*>(ws);
  void* h = a.h_out ? a.h_out : static_cast<void*>(w);
  float* part = reinterpret_cast<float*>(w + align256((size_t)(a.T * a.d * es)));
  const int HD = a.Hkv * a.D;
  // GEMM 1: h_ctx = concat(hiddens) W_f^T + b_f
  {
    GemmP p{};
    p.M = (int)a.T; p.N = a.d; p.K = a.m * a.d;
    for (int s = 0; s < a.m; ++s) p.a[s] = a.hiddens[s];
    p.a_seg = a.d;
    p.b = a.W_f; p.ldb = (int64_t)a.m * a.d;
    p.b_layered = 0;
    p.part = part;
    p.bias = a.b_f;
    p.out = h;
    run_gemm(bf16, p, EPI_DENSE, st);
  }
  // GEMM 2: every layer's K and V in one product, scattered into the caches.
  // Layers are processed kML at a time.
  for (int l0 = 0; l0 < a.n_layers; l0 += kML) {
    const int nl = std::min(kML, a.n_layers - l0);
    GemmP p{};
    p.M = (int)a.T; p.N = 2 * nl * HD; p.K = a.d;
    p.a[0] = h;
    p.a_seg = a.d;
    p.b_layered = 1;
    for (int l = 0; l < nl; ++l) {
      p.wk[l] = a.W_K[l0 + l];
      p.wv[l] = a.W_V[l0 + l];
      p.ck[l] = a.cache_k[l0 + l];
      p.cv[l] = a.cache_v[l0 + l];
      p.np[l] = a.num_pages[l0 + l];
    }
    p.HD = HD;
    p.part = part;
    p.bt = a.block_table;
    p.max_pages = a.max_pages;
    p.rows_per_seq = a.rows_per_seq;
    p.seq_start = a.seq_start;
    p.commit = a.commit_lens;
    run_gemm(bf16, p, EPI_PAGED, st);
  }
  return hipGetLastError();
}

}  // namespace dflash
