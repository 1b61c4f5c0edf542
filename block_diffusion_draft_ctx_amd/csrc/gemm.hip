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
constexpr int BM = 128, BN = 128, BK = 64, LS = BK + 8;

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

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmP p) {
  __shared__ __align__(16) uint16_t As[BM * LS];
  __shared__ __align__(16) uint16_t Bs[BN * LS];
  const int tid = threadIdx.x;
  const int n_nt = p.N / BN;
  const int tiles = (int)gridDim.x;
  int id = blockIdx.x;
  // Consecutive workgroups land on different XCDs; renumber so that each XCD
  // owns a contiguous run of tiles (neighbouring tiles share A rows in L2).
  if ((tiles & 7) == 0) id = (id & 7) * (tiles >> 3) + (id >> 3);
  const int mt = id / n_nt, nt = id - mt * n_nt;
  const int m0 = mt * BM, n0 = nt * BN;
  const int split = blockIdx.y;
  const int kbeg = split * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);

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

  u32x4 ar[4], br[4];
  auto gload = [&](int k0) __attribute__((always_inline)) {
    const int src = k0 / p.a_seg;
    const int kc = k0 - src * p.a_seg;
    const uint16_t* asrc = static_cast<const uint16_t*>(pick(p.a, src));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = tid + 256 * c;
      const int row = e >> 3;
      const int cc = (e & 7) * 8;
      const int gr = m0 + row;
      ar[c] = gr < p.M ? *reinterpret_cast<const u32x4*>(asrc + (int64_t)gr * p.a_seg + kc + cc)
                       : u32x4{0u, 0u, 0u, 0u};
      br[c] = *reinterpret_cast<const u32x4*>(bbase + (int64_t)row * ldb + k0 + cc);
    }
  };

  const int lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int r32 = lane & 31, hh = lane >> 5;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  if (kbeg < kend) gload(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = tid + 256 * c;
      const int row = e >> 3;
      const int cc = (e & 7) * 8;
      *reinterpret_cast<u32x4*>(As + row * LS + cc) = ar[c];
      *reinterpret_cast<u32x4*>(Bs + row * LS + cc) = br[c];
    }
    __syncthreads();
    if (k0 + BK < kend) gload(k0 + BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              As + (64 * wm + 32 * i + r32) * LS + 16 * s + 8 * hh));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                              Bs + (64 * wn + 32 * j + r32) * LS + 16 * s + 8 * hh));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // C layout of the 32x32 MFMA: lane holds column (lane % 32); accumulator q
  // holds row 8*(q/4) + 4*(lane/32) + q%4.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int row = m0 + 64 * wm + 32 * i + 8 * (q >> 2) + 4 * hh + (q & 3);
      if (row >= p.M) continue;
      int64_t slot = -1;
      if (EPI == EPI_PAGED) slot = row_slot(p, row, (n0 + 64 * wn) / (2 * p.HD));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + 64 * wn + 32 * j + r32;
        const float v = acc[i][j][q];
        if (EPI == EPI_PARTIAL)
          p.part[((int64_t)split * p.M + row) * p.N + col] = v;
        else
          emit<uint16_t, EPI>(p, row, col, v, slot);
      }
    }
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
  int ksplit, kchunk;
};

Plan plan_gemm(int64_t M, int64_t N, int64_t K, bool bf16) {
  const int bk = bf16 ? BK : 16;
  const int64_t tiles = bf16 ? cdiv(M, BM) * (N / BN) : cdiv(M, 64) * cdiv(N, 64);
  int64_t ks = 1;
  if (tiles < 512) ks = std::min<int64_t>(cdiv(1024, tiles), std::max<int64_t>(1, K / (4 * bk)));
  int64_t kchunk = cdiv(cdiv(K, ks), bk) * bk;
  ks = cdiv(K, kchunk);
  return Plan{(int)ks, (int)kchunk};
}

void run_gemm(bool bf16, GemmP p, int epi_final, hipStream_t st) {
  const Plan pl = plan_gemm(p.M, p.N, p.K, bf16);
  p.ksplit = pl.ksplit;
  p.kchunk = pl.kchunk;
  const int epi = pl.ksplit > 1 ? EPI_PARTIAL : epi_final;
  dim3 grid;
  if (bf16) grid = dim3((unsigned)(cdiv(p.M, BM) * (p.N / BN)), (unsigned)pl.ksplit);
  else grid = dim3((unsigned)(cdiv(p.M, 64) * cdiv(p.N, 64)), (unsigned)pl.ksplit);
  if (bf16) {
    if (epi == EPI_DENSE) hipLaunchKernelGGL(k_gemm_bf16<EPI_DENSE>, grid, dim3(256), 0, st, p);
    else if (epi == EPI_PAGED) hipLaunchKernelGGL(k_gemm_bf16<EPI_PAGED>, grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL(k_gemm_bf16<EPI_PARTIAL>, grid, dim3(256), 0, st, p);
  } else {
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
