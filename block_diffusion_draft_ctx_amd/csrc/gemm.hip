// Target-context KV injection: two GEMMs.
//
// [DFlash overview], section "KV 注入", steps 2-3: h_ctx = [h_1;...;h_m] W_f^T
// + b_f, then K^(l) = h_ctx W_K^(l)^T and V^(l) = h_ctx W_V^(l)^T for every
// draft layer l.  [SGLang DFlash], section 4.1: only the committed rows of a
// request go into its paged draft KV cache.
//
// Design.  Both products are "NT" GEMMs (every operand row is contiguous
// along the contraction), run on the gfx950 bf16 MFMAs: 16x16x32 on the
// large tiles, 32x32x16 on the smaller ones.
//  * Tiles: 256 x 256 (or 192 x 256 when one round of those fills more CUs)
//    with eight wavefronts (2 x 4, two per SIMD) when there are enough of
//    them to fill the chip, else 128 x 128 with four, or BM x 256 for
//    products of few rows; operands stream straight from global memory into
//    LDS (no staging registers) through a software pipeline of 64-column
//    steps, 2 or 3 stages deep, each step's loads issued right behind the
//    barrier that frees their stage.
//  * GEMM 1 reads A as a virtual concatenation: the contraction index picks
//    one of the m hidden-state buffers, so the [T, m*d] matrix never exists.
//  * GEMM 2 fuses all layers' K and V projections horizontally: output column
//    n belongs to layer n / (2*Hkv*D), to K or V by (n / (Hkv*D)) mod 2, and
//    a column tile never straddles two weight matrices.
//  * The GEMM 2 epilogue turns each output row into its physical cache slot
//    (request, logical position, block table) and drops rows past the
//    request's committed length, so K/V go straight from accumulators to the
//    paged cache, as whole 16-byte row pieces staged through LDS.
//  * When rows are few (decode), the contraction is split across workgroups
//    (fp32 partials in the workspace, then a reduction kernel that applies
//    the same epilogue) so that enough workgroups stream the weights.
//  * Tile order is XCD-aware: each XCD owns a contiguous run of tiles,
//    walked in groups of 8 row tiles so their B columns stay in its L2.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace dflash {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kML = 16;  // layers a single launch can address
constexpr int BK = 64;   // granularity of split-K chunks (a multiple of the pipeline step)

#ifndef DFLASH_GEMM_GM
#define DFLASH_GEMM_GM 2     // row tiles per group in the XCD-local tile walk (more than 8 row tiles)
#endif

// Tuning knobs: the block-tile height used below 256 x 256 (128 or 256, with
// 128 columns), and the workgroup count split-K aims for.
#ifndef DFLASH_GEMM_SMALL_BM
#define DFLASH_GEMM_SMALL_BM 128
#endif
// Non-temporal stores for the products' outputs: split partials (read once by
// the reduction), paged K/V rows (read by attention much later) and dense
// outputs.  Written back lazily, tens of MB of dirty lines cost the next
// streaming kernel (block attention after the K/V materialisation) far more
// than their size in HBM time; written non-temporally they do not linger.
#ifndef DFLASH_GEMM_NT_PARTIAL
#define DFLASH_GEMM_NT_PARTIAL 1
#endif
#ifndef DFLASH_GEMM_NT_CACHE
#define DFLASH_GEMM_NT_CACHE 1
#endif
#ifndef DFLASH_GEMM_NT_DENSE
#define DFLASH_GEMM_NT_DENSE 1
#endif
#ifndef DFLASH_GEMM_SPLIT_MIN_K
#define DFLASH_GEMM_SPLIT_MIN_K 4096   // shortest contraction split of the 256 x 256 plan
#endif
#ifndef DFLASH_GEMM_WGS
#define DFLASH_GEMM_WGS 512
#endif
// Few-row products (at most DFLASH_GEMM_SKINNY_M rows: decode and the
// drafter at up to sixteen blocks of 16) stream their weights: BM x 256
// tiles (BM = 32, 64 or 128, four wavefronts) keep more weight bytes in
// flight per CU than 128 x 128 tiles; the split count comes from the cost
// model of pick_splits, with rounds of DFLASH_GEMM_SKINNY_WGS workgroups.
#ifndef DFLASH_GEMM_SKINNY_M
#define DFLASH_GEMM_SKINNY_M 256
#endif
// The 128 x 128 plan picks its split count with the same cost model (1) or
// aims at DFLASH_GEMM_WGS workgroups (0).
// Bytes charged per fp32 partial element in that cost: 16, twice its write
// and read, since the reduce pass streams them less efficiently than the
// GEMM streams weights (measured better than 8 at batch 1 to 32).
#ifndef DFLASH_GEMM_PART_W
#define DFLASH_GEMM_PART_W 16.0
#endif
#ifndef DFLASH_GEMM_SMALL_COST
#define DFLASH_GEMM_SMALL_COST 1
#endif
#ifndef DFLASH_GEMM_SKINNY_WGS
#define DFLASH_GEMM_SKINNY_WGS 256
#endif
// Pipeline shape (contraction columns per step, stages) for the 256 x 256
// tile and for the smaller tiles.
#ifndef DFLASH_GEMM_KB_BIG
#define DFLASH_GEMM_KB_BIG 64
#endif
#ifndef DFLASH_GEMM_NSTG_BIG
#define DFLASH_GEMM_NSTG_BIG 2
#endif
#ifndef DFLASH_GEMM_KB_SMALL
#define DFLASH_GEMM_KB_SMALL 64
#endif
#ifndef DFLASH_GEMM_NSTG_SMALL
#define DFLASH_GEMM_NSTG_SMALL 3
#endif
// Wavefront columns of the 256 x 256 and 128 x 128 tiles (two rows of
// wavefronts): 2 gives four wavefronts (one per SIMD), 4 gives eight.
#ifndef DFLASH_GEMM_BIG_WN
#define DFLASH_GEMM_BIG_WN 4
#endif
#ifndef DFLASH_GEMM_BIG_WM
#define DFLASH_GEMM_BIG_WM 2
#endif
#ifndef DFLASH_GEMM_SMALL_WN
#define DFLASH_GEMM_SMALL_WN 2
#endif
// Workgroups a 256 x 256 split-K aims for (one per CU), and the fewest
// 256 x 256 tiles that are used without a split.
#ifndef DFLASH_GEMM_BIG_MIN_TILES
#define DFLASH_GEMM_BIG_MIN_TILES 256
#endif
#ifndef DFLASH_GEMM_BIG_UNSPLIT_MIN
#define DFLASH_GEMM_BIG_UNSPLIT_MIN 128
#endif
// Rotation of each tile's contraction start, in elements per workgroup
// (0: every tile starts at the beginning of its range).
#ifndef DFLASH_GEMM_ROT
#define DFLASH_GEMM_ROT 0
#endif
// With two stages, the DMA of a step is issued during this many sub-steps.
#ifndef DFLASH_GEMM_SPREAD2
#define DFLASH_GEMM_SPREAD2 1
#endif
// 1: the DMA of step k + NSTG goes out during the last sub-step of step k,
// right behind the barrier that frees its stage (every stage is loaded
// before the first step); 0: the DMA of step k + NSTG - 1 goes out during
// the sub-steps of step k before its last.
#ifndef DFLASH_GEMM_EARLY
#define DFLASH_GEMM_EARLY 1
#endif

// MFMA shape of the 256 x 256 tiles (32: 32x32x16, 16: 16x16x32)
#ifndef DFLASH_GEMM_MT_BIG
#define DFLASH_GEMM_MT_BIG 16
#endif
// MFMA shape of the smaller tiles
#ifndef DFLASH_GEMM_MT_SMALL
#define DFLASH_GEMM_MT_SMALL 32
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
  int D;             // head dim (paged cache offsets)
  int ksplit, kchunk;
  float* part;       // [ksplit, M, N]
  const void* bias;  // [N] or null (dense epilogue)
  const void* resid; // [M, N] or null (dense epilogue): out = resid + (product rounded to storage)
  void* out;         // dense epilogue output [M, N] (may be resid itself)
  int64_t ldc;       // row stride of out and resid (dense epilogue)
  void* ck[kML];
  void* cv[kML];
  int np[kML];
  const int32_t* bt;
  int max_pages;
  int rows_per_seq;
  const int32_t* seq_start;
  const int32_t* commit;
};

// Whether every operand byte offset of a BN-column tile fits the 32-bit
// offsets of the buffer-resource loads: A rows of all M rows of a source,
// B rows of one tile plus the contraction.
inline bool buf_offsets_fit(const GemmP& p, int bn) {
  const uint64_t lim = 0xFFFFFFFFull;
  const uint64_t ldb = p.b_layered ? (uint64_t)p.K : (uint64_t)p.ldb;
  return (uint64_t)p.M * p.a_seg * 2 <= lim && ((uint64_t)bn * ldb + p.K) * 2 <= lim;
}

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

// Element offset of (slot, column hd of the Hkv*D row) in a head-major paged
// cache [num_pages, Hkv, 16, D]: a page's 16 positions of one kv-head are
// contiguous.  8 consecutive columns never straddle a head (D % 8 == 0).
__device__ __forceinline__ int64_t kv_off(const GemmP& p, int64_t slot, int hd) {
  const int h = hd / p.D;
  return (slot >> 4) * 16 * (int64_t)p.HD + ((int64_t)h * 16 + (slot & 15)) * p.D + (hd - h * p.D);
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
    const int64_t i = (int64_t)row * p.ldc + col;
    if (p.resid) {
      // the product is stored (rounded), then added to the residual
      if (sizeof(T) == 2) v = bf16_to_f32(f32_to_bf16(v));
      v += static_cast<float>(load1(static_cast<const T*>(p.resid) + i));
    }
    store_val<T>(static_cast<T*>(p.out), i, v);
  } else {
    if (slot < 0) return;
    const int l = col / (2 * p.HD);
    const int kv = (col / p.HD) & 1;
    const int hd = col - (col / p.HD) * p.HD;
    T* cache = static_cast<T*>(kv ? pick(p.cv, l) : pick(p.ck, l));
    store_val<T>(cache, kv_off(p, slot, hd), v);
  }
}

// bf16 MFMA GEMM, C[M x N] = A[M x K] . B[N x K]^T, one BM x BN tile per
// workgroup of WM x WN wavefronts (each BM/WM x BN/WN, built from MFMA
// 32x32x16 blocks).  Operands stream into LDS with direct global->LDS loads
// (no staging registers, no LDS store instructions) through NSTG stages of
// KB contraction columns: step k is computed while steps k+1..k+NSTG-1 are
// in flight.  An operand row of a stage is KB*2 bytes made of 16-byte chunks
// stored in XOR-swizzled order (chunk c of row r at slot c ^ swz(r), with
// swz cycling once per 256 bytes of LDS), which keeps the MFMA operand reads
// free of bank conflicts.
#define LPTR(p) ((void __attribute__((address_space(3)))*)(p))

template <int BM_, int BN_, int KB_, int NSTG_>
constexpr size_t gemm_lds_bytes() {
  return std::max<size_t>((size_t)NSTG_ * (BM_ + BN_) * KB_ * 2, (size_t)BM_ * (BN_ + 8) * 2);
}

// Wait for all LDS and scalar-memory operations, as an instruction the
// compiler's wait-count tracking sees (inline assembly it does not): once no
// scalar load is pending, it can wait for individual LDS reads by count.
__device__ __forceinline__ void lgkm_drain() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// One direct global->LDS load of 16 bytes per lane: lane L's bytes land at
// LDS address lds_addr + 16*L.  Written as inline assembly on purpose: the
// compiler's wait-count tracking treats its own LDS-DMA instruction as an
// LDS event of another kind and would then drain the LDS counter before
// every MFMA.  The kernel waits for these loads itself (vmcnt + barrier).
// M0 must settle for one cycle before the load reads it.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gptr), "s"(lds_addr) : "memory", "m0");
}

// The same load through a buffer resource: lane L reads 16 bytes at byte
// offset voff + soff of the resource (voff per lane, soff uniform), so a step
// advance is one scalar add instead of a 64-bit address update per lane.
__device__ __forceinline__ void dma16_buf(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr) : "memory", "m0");
}

// Raw buffer resource over [base, base + bytes) (untyped, range checked).
__device__ __forceinline__ u32x4 buf_rsrc(const void* base, uint64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r[0] = (uint32_t)a;
  r[1] = (uint32_t)(a >> 32) & 0xFFFFu;
  r[2] = (uint32_t)min(bytes, (uint64_t)0xFFFFFFFFu);
  r[3] = 0x00020000u;
  return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Operand fragments of one sub-step (A blocks 0..MI-1, then B blocks as
// MI..MI+NJ-1) in the order the sub-step's MFMAs (A block t / NJ, B block
// t % NJ) first use them.  Reads issued in this order, one per MFMA of the
// sub-step before, give every fragment about one sub-step of lead.
template <int MI, int NJ>
struct FragOrder {
  int f[MI + NJ];
  constexpr FragOrder() : f() {
    bool a[MI] = {}, b[NJ] = {};
    int n = 0;
    for (int t = 0; t < MI * NJ; ++t) {
      if (!a[t / NJ]) { a[t / NJ] = true; f[n++] = t / NJ; }
      if (!b[t % NJ]) { b[t % NJ] = true; f[n++] = MI + t % NJ; }
    }
  }
};

template <int BM_, int BN_, int WM_, int WN_, int KB_, int NSTG_, int EPI, int MT_ = 32, bool BUF = false>
__global__ __launch_bounds__(64 * WM_ * WN_) void k_gemm_bf16(GemmP p) {
  constexpr int NW = WM_ * WN_, NT = 64 * NW;     // wavefronts (WM x WN grid), threads
  // MFMA shape: 32x32x16 (MT 32) or 16x16x32 (MT 16); MI x NJ blocks per wave
  static_assert(MT_ == 32 || MT_ == 16, "MFMA shape");
  constexpr int MI = BM_ / (MT_ * WM_), NJ = BN_ / (MT_ * WN_);
  constexpr int ROWB = KB_ * 2;                   // bytes per operand row per stage
  constexpr int CH = KB_ / 8;                     // 16-byte chunks per row
  constexpr int RP256 = 256 / ROWB;               // rows per 256 bytes of LDS
  constexpr int RPI = 64 / CH;                    // rows one DMA instruction fills
  constexpr int STG = (BM_ + BN_) * ROWB;         // bytes per stage
  constexpr int AI = BM_ / RPI / NW, BI = BN_ / RPI / NW;   // DMA instructions per wave per step
  static_assert(AI * RPI * NW == BM_ && BI * RPI * NW == BN_, "DMA rows per wave");
  constexpr int DMA_PER_STEP = AI + BI;
  static_assert(NSTG_ >= 2 && NSTG_ <= 4 && (NSTG_ - 1) * DMA_PER_STEP <= 63, "vmcnt range");
  static_assert(BK % KB_ == 0 && (KB_ == 32 || KB_ == 64), "pipeline step");
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
  // With many row tiles (prefill) and at most 32 column tiles, the groups
  // are 2 row tiles wide: the 32 CUs of an XCD then share each A tile 16
  // ways in their L2 and stream the B columns (which stay in the MALL).
  // Measured at T = 131072: the fusion GEMM (16 column tiles) 3% faster than
  // with 8-wide groups; the K/V GEMM (40 column tiles) 1% slower, so it keeps
  // 8.  With at most 8 row tiles (decode) one group holds them all.
  const int n_mt = (p.M + BM_ - 1) / BM_;
  const int GM = (n_mt > 8 && n_nt <= 32) ? DFLASH_GEMM_GM : 8;
  const int group = id / (GM * n_nt);
  const int first_m = group * GM;
  const int gsz = min(GM, n_mt - first_m);
  const int mt = first_m + (id % (GM * n_nt)) % gsz;
  const int nt = (id % (GM * n_nt)) / gsz;
  const int m0 = mt * BM_, n0 = nt * BN_;
  const int split = blockIdx.y;
  const int kbeg = split * p.kchunk;
  const int kend = min(p.K, kbeg + p.kchunk);
  const int nk = (kend - kbeg) / KB_;

  const uint16_t* bbase;
  int64_t ldb, brows;
  if (p.b_layered) {
    const int l = n0 / (2 * p.HD);
    const int kv = (n0 / p.HD) & 1;
    const int hd0 = n0 - (n0 / p.HD) * p.HD;
    bbase = static_cast<const uint16_t*>(kv ? pick(p.wv, l) : pick(p.wk, l)) + (int64_t)hd0 * p.K;
    ldb = p.K;
    brows = p.HD - hd0;
  } else {
    bbase = static_cast<const uint16_t*>(p.b) + (int64_t)n0 * p.ldb;
    ldb = p.ldb;
    brows = p.N - n0;
  }

  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6), wm = w / WN_, wn = w % WN_;
  // DMA geometry: one instruction fills RPI rows; lane L writes slot L%CH of
  // row L/CH, which holds logical chunk (L%CH) ^ swz(row).
  auto swz = [](int row) __attribute__((always_inline)) { return (row / RP256) % CH; };
  const int drow = lane / CH;
  int64_t aoff[AI], boff[BI];
  int achk[AI], bchk[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (w * AI + i) * RPI + drow;
    achk[i] = 8 * ((lane % CH) ^ swz(row));
    aoff[i] = (int64_t)min(m0 + row, p.M - 1) * p.a_seg;   // rows past M load a valid row
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int row = (w * BI + i) * RPI + drow;
    bchk[i] = 8 * ((lane % CH) ^ swz(row));
    boff[i] = (int64_t)row * ldb;
  }
  // Steps are issued strictly in order; the issue position advances by KB
  // contraction columns and moves to the next A source at a segment end.
  // The contraction range of a tile may start at a rotated offset and wrap
  // around (summation order only), so that workgroups running side by side
  // read different address ranges at the same time.
  int rot = 0;
  if (DFLASH_GEMM_ROT > 0) {
    rot = (int)(((int64_t)(blockIdx.x >> 3) * DFLASH_GEMM_ROT) % (kend - kbeg));
    rot -= rot % KB_;
  }
  int is_k, is_src, is_off;
  const uint16_t* acur;
  auto set_pos = [&](int k) __attribute__((always_inline)) {
    is_k = k;
    is_src = k / p.a_seg;
    is_off = k - is_src * p.a_seg;
    acur = static_cast<const uint16_t*>(pick(p.a, is_src)) + is_off;
  };
  set_pos(kbeg + rot);
  const uint32_t lds0 = (uint32_t)(uintptr_t)LPTR(lb);
  uint32_t avo[AI], bvo[BI];
  u32x4 arsrc, brsrc;
  const uint64_t a_bytes = (uint64_t)p.M * p.a_seg * 2;
  if (BUF) {
#pragma unroll
    for (int q = 0; q < AI; ++q) avo[q] = (uint32_t)((aoff[q] + achk[q]) * 2);
#pragma unroll
    for (int i = 0; i < BI; ++i) bvo[i] = (uint32_t)((boff[i] + bchk[i]) * 2);
    arsrc = buf_rsrc(pick(p.a, is_src), a_bytes);
    brsrc = buf_rsrc(bbase, (uint64_t)brows * ldb * 2);
  }
  // DMA instruction q (< AI + BI) of the step at the issue position into
  // stage st; the last one moves the position to the next step.
  auto dma_one = [&](int st, int q) __attribute__((always_inline)) {
    const uint32_t base = lds0 + st * STG;
    if (BUF) {
      if (q < AI)
        dma16_buf(arsrc, avo[q], (uint32_t)is_off * 2, base + (w * AI + q) * 1024);
      else
        dma16_buf(brsrc, bvo[q - AI], (uint32_t)is_k * 2, base + BM_ * ROWB + (w * BI + q - AI) * 1024);
    } else if (q < AI) {
      dma16(acur + aoff[q] + achk[q], base + (w * AI + q) * 1024);
    } else {
      const int i = q - AI;
      dma16(bbase + boff[i] + is_k + bchk[i], base + BM_ * ROWB + (w * BI + i) * 1024);
    }
    if (q == AI + BI - 1) {
      is_k += KB_;
      is_off += KB_;
      acur += KB_;
      if (DFLASH_GEMM_ROT > 0 && is_k == kend) {
        set_pos(kbeg);
        if (BUF) arsrc = buf_rsrc(pick(p.a, is_src), a_bytes);
        lgkm_drain();   // the pointer may come from a scalar load
      } else if (is_off == p.a_seg) {
        is_off = 0;
        ++is_src;
        acur = static_cast<const uint16_t*>(pick(p.a, is_src));
        if (BUF) arsrc = buf_rsrc(acur, a_bytes);
        lgkm_drain();   // the pointer may come from a scalar load
      }
    }
  };
  auto issue = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < AI + BI; ++q) dma_one(st, q);
  };

  // Operand layout of both MFMA shapes: lane L holds 8 contraction values
  // (16 bytes) of block row L % MT, chunk L / MT of the sub-step's columns.
  // Result layout: lane L holds block column L % MT; accumulator q holds
  // block row crow(q).
  const int rb = lane % MT_, kq = lane / MT_;
  using AccT = std::conditional_t<MT_ == 32, f32x16, f32x4v>;
  constexpr int NACC = MT_ == 32 ? 16 : 4;
  auto crow = [&](int q) __attribute__((always_inline)) {
    return MT_ == 32 ? 8 * (q >> 2) + 4 * kq + (q & 3) : 4 * kq + q;
  };
  auto mfma = [](bf16x8 a, bf16x8 b, AccT c) __attribute__((always_inline)) {
    if constexpr (MT_ == 32) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    else return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  };
  AccT acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < NACC; ++q) acc[i][j][q] = 0.f;

  // operand read offsets within a stage (row, swizzled chunk), per sub-step
  constexpr int SS = KB_ / (MT_ == 32 ? 16 : 32);
  constexpr int CPS = 64 / MT_;   // 16-byte chunks per row per sub-step
  // the fragment register sets alternate by sub-step parity across steps
  static_assert(SS % 2 == 0, "an even number of sub-steps per step");
  // Block rows differ by multiples of MT (and the wave offsets by multiples
  // of the wave tile), which the swizzle ignores: one base per operand and sub-step,
  // plus a constant per block (an instruction offset).
  static_assert((MT_ / RP256) % CH == 0 && (BM_ / WM_ / RP256) % CH == 0 && (BN_ / WN_ / RP256) % CH == 0,
                "swizzle period");
  int aro0[SS], bro0[SS];
#pragma unroll
  for (int ss = 0; ss < SS; ++ss) {
    aro0[ss] = (BM_ / WM_ * wm + rb) * ROWB + 16 * ((CPS * ss + kq) ^ swz(rb));
    bro0[ss] = (BM_ + BN_ / WN_ * wn + rb) * ROWB + 16 * ((CPS * ss + kq) ^ swz(rb));
  }

  // Software pipeline over steps of KB contraction columns, SS sub-steps of
  // one MFMA's contraction (16 or 32 columns) each.
  //  * Operand fragments of sub-step s+1 are read from LDS while the MFMAs of
  //    sub-step s run.
  //  * At the start of the last sub-step of step k every wave waits for its
  //    DMA of step k+1, finishes its reads of stage k and meets the others
  //    at a barrier; it then reads the first fragments of step k+1.
  //  * Default (EARLY): the DMA of step k+NSTG goes into stage k right behind
  //    that barrier, one instruction every few MFMAs of the last sub-step, so
  //    every step's loads have NSTG-1 whole steps to land.  Otherwise the DMA
  //    of step k+NSTG-1 goes into the stage of step k-1 during the sub-steps
  //    before the last.
  bf16x8 fa[2][MI], fb[2][NJ];
  // fragment f of sub-step ss: A blocks first (f < MI), then B blocks
  auto read_one = [&](int set, const uint8_t* sb, int ss, int f) __attribute__((always_inline)) {
    if (f < MI)
      fa[set][f] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + aro0[ss] + MT_ * f * ROWB));
    else
      fb[set][f - MI] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sb + bro0[ss] + MT_ * (f - MI) * ROWB));
  };
  // wait until at most `ahead` steps of DMA are outstanding (ahead < NSTG - 1)
  auto wait_steps = [&](int ahead) __attribute__((always_inline)) {
    if (NSTG_ >= 4 && ahead >= 2) wait_vmcnt<(NSTG_ >= 4 ? 2 * DMA_PER_STEP : 0)>();
    else if (NSTG_ >= 3 && ahead == 1) wait_vmcnt<DMA_PER_STEP>();
    else wait_vmcnt<0>();
  };
  constexpr int MF = MI * NJ;              // MFMAs per sub-step
  constexpr int NF = MI + NJ;              // operand fragments per sub-step
  // MFMA slots that carry DMA issue: all sub-steps before the last, or only
  // the first ones (with two stages the loads need the rest of the step to
  // land)
  constexpr int SPREAD = NSTG_ == 2 ? (SS - 1 < DFLASH_GEMM_SPREAD2 ? SS - 1 : DFLASH_GEMM_SPREAD2) : SS - 1;
  constexpr int SLOTS = SPREAD * MF;   // (with more DMA instructions than slots, several share one)

  constexpr bool EARLY = DFLASH_GEMM_EARLY;
  for (int s = 0; s < NSTG_ - (EARLY ? 0 : 1) && s < nk; ++s) issue(s);
  if (nk > 0) {
    if (EARLY && nk >= NSTG_) wait_vmcnt<(NSTG_ - 1) * DMA_PER_STEP>();   // step 0 of NSTG
    else wait_steps(min(NSTG_ - 2, nk - 1));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int f = 0; f < NF; ++f) read_one(0, lb, 0, f);
  }
  lgkm_drain();
  // mode 0: issue the DMA of a later step (kt+NSTG, or kt+NSTG-1 without
  // EARLY); 1: nothing left to issue; 2: the final step (no hand-over to a
  // next step)
  auto step = [&](int kt, int mode) __attribute__((always_inline)) {
    const uint8_t* sb = lb + (kt % NSTG_) * STG;
    const int dst = (kt + NSTG_ - 1) % NSTG_;
#pragma unroll
    for (int ss = 0; ss < SS; ++ss) {
      const int c = ss & 1;
      // fragments for the next sub-step: this stage, or the next stage once
      // every wave has its DMA and is done with this stage
      const uint8_t* rsb = sb;
      int rss = ss + 1;
      const bool rd = ss + 1 < SS || mode != 2;
      if (ss + 1 == SS && mode != 2) {
        wait_steps(min(NSTG_ - 2, nk - 2 - kt));
        lgkm_drain();   // own reads of this stage are done
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        rsb = lb + ((kt + 1) % NSTG_) * STG;
        rss = 0;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < MF; ++t) {
        const int i = t / NJ, j = t % NJ;
        acc[i][j] = mfma(fa[c][i], fb[c][j], acc[i][j]);
        // the t-th fragment in first-use order rides on MFMA t; any beyond
        // the last MFMA follow it
        if (rd) {
          constexpr FragOrder<MI, NJ> fo;
          if (t < NF) read_one(c ^ 1, rsb, rss, fo.f[t]);
          if (t == MF - 1) {
#pragma unroll
            for (int u = MF; u < NF; ++u) read_one(c ^ 1, rsb, rss, fo.f[u]);
          }
        }
        if (EARLY && mode == 0 && ss + 1 == SS) {
          // DMA instructions q with q * MF / DMA_PER_STEP == t
#pragma unroll
          for (int q = (t * DMA_PER_STEP + MF - 1) / MF; q < ((t + 1) * DMA_PER_STEP + MF - 1) / MF; ++q) {
            __builtin_amdgcn_sched_barrier(0);
            dma_one(kt % NSTG_, q);
          }
        }
        if (!EARLY && mode == 0 && ss < SPREAD) {
          const int slot = ss * MF + t;
#pragma unroll
          for (int q = 0; q < DMA_PER_STEP; ++q)
            if (q * SLOTS / DMA_PER_STEP == slot) {
              __builtin_amdgcn_sched_barrier(0);
              dma_one(dst, q);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  const int n_issue = max(0, nk - (NSTG_ - (EARLY ? 0 : 1)));   // steps that still issue a DMA
  int kt = 0;
  for (; kt < n_issue; ++kt) step(kt, 0);
  for (; kt < nk - 1; ++kt) step(kt, 1);
  if (nk > 0) step(nk - 1, 2);
  wait_vmcnt<0>();
  __syncthreads();   // every wave is done with the stages before they are reused

  if (EPI == EPI_PARTIAL) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < NACC; ++q) {
        const int row = m0 + BM_ / WM_ * wm + MT_ * i + crow(q);
        if (row >= p.M) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          float* dst = p.part + ((int64_t)split * p.M + row) * p.N + n0 + BN_ / WN_ * wn + MT_ * j + rb;
          if (DFLASH_GEMM_NT_PARTIAL) __builtin_nontemporal_store(acc[i][j][q], dst);
          else *dst = acc[i][j][q];
        }
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
    const int cl = BN_ / WN_ * wn + MT_ * j + rb;
    const float bias = (EPI == EPI_DENSE && p.bias)
                           ? bf16_to_f32(static_cast<const uint16_t*>(p.bias)[n0 + cl]) : 0.f;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < NACC; ++q) {
        const int rl = BM_ / WM_ * wm + MT_ * i + crow(q);
        ot[rl * OS + cl] = f32_to_bf16(acc[i][j][q] + bias);
      }
  }
  __syncthreads();
  uint16_t* dst_base;
  int hd0 = 0, layer = 0;
  if (EPI == EPI_DENSE) {
    dst_base = static_cast<uint16_t*>(p.out) + n0;
  } else {
    layer = n0 / (2 * p.HD);
    const int kv = (n0 / p.HD) & 1;
    hd0 = n0 - (n0 / p.HD) * p.HD;
    dst_base = static_cast<uint16_t*>(kv ? pick(p.cv, layer) : pick(p.ck, layer));
  }
  constexpr int CPRW = BN_ / 8;            // 16-byte chunks per output row
  for (int e = tid; e < BM_ * CPRW; e += NT) {
    const int rl = e / CPRW, c = e - rl * CPRW;
    const int row = m0 + rl;
    if (row >= p.M) continue;
    int64_t dst;                           // element offset of the chunk from dst_base
    if (EPI == EPI_DENSE) {
      dst = (int64_t)row * p.ldc + 8 * c;
    } else {
      const int64_t slot = row_slot(p, row, layer);
      if (slot < 0) continue;
      dst = kv_off(p, slot, hd0 + 8 * c);
    }
    u32x4 o = *reinterpret_cast<const u32x4*>(ot + rl * OS + 8 * c);
    if (EPI == EPI_DENSE && p.resid) {   // residual add on the rounded product
      const u32x4 r = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.resid) + n0 + dst);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = pack_bf16x2(bf16_lo(o[j]) + bf16_lo(r[j]), bf16_hi(o[j]) + bf16_hi(r[j]));
    }
    u32x4* d = reinterpret_cast<u32x4*>(dst_base + dst);
    if ((EPI == EPI_PAGED && DFLASH_GEMM_NT_CACHE) || (EPI == EPI_DENSE && DFLASH_GEMM_NT_DENSE))
      __builtin_nontemporal_store(o, d);
    else
      *d = o;
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

// Sum the split-K partials in split order, then the final epilogue.  With
// bf16 storage and N a multiple of 8, a thread takes 8 consecutive columns of
// one row: vector loads of the partials, one cache-slot lookup, one 16-byte
// store (8 columns never straddle a layer or K/V block: HD is a multiple of
// 128).
template <typename T, int EPI>
__global__ __launch_bounds__(256) void k_splitk_reduce(GemmP p) {
  const int64_t total = (int64_t)p.M * p.N;
  if (sizeof(T) == 2 && p.N % 8 == 0) {
    const int n8 = p.N / 8;
    const int64_t total8 = (int64_t)p.M * n8;
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total8; e += (int64_t)gridDim.x * 256) {
      const int row = (int)(e / n8);
      const int col = (int)(e - (int64_t)row * n8) * 8;
      const int64_t base = (int64_t)row * p.N + col;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      // in split order (deterministic); unrolled so several splits' loads are
      // in flight at once
#pragma unroll 8
      for (int s = 0; s < p.ksplit; ++s) {
        const f32x4v* src = reinterpret_cast<const f32x4v*>(p.part + (int64_t)s * total + base);
        const f32x4v lo = src[0], hi = src[1];
#pragma unroll
        for (int j = 0; j < 4; ++j) { v[j] += lo[j]; v[4 + j] += hi[j]; }
      }
      uint16_t* dst;
      if (EPI == EPI_DENSE) {
        if (p.bias) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] += bf16_to_f32(static_cast<const uint16_t*>(p.bias)[col + j]);
        }
        dst = static_cast<uint16_t*>(p.out) + (int64_t)row * p.ldc + col;
      } else {
        const int l = col / (2 * p.HD);
        const int64_t slot = row_slot(p, row, l);
        if (slot < 0) continue;
        const int kv = (col / p.HD) & 1;
        const int hd = col - (col / p.HD) * p.HD;
        dst = static_cast<uint16_t*>(kv ? pick(p.cv, l) : pick(p.ck, l)) + kv_off(p, slot, hd);
      }
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
      if (EPI == EPI_DENSE && p.resid) {   // residual add on the rounded product
        const u32x4 r = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.resid) +
                                                        (int64_t)row * p.ldc + col);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = pack_bf16x2(bf16_lo(o[j]) + bf16_lo(r[j]), bf16_hi(o[j]) + bf16_hi(r[j]));
      }
      if ((EPI == EPI_PAGED && DFLASH_GEMM_NT_CACHE) || (EPI == EPI_DENSE && DFLASH_GEMM_NT_DENSE))
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst));
      else
        *reinterpret_cast<u32x4*>(dst) = o;
    }
    return;
  }
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

// The drafter's gate/up product [M, 2I] split over the contraction, reduced
// straight into h[M, I] = silu(gate) * up: per 8 columns c of h, the partials
// of gate column c and up column I + c are summed in split order, each sum
// rounded to storage (as the stored product would be), then combined.
// Element-wise identical to the stored product followed by the SiLU kernel.
template <typename T>
__global__ __launch_bounds__(256) void k_splitk_reduce_silu(GemmP p, int I) {
  const int64_t total = (int64_t)p.M * p.N;   // N = 2 I
  const int i8 = I / 8;
  const int64_t n = (int64_t)p.M * i8;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int row = (int)(e / i8);
    const int col = (int)(e - (int64_t)row * i8) * 8;
    const int64_t gb = (int64_t)row * p.N + col;
    float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = 0; s < p.ksplit; ++s) {
      const f32x4v* sg = reinterpret_cast<const f32x4v*>(p.part + (int64_t)s * total + gb);
      const f32x4v* su = reinterpret_cast<const f32x4v*>(p.part + (int64_t)s * total + gb + I);
      const f32x4v g0 = sg[0], g1 = sg[1], u0 = su[0], u1 = su[1];
#pragma unroll
      for (int j = 0; j < 4; ++j) { g[j] += g0[j]; g[4 + j] += g1[j]; u[j] += u0[j]; u[4 + j] += u1[j]; }
    }
    float h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float gr = sizeof(T) == 2 ? bf16_to_f32(f32_to_bf16(g[j])) : g[j];
      const float ur = sizeof(T) == 2 ? bf16_to_f32(f32_to_bf16(u[j])) : u[j];
      h[j] = gr / (1.f + __expf(-gr)) * ur;
    }
    T* dst = static_cast<T*>(p.out) + (int64_t)row * p.ldc + col;
    if constexpr (sizeof(T) == 2) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(h[2 * j], h[2 * j + 1]);
      *reinterpret_cast<u32x4*>(dst) = o;
    } else {
      reinterpret_cast<f32x4v*>(dst)[0] = f32x4v{h[0], h[1], h[2], h[3]};
      reinterpret_cast<f32x4v*>(dst)[1] = f32x4v{h[4], h[5], h[6], h[7]};
    }
  }
}

// K epilogue of materialisation ([SGLang DFlash], section 4.1: the K
// projection goes through k_norm, then the rotary embedding at the row's
// position, before the prefix-valid write), applied in place to the K rows
// GEMM 2 has just written.  A group of D/8 consecutive lanes owns one (row,
// layer), 8 dims of every head per lane: it evaluates its row's rotation
// angles once for all heads, issues the loads of 8 heads together, and per
// head takes the mean square as a shuffle sum over the group; the rotation
// partner of dim i (i + D/2 or i - D/2) sits D/16 lanes away.  Angles are
// reduced in double precision (revolutions = pos * theta^(-2i/D) / (2 pi),
// fractional part kept) before the hardware sine and cosine, so they stay
// accurate at long positions.
struct KEpi {
  const void* w[kML];   // per layer [D] norm weight (storage dtype), used when norm
  float eps;
  int norm, rope;
  double l2theta;       // log2(rotary base)
  int D, nl;
};

__device__ __forceinline__ void load8v(const uint16_t* p, float (&v)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[2 * j] = bf16_lo(w[j]); v[2 * j + 1] = bf16_hi(w[j]); }
}
__device__ __forceinline__ void load8v(const float* p, float (&v)[8]) {
  const f32x4v a = reinterpret_cast<const f32x4v*>(p)[0], b = reinterpret_cast<const f32x4v*>(p)[1];
#pragma unroll
  for (int j = 0; j < 4; ++j) { v[j] = a[j]; v[4 + j] = b[j]; }
}
__device__ __forceinline__ void store8v(uint16_t* p, const float (&v)[8]) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
  *reinterpret_cast<u32x4*>(p) = o;
}
__device__ __forceinline__ void store8v(float* p, const float (&v)[8]) {
  reinterpret_cast<f32x4v*>(p)[0] = f32x4v{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4v*>(p)[1] = f32x4v{v[4], v[5], v[6], v[7]};
}

template <typename T>
__global__ __launch_bounds__(256) void k_k_epilogue(GemmP p, KEpi e) {
  __shared__ double rev_rate[64];   // theta^(-2i/D) / (2 pi): revolutions per position, i < D/2
  const int half = e.D / 2;
  for (int i = threadIdx.x; i < half; i += 256)
    rev_rate[i] = exp2(-(2.0 * i / e.D) * e.l2theta) * 0.15915494309189535;
  __syncthreads();
  const int G = e.D / 8;            // lanes per head (8 or 16: groups never straddle a wavefront)
  const int Hkv = p.HD / e.D;
  const int64_t items = (int64_t)p.M * e.nl;
  const int lig = threadIdx.x % G;
  const bool first = lig < G / 2;   // dims i < D/2: (x, y) -> (x c - y s, y c + x s)
  const int64_t istride = (int64_t)gridDim.x * (256 / G);
  constexpr int HB = 8;             // heads whose loads are in flight together
  for (int64_t it = ((int64_t)blockIdx.x * 256 + threadIdx.x) / G; it < items; it += istride) {
    // item -> (row, layer), rows fastest: the groups of a wavefront read
    // consecutive rows, which sit in adjacent slots of one page
    const int l = (int)(it / p.M);
    const int row = (int)(it - (int64_t)l * p.M);
    const int64_t slot = row_slot(p, row, l);
    if (slot < 0) continue;         // uniform over the group
    float cs[8], sn[8];
    if (e.rope) {
      const int s = row / p.rows_per_seq;
      const int pos = p.seq_start[s] + (row - s * p.rows_per_seq);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        double rev = (double)pos * rev_rate[8 * (lig % (G / 2)) + j];
        rev -= floor(rev);
        // the hardware sine and cosine take their argument in revolutions
        sn[j] = __builtin_amdgcn_sinf((float)rev);
        cs[j] = __builtin_amdgcn_cosf((float)rev);
      }
    }
    float w[8];
    if (e.norm) load8v(static_cast<const T*>(pick(e.w, l)) + 8 * lig, w);
    // head h of this slot sits at kp + h * 16 * D (head-major pages)
    T* kp = static_cast<T*>(pick(p.ck, l)) + kv_off(p, slot, 8 * lig);
    for (int h0 = 0; h0 < Hkv; h0 += HB) {
      float v[HB][8];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        if (h0 + hb < Hkv) load8v(kp + (int64_t)(h0 + hb) * 16 * e.D, v[hb]);
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        if (h0 + hb >= Hkv) break;   // uniform
        if (e.norm) {
          float ss = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) ss = fmaf(v[hb][j], v[hb][j], ss);
          for (int o = G / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
          const float r = 1.f / sqrtf(ss / e.D + e.eps);
#pragma unroll
          for (int j = 0; j < 8; ++j) v[hb][j] *= r * w[j];
        }
        if (e.rope) {
          float pr[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pr[j] = __shfl_xor(v[hb][j], G / 2, 64);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            v[hb][j] = first ? fmaf(v[hb][j], cs[j], -pr[j] * sn[j]) : fmaf(v[hb][j], cs[j], pr[j] * sn[j]);
        }
        store8v(kp + (int64_t)(h0 + hb) * 16 * e.D, v[hb]);
      }
    }
  }
}

struct Plan {
  int bm, bn;          // block tile (bf16)
  int ksplit, kchunk;
};

// col_block: the width of the column blocks no tile may straddle (the K/V
// GEMM's Hkv*D-wide blocks, one per layer and K or V, each with its own
// weight matrix and cache), or 0 for a dense product.  256-wide tiles need
// it to be a multiple of 256; 128 always divides it.
// Split count for tiles that run one workgroup per CU, in rounds of W.
// Cost of k splits, in bytes per CU: each round streams one tile's operands
// over K / k columns (512 K / k bytes for 256 operand rows), and the fp32
// partials are written and read back (DFLASH_GEMM_PART_W k M N bytes over
// the CUs).  The
// cheapest count wins, the fewest splits on a tie; no split is shorter than
// 4 steps.
int64_t pick_splits(int64_t tiles, int64_t M, int64_t N, int64_t K, int64_t W) {
  const int64_t ks_max = std::max<int64_t>(1, K / (4 * BK));
  int64_t ks = 1;
  double best = (double)cdiv(tiles, W) * 512.0 * (double)K;
  for (int64_t k = 2; k <= ks_max; ++k) {
    const double cost = (double)cdiv(tiles * k, W) * 512.0 * (double)K / (double)k +
                        DFLASH_GEMM_PART_W * (double)k * (double)M * (double)N / (double)W;
    if (cost < best) { best = cost; ks = k; }
  }
  return ks;
}

Plan plan_gemm(int64_t M, int64_t N, int64_t K, bool bf16, int64_t col_block) {
  if (!bf16) {
    const int64_t tiles = cdiv(M, 64) * cdiv(N, 64);
    int64_t ks = 1;
    if (tiles < 512) ks = std::min<int64_t>(cdiv(1024, tiles), std::max<int64_t>(1, K / 64));
    int64_t kchunk = cdiv(cdiv(K, ks), 16) * 16;
    return Plan{64, 64, (int)cdiv(K, kchunk), (int)kchunk};
  }
  // Per CU the operand feed from L2 bounds a tile's rate, and a 256 x 256
  // tile does twice the work per byte of a 128 x 128 one, so 256 x 256 is
  // preferred:
  //  * split over the contraction to one workgroup per CU when every split
  //    stays at least 4096 columns long (shorter splits lose to their
  //    partials), or whole when the tiles alone fill the CUs;
  //  * unsplit when at least DFLASH_GEMM_BIG_UNSPLIT_MIN tiles exist;
  //  * else 128-row tiles, the contraction split until about
  //    DFLASH_GEMM_WGS workgroups exist.
  const bool w256 = N % 256 == 0 && col_block % 256 == 0;
  if (M <= DFLASH_GEMM_SKINNY_M && w256) {
    const int bm = M <= 32 ? 32 : (M <= 64 ? 64 : 128);
    const int64_t tiles = cdiv(M, bm) * (N / 256);
    const int64_t ks = pick_splits(tiles, M, N, K, DFLASH_GEMM_SKINNY_WGS);
    const int64_t kchunk = cdiv(cdiv(K, ks), BK) * BK;
    return Plan{bm, 256, (int)cdiv(K, kchunk), (int)kchunk};
  }
  constexpr int64_t kCUs = DFLASH_GEMM_BIG_MIN_TILES;
  const int64_t t256 = w256 ? cdiv(M, 256) * (N / 256) : 0;
  const bool split_ok = t256 > 0 && K / cdiv(kCUs, t256) >= DFLASH_GEMM_SPLIT_MIN_K;
  if (split_ok || t256 >= DFLASH_GEMM_BIG_UNSPLIT_MIN) {
    const int64_t ks0 = split_ok ? cdiv(kCUs, t256) : 1;
    const int64_t kchunk = cdiv(cdiv(K, ks0), BK) * BK;
    // Unsplit, 192-row tiles when their rounds of workgroups take clearly
    // less time (rounds x tile rows): 160 256-row tiles of a 1024-row product
    // leave 96 CUs idle, 240 192-row ones fill them.
    const int64_t t192 = cdiv(M, 192) * (N / 256);
    if (ks0 == 1 && 10 * cdiv(t192, kCUs) * 192 < 9 * cdiv(t256, kCUs) * 256)
      return Plan{192, 256, 1, (int)cdiv(K, BK) * BK};
    return Plan{256, 256, (int)cdiv(K, kchunk), (int)kchunk};
  }
  const int bm = DFLASH_GEMM_SMALL_BM, bn = 128;
  const int64_t tiles = cdiv(M, bm) * (N / bn);
  int64_t ks = 1;
  if (DFLASH_GEMM_SMALL_COST)   // one workgroup per CU: the same cost model
    ks = pick_splits(tiles, M, N, K, DFLASH_GEMM_SKINNY_WGS);
  else if (tiles < DFLASH_GEMM_WGS)
    ks = std::min<int64_t>(cdiv(DFLASH_GEMM_WGS, tiles), std::max<int64_t>(1, K / (4 * BK)));
  const int64_t kchunk = cdiv(cdiv(K, ks), BK) * BK;
  ks = cdiv(K, kchunk);
  return Plan{bm, bn, (int)ks, (int)kchunk};
}

template <int BM_, int BN_, int WM_, int WN_, int KB_, int NSTG_, int MT_ = 32, bool BUF = false>
void launch_bf16_gemm(GemmP p, int epi, dim3 grid, hipStream_t st) {
  const size_t lds = gemm_lds_bytes<BM_, BN_, KB_, NSTG_>();
  const dim3 block(64 * WM_ * WN_);
  if (epi == EPI_DENSE)
    hipLaunchKernelGGL((k_gemm_bf16<BM_, BN_, WM_, WN_, KB_, NSTG_, EPI_DENSE, MT_, BUF>), grid, block, lds, st, p);
  else if (epi == EPI_PAGED)
    hipLaunchKernelGGL((k_gemm_bf16<BM_, BN_, WM_, WN_, KB_, NSTG_, EPI_PAGED, MT_, BUF>), grid, block, lds, st, p);
  else
    hipLaunchKernelGGL((k_gemm_bf16<BM_, BN_, WM_, WN_, KB_, NSTG_, EPI_PARTIAL, MT_, BUF>), grid, block, lds, st, p);
}

// The bf16 tile kernel of plan pl (tile shape, MFMA shape, operand loads).
void launch_plan_bf16(GemmP p, const Plan& pl, int epi, dim3 grid, hipStream_t st) {
  if (pl.bm == 256 && pl.bn == 256) {
    if (buf_offsets_fit(p, 256))
      launch_bf16_gemm<256, 256, DFLASH_GEMM_BIG_WM, DFLASH_GEMM_BIG_WN, DFLASH_GEMM_KB_BIG, DFLASH_GEMM_NSTG_BIG,
                       DFLASH_GEMM_MT_BIG, true>(p, epi, grid, st);
    else
      launch_bf16_gemm<256, 256, DFLASH_GEMM_BIG_WM, DFLASH_GEMM_BIG_WN, DFLASH_GEMM_KB_BIG, DFLASH_GEMM_NSTG_BIG,
                       DFLASH_GEMM_MT_BIG>(p, epi, grid, st);
  }
  else if (pl.bm == 192) {
    if (buf_offsets_fit(p, 256))
      launch_bf16_gemm<192, 256, 2, 4, 64, 2, DFLASH_GEMM_MT_BIG, true>(p, epi, grid, st);
    else
      launch_bf16_gemm<192, 256, 2, 4, 64, 2, DFLASH_GEMM_MT_BIG>(p, epi, grid, st);
  }
  else if (pl.bm == 32)
    launch_bf16_gemm<32, 256, 1, 4, 64, 4, DFLASH_GEMM_MT_SMALL>(p, epi, grid, st);
  else if (pl.bm == 64)
    launch_bf16_gemm<64, 256, 1, 4, 64, 3, DFLASH_GEMM_MT_SMALL>(p, epi, grid, st);
  else if (pl.bm == 128 && pl.bn == 256)
    launch_bf16_gemm<128, 256, 2, 2, 64, 3, DFLASH_GEMM_MT_SMALL>(p, epi, grid, st);
  else if (pl.bm == 256)
    launch_bf16_gemm<256, 128, 2, 2, DFLASH_GEMM_KB_SMALL, DFLASH_GEMM_NSTG_SMALL, DFLASH_GEMM_MT_SMALL>(p, epi, grid, st);
  else
    launch_bf16_gemm<128, 128, 2, DFLASH_GEMM_SMALL_WN, DFLASH_GEMM_KB_SMALL, DFLASH_GEMM_NSTG_SMALL,
                     DFLASH_GEMM_MT_SMALL>(p, epi, grid, st);
}

void run_gemm(bool bf16, GemmP p, int epi_final, hipStream_t st) {
  const Plan pl = plan_gemm(p.M, p.N, p.K, bf16, p.b_layered ? p.HD : 0);
  p.ksplit = pl.ksplit;
  p.kchunk = pl.kchunk;
  const int epi = pl.ksplit > 1 ? EPI_PARTIAL : epi_final;
  if (bf16) {
    const dim3 grid((unsigned)(cdiv(p.M, pl.bm) * (p.N / pl.bn)), (unsigned)pl.ksplit);
    launch_plan_bf16(p, pl, epi, grid, st);
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

size_t partial_bytes(int64_t M, int64_t N, int64_t K, bool bf16, int64_t col_block = 0) {
  const Plan pl = plan_gemm(M, N, K, bf16, col_block);
  return pl.ksplit > 1 ? align256(sizeof(float) * pl.ksplit * M * N) : 0;
}

}  // namespace

size_t dense_gemm_ws_bytes(int64_t M, int64_t N, int64_t K, bool bf16) {
  if (bf16 && N > 256 && N % 256 == 128)
    return std::max(partial_bytes(M, N - 128, K, bf16), partial_bytes(M, 128, K, bf16));
  return partial_bytes(M, N, K, bf16);
}

hipError_t launch_dense_gemm(bool bf16, int M, int N, int K, const void* A, const void* B,
                             const void* bias, const void* resid, void* out, void* ws,
                             hipStream_t st) {
  // 256-column tiles need N % 256 == 0: a width of 256j + 128 runs as the
  // first 256j columns plus one 128-column strip (same output rows).
  const int tail = (bf16 && N > 256 && N % 256 == 128) ? 128 : 0;
  for (int part = 0; part < (tail ? 2 : 1); ++part) {
    const int c0 = part == 0 ? 0 : N - tail;
    const int n = tail ? (part == 0 ? N - tail : tail) : N;
    const int64_t es = bf16 ? 2 : 4;
    GemmP p{};
    p.M = M; p.N = n; p.K = K;
    p.a[0] = A;
    p.a_seg = K;
    p.b = static_cast<const char*>(B) + (int64_t)c0 * K * es; p.ldb = K;
    p.b_layered = 0;
    p.part = static_cast<float*>(ws);
    p.bias = bias ? static_cast<const char*>(bias) + c0 * es : nullptr;
    p.resid = resid ? static_cast<const char*>(resid) + c0 * es : nullptr;
    p.out = static_cast<char*>(out) + c0 * es;
    p.ldc = N;
    run_gemm(bf16, p, EPI_DENSE, st);
  }
  return hipGetLastError();
}

bool dense_gemm_splits(int M, int N, int K, bool bf16) {
  if (bf16 && N > 256 && N % 256 == 128) return false;
  return plan_gemm(M, N, K, bf16, 0).ksplit > 1;
}

hipError_t launch_dense_gemm_silu(bool bf16, int M, int I, int K, const void* A, const void* B, void* h,
                                  void* ws, hipStream_t st) {
  if (!dense_gemm_splits(M, 2 * I, K, bf16) || I % 8) return hipErrorInvalidValue;
  const Plan pl = plan_gemm(M, 2 * I, K, bf16, 0);
  GemmP p{};
  p.M = M; p.N = 2 * I; p.K = K;
  p.a[0] = A;
  p.a_seg = K;
  p.b = B; p.ldb = K;
  p.b_layered = 0;
  p.part = static_cast<float*>(ws);
  p.out = h;
  p.ldc = I;
  p.ksplit = pl.ksplit;
  p.kchunk = pl.kchunk;
  if (bf16) {
    const dim3 grid((unsigned)(cdiv(p.M, pl.bm) * (p.N / pl.bn)), (unsigned)pl.ksplit);
    launch_plan_bf16(p, pl, EPI_PARTIAL, grid, st);
  } else {
    const dim3 grid((unsigned)(cdiv(p.M, 64) * cdiv(p.N, 64)), (unsigned)pl.ksplit);
    hipLaunchKernelGGL(k_gemm_f32<EPI_PARTIAL>, grid, dim3(256), 0, st, p);
  }
  const unsigned blocks = (unsigned)std::min<int64_t>(cdiv((int64_t)M * I / 8, 256), 8192);
  if (bf16) hipLaunchKernelGGL(k_splitk_reduce_silu<uint16_t>, dim3(blocks), dim3(256), 0, st, p, I);
  else hipLaunchKernelGGL(k_splitk_reduce_silu<float>, dim3(blocks), dim3(256), 0, st, p, I);
  return hipGetLastError();
}

size_t materialize_ws_bytes(int64_t T, int m, int d, int n_layers, int Hkv, int D, bool bf16) {
  const int64_t es = bf16 ? 2 : 4;
  const size_t h = align256((size_t)(T * d * es));
  const size_t p1 = partial_bytes(T, d, (int64_t)m * d, bf16);
  // the K/V GEMM runs in groups of up to kML layers: size for every group
  // width that occurs (a narrower last group may plan more splits)
  const int64_t HD = (int64_t)Hkv * D;
  size_t p2 = partial_bytes(T, 2LL * std::min(n_layers, kML) * HD, d, bf16, HD);
  if (n_layers > kML && n_layers % kML)
    p2 = std::max(p2, partial_bytes(T, 2LL * (n_layers % kML) * HD, d, bf16, HD));
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
    p.ldc = a.d;
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
    p.D = a.D;
    p.part = part;
    p.bt = a.block_table;
    p.max_pages = a.max_pages;
    p.rows_per_seq = a.rows_per_seq;
    p.seq_start = a.seq_start;
    p.commit = a.commit_lens;
    run_gemm(bf16, p, EPI_PAGED, st);
    if (a.k_norm_on || a.rope_theta > 0.f) {
      KEpi e{};
      for (int l = 0; l < nl; ++l) e.w[l] = a.k_norm_w[l0 + l];
      e.eps = a.k_norm_eps;
      e.norm = a.k_norm_on ? 1 : 0;
      e.rope = a.rope_theta > 0.f ? 1 : 0;
      e.l2theta = a.rope_theta > 0.f ? std::log2((double)a.rope_theta) : 0.0;
      e.D = a.D;
      e.nl = nl;
      const int64_t threads = (int64_t)a.T * nl * (a.D / 8);
      const unsigned grid = (unsigned)std::min<int64_t>(cdiv(threads, 256), 16384);
      if (bf16) hipLaunchKernelGGL(k_k_epilogue<uint16_t>, dim3(grid), dim3(256), 0, st, p, e);
      else hipLaunchKernelGGL(k_k_epilogue<float>, dim3(grid), dim3(256), 0, st, p, e);
    }
  }
  return hipGetLastError();
}

}  // namespace dflash
