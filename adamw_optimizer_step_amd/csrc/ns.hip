// Newton-Schulz orthogonalisation kernels for gfx950.
//
// Per independent matrix (slice) the iteration X <- a X + (b A + c A^2) X,
// A = X X^T, runs on the short side (NorMuon paper section 2.2 eq. (5); OMN
// "Dual-Manifold Optimization", Muon-path paragraphs).  Every slice lives in a
// zero-padded pool as X (s x l, padded to the GEMM tile), with two iterate
// buffers used in turn.  The batched GEMM path runs per iteration:
//   Gram    P[i][j] = a [i == j] + b sum_k X[i][k] X[j][k]   (symmetric: tiles
//           i <= j, the lower triangle written as the mirror)
//   or      A = X X^T, then P = a I + b A + c A A (A symmetric: its own
//           transposed operand and its own E term)
//   Update  X'[i][n] = sum_k P[i][k] X[k][n], X read K-major through LDS
//           transpose reads; a X is folded into P's diagonal, so the update is
//           a plain product stored straight from registers.
// Zero padding stays zero through every product (a zero row of X gives a
// zero row of X X^T and of P X; a on a padded diagonal entry meets a zero row
// of X), so no bounds checks are needed inside the GEMM.  Head-sized slices
// (short side at most 128, bf16) run all iterations in one slice-resident
// kernel instead.
#include <atomic>
#include <type_traits>

#include <cstdlib>
#include <cstring>

#include "kernels.hpp"

namespace mo {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Statistics, scale and the padded, scaled copy X0 in both orientations.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_ns_stats(const PrepItem* __restrict__ items, int n,
                                                       StatPartial* __restrict__ partials) {
  const int64_t tile = blockIdx.x;
  const PrepItem it = items[find_segment(items, n, tile)];
  const int64_t lt = tile - it.start;
  const int r0 = static_cast<int>(lt / it.tiles_c) * kPrepTile;
  const int c0 = static_cast<int>(lt % it.tiles_c) * kPrepTile;
  const int col = c0 + (threadIdx.x & 63);
  float amax = 0.f;
  double ss = 0.0;
  for (int q = 0; q < kPrepTile / 4; ++q) {
    const int row = r0 + (threadIdx.x >> 6) + 4 * q;
    if (row < it.r && col < it.c) {
      const float v = fabsf(load_as_f32(it.in, static_cast<int64_t>(row) * it.ld_in + col, it.in_dt));
      amax = fmaxf(amax, v);
      ss += static_cast<double>(v) * v;
    }
  }
  block_stat_reduce(amax, ss, &partials[tile]);
}

__global__ __launch_bounds__(kThreads) void k_ns_scale(const PrepItem* __restrict__ items,
                                                       const StatPartial* __restrict__ partials,
                                                       float* __restrict__ scale,
                                                       int32_t* __restrict__ range_fb) {
  const PrepItem it = items[blockIdx.x];
  float amax = 0.f;
  double ss = 0.0;
  for (int64_t i = it.stat_begin + threadIdx.x; i < it.stat_end; i += kThreads) {
    amax = fmaxf(amax, partials[i].amax);
    ss += partials[i].sumsq;
  }
  __shared__ StatPartial red;
  block_stat_reduce(amax, ss, &red);
  __syncthreads();
  if (threadIdx.x == 0) {
    // X = D / alpha, X <- X / (||X||_F + 1e-7)  ==  D / (||D||_F + 1e-7 alpha)
    const double alpha = fmax(static_cast<double>(red.amax), 1e-7);
    scale[blockIdx.x] = static_cast<float>(1.0 / (sqrt(red.sumsq) + 1e-7 * alpha));
    // unscaled products D D^T (K <= 2^16 terms) stay normal fp32 numbers, and
    // s^2 too, while max|D| is in [2^-50, 2^40]
    if (range_fb)
      range_fb[blockIdx.x] = !(red.amax >= 0x1p-50f && red.amax <= 0x1p40f);
  }
}

template <typename T>
__device__ __forceinline__ T to_elem(float v);
template <>
__device__ __forceinline__ uint16_t to_elem<uint16_t>(float v) { return f32_to_bf16(v); }
template <>
__device__ __forceinline__ float to_elem<float>(float v) { return v; }

template <typename T>
__global__ __launch_bounds__(kThreads) void k_ns_final(const FinalItem* __restrict__ items, int n,
                                                       int64_t total_rows,
                                                       const T* __restrict__ pool) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  const FinalItem it = items[find_segment(items, n, row)];
  const int64_t r = row - it.start;
  const T* src = pool + it.src + r * it.ld_src;
  for (int c = lane; c < it.cols; c += 64) {
    float v;
    if constexpr (sizeof(T) == 2)
      v = bf16_to_f32(src[c]);
    else
      v = src[c];
    store_from_f32(it.out, r * it.ld_out + c, it.out_dt, v);
  }
}

// ---------------------------------------------------------------------------
// Batched NT GEMM on MFMA (32x32x16 bf16, or 32x32x2 fp32), templated on the
// workgroup tile BM x BN and the wave grid WM x WN (64 * WM * WN threads).
// Each wave owns a (BM/WM) x (BN/WN) sub-tile of FM x FN 32x32 blocks.  K is
// staged through LDS 128 bytes of every row at a time (64 bf16 / 32 fp32),
// double-buffered, with the next slab prefetched into registers while the
// current one is multiplied.  The LDS traffic per MFMA falls as the wave
// sub-tile grows: (FM + FN) fragment reads feed FM * FN MFMAs.
// ---------------------------------------------------------------------------
// LDS slabs of kRowB-byte rows (one K slab of A, or of B stored N x K):
// 16-byte chunk c of row r sits at chunk c ^ ((r >> kSh) & (chunks - 1)) with
// kSh = log2(256 / kRowB).  The LDS has 64 four-byte banks; the rows that
// share one 256-byte bank line differ in the bits below kSh, and XOR-ing the
// next bits spreads the 32 rows x one chunk of an MFMA operand read over all
// banks.  Measured on gfx950 with the LDS bank-conflict counter: no conflict
// cycles for these reads, where a row-parity swizzle doubles their cycles.
// Tile order inside one problem.  Non-symmetric problems go by groups of 8
// tile-rows (column-major inside a group), so the workgroups resident at one
// time share both operand row blocks; symmetric problems (upper triangle
// only) go by 4 x 4 super-tiles of the triangle.
constexpr int kGroupRows = 8;
constexpr int kXcdChunk = 32;
constexpr int kSuper = 4;

__device__ __forceinline__ void decode_tile(int t, int tm, int tn, int sym, int& ti, int& tj) {
  if (!sym) {
    const int per = kGroupRows * tn;
    const int g = t / per;
    const int first = g * kGroupRows;
    const int gsz = min(tm - first, kGroupRows);
    const int r = t - g * per;
    ti = first + r % gsz;
    tj = r / gsz;
    return;
  }
  const int ts = (tm + kSuper - 1) / kSuper;
  for (int bi = 0; bi < ts; ++bi) {
    const int hi = min(kSuper, tm - bi * kSuper);
    for (int bj = bi; bj < ts; ++bj) {
      const int wj = min(kSuper, tm - bj * kSuper);
      const int cnt = bi == bj ? hi * (hi + 1) / 2 : hi * wj;
      if (t < cnt) {
        if (bi == bj) {
          int i = 0, len = hi;
          while (t >= len) { t -= len; ++i; --len; }
          ti = bi * kSuper + i;
          tj = bi * kSuper + i + t;
        } else {
          ti = bi * kSuper + t / wj;
          tj = bj * kSuper + t % wj;
        }
        return;
      }
      t -= cnt;
    }
  }
  ti = tj = 0;  // unreachable for t inside the problem's tile count
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// s_waitcnt immediate (gfx9 encoding): vmcnt(n) (6 bits: [3:0] and [15:14]),
// lgkmcnt(0), expcnt not waited on.
constexpr int vm_wait_imm(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4); }

// Wait until at most min(younger, K) groups of INST vector-memory
// instructions are outstanding: an if / else chain tested from the largest
// count down, so the common case (younger >= K) takes one compare.
template <int K, int INST>
__device__ __forceinline__ void wait_vm_groups(int younger) {
  static_assert(K * INST <= 63, "vmcnt immediate");
  if constexpr (K == 0) {
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
  } else {
    if (younger >= K)
      __builtin_amdgcn_s_waitcnt(vm_wait_imm(K * INST));
    else
      wait_vm_groups<K - 1, INST>(younger);
  }
}

// Buffer resource (raw, stride 0) over `bytes` bytes from `base`; accesses
// past the range read zero instead of faulting.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes,
               0x00020000u};
}

// Direct-to-LDS load (buffer_load_dwordx4 ... lds): lane i's 16 bytes from
// base + voff + soff land at LDS byte lds_byte + 16 i.  M0, which carries the
// LDS address, is saved and restored around it.  The compiler does not see
// this as an LDS store: the caller waits for the vector memory counter and
// synchronises the workgroup before the data is read.
// NT: non-temporal hint, for data that no other workgroup reads from L2.
template <bool NT = false>
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t lds_byte, int voff,
                                          int soff) {
  // every operand but the lane offset must live in scalar registers
  u32x4 rs;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    rs[k] = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(rsrc[k])));
  const uint32_t lb =
      static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds_byte)));
  const int so = __builtin_amdgcn_readfirstlane(soff);
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen nt lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lb), "v"(voff), "s"(rs), "s"(so)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lb), "v"(voff), "s"(rs), "s"(so)
        : "memory");
}

template <typename T>
__device__ __forceinline__ void mma(const u32x4& a, const u32x4& b, f32x16& acc);

template <>
__device__ __forceinline__ void mma<uint16_t>(const u32x4& a, const u32x4& b, f32x16& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma<float>(const u32x4& a, const u32x4& b, f32x16& acc) {
  // Each lane group supplies 4 consecutive k per 16-byte chunk; component e
  // of A and of B go to the same MFMA, so the k ordering is consistent.
  const f32x4 fa = __builtin_bit_cast(f32x4, a);
  const f32x4 fb = __builtin_bit_cast(f32x4, b);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[0], fb[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[1], fb[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[2], fb[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[3], fb[3], acc, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ void ld8(const T* p, float* v);
template <>
__device__ __forceinline__ void ld8<uint16_t>(const uint16_t* p, float* v) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = __uint_as_float(u[k] << 16);
    v[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void ld8<float>(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int k = 0; k < 4; ++k) { v[k] = a[k]; v[4 + k] = b[k]; }
}

// 4 values to 4 consecutive elements (8 bytes of bf16, 16 of fp32).
template <typename T, bool NT = false>
__device__ __forceinline__ void st4(T* p, float v0, float v1, float v2, float v3) {
  if constexpr (sizeof(T) == 2) {
    const u32x2 u{pk_bf16(v0, v1),
                  pk_bf16(v2, v3)};
    if constexpr (NT)
      __builtin_nontemporal_store(u, reinterpret_cast<u32x2*>(p));
    else
      *reinterpret_cast<u32x2*>(p) = u;
  } else {
    const f32x4 a{v0, v1, v2, v3};
    if constexpr (NT)
      __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
    else
      *reinterpret_cast<f32x4*>(p) = a;
  }
}

// 8 values to 8 consecutive elements; NT = non-temporal (streaming) stores,
// for outputs that the same launch does not read again.
template <typename T, bool NT = false>
__device__ __forceinline__ void st8(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    u32x4 u;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      u[k] = pk_bf16(v[2 * k], v[2 * k + 1]);
    if constexpr (NT)
      __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
    else
      *reinterpret_cast<u32x4*>(p) = u;
  } else {
    const f32x4 a{v[0], v[1], v[2], v[3]}, b{v[4], v[5], v[6], v[7]};
    if constexpr (NT) {
      __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
      __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + 4));
    } else {
      *reinterpret_cast<f32x4*>(p) = a;
      *reinterpret_cast<f32x4*>(p + 4) = b;
    }
  }
}

template <typename T>
__device__ __forceinline__ void ld4(const T* p, float* v);
template <>
__device__ __forceinline__ void ld4<uint16_t>(const uint16_t* p, float* v) {
  const u32x2 u = *reinterpret_cast<const u32x2*>(p);
  v[0] = __uint_as_float(u[0] << 16);
  v[1] = __uint_as_float(u[0] & 0xffff0000u);
  v[2] = __uint_as_float(u[1] << 16);
  v[3] = __uint_as_float(u[1] & 0xffff0000u);
}
template <>
__device__ __forceinline__ void ld4<float>(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = a[k];
}

template <typename T>
__device__ __forceinline__ void st4(T* p, const float* v);
template <>
__device__ __forceinline__ void st4<uint16_t>(uint16_t* p, const float* v) {
  u32x2 u;
  u[0] = pk_bf16(v[0], v[1]);
  u[1] = pk_bf16(v[2], v[3]);
  *reinterpret_cast<u32x2*>(p) = u;
}
template <>
__device__ __forceinline__ void st4<float>(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

template <typename T>
__device__ __forceinline__ float from_elem(T v);
template <>
__device__ __forceinline__ float from_elem<uint16_t>(uint16_t v) { return bf16_to_f32(v); }
template <>
__device__ __forceinline__ float from_elem<float>(float v) { return v; }

// X0 = scale * D over one 64 x 64 tile of the padded stored orientation:
// 16-byte global accesses (8 elements per thread and row pass), zeros in the
// padding; tall slices go through an LDS tile and are written transposed.
// One 64 x 64 tile (number lt of item `it`) of X0 = s D into the pool, in
// the stored orientation (sbuf) or transposed through LDS (stbuf).
template <typename T>
__device__ __forceinline__ void prep_tile(const PrepItem& it, float sc, int64_t lt, T* pool,
                                          T (*tile_s)[kPrepTile + 2]) {
  const int r0 = static_cast<int>(lt / it.tiles_c) * kPrepTile;
  const int c0 = static_cast<int>(lt % it.tiles_c) * kPrepTile;
  const int lr = threadIdx.x >> 3, lc = (threadIdx.x & 7) * 8;
  float v[2][8];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int row = r0 + lr + 32 * k, col = c0 + lc;
    if (it.vec && row < it.r && col + 8 <= it.c) {
      load8(it.in, static_cast<int64_t>(row) * it.ld_in + col, it.in_dt, v[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[k][e] *= sc;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[k][e] = row < it.r && col + e < it.c
                      ? load_as_f32(it.in, static_cast<int64_t>(row) * it.ld_in + col + e,
                                    it.in_dt) * sc
                      : 0.f;
    }
  }
  if (it.sbuf >= 0) {  // uniform over the block
#pragma unroll
    for (int k = 0; k < 2; ++k)
      st8<T>(pool + it.sbuf + static_cast<int64_t>(r0 + lr + 32 * k) * it.cp + c0 + lc, v[k]);
    return;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) tile_s[lr + 32 * k][lc + e] = to_elem<T>(v[k][e]);
  __syncthreads();
  // output row = stored column c0 + lr + 32 k, 8 output columns = stored rows
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = from_elem<T>(tile_s[lc + e][lr + 32 * k]);
    st8<T>(pool + it.stbuf + static_cast<int64_t>(c0 + lr + 32 * k) * it.rp + r0 + lc, w);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_ns_prep(const PrepItem* __restrict__ items, int n,
                                                      const float* __restrict__ scale,
                                                      T* __restrict__ pool) {
  static_assert(kPrepTile == 64 && kThreads == 256, "prep tile split");
  __shared__ T tile_s[kPrepTile][kPrepTile + 2];
  const int64_t tile = blockIdx.x;
  const int idx = find_segment(items, n, tile);
  const PrepItem it = items[idx];
  if (it.sbuf < 0 && it.stbuf < 0) return;   // read in place
  prep_tile<T>(it, scale[idx], tile - it.start, pool, tile_s);
}

// The prep copy of the items whose range flag is set (see k_ns_scale): every
// workgroup checks the flags of kThreads items at a time, one per thread, and
// takes every gridDim.x-th tile of the flagged ones (none, normally).
__global__ __launch_bounds__(kThreads) void k_ns_prep_fb(const PrepItem* __restrict__ items,
                                                         int n, const float* __restrict__ scale,
                                                         const int32_t* __restrict__ range_fb,
                                                         uint16_t* __restrict__ pool) {
  __shared__ uint16_t tile_s[kPrepTile][kPrepTile + 2];
  for (int k0 = 0; k0 < n; k0 += kThreads) {
    const int mine = k0 + static_cast<int>(threadIdx.x);
    const int flagged = mine < n && range_fb[items[mine].slice] != 0;
    if (!__syncthreads_or(flagged)) continue;
    for (int k = k0; k < min(n, k0 + kThreads); ++k) {
      const PrepItem it = items[k];
      if (range_fb[it.slice] == 0) continue;   // uniform over the block
      const int64_t nt = static_cast<int64_t>(it.rp / kPrepTile) * it.tiles_c;
      const float sc = scale[it.slice];
      for (int64_t lt = blockIdx.x; lt < nt; lt += gridDim.x) {
        prep_tile<uint16_t>(it, sc, lt, pool, tile_s);
        __syncthreads();   // before the next tile reuses tile_s
      }
    }
  }
}

template <int N>
using Int = std::integral_constant<int, N>;

// f(Int<I>{}), ..., f(Int<N-1>{}) with compile-time indices.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<I + 1, N>(f);
  }
}

template <typename T, int BM, int BN, int WM, int WN, bool BK, int ST = 4, int SRB = 64>
struct GemmCfg {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kWaves = WM * WN;
  static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
  static constexpr int FM = kWaveM / 32, FN = kWaveN / 32;
  // K slab: SRB-byte rows (64: 32 bf16 / 16 fp32 of k; 128: twice that); ST
  // LDS stages (a power of two), ST - 1 slabs in flight
  static constexpr int kRowB = SRB;
  static_assert(SRB == 64 || SRB == 128, "slab rows of 64 or 128 bytes");
  static constexpr int kStages = ST;
  static_assert(ST >= 2 && (ST & (ST - 1)) == 0, "stage count is a power of two");
  static constexpr int kSub = kRowB / 32;                   // 16-k substeps per slab
  static constexpr int kChunks = kRowB / 16;                // 16-byte chunks per row
  static constexpr int kSh = kRowB == 64 ? 2 : 1;           // swizzle shift
  static constexpr int kSlabK = kRowB / static_cast<int>(sizeof(T));
  // Slabs are filled by direct-to-LDS loads: one instruction moves 64 lanes x
  // 16 bytes into 1 KiB of contiguous LDS.  A (and B stored N x K): 1024 / kRowB
  // rows per instruction.  B stored K x N (BK): rows of BN elements.
  static constexpr int kRowsPerInst = 1024 / kRowB;
  static constexpr int kBkRowBytes = BN * static_cast<int>(sizeof(T));
  static constexpr int kBkRowsPerInst = 1024 / kBkRowBytes;
  static constexpr int kBkChunksPerRow = kBkRowBytes / 16;
  static constexpr int kInstA = BM * kRowB / 1024 / kWaves;    // per wave and slab
  static constexpr int kBStageBytes = BK ? kSlabK * kBkRowBytes : BN * kRowB;
  static constexpr int kInstB = kBStageBytes / 1024 / kWaves;
  static constexpr int kInst = kInstA + kInstB;
  static constexpr int kStageBytes = BM * kRowB + kBStageBytes;
  static constexpr int kBandLd = BN + 4;                    // epilogue band stride (floats)
  static constexpr int kBandBytes = kWaveM / 2 * kBandLd * 4;   // one epilogue band of C
  static constexpr int kLdsBytes =
      kStages * kStageBytes > kBandBytes ? kStages * kStageBytes : kBandBytes;
  static_assert(FM >= 1 && FN >= 1 && kInstA >= 1 && kInstB >= 1, "bad tile");
  static_assert(kInstA * kWaves * 1024 == BM * kRowB, "A slab split");
  static_assert(kInstB * kWaves * 1024 == kBStageBytes, "B slab split");
  static_assert(!BK || (kBkRowsPerInst >= 1 && kBkRowsPerInst * kBkRowBytes == 1024),
                "K-major B rows per instruction");
  static_assert(kInst <= 31, "vector-memory wait counts below assume at most 31 loads per slab");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget of a gfx950 CU");
};

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element
// (i & 3) of the 4-element words addressed by lanes 4e + (i >> 2), e = 0..3.
// With lane j pointing at row k0 + (j >> 2), columns n0 + 4 (j & 3) .. + 3 of
// a K x N row-major array, lane i therefore gets column n0 + i, rows
// k0 .. k0 + 3: an MFMA B fragment piece read from K-major data.  A lane's
// result depends on the addresses of other lanes, so all 16 lanes of a group
// must execute it (never under a lane-dependent branch).
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Logical tile `bid` of a launch of G logical tiles (k_ns_gemm's body).
template <typename T, int BM, int BN, int WM, int WN, bool BK, int ST, int SRB>
__device__ __forceinline__ void ns_gemm_tile(
    const int bid, const int G,
    const GemmProb* __restrict__ probs, int nprob, T* __restrict__ pool, float c0, float c1_arg,
    int has_e, float cd, const RowSeg* __restrict__ wt, float lr_arg,
    const float* __restrict__ lrs, const float* __restrict__ pscale,
    const int32_t* __restrict__ pfb, float c1b_arg, float cdb) {
  using C = GemmCfg<T, BM, BN, WM, WN, BK, ST, SRB>;
  constexpr int NT = C::kThreads, FM = C::FM, FN = C::FN;
  __shared__ __attribute__((aligned(16))) char smem[C::kLdsBytes];
  // XCD-aware order: consecutive workgroup ids go round-robin over the 8
  // XCDs.  Each XCD receives chunks of kXcdChunk consecutive logical tiles
  // (neighbouring tiles share operand panels in that XCD's L2), the chunks
  // dealt round-robin so that every XCD gets a similar mix of long and short
  // problems; the last partial round is split into contiguous runs.
  const int xcd = bid & 7, ord = bid >> 3;
  const int full = G / (8 * kXcdChunk);
  int tile;
  if (ord < full * kXcdChunk) {
    tile = ((ord / kXcdChunk) * 8 + xcd) * kXcdChunk + ord % kXcdChunk;
  } else {
    const int rest = G - full * 8 * kXcdChunk;
    const int q8 = rest >> 3, r8 = rest & 7;
    tile = full * 8 * kXcdChunk + xcd * q8 + min(xcd, r8) + (ord - full * kXcdChunk);
  }
  const GemmProb pr = probs[find_segment(probs, nprob, tile)];
  int ti, tj;
  decode_tile(tile - pr.start, pr.tiles_m, pr.tiles_n, pr.sym, ti, tj);
  // iteration 0 on the unscaled input D: (s D)(s D)^T = s^2 D D^T for the
  // Gram, P (s D) = s P D for the update; a slice whose range flag is set
  // reads the prepared X0 (alt_off) as later iterations do
  float c1 = c1_arg, c1b = c1b_arg;
  int64_t a_off = pr.a_off, b_off = pr.b_off;
  if (pscale != nullptr && pr.sitem >= 0) {
    if (pfb != nullptr && pfb[pr.sitem] != 0) {
      if (!BK) a_off = pr.alt_off;
      b_off = pr.alt_off;
    } else {
      const float sc = pscale[pr.sitem];
      c1 = BK ? c1_arg * sc : c1_arg * (sc * sc);
      c1b = c1b_arg * (sc * sc);
    }
  }

  // (opaque per tile in a persistent kernel, which then recomputes the
  // per-lane offsets below for each tile rather than holding them in
  // registers across the whole tile)
  int tid = threadIdx.x;
  if constexpr (BM == kGemmTile) asm volatile("" : "+v"(tid));
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int fr = lane & 31, fg = lane >> 5;
  static_assert(FM % 2 == 0, "wave tiles span an even number of 32-row blocks");
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave index as a scalar

  // Global -> LDS through buffer resources (hardware range-checked).  A (and
  // B stored N x K) spans this tile's operand rows; the K slab goes into the
  // scalar offset.  B stored K x N spans the columns tj*BN.. of the slab's
  // kSlabK rows; its resource moves with the slab so offsets stay small.
  const uint32_t lda_b = static_cast<uint32_t>(pr.lda) * sizeof(T);
  const uint32_t ldb_b = static_cast<uint32_t>(pr.ldb) * sizeof(T);
  const char* abase = reinterpret_cast<const char*>(pool + a_off) +
                      static_cast<size_t>(ti) * BM * lda_b;
  // In 128 x 128 tiles, A's resource (and B's, stored N x K) ends at the
  // operand's last row that holds data (a_rows, b_rows): rows past it (a
  // slice's padding) read zero without a memory access, and a slice read in
  // place needs no padded copy.  (The K slab's offset goes in the scalar
  // offset, outside the range check; rows are in the lane offset, inside it.)
  // K-major B needs no such limit: K stops at the last slab holding data, and
  // a slice read in place has a multiple of the slab depth as its K (no
  // per-slab arithmetic in the loop, where it cost 1%).  The 256 x 256 tiles
  // read whole tiles: their slices are read in place only unpadded, and the
  // limit's scalar registers cost them 0.3%.
  auto rows_in = [](int32_t valid, int first, int n) __attribute__((always_inline)) {
    if constexpr (BM == kGemmTile) return valid > 0 ? max(0, min(n, valid - first)) : n;
    else return n;
  };
  const u32x4 rsa = buffer_rsrc(abase, rows_in(pr.a_rows, ti * BM, BM) * lda_b);
  const char* bbase = BK ? reinterpret_cast<const char*>(pool + b_off + tj * BN)
                         : reinterpret_cast<const char*>(pool + b_off) +
                               static_cast<size_t>(tj) * BN * ldb_b;
  const int rows_b = BK ? 0 : rows_in(pr.b_rows, tj * BN, BN);
  auto rsb_at = [&](int kt) __attribute__((always_inline)) {
    if constexpr (BK)
      return buffer_rsrc(bbase + static_cast<size_t>(kt) * C::kSlabK * ldb_b, C::kSlabK * ldb_b);
    else
      return buffer_rsrc(bbase, rows_b * ldb_b);
  };

  // LDS slab layout (kRowB-byte rows): chunk c of row r at chunk
  // c ^ swz(r).  Load instruction t of the workgroup fills rows
  // kRowsPerInst * t .. + kRowsPerInst - 1; lane i lands at row + i / kChunks,
  // physical chunk i % kChunks, so it fetches logical chunk
  // (i % kChunks) ^ swz(row).
  auto swz = [](int r) __attribute__((always_inline)) {
    return (r >> C::kSh) & (C::kChunks - 1);
  };
  int voa[C::kInstA], vob[C::kInstB];
#pragma unroll
  for (int q = 0; q < C::kInstA; ++q) {
    const int row = (wv * C::kInstA + q) * C::kRowsPerInst + lane / C::kChunks;
    voa[q] = static_cast<int>(row * lda_b) + (((lane % C::kChunks) ^ swz(row)) << 4);
  }
  // B stored K x N: row r of the slab (kBkRowBytes bytes) holds 16-byte chunk
  // c at c ^ ((r & 3) << 2) (bf16; the four rows read together by a
  // transpose read then use four different 64-byte bank windows).
  auto bk_swz = [](int r) __attribute__((always_inline)) {
    return sizeof(T) == 2 ? (r & 3) << 2 : 0;
  };
#pragma unroll
  for (int q = 0; q < C::kInstB; ++q) {
    if constexpr (BK) {
      const int row = (wv * C::kInstB + q) * C::kBkRowsPerInst + lane / C::kBkChunksPerRow;
      vob[q] = static_cast<int>(row * ldb_b) +
               (((lane % C::kBkChunksPerRow) ^ bk_swz(row)) << 4);
    } else {
      const int row = (wv * C::kInstB + q) * C::kRowsPerInst + lane / C::kChunks;
      vob[q] = static_cast<int>(row * ldb_b) + (((lane % C::kChunks) ^ swz(row)) << 4);
    }
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(smem))));
  // all direct-to-LDS loads of slab kt into `stage` (kInst per wave)
  auto issue_a = [&](int kt, int stage) __attribute__((always_inline)) {
    const uint32_t sb = lds0 + stage * C::kStageBytes;
#pragma unroll
    for (int q = 0; q < C::kInstA; ++q)
      lds_dma16(rsa, sb + (wv * C::kInstA + q) * 1024, voa[q], kt * C::kRowB);
  };
  auto issue_b = [&](int kt, int stage) __attribute__((always_inline)) {
    const uint32_t sb = lds0 + stage * C::kStageBytes;
    const u32x4 rsb = rsb_at(kt);
#pragma unroll
    for (int q = 0; q < C::kInstB; ++q)
      lds_dma16(rsb, sb + BM * C::kRowB + (wv * C::kInstB + q) * 1024, vob[q],
                BK ? 0 : kt * C::kRowB);
  };
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    issue_a(kt, stage);
    issue_b(kt, stage);
  };

  // Fragment reads.  A / NxK B: lane reads row (wave row base + fr), logical
  // chunk 2 ks + fg; the row offsets added are multiples of 32, so the
  // swizzle is a per-thread constant.  KxN B (bf16): transpose reads, lane j
  // of 16-lane group g covering rows 16 ks + 8 (g / 2) + 4 h + j / 4 and
  // columns wn * kWaveN + 32 ni + 16 (g % 2) + 4 (j % 4); fp32: rows
  // 8 ks + 4 fg + e, column wn * kWaveN + 32 ni + fr.
  const int f_r = swz(fr);
  const int rd_a = (wm * C::kWaveM + fr) * C::kRowB;
  const int rd_b = BM * C::kRowB + (wn * C::kWaveN + fr) * C::kRowB;
  auto rd_chunk = [&](int ks) __attribute__((always_inline)) {
    return ((ks * 2 + fg) ^ f_r) << 4;
  };
  const int g16 = lane >> 4, j16 = lane & 15;
  int rd_bk[FN];
#pragma unroll
  for (int ni = 0; ni < FN; ++ni) {
    if constexpr (sizeof(T) == 2) {
      const int row = 8 * (g16 >> 1) + (j16 >> 2);
      const int colb = (wn * C::kWaveN + ni * 32 + 16 * (g16 & 1) + 4 * (j16 & 3)) * 2;
      rd_bk[ni] = BM * C::kRowB + row * C::kBkRowBytes +
                  (((colb >> 4) ^ bk_swz(row)) << 4) + (colb & 15);
    } else {
      rd_bk[ni] = BM * C::kRowB + 4 * fg * C::kBkRowBytes + (wn * C::kWaveN + ni * 32 + fr) * 4;
    }
  }

  f32x16 acc[FM][FN];
#pragma unroll
  for (int mi = 0; mi < FM; ++mi)
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  // Operand fragments of one k-substep (32 bytes of every row); two sets so
  // that the reads of the next substep are in flight while one is multiplied.
  u32x4 av[2][FM], bv[2][FN];
  auto fload = [&](int stage, int ks, auto setc) __attribute__((always_inline)) {
    constexpr int set = decltype(setc)::value;
    const char* base = smem + stage * C::kStageBytes;
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
      av[set][mi] = *reinterpret_cast<const u32x4*>(base + rd_a + mi * 32 * C::kRowB +
                                                    rd_chunk(ks));
    if constexpr (!BK) {
#pragma unroll
      for (int ni = 0; ni < FN; ++ni)
        bv[set][ni] = *reinterpret_cast<const u32x4*>(base + rd_b + ni * 32 * C::kRowB +
                                                      rd_chunk(ks));
    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) {
        const char* p = base + rd_bk[ni] + ks * 16 * C::kBkRowBytes;
        const u32x2 lo = lds_read_tr16(p);
        const u32x2 hi = lds_read_tr16(p + 4 * C::kBkRowBytes);
        bv[set][ni] = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    } else {
#pragma unroll
      for (int ni = 0; ni < FN; ++ni) {
        const char* p = base + rd_bk[ni] + ks * 8 * C::kBkRowBytes;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bv[set][ni][e] = *reinterpret_cast<const uint32_t*>(p + e * C::kBkRowBytes);
      }
    }
  };
  // The update (K-major B) writes C = A B row-major from registers: with the
  // operands swapped (SW), the MFMA produces C^T tiles, whose lane layout
  // holds 4 consecutive columns of one row of C.  A problem with a transposed
  // output (ct_off) keeps the plain order, whose lanes hold 4 consecutive rows
  // of one column of C, i.e. 4 consecutive elements of a row of C^T.  The
  // order is a compile-time choice: the main loop exists once per order.
  auto mfma_block = [&](auto setc, auto swc) __attribute__((always_inline)) {
    constexpr int set = decltype(setc)::value;
    if constexpr (decltype(swc)::value) {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) mma<T>(bv[set][ni], av[set][mi], acc[mi][ni]);
    } else {
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni) mma<T>(av[set][mi], bv[set][ni], acc[mi][ni]);
    }
  };
  // Wait until this wave's loads of all but the `younger` most recent slabs
  // have landed (the direct-to-LDS loads are counted by the vector memory
  // counter, kInst per slab, completing in order) and its LDS reads are done
  // (the stage they read is refilled after the next barrier).
  auto wait_slab = [](int younger) __attribute__((always_inline)) {
    wait_vm_groups<C::kStages - 2, C::kInst>(younger);
  };
  // Software pipeline over K slabs (kSub = 2 or 4 substeps of 16 k), two
  // fragment register sets used in turn, S = kStages LDS stages with the
  // loads of S - 1 slabs in flight.  Per slab kt (shown for kSub = 2):
  //   loads of slab kt+S-1 into stage (kt+S-1) % S (last read in slab kt-1,
  //   which ended with a barrier)
  //   read frags ks1              | MFMAs ks0
  //   wait for slab kt+1; barrier
  //   read frags ks0 of slab kt+1 | MFMAs ks1
  // With two stages the slab's loads are the only ones in flight, so they
  // are issued as early as the stage allows: right after the barrier that
  // ends slab kt - 1 (the barrier waits for every wave's LDS reads), before
  // that slab's last MFMAs, which gives them a whole slab of MFMAs to land
  // (1% faster on the dense decoder's launches; the four-stage launches of
  // few tiles ran 2.5% slower that way and keep the issue at the slab start).
  static_assert(C::kSub % 2 == 0, "an even number of substeps per slab");
  constexpr bool kEarly = C::kStages == 2;
  // 256 x 256 tiles issue those loads in two halves: A's right after the
  // barrier, B's at the start of the next slab, once the slab's last MFMAs
  // are issued.  The dense-decoder launches ran 4% faster than with all of a
  // wave's loads issued at the barrier (B a substep later, or the loads in
  // four parts, were no faster or slower); the 128 x 128 tiles gained
  // nothing and issue them together.
  constexpr bool kSplitIssue = kEarly && BM == 256;
  const int KT = pr.K / C::kSlabK;
  // slab_hook(kt, stage): called at the start of slab kt, whose stage is
  // complete in LDS and stays intact until the barrier of that slab
  auto main_loop = [&](auto swc, auto slab_hook) __attribute__((always_inline)) {
    const int pre = KT < C::kStages - 1 ? KT : C::kStages - 1;
    for (int k = 0; k < pre; ++k) issue(k, k);
    wait_slab(pre - 1);
    __syncthreads();
    if (kEarly && C::kStages - 1 < KT) issue(C::kStages - 1, C::kStages - 1);
    fload(0, 0, Int<0>{});
    int pend_b = -1;   // slab whose B half is still to be issued (split issue)
    for (int kt = 0; kt < KT; ++kt) {
      const int stage = kt & (C::kStages - 1);
      if (kSplitIssue && pend_b >= 0) {
        issue_b(pend_b, pend_b & (C::kStages - 1));
        pend_b = -1;
      }
      if (!kEarly && kt + C::kStages - 1 < KT)
        issue(kt + C::kStages - 1, (kt + C::kStages - 1) & (C::kStages - 1));
      slab_hook(kt, stage);
      __builtin_amdgcn_sched_barrier(0);
      // substep ks multiplies set ks & 1 while the next substep's fragments
      // load into the other set; before the last substep, wait for slab
      // kt + 1 and load its first substep
      static_for<0, C::kSub>([&](auto ksc) {
        constexpr int ks = decltype(ksc)::value;
        if constexpr (ks + 1 < C::kSub) {
          fload(stage, ks + 1, Int<(ks + 1) & 1>{});
        } else {
          const int last = min(KT - 1, kt + C::kStages - 1);
          wait_slab(last - (kt + 1));
          __syncthreads();
          // slab kt's stage is free from here: it takes slab kt + S
          if (kEarly && kt + C::kStages < KT) {
            if constexpr (kSplitIssue) {
              issue_a(kt + C::kStages, stage);
              pend_b = kt + C::kStages;
            } else {
              issue(kt + C::kStages, stage);
            }
          }
          if (kt + 1 < KT) fload((kt + 1) & (C::kStages - 1), 0, Int<0>{});
        }
        if constexpr (ks + 1 < C::kSub && sizeof(T) == 2) {
          // (bf16) the next substep's fragment reads interleaved with this
          // one's MFMAs, alternately one LDS read (scheduling group 0x100)
          // and one MFMA (0x008), rather than all reads first: the dense
          // decoder's GEMM launches 1.3% faster
          constexpr int kReads = FM + (BK ? 2 * FN : FN), kMf = FM * FN;
          constexpr int kPairs = kReads < kMf ? kReads : kMf;
          mfma_block(Int<ks & 1>{}, swc);
          static_for<0, kPairs>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          });
          if constexpr (kReads > kPairs) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kPairs, 0);
          if constexpr (kMf > kPairs) __builtin_amdgcn_sched_group_barrier(0x008, kMf - kPairs, 0);
        } else {
          __builtin_amdgcn_sched_barrier(0);
          mfma_block(Int<ks & 1>{}, swc);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  };

  if constexpr (BK) {
    // Update epilogue.  32x32 MFMA output: lane l holds column l % 32 and rows
    // 8 (v / 4) + 4 (l / 32) + v % 4 of its tile, which with swapped operands
    // is a tile of C^T: 4 consecutive columns of one row of C per lane (and,
    // in plain order, 4 consecutive elements of one row of C^T).  bf16: the
    // whole output tile (row-major C, or C^T for a transposed output) is
    // staged once in LDS, rows of BN * 2 bytes with 16-byte chunk c at
    // c ^ row (8-byte writes of 32 rows and 16-byte reads of a row are both
    // conflict-free), then every 32 lanes store one contiguous row segment.
    // fp32: 16-byte stores straight from registers.  The output is read only
    // by the next launch: streaming stores.
    const bool to_c = pr.ct_off < 0;
    auto none = [](int, int) __attribute__((always_inline)) {};
    if (to_c)
      main_loop(std::true_type{}, none);
    else
      main_loop(std::false_type{}, none);
    // tile-local (row, col) of value 4q of acc[mi][ni] in the staged tile
    auto at = [&](int mi, int ni, int q, int& r, int& c) __attribute__((always_inline)) {
      const int m = wm * C::kWaveM + mi * 32, n = wn * C::kWaveN + ni * 32;
      if (to_c) { r = m + fr; c = n + 8 * q + 4 * fg; }
      else      { r = n + fr; c = m + 8 * q + 4 * fg; }
    };
    if constexpr (sizeof(T) == 2) {
      static_assert(BM == BN, "square output tiles");
      constexpr int RB = BN * 2, NCH = RB / 16;
      static_assert(BM * RB <= C::kLdsBytes, "staged output tile fits the stages");
      __syncthreads();   // every wave is done reading the operand stages
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int r, c;
            at(mi, ni, q, r, c);
            const f32x16& a = acc[mi][ni];
            const u32x2 u{pk_bf16(c1 * a[4 * q], c1 * a[4 * q + 1]),
                          pk_bf16(c1 * a[4 * q + 2], c1 * a[4 * q + 3])};
            *reinterpret_cast<u32x2*>(smem + r * RB + ((((c >> 3) ^ r) & (NCH - 1)) << 4) +
                                      (c & 7) * 2) = u;
          }
      __syncthreads();
      if (wt != nullptr && pr.item >= 0) {
        // last update of a slice: apply the Muon step to its weights from the
        // staged (bf16-rounded) output tile, rows and columns in the weight's
        // stored orientation, clipped to the slice's real extent
        // (every weight load of the thread is issued before the first update)
        const RowSeg w = wt[pr.item];
        const int orow0 = to_c ? ti * BM : tj * BN, ocol0 = to_c ? tj * BN : ti * BM;
        const float lr = lrs ? lrs[w.lr_slot] : lr_arg;
        const float decay = 1.f - lr * w.wd, coef = lr * w.scale;
        constexpr int NP = BM * NCH / NT;
        W8 wr[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int idx = p * NT + tid, r = idx / NCH, c = idx % NCH;
          const int orow = orow0 + r, ocol = ocol0 + c * 8;
          if (orow < w.rows && ocol < w.cols)
            wr[p] = load_w8(w.w, static_cast<int64_t>(orow) * w.ld_w + ocol, w.w_dt);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int idx = p * NT + tid, r = idx / NCH, c = idx % NCH;
          const int orow = orow0 + r, ocol = ocol0 + c * 8;
          if (orow < w.rows && ocol < w.cols) {
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(smem + r * RB + (((c ^ r) & (NCH - 1)) << 4));
            apply_w8(w.w, static_cast<int64_t>(orow) * w.ld_w + ocol, w.w_dt, wr[p], v, decay,
                     coef);
          }
        }
        return;
      }
      T* const g = to_c ? pool + pr.c_off + static_cast<size_t>(ti * BM) * pr.ldc + tj * BN
                        : pool + pr.ct_off + static_cast<size_t>(tj * BN) * pr.ldct + ti * BM;
      const size_t ld = to_c ? pr.ldc : pr.ldct;
#pragma unroll
      for (int p = 0; p < BM * NCH / NT; ++p) {
        const int idx = p * NT + tid, r = idx / NCH, c = idx % NCH;
        const u32x4 v = *reinterpret_cast<const u32x4*>(smem + r * RB + (((c ^ r) & (NCH - 1)) << 4));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(g + r * ld + c * 8));
      }
    } else {
      T* const g = to_c ? pool + pr.c_off + static_cast<size_t>(ti * BM) * pr.ldc + tj * BN
                        : pool + pr.ct_off + static_cast<size_t>(tj * BN) * pr.ldct + ti * BM;
      const size_t ld = to_c ? pr.ldc : pr.ldct;
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int r, c;
            at(mi, ni, q, r, c);
            const f32x16& a = acc[mi][ni];
            st4<T>(g + r * ld + c, c1 * a[4 * q], c1 * a[4 * q + 1], c1 * a[4 * q + 2],
                   c1 * a[4 * q + 3]);
          }
    }
    return;
  } else {
    if constexpr (sizeof(T) == 2) {
      // has_e == 2: the E term is the product's own left factor (E = U, as
      // for T = a A + b A A), so E's tile (ti, tj) is the A operand's slab
      // of columns tj * BN .. and passes through LDS in the K loop: each wave
      // adds (c0 / c1) E to its accumulators from the one slab holding its
      // columns, and the product takes the epilogue below.
      // (compiled into the two-stage variants only: the few-tile variant's
      // launches read E, and an extra copy of its K loop measured slower)
      const bool e_in_loop = ST == 2 && has_e == 2 && c1 != 0.f && pr.c2_off < 0;
      if (!has_e || e_in_loop) {
        // Gram epilogue (bf16): with swapped operands each lane holds 4
        // consecutive columns of one row of the tile.  The tile c1 C + cd I
        // is staged once in LDS as bf16 (layout as in the update epilogue);
        // C's rows are stored as contiguous row segments, and the mirror (the
        // transposed tile, for the lower triangle) is read with transpose
        // reads: per 16-lane group, two reads give lane i 8 consecutive
        // elements of row n0 + i of C^T, and the 4 groups of a wave cover 32
        // consecutive columns, 64 contiguous bytes per row.
        if constexpr (ST != 2) {
          main_loop(std::true_type{}, [](int, int) __attribute__((always_inline)) {});
        } else if (e_in_loop) {
          // (separate copies of the K loop for the two cases)
          const float eratio = c0 / c1;
          const int e_col0 = tj * BN + wn * C::kWaveN;   // the wave's first column
          static_assert(C::kSlabK % C::kWaveN == 0, "a wave's columns lie in one K slab");
          const int kt_e = e_col0 / C::kSlabK, kk0 = e_col0 - kt_e * C::kSlabK;
          main_loop(std::true_type{}, [&](int kt, int stage) __attribute__((always_inline)) {
            if (kt != kt_e) return;
            const char* const slab = smem + stage * C::kStageBytes;   // A rows first
#pragma unroll
            for (int mi = 0; mi < FM; ++mi)
#pragma unroll
              for (int ni = 0; ni < FN; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  // acc[mi][ni][4 q + e] = C[r][c + e]: E[r][c + e] = U[row r][k = kk + e]
                  const int r = wm * C::kWaveM + mi * 32 + fr;
                  const int kk = kk0 + ni * 32 + 8 * q + 4 * fg;
                  const u32x2 ev = *reinterpret_cast<const u32x2*>(
                      slab + r * C::kRowB + ((((kk >> 3) ^ swz(r)) & (C::kChunks - 1)) << 4) +
                      (kk & 7) * 2);
                  acc[mi][ni][4 * q] += eratio * __uint_as_float(ev[0] << 16);
                  acc[mi][ni][4 * q + 1] += eratio * __uint_as_float(ev[0] & 0xffff0000u);
                  acc[mi][ni][4 * q + 2] += eratio * __uint_as_float(ev[1] << 16);
                  acc[mi][ni][4 * q + 3] += eratio * __uint_as_float(ev[1] & 0xffff0000u);
                }
          });
        } else {
          main_loop(std::true_type{}, [](int, int) __attribute__((always_inline)) {});
        }
        static_assert(BM == BN, "square output tiles");
        constexpr int RB = BN * 2, NCH = RB / 16;
        static_assert(BM * RB <= C::kLdsBytes, "staged output tile fits the stages");
        auto soff = [](int r, int c) __attribute__((always_inline)) {
          return r * RB + ((((c >> 3) ^ r) & (NCH - 1)) << 4) + (c & 7) * 2;
        };
        const bool diag = ti == tj;
        // stage cc1 C + ccd I and store it to `off_c` (rows) and, for the
        // lower triangle, to `off_ct` (mirror)
        auto emit = [&](float cc1, float ccd, int64_t off_c, int64_t off_ct)
            __attribute__((always_inline)) {
#pragma unroll
          for (int mi = 0; mi < FM; ++mi)
#pragma unroll
            for (int ni = 0; ni < FN; ++ni)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int r = wm * C::kWaveM + mi * 32 + fr;
                const int c = wn * C::kWaveN + ni * 32 + 8 * q + 4 * fg;
                float x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  x[e] = cc1 * acc[mi][ni][4 * q + e] + (diag && r == c + e ? ccd : 0.f);
                const u32x2 u{pk_bf16(x[0], x[1]),
                              pk_bf16(x[2], x[3])};
                *reinterpret_cast<u32x2*>(smem + soff(r, c)) = u;
              }
          __syncthreads();
          if (off_c >= 0) {
            T* const g = pool + off_c + static_cast<size_t>(ti * BM) * pr.ldc + tj * BN;
#pragma unroll
            for (int p = 0; p < BM * NCH / NT; ++p) {
              const int idx = p * NT + tid, r = idx / NCH, c = idx % NCH;
              *reinterpret_cast<u32x4*>(g + static_cast<size_t>(r) * pr.ldc + c * 8) =
                  *reinterpret_cast<const u32x4*>(smem + r * RB + (((c ^ r) & (NCH - 1)) << 4));
            }
          }
          if (off_ct >= 0 && !(pr.sym && diag)) {
            T* const g = pool + off_ct + static_cast<size_t>(tj * BN) * pr.ldct + ti * BM;
            constexpr int kUnits = (BN / 16) * (BM / 32);   // 16 rows x 32 columns of C^T
            static_assert(kUnits % C::kWaves == 0, "mirror units per wave");
            for (int u = wv; u < kUnits; u += C::kWaves) {
              const int n0 = (u % (BN / 16)) * 16, k0 = (u / (BN / 16)) * 32 + 8 * g16;
              const int col = n0 + 4 * (j16 & 3);
              const u32x2 lo = lds_read_tr16(smem + soff(k0 + (j16 >> 2), col));
              const u32x2 hi = lds_read_tr16(smem + soff(k0 + 4 + (j16 >> 2), col));
              *reinterpret_cast<u32x4*>(g + static_cast<size_t>(n0 + j16) * pr.ldct + k0) =
                  u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
          }
        };
        __syncthreads();   // every wave is done reading the operand stages
        emit(c1, cd, pr.c_off, pr.ct_off);
        if (pr.c2_off >= 0) {
          // second output of the same product (same layout and mirror):
          // c1b C + cdb I, e.g. A = X X^T and P = a I + b A together
          __syncthreads();   // the staged tile has been read
          emit(c1b, cdb, pr.c2_off, pr.c2_off);
        }
        return;
      }
    }
    main_loop(std::false_type{}, [](int, int) __attribute__((always_inline)) {});
  }
  __syncthreads();

  // Epilogue, one band of kWaveM / 2 rows (half of one row of waves) at a
  // time: the band's waves stage their fp32 accumulators in LDS, then all
  // threads make coalesced direct stores (with the E term) and, when asked,
  // write the values back for the transposed stores.  32x32 MFMA output: lane l holds column l % 32 and rows
  // 8 (v / 4) + 4 (l / 32) + v % 4 for v = 0..15.
  float* cs = reinterpret_cast<float*>(smem);
  const bool need_c = pr.c_off >= 0;
  const bool need_t = pr.ct_off >= 0 && !(pr.sym && ti == tj);
  constexpr int HM = FM / 2;                 // 32-row blocks per band
  constexpr int BR = HM * 32;                // band rows
  constexpr int kIters = (BR * BN) / (NT * 8);
  static_assert(FM % 2 == 0 && kIters >= 1 && (BR * BN) % (NT * 8) == 0, "epilogue split");
  // bf16: the whole tile's E values are requested before the first store
  // (the compiler orders a load after every earlier store it cannot prove
  // disjoint, so loads issued between bands would wait for their stores).
  u32x4 er[2 * WM][kIters];
  if constexpr (sizeof(T) == 2) {
    if (has_e) {
#pragma unroll
      for (int band = 0; band < 2 * WM; ++band) {
        const T* eg = pool + pr.e_off + static_cast<size_t>(ti * BM + band * BR) * pr.lde + tj * BN;
#pragma unroll
        for (int p = 0; p < kIters; ++p) {
          const int idx = p * NT + tid;
          const int i = idx / (BN / 8), j = (idx % (BN / 8)) * 8;
          er[band][p] = *reinterpret_cast<const u32x4*>(eg + static_cast<size_t>(i) * pr.lde + j);
        }
      }
    }
  }
#pragma unroll
  for (int band = 0; band < 2 * WM; ++band) {
    const int row0 = ti * BM + band * BR;
    T* cg = need_c ? pool + pr.c_off + static_cast<size_t>(row0) * pr.ldc + tj * BN : nullptr;
    const T* eg = has_e ? pool + pr.e_off + static_cast<size_t>(row0) * pr.lde + tj * BN
                        : nullptr;
    if (wm == (band >> 1)) {
      const int h = band & 1;
#pragma unroll
      for (int hm = 0; hm < HM; ++hm)
#pragma unroll
        for (int ni = 0; ni < FN; ++ni)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int i = hm * 32 + 8 * (v >> 2) + 4 * fg + (v & 3);
            const int j = wn * C::kWaveN + ni * 32 + fr;
            cs[i * C::kBandLd + j] = h ? acc[HM + hm][ni][v] : acc[hm][ni][v];
          }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kIters; ++p) {
      const int idx = p * NT + tid;
      const int i = idx / (BN / 8), j = (idx % (BN / 8)) * 8;
      float v[8];
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(cs + i * C::kBandLd + j);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(cs + i * C::kBandLd + j + 4);
#pragma unroll
      for (int k = 0; k < 4; ++k) { v[k] = c1 * x0[k]; v[4 + k] = c1 * x1[k]; }
      if (has_e) {
        float e[8];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            e[2 * k] = __uint_as_float(er[band][p][k] << 16);
            e[2 * k + 1] = __uint_as_float(er[band][p][k] & 0xffff0000u);
          }
        } else {
          ld8<T>(eg + static_cast<size_t>(i) * pr.lde + j, e);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] += c0 * e[k];
      }
      // + cd I (the update's a X folded into P); diagonal tiles only
      if (ti == tj) {
        const int d = band * BR + i - j;
        if (d >= 0 && d < 8) v[d] += cd;
      }
      // the update's output is read only by the next launch: stream it past
      // L2, which holds this launch's operand panels (the Gram's stores are
      // kept: its mirror writes rely on write combining in L2)
      if (need_c) st8<T, BK>(cg + static_cast<size_t>(i) * pr.ldc + j, v);
      if (need_t) {
        *reinterpret_cast<f32x4*>(cs + i * C::kBandLd + j) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(cs + i * C::kBandLd + j + 4) = f32x4{v[4], v[5], v[6], v[7]};
      }
    }
    if (need_t) {
      __syncthreads();
      T* ctg = pool + pr.ct_off + static_cast<size_t>(tj) * BN * pr.ldct + row0;
#pragma unroll
      for (int p = 0; p < kIters; ++p) {
        const int idx = p * NT + tid;
        const int j = idx % BN, i = (idx / BN) * 8;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = cs[(i + k) * C::kBandLd + j];
        st8<T>(ctg + static_cast<size_t>(j) * pr.ldct + i, v);
      }
    }
    __syncthreads();
  }
}

// Batched GEMM over a problem table (GemmProb), one 64 WM x 64 WN-thread
// workgroup per output tile at a time.  128 x 128 tiles: with gridDim.x
// below ntiles the launch is persistent, workgroup b taking logical tiles b,
// b + gridDim.x, ... (gridDim.x a multiple of 8, so each keeps its XCD,
// b mod 8, and the workgroups of one round hold consecutive logical tiles as
// one workgroup per tile would), without a workgroup launch per tile.
// 256 x 256 tiles: one per workgroup (the tile loop's registers cost the
// dense-decoder launches 1.6%).
template <typename T, int BM, int BN, int WM, int WN, int MINW, bool BK, int ST, int SRB>
__global__ __launch_bounds__(64 * WM * WN, MINW) void k_ns_gemm(
    const GemmProb* __restrict__ probs, int nprob, T* __restrict__ pool, float c0,
    float c1_arg, int has_e, float cd, const RowSeg* __restrict__ wt, float lr_arg,
    const float* __restrict__ lrs, const float* __restrict__ pscale,
    const int32_t* __restrict__ pfb, float c1b_arg, float cdb, int ntiles) {
  if constexpr (BM == kGemmTile) {
    for (int vb = blockIdx.x; vb < ntiles; vb += gridDim.x) {
      // the previous tile's reads of LDS are done before its stages refill
      if (vb != static_cast<int>(blockIdx.x)) __syncthreads();
      ns_gemm_tile<T, BM, BN, WM, WN, BK, ST, SRB>(vb, ntiles, probs, nprob, pool, c0, c1_arg,
                                                    has_e, cd, wt, lr_arg, lrs, pscale, pfb,
                                                    c1b_arg, cdb);
    }
  } else {
    ns_gemm_tile<T, BM, BN, WM, WN, BK, ST, SRB>(blockIdx.x, gridDim.x, probs, nprob, pool, c0,
                                                  c1_arg, has_e, cd, wt, lr_arg, lrs, pscale,
                                                  pfb, c1b_arg, cdb);
  }
}


// ---------------------------------------------------------------------------
// Slice-resident Newton-Schulz for bf16 slices whose padded short side is
// 128 (head-sized slices).  One workgroup of 8 waves owns one slice for all
// iterations.  X (128 x lp) streams through LDS in 128 x 128 column blocks;
// P = a I + b A (+ c A^2), A = X X^T, lives in LDS (a X folded into P's
// diagonal, as in the GEMM path).  Per block of iteration k:
//   X'_b = P X_b                (B operand read from the staged block)
//   X'_b -> global, and A' += X'_b X'_b^T for iteration k + 1 (registers)
// so each iteration reads and writes X once; one extra read of X0 forms the
// first Gram.  Same iterate buffers and conventions as the GEMM path: the
// last iteration of a tall slice is written transposed (lp x 128).
// ---------------------------------------------------------------------------
constexpr int kSmThreads = 512;                 // 8 waves: 2 (rows) x 4 (cols), 64 x 32 each
constexpr int kSmTile = kSmallS * kSmallS * 2;  // one 128 x 128 bf16 tile (32 KiB)
constexpr int kSmStages = 3;                    // X blocks in LDS (2 loads ahead)

// 128 x 128 bf16 tiles in LDS: rows of 256 bytes, 16-byte chunk c of row r at
// c ^ swz(r), swz XOR-ing (r1, r0, r0 ^ r2, r1 ^ r3) into chunk bits 0..3.
// Chosen by search: conflict-free for the MFMA operand reads (32 rows x one
// chunk) under every lane grouping consistent with the gfx950 bank-conflict
// measurements, and for the transpose reads (4 rows x 64 bytes per 16 lanes).
__device__ __forceinline__ int sm_swz(int r) {
  return ((r >> 1) & 1) | ((r & 1) << 1) | (((r ^ (r >> 2)) & 1) << 2) |
         ((((r >> 1) ^ (r >> 3)) & 1) << 3);
}
__device__ __forceinline__ int sm_off(int row, int col) {
  return row * 256 + ((((col >> 3) ^ sm_swz(row)) & 15) << 4) + (col & 7) * 2;
}

// The Newton-Schulz iterations in Gram space for one 128 x 128 slice Gram,
// by the 8 waves of the slice-resident kernel (2 x 4 waves of 64 x 32
// outputs).  With P_k = a_k I + R_k, R_k = b_k A_k + c_k A_k^2:
// Q_1 = P_0, Q_{k+1} = P_k Q_k, T_k = P_k A_k, A_{k+1} = T_k P_k.  All
// factors are polynomials in A_0; the products are nonetheless formed
// exactly as U V (the right factor read by columns), since after rounding
// the factors no longer commute exactly.  In: A_0 (bf16) in xa.  Out: Q_N
// (bf16) in qs.  xa and yb are scratch tiles (A, the quintic T; the cubic T
// or the quintic R).  E terms are read one value at a time, so that the
// phase needs no registers beyond one accumulator block.
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
__device__ __forceinline__ void sm_gram_space(lds_char* qs, lds_char* xa, lds_char* yb,
                                           const NsCoeffTable* cfp, int steps) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3, fr = lane & 31, fg = lane >> 5;
  auto frag = [&](const lds_char* t, int m, int ks) __attribute__((always_inline)) {
    return *reinterpret_cast<const lds_u32x4*>(t + m * 256 +
                                               ((((2 * ks + fg) ^ sm_swz(m)) & 15) << 4));
  };
  // x = U V over the wave's 64 x 32 block: U by rows, V by columns
  // (transpose reads of its 16-row slabs), so the product is exact whether
  // or not the rounded factors are still exactly symmetric.  The operands go
  // into the MFMA swapped, which yields the transposed tile: each lane then
  // holds 4 consecutive columns of one row, x[mi][4 q + e] = (U V)[rw(mi)]
  // [cl(q) + e], so E terms and results move as 8-byte LDS accesses.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int trow = 8 * (g16 >> 1) + (j16 >> 2);
  const int tcol = wn * 32 + 16 * (g16 & 1) + 4 * (j16 & 3);
  auto prod = [&](const lds_char* u, const lds_char* v, f32x16 (&x)[2])
      __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int e = 0; e < 16; ++e) x[mi][e] = 0.f;
    u32x4 fv[2], fu[2][2];
    auto load = [&](int set, int ks) __attribute__((always_inline)) {
      const u32x2 lo = lds_read_tr16((const char*)(v + sm_off(16 * ks + trow, tcol)));
      const u32x2 hi = lds_read_tr16((const char*)(v + sm_off(16 * ks + trow + 4, tcol)));
      fv[set] = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) fu[set][mi] = frag(u, wm * 64 + mi * 32 + fr, ks);
    };
    load(0, 0);
    static_for<0, 8>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value, c = ks & 1;
      if constexpr (ks + 1 < 8) load(c ^ 1, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) mma<uint16_t>(fv[c], fu[c][mi], x[mi]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto rw = [&](int mi) { return wm * 64 + mi * 32 + fr; };
  auto cl = [&](int q) { return wn * 32 + 8 * q + 4 * fg; };
  auto put = [&](lds_char* dst, const f32x16 (&x)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<lds_u32x2*>(dst + sm_off(rw(mi), cl(q))) =
            u32x2{pk_bf16(x[mi][4 * q], x[mi][4 * q + 1]),
                  pk_bf16(x[mi][4 * q + 2], x[mi][4 * q + 3])};
  };
  // the 4 values of `src` at the place of x[mi][4 q .. 4 q + 3]
  auto at4 = [&](const lds_char* src, int mi, int q, float (&e)[4]) __attribute__((always_inline)) {
    const u32x2 w = *reinterpret_cast<const lds_u32x2*>(src + sm_off(rw(mi), cl(q)));
    e[0] = __uint_as_float(w[0] << 16);
    e[1] = __uint_as_float(w[0] & 0xffff0000u);
    e[2] = __uint_as_float(w[1] << 16);
    e[3] = __uint_as_float(w[1] & 0xffff0000u);
  };
  // x = alpha E + beta x, E from the tile `src` (read before any write)
  auto axpy = [&](f32x16 (&x)[2], float alpha, const lds_char* src, float beta)
      __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float e[4];
        at4(src, mi, q, e);
#pragma unroll
        for (int t = 0; t < 4; ++t) x[mi][4 * q + t] = alpha * e[t] + beta * x[mi][4 * q + t];
      }
  };
  f32x16 x[2];
  for (int k = 0; k < steps; ++k) {
    const float ak = cfp->a[k], bk = cfp->b[k], ck = cfp->c[k];
    const bool quint = ck != 0.f;
    if (quint) {        // R = b A + c A A into yb
      prod(xa, xa, x);
      axpy(x, bk, xa, ck);
      put(yb, x);
      __syncthreads();
    }
    // the left factor: R (quintic), or A scaled by b (cubic)
    const lds_char* const rt = quint ? yb : xa;
    const float rs = quint ? 1.f : bk;
    if (k == 0) {       // Q_1 = a_0 I + R_0
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float e[4];
          at4(rt, mi, q, e);
#pragma unroll
          for (int t = 0; t < 4; ++t)
            x[mi][4 * q + t] = rs * e[t] + (rw(mi) == cl(q) + t ? ak : 0.f);
        }
      put(qs, x);
    } else {            // Q' = a Q + rs (R Q)
      prod(rt, qs, x);
      axpy(x, ak, qs, rs);
      __syncthreads();
      put(qs, x);
    }
    __syncthreads();
    if (k + 1 == steps) break;
    // T = a A + rs (R A): into yb (cubic) or over A (quintic)
    prod(rt, xa, x);
    axpy(x, ak, xa, rs);
    if (quint) __syncthreads();
    lds_char* const tt = quint ? xa : yb;
    put(tt, x);
    __syncthreads();
    // A' = a T + rs (T R), over A
    prod(tt, rt, x);
    axpy(x, ak, tt, rs);
    __syncthreads();
    put(xa, x);
    __syncthreads();
  }
}

template <bool GS>
__global__ __launch_bounds__(kSmThreads, 1) void k_ns_small(const SmallProb* __restrict__ probs,
                                                            uint16_t* __restrict__ pool,
                                                            const PrepItem* __restrict__ items,
                                                            const float* __restrict__ scale,
                                                            NsCoeffTable cf, int steps,
                                                            const RowSeg* __restrict__ wt,
                                                            float lr_arg,
                                                            const float* __restrict__ lrs,
                                                            const int32_t* __restrict__ range_fb) {
  __shared__ __attribute__((aligned(16))) char smem[kSmTile * (2 + kSmStages)];
  char* const Ps = smem;             // P (A operand of the update)
  char* const Xn = smem + kSmTile;   // the new block X'_b (and A in a quintic step)
  const SmallProb pr = probs[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave >> 2, wn = wave & 3;
  const int fr = lane & 31, fg = lane >> 5, g16 = lane >> 4, j16 = lane & 15;
  const int NB = pr.lp / kSmallS;
  // Workgroup w walks the column blocks starting at block w % NB: the
  // workgroups that start together then read different column offsets of
  // their row-strided slabs instead of all the same ones.
  const int rot = static_cast<int>(blockIdx.x % static_cast<unsigned>(NB));
  auto col_of = [&](int b) __attribute__((always_inline)) {
    return b + rot >= NB ? b + rot - NB : b + rot;
  };
  // passes over X: pass 0 forms the first Gram; pass k + 1 runs iteration k.
  // Gram space: pass 0, then all iterations on 128 x 128 matrices in LDS,
  // then one pass for X_N = Q_N X0.
  const int npass = GS ? 1 : steps;
  const int total = NB * (npass + 1);
  const uint32_t ld_b = static_cast<uint32_t>(pr.lp) * 2;
  uint16_t* const X0 = pool + pr.x_off[0];
  uint16_t* const X1 = pool + pr.x_off[1];
  // In-place input: passes 0 and 1 read D itself (128 x lp bf16, row stride
  // lp, the layout of X0) and form X0 = bf16(s D) in LDS, with the same fp32
  // product and rounding as the prep kernel.
  const bool direct = pr.direct != 0;
  const u32x4 rs0 = buffer_rsrc(X0, kSmallS * ld_b), rs1 = buffer_rsrc(X1, kSmallS * ld_b);
  const u32x4 rsin = direct ? buffer_rsrc(items[pr.item].in, kSmallS * ld_b) : rs0;
  const float dscale = direct ? scale[pr.item] : 1.f;
  // With range flags (grouped step), an in-place slice whose max|D| is in
  // the range where unscaled products stay normal fp32 numbers (range flag
  // clear) skips the conversion: the passes that read D multiply D instead
  // of bf16(s D), and the scale is applied to the results, s^2 to the first
  // Gram and s to the first update, as the batched GEMM's first iteration
  // does.  Otherwise X0 = bf16(s D) is formed in LDS.
  const bool fold = direct && range_fb != nullptr && range_fb[pr.item] == 0;

  // Direct-to-LDS loads of one 128 x 128 block: 32 instructions of 4 rows
  // (1 KiB), 4 per wave; lane i lands at row + i / 16, physical chunk i % 16
  // and fetches logical chunk (i % 16) ^ swz(row).  Non-temporal: each block
  // is read once per pass by this workgroup only (9% faster than cached
  // loads; non-temporal stores of X'_b were slower).
  int vo[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = (wv * 4 + q) * 4 + (lane >> 4);
    vo[q] = static_cast<int>(row * ld_b) + (((lane & 15) ^ sm_swz(row)) << 4);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(smem))));
  auto issue = [&](int e) __attribute__((always_inline)) {
    const int pass = e / NB, b = col_of(e - pass * NB);
    // iteration k reads X[k % 2]; passes 0 and 1 read X0 (or D in place).
    // Selected per 32-bit word: a select between whole descriptors made the
    // compiler keep them in scratch memory.
    const bool from1 = pass >= 2 && ((pass - 1) & 1);
    u32x4 rs;
#pragma unroll
    for (int k = 0; k < 4; ++k) rs[k] = pass < 2 ? rsin[k] : from1 ? rs1[k] : rs0[k];
    const uint32_t st = lds0 + (2 + e % kSmStages) * kSmTile;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      lds_dma16<true>(rs, st + (wv * 4 + q) * 1024, vo[q], b * 256);
  };

  // Operand reads.  NT fragment: row m, logical chunk 2 ks + fg (both
  // operands of the Grams, P in the update).  K-major fragment (X_b^T in the
  // update): two transpose reads, lane j of 16-lane group g at row
  // 16 ks + 8 (g / 2) + 4 h + j / 4, columns c + 16 (g % 2) + 4 (j % 4).
  auto nt_frag = [&](const char* t, int m, int ks) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(t + m * 256 +
                                           ((((2 * ks + fg) ^ sm_swz(m)) & 15) << 4));
  };
  const int trow = 8 * (g16 >> 1) + (j16 >> 2);
  // C[m][n] += sum_k A[m][k] B[n][k] over a 128-wide K, both operands NT
  // (the fragments of step ks + 1 are read while step ks is multiplied: two
  // register sets, as in the batched GEMM; here and in the update and the
  // Gram-space products: 1% on the head-batched set)
  auto gram_acc = [&](const char* ta, const char* tb, f32x16 (&acc)[2]) __attribute__((always_inline)) {
    u32x4 fb[2], fa[2][2];
    auto load = [&](int set, int ks) __attribute__((always_inline)) {
      fb[set] = nt_frag(tb, wn * 32 + fr, ks);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) fa[set][mi] = nt_frag(ta, wm * 64 + mi * 32 + fr, ks);
    };
    load(0, 0);
    static_for<0, 8>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value, c = ks & 1;
      if constexpr (ks + 1 < 8) load(c ^ 1, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) mma<uint16_t>(fa[c][mi], fb[c], acc[mi]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto zero = [](f32x16 (&acc)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][v] = 0.f;
  };
  // element (row, col) of the wave's accumulator value (mi, v)
  auto acc_row = [&](int mi, int v) __attribute__((always_inline)) {
    return wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * fg + (v & 3);
  };
  const int acc_col = wn * 32 + fr;

  f32x16 accg[2], accu[2];
  zero(accg);
  // Load issue bookkeeping (uniform): element e is issued while processing
  // element at_e; stores of elements up to at(cur) - 1 are older than the loads
  // of `cur` and have completed once those are waited for (vector memory
  // operations complete in order).
  // at_k: element at which element cur + k was issued (k = 0, 1, 2)
  // (value selects, not a branch chain: the compiler turned the chain into a
  // store at a computed index, which kept the three values in scratch memory,
  // and every reload of them waited for all loads in flight)
  int next = 0, at_0 = 0, at_1 = 0, at_2 = 0;
  // Stores per wave of an update element, as the waits below count them: 4
  // (one 16-byte store per q; the fp32 weight update's 8 are counted as 4, a
  // smaller count only makes a wait stronger).  A fused weight update whose
  // weight rows (tall: rows or columns) do not fill the 128 x 128 blocks
  // leaves some waves without a valid row in some q, and their stores may
  // then not be issued at all: none are counted.
  int st_upd = 4;
  if (wt != nullptr) {
    const RowSeg& w = wt[pr.item];
    const bool full = pr.tall ? w.rows % kSmallS == 0 && w.cols >= kSmallS : w.rows >= kSmallS;
    if (!full) st_upd = 0;
  }
  auto note_issue = [&](int e, int cur) __attribute__((always_inline)) {
    at_0 = e == cur ? cur : at_0;
    at_1 = e == cur + 1 ? cur : at_1;
    at_2 = e != cur && e != cur + 1 ? cur : at_2;
  };

  // One element of the pipeline: block b of pass `pass`.  PC >= 0 fixes the
  // pass at compile time (the Gram-space kernel runs its two passes as two
  // loops, so that each loop only holds the registers its pass needs).
  auto element = [&](int cur, int pass_rt, auto pc) __attribute__((always_inline)) {
    constexpr int PC = decltype(pc)::value;
    const int pass = PC >= 0 ? PC : pass_rt, b = cur - pass * NB;
    const int pb = col_of(b);   // the column block it covers
    // A fused bf16 weight update (not tall) loads its weights here, before
    // the block wait, so that they arrive while the block's MFMAs run rather
    // than after them (the kernel: 1.45 -> 1.41 ms on the head-batched set).
    // The wait below counts these loads (when every wave issues all four).
    const bool wpre = wt != nullptr && !pr.tall && pass >= 1 && (GS || pass == npass) &&
                      wt[pr.item].w_dt == MO_BF16;
    W8 wrp[4];
    if (wpre) {
      const RowSeg& w = wt[pr.item];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int id = q * kSmThreads + tid;
        const int row = id >> 4, c = id & 15;
        const int ocol = pb * kSmallS + c * 8;
        if (row < w.rows && ocol < w.cols)
          wrp[q] = load_w8(w.w, static_cast<int64_t>(row) * w.ld_w + ocol, MO_BF16);
      }
    }
    int done;   // stores of elements <= done are complete after the wait below
    if (next == cur) {
      // not issued ahead (its block was written too recently): drain, then load
      __builtin_amdgcn_s_waitcnt(0x0070);
      __syncthreads();
      issue(cur);
      at_0 = cur;
      ++next;
      __builtin_amdgcn_s_waitcnt(0x0070);
      done = cur - 1;
    } else {
      // operations of this wave younger than the loads of `cur`: loads of
      // later elements (4 each) and the stores (st_upd each) of update
      // elements processed since those loads were issued
      const int a = at_0;
      const int first_store = a > NB ? a : NB;
      const int young = 4 * (next - 1 - cur) +
                        st_upd * (cur > first_store ? cur - first_store : 0) +
                        (wpre && st_upd == 4 ? 4 : 0);
      switch (young >> 2) {
        case 0: __builtin_amdgcn_s_waitcnt(vm_wait_imm(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(vm_wait_imm(4)); break;
        case 2: __builtin_amdgcn_s_waitcnt(vm_wait_imm(8)); break;
        case 3: __builtin_amdgcn_s_waitcnt(vm_wait_imm(12)); break;
        default: __builtin_amdgcn_s_waitcnt(vm_wait_imm(16)); break;
      }
      done = a - 1;
    }
    __syncthreads();   // B1: block `cur` in LDS; element cur - 1 fully done
    if (direct && !fold && cur < 2 * NB) {
      // D block -> X0 block in place (16 bytes = 8 elements per access; the
      // chunk swizzle does not matter for an elementwise pass)
      char* const blk = smem + (2 + cur % kSmStages) * kSmTile;
#pragma unroll
      for (int q = 0; q < kSmTile / (16 * kSmThreads); ++q) {
        u32x4* const p = reinterpret_cast<u32x4*>(blk + (q * kSmThreads + tid) * 16);
        u32x4 v = *p;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          v[k] = pk_bf16(dscale * __uint_as_float(v[k] << 16),
                         dscale * __uint_as_float(v[k] & 0xffff0000u));
        *p = v;
      }
      __syncthreads();
    }
    // Loads ahead: at most 2 elements ahead (their stage was last read by
    // element cur - 1), and a block written by an earlier pass only once its
    // stores are known complete.
    while (next < total && next <= cur + 2 && (next < 2 * NB || next - NB <= done)) {
      issue(next);
      note_issue(next, cur);
      ++next;
    }
    const char* stg = smem + (2 + cur % kSmStages) * kSmTile;
    if (pass == 0) {
      gram_acc(stg, stg, accg);
    } else {
      // update, computed transposed: (P X_b)^T = X_b^T P (P is symmetric), so
      // that each lane's accumulator holds 4 consecutive columns of one row of
      // X'_b.  A operand X_b^T: rows = block columns, read K-major (transpose
      // reads); B operand P: rows read as stored.
      zero(accu);
      {
        u32x4 fp[2], fx[2][2];
        auto load = [&](int set, int ks) __attribute__((always_inline)) {
          fp[set] = nt_frag(Ps, wn * 32 + fr, ks);
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) {
            const int c0 = wm * 64 + mi * 32 + 16 * (g16 & 1) + 4 * (j16 & 3);
            const u32x2 lo = lds_read_tr16(stg + sm_off(16 * ks + trow, c0));
            const u32x2 hi = lds_read_tr16(stg + sm_off(16 * ks + trow + 4, c0));
            fx[set][mi] = u32x4{lo[0], lo[1], hi[0], hi[1]};
          }
        };
        load(0, 0);
        static_for<0, 8>([&](auto ksc) {
          constexpr int ks = decltype(ksc)::value, c = ks & 1;
          if constexpr (ks + 1 < 8) load(c ^ 1, ks + 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mi = 0; mi < 2; ++mi) mma<uint16_t>(fx[c][mi], fp[c], accu[mi]);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      if (fold && pass == 1) {   // (s D)-based result: s times the product with D
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int v = 0; v < 16; ++v) accu[mi][v] *= dscale;
      }
      // accu[mi][4 q + e] = X'_b[i][j0 + e], i = wn * 32 + fr,
      // j0 = wm * 64 + mi * 32 + 8 q + 4 fg: 8-byte E reads and X'_b writes
      // (a X_b is on P's diagonal: P = a I + b A + c A^2)
      const int xi = wn * 32 + fr;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int off = sm_off(xi, wm * 64 + mi * 32 + 8 * q + 4 * fg);
          const f32x16& x = accu[mi];
          *reinterpret_cast<u32x2*>(Xn + off) =
              u32x2{pk_bf16(x[4 * q], x[4 * q + 1]), pk_bf16(x[4 * q + 2], x[4 * q + 3])};
        }
      __syncthreads();   // B2: X'_b complete in LDS
      const bool last = GS || pass == npass;
      if (last && wt != nullptr) {
        // apply the Muon step to the slice's weights (stored orientation,
        // clipped to the real extent) instead of writing O
        const RowSeg w = wt[pr.item];
        const float lr = lrs ? lrs[w.lr_slot] : lr_arg;
        const float decay = 1.f - lr * w.wd, coef = lr * w.scale;
        // (one chunk at a time: holding all four weight chunks of a thread
        // in registers would spill in this kernel)
        if (pr.tall) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int T = q * 32 + wv * 4 + g16;
            const int n0 = 16 * (T & 7), k0 = 8 * (T >> 3);
            // transpose reads exchange data between the lanes of a 16-lane
            // group: every lane takes part, whatever its row
            const u32x2 lo = lds_read_tr16(Xn + sm_off(k0 + (j16 >> 2), n0 + 4 * (j16 & 3)));
            const u32x2 hi = lds_read_tr16(Xn + sm_off(k0 + 4 + (j16 >> 2), n0 + 4 * (j16 & 3)));
            const int orow = pb * kSmallS + n0 + j16;
            if (orow < w.rows && k0 < w.cols) {
              const int64_t at = static_cast<int64_t>(orow) * w.ld_w + k0;
              apply_w8(w.w, at, w.w_dt, load_w8(w.w, at, w.w_dt),
                       u32x4{lo[0], lo[1], hi[0], hi[1]}, decay, coef);
            }
          }
        } else if (w.w_dt == MO_BF16) {
          W8 (&wr)[4] = wrp;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int id = q * kSmThreads + tid;
            const int row = id >> 4, c = id & 15;
            const int ocol = pb * kSmallS + c * 8;
            if (row < w.rows && ocol < w.cols)
              apply_w8(w.w, static_cast<int64_t>(row) * w.ld_w + ocol, MO_BF16, wr[q],
                       *reinterpret_cast<const u32x4*>(Xn + row * 256 +
                                                       (((c ^ sm_swz(row)) & 15) << 4)),
                       decay, coef);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int id = q * kSmThreads + tid;
            const int row = id >> 4, c = id & 15;
            const int ocol = pb * kSmallS + c * 8;
            if (row < w.rows && ocol < w.cols) {
              const int64_t at = static_cast<int64_t>(row) * w.ld_w + ocol;
              apply_w8(w.w, at, w.w_dt, load_w8(w.w, at, w.w_dt),
                       *reinterpret_cast<const u32x4*>(Xn + row * 256 +
                                                       (((c ^ sm_swz(row)) & 15) << 4)),
                       decay, coef);
            }
          }
        }
      } else if (last && pr.tall) {
        // stored orientation: out[b * 128 + n][k] = X'_b[k][n], ld 128
        uint16_t* out = (npass & 1) ? X1 : X0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int T = q * 32 + wv * 4 + g16;
          const int n0 = 16 * (T & 7), k0 = 8 * (T >> 3);
          const u32x2 lo = lds_read_tr16(Xn + sm_off(k0 + (j16 >> 2), n0 + 4 * (j16 & 3)));
          const u32x2 hi = lds_read_tr16(Xn + sm_off(k0 + 4 + (j16 >> 2), n0 + 4 * (j16 & 3)));
          *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(pb * kSmallS + n0 + j16) * kSmallS +
                                    k0) = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      } else {
        uint16_t* out = (pass & 1) ? X1 : X0;   // iteration k writes X[(k + 1) % 2]
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int id = q * kSmThreads + tid;
          const int row = id >> 4, c = id & 15;
          const u32x4 v = *reinterpret_cast<const u32x4*>(Xn + row * 256 +
                                                         (((c ^ sm_swz(row)) & 15) << 4));
          *reinterpret_cast<u32x4*>(out + static_cast<int64_t>(row) * pr.lp + pb * kSmallS +
                                    c * 8) = v;
        }
      }
      if (!last) gram_acc(Xn, Xn, accg);
    }
    if (fold && b == NB - 1 && pass == 0) {   // the first Gram: s^2 D D^T
      const float s2 = dscale * dscale;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v) accg[mi][v] *= s2;
    }
    if (GS && b == NB - 1 && pass == 0) {
      // Gram space: A_0 (as stored, bf16) into Xn, then every iteration on
      // 128 x 128 matrices in LDS; Q_N lands in Ps for the final pass.  The
      // stage this element's block has just left is free for the phase.
      __syncthreads();   // every wave is done with this element's staged block
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          *reinterpret_cast<uint16_t*>(Xn + sm_off(acc_row(mi, v), acc_col)) =
              f32_to_bf16(accg[mi][v]);
      __syncthreads();
      // (C-style casts: generic pointers to LDS, into the LDS address space)
      sm_gram_space((lds_char*)(Ps), (lds_char*)(Xn),
                    (lds_char*)(smem + (2 + cur % kSmStages) * kSmTile), &cf, steps);
      zero(accg);
    } else if (!GS && b == NB - 1 && pass < steps) {
      // P = a I + b A (+ c A^2) for iteration `pass`, from A = accg
      const float ak = cf.a[pass], bk = cf.b[pass], ck = cf.c[pass];
      if (ck == 0.f) {
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            *reinterpret_cast<uint16_t*>(Ps + sm_off(acc_row(mi, v), acc_col)) =
                f32_to_bf16(bk * accg[mi][v] + (acc_row(mi, v) == acc_col ? ak : 0.f));
      } else {
        __syncthreads();   // X'_b reads of this element are done
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint16_t h = f32_to_bf16(accg[mi][v]);
            accg[mi][v] = bf16_to_f32(h);   // A as stored
            *reinterpret_cast<uint16_t*>(Xn + sm_off(acc_row(mi, v), acc_col)) = h;
          }
        __syncthreads();
        zero(accu);
        gram_acc(Xn, Xn, accu);   // A A (A is symmetric, so it is its own transpose)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            *reinterpret_cast<uint16_t*>(Ps + sm_off(acc_row(mi, v), acc_col)) =
                f32_to_bf16(bk * accg[mi][v] + ck * accu[mi][v] +
                            (acc_row(mi, v) == acc_col ? ak : 0.f));
      }
      zero(accg);
    }
    at_0 = at_1;
    at_1 = at_2;
  };
  if constexpr (GS) {
#pragma unroll 1
    for (int cur = 0; cur < NB; ++cur) element(cur, 0, Int<0>{});
#pragma unroll 1
    for (int cur = NB; cur < total; ++cur) element(cur, 1, Int<1>{});
  } else {
#pragma unroll 1
    for (int pass = 0; pass <= npass; ++pass)
#pragma unroll 1
      for (int cur = pass * NB; cur < (pass + 1) * NB; ++cur) element(cur, pass, Int<-1>{});
  }
}

}  // namespace

mo_status launch_ns_stats(const PrepItem* items, int n, int64_t ntiles, StatPartial* partials,
                          hipStream_t st) {
  if (ntiles <= 0) return MO_OK;
  KTimer tm(MO_KC_NS_STATS, st);
  k_ns_stats<<<dim3(static_cast<unsigned>(ntiles)), kThreads, 0, st>>>(items, n, partials);
  MO_LAUNCH_CHECK("k_ns_stats");
  return MO_OK;
}

mo_status launch_ns_scale(const PrepItem* items, int n, const StatPartial* partials,
                          float* scale, int32_t* range_fb, hipStream_t st) {
  if (n <= 0) return MO_OK;
  KTimer tm(MO_KC_NS_SCALE, st);
  k_ns_scale<<<dim3(n), kThreads, 0, st>>>(items, partials, scale, range_fb);
  MO_LAUNCH_CHECK("k_ns_scale");
  return MO_OK;
}

mo_status launch_ns_prep(const PrepItem* items, int n, int64_t ntiles, const float* scale,
                         void* pool, int elem, hipStream_t st) {
  if (ntiles <= 0) return MO_OK;
  KTimer tm(MO_KC_NS_PREP, st);
  if (elem == 2)
    k_ns_prep<uint16_t><<<dim3(static_cast<unsigned>(ntiles)), kThreads, 0, st>>>(
        items, n, scale, static_cast<uint16_t*>(pool));
  else
    k_ns_prep<float><<<dim3(static_cast<unsigned>(ntiles)), kThreads, 0, st>>>(
        items, n, scale, static_cast<float*>(pool));
  MO_LAUNCH_CHECK("k_ns_prep");
  return MO_OK;
}

mo_status launch_ns_prep_fallback(const PrepItem* items, int n, const float* scale,
                                  const int32_t* range_fb, void* pool, hipStream_t st) {
  if (n <= 0) return MO_OK;
  KTimer tm(MO_KC_NS_PREP, st);
  k_ns_prep_fb<<<dim3(1024), kThreads, 0, st>>>(items, n, scale, range_fb,
                                                static_cast<uint16_t*>(pool));
  MO_LAUNCH_CHECK("k_ns_prep_fb");
  return MO_OK;
}

// Workgroups of `kernel` (nt threads) resident on the current device at once:
// CUs x workgroups per CU, rounded down to a multiple of the 8 XCDs; 0 when
// the runtime cannot tell.  Cached per kernel and device.
template <typename K>
int resident_wgs(K kernel, int nt) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int ncu = 0, occ = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, nt, 0) != hipSuccess)
      return 0;
    v = (ncu * occ) & ~7;
    if (v <= 0) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <typename T, int BM, int WM, int WN, int ST = 4, int SRB = 64>
void launch_gemm_shape(const GemmProb* probs, int n, int ntiles, bool persist, int bk, T* pool,
                       float c0, float c1, int has_e, float cd, const RowSeg* wt, float lr,
                       const float* lrs, const float* pscale, const int32_t* pfb, float c1b,
                       float cdb, hipStream_t st) {
  constexpr int NT = 64 * WM * WN;
  auto run = [&](auto kernel) {
    // (only 128 x 128 tiles loop over tiles; others take one per workgroup)
    const int res = persist && BM == kGemmTile ? resident_wgs(kernel, NT) : 0;
    const dim3 grid(static_cast<unsigned>(res > 0 && res < ntiles ? res : ntiles));
    kernel<<<grid, NT, 0, st>>>(probs, n, pool, c0, c1, has_e, cd, wt, lr, lrs, pscale, pfb,
                                c1b, cdb, ntiles);
  };
  if (bk)
    run(k_ns_gemm<T, BM, BM, WM, WN, 2, true, ST, SRB>);
  else
    run(k_ns_gemm<T, BM, BM, WM, WN, 2, false, ST, SRB>);
}

mo_status launch_ns_gemm(const GemmProb* probs, int n, int64_t ntiles, bool persist, int tile,
                         int64_t few_max, int bk,
                         void* pool, int elem, float c0, float c1, int has_e, float cd,
                         const RowSeg* wt, float lr, const float* lrs, const float* pscale,
                         const int32_t* pfb, hipStream_t st, float c1b, float cdb) {
  if (ntiles <= 0) return MO_OK;
  if (bk && has_e) return fail(MO_EINVAL, "the K-major-B GEMM takes no E term");
  if (wt && (!bk || elem != 2))
    return fail(MO_EINVAL, "the fused weight update needs the bf16 K-major-B GEMM");
  if (ntiles > INT32_MAX) return fail(MO_EINVAL, "%lld GEMM tiles in one launch", static_cast<long long>(ntiles));
  KTimer tm(MO_KC_NS_GEMM, st);
  const int nt = static_cast<int>(ntiles);
  if (tile == 256) {
    // bf16: 64-deep K slabs (128-byte rows) in 2 stages (128 KiB), one slab
    // in flight while the other is multiplied: half the waits and barriers
    // per unit of k of 4 stages of 32-deep slabs, and 2% faster on the
    // dense-decoder batch.  One workgroup per tile: persistent launches of
    // these long tiles ran no faster alone, and left no CU to a concurrent
    // launch on another stream (the dense-decoder step: 1.2 ms slower).
    if (elem == 2)
      launch_gemm_shape<uint16_t, 256, 2, 4, 2, 128>(probs, n, nt, persist, bk,
                                                     static_cast<uint16_t*>(pool), c0, c1, has_e,
                                                     cd, wt, lr, lrs, pscale, pfb, c1b, cdb, st);
    else
      launch_gemm_shape<float, 256, 2, 4>(probs, n, nt, persist, bk, static_cast<float*>(pool), c0, c1,
                                          has_e, cd, wt, lr, lrs, pscale, pfb, c1b, cdb, st);
  } else if (tile == 128) {
    // Persistent when every problem has one K: a workgroup launch per tile
    // left the CU idle for about 3 us between two tiles, a large share of
    // these short tiles (the head-batched set's launches: 2-8% faster).
    // A launch with few tiles leaves most CUs idle and lasts as long as one
    // tile's K loop, whose length is set by the fixed cost of each K slab
    // (wait, barrier, fragment reads): split each tile over 8 waves of
    // 64 x 32 instead of 4 of 64 x 64, and take 64-deep slabs (128-byte
    // rows; 4 stages, 128 KiB) instead of 32-deep ones.  15-20% faster on the
    // single-matrix sweeps; 8 stages of 32-deep slabs were slower.
    if (elem == 2 && ntiles < few_max)
      launch_gemm_shape<uint16_t, 128, 2, 4, 4, 128>(probs, n, nt, persist, bk,
                                                     static_cast<uint16_t*>(pool), c0, c1, has_e,
                                                     cd, wt, lr, lrs, pscale, pfb, c1b, cdb, st);
    else if (elem == 2)  // 2 stages of 64-deep slabs, as for 256 x 256 tiles (64 KiB)
      launch_gemm_shape<uint16_t, 128, 2, 2, 2, 128>(probs, n, nt, persist, bk,
                                                     static_cast<uint16_t*>(pool), c0, c1, has_e,
                                                     cd, wt, lr, lrs, pscale, pfb, c1b, cdb, st);
    else
      launch_gemm_shape<float, 128, 2, 2>(probs, n, nt, persist, bk, static_cast<float*>(pool), c0, c1,
                                          has_e, cd, wt, lr, lrs, pscale, pfb, c1b, cdb, st);
  } else {
    return fail(MO_EINVAL, "unsupported GEMM tile %d", tile);
  }
  MO_LAUNCH_CHECK("k_ns_gemm");
  return MO_OK;
}

mo_status launch_ns_small(const SmallProb* probs, int n, void* pool, const PrepItem* items,
                          const float* scale, const float* coeffs, int steps, const RowSeg* wt,
                          float lr, const float* lrs, hipStream_t st, int gspace,
                          const int32_t* range_fb) {
  if (n <= 0) return MO_OK;
  if (steps < 1 || steps > MO_NS_MAX_STEPS) return fail(MO_EINVAL, "bad step count %d", steps);
  NsCoeffTable cf;
  std::memset(&cf, 0, sizeof(cf));
  for (int k = 0; k < steps; ++k) {
    cf.a[k] = coeffs[3 * k];
    cf.b[k] = coeffs[3 * k + 1];
    cf.c[k] = coeffs[3 * k + 2];
  }
  KTimer tm(MO_KC_NS_SMALL, st);
  if (gspace)
    k_ns_small<true><<<dim3(static_cast<unsigned>(n)), kSmThreads, 0, st>>>(
        probs, static_cast<uint16_t*>(pool), items, scale, cf, steps, wt, lr, lrs, range_fb);
  else
    k_ns_small<false><<<dim3(static_cast<unsigned>(n)), kSmThreads, 0, st>>>(
        probs, static_cast<uint16_t*>(pool), items, scale, cf, steps, wt, lr, lrs, range_fb);
  MO_LAUNCH_CHECK("k_ns_small");
  return MO_OK;
}

mo_status launch_ns_final(const FinalItem* items, int n, int64_t total_rows, const void* pool,
                          int elem, hipStream_t st) {
  if (total_rows <= 0) return MO_OK;
  const unsigned grid = static_cast<unsigned>(ceil_div(total_rows, kThreads / 64));
  KTimer tm(MO_KC_NS_FINAL, st);
  if (elem == 2)
    k_ns_final<uint16_t><<<grid, kThreads, 0, st>>>(items, n, total_rows,
                                                     static_cast<const uint16_t*>(pool));
  else
    k_ns_final<float><<<grid, kThreads, 0, st>>>(items, n, total_rows,
                                                  static_cast<const float*>(pool));
  MO_LAUNCH_CHECK("k_ns_final");
  return MO_OK;
}

}  // namespace mo
