// Newton-Schulz orthogonalisation kernels for gfx950.
//
// Per independent matrix (slice) the iteration X <- a X + (b A + c A^2) X,
// A = X X^T, runs on the short side (NorMuon paper section 2.2 eq. (5); OMN
// "Dual-Manifold Optimization", Muon-path paragraphs).  Every slice lives in a
// zero-padded pool in two layouts: X (s x l) and X^T (l x s), padded to
// multiples of 128, so that all three products are "NT" GEMMs with the
// contraction index contiguous in memory for both operands:
//   Gram    A[i][j]  = sum_k X[i][k]  X[j][k]        (symmetric: tiles i <= j)
//   Square  P[i][j]  = b A[i][j] + c sum_k A[i][k] A[j][k]   (A symmetric)
//   Update  X'[i][n] = a X[i][n] + sum_k P[i][k] Xt[n][k]
// The update writes X' in place and its transpose into the other X^T buffer.
// Zero padding stays zero through every product, so no bounds checks are
// needed inside the GEMM.
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
                                                       float* __restrict__ scale) {
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
  }
}

template <typename T>
__device__ __forceinline__ T to_elem(float v);
template <>
__device__ __forceinline__ uint16_t to_elem<uint16_t>(float v) { return f32_to_bf16(v); }
template <>
__device__ __forceinline__ float to_elem<float>(float v) { return v; }

template <typename T>
__global__ __launch_bounds__(kThreads) void k_ns_prep(const PrepItem* __restrict__ items, int n,
                                                      const float* __restrict__ scale,
                                                      T* __restrict__ pool) {
  __shared__ T tile_s[kPrepTile][kPrepTile + 1];
  const int64_t tile = blockIdx.x;
  const int idx = find_segment(items, n, tile);
  const PrepItem it = items[idx];
  const float s = scale[idx];
  const int64_t lt = tile - it.start;
  const int r0 = static_cast<int>(lt / it.tiles_c) * kPrepTile;
  const int c0 = static_cast<int>(lt % it.tiles_c) * kPrepTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  T* sb = pool + it.sbuf;
  T* st = pool + it.stbuf;
  for (int q = 0; q < kPrepTile / 4; ++q) {
    const int lr = ty + 4 * q;
    const int row = r0 + lr, col = c0 + tx;
    float v = 0.f;
    if (row < it.r && col < it.c)
      v = load_as_f32(it.in, static_cast<int64_t>(row) * it.ld_in + col, it.in_dt) * s;
    const T e = to_elem<T>(v);
    sb[static_cast<int64_t>(row) * it.cp + col] = e;
    tile_s[lr][tx] = e;
  }
  __syncthreads();
  for (int q = 0; q < kPrepTile / 4; ++q) {
    const int lc = ty + 4 * q;  // column of the stored tile = row of the transpose
    st[static_cast<int64_t>(c0 + lc) * it.rp + r0 + tx] = tile_s[tx][lc];
  }
}

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
// Batched NT GEMM on MFMA: 128 x 128 tile per 256-thread workgroup, 4 waves
// in 2 x 2, each wave 64 x 64 = 2 x 2 blocks of the 32x32 MFMA.  K is staged
// through LDS 128 bytes of every row at a time (64 bf16 / 32 fp32) with a
// 16-byte XOR swizzle, double-buffered; the next K slab is prefetched into
// registers while the current one is multiplied.
// ---------------------------------------------------------------------------
constexpr int kRowBytes = 128;
constexpr int kStageBytes = 2 * kGemmTile * kRowBytes;   // A + B slabs: 32 KiB
constexpr int kCsLd = 132;                               // epilogue tile stride (floats)
constexpr int kLdsBytes = kGemmTile * kCsLd * 4;         // 66 KiB (>= 2 stages)
static_assert(kLdsBytes >= 2 * kStageBytes, "epilogue tile must cover both stages");

__device__ __forceinline__ int swz(int row, int c16) {
  return row * kRowBytes + ((c16 ^ (row & 7)) << 4);
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

template <typename T>
__device__ __forceinline__ void st8(T* p, const float* v);
template <>
__device__ __forceinline__ void st8<uint16_t>(uint16_t* p, const float* v) {
  u32x4 u;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    u[k] = f32_to_bf16(v[2 * k]) | (static_cast<uint32_t>(f32_to_bf16(v[2 * k + 1])) << 16);
  *reinterpret_cast<u32x4*>(p) = u;
}
template <>
__device__ __forceinline__ void st8<float>(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void k_ns_gemm(const GemmProb* __restrict__ probs,
                                                         int nprob, T* __restrict__ pool,
                                                         float c0, float c1, int has_e) {
  __shared__ __attribute__((aligned(16))) char smem[kLdsBytes];
  // XCD-aware order: consecutive workgroup ids go round-robin over the 8
  // XCDs; give each XCD a contiguous run of logical tiles so neighbouring
  // tiles (which share operand rows) meet in the same L2.
  const int G = gridDim.x, bid = blockIdx.x;
  const int q8 = G >> 3, r8 = G & 7, xcd = bid & 7;
  const int tile = xcd * q8 + min(xcd, r8) + (bid >> 3);
  const GemmProb pr = probs[find_segment(probs, nprob, tile)];
  int t = tile - pr.start, ti, tj;
  if (pr.sym) {
    ti = 0;
    int len = pr.tiles_m;
    while (t >= len) { t -= len; ++ti; --len; }
    tj = ti + t;
  } else {
    ti = t / pr.tiles_n;
    tj = t - ti * pr.tiles_n;
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int fr = lane & 31, fg = lane >> 5;
  const int lrow = tid >> 3, lc = tid & 7;
  const size_t lda_b = static_cast<size_t>(pr.lda) * sizeof(T);
  const size_t ldb_b = static_cast<size_t>(pr.ldb) * sizeof(T);
  const char* ag = reinterpret_cast<const char*>(pool + pr.a_off) +
                   static_cast<size_t>(ti) * kGemmTile * lda_b + lrow * lda_b + lc * 16;
  const char* bg = reinterpret_cast<const char*>(pool + pr.b_off) +
                   static_cast<size_t>(tj) * kGemmTile * ldb_b + lrow * ldb_b + lc * 16;

  u32x4 ra[4], rb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ra[q] = *reinterpret_cast<const u32x4*>(ag + q * 32 * lda_b);
    rb[q] = *reinterpret_cast<const u32x4*>(bg + q * 32 * ldb_b);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    *reinterpret_cast<u32x4*>(smem + swz(lrow + 32 * q, lc)) = ra[q];
    *reinterpret_cast<u32x4*>(smem + kGemmTile * kRowBytes + swz(lrow + 32 * q, lc)) = rb[q];
  }
  __syncthreads();

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.f;

  const int KT = pr.K / (kRowBytes / static_cast<int>(sizeof(T)));
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) {
      ag += kRowBytes;
      bg += kRowBytes;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ra[q] = *reinterpret_cast<const u32x4*>(ag + q * 32 * lda_b);
        rb[q] = *reinterpret_cast<const u32x4*>(bg + q * 32 * ldb_b);
      }
    }
    const char* as = smem + (kt & 1) * kStageBytes;
    const char* bs = as + kGemmTile * kRowBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 av[2], bv[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        av[mi] = *reinterpret_cast<const u32x4*>(as + swz(wm * 64 + mi * 32 + fr, ks * 2 + fg));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bv[ni] = *reinterpret_cast<const u32x4*>(bs + swz(wn * 64 + ni * 32 + fr, ks * 2 + fg));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) mma<T>(av[mi], bv[ni], acc[mi][ni]);
    }
    if (more) {
      char* nas = smem + ((kt + 1) & 1) * kStageBytes;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<u32x4*>(nas + swz(lrow + 32 * q, lc)) = ra[q];
        *reinterpret_cast<u32x4*>(nas + kGemmTile * kRowBytes + swz(lrow + 32 * q, lc)) = rb[q];
      }
    }
    __syncthreads();
  }

  // Epilogue: stage the fp32 tile in LDS, then coalesced direct (and
  // transposed) stores.  32x32 MFMA output: lane l holds column l % 32 and
  // rows 8 (v / 4) + 4 (l / 32) + v % 4 for v = 0..15.
  float* cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = wm * 64 + mi * 32 + 8 * (v >> 2) + 4 * fg + (v & 3);
        const int j = wn * 64 + ni * 32 + fr;
        cs[i * kCsLd + j] = acc[mi][ni][v];
      }
  __syncthreads();
  const bool need_t = pr.ct_off >= 0 && !(pr.sym && ti == tj);
  T* cg = pool + pr.c_off + static_cast<size_t>(ti) * kGemmTile * pr.ldc + tj * kGemmTile;
  const T* eg = has_e ? pool + pr.e_off + static_cast<size_t>(ti) * kGemmTile * pr.lde +
                            tj * kGemmTile
                      : nullptr;
#pragma unroll 2
  for (int p = 0; p < (kGemmTile * kGemmTile) / (kThreads * 8); ++p) {
    const int idx = p * kThreads + tid;
    const int i = idx >> 4, j = (idx & 15) * 8;
    float v[8];
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(cs + i * kCsLd + j);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(cs + i * kCsLd + j + 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) { v[k] = c1 * x0[k]; v[4 + k] = c1 * x1[k]; }
    if (has_e) {
      float e[8];
      ld8<T>(eg + static_cast<size_t>(i) * pr.lde + j, e);
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] += c0 * e[k];
    }
    st8<T>(cg + static_cast<size_t>(i) * pr.ldc + j, v);
    if (need_t) {
      *reinterpret_cast<f32x4*>(cs + i * kCsLd + j) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(cs + i * kCsLd + j + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
  }
  if (need_t) {
    __syncthreads();
    T* ctg = pool + pr.ct_off + static_cast<size_t>(tj) * kGemmTile * pr.ldct + ti * kGemmTile;
#pragma unroll 2
    for (int p = 0; p < (kGemmTile * kGemmTile) / (kThreads * 8); ++p) {
      const int idx = p * kThreads + tid;
      const int j = idx & (kGemmTile - 1), i = (idx >> 7) * 8;
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = cs[(i + k) * kCsLd + j];
      st8<T>(ctg + static_cast<size_t>(j) * pr.ldct + i, v);
    }
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
                          float* scale, hipStream_t st) {
  if (n <= 0) return MO_OK;
  KTimer tm(MO_KC_NS_SCALE, st);
  k_ns_scale<<<dim3(n), kThreads, 0, st>>>(items, partials, scale);
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

mo_status launch_ns_gemm(const GemmProb* probs, int n, int64_t ntiles, void* pool, int elem,
                         float c0, float c1, int has_e, hipStream_t st) {
  if (ntiles <= 0) return MO_OK;
  KTimer tm(MO_KC_NS_GEMM, st);
  if (elem == 2)
    k_ns_gemm<uint16_t><<<dim3(static_cast<unsigned>(ntiles)), kThreads, 0, st>>>(
        probs, n, static_cast<uint16_t*>(pool), c0, c1, has_e);
  else
    k_ns_gemm<float><<<dim3(static_cast<unsigned>(ntiles)), kThreads, 0, st>>>(
        probs, n, static_cast<float*>(pool), c0, c1, has_e);
  MO_LAUNCH_CHECK("k_ns_gemm");
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
