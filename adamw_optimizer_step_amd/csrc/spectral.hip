// Power-iteration estimate of each matrix's largest singular value, for the
// spectral-cap guard on the Muon buffer (OMN "Dual-Manifold Optimization"
// page, Muon-path paragraph: an optional guard with a power-iteration
// estimate, inactive by default).  Per matrix B (fp32, rows x cols):
//   v_0 = ones / sqrt(cols);  v_{k+1} = B^T B v_k / ||B^T B v_k||;
//   sigma = ||B v_K||.
// One iteration is a row pass (u = B v: one fp64 dot product per row, one
// wave per row, with the partial sums of u^2), a column pass (B^T u over
// chunks of 256 rows, 4 columns per thread, into per-chunk partials), a fold
// (w = the sum of the chunks' partials, with the partial sums of w^2) and a
// per-matrix norm; the estimate is the row pass after the last iteration.
// All sums are fp64, in a fixed order: the cap rescales an fp32 state, so
// the estimate must be good to far below fp32's unit roundoff relative to
// itself.  HBM-bound: the row and column passes each read B once, with
// 16-byte accesses where the rows allow them.
#include "kernels.hpp"

namespace mo {

namespace {

constexpr int kPowRowsPerBlock = 64;    // row pass: 4 waves x 16 rows
constexpr int kPowRowsPerChunk = 256;   // column pass: rows per block
constexpr int kPowColsPerBlock = 4 * kThreads;   // column pass: 4 columns per thread
constexpr int kPowFoldCols = kThreads;  // fold: one column per thread
constexpr int kPowWLds = 6144;          // row pass: w staged in LDS up to this many columns

template <typename S>
__device__ __forceinline__ int find_by(const S* segs, int n, int64_t key, int64_t S::*field) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].*field <= key) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// 16-byte accesses along rows: 16-byte aligned rows and columns a multiple
// of 4 (otherwise one element at a time)
__device__ __forceinline__ bool pow_vec(const PowSeg& sg) {
  return (reinterpret_cast<uintptr_t>(sg.b) & 15) == 0 && (sg.ld & 3) == 0 && (sg.cols & 3) == 0;
}

// The dot products of one row with v, over 16-byte groups when kVec:
// kFirst: v = v_0 (the constant is applied by the caller); else v = w (from
// wv, which is LDS or global memory).
template <bool kFirst, bool kVec, typename WP>
__device__ __forceinline__ double pow_row_dot(const float* row, int cols, WP wv, int lane) {
  double d0 = 0.0, d1 = 0.0;   // two accumulators, over alternate groups of 256 columns
  if constexpr (kVec) {
    auto grp = [&](int j) __attribute__((always_inline)) {
      const float4 a = *reinterpret_cast<const float4*>(row + j);
      if constexpr (kFirst)
        return (static_cast<double>(a.x) + a.y) + (static_cast<double>(a.z) + a.w);
      else
        return static_cast<double>(a.x) * wv[j] + static_cast<double>(a.y) * wv[j + 1] +
               static_cast<double>(a.z) * wv[j + 2] + static_cast<double>(a.w) * wv[j + 3];
    };
    int j = 4 * lane;
    for (; j + 256 < cols; j += 512) {
      d0 += grp(j);
      d1 += grp(j + 256);
    }
    if (j < cols) d0 += grp(j);
  } else {
#pragma unroll 4
    for (int j = lane; j < cols; j += 64)
      d0 += static_cast<double>(row[j]) * (kFirst ? 1.0 : static_cast<double>(wv[j]));
  }
  return d0 + d1;
}

// u = B v for every row of every matrix (v_0 on the first pass, else
// w * inv), with one partial of sum u^2 per block.  One wave per row; the
// block's rows all belong to one matrix, which reads w from LDS when it fits.
template <bool kFirst>
__global__ __launch_bounds__(kThreads) void k_pow_rows(const PowSeg* __restrict__ segs, int nseg,
                                                       const double* __restrict__ w,
                                                       const double* __restrict__ inv,
                                                       double* __restrict__ u,
                                                       double* __restrict__ rpart) {
  __shared__ double red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) double wl[kFirst ? 1 : kPowWLds];
  const int64_t blk = blockIdx.x;
  const int si = find_by(segs, nseg, blk, &PowSeg::rblk0);
  const PowSeg sg = segs[si];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = static_cast<int>(blk - sg.rblk0) * kPowRowsPerBlock;
  const double v0 = 1.0 / sqrt(static_cast<double>(sg.cols));
  const double sc = kFirst ? 0.0 : inv[si];
  const double* ws = w + sg.w_off;
  const bool vec = pow_vec(sg);
  const bool lds = !kFirst && sg.cols <= kPowWLds;
  if (lds) {
    for (int j = threadIdx.x; j < sg.cols; j += kThreads) wl[j] = ws[j];
    __syncthreads();
  }
  double usq = 0.0;
  for (int k = 0; k < kPowRowsPerBlock / 4; ++k) {
    const int r = r0 + wave + 4 * k;
    if (r >= sg.rows) break;
    const float* row = sg.b + static_cast<int64_t>(r) * sg.ld;
    double d;
    if (lds)
      d = vec ? pow_row_dot<kFirst, true>(row, sg.cols, (const double*)wl, lane)
              : pow_row_dot<kFirst, false>(row, sg.cols, (const double*)wl, lane);
    else
      d = vec ? pow_row_dot<kFirst, true>(row, sg.cols, ws, lane)
              : pow_row_dot<kFirst, false>(row, sg.cols, ws, lane);
    double dot = wave_sum(d);
    dot *= kFirst ? v0 : sc;
    if (lane == 0) u[sg.u_off + r] = dot;
    usq += dot * dot;   // the same value in every lane after the reduction
  }
  if (lane != 0) usq = 0.0;
  usq = block_sum(usq, red);
  if (threadIdx.x == 0) rpart[blk] = usq;
}

// B^T u over one chunk of kPowRowsPerChunk rows: 4 consecutive columns per
// thread (one 16-byte load per row), into the chunk's partial wpart.
__global__ __launch_bounds__(kThreads) void k_pow_cols(const PowSeg* __restrict__ segs, int nseg,
                                                       const double* __restrict__ u,
                                                       double* __restrict__ wpart) {
  const int64_t blk = blockIdx.x;
  const PowSeg sg = segs[find_by(segs, nseg, blk, &PowSeg::cblk0)];
  const int ncb = static_cast<int>((sg.cols + kPowColsPerBlock - 1) / kPowColsPerBlock);
  const int local = static_cast<int>(blk - sg.cblk0);
  const int ch = local / ncb, cb = local - ch * ncb;
  const int r0 = ch * kPowRowsPerChunk;
  const int r1 = min(sg.rows, r0 + kPowRowsPerChunk);
  const int c = cb * kPowColsPerBlock + 4 * static_cast<int>(threadIdx.x);
  if (c >= sg.cols) return;
  const double* uu = u + sg.u_off;
  double* out = wpart + sg.wp_off + static_cast<int64_t>(ch) * sg.cols;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  if (pow_vec(sg)) {
    const float* col = sg.b + c;
    int r = r0;
    for (; r + 4 <= r1; r += 4) {
      const float4 x0 = *reinterpret_cast<const float4*>(col + static_cast<int64_t>(r) * sg.ld);
      const float4 x1 = *reinterpret_cast<const float4*>(col + static_cast<int64_t>(r + 1) * sg.ld);
      const float4 x2 = *reinterpret_cast<const float4*>(col + static_cast<int64_t>(r + 2) * sg.ld);
      const float4 x3 = *reinterpret_cast<const float4*>(col + static_cast<int64_t>(r + 3) * sg.ld);
      const double u0 = uu[r], u1 = uu[r + 1], u2 = uu[r + 2], u3 = uu[r + 3];
      a0 += x0.x * u0; a1 += x0.y * u0; a2 += x0.z * u0; a3 += x0.w * u0;
      a0 += x1.x * u1; a1 += x1.y * u1; a2 += x1.z * u1; a3 += x1.w * u1;
      a0 += x2.x * u2; a1 += x2.y * u2; a2 += x2.z * u2; a3 += x2.w * u2;
      a0 += x3.x * u3; a1 += x3.y * u3; a2 += x3.z * u3; a3 += x3.w * u3;
    }
    for (; r < r1; ++r) {
      const float4 x = *reinterpret_cast<const float4*>(col + static_cast<int64_t>(r) * sg.ld);
      const double ur = uu[r];
      a0 += x.x * ur; a1 += x.y * ur; a2 += x.z * ur; a3 += x.w * ur;
    }
    *reinterpret_cast<double2*>(out + c) = double2{a0, a1};
    *reinterpret_cast<double2*>(out + c + 2) = double2{a2, a3};
  } else {
    const int nc = min(4, sg.cols - c);
    for (int r = r0; r < r1; ++r) {
      const float* row = sg.b + static_cast<int64_t>(r) * sg.ld + c;
      const double ur = uu[r];
      a0 += static_cast<double>(row[0]) * ur;
      if (nc > 1) a1 += static_cast<double>(row[1]) * ur;
      if (nc > 2) a2 += static_cast<double>(row[2]) * ur;
      if (nc > 3) a3 += static_cast<double>(row[3]) * ur;
    }
    out[c] = a0;
    if (nc > 1) out[c + 1] = a1;
    if (nc > 2) out[c + 2] = a2;
    if (nc > 3) out[c + 3] = a3;
  }
}

// w = the sum of the chunks' partials (in chunk order), with one partial of
// sum w^2 per block.
__global__ __launch_bounds__(kThreads) void k_pow_fold(const PowSeg* __restrict__ segs, int nseg,
                                                       const double* __restrict__ wpart,
                                                       double* __restrict__ w,
                                                       double* __restrict__ cpart) {
  __shared__ double red[kThreads / 64];
  const int64_t blk = blockIdx.x;
  const PowSeg sg = segs[find_by(segs, nseg, blk, &PowSeg::kblk0)];
  const int c = static_cast<int>(blk - sg.kblk0) * kPowFoldCols + threadIdx.x;
  double s = 0.0;
  if (c < sg.cols) {
    const int nch = (sg.rows + kPowRowsPerChunk - 1) / kPowRowsPerChunk;
    const double* p = wpart + sg.wp_off + c;
    for (int ch = 0; ch < nch; ++ch) s += p[static_cast<int64_t>(ch) * sg.cols];
    w[sg.w_off + c] = s;
  }
  const double q = block_sum(s * s, red);
  if (threadIdx.x == 0) cpart[blk] = q;
}

// Per matrix: inv = 1 / ||w|| (0 when w vanishes) from the fold partials;
// or, after the last row pass, sigma = ||u|| and the cap factor.
template <bool kFinal>
__global__ __launch_bounds__(kThreads) void k_pow_norm(const PowSeg* __restrict__ segs, int nseg,
                                                       const double* __restrict__ part,
                                                       double* __restrict__ inv,
                                                       double* __restrict__ sigma,
                                                       float* __restrict__ kappa, float cap) {
  const int si = blockIdx.x * kThreads + threadIdx.x;
  if (si >= nseg) return;
  const PowSeg sg = segs[si];
  const int64_t p0 = kFinal ? sg.rblk0 : sg.kblk0;
  const int64_t np = kFinal ? (sg.rows + kPowRowsPerBlock - 1) / kPowRowsPerBlock
                            : (sg.cols + kPowFoldCols - 1) / kPowFoldCols;
  double s = 0.0;
  for (int64_t k = 0; k < np; ++k) s += part[p0 + k];
  const double n = sqrt(s);
  if (!kFinal) {
    inv[si] = n > 0.0 ? 1.0 / n : 0.0;
    return;
  }
  if (sigma) sigma[si] = n;
  if (kappa) kappa[si] = (cap > 0.f && n > static_cast<double>(cap))
                             ? static_cast<float>(static_cast<double>(cap) / n)
                             : 1.f;
}

}  // namespace

int64_t pow_row_blocks(int64_t rows) { return ceil_div(rows, kPowRowsPerBlock); }
int64_t pow_row_chunks(int64_t rows) { return ceil_div(rows, kPowRowsPerChunk); }
int64_t pow_col_blocks(int64_t rows, int64_t cols) {
  return pow_row_chunks(rows) * ceil_div(cols, kPowColsPerBlock);
}
int64_t pow_fold_blocks(int64_t cols) { return ceil_div(cols, kPowFoldCols); }

mo_status launch_power_iteration(const PowSeg* segs, int nseg, const PowGrid& g, int iters,
                                 const PowWork& wk, float cap, hipStream_t st) {
  if (nseg <= 0) return MO_OK;
  KTimer tm(MO_KC_SPECTRAL, st);
  const unsigned gr = static_cast<unsigned>(g.row_blocks), gc = static_cast<unsigned>(g.col_blocks);
  const unsigned gf = static_cast<unsigned>(g.fold_blocks);
  const unsigned gn = static_cast<unsigned>(ceil_div(nseg, kThreads));
  k_pow_rows<true><<<gr, kThreads, 0, st>>>(segs, nseg, wk.w, wk.inv, wk.u, wk.rpart);
  MO_LAUNCH_CHECK("k_pow_rows");
  for (int k = 0; k < iters; ++k) {
    k_pow_cols<<<gc, kThreads, 0, st>>>(segs, nseg, wk.u, wk.wpart);
    MO_LAUNCH_CHECK("k_pow_cols");
    k_pow_fold<<<gf, kThreads, 0, st>>>(segs, nseg, wk.wpart, wk.w, wk.cpart);
    MO_LAUNCH_CHECK("k_pow_fold");
    k_pow_norm<false><<<gn, kThreads, 0, st>>>(segs, nseg, wk.cpart, wk.inv, nullptr, nullptr,
                                                0.f);
    MO_LAUNCH_CHECK("k_pow_norm");
    k_pow_rows<false><<<gr, kThreads, 0, st>>>(segs, nseg, wk.w, wk.inv, wk.u, wk.rpart);
    MO_LAUNCH_CHECK("k_pow_rows");
  }
  k_pow_norm<true><<<gn, kThreads, 0, st>>>(segs, nseg, wk.rpart, nullptr, wk.sigma, wk.kappa,
                                             cap);
  MO_LAUNCH_CHECK("k_pow_norm");
  return MO_OK;
}

}  // namespace mo
