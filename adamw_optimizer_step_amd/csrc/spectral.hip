// Power-iteration estimate of each matrix's largest singular value, for the
// spectral-cap guard on the Muon buffer (OMN "Dual-Manifold Optimization"
// page, Muon-path paragraph: an optional guard with a power-iteration
// estimate, inactive by default).  Per matrix B (fp32, rows x cols):
//   v_0 = ones / sqrt(cols);  v_{k+1} = B^T B v_k / ||B^T B v_k||;
//   sigma = ||B v_K||.
// One iteration is a row pass (u = B v, one fp64 dot product per row, with
// the partial sums of u^2), a column pass (w = B^T u, one column per thread,
// with the partial sums of w^2) and a per-matrix norm; the estimate is the
// row pass after the last iteration.  All sums are fp64: the cap rescales an
// fp32 state, so the estimate must be good to far below fp32's unit
// roundoff relative to itself.  HBM-bound: each pass reads B once.
#include "kernels.hpp"

namespace mo {

namespace {

constexpr int kPowRowsPerBlock = 64;   // 4 waves x 16 rows
constexpr int kPowColsPerBlock = kThreads;

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

// u = B v for every row of every matrix (v_0 on the first pass, else
// w * inv), with one partial of sum u^2 per block.
template <bool kFirst>
__global__ __launch_bounds__(kThreads) void k_pow_rows(const PowSeg* __restrict__ segs, int nseg,
                                                       const double* __restrict__ w,
                                                       const double* __restrict__ inv,
                                                       double* __restrict__ u,
                                                       double* __restrict__ rpart) {
  __shared__ double red[kThreads / 64];
  const int64_t blk = blockIdx.x;
  const int si = find_by(segs, nseg, blk, &PowSeg::rblk0);
  const PowSeg sg = segs[si];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = static_cast<int>(blk - sg.rblk0) * kPowRowsPerBlock;
  const double v0 = 1.0 / sqrt(static_cast<double>(sg.cols));
  const double sc = kFirst ? 0.0 : inv[si];
  double usq = 0.0;
  for (int k = 0; k < kPowRowsPerBlock / 4; ++k) {
    const int r = r0 + wave + 4 * k;
    if (r >= sg.rows) break;
    const float* row = sg.b + static_cast<int64_t>(r) * sg.ld;
    double dot = 0.0;
#pragma unroll 4
    for (int j = lane; j < sg.cols; j += 64)
      dot += static_cast<double>(row[j]) * (kFirst ? v0 : w[sg.w_off + j] * sc);
    dot = wave_sum(dot);
    if (lane == 0) u[sg.u_off + r] = dot;
    usq += dot * dot;   // the same value in every lane after the reduction
  }
  if (lane != 0) usq = 0.0;
  usq = block_sum(usq, red);
  if (threadIdx.x == 0) rpart[blk] = usq;
}

// w = B^T u: one column per thread, every row in turn, with one partial of
// sum w^2 per block.
__global__ __launch_bounds__(kThreads) void k_pow_cols(const PowSeg* __restrict__ segs, int nseg,
                                                       const double* __restrict__ u,
                                                       double* __restrict__ w,
                                                       double* __restrict__ cpart) {
  __shared__ double red[kThreads / 64];
  const int64_t blk = blockIdx.x;
  const PowSeg sg = segs[find_by(segs, nseg, blk, &PowSeg::cblk0)];
  const int c = static_cast<int>(blk - sg.cblk0) * kPowColsPerBlock + threadIdx.x;
  double acc = 0.0;
  if (c < sg.cols) {
    const float* col = sg.b + c;
    const double* uu = u + sg.u_off;
    int r = 0;
    for (; r + 4 <= sg.rows; r += 4) {
      const float b0 = col[static_cast<int64_t>(r) * sg.ld];
      const float b1 = col[static_cast<int64_t>(r + 1) * sg.ld];
      const float b2 = col[static_cast<int64_t>(r + 2) * sg.ld];
      const float b3 = col[static_cast<int64_t>(r + 3) * sg.ld];
      acc += static_cast<double>(b0) * uu[r];
      acc += static_cast<double>(b1) * uu[r + 1];
      acc += static_cast<double>(b2) * uu[r + 2];
      acc += static_cast<double>(b3) * uu[r + 3];
    }
    for (; r < sg.rows; ++r) acc += static_cast<double>(col[static_cast<int64_t>(r) * sg.ld]) * uu[r];
    w[sg.w_off + c] = acc;
  }
  const double s = block_sum(acc * acc, red);
  if (threadIdx.x == 0) cpart[blk] = s;
}

// Per matrix: inv = 1 / ||w|| (0 when w vanishes) from the column partials;
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
  const int64_t p0 = kFinal ? sg.rblk0 : sg.cblk0;
  const int64_t np = kFinal ? (sg.rows + kPowRowsPerBlock - 1) / kPowRowsPerBlock
                            : (sg.cols + kPowColsPerBlock - 1) / kPowColsPerBlock;
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
int64_t pow_col_blocks(int64_t cols) { return ceil_div(cols, kPowColsPerBlock); }

mo_status launch_power_iteration(const PowSeg* segs, int nseg, int64_t row_blocks,
                                 int64_t col_blocks, int iters, const PowWork& wk, float cap,
                                 hipStream_t st) {
  if (nseg <= 0) return MO_OK;
  KTimer tm(MO_KC_SPECTRAL, st);
  const unsigned gr = static_cast<unsigned>(row_blocks), gc = static_cast<unsigned>(col_blocks);
  const unsigned gn = static_cast<unsigned>(ceil_div(nseg, kThreads));
  k_pow_rows<true><<<gr, kThreads, 0, st>>>(segs, nseg, wk.w, wk.inv, wk.u, wk.rpart);
  MO_LAUNCH_CHECK("k_pow_rows");
  for (int k = 0; k < iters; ++k) {
    k_pow_cols<<<gc, kThreads, 0, st>>>(segs, nseg, wk.u, wk.w, wk.cpart);
    MO_LAUNCH_CHECK("k_pow_cols");
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
