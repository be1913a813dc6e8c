// Memory-bound kernels: Muon momentum, AdamW with the global-norm clip, and
// the row kernels (NorMuon row normalisation, scaled Muon update).
//
// All are HBM-bound streaming passes over 2048 elements per 256-thread block,
// one launch over every tensor of a call (segment table + binary search).
// Momentum and AdamW give each thread two groups of 4 consecutive elements,
// 1024 apart, so that each access instruction of a wave covers one contiguous
// span (1 KiB of fp32, 512 bytes of bf16) and whole cache lines of every array.
#include "kernels.hpp"

namespace mo {

namespace {

typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// 4 consecutive elements <-> 4 floats: one 16-byte fp32 or 8-byte bf16
// access.  `i` is a multiple of 4 and the base pointer 16-byte aligned.
template <bool NT>
__device__ __forceinline__ void load4(const void* p, int64_t i, int32_t dt, float* v) {
  if (dt == MO_F32) {
    const f32x4_t a = ldv<f32x4_t, NT>(reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i));
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = a[k];
  } else {
    const u32x2_t u =
        ldv<u32x2_t, NT>(reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(p) + i));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      v[2 * k] = __uint_as_float(u[k] << 16);
      v[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
  }
}

template <bool NT>
__device__ __forceinline__ void store4(void* p, int64_t i, int32_t dt, const float* v) {
  if (dt == MO_F32) {
    stv<f32x4_t, NT>(reinterpret_cast<f32x4_t*>(static_cast<float*>(p) + i),
                     f32x4_t{v[0], v[1], v[2], v[3]});
  } else {
    u32x2_t u;
#pragma unroll
    for (int k = 0; k < 2; ++k)
      u[k] = pk_bf16(v[2 * k], v[2 * k + 1]);
    stv<u32x2_t, NT>(reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p) + i), u);
  }
}

// Groups of 4 per thread in a block, and the distance between a thread's groups.
constexpr int kGroups = kEltPerBlock / (kThreads * 4);
constexpr int kGroupStride = kThreads * 4;

// (1 - beta^t) by binary exponentiation in fp64 (t >= 1).
__device__ double one_minus_pow(double beta, int t) {
  double r = 1.0, b = beta;
  while (t > 0) {
    if (t & 1) r *= b;
    b *= b;
    t >>= 1;
  }
  return 1.0 - r;
}

// ---------------------------------------------------------------------------
// Momentum: B <- mu B + G ; D <- G + mu B (Nesterov) or B.
// (OMN "Dual-Manifold Optimization", Muon-path paragraph; NorMuon eq. (1).)
// ---------------------------------------------------------------------------
template <bool kStats, int kPhase>
__global__ __launch_bounds__(kThreads) void k_momentum(const MomSeg* __restrict__ segs, int nseg,
                                                       float mu, int nesterov,
                                                       StatPartial* __restrict__ stats,
                                                       const float* __restrict__ kappa) {
  const int64_t blk = blockIdx.x;
  const int si = find_segment(segs, nseg, blk);
  const MomSeg sg = segs[si];
  // phase 2: the spectral-cap factor of this segment (1 leaves B as stored)
  const float kap = kPhase == 2 ? kappa[si] : 1.f;
  const int64_t base = (blk - sg.start) * kEltPerBlock;
  float amax = 0.f;
  double ss = 0.0;
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const int64_t e0 = base + q * kGroupStride + threadIdx.x * 4;
    if (e0 >= sg.numel) break;
    float g[4], b[4], d[4];
    const int cnt = sg.numel - e0 >= 4 ? 4 : static_cast<int>(sg.numel - e0);
    const bool vec = cnt == 4 && sg.vec;
    if (vec) {
      load4<true>(sg.g, e0, sg.gdt, g);
      load4<true>(sg.b, e0, MO_F32, b);
    } else {
      for (int k = 0; k < 4; ++k) {
        g[k] = k < cnt ? load_as_f32(sg.g, e0 + k, sg.gdt) : 0.f;
        b[k] = k < cnt ? sg.b[e0 + k] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      b[k] = kPhase == 2 ? kap * b[k] : mu * b[k] + g[k];
      d[k] = nesterov ? g[k] + mu * b[k] : b[k];
    }
    const bool store_b = kPhase != 2 || kap != 1.f;
    void* const dst = kPhase == 1 ? nullptr : sg.d;
    if (vec) {
      if (store_b) store4<true>(sg.b, e0, MO_F32, b);
      if (dst) store4<true>(dst, e0, sg.ddt, d);
    } else {
      for (int k = 0; k < cnt; ++k) {
        if (store_b) sg.b[e0 + k] = b[k];
        if (dst) store_from_f32(dst, e0 + k, sg.ddt, d[k]);
      }
    }
    if (kStats) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // statistics of the value as stored
        const float dv = sg.ddt == MO_BF16 ? bf16_to_f32(f32_to_bf16(d[k])) : d[k];
        const float a = k < cnt ? fabsf(dv) : 0.f;
        amax = fmaxf(amax, a);
        ss += static_cast<double>(a) * a;
      }
    }
  }
  if (kStats) block_stat_reduce(amax, ss, &stats[blk]);
}

// ---------------------------------------------------------------------------
// AdamW (OMN page, recipe paragraph; Qwen3.8 optimizer notes, Adam/AdamW).
// ---------------------------------------------------------------------------
// Sum of squares of the gradients: each block covers kSumsqSub blocks of the
// apply kernel's partition, one 16-byte load of 8 elements per thread and
// block, all issued before the reduction (four independent fp64 sums), and
// writes one partial.
constexpr int kSumsqSub = kSumsqBlocksPerPartial;
static_assert(kEltPerBlock == kThreads * 8,
              "k_adam_sumsq covers a block with one 8-element chunk per thread");
__host__ __device__ constexpr int64_t sumsq_partials(int64_t nblocks) {
  return sumsq_partial_count(nblocks);
}

__global__ __launch_bounds__(kThreads) void k_adam_sumsq(const AdamSeg* __restrict__ segs, int nseg,
                                                         int64_t nblocks,
                                                         double* __restrict__ partials) {
  float g[kSumsqSub][8];
#pragma unroll
  for (int j = 0; j < kSumsqSub; ++j) {
    const int64_t ab = static_cast<int64_t>(blockIdx.x) * kSumsqSub + j;
    const AdamSeg* sp = ab < nblocks ? &segs[find_segment(segs, nseg, ab)] : nullptr;
    const int64_t e0 = sp ? (ab - sp->start) * kEltPerBlock + threadIdx.x * 8 : 0;
    const int64_t left = sp ? sp->numel - e0 : 0;
    if (left >= 8) {
      load8(sp->g, e0, sp->dt, g[j]);
    } else {
      for (int k = 0; k < 8; ++k) g[j][k] = k < left ? load_as_f32(sp->g, e0 + k, sp->dt) : 0.f;
    }
  }
  double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int j = 0; j < kSumsqSub; ++j)
#pragma unroll
    for (int k = 0; k < 8; ++k) s4[k & 3] += static_cast<double>(g[j][k]) * g[j][k];
  double ss = (s4[0] + s4[1]) + (s4[2] + s4[3]);
  __shared__ double s_ss[4];
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) s_ss[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) partials[blockIdx.x] = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
}

constexpr int kNormThreads = 1024;
__global__ __launch_bounds__(kNormThreads) void k_adam_norm(const double* __restrict__ partials,
                                                            int64_t n, float max_norm,
                                                            double* __restrict__ scal,
                                                            double* __restrict__ norm_out) {
  double s = 0.0;
#pragma unroll 4
  for (int64_t i = threadIdx.x; i < n; i += kNormThreads) s += partials[i];
  __shared__ double s_ss[kNormThreads / 64];
  s = wave_sum(s);
  if ((threadIdx.x & 63) == 0) s_ss[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int k = 0; k < kNormThreads / 64; ++k) t += s_ss[k];
    const double T = sqrt(t);
    const double kappa = (max_norm > 0.f && T > static_cast<double>(max_norm))
                             ? static_cast<double>(max_norm) / T
                             : 1.0;
    scal[0] = T;
    reinterpret_cast<float*>(scal + 1)[0] = static_cast<float>(kappa);
    if (norm_out) *norm_out = T;
  }
}

__global__ __launch_bounds__(kThreads) void k_adam_apply(const AdamSeg* __restrict__ segs, int nseg,
                                                         const double* __restrict__ scal,
                                                         float lr_arg,
                                                         const float* __restrict__ lrs,
                                                         int32_t tdelta,
                                                         const int32_t* __restrict__ tcount) {
  const int64_t blk = blockIdx.x;
  const AdamSeg sg = segs[find_segment(segs, nseg, blk)];
  // steps since the tables were built: the device counter (advanced at the
  // start of every grouped step, so that a step replayed from a graph still
  // takes the next step's bias correction), else the argument
  if (tcount != nullptr) tdelta = *tcount - 1;
  const int64_t base = (blk - sg.start) * kEltPerBlock;
  const float kappa = reinterpret_cast<const float*>(scal + 1)[0];
  const float lr = lrs ? lrs[sg.lr_slot] : lr_arg;
  const float beta1 = sg.beta1, beta2 = sg.beta2, eps = sg.eps;
  const int t = sg.t0 + tdelta;
  const double bc1 = one_minus_pow(beta1, t);
  const double bc2 = one_minus_pow(beta2, t);
  const float step = static_cast<float>(lr / bc1);
  const float ibc2 = static_cast<float>(1.0 / sqrt(bc2));
  const float decay = 1.f - lr * sg.wd;
  const float omb1 = 1.f - beta1, omb2 = 1.f - beta2;
#pragma unroll
  for (int q = 0; q < kGroups; ++q) {
    const int64_t e0 = base + q * kGroupStride + threadIdx.x * 4;
    if (e0 >= sg.numel) break;
    float g[4], w[4], m[4], v[4];
    const int cnt = sg.numel - e0 >= 4 ? 4 : static_cast<int>(sg.numel - e0);
    if (cnt == 4) {
      load4<true>(sg.g, e0, sg.dt, g);
      load4<true>(sg.p, e0, sg.dt, w);
      load4<true>(sg.m, e0, MO_F32, m);
      load4<true>(sg.v, e0, MO_F32, v);
    } else {
      for (int k = 0; k < 4; ++k) {
        const bool in = k < cnt;
        g[k] = in ? load_as_f32(sg.g, e0 + k, sg.dt) : 0.f;
        w[k] = in ? load_as_f32(sg.p, e0 + k, sg.dt) : 0.f;
        m[k] = in ? sg.m[e0 + k] : 0.f;
        v[k] = in ? sg.v[e0 + k] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float gk = kappa * g[k];
      m[k] = beta1 * m[k] + omb1 * gk;
      v[k] = beta2 * v[k] + omb2 * gk * gk;
      const float denom = sqrtf(v[k]) * ibc2 + eps;
      w[k] = w[k] * decay - step * (m[k] / denom);
    }
    if (cnt == 4) {
      store4<true>(sg.p, e0, sg.dt, w);
      store4<true>(sg.m, e0, MO_F32, m);
      store4<true>(sg.v, e0, MO_F32, v);
    } else {
      for (int k = 0; k < cnt; ++k) {
        store_from_f32(sg.p, e0 + k, sg.dt, w[k]);
        sg.m[e0 + k] = m[k];
        sg.v[e0 + k] = v[k];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row kernels: one wavefront per row.
//   NorMuon (NorMuon paper section 3.1): ms = mean_j O_ij^2,
//     v_i <- beta2 v_i + (1 - beta2) ms, O_ij <- O_ij / (sqrt(v_i) + eps).
//   Update (NorMuon eq. (3); OMN rectangular-scaling paragraph):
//     W <- W (1 - lr wd) - lr scale O.
// ---------------------------------------------------------------------------
template <int kMode>
__global__ __launch_bounds__(kThreads) void k_rows(const RowSeg* __restrict__ segs, int nseg,
                                                   RowSeg one, int64_t total_rows, float lr_arg,
                                                   const float* __restrict__ lrs, float beta2,
                                                   float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  // nseg == 0: a single matrix passed by value
  const RowSeg sg = nseg == 0 ? one : segs[find_segment(segs, nseg, row)];
  const int64_t r = row - sg.start;
  const int cols = sg.cols;
  const int64_t obase = r * sg.ld_o;
  const int64_t wbase = r * sg.ld_w;
  // vector path when every row start is 16-byte aligned and cols % 8 == 0
  const bool vec_o = (cols % 8 == 0) && ((sg.ld_o * (sg.o_dt == MO_F32 ? 4 : 2)) % 16 == 0) &&
                     aligned16(sg.o);
  const bool vec_w = (cols % 8 == 0) && ((sg.ld_w * (sg.w_dt == MO_F32 ? 4 : 2)) % 16 == 0) &&
                     aligned16(sg.w);
  float inv = 1.f;
  if (kMode != kRowUpdate) {
    double ss = 0.0;
    if (vec_o) {
      for (int c0 = lane * 8; c0 < cols; c0 += 64 * 8) {
        float o[8];
        load8(sg.o, obase + c0, sg.o_dt, o);
#pragma unroll
        for (int k = 0; k < 8; ++k) ss += static_cast<double>(o[k]) * o[k];
      }
    } else {
      for (int c = lane; c < cols; c += 64) {
        const float o = load_as_f32(sg.o, obase + c, sg.o_dt);
        ss += static_cast<double>(o) * o;
      }
    }
    ss = wave_sum(ss);
    const double ms = ss / cols;
    const float vnew = static_cast<float>(beta2 * static_cast<double>(sg.nv[r]) +
                                          (1.0 - beta2) * ms);
    if (lane == 0) sg.nv[r] = vnew;
    inv = 1.f / (sqrtf(vnew) + eps);
  }
  if (kMode == kRowNormInPlace) {
    if (vec_o) {
      for (int c0 = lane * 8; c0 < cols; c0 += 64 * 8) {
        float o[8];
        load8(sg.o, obase + c0, sg.o_dt, o);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] *= inv;
        store8(sg.o, obase + c0, sg.o_dt, o);
      }
    } else {
      for (int c = lane; c < cols; c += 64)
        store_from_f32(sg.o, obase + c, sg.o_dt, load_as_f32(sg.o, obase + c, sg.o_dt) * inv);
    }
    return;
  }
  const float lr = lrs ? lrs[sg.lr_slot] : lr_arg;
  const float decay = 1.f - lr * sg.wd;
  const float coef = lr * sg.scale * inv;
  if (vec_o && vec_w) {
#pragma unroll 2
    for (int c0 = lane * 8; c0 < cols; c0 += 64 * 8) {
      float o[8], w[8];
      load8<true>(sg.o, obase + c0, sg.o_dt, o);
      load8<true>(sg.w, wbase + c0, sg.w_dt, w);
#pragma unroll
      for (int k = 0; k < 8; ++k) w[k] = muon_apply(w[k], o[k], decay, coef);
      store8<true>(sg.w, wbase + c0, sg.w_dt, w);
    }
  } else {
    for (int c = lane; c < cols; c += 64) {
      const float o = load_as_f32(sg.o, obase + c, sg.o_dt);
      const float w = load_as_f32(sg.w, wbase + c, sg.w_dt);
      store_from_f32(sg.w, wbase + c, sg.w_dt, muon_apply(w, o, decay, coef));
    }
  }
}

}  // namespace

mo_status launch_momentum(const MomSeg* segs, int nseg, int64_t nblocks, float mu, int nesterov,
                          StatPartial* stats, hipStream_t st, int phase, const float* kappa) {
  if (nblocks <= 0) return MO_OK;
  if (phase == 2 && !kappa) return fail(MO_EINVAL, "momentum phase 2 needs the cap factors");
  KTimer tm(MO_KC_MOMENTUM, st);
  const dim3 grid(static_cast<unsigned>(nblocks));
  if (phase == 1)
    k_momentum<false, 1><<<grid, dim3(kThreads), 0, st>>>(segs, nseg, mu, nesterov, nullptr,
                                                           nullptr);
  else if (phase == 2 && stats)
    k_momentum<true, 2><<<grid, dim3(kThreads), 0, st>>>(segs, nseg, mu, nesterov, stats, kappa);
  else if (phase == 2)
    k_momentum<false, 2><<<grid, dim3(kThreads), 0, st>>>(segs, nseg, mu, nesterov, nullptr,
                                                           kappa);
  else if (stats)
    k_momentum<true, 0><<<grid, dim3(kThreads), 0, st>>>(segs, nseg, mu, nesterov, stats,
                                                          nullptr);
  else
    k_momentum<false, 0><<<grid, dim3(kThreads), 0, st>>>(segs, nseg, mu, nesterov, nullptr,
                                                           nullptr);
  MO_LAUNCH_CHECK("k_momentum");
  return MO_OK;
}

mo_status launch_adam_sumsq(const AdamSeg* segs, int nseg, int64_t nblocks, double* partials,
                            hipStream_t st) {
  if (nblocks <= 0) return MO_OK;
  KTimer tm(MO_KC_ADAM_SUMSQ, st);
  k_adam_sumsq<<<dim3(static_cast<unsigned>(sumsq_partials(nblocks))), dim3(kThreads), 0, st>>>(
      segs, nseg, nblocks, partials);
  MO_LAUNCH_CHECK("k_adam_sumsq");
  return MO_OK;
}

mo_status launch_adam_norm(const double* partials, int64_t nblocks, float max_norm, double* scal,
                           double* norm_out, hipStream_t st) {
  KTimer tm(MO_KC_ADAM_NORM, st);
  k_adam_norm<<<dim3(1), dim3(kNormThreads), 0, st>>>(partials, sumsq_partials(nblocks), max_norm,
                                                       scal, norm_out);
  MO_LAUNCH_CHECK("k_adam_norm");
  return MO_OK;
}

mo_status launch_adam_apply(const AdamSeg* segs, int nseg, int64_t nblocks, const double* scal,
                            float lr, const float* lrs, int32_t tdelta, hipStream_t st,
                            const int32_t* tcount) {
  if (nblocks <= 0) return MO_OK;
  KTimer tm(MO_KC_ADAM_APPLY, st);
  k_adam_apply<<<dim3(static_cast<unsigned>(nblocks)), dim3(kThreads), 0, st>>>(
      segs, nseg, scal, lr, lrs, tdelta, tcount);
  MO_LAUNCH_CHECK("k_adam_apply");
  return MO_OK;
}

mo_status launch_rows(int32_t mode, const RowSeg* segs, int nseg, const RowSeg& one,
                      int64_t total_rows, float lr, const float* lrs, float beta2, float eps,
                      hipStream_t st) {
  if (total_rows <= 0) return MO_OK;
  const unsigned grid = static_cast<unsigned>(ceil_div(total_rows, kThreads / 64));
  KTimer tm(MO_KC_ROWS, st);
  switch (mode) {
    case kRowUpdate:
      k_rows<kRowUpdate><<<grid, kThreads, 0, st>>>(segs, nseg, one, total_rows, lr, lrs, beta2,
                                                     eps);
      break;
    case kRowNormUpdate:
      k_rows<kRowNormUpdate><<<grid, kThreads, 0, st>>>(segs, nseg, one, total_rows, lr, lrs,
                                                         beta2, eps);
      break;
    default:
      k_rows<kRowNormInPlace><<<grid, kThreads, 0, st>>>(segs, nseg, one, total_rows, lr, lrs,
                                                          beta2, eps);
      break;
  }
  MO_LAUNCH_CHECK("k_rows");
  return MO_OK;
}

// ---------------------------------------------------------------------------
// Per-step learning-rate table, written from the kernel's arguments.
// ---------------------------------------------------------------------------
struct LrArgs {
  float v[kMaxLrSlots];
};

__global__ __launch_bounds__(kThreads) void k_set_lrs(float* __restrict__ dst, LrArgs a, int n,
                                                      int32_t* __restrict__ tcount) {
  for (int i = threadIdx.x; i < n; i += kThreads) dst[i] = a.v[i];
  if (tcount != nullptr && threadIdx.x == 0) *tcount += 1;
}

mo_status launch_set_lrs(float* dst, const float* vals, int n, hipStream_t st, int32_t* tcount) {
  if (n <= 0 && tcount == nullptr) return MO_OK;
  if (n > kMaxLrSlots) return fail(MO_EINVAL, "%d learning-rate slots (at most %d)", n,
                                   kMaxLrSlots);
  LrArgs a;
  for (int i = 0; i < kMaxLrSlots; ++i) a.v[i] = i < n ? vals[i] : 0.f;
  k_set_lrs<<<1, kThreads, 0, st>>>(dst, a, n, tcount);
  MO_LAUNCH_CHECK("k_set_lrs");
  return MO_OK;
}

// ---------------------------------------------------------------------------
// Plain device copy of a known byte count (one non-temporal 16-byte load and
// store per thread): the reference point that scales hardware byte counters,
// and the practical ceiling of a read + write stream.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_diag_copy(const u32x4_t* __restrict__ src,
                                                        u32x4_t* __restrict__ dst, int64_t n16) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n16) stv<u32x4_t, true>(dst + i, ldv<u32x4_t, true>(src + i));
}

mo_status launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  if (bytes <= 0) return MO_OK;
  const int64_t n16 = bytes / 16;
  const int64_t grid = ceil_div(n16, kThreads);
  if (grid > 0x7fffffff) return fail(MO_EINVAL, "copy of %lld bytes is too large",
                                     static_cast<long long>(bytes));
  k_diag_copy<<<static_cast<unsigned>(grid), kThreads, 0, st>>>(
      static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), n16);
  MO_LAUNCH_CHECK("k_diag_copy");
  return MO_OK;
}

}  // namespace mo
