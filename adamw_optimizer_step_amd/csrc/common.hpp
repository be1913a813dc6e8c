// Shared host/device helpers of the hybrid Muon + AdamW library (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/muon_adamw.h"

namespace mo {

// ---------------------------------------------------------------------------
// Error reporting (thread-local message, status returned to the caller)
// ---------------------------------------------------------------------------
mo_status fail(mo_status s, const char* fmt, ...);
void clear_error();

#define MO_HIP_TRY(expr)                                                          \
  do {                                                                            \
    hipError_t e_ = (expr);                                                       \
    if (e_ != hipSuccess)                                                         \
      return ::mo::fail(MO_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));  \
  } while (0)

#define MO_LAUNCH_CHECK(name)                                                     \
  do {                                                                            \
    hipError_t e_ = hipGetLastError();                                            \
    if (e_ != hipSuccess)                                                         \
      return ::mo::fail(MO_EHIP, "launch of %s failed: %s", name,                 \
                        hipGetErrorString(e_));                                   \
  } while (0)

inline bool valid_dtype(int32_t d) { return d == MO_F32 || d == MO_BF16; }
inline size_t dtype_size(int32_t d) { return d == MO_F32 ? 4 : 2; }
__host__ __device__ inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Bump allocator over the caller's workspace (offsets only; no memory touched).
struct WsCursor {
  size_t off = 0;
  size_t take(size_t bytes, size_t align = 256) {
    off = align_up(off, align);
    size_t at = off;
    off += bytes;
    return at;
  }
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.  The casts
// select gfx950's v_cvt_pk_bf16_f32, whose results equal the integer
// rounding (add 0x7fff plus the kept lsb, truncate) for every non-NaN input.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two values -> packed bf16, lo | hi << 16 (one conversion instruction).
__device__ __forceinline__ uint32_t pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float load_as_f32(const void* p, int64_t i, int32_t dt) {
  return dt == MO_F32 ? static_cast<const float*>(p)[i]
                      : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

__device__ __forceinline__ void store_from_f32(void* p, int64_t i, int32_t dt, float v) {
  if (dt == MO_F32)
    static_cast<float*>(p)[i] = v;
  else
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
}

// 8 consecutive elements <-> 8 floats.  Pointers must be 16-byte aligned.
// NT = non-temporal (streaming) access, for data a launch touches once.
// Device memory only, never LDS: through a global-address-space pointer the
// access is a global instruction, counted by the vector-memory counter alone
// (a flat one, which a pointer read from memory would otherwise give, also
// counts as an LDS access, so that every wait on LDS accesses waited for it).
template <typename V>
using gptr = __attribute__((address_space(1))) V*;
template <typename V, bool NT>
__device__ __forceinline__ V ldv(const V* q) {
  const gptr<const V> g = (gptr<const V>)(q);
  if constexpr (NT)
    return __builtin_nontemporal_load(g);
  else
    return *g;
}
template <typename V, bool NT>
__device__ __forceinline__ void stv(V* q, const V& v) {
  const gptr<V> g = (gptr<V>)(q);
  if constexpr (NT)
    __builtin_nontemporal_store(v, g);
  else
    *g = v;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <bool NT = false>
__device__ __forceinline__ void load8(const void* p, int64_t i, int32_t dt, float* v) {
  if (dt == MO_F32) {
    const f32x4_t* q = reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p) + i);
    const f32x4_t a = ldv<f32x4_t, NT>(q), b = ldv<f32x4_t, NT>(q + 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) { v[k] = a[k]; v[4 + k] = b[k]; }
  } else {
    const u32x4_t u =
        ldv<u32x4_t, NT>(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(p) + i));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(u[k] << 16);
      v[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
  }
}

template <bool NT = false>
__device__ __forceinline__ void store8(void* p, int64_t i, int32_t dt, const float* v) {
  if (dt == MO_F32) {
    f32x4_t* q = reinterpret_cast<f32x4_t*>(static_cast<float*>(p) + i);
    stv<f32x4_t, NT>(q, f32x4_t{v[0], v[1], v[2], v[3]});
    stv<f32x4_t, NT>(q + 1, f32x4_t{v[4], v[5], v[6], v[7]});
  } else {
    u32x4_t u;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      u[k] = pk_bf16(v[2 * k], v[2 * k + 1]);
    stv<u32x4_t, NT>(reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p) + i), u);
  }
}

__device__ __forceinline__ float4 ld_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }

// Muon weight update of one element, W (1 - lr wd) - lr scale O: one rounded
// product W * decay, then one fused multiply-add.  Every kernel that applies
// the update uses this exact sequence, so the separate pass and the update
// fused into the last Newton-Schulz launch give identical bits.
__device__ __forceinline__ float muon_apply(float w, float o, float decay, float coef) {
  return __builtin_fmaf(-coef, o, w * decay);
}

// 8 consecutive weights (dtype dt, 16-byte aligned) as raw bits: one
// streaming 16-byte load for bf16, two for fp32.  Loaded ahead of the
// updates below so that a thread's loads are all in flight at once.
struct W8 {
  u32x4_t a, b;
};
__device__ __forceinline__ W8 load_w8(const void* w, int64_t i, int32_t dt) {
  W8 r;
  if (dt == MO_F32) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(static_cast<const float*>(w) + i);
    r.a = ldv<u32x4_t, true>(q);
    r.b = ldv<u32x4_t, true>(q + 1);
  } else {
    r.a = ldv<u32x4_t, true>(reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(w) + i));
    r.b = u32x4_t{0u, 0u, 0u, 0u};
  }
  return r;
}

// The update on those 8 weights from 8 bf16 values of O packed in `o`, low
// half first; the result is stored (streaming) in the weights' dtype.
__device__ __forceinline__ void apply_w8(void* w, int64_t i, int32_t dt, const W8& raw,
                                         const u32x4_t& o, float decay, float coef) {
  float wf[8];
  if (dt == MO_F32) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      wf[k] = __uint_as_float(raw.a[k]);
      wf[4 + k] = __uint_as_float(raw.b[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      wf[2 * k] = __uint_as_float(raw.a[k] << 16);
      wf[2 * k + 1] = __uint_as_float(raw.a[k] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    wf[2 * k] = muon_apply(wf[2 * k], __uint_as_float(o[k] << 16), decay, coef);
    wf[2 * k + 1] = muon_apply(wf[2 * k + 1], __uint_as_float(o[k] & 0xffff0000u), decay, coef);
  }
  store8<true>(w, i, dt, wf);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Largest index p in [0, n) with start[p] <= key (start ascending, start[0] == 0).
template <typename S, typename K>
__device__ __forceinline__ int find_segment(const S* segs, int n, K key) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (segs[mid].start <= key) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Per-block partial statistics of a Newton-Schulz input (max |d| and sum d^2).
struct StatPartial {
  float amax;
  float pad;
  double sumsq;
};

// Block-wide reduction of (amax, sumsq) over 256 threads in a fixed order.
__device__ __forceinline__ void block_stat_reduce(float amax, double ss, StatPartial* out) {
  __shared__ float s_amax[4];
  __shared__ double s_ss[4];
  amax = wave_max(amax);
  ss = wave_sum(ss);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s_amax[w] = amax; s_ss[w] = ss; }
  __syncthreads();
  if (threadIdx.x == 0) {
    StatPartial p;
    p.amax = fmaxf(fmaxf(s_amax[0], s_amax[1]), fmaxf(s_amax[2], s_amax[3]));
    p.pad = 0.f;
    p.sumsq = (s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3]);
    *out = p;
  }
}

}  // namespace mo
