// Allocation-free variant of adamw_clip_step for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  The workspace of adamw_clip_step (segment table, fp64 partial
// sums, the norm T and the clip factor) lives in a file-scope device array of
// fixed size instead; each device holds its own copy, whose address is looked
// up once per device.  The kernels are the ones adamw_clip_step launches.
//
// Every byte a call reads from the array is written earlier in the same call
// on the same stream (the table by k_put_adam_table, every partial by
// k_adam_sumsq, T and the clip factor by k_adam_norm), so nothing has to be
// cleared between calls.  Calls on one device share the array: calls that
// overlap (on different streams, without ordering) race.
#include <mutex>

#include "host.hpp"

namespace mo {

namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;
constexpr int kNoAllocMaxItems = 64;            // AdamW items with a gradient per call
constexpr int kTableChunk = 32;                 // items per table-writing launch
constexpr size_t kTableBytes = 8192;            // segment table
constexpr size_t kScalOff = kTableBytes;        // T (fp64), clip factor
constexpr size_t kPartialsOff = kTableBytes + 256;
constexpr int64_t kMaxPartials =
    static_cast<int64_t>((kScratchBytes - kPartialsOff) / sizeof(double));
constexpr int kMaxDevices = 64;
static_assert(kNoAllocMaxItems * sizeof(AdamSeg) <= kTableBytes, "table fits");

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
char* g_ptr[kMaxDevices] = {};

struct TableChunk {
  AdamSeg s[kTableChunk];
};

__global__ __launch_bounds__(64) void k_put_adam_table(AdamSeg* __restrict__ dst, TableChunk c,
                                                       int n) {
  const int i = threadIdx.x;
  if (i < n) dst[i] = c.s[i];
}

// Device address of the current device's copy of `scratch` (looked up once
// per device, with that device current).
mo_status scratch_ptr(char** out) {
  int dev = 0;
  MO_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(MO_EINVAL, "device %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MO_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_ptr[dev];
  return MO_OK;
}

}  // namespace
}  // namespace mo

using namespace mo;

extern "C" mo_status adamw_clip_step_noalloc(const mo_adamw_item* items, int32_t n, float lr,
                                             float beta1, float beta2, float eps,
                                             float max_norm, double* norm_out, void* stream) {
  clear_error();
  if (n < 0 || (n > 0 && !items)) return fail(MO_EINVAL, "bad item list");
  AdamSeg segs[kNoAllocMaxItems];
  int nseg = 0;
  int64_t nblocks = 0;
  mo_status s = adam_segments(items, n, lr, beta1, beta2, eps, max_norm, segs, kNoAllocMaxItems,
                              &nseg, &nblocks);
  if (s != MO_OK) return s;
  if (sumsq_partial_count(nblocks) > kMaxPartials)
    return fail(MO_EWORKSPACE,
                "%lld AdamW blocks need %lld partial sums; the fixed scratch holds %lld "
                "(about %lld elements)",
                static_cast<long long>(nblocks),
                static_cast<long long>(sumsq_partial_count(nblocks)),
                static_cast<long long>(kMaxPartials),
                static_cast<long long>(kMaxPartials * kSumsqBlocksPerPartial * kEltPerBlock));
  char* base = nullptr;
  if ((s = scratch_ptr(&base)) != MO_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const KTimerOff quiet;   // no timing events: this path creates nothing
  AdamSeg* dsegs = reinterpret_cast<AdamSeg*>(base);
  for (int c0 = 0; c0 < nseg; c0 += kTableChunk) {
    TableChunk c;
    const int m = nseg - c0 < kTableChunk ? nseg - c0 : kTableChunk;
    for (int k = 0; k < m; ++k) c.s[k] = segs[c0 + k];
    k_put_adam_table<<<1, 64, 0, st>>>(dsegs + c0, c, m);
    MO_LAUNCH_CHECK("k_put_adam_table");
  }
  double* scal = reinterpret_cast<double*>(base + kScalOff);
  double* partials = reinterpret_cast<double*>(base + kPartialsOff);
  if ((s = launch_adam_sumsq(dsegs, nseg, nblocks, partials, st)) != MO_OK) return s;
  if ((s = launch_adam_norm(partials, nblocks, max_norm, scal, norm_out, st)) != MO_OK) return s;
  return launch_adam_apply(dsegs, nseg, nblocks, scal, lr, nullptr, 0, st);
}
