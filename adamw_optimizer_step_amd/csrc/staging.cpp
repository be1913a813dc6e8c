// Host -> device upload of descriptor tables through pinned staging buffers.
//
// A small ring of pinned buffers per thread; each buffer carries the event
// recorded after its last copy, and is reused only after that event has
// completed, so the caller's host data may be released as soon as the call
// returns while the copy itself stays asynchronous on the caller's stream.
#include <cstring>

#include "host.hpp"

namespace mo {

namespace {
struct StageBuf {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

struct StageRing {
  StageBuf bufs[4];
  int next = 0;
  ~StageRing() {
    for (StageBuf& b : bufs) {
      if (b.pending) (void)hipEventSynchronize(b.ev);
      if (b.ev) (void)hipEventDestroy(b.ev);
      if (b.host) (void)hipHostFree(b.host);
    }
  }
};

thread_local StageRing g_ring;
}  // namespace

mo_status stage_upload(void* dst, const void* src, size_t bytes, hipStream_t st) {
  if (bytes == 0) return MO_OK;
  StageBuf& b = g_ring.bufs[g_ring.next];
  g_ring.next = (g_ring.next + 1) % 4;
  if (b.pending) {
    MO_HIP_TRY(hipEventSynchronize(b.ev));
    b.pending = false;
  }
  if (!b.ev) MO_HIP_TRY(hipEventCreateWithFlags(&b.ev, hipEventDisableTiming));
  if (b.cap < bytes) {
    if (b.host) MO_HIP_TRY(hipHostFree(b.host));
    b.host = nullptr;
    b.cap = 0;
    const size_t cap = align_up(bytes, 1 << 16);
    MO_HIP_TRY(hipHostMalloc(&b.host, cap, hipHostMallocDefault));
    b.cap = cap;
  }
  std::memcpy(b.host, src, bytes);
  MO_HIP_TRY(hipMemcpyAsync(dst, b.host, bytes, hipMemcpyHostToDevice, st));
  MO_HIP_TRY(hipEventRecord(b.ev, st));
  b.pending = true;
  return MO_OK;
}

}  // namespace mo
