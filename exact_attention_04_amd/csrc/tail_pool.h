// Host side of the dynamic tail of the causal kernels (attn_fwd, attn_bwd).
//
// The light end of a causal grid (the query or key blocks with the least
// work) is handed out at run time through counters, so XCDs that run faster
// under load take more of it and the whole grid finishes together.  The
// counters live in a static device array of the kernel's file (zero when
// the library loads), kTailSlots slots per GPU.  Every call takes the next
// slot in turn and, before its kernels, makes its stream wait for a HIP
// event recorded after the previous call that used the slot; the last
// claimer of each counter returns it to zero.  So two calls in flight never
// share a counter, on any streams.  A call made while its stream is being
// captured into a graph gets no slot (a captured call would reuse it at
// every replay without the wait) and runs the fixed order.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>

namespace attn {

constexpr int kTailSlots = 64;
constexpr int kTailStride = 64;  // unsigned ints per slot: room for two counters on separate 128-byte lines
constexpr int kTailMaxDevices = 64;

struct TailPoolState {
  std::mutex mu;
  unsigned* base = nullptr;  // the array's address on this device
  unsigned next = 0;
  hipEvent_t done[kTailSlots] = {};
};

// Calls launch(counters) with the kTailStride counters of a fresh slot, or
// launch(nullptr) when the call must run the fixed order (stream capture, or
// any failure to get a slot).  get_symbol(void**) returns the device array's
// address on the current device (hipGetSymbolAddress in the defining file).
template <class GetSymbol, class Launch>
hipError_t with_tail_slot(TailPoolState (&states)[kTailMaxDevices], GetSymbol get_symbol, hipStream_t s,
                          Launch launch) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return launch(nullptr);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kTailMaxDevices) {
    (void)hipGetLastError();
    return launch(nullptr);
  }
  TailPoolState& ps = states[dev];
  std::lock_guard<std::mutex> lock(ps.mu);
  if (ps.base == nullptr) {
    void* p = nullptr;
    if (get_symbol(&p) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return launch(nullptr);
    }
    ps.base = static_cast<unsigned*>(p);
  }
  const int slot = (int)(ps.next++ % kTailSlots);
  hipError_t e = ps.done[slot] == nullptr ? hipEventCreateWithFlags(&ps.done[slot], hipEventDisableTiming)
                                          : hipStreamWaitEvent(s, ps.done[slot], 0);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return launch(nullptr);  // nothing ran on this slot
  }
  e = launch(ps.base + (size_t)slot * kTailStride);
  if (e != hipSuccess) return e;
  return hipEventRecord(ps.done[slot], s);
}

}  // namespace attn
