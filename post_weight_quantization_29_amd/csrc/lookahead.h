// A second stream per device for block lookahead in GPTQ's lazy-batch column
// loop.  Block k's trailing update is split: the part that the next block reads runs on the
// caller's stream right after panel k, the rest runs on the side stream while
// the caller's stream goes on to panel k + 1.  Two events order the streams:
// `panel_done` (recorded on the caller's stream after a panel, waited on by the
// side stream) and `trail_done` (recorded on the side stream after a trailing
// update, waited on by the caller's stream before the next update that touches
// the same rows).  Each event is waited on before it is recorded again, in host
// order, so one pair per device suffices; a per-device lock keeps the enqueue
// of one call in one piece when several host threads share a device.  Before
// returning, the caller's stream waits for the side stream's last update, so
// the call's work is complete, as seen from the caller's stream, exactly as if
// it had all been issued there.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdlib>
#include <cstring>
#include <mutex>

namespace gptq {

struct Lookahead {
  std::mutex mu;
  bool tried = false;
  bool ok = false;
  hipStream_t side = nullptr;
  hipEvent_t panel_done = nullptr;
  hipEvent_t trail_done = nullptr;
};

// The current device's lookahead state, created on first use (a non-blocking
// stream at the default priority, two events without timing); nullptr when
// the device cannot be queried, the objects cannot be created, or the
// environment sets GPTQ_LOOKAHEAD=0, and the loops then run on the caller's
// stream alone (same kernels, same results bit for bit).
inline Lookahead* lookahead_for_current_device() {
  static Lookahead table[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  Lookahead* la = &table[dev];
  std::lock_guard<std::mutex> g(la->mu);
  if (!la->tried) {
    la->tried = true;
    const char* env = std::getenv("GPTQ_LOOKAHEAD");
    if (env && std::strcmp(env, "0") == 0) return nullptr;
    la->ok = hipStreamCreateWithFlags(&la->side, hipStreamNonBlocking) == hipSuccess &&
             hipEventCreateWithFlags(&la->panel_done, hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&la->trail_done, hipEventDisableTiming) == hipSuccess;
  }
  return la->ok ? la : nullptr;
}

}  // namespace gptq
