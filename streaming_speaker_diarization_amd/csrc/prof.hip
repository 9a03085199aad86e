// Per-kernel-class timing for benchmarks. While a class is being profiled,
// every launch of that class carries a start/stop event pair that the
// dispatch records around the kernel itself (hipExtLaunchKernelGGL), and the
// launch's algorithmic flop and byte counts are accumulated (what the
// operation must compute and move, independent of how the kernel tiles it).
#include <vector>

#include "kernels.h"

namespace sf {

namespace {
struct Prof {
  bool on = false;
  int cls = 0;
  std::vector<hipEvent_t> ev;
  size_t used = 0;
  double flops = 0, bytes = 0;
  long long launches = 0;
};
Prof& P() {
  static Prof p;
  return p;
}
}  // namespace

bool profiling() { return P().on; }

bool prof_active(int cls) {
  Prof& p = P();
  return p.on && p.cls == cls && p.used + 2 <= p.ev.size();
}

void prof_next(hipEvent_t* start, hipEvent_t* stop, double flops, double bytes) {
  Prof& p = P();
  *start = p.ev[p.used];
  *stop = p.ev[p.used + 1];
  p.used += 2;
  p.flops += flops;
  p.bytes += bytes;
  p.launches += 1;
}

int prof_start(int cls, int max_launches) {
  Prof& p = P();
  if (p.on || max_launches < 1) return -1;
  for (auto e : p.ev) (void)hipEventDestroy(e);
  p.ev.assign((size_t)2 * max_launches, nullptr);
  for (auto& e : p.ev)
    if (hipEventCreate(&e) != hipSuccess) return -4;
  p.used = 0;
  p.flops = p.bytes = 0;
  p.launches = 0;
  p.cls = cls;
  p.on = true;
  return 0;
}

int prof_stop(double* ms, long long* launches, double* flops, double* bytes) {
  Prof& p = P();
  if (!p.on) return -5;
  p.on = false;
  double total = 0;
  for (size_t i = 0; i < p.used; i += 2) {
    if (hipEventSynchronize(p.ev[i + 1]) != hipSuccess) return -4;
    float t = 0;
    if (hipEventElapsedTime(&t, p.ev[i], p.ev[i + 1]) != hipSuccess) return -4;
    total += t;
  }
  if (ms) *ms = total;
  if (launches) *launches = p.launches;
  if (flops) *flops = p.flops;
  if (bytes) *bytes = p.bytes;
  return 0;
}

}  // namespace sf
