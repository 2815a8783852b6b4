// Launching kernels whose workgroups wait on each other (the persistent
// conv + normalisation and the one-launch GEMM + row-min): how many
// workgroups the current device keeps resident at once, and the launch.
//
// Such a kernel is correct only if every workgroup it waits for is resident
// together with it.  The launch paths check grid <= resident_capacity() and
// then either
//   - launch it as an ordinary kernel (the default): on a device that runs
//     nothing else at the same time, the dispatcher places every workgroup of
//     a grid that fits at once, and the stream's order means the kernels
//     before it have finished; or
//   - launch it cooperatively (hipLaunchCooperativeKernel), for callers that
//     run other work on the device concurrently: the runtime then guarantees
//     co-residency, at the price of a queue synchronisation on each side of
//     the launch (~11 us each on MI355X).
// Every wait is bounded either way (grid_sync.hpp), so a workgroup denied
// co-residency gives up and poisons its output with NaN instead of hanging.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <mutex>

#include "launch.hpp"

namespace c1g {
namespace {

struct CapEntry {
  int dev;
  const void* kernel;
  int threads;
  int value;
};

constexpr int kMaxEntries = 64;
std::mutex cap_mutex;
CapEntry cap_table[kMaxEntries];
int cap_used = 0;

int query_capacity(int dev, const void* kernel, int threads) {
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
    return 0;
  return cus * per_cu;
}

// The environment variable C1G_RESIDENT_LIMIT (a positive integer, read at
// each call) caps the capacity reported below, so that the paths of a device
// that keeps fewer workgroups resident (fewer samples per round of the
// persistent conv, the split route in its place, two launches instead of the
// one-launch row-min) can be exercised on any device.  0: no cap.
int resident_limit() {
  const char* e = std::getenv("C1G_RESIDENT_LIMIT");
  if (e == nullptr || *e == '\0') return 0;
  char* end = nullptr;
  const long v = std::strtol(e, &end, 10);
  return (end != nullptr && *end == '\0' && v > 0 && v < (1l << 30)) ? (int)v : 0;
}

int capped(int v) {
  const int lim = resident_limit();
  return (lim > 0 && lim < v) ? lim : v;
}

}  // namespace

int resident_capacity(const void* kernel, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(cap_mutex);
  for (int i = 0; i < cap_used; ++i)
    if (cap_table[i].dev == dev && cap_table[i].kernel == kernel &&
        cap_table[i].threads == threads)
      return capped(cap_table[i].value);
  const int v = query_capacity(dev, kernel, threads);
  // a failed query is not cached (the next call asks again); a full table
  // just means asking the runtime every time
  if (v > 0 && cap_used < kMaxEntries) cap_table[cap_used++] = CapEntry{dev, kernel, threads, v};
  return capped(v);
}

hipError_t launch_coresident(const void* kernel, unsigned grid, int threads, void** args,
                             bool cooperative, hipStream_t s) {
  if (grid < 1 || (int64_t)grid > (int64_t)resident_capacity(kernel, threads))
    return hipErrorInvalidValue;
  if (cooperative)
    return hipLaunchCooperativeKernel(kernel, dim3(grid), dim3((unsigned)threads), args, 0, s);
  hipError_t e = hipLaunchKernel(kernel, dim3(grid), dim3((unsigned)threads), args, 0, s);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace c1g
