// Dedicated-row notify/wait barrier on one GPU.
//
// [BAR] = "Barrier: Signals Only" (pypto documentation).  Section The idea:
// a rank adds 1 to its own row's cell in every other rank's signal window,
// then waits until every other row of its own window reaches the threshold;
// each cell has exactly one writer, so the barrier costs P-1 notifies and P-1
// waits per rank and moves no data.  Section Edge cases: the cells are
// monotonic, so generation g waits for >= g instead of resetting.
//
// The P windows are stacked as W[P][P] int32; W[q][s] is the cell of row s in
// rank q's window, written only by rank s.  One 64-lane wave per simulated
// rank, built on the device calls of tc_device.h: lane q notifies rank q
// (tc_notify, a release add), and the wave waits with lane s on row s
// (tc_wait_ge: relaxed polls, a wave vote so the whole wave leaves the loop
// together, then one acquire).  Polls are counted and bounded, so every wave
// exits even if a peer never arrives.
#include <hip/hip_runtime.h>

#include "internal.h"
#include "plan_internal.h"
#include "tc.h"
#include "tc_device.h"

using tc::fail;

namespace {

struct BarrierArgs {
  int32_t* W;
  int32_t* x;
  int32_t* y;
  int32_t* snap;
  uint32_t* status;
  uint32_t P, first_gen, n_gen, max_polls;
};

__global__ __launch_bounds__(64) void barrier_kernel(BarrierArgs a) {
  const uint32_t m = blockIdx.x;
  const uint32_t lane = threadIdx.x;
  const uint32_t P = a.P;
  for (uint32_t i = 0; i < a.n_gen; ++i) {
    const uint32_t g = a.first_gen + i;
    if (a.x && lane == 0) a.x[(g & 1) * P + m] = (int32_t)((g << 8) | m);  // stage
    __syncthreads();
    tc_notify(a.W, P, m, lane);  // lane q notifies rank q
    if (!tc_wait_ge(a.W, P, m, lane, (int32_t)g, a.max_polls)) {  // lane s waits on row s
      if (lane == 0) {
        uint32_t expected = 0;
        __hip_atomic_compare_exchange_strong(a.status, &expected, 1 + m, __ATOMIC_RELAXED,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
      return;
    }
    if (a.snap && lane < P)
      a.snap[((uint64_t)i * P + m) * P + lane] =
          __hip_atomic_load(a.W + m * P + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (a.y && lane == 0)
      a.y[(uint64_t)i * P + m] = __hip_atomic_load(a.x + (g & 1) * P + (m + 1) % P,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
}

}  // namespace

extern "C" int tc_barrier_run(int32_t* W, uint32_t P, uint32_t first_gen, uint32_t n_gen,
                              int32_t* x, int32_t* y, int32_t* snap, uint32_t max_polls,
                              uint32_t* status, void* stream) {
  if (!W || !status) return fail(TC_EINVAL, "barrier: NULL W or status");
  if (P < 2 || P > TC_MAX_RANKS) return fail(TC_EINVAL, "barrier: P must be in 2..16");
  if (first_gen == 0) return fail(TC_EINVAL, "barrier: generations start at 1");
  if ((uint64_t)first_gen + n_gen > (1u << 23)) return fail(TC_EINVAL, "barrier: generation overflow");
  if (n_gen == 0) return TC_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TC_EHIP, "barrier: hipGetDevice failed");
  const uint64_t pp = (uint64_t)P * P * 4;
  if (int rc = tc::check_device_range(W, pp, dev, "barrier: W")) return rc;
  if (int rc = tc::check_device_range(status, 4, dev, "barrier: status")) return rc;
  if (x)
    if (int rc = tc::check_device_range(x, 2ull * P * 4, dev, "barrier: x")) return rc;
  if (y)
    if (int rc = tc::check_device_range(y, (uint64_t)n_gen * P * 4, dev, "barrier: y")) return rc;
  if (snap)
    if (int rc = tc::check_device_range(snap, (uint64_t)n_gen * pp, dev, "barrier: snap")) return rc;
  BarrierArgs a{W, x, y, snap, status, P, first_gen, n_gen, max_polls};
  hipLaunchKernelGGL(barrier_kernel, dim3(P), dim3(64), 0, (hipStream_t)stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return tc::hip_fail(e, "barrier launch");
  return TC_OK;
}
