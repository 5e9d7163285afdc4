// A user kernel built on the library's exported device calls alone
// (include/tc_device.h), compiled into its own shared library for the GPU
// tests: it is how a kernel outside the library builds a rendezvous on the
// dedicated-row signals of "Barrier: Signals Only" (sections The idea and
// Walkthrough: notify the peers, then wait for their rows).
//
// gather_kernel: one CTA of 256 threads per simulated rank m.  In each
// generation g the CTA writes its 256-word payload into stage[g % 2][m], every
// wave waits for its stores and the CTA syncs, then wave 0 notifies every
// peer (tc_notify, lane q -> rank q) and waits for every row (tc_wait_ge,
// lane s on row s).  The CTA then reads every rank's payload of generation g
// into out[g - first][m][s][*].  Seeing row s at >= g means rank s released
// its payload of generation g before notifying, so every word read must be
// that generation's; the double buffer is safe because no rank can write
// generation g + 2 before every rank has notified in generation g + 1, which
// each does only after its reads of generation g.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tc_device.h"

namespace {

constexpr uint32_t kWords = 256;

__device__ inline int32_t payload(uint32_t g, uint32_t rank, uint32_t t) {
  return (int32_t)((g * 2654435761u) ^ (rank << 24) ^ (t * 40503u));
}

__global__ __launch_bounds__(kWords) void gather_kernel(int32_t* W, uint32_t P, uint32_t first,
                                                        uint32_t n, int32_t* stage, int32_t* out,
                                                        uint32_t max_polls, uint32_t* status) {
  __shared__ uint32_t ok_flag;
  const uint32_t m = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const bool wave0 = __builtin_amdgcn_readfirstlane(t >> 6) == 0;
  for (uint32_t i = 0; i < n; ++i) {
    const uint32_t g = first + i;
    int32_t* buf = stage + (uint64_t)(g & 1) * P * kWords;
    buf[m * kWords + t] = payload(g, m, t);
    __builtin_amdgcn_s_waitcnt(TC_WAITCNT_VMCNT0);  // this wave's stores are done
    __syncthreads();                                // ... and every wave's
    if (wave0) {
      tc_notify(W, P, m, lane);
      const bool ok = tc_wait_ge(W, P, m, lane, (int32_t)g, max_polls);
      if (lane == 0) ok_flag = ok ? 1u : 0u;
    }
    __syncthreads();
    if (tc_uniform(ok_flag) == 0) {
      if (t == 0) atomicCAS(status, 0u, 1u + m);
      return;
    }
    for (uint32_t s = 0; s < P; ++s)
      out[(((uint64_t)i * P + m) * P + s) * kWords + t] = buf[s * kWords + t];
    __syncthreads();
  }
}

}  // namespace

// W: device int32 [P][P], zero before generation 1.  stage: device int32
// [2][P][256].  out: device int32 [n][P][P][256].  status: device u32, set to
// 1 + rank when that rank's wait ran out of polls.
extern "C" int tcu_gather(int32_t* W, uint32_t P, uint32_t first, uint32_t n, int32_t* stage,
                          int32_t* out, uint32_t max_polls, uint32_t* status, void* stream) {
  if (!W || !stage || !out || !status || P < 2 || P > TC_MAX_RANKS || first == 0 || n == 0 ||
      (uint64_t)first + n > (1u << 30))
    return -1;
  hipLaunchKernelGGL(gather_kernel, dim3(P), dim3(kWords), 0, (hipStream_t)stream, W, P, first, n,
                     stage, out, max_polls, status);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
