/*
 * tc_device.h -- device view of a triggered plan, for HIP kernels on gfx950.
 *
 * Producer side ([TP] = "Triggered Plans", section Memory ordering): a chunk's
 * data must be in memory before its gate opens.  Every wave waits for its own
 * stores (s_waitcnt vmcnt(0)), the CTA barrier makes that true for every wave,
 * then one thread releases (writing back this XCD's L2) and adds 1 to the
 * chunk's writer count.  The count is striped over TC_MARK_STRIPES words so
 * that hundreds of writer CTAs finishing together do not serialize on one
 * address; the gate of round r is open once the stripes sum to r * writers.
 * Nobody needs to learn that it was the last writer, so the increment does
 * not wait for its result.
 *
 * Consumer side (same section; [TP] The kernel author's contract: every wave
 * of the CTA makes the same arrived/wait calls):
 * arrived/wait read the arrival counter, then acquire at system scope.  One
 * wave reads, the CTA barrier hands the result to every wave, and polling
 * loops count polls instead of reading a clock, so every wave takes the same
 * exit.  All tc_mark_ready / tc_arrived / tc_wait calls are whole-CTA calls:
 * every thread of the CTA must make them, outside divergent branches.
 *
 * Gate rows: rank src's chunk c has global id chunk_base[src] + c; its row in
 * rank q's table is at gates + q * gate_stride + id * 64, and holds the
 * chunk's `arrival` at q.  The mark stripes of global chunk g start at
 * marks + g * TC_MARK_STRIPES * TC_MARK_STRIPE_BYTES.  A rank's own chunk
 * never "arrives" at itself: tc_arrived(dst == src) means its gate is open.
 */
#ifndef TC_DEVICE_H
#define TC_DEVICE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tc.h"

/* s_waitcnt with vmcnt = 0 and expcnt / lgkmcnt left at their maxima (gfx9
 * encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
 * On gfx9 stores are counted by vmcnt, so this waits for the wave's stores,
 * buffer stores included. */
#define TC_WAITCNT_VMCNT0 0x0F70

__device__ inline tc_gate_row* tc_gate_row_ptr(const tc_handle& h, uint32_t table_rank,
                                               uint32_t src, uint32_t chunk) {
  return reinterpret_cast<tc_gate_row*>(h.gates + (uint64_t)table_rank * h.gate_stride +
                                        (uint64_t)(h.chunk_base[src] + chunk) * TC_GATE_ROW_BYTES);
}

__device__ inline bool tc_is_cta_leader() {
  return threadIdx.x == 0 && threadIdx.y == 0 && threadIdx.z == 0;
}

/* Linear thread id in the CTA; threads 0..63 form wave 0. */
__device__ inline uint32_t tc_linear_tid() {
  return threadIdx.x + blockDim.x * (threadIdx.y + blockDim.y * threadIdx.z);
}

/* Lane index within the 64-lane wave. */
__device__ inline uint32_t tc_lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

/* A value read back as a wave-uniform scalar (the first active lane's).
 * Branches on it are scalar branches.  Code in these headers never branches
 * per lane inside a loop that synchronizes: a loop exit or a leader-only
 * block that the compiler must treat as per-lane may be lowered so that one
 * lane leaves the loop while the rest of its wave keeps iterating, which
 * deadlocks against barriers or cross-lane reads.  Leader work is therefore
 * done by a whole wave, with lane-specific values chosen by select, except
 * where a single-lane block holds no loop and ends at a barrier. */
__device__ inline uint32_t tc_uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ inline uint64_t tc_uniform64(uint64_t v) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  return ((uint64_t)hi << 32) | lo;
}

/* Mark stripe s of rank src's chunk c. */
__device__ inline uint64_t* tc_mark_stripe(const tc_handle& h, uint32_t src, uint32_t chunk,
                                           uint32_t s) {
  return reinterpret_cast<uint64_t*>(
      h.marks + ((uint64_t)(h.chunk_base[src] + chunk) * TC_MARK_STRIPES + s) * TC_MARK_STRIPE_BYTES);
}

/* mark_ready(chunk) by one writer CTA of rank `rank`.  Whole CTA.  Every
 * wave waits for its stores, the barrier makes that true for the CTA, then
 * the leader thread releases at agent scope (the L2 write-back that makes
 * the chunk's bytes visible to every XCD) and adds 1 to one of the chunk's
 * mark stripes, chosen by the CTA index, without waiting for the result.
 * Whoever polls the gate sums the stripes.  kWriteBack = false skips the
 * write-back: only for producers whose every store to the chunk was issued
 * write-through at system scope, so that its completion (vmcnt) already
 * made the bytes visible.  The leader block holds no loop and is followed by
 * the closing barrier, so it cannot be merged into a caller's loop back-edge. */
template <bool kWriteBack>
__device__ inline void tc_mark_ready_impl(const tc_handle& h, uint32_t rank, uint32_t chunk) {
  __builtin_amdgcn_s_waitcnt(TC_WAITCNT_VMCNT0);  // wait for this wave's own stores
  __syncthreads();                                // ... and so are every other wave's
  if (tc_is_cta_leader()) {
    uint64_t* stripe = tc_mark_stripe(h, rank, chunk, blockIdx.x % TC_MARK_STRIPES);
    if (kWriteBack) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_fetch_add(stripe, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

__device__ inline void tc_mark_ready(const tc_handle& h, uint32_t rank, uint32_t chunk) {
  tc_mark_ready_impl<true>(h, rank, chunk);
}

/* mark_ready for producers that store the chunk with system-scope
 * write-through stores (cache policy sc0 sc1) only. */
__device__ inline void tc_mark_ready_wt(const tc_handle& h, uint32_t rank, uint32_t chunk) {
  tc_mark_ready_impl<false>(h, rank, chunk);
}

/* The chunk's mark count: the sum of its stripes (relaxed, wave-uniform). */
__device__ inline uint64_t tc_mark_count(const tc_handle& h, uint32_t src, uint32_t chunk) {
  uint64_t sum = 0;
#pragma unroll
  for (uint32_t s = 0; s < TC_MARK_STRIPES; ++s)
    sum += tc_uniform64(__hip_atomic_load(tc_mark_stripe(h, src, chunk, s), __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT));
  return sum;
}

/* One relaxed poll of chunk (src, chunk) as seen by rank dst, wave-uniform:
 * every lane reads the same words.  dst == src: the gate is open (the mark
 * count reached round * writers); otherwise the chunk's arrival at dst
 * reached the round.  The caller acquires after a true result. */
__device__ inline bool tc_poll_once(const tc_handle& h, uint32_t dst, uint32_t src,
                                    uint32_t chunk) {
  if (dst == src) {
    const uint32_t* writers = reinterpret_cast<const uint32_t*>(h.writers);
    const uint64_t w = writers[h.chunk_base[src] + chunk];
    return tc_mark_count(h, src, chunk) >= (uint64_t)h.round * w;
  }
  const tc_gate_row* row = tc_gate_row_ptr(h, dst, src, chunk);
  const uint32_t lo = tc_uniform(
      (uint32_t)__hip_atomic_load(&row->arrival, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM));
  return lo >= h.round;
}

/* arrived(chunk): has rank src's chunk of this round arrived at rank dst?
 * Wave 0 reads the arrival word once; the result reaches every wave through
 * the CTA barrier.  Data read after a true return is this round's. */
__device__ inline bool tc_arrived(const tc_handle& h, uint32_t dst, uint32_t src, uint32_t chunk) {
  __shared__ uint32_t tc_flag;
  if (tc_linear_tid() < 64) {
    const bool ok = tc_poll_once(h, dst, src, chunk);
    if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");  // system-scope acquire
    tc_flag = ok ? 1u : 0u;
  }
  __syncthreads();
  const bool ok = tc_uniform(tc_flag) != 0;
  __syncthreads();
  return ok;
}

/* wait(chunk) with at most max_polls polls (counted, never timed); returns
 * whether the chunk arrived.  Data read after a true return is this round's. */
__device__ inline bool tc_wait(const tc_handle& h, uint32_t dst, uint32_t src, uint32_t chunk,
                               uint32_t max_polls) {
  __shared__ uint32_t tc_flag;
  if (tc_linear_tid() < 64) {
    uint32_t ok = 0;
    for (uint32_t i = 0; i < max_polls; ++i) {
      if (tc_poll_once(h, dst, src, chunk)) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");    // system-scope acquire
    tc_flag = ok;
  }
  __syncthreads();
  const bool ok = tc_uniform(tc_flag) != 0;
  __syncthreads();
  return ok;
}

/* ---------------------------------------------------------------- barrier
 *
 * Dedicated-row signals ([BAR] = "Barrier: Signals Only", sections The idea
 * and Walkthrough).  Every rank owns a signal window of P int32 cells, one
 * row per rank, and cell s of a window is written by rank s alone, so no two
 * ranks ever update the same word.  W holds the P windows stacked: W[q*P + s]
 * is the cell of row s in rank q's window.  The cells only grow ([BAR] Edge
 * cases): generation g of a rendezvous waits for >= g instead of resetting.
 * Every collective lowers to these two calls: notify the peers, then wait
 * for the rows one expects.
 */

/* notify: rank `me` adds 1 to its own row's cell in rank `peer`'s window,
 * W[peer][me] += 1, as a release at system scope: stores this wave made
 * before the call are visible to any thread that sees the new count.  To
 * publish a whole CTA's stores, every wave first waits for its own stores
 * (s_waitcnt vmcnt(0)) and the CTA syncs, as in mark_ready.  Per lane: each
 * calling lane notifies the peer it names, so one wave can notify every peer
 * at once (lane q notifying rank q); a lane naming peer >= P or peer == me
 * does nothing. */
__device__ inline void tc_notify(int32_t* W, uint32_t P, uint32_t me, uint32_t peer) {
  if (peer < P && peer != me)
    __hip_atomic_fetch_add(W + (uint64_t)peer * P + me, 1, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_SYSTEM);
}

/* wait_ge: rank `me` waits until row `src` of its own window holds at least
 * `expected`, W[me][src] >= expected.  Whole wave, wave-uniform result.  Each
 * lane names its own src, so one wave can wait on every row at once (lane s
 * on row s); a lane naming src >= P or src == me waits for nothing.  Polls
 * are relaxed and counted (at most max_polls + 1, never a clock); the wave
 * leaves the loop together on a vote once every lane's cell is high enough,
 * then acquires at system scope, so whatever a notifier released before its
 * notify is visible afterwards.  Returns false when the polls ran out. */
__device__ inline bool tc_wait_ge(const int32_t* W, uint32_t P, uint32_t me, uint32_t src,
                                  int32_t expected, uint32_t max_polls) {
  const bool mine = src < P && src != me;
  const int32_t* cell = W + (uint64_t)me * P + (mine ? src : 0u);
  for (uint32_t polls = 0;; ++polls) {
    bool ok = true;
    if (mine)
      ok = __hip_atomic_load(cell, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) >= expected;
    if (__all(ok)) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");  // system-scope acquire
      return true;
    }
    if (polls >= max_polls) return false;
    __builtin_amdgcn_s_sleep(1);
  }
}

/* The producer's step->tile map: group_m tile-rows walked column by column,
 * then the next band of rows (the grouped order [TP] Model's tile_of stands
 * for).  Plain integer arithmetic, shared by host and device so the schedule
 * and the kernel cannot drift. */
__host__ __device__ inline uint32_t tc_tile_of(uint32_t step, uint32_t tm, uint32_t tn,
                                               uint32_t group_m) {
  const uint32_t width = group_m * tn;
  const uint32_t first_m = (step / width) * group_m;
  const uint32_t left = tm - first_m;
  const uint32_t size_m = left < group_m ? left : group_m;
  const uint32_t in_band = step % width;
  return (first_m + in_band % size_m) * tn + in_band / size_m;
}

#endif /* TC_DEVICE_H */
