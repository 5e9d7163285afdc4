/*
 * A plain C user of the boundary in include/tc.h: device buffers from
 * hipMalloc, a stream from hipStreamCreate, no Python and no PyTorch.
 *
 * Three ranks, each rank's rows of a u32 [3 * 40, 96] buffer as one whole()
 * chunk with two writers ([TP] Model: whole(), writers); the library's
 * hash-fill producer writes and marks each rank's chunk in its own replica;
 * the copy engine delivers it to the other two.  Two rounds ([TP] Gates and
 * rounds: monotonic rounds, no reset).  After each wait() the program checks
 * that
 *   - every replica holds each rank's block exactly as the producer wrote it
 *     into that rank's own replica, and the sentinel everywhere else;
 *   - the second round's blocks differ from the first's (no stale data);
 *   - the gate rows read arrival = round at the peers and 0 in the sender's
 *     own table, where the writer count reads 2 * round.
 * Exit status 0 when all hold; otherwise the first failure is printed.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tc.h"

#define P 3
#define ROWS 40
#define COLS 960
#define SENTINEL 0xA5

#define CHECK_TC(call)                                                              \
  do {                                                                              \
    int rc_ = (call);                                                               \
    if (rc_ != TC_OK) {                                                             \
      fprintf(stderr, "%s returned %d: %s\n", #call, rc_, tc_last_error());         \
      return 1;                                                                     \
    }                                                                               \
  } while (0)
#define CHECK_HIP(call)                                                             \
  do {                                                                              \
    hipError_t e_ = (call);                                                         \
    if (e_ != hipSuccess) {                                                         \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
      return 1;                                                                     \
    }                                                                               \
  } while (0)

int main(void) {
  const uint64_t rank_bytes = (uint64_t)ROWS * COLS * 4;
  const uint64_t B = P * rank_bytes;  /* 46080 bytes, a multiple of 256 */
  void* rep[P];
  uint8_t* host[P];
  uint8_t* prev = (uint8_t*)malloc(B);
  tc_view views[P];
  tc_schedule* sched[P];
  if (!prev) return 1;
  memset(prev, 0, B);
  for (int p = 0; p < P; ++p) {
    CHECK_HIP(hipMalloc(&rep[p], B));
    CHECK_HIP(hipMemset(rep[p], SENTINEL, B));
    host[p] = (uint8_t*)malloc(B);
    if (!host[p]) return 1;
    memset(&views[p], 0, sizeof(views[p]));
    views[p].byte_offset = (uint64_t)p * rank_bytes;
    views[p].rows = ROWS;
    views[p].cols = COLS;
    views[p].row_stride = COLS;
    views[p].elem_bytes = 4;
    CHECK_TC(tc_schedule_whole(&views[p], 2, &sched[p]));
  }
  CHECK_HIP(hipDeviceSynchronize());
  uint64_t ws_bytes = 0;
  CHECK_TC(tc_plan_workspace_bytes(P, (const tc_schedule* const*)sched, 0, &ws_bytes));
  void* ws = NULL;
  CHECK_HIP(hipMalloc(&ws, ws_bytes));

  tc_plan_desc d;
  memset(&d, 0, sizeof(d));
  d.nranks = P;
  d.flags = TC_CHECK_OWN_ROWS;
  d.replicas = rep;
  d.buffer_bytes = B;
  d.schedules = (const tc_schedule* const*)sched;
  d.workspace = ws;
  d.workspace_bytes = ws_bytes;
  d.rows_per_rank_bytes = rank_bytes;
  d.engine_backstop_us = 20u * 1000u * 1000u;
  tc_plan* plan = NULL;
  CHECK_TC(tc_plan_create(&d, &plan));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreateWithFlags(&stream, hipStreamNonBlocking));

  tc_gate_row gates[P * P];  /* P tables x G = P chunks */
  for (uint32_t round = 1; round <= 3; ++round) {
    tc_handle h;
    CHECK_TC(tc_plan_start(plan, stream, &h));
    tc_fill_desc f;
    memset(&f, 0, sizeof(f));
    f.views = views;
    f.seed = 0x7C0FFEEull;
    f.kind = TC_FILL_U32;
    f.mark_mode = TC_MARK_INKERNEL;
    f.mode = round == 1 ? TC_FILL_PARALLEL : TC_FILL_ONESHOT;  /* one CTA per writer, then per 16 KiB */
    CHECK_TC(tc_produce_fill(plan, &h, &f, stream));
    CHECK_TC(tc_plan_wait(plan, 10u * 1000u * 1000u));
    CHECK_HIP(hipDeviceSynchronize());
    for (int q = 0; q < P; ++q) CHECK_HIP(hipMemcpy(host[q], rep[q], B, hipMemcpyDeviceToHost));

    for (int p = 0; p < P; ++p) {
      const uint8_t* own = host[p] + p * rank_bytes;
      for (int q = 0; q < P; ++q) {
        if (memcmp(host[q] + p * rank_bytes, own, rank_bytes) != 0) {
          fprintf(stderr, "round %u: replica %d differs from rank %d's block\n", round, q, p);
          return 1;
        }
      }
      uint64_t same_as_prev = 0, sentinel = 0;
      for (uint64_t i = 0; i < rank_bytes; ++i) {
        same_as_prev += own[i] == prev[p * rank_bytes + i];
        sentinel += own[i] == SENTINEL;
      }
      if (sentinel * 16 > rank_bytes || (round > 1 && same_as_prev * 16 > rank_bytes)) {
        fprintf(stderr, "round %u: rank %d's block looks unwritten or stale\n", round, p);
        return 1;
      }
    }
    memcpy(prev, host[0], B);

    CHECK_TC(tc_plan_read_gates(plan, gates, sizeof(gates)));
    for (int table = 0; table < P; ++table)
      for (int g = 0; g < P; ++g) {  /* chunk g is rank g's only chunk */
        const tc_gate_row* r = &gates[table * P + g];
        const uint64_t want_arrival = table == g ? 0 : round;
        if (r->arrival != want_arrival) {
          fprintf(stderr, "round %u: table %d chunk %d arrival %llu, want %llu\n", round, table, g,
                  (unsigned long long)r->arrival, (unsigned long long)want_arrival);
          return 1;
        }
        if (table == g && (r->writers != 2ull * round || r->ready != round)) {
          fprintf(stderr, "round %u: rank %d's own gate row writers %llu ready %llu\n", round, g,
                  (unsigned long long)r->writers, (unsigned long long)r->ready);
          return 1;
        }
      }
    CHECK_TC(tc_plan_next_round(plan));
  }
  int closing = 0;
  CHECK_TC(tc_plan_close(plan, &closing));
  for (int p = 0; p < P; ++p) {
    tc_schedule_free(sched[p]);
    CHECK_HIP(hipFree(rep[p]));
    free(host[p]);
  }
  CHECK_HIP(hipFree(ws));
  CHECK_HIP(hipStreamDestroy(stream));
  free(prev);
  printf("c_abi round_trip: OK (3 ranks, 3 rounds)\n");
  return 0;
}
