// Triggered plan runtime and its two kernels: the copy engine and the
// completion check.
//
// [TP] = "Triggered Plans" (Iris documentation), [PR] = "Triggered SDMA
// Plans" (Iris pull request).
//
// The pages' copy engine is a DMA engine fed, per peer, one in-order queue of
// chains: poll the chunk's gate against the round, copy each region, add 1 to
// the peer's arrival counter ([TP] opening diagram; [PR] Design notes).  Here
// the engine is a persistent kernel on the same GPU:
//
//  * Work units ("pieces") are whole rows of one region, about piece_bytes
//    each (8 KiB by default), listed per source rank in schedule order.  Every
//    64-lane wave is an independent worker that claims pieces of a source
//    with an atomic ticket, so consecutive pieces are in flight on different
//    CUs at once and the addresses in flight stay within a narrow window.
//  * A wave reading a chunk for the first time polls its gate: the chunk's
//    mark count (the sum of its stripes) >= round * writers, or the plan's
//    force word set by a close() in mid-round.  Data is read with loads of
//    device-scope coherence (sc1, the policy of a device-scope atomic load),
//    each of which reads the coherent copy, so no cache invalidate is needed
//    after the gate (it would be for ordinary loads).
//  * A piece is read once and written to all P-1 other replicas (fan-out): the
//    P per-peer queues of one source see the same gates, so they advance
//    together and delivering to all of them at once changes no outcome.
//    Stores are system-scope write-through, so once the wave's store counter
//    drains the bytes are visible without an L2 write-back.
//  * Every wave counts its finished piece without waiting for the atomic's
//    result; the wave holding a chunk's last piece waits for the others'
//    counts, then until every earlier chunk of the same source has been
//    signalled (head-of-line order, [TP] The kernel author's contract: a
//    queue delivers a source's chunks in schedule order), then stores the
//    round into `arrival` in every receiver's gate row and advances the
//    queue cursors.
//  * All control flow is wave-uniform; lanes past the end of a piece are
//    masked by the buffer range check.
//
// Every poll loop also watches a device stop word, an abort word in pinned
// host memory and a wall-clock backstop, so every wave of the engine exits
// even when a gate never opens.  A round interrupted that way is resumed by launching the
// engine again: pieces are re-copied (same bytes), chunks already signalled
// are not signalled twice.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include "internal.h"
#include "plan_internal.h"
#include "tc.h"
#include "tc_device.h"

using tc::fail;

namespace tc {

// ------------------------------------------------------------ layout

Layout compute_layout(uint32_t P, uint32_t G, uint64_t npieces, uint64_t nwriters) {
  Layout L{};
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align_up(off + std::max<uint64_t>(bytes, 1), 256);
    return at;
  };
  L.gate_stride = align_up((uint64_t)std::max<uint32_t>(G, 1) * TC_GATE_ROW_BYTES, 256);
  L.gates = take(L.gate_stride * P);
  L.pieces = take(npieces * sizeof(PieceD));
  L.chunks = take((uint64_t)G * sizeof(ChunkD));
  L.writers = take((uint64_t)G * 4);
  L.marks = take((uint64_t)G * TC_MARK_STRIPES * TC_MARK_STRIPE_BYTES);
  L.wprefix = take((uint64_t)(G + 1) * 8);
  // tickets (one line per source) | stats | stop word | done (one line per chunk)
  L.launch_bytes = align_up((uint64_t)P * kTicketStride * 4 + kStatsWords * 8 + 128 +
                                (uint64_t)G * kTicketStride * 4, 256);
  L.launch[0] = take(L.launch_bytes);
  L.launch[1] = take(L.launch_bytes);
  L.round_bytes = align_up((uint64_t)P * kTicketStride * 4 + (uint64_t)P * P * 4, 256);
  L.round_blk[0] = take(L.round_bytes);
  L.round_blk[1] = take(L.round_bytes);
  L.status = take(256);
  L.hostio = take(kHostioFlags + (uint64_t)G * 4);
  L.shares = take((nwriters + 1) * sizeof(ShareD));
  L.share_ctr = take(nwriters * 64);  // one counter per 64-byte line
  L.total = off;
  return L;
}

// ------------------------------------------------------------ kernels

__global__ void zero_words_kernel(uint32_t* p, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kEngineThreads = 256;     // 4 independent waves per CTA
constexpr int kUnroll = 2;              // 16-byte vectors in flight per lane per step
constexpr int kBufWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 family)
// Cache policy of the engine's buffer accesses: loads at device scope (sc1,
// as a device-scope atomic load) read the coherent copy, so no L2
// invalidate is needed after a gate opens; stores at system scope (sc0 sc1)
// are written through, so their completion (vmcnt) already means
// "visible", and no L2 write-back is needed before an arrival is signalled.
constexpr int kLoadPolicy = 16;
constexpr int kStorePolicy = 17;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;  // offset past every buffer: access dropped
constexpr uint32_t kQuickCountGrid = 512;      // engine grids below this many CTAs: see engine_kernel

struct EngineArgs {
  uint64_t rep[TC_MAX_RANKS];
  const PieceD* pieces;
  const ChunkD* chunks;
  uint8_t* gates;
  uint64_t gate_stride;
  const uint8_t* marks;   // mark stripes, TC_MARK_STRIPES per chunk
  uint32_t* tickets;      // this launch: one per source, kTicketStride apart
  uint32_t* done;         // this launch: pieces finished, per chunk, kTicketStride apart
  uint32_t* stats;        // this launch: [0] ~first gate seen, [1] last signal (low 32 bits
                          // of the 100 MHz clock; the window is taken modulo 2^32)
  uint32_t* stop;         // this launch: set once any wave saw the abort or backstop
  uint32_t* all_open;     // this launch: set by the publisher once every gate is open
  uint32_t* zero_launch;  // the other launch block, cleared for the next launch
  uint32_t zero_launch_words;
  uint32_t zero_round_words;
  uint32_t* sig;          // this round: chunks signalled per source, kTicketStride apart
  uint32_t* cur;          // this round: cursor[p*P + q]
  uint32_t* zero_round;   // the other round block, cleared for the next round
  const uint32_t* abort_word;  // pinned host word: launches <= it must stop
  const uint32_t* force;       // device word: nonzero once close() sends chunks as they stand
  uint32_t* status;
  uint32_t piece_base[TC_MAX_RANKS + 1];
  uint32_t round;
  uint32_t nranks;
  uint32_t launch_id;
  uint32_t nchunks;       // G
  uint64_t backstop_ticks;
  // The completion check, run by the publisher once every chunk is
  // signalled and the host has asked for it (chk_seq == 0: not this launch).
  uint32_t chk_seq;             // sequence number of the check this launch may run
  uint32_t pad2;
  const uint32_t* chk_req;      // mapped host word: the host writes chk_seq to ask
  uint32_t* chk_exit;           // mapped host word: launch id, when it left without checking
  uint32_t* chk_flags;          // mapped host memory: one flag word per chunk
  uint32_t* chk_status;         // mapped host word: the engine status handed over
  uint32_t* chk_seq_host;       // mapped host word: chk_seq once the flags are written
  uint32_t chunk_base[TC_MAX_RANKS + 1];
  uint32_t pad3;
};

__device__ inline uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufWord3);
}

// Adds 1 to the word at p, from lane 0 only and without a lane branch: the
// other lanes' offsets fall outside the one-word buffer and are dropped.
// The compiler issues it and moves on.  The same count through the compiler's
// wave-level atomic form (a scan over the lanes inside a masked branch) kept
// the atomic's round trip, about 2.6 us here, on the path of every piece.
__device__ inline void wave_count(uint32_t* p) {
  (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, rsrc(p, 4), tc_lane_id() == 0 ? 0 : (int)kOutOfRange,
                                                       0, 0);
}

// Whole-wave atomic add where only lane 0 contributes `v`; every lane gets
// lane 0's old value.  Device (agent) scope: the engine's own counters are
// only ever read on this GPU.
__device__ inline uint32_t wave_add(uint32_t* p, uint32_t v) {
  const uint32_t mine = tc_lane_id() == 0 ? v : 0u;
  return tc_uniform(__hip_atomic_fetch_add(p, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// The same without waiting for the result.
__device__ inline void wave_add_noret(uint32_t* p, uint32_t v) {
  const uint32_t mine = tc_lane_id() == 0 ? v : 0u;
  __hip_atomic_fetch_add(p, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline uint32_t wave_load(const uint32_t* p) {
  return tc_uniform(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Gates, the abort word and the cursors are shared with the host and with
// other kernels: system scope.
__device__ inline uint32_t wave_load_sys(const uint32_t* p) {
  return tc_uniform(__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM));
}
// 32-bit max (the compiler merges a wave's lanes into one atomic; a 64-bit
// one would be 64 serialized atomics).
__device__ inline void wave_max32(uint32_t* p, uint32_t v) {
  const uint32_t mine = tc_lane_id() == 0 ? v : 0u;
  __hip_atomic_fetch_max(p, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void wave_wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// True when this launch must give up.  Uniform.  Checked every 16 spins:
// the device stop word (cheap) and the backstop clock; every 512 spins (about
// 1.5 ms of waiting) the waiting wave also reads the host's abort word (a
// PCIe read) and, when it is set, raises the stop word for all.
__device__ inline bool must_stop(const EngineArgs& a, uint64_t t0, uint32_t spins) {
  if (spins % 16 != 0) return false;
  if (wave_load(a.stop) != 0) return true;
  uint32_t flag = 0;
  if (now_ticks() - t0 > a.backstop_ticks) flag = kStatusExpired;
  else if (spins % 512 == 0 && wave_load_sys(a.abort_word) >= a.launch_id) flag = kStatusAborted;
  if (flag == 0) return false;
  __hip_atomic_fetch_or(a.status, tc_lane_id() == 0 ? flag : 0u, __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(a.stop, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  return true;
}

// How a waiting wave backs off between polls.  Gate polls by most waves of a
// large grid are "reserve" polls: about 3.4 us between polls once the wave
// has waited a little, so thousands of idle workers put little load on the
// memory system while a producer runs.  (7 and 20 us measured slower on
// 8-rank rounds of whole chunks, 110.5 and 125-128 us p90 against 106.6: a
// chunk waits for the last of its pieces' waves to wake.)  Other gate polls
// ("normal") come 0.4 us apart for the first 16, then about 3.4 us apart: a
// short producer is caught at once, a long one (a GEMM) is not slowed by the
// polling (7 us apart measured the same beside GEMM producers, and 2-rank
// rounds 43 us p90 against 41).  The few waves waiting on another wave of the
// engine (a chunk's last pieces, its turn to signal) poll briskly: they are
// on the round's critical path.  The mode must be a scalar (wave-uniform)
// value: see gate_mode.
constexpr int kPollNormal = 0, kPollReserve = 1, kPollBrisk = 2;

// The pause after the spins-th fruitless poll in a row.
__device__ inline void backoff(int mode, uint32_t spins) {
  if (spins < 8 || mode == kPollBrisk)
    __builtin_amdgcn_s_sleep(1);
  else if (mode == kPollNormal && spins < 16)
    __builtin_amdgcn_s_sleep(16);
  else
    __builtin_amdgcn_s_sleep(127);
}

// Uniform spin until ready() holds.
template <typename Ready>
__device__ inline bool poll_until(const EngineArgs& a, uint64_t t0, int mode, Ready ready) {
  uint32_t spins = 0;
  for (;;) {
    if (ready()) {
      asm volatile("" ::: "memory");  // no later access is moved above the poll
      return true;
    }
    if (must_stop(a, t0, ++spins)) return false;
    backoff(mode, spins);
  }
}

__device__ inline tc_gate_row* gate_row(const EngineArgs& a, uint32_t table, uint32_t g) {
  return reinterpret_cast<tc_gate_row*>(a.gates + (uint64_t)table * a.gate_stride +
                                        (uint64_t)g * TC_GATE_ROW_BYTES);
}

// Signal chunk `c` (global id g) of source p once every earlier chunk of p
// has been signalled, then every following chunk of p that is already
// complete, in order, and only then publish how far p is signalled.  Every
// piece's stores completed (at system scope) before its `done` increment,
// so a chunk whose count has reached its piece count is visible in full.
// A chunk signalled here on its last-piece wave's behalf is seen by that
// wave as already signalled (sig past it), as is one an earlier launch of
// this round signalled.  (Handing each chunk's turn to the next chunk's
// wave instead cost a poll of sig per chunk: 2-rank rounds of four chunks
// per source 38-42 us against 35.)  The engine is the only writer of
// arrival counters and signals each chunk once per round, so the increment
// is a plain store of the round (a store completes in a fraction of the
// time an atomic takes).
__device__ bool signal_in_order(const EngineArgs& a, uint32_t p, uint32_t c, uint32_t g,
                                uint64_t t0) {
  uint32_t* sig = a.sig + p * kTicketStride;
  uint32_t seen = 0;
  if (!poll_until(a, t0, kPollBrisk, [&] { return (seen = wave_load_sys(sig)) >= c; })) return false;
  if (seen > c) return true;
  const uint32_t nc = a.chunk_base[p + 1] - a.chunk_base[p];
  for (;;) {
    for (uint32_t q = 0; q < a.nranks; ++q) {
      if (q == p) continue;
      __hip_atomic_store(&gate_row(a, q, g)->arrival, (uint64_t)a.round, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(a.cur + p * a.nranks + q, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    wave_wait_stores();  // this chunk's arrivals land before the next chunk's
    if (c + 1 >= nc) break;
    const ChunkD next = a.chunks[g + 1];
    if (wave_load(a.done + (uint64_t)(g + 1) * kTicketStride) < next.npieces) break;
    ++c;
    ++g;
  }
  __hip_atomic_store(sig, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  wave_max32(&a.stats[1], (uint32_t)now_ticks());
  return true;
}

// Whole wave: copy `len` bytes at `off` of replica p to every other replica.
// Lanes past the end are masked by the buffer range check, not by branches.
__device__ void copy_linear(const EngineArgs& a, uint32_t p, uint64_t off, uint32_t len) {
  const uint32_t lane = tc_lane_id();
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.rep[p]);
  uint32_t head = (uint32_t)((16 - (off & 15)) & 15);
  if (head > len) head = len;
  const uint32_t body = (len - head) & ~15u;
  const uint32_t tail = len - head - body;
  if (head + tail) {  // unaligned bytes at both ends (at most 30)
    const __amdgpu_buffer_rsrc_t rs = rsrc(src + off, len);
    const uint32_t o = lane < head ? lane : (lane < head + tail ? head + body + (lane - head) : kOutOfRange);
    const uint8_t v = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)o, 0, kLoadPolicy);
    for (uint32_t q = 0; q < a.nranks; ++q)
      if (q != p)
        __builtin_amdgcn_raw_buffer_store_b8(v, rsrc(reinterpret_cast<const uint8_t*>(a.rep[q]) + off, len),
                                             (int)o, 0, kStorePolicy);
  }
  if (body == 0) return;
  const uint64_t start = off + head;
  const __amdgpu_buffer_rsrc_t rs = rsrc(src + start, body);
  const uint32_t nv = body / 16;
  for (uint32_t base = 0; base < nv; base += 64 * kUnroll) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)((base + u * 64 + lane) * 16), 0, kLoadPolicy);
    for (uint32_t q = 0; q < a.nranks; ++q) {
      if (q == p) continue;
      const __amdgpu_buffer_rsrc_t rd = rsrc(reinterpret_cast<const uint8_t*>(a.rep[q]) + start, body);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, (int)((base + u * 64 + lane) * 16), 0,
                                               kStorePolicy);
    }
  }
}

// Whole wave: copy a 2-D piece (rows x row_bytes at pitch; its extent fits in
// 31 bits by construction).
__device__ void copy_2d(const EngineArgs& a, uint32_t p, const PieceD& pc) {
  const uint32_t lane = tc_lane_id();
  const uint32_t extent = (uint32_t)((uint64_t)(pc.rows - 1) * pc.pitch + pc.row_bytes);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.rep[p]) + pc.off;
  const __amdgpu_buffer_rsrc_t rs = rsrc(src, extent);
  auto rd = [&](uint32_t q) {
    return rsrc(reinterpret_cast<const uint8_t*>(a.rep[q]) + pc.off, extent);
  };
  const uint32_t pitch = (uint32_t)pc.pitch;
  if (((pc.off | pc.pitch | pc.row_bytes) & 15) == 0) {
    const uint32_t vpr = pc.row_bytes / 16;
    const uint32_t nv = pc.rows * vpr;
    for (uint32_t base = 0; base < nv; base += 64 * kUnroll) {
      u32x4 v[kUnroll];
      uint32_t at[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t i = base + u * 64 + lane;
        const uint32_t r = i / vpr, c = i - r * vpr;
        at[u] = i < nv ? r * pitch + c * 16 : kOutOfRange;
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)at[u], 0, kLoadPolicy);
      }
      for (uint32_t q = 0; q < a.nranks; ++q) {
        if (q == p) continue;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
          __builtin_amdgcn_raw_buffer_store_b128(v[u], rd(q), (int)at[u], 0, kStorePolicy);
      }
    }
  } else {
    const uint32_t n = pc.rows * pc.row_bytes;
    for (uint32_t base = 0; base < n; base += 64) {
      const uint32_t i = base + lane;
      const uint32_t r = i / pc.row_bytes, c = i - r * pc.row_bytes;
      const uint32_t at = i < n ? r * pitch + c : kOutOfRange;
      const uint8_t v = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)at, 0, kLoadPolicy);
      for (uint32_t q = 0; q < a.nranks; ++q)
        if (q != p) __builtin_amdgcn_raw_buffer_store_b8(v, rd(q), (int)at, 0, kStorePolicy);
    }
  }
}

// What the completion check reads: the workspace's chunk descriptors, gate
// tables and mark stripes, against round `round`.
struct CheckView {
  const ChunkD* chunks;
  const uint8_t* gates;
  uint64_t gate_stride;
  const uint8_t* marks;
  uint32_t nranks, round;
};

__device__ inline uint64_t ld(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// A chunk's counters against what a complete round r leaves ([TP] Gates and
// rounds: this rank's chunk marked by all its writers and arrived at every
// peer).  Every word is loaded before any is judged, and the judging has no
// branch, so that one wait covers all the loads of a lane.

// One gate row (rank q's row of chunk g), as loaded.
struct RowWords {
  uint64_t ready, arrival, other;  // other: writers | rsvd[0..4], all zero
};

__device__ inline RowWords load_row(const CheckView& a, uint32_t g, uint32_t q) {
  const tc_gate_row* r = reinterpret_cast<const tc_gate_row*>(
      a.gates + (uint64_t)q * a.gate_stride + (uint64_t)g * TC_GATE_ROW_BYTES);
  uint64_t w[5];
  for (int k = 0; k < 5; ++k) w[k] = ld(&r->rsvd[k]);
  const uint64_t wr = ld(&r->writers), arr = ld(&r->arrival), rdy = ld(&r->ready);
  return RowWords{rdy, arr, wr | w[0] | w[1] | w[2] | w[3] | w[4]};
}

// Rank q's row is the sender's own when own: no arrival there, and `ready`
// is this round once the gate has opened (it is stored before the chunk is
// signalled anywhere).  Every other row holds an arrival and no `ready`.
__device__ inline uint32_t judge_row(const RowWords& w, bool own, uint32_t round) {
  const uint32_t f_own = ((w.arrival != 0 || w.ready > round) ? kFlagCorrupt : 0u) |
                         (w.ready < round ? kFlagNotArrived : 0u);
  const uint32_t f_peer = ((w.ready != 0 || w.arrival > round) ? kFlagCorrupt : 0u) |
                          (w.arrival < round ? kFlagNotArrived : 0u);
  return (w.other != 0 ? kFlagCorrupt : 0u) | (own ? f_own : f_peer);
}

// The sum of chunk g's mark stripes.
__device__ inline uint64_t load_marks(const CheckView& a, uint32_t g) {
  uint64_t m[TC_MARK_STRIPES];
  for (uint32_t k = 0; k < TC_MARK_STRIPES; ++k)
    m[k] = ld(reinterpret_cast<const uint64_t*>(
        a.marks + ((uint64_t)g * TC_MARK_STRIPES + k) * TC_MARK_STRIPE_BYTES));
  uint64_t sum = 0;
  for (uint32_t k = 0; k < TC_MARK_STRIPES; ++k) sum += m[k];
  return sum;
}

__device__ inline uint32_t judge_marks(uint64_t marks, uint32_t writers, uint32_t round) {
  const uint64_t want = (uint64_t)round * writers;
  return (marks > want ? kFlagExtra : 0u) | (marks < want ? kFlagShortMarks : 0u);
}

// Every flag of chunk g, one lane alone (the check kernel's way).
__device__ uint32_t check_chunk(const CheckView& a, uint32_t g) {
  const ChunkD cd = a.chunks[g];
  uint32_t f = judge_marks(load_marks(a, g), cd.writers, a.round);
  for (uint32_t q = 0; q < a.nranks; ++q) f |= judge_row(load_row(a, g, q), q == cd.rank, a.round);
  return f;
}

struct CheckArgs {
  CheckView v;
  uint32_t* flags;        // mapped pinned host memory, one word per chunk
  uint32_t* status;       // device engine status word: read, reported, cleared
  uint32_t* status_host;  // mapped pinned host memory
  uint32_t* seq_host;     // mapped pinned host memory: `seq` once every flag is written
  uint32_t G, seq;
};

constexpr int kCheckThreads = 1024;
// Plans of up to this many chunks have their completion check run by the
// engine's publisher (one wave, by chunks or by gate rows, see engine_check);
// larger ones by the check kernel.
constexpr uint32_t kEngineCheckMaxChunks = 256;

// The sum of global chunk g's mark stripes, per lane (each lane its own g).
__device__ inline uint64_t lane_mark_count(const EngineArgs& a, uint32_t g) {
  const uint64_t* s = reinterpret_cast<const uint64_t*>(a.marks + (uint64_t)g * TC_MARK_STRIPES *
                                                                       TC_MARK_STRIPE_BYTES);
  uint64_t sum = 0;
#pragma unroll
  for (uint32_t k = 0; k < TC_MARK_STRIPES; ++k)
    sum += __hip_atomic_load(s + k * (TC_MARK_STRIPE_BYTES / 8), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  return sum;
}

// The gate publisher: one wave of the engine stands in for the pages' last
// writer, whose increment returns the count and who then stores the round
// into the gate's `ready` word ([TP] Memory ordering).  Marks here add to
// striped counters without learning the total, so this wave watches every
// chunk's stripes (lane i takes chunks i, i + 64, ...) and stores the round
// into `ready`, in the sender's own gate row, once the count reaches
// round * writers.  It does this for every chunk as its marks complete,
// whatever the copy queues are doing (a chunk held back behind a shut
// earlier chunk still shows its gate open), and leaves once every gate of
// the round is published, or when close() forces the gates open, or when
// the launch must stop.  The copy waves poll the stripes themselves, so
// the publisher is never on a copy's critical path; the engine's exit, and
// so the completion check, come after every `ready` store.
__device__ bool publish_gates(const EngineArgs& a, uint64_t t0) {
  const uint32_t lane = tc_lane_id();
  for (uint32_t spins = 0;;) {
    uint32_t shut = 0;
    for (uint32_t base = 0; base < a.nchunks; base += 64) {
      const uint32_t g = base + lane;
      if (g < a.nchunks) {
        uint64_t* ready = &gate_row(a, a.chunks[g].rank, g)->ready;
        if (__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) < a.round) {
          if (lane_mark_count(a, g) >= (uint64_t)a.round * a.chunks[g].writers)
            __hip_atomic_store(ready, (uint64_t)a.round, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
          else
            shut = 1;
        }
      }
    }
    if (__all(shut == 0)) return true;
    if (wave_load_sys(a.force) != 0) return false;
    if (must_stop(a, t0, ++spins)) return false;
    // Brisk polling: the engine cannot end before the publisher, so its pass
    // interval is on the round's critical path.
    __builtin_amdgcn_s_sleep(2);
  }
}

// The completion check, in the engine (the publisher runs it after its
// gates): once every source's chunks are signalled, and only if the host has
// asked (its producers are done, so their marks are all counted), the same
// flags as the check kernel's, the engine status handed over, then the
// sequence word.  Otherwise -- no request within kRequestPolls polls, or the
// launch must stop -- it reports leaving unchecked through chk_exit, and the
// host runs the check kernel instead.  Whole wave.
constexpr uint32_t kRequestPolls = 48;

__device__ void engine_check(const EngineArgs& a, uint64_t t0) {
  const uint32_t lane = tc_lane_id();
  bool checked = false;
  for (uint32_t spins = 0;;) {  // every chunk signalled
    bool ok = true;
    if (lane < a.nranks)
      ok = __hip_atomic_load(a.sig + lane * kTicketStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) >=
           a.chunk_base[lane + 1] - a.chunk_base[lane];
    if (__all(ok)) break;
    if (must_stop(a, t0, ++spins)) goto leave;
    __builtin_amdgcn_s_sleep(2);
  }
  for (uint32_t polls = 0;; ++polls) {  // the host's request
    if (wave_load_sys(a.chk_req) == a.chk_seq) break;
    if (polls >= kRequestPolls) goto leave;
    __builtin_amdgcn_s_sleep(16);
  }
  {
    // The engine's status word is taken (read and cleared in one atomic, so
    // that no flag set meanwhile is lost) along with the first loads.
    uint32_t st = 0;
    if (lane == 0) st = __hip_atomic_exchange(a.status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    // Two ways to cover the chunks.  One lane per chunk, 64 chunks a pass,
    // waits for P + 1 rounds of loads a pass (the mark stripes, then each
    // receiver's row).  One (chunk, receiver) row per lane, 64 / P chunks a
    // pass, issues all of a lane's loads under one wait, but a pass costs
    // about two such rounds (more loads, the combining shuffles): the wave
    // takes the way with fewer rounds (8 ranks' whole() round: 6.4 us -> 3.1;
    // 40 chunks of 8 ranks: 5.4 us one lane per chunk, 6.9 us by rows).
    const CheckView v{a.chunks, a.gates, a.gate_stride, a.marks, a.nranks, a.round};
    static_assert(TC_MAX_RANKS <= 64, "a pass by rows holds every receiver of a chunk in one wave");
    const uint32_t P = a.nranks, per = 64 / P, nb = 64 / per, B = per * nb;
    const uint32_t row_passes = (a.nchunks + per - 1) / per;
    const uint32_t chunk_rounds = (a.nchunks + 63) / 64 * (P + 1);
    if (2 * row_passes > chunk_rounds) {
      for (uint32_t g = lane; g < a.nchunks; g += 64)
        __hip_atomic_store(a.chk_flags + g, check_chunk(v, g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    } else {
      // By rows: every lane also sums its chunk's mark stripes (the chunk's
      // first lane's sum is used), so no load sits under a lane condition;
      // idle lanes load chunk G-1's words and drop them.  A chunk's lanes
      // are combined in its first lane, and each pass's results move to the
      // lane of their chunk in a batch of up to 64, stored together: the
      // stores go to host memory, and a store per pass would put its round
      // trip in front of the next pass's loads.
      const uint32_t lg = lane / P, q = lane - lg * P;
      for (uint32_t b0 = 0; b0 < a.nchunks; b0 += B) {
        uint32_t acc = 0;
        for (uint32_t k = 0; k < nb && b0 + k * per < a.nchunks; ++k) {
          const uint32_t g = b0 + k * per + lg;
          const bool mine = lg < per && g < a.nchunks;
          const uint32_t gl = mine ? g : a.nchunks - 1;
          const RowWords w = load_row(v, gl, q);
          const uint64_t marks = load_marks(v, gl);
          const ChunkD& cd = a.chunks[gl];
          const uint32_t rank = cd.rank, writers = cd.writers;
          uint32_t f = judge_row(w, q == rank, a.round) | (q == 0 ? judge_marks(marks, writers, a.round) : 0u);
          f = mine ? f : 0u;
          uint32_t all = f;  // valid in each chunk's first lane
          for (uint32_t j = 1; j < P; ++j) all |= (uint32_t)__shfl((int)f, (int)(lane + j));
          const uint32_t t = lane - k * per;  // wraps below this pass's lanes
          const uint32_t got = (uint32_t)__shfl((int)all, (int)(t * P));
          acc = t < per ? got : acc;
        }
        if (lane < B && b0 + lane < a.nchunks)
          __hip_atomic_store(a.chk_flags + b0 + lane, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      }
    }
    if (lane == 0) __hip_atomic_store(a.chk_status, st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    wave_wait_stores();
    if (lane == 0)
      __hip_atomic_store(a.chk_seq_host, a.chk_seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    checked = true;
  }
leave:
  if (!checked && lane == 0)
    __hip_atomic_store(a.chk_exit, a.launch_id, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The copy engine.  Every wave is an independent worker; all control flow is
// wave-uniform (no per-lane branch in any loop), so no lane can be left
// behind in a loop its wave has to leave together.
__global__ __launch_bounds__(kEngineThreads) void engine_kernel(EngineArgs a) {
  const uint32_t gw = tc_uniform((blockIdx.x * kEngineThreads + threadIdx.x) >> 6);

  // Clear the blocks the next launch and the next round will use; nothing
  // touches them while this launch runs.
  for (uint32_t i = blockIdx.x * kEngineThreads + threadIdx.x; i < a.zero_launch_words;
       i += gridDim.x * kEngineThreads)
    a.zero_launch[i] = 0;
  for (uint32_t i = blockIdx.x * kEngineThreads + threadIdx.x; i < a.zero_round_words;
       i += gridDim.x * kEngineThreads)
    a.zero_round[i] = 0;

  const uint64_t t0 = now_ticks();
  // The grid's last wave publishes the gates' `ready` words and copies
  // nothing.  (Measured beside the GEMM producers: a wave of the first CTA
  // that leaves the copy loop, even one that does nothing at all, costs
  // the GEMMs running beside the engine about 25%; the last CTA's costs
  // nothing measurable.)
  if (gw == gridDim.x * (kEngineThreads / 64) - 1) {
    const bool all = publish_gates(a, t0);
    if (all && tc_lane_id() == 0)
      __hip_atomic_store(a.all_open, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    if (a.chk_seq != 0) {
      if (all) engine_check(a, t0);
      else if (tc_lane_id() == 0)
        __hip_atomic_store(a.chk_exit, a.launch_id, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    return;
  }
  uint32_t acquired = 0xFFFFFFFFu;  // last chunk whose gate this wave has seen open
  // Large grids keep one wave in eight polling briskly and let the rest back
  // off; small grids poll with every wave.  The mode is read back as a scalar
  // so that backoff() branches on it: lowered as a per-lane branch with no
  // skip, the reserve sleeps (scalar instructions, which run whatever the
  // lane mask) would be taken in every mode.
  const int gate_mode = (int)tc_uniform(gridDim.x >= 256 && gw % 8 != 0 ? kPollReserve : kPollNormal);
  // Grids under kQuickCountGrid CTAs count pieces with wave_count once the
  // publisher has seen every gate open (checked with each ticket until then).
  // Counted that way from the start, the copies beside 4 GEMM producers ran
  // faster while the producers ran and slowed them by 8-9% (against 6%); at
  // 1024 CTAs it cost the all-gather 0.5 points of HBM peak.  Switched on once
  // every gate is open: GEMM rounds 126 us against 135 at the same slowdown,
  // 2-rank rounds 37-39 us against 42, 8-rank rounds 97 against 99.
  const bool small_grid = gridDim.x < kQuickCountGrid;
  bool quick = false;

  for (uint32_t s = 0; s < a.nranks; ++s) {
    const uint32_t p = (gw + s) % a.nranks;
    const uint32_t np = a.piece_base[p + 1] - a.piece_base[p];
    if (np == 0) continue;
    for (;;) {
      const uint32_t opened = small_grid && !quick ? wave_load(a.all_open) : 0u;
      const uint32_t t = wave_add(a.tickets + p * kTicketStride, 1u);
      if (opened != 0) quick = true;
      if (t >= np) break;
      const PieceD pc = a.pieces[a.piece_base[p] + t];
      const uint32_t g = tc_uniform(pc.chunk);
      if (g != acquired) {
        // The gate of round r is open once the chunk's marks reach r * writers
        // (or once close() forces every gate of the plan open).  Waiting
        // waves read the one `ready` word the publisher stores when it sees
        // the count complete, not the stripes: a poll is then one load (and
        // the force word one poll in 16).  Hundreds of waves polling nine
        // words each at short intervals made the memory channels holding
        // them hot enough to slow GEMM producers running beside the engine
        // by about 30%.
        const uint64_t* ready = &gate_row(a, a.chunks[g].rank, g)->ready;
        uint32_t polls = 0;
        if (!poll_until(a, t0, gate_mode, [&] {
              return tc_uniform64(__hip_atomic_load(ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM)) >=
                         a.round ||
                     (++polls % 16 == 0 && wave_load_sys(a.force) != 0);
            }))
          return;
        // The wave holding a chunk's first piece records when it saw the gate open.
        if (a.piece_base[p] + t == a.chunks[g].first_piece) wave_max32(&a.stats[0], ~(uint32_t)now_ticks());
        acquired = g;
      }
      if (pc.rows == 1)
        copy_linear(a, p, pc.off, pc.row_bytes);
      else
        copy_2d(a, p, pc);
      wave_wait_stores();  // this piece's bytes are visible at system scope
      // Every piece is counted done without waiting for the atomic's result;
      // the wave holding a chunk's last piece then signals the chunk once all
      // of them are counted (a count that reaches npieces means the whole
      // chunk is visible, which lets an earlier chunk's signaller take it).
      const ChunkD cd = a.chunks[g];
      uint32_t* done = a.done + (uint64_t)g * kTicketStride;
      if (quick)
        wave_count(done);
      else
        wave_add_noret(done, 1u);
      if (a.piece_base[p] + t + 1 != cd.first_piece + cd.npieces) continue;
      if (!poll_until(a, t0, kPollBrisk, [&] { return wave_load(done) >= cd.npieces; })) return;
      if (!signal_in_order(a, p, cd.local, g, t0)) return;
    }
  }
}

// One CTA: every chunk's flags into host memory, the engine's status handed
// over (and cleared for the next launch), then the sequence number the host
// waits for.
__global__ __launch_bounds__(kCheckThreads) void check_kernel(CheckArgs a) {
  for (uint32_t g = threadIdx.x; g < a.G; g += kCheckThreads)
    __hip_atomic_store(a.flags + g, check_chunk(a.v, g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  if (threadIdx.x == 0) {
    const uint32_t st = __hip_atomic_exchange(a.status, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __hip_atomic_store(a.status_host, st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }
  // Every wave waits for its own flag stores (written through to host
  // memory) before the barrier: thread 0's release of the sequence word
  // waits only for its own wave's stores, and the barrier does not wait for
  // stores, so without this the host could see the sequence word before
  // another wave's flags.
  wave_wait_stores();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(a.seq_host, a.seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace

// ------------------------------------------------------------ host side

// The workspace of no-allocation plans (tc_plan_create_noalloc): one array
// per device, for the life of the process.  In host code the name stands in
// for the symbol only; its address on a device comes from
// hipGetSymbolAddress, once per device, and kernels get that address.
static __device__ __align__(256) uint8_t scratch[TC_NOALLOC_WORKSPACE_BYTES];

int hip_fail(hipError_t e, const char* what) {
  return fail(TC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define TC_HIP(call)                                   \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return hip_fail(e_, #call);  \
  } while (0)

// Engine streams are shared by every plan on the same device with the same
// CU mask: each one owns a hardware queue (and its wave save area), which
// are too costly to create per plan.  Plans that share a stream run their
// engines in the order they were started.  The registry also lists the live
// plans, so that close() can tell whether a plan's launch is queued behind
// another plan's waiting engine, and tc_release() can destroy the streams
// once no plan is left.  It is never destroyed itself, so nothing of it runs
// in the process's exit-time destructors.
struct NoallocDevice {
  uint8_t* scratch = nullptr;  // this device's copy of `scratch`, from hipGetSymbolAddress
  hipStream_t aux = nullptr;   // side stream shared by the device's no-allocation plans
  bool in_use = false;         // a no-allocation plan is open on the device
};

struct Registry {
  std::mutex mu;
  std::map<std::pair<int, std::vector<uint32_t>>, hipStream_t> streams;
  std::vector<tc_plan*> live;
  uint64_t submits = 0;  // engine launches so far, in submission order
  std::map<int, NoallocDevice> noalloc;
};

static Registry& registry() {
  static Registry* r = new Registry();
  return *r;
}

static int engine_stream_for(int device, const std::vector<uint32_t>& mask, hipStream_t* out) {
  Registry& R = registry();
  std::lock_guard<std::mutex> lock(R.mu);
  auto key = std::make_pair(device, mask);
  auto it = R.streams.find(key);
  if (it != R.streams.end()) {
    *out = it->second;
    return TC_OK;
  }
  hipStream_t s = nullptr;
  const hipError_t e = hipExtStreamCreateWithCUMask(&s, (uint32_t)mask.size(), mask.data());
  if (e != hipSuccess) return hip_fail(e, "hipExtStreamCreateWithCUMask (engine stream)");
  R.streams.emplace(key, s);
  *out = s;
  return TC_OK;
}

static int zero_device(void* p, uint64_t bytes, hipStream_t s) {
  const uint64_t words = bytes / 4;
  if (words == 0) return TC_OK;
  const uint32_t blocks = (uint32_t)std::min<uint64_t>((words + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, words);
  TC_HIP(hipGetLastError());
  return TC_OK;
}

static int launch_engine(tc_plan* P) {
  const Layout& L = P->L;
  EngineArgs a{};
  for (uint32_t p = 0; p < P->P; ++p) a.rep[p] = (uint64_t)P->rep[p];
  a.pieces = reinterpret_cast<const PieceD*>(P->ws + L.pieces);
  a.chunks = reinterpret_cast<const ChunkD*>(P->ws + L.chunks);
  a.gates = P->ws + L.gates;
  a.gate_stride = L.gate_stride;
  a.marks = P->ws + L.marks;
  const uint32_t lb = P->launch_seq & 1u;  // launch block of this launch
  uint8_t* cur_launch = P->ws + L.launch[lb];
  a.tickets = reinterpret_cast<uint32_t*>(cur_launch);
  a.stats = reinterpret_cast<uint32_t*>(cur_launch + (uint64_t)P->P * kTicketStride * 4);
  a.stop = reinterpret_cast<uint32_t*>(cur_launch + (uint64_t)P->P * kTicketStride * 4 + kStatsWords * 8);
  a.all_open = a.stop + 16;  // the stop word's line, 64 bytes in
  a.done = reinterpret_cast<uint32_t*>(cur_launch + (uint64_t)P->P * kTicketStride * 4 + kStatsWords * 8 + 128);
  a.zero_launch = reinterpret_cast<uint32_t*>(P->ws + L.launch[lb ^ 1u]);
  a.zero_launch_words = (uint32_t)(L.launch_bytes / 4);
  const uint32_t rb = P->round & 1u;
  uint8_t* cur_round = P->ws + L.round_blk[rb];
  a.sig = reinterpret_cast<uint32_t*>(cur_round);
  a.cur = reinterpret_cast<uint32_t*>(cur_round + (uint64_t)P->P * kTicketStride * 4);
  a.zero_round = reinterpret_cast<uint32_t*>(P->ws + L.round_blk[rb ^ 1u]);
  a.zero_round_words = (uint32_t)(L.round_bytes / 4);
  a.abort_word = P->abort_dev;
  a.status = reinterpret_cast<uint32_t*>(P->ws + L.status);
  a.force = reinterpret_cast<const uint32_t*>(P->ws + L.status + kForceOffset);
  for (uint32_t p = 0; p <= P->P; ++p) a.piece_base[p] = P->piece_base[p];
  a.round = P->round;
  a.nranks = P->P;
  a.nchunks = P->G;
  a.launch_id = ++P->launch_id;
  for (uint32_t p = 0; p <= P->P; ++p) a.chunk_base[p] = P->chunk_base[p];
  // The completion check rides on this launch (the publisher runs it when
  // wait() asks) unless the plan has no mapped host words, more chunks than
  // a wave checks quickly, or is being closed.
  P->engine_chk_seq = 0;
  if (!P->noalloc && P->G <= kEngineCheckMaxChunks && !P->forced) {
    P->engine_chk_seq = ++P->check_seq;
    a.chk_seq = P->engine_chk_seq;
    a.chk_req = P->req_dev;
    a.chk_exit = P->exit_dev;
    a.chk_flags = P->flags_dev;
    a.chk_status = P->status_dev;
    a.chk_seq_host = P->seq_dev;
  }
  a.backstop_ticks = P->backstop_ticks;
  P->cur_launch_block = lb;
  P->launch_seq++;
  // Timing events alternate between two pairs, so a launch never waits for
  // the previous one (still ending after wait() returned) to read its time:
  // a pair is reused two launches later, and read then if still unread.
  if (P->engine_ms_pending && P->pending_pair == lb) {
    TC_HIP(hipEventSynchronize(P->ev_eng_done[lb]));
    TC_HIP(hipEventElapsedTime(&P->last_engine_ms, P->ev_eng_start[lb], P->ev_eng_done[lb]));
    P->engine_ms_pending = false;
  }
  P->ev_engine_start = P->ev_eng_start[lb];
  P->ev_engine_done = P->ev_eng_done[lb];
  {
    Registry& R = registry();
    std::lock_guard<std::mutex> lock(R.mu);
    // (Events attached to the dispatch itself, hipExtLaunchKernelGGL,
    // measured slower: 2-rank rounds 76 against 62-66 us, and the GEMMs
    // beside the engine 7% against 4% slower.)
    TC_HIP(hipEventRecord(P->ev_engine_start, P->engine_stream));
    hipLaunchKernelGGL(engine_kernel, dim3(P->engine_ctas), dim3(kEngineThreads), 0, P->engine_stream, a);
    P->last_submit = ++R.submits;
  }
  TC_HIP(hipGetLastError());
  TC_HIP(hipEventRecord(P->ev_engine_done, P->engine_stream));
  P->launches_this_round++;
  return TC_OK;
}

// Orders the engine stream after the work queued so far on the producer's
// stream `ps`.  A stream whose work has all completed needs no dependency:
// that skips a barrier packet on the device and 10-15 us of host time in the
// runtime's event calls.
static int order_engine_after(tc_plan* P, hipStream_t ps, hipEvent_t ev) {
  const hipError_t q = hipStreamQuery(ps);
  if (q == hipSuccess) return TC_OK;
  if (q != hipErrorNotReady) return hip_fail(q, "hipStreamQuery(producer stream)");
  TC_HIP(hipEventRecord(ev, ps));
  TC_HIP(hipStreamWaitEvent(P->engine_stream, ev, 0));
  return TC_OK;
}

// Queues the check kernel on the engine stream behind the engine and behind
// the producer's work queued so far; it writes its per-chunk flags and the
// engine status straight into mapped pinned memory.
static int queue_check(tc_plan* P) {
  if (int rc = order_engine_after(P, P->producer_stream, P->ev_prod_end)) return rc;
  CheckArgs c{};
  c.v.chunks = reinterpret_cast<const ChunkD*>(P->ws + P->L.chunks);
  c.v.gates = P->ws + P->L.gates;
  c.v.gate_stride = P->L.gate_stride;
  c.v.marks = P->ws + P->L.marks;
  c.v.nranks = P->P;
  c.v.round = P->round;
  c.flags = P->flags_dev;
  c.status = reinterpret_cast<uint32_t*>(P->ws + P->L.status);
  c.status_host = P->status_dev;
  c.seq_host = P->seq_dev;
  c.G = P->G;
  c.seq = ++P->check_seq;
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kCheckThreads), 0, P->engine_stream, c);
  TC_HIP(hipGetLastError());
  TC_HIP(hipEventRecord(P->ev_check_done, P->engine_stream));  // for close()
  P->check_queued = true;
  return TC_OK;
}

// Spins until `ev` completes or the deadline passes.  1 = done, 0 = deadline.
static int event_done_by(hipEvent_t ev, std::chrono::steady_clock::time_point deadline,
                         hipError_t* err) {
  int spins = 0;
  for (;;) {
    const hipError_t e = hipEventQuery(ev);
    if (e == hipSuccess) return 1;
    if (e != hipErrorNotReady) {
      *err = e;
      return -1;
    }
    if (std::chrono::steady_clock::now() >= deadline) return 0;
    if (++spins > 2000) std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
}

// Spins until the check kernel has published sequence number `seq`, or the
// deadline passes.  1 = done, 0 = deadline, negative = error.  A plan
// without mapped host words (the no-allocation plans) waits for the check's
// event instead and then copies its flags and status word back.
static int check_done_by(tc_plan* P, uint32_t seq, std::chrono::steady_clock::time_point deadline) {
  int spins = 0;
  for (;;) {
    if (P->noalloc) {
      const hipError_t e = hipEventQuery(P->ev_check_done);
      if (e == hipSuccess) {
        const uint8_t* io = P->ws + P->L.hostio;
        TC_HIP(hipMemcpyAsync(&P->status_word, io + kHostioStatus, 4, hipMemcpyDeviceToHost,
                              P->aux_stream));
        if (P->G)
          TC_HIP(hipMemcpyAsync(P->flags_buf.data(), io + kHostioFlags, (size_t)P->G * 4,
                                hipMemcpyDeviceToHost, P->aux_stream));
        TC_HIP(hipStreamSynchronize(P->aux_stream));
        return 1;
      }
      if (e != hipErrorNotReady) return hip_fail(e, "wait: hipEventQuery (completion check)");
    } else if (__atomic_load_n(P->seq_host, __ATOMIC_ACQUIRE) == seq) {
      return 1;
    }
    if (std::chrono::steady_clock::now() >= deadline) return 0;
    if (++spins > 20000) std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
}

// After wait() asked the running engine for the completion check: 1 once
// the check's sequence word is published, 2 once the engine reports that it
// left without checking (the check kernel must run), 0 at the deadline.
static int engine_check_by(const tc_plan* P, std::chrono::steady_clock::time_point deadline) {
  int spins = 0;
  for (;;) {
    if (__atomic_load_n(P->seq_host, __ATOMIC_ACQUIRE) == P->engine_chk_seq) return 1;
    if (__atomic_load_n(P->exit_host, __ATOMIC_ACQUIRE) == P->launch_id) return 2;
    if (std::chrono::steady_clock::now() >= deadline) return 0;
    if (++spins > 20000) std::this_thread::sleep_for(std::chrono::microseconds(20));
  }
}

// Raises the abort word for the plan's newest engine launch: a store to
// pinned host memory, or for a no-allocation plan a copy into its device
// word on the side stream.
static int set_abort(tc_plan* P) {
  if (!P->noalloc) {
    __atomic_store_n(P->abort_host, P->launch_id, __ATOMIC_SEQ_CST);
    return TC_OK;
  }
  P->abort_value = P->launch_id;
  TC_HIP(hipMemcpyAsync(P->abort_dev, &P->abort_value, 4, hipMemcpyHostToDevice, P->aux_stream));
  TC_HIP(hipStreamSynchronize(P->aux_stream));
  return TC_OK;
}

// Whether every gate of plan Q is open in its current round (or forced
// open by close()), from its mark stripes read now.
static int gates_all_open(tc_plan* Q, bool* open) {
  *open = true;
  if (Q->forced || Q->G == 0) return TC_OK;
  std::vector<uint64_t> marks((size_t)Q->G * TC_MARK_STRIPES * (TC_MARK_STRIPE_BYTES / 8));
  TC_HIP(hipMemcpyAsync(marks.data(), Q->ws + Q->L.marks, marks.size() * 8, hipMemcpyDeviceToHost,
                        Q->aux_stream));
  TC_HIP(hipStreamSynchronize(Q->aux_stream));
  for (uint32_t g = 0; g < Q->G; ++g) {
    uint64_t count = 0;
    for (uint32_t k = 0; k < TC_MARK_STRIPES; ++k)
      count += marks[((size_t)g * TC_MARK_STRIPES + k) * (TC_MARK_STRIPE_BYTES / 8)];
    if (count < (uint64_t)Q->round * Q->chunks[g].writers) {
      *open = false;
      return TC_OK;
    }
  }
  return TC_OK;
}

// Whether P's newest engine launch is queued behind an earlier launch on
// the same stream that cannot finish by itself: a plan whose engine has not
// finished and some of whose gates are shut and not forced.  Plans behind
// such a plan are caught too, since their launches are earlier than P's.
static int queued_behind_blocked_plan(tc_plan* P, bool* blocked) {
  *blocked = false;
  Registry& R = registry();
  std::lock_guard<std::mutex> lock(R.mu);
  for (tc_plan* Q : R.live) {
    if (Q == P || Q->engine_stream != P->engine_stream || Q->last_submit == 0 ||
        Q->last_submit > P->last_submit)
      continue;
    const hipError_t e = hipEventQuery(Q->ev_engine_done);
    if (e == hipSuccess) continue;
    if (e != hipErrorNotReady) return hip_fail(e, "close: hipEventQuery (earlier plan)");
    bool open = true;
    if (int rc = gates_all_open(Q, &open)) return rc;
    if (!open) {
      *blocked = true;
      return TC_OK;
    }
  }
  return TC_OK;
}

}  // namespace tc

using namespace tc;

extern "C" {

int tc_plan_workspace_bytes(uint32_t nranks, const tc_schedule* const* schedules,
                            uint64_t piece_bytes, uint64_t* out_bytes) {
  if (!out_bytes || nranks == 0 || nranks > TC_MAX_RANKS)
    return fail(TC_EINVAL, "workspace_bytes: bad rank count or NULL out");
  if (piece_bytes == 0) piece_bytes = kDefaultPieceBytes;
  std::vector<PieceD> pieces;
  std::vector<ChunkD> chunks;
  std::vector<uint32_t> pb, cb;
  build_pieces(nranks, schedules, piece_bytes, pieces, chunks, pb, cb);
  uint64_t nw = 0;
  for (const ChunkD& c : chunks) nw += c.writers;
  *out_bytes = compute_layout(nranks, (uint32_t)chunks.size(), pieces.size(), nw).total;
  return TC_OK;
}

int tc_plan_validate(const tc_plan_desc* d) {
  if (!d) return fail(TC_EINVAL, "desc is NULL");
  if (d->nranks == 0 || d->nranks > TC_MAX_RANKS)
    return fail(TC_EINVAL, "nranks must be in 1.." + std::to_string(TC_MAX_RANKS));
  if (d->buffer_bytes == 0) return fail(TC_EINVAL, "buffer_bytes is 0");
  if ((d->flags & TC_CHECK_OWN_ROWS) && d->rows_per_rank_bytes == 0)
    return fail(TC_EINVAL, "TC_CHECK_OWN_ROWS needs rows_per_rank_bytes");
  if (d->piece_bytes && (d->piece_bytes % 256 || d->piece_bytes > (1ull << 30)))
    return fail(TC_EINVAL, "piece_bytes must be a multiple of 256 and at most 1 GiB");
  uint64_t G = 0;
  for (uint32_t p = 0; p < d->nranks; ++p)
    if (d->schedules && d->schedules[p]) G += d->schedules[p]->chunks.size();
  if (G >= (1ull << 31)) return fail(TC_EINVAL, "too many chunks");
  return validate_schedules(d->nranks, d->schedules, d->buffer_bytes,
                            (d->flags & TC_CHECK_OWN_ROWS) != 0, d->rows_per_rank_bytes);
}

static void destroy(tc_plan* P) {
  if (!P) return;
  {
    Registry& R = registry();
    std::lock_guard<std::mutex> lock(R.mu);
    R.live.erase(std::remove(R.live.begin(), R.live.end(), P), R.live.end());
  }
  for (hipEvent_t e : {P->ev_prod_start, P->ev_prod_end, P->ev_eng_start[0], P->ev_eng_done[0],
                       P->ev_eng_start[1], P->ev_eng_done[1], P->ev_check_done})
    if (e) (void)hipEventDestroy(e);
  if (P->noalloc) {
    // The side stream and the workspace belong to the device, not the plan.
    Registry& R = registry();
    std::lock_guard<std::mutex> lock(R.mu);
    R.noalloc[P->device].in_use = false;
  } else {
    if (P->aux_stream) (void)hipStreamDestroy(P->aux_stream);
    if (P->abort_host) (void)hipHostFree((void*)P->abort_host);
    if (P->flags_host) (void)hipHostFree(P->flags_host);
    if (P->status_host) (void)hipHostFree(P->status_host);
    if (P->seq_host) (void)hipHostFree((void*)P->seq_host);
    if (P->req_host) (void)hipHostFree((void*)P->req_host);
  }
  delete P;
}

extern "C++" {
// TC_OK when [p, p + bytes) lies in one device allocation of `device`;
// otherwise an error naming `what`.  A wrong pointer or size then fails on
// the host rather than as a memory fault in a kernel.
int tc::check_device_range(const void* p, uint64_t bytes, int device, const char* what) {
  hipPointerAttribute_t attr{};
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(TC_EINVAL, std::string(what) + " is not memory the HIP runtime knows");
  }
  if (attr.type != hipMemoryTypeDevice || attr.device != device)
    return fail(TC_EINVAL, std::string(what) + " is not device memory of the current device " +
                               std::to_string(device));
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();
    return fail(TC_EINVAL, std::string(what) + ": allocation range unknown");
  }
  if ((uintptr_t)p + bytes > (uintptr_t)base + size)
    return fail(TC_EBOUNDS, std::string(what) + ": " + std::to_string(bytes) +
                                " bytes run past the end of its allocation");
  return TC_OK;
}
}  // extern "C++"

// Creates a plan over workspace `ws` (ws_bytes).  noalloc_aux != NULL: a
// no-allocation plan, whose workspace is the device's `scratch` array, whose
// side stream is the device's shared one, and whose host-visible words live
// in its workspace instead of mapped host memory.
static int create_plan(const tc_plan_desc* d, uint8_t* ws, uint64_t ws_bytes,
                       hipStream_t noalloc_aux, int noalloc_device, tc_plan** out) {
  if (!out) return fail(TC_EINVAL, "out is NULL");
  *out = nullptr;
  if (int rc = tc_plan_validate(d)) return rc;
  if (!d->replicas || !ws) return fail(TC_EINVAL, "replicas or workspace is NULL");
  for (uint32_t p = 0; p < d->nranks; ++p)
    if (!d->replicas[p] || ((uintptr_t)d->replicas[p] & 255))
      return fail(TC_EINVAL, "replica pointers must be non-NULL and 256-byte aligned");
  if ((uintptr_t)ws & 255) return fail(TC_EINVAL, "workspace must be 256-byte aligned");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0) return fail(TC_ENODEV, "no GPU visible");
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(TC_EHIP, "hipGetDevice failed");
    for (uint32_t p = 0; p < d->nranks; ++p)
      if (int rc = check_device_range(d->replicas[p], d->buffer_bytes, dev,
                                      ("replica " + std::to_string(p)).c_str()))
        return rc;
    if (!noalloc_aux)
      if (int rc = check_device_range(ws, ws_bytes, dev, "workspace")) return rc;
  }

  auto* P = new tc_plan();
  P->P = d->nranks;
  P->buffer_bytes = d->buffer_bytes;
  for (uint32_t p = 0; p < d->nranks; ++p) P->rep[p] = (uint8_t*)d->replicas[p];
  P->ws = ws;
  P->ws_bytes = ws_bytes;
  const uint64_t piece_bytes = d->piece_bytes ? d->piece_bytes : kDefaultPieceBytes;
  build_pieces(P->P, d->schedules, piece_bytes, P->pieces, P->chunks, P->piece_base, P->chunk_base);
  P->G = (uint32_t)P->chunks.size();
  for (const ChunkD& c : P->chunks) P->total_writers += c.writers;
  P->L = compute_layout(P->P, P->G, P->pieces.size(), P->total_writers);
  if (P->L.total > ws_bytes) {
    const uint64_t need = P->L.total;
    delete P;
    return fail(TC_ENOMEM, std::string(noalloc_aux ? "the no-allocation workspace (" +
                                                         std::to_string(ws_bytes) + " bytes)"
                                                   : std::string("workspace")) +
                               " is too small: the plan needs " + std::to_string(need) + " bytes");
  }
  if (noalloc_aux) {
    P->noalloc = true;
    P->device = noalloc_device;
    P->aux_stream = noalloc_aux;
  }
  auto bail = [&](int rc) {
    destroy(P);
    return rc;
  };
  int rc = TC_OK;
#define TC_HIP_C(call)                                       \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) return bail(hip_fail(e_, #call));  \
  } while (0)
  TC_HIP_C(hipGetDevice(&P->device));
  int cus = 0;
  TC_HIP_C(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, P->device));
  // The engine is launched before the producer it waits for, so it must not
  // share a hardware queue with the producer's stream (kernels of streams
  // that share one run in submission order).  A CU-masked stream always gets
  // a queue of its own, so the engine stream is always created with a mask:
  // the caller's, or every CU.
  std::vector<uint32_t> mask;
  if (d->cu_mask && d->cu_mask_words) {
    mask.assign(d->cu_mask, d->cu_mask + d->cu_mask_words);
  } else {
    mask.assign((cus + 31) / 32, 0u);
    for (int i = 0; i < cus; ++i) mask[i / 32] |= 1u << (i % 32);
  }
  uint32_t usable = 0;
  for (uint32_t m : mask) usable += __builtin_popcount(m);
  if (usable == 0) return bail(fail(TC_EINVAL, "cu_mask selects no CU"));
  if ((rc = engine_stream_for(P->device, mask, &P->engine_stream))) return bail(rc);
  if (!P->noalloc) TC_HIP_C(hipStreamCreateWithFlags(&P->aux_stream, hipStreamNonBlocking));
  TC_HIP_C(hipEventCreateWithFlags(&P->ev_prod_start, hipEventDisableTiming));
  TC_HIP_C(hipEventCreateWithFlags(&P->ev_prod_end, hipEventDisableTiming));
  for (int k = 0; k < 2; ++k) {
    TC_HIP_C(hipEventCreate(&P->ev_eng_start[k]));
    TC_HIP_C(hipEventCreate(&P->ev_eng_done[k]));
  }
  P->ev_engine_start = P->ev_eng_start[0];
  P->ev_engine_done = P->ev_eng_done[0];
  TC_HIP_C(hipEventCreateWithFlags(&P->ev_check_done, hipEventDisableTiming));
  if (P->noalloc) {
    // The engine's abort word and the check's outputs live in the
    // workspace; the host copies them over the side stream.
    uint8_t* io = P->ws + P->L.hostio;
    P->abort_dev = reinterpret_cast<uint32_t*>(io + kHostioAbort);
    P->status_dev = reinterpret_cast<uint32_t*>(io + kHostioStatus);
    P->seq_dev = reinterpret_cast<uint32_t*>(io + kHostioSeq);
    P->flags_dev = reinterpret_cast<uint32_t*>(io + kHostioFlags);
    P->flags_buf.assign(std::max<uint32_t>(P->G, 1), 0u);
    P->flags_host = P->flags_buf.data();
    P->status_host = &P->status_word;
  } else {
    void* hp = nullptr;
    TC_HIP_C(hipHostMalloc(&hp, 64, hipHostMallocMapped | hipHostMallocCoherent));
    P->abort_host = (volatile uint32_t*)hp;
    P->abort_host[0] = 0;
    TC_HIP_C(hipHostGetDevicePointer((void**)&P->abort_dev, hp, 0));
    TC_HIP_C(hipHostMalloc((void**)&P->flags_host, (size_t)std::max<uint32_t>(P->G, 1) * 4,
                           hipHostMallocMapped | hipHostMallocCoherent));
    TC_HIP_C(hipHostGetDevicePointer((void**)&P->flags_dev, P->flags_host, 0));
    TC_HIP_C(hipHostMalloc((void**)&P->status_host, 64, hipHostMallocMapped | hipHostMallocCoherent));
    TC_HIP_C(hipHostGetDevicePointer((void**)&P->status_dev, P->status_host, 0));
    TC_HIP_C(hipHostMalloc((void**)&P->seq_host, 64, hipHostMallocMapped | hipHostMallocCoherent));
    *P->seq_host = 0;
    TC_HIP_C(hipHostGetDevicePointer((void**)&P->seq_dev, (void*)P->seq_host, 0));
    // The in-engine check's request word (host writes) and exit note (the
    // engine writes), 64 bytes apart.
    TC_HIP_C(hipHostMalloc((void**)&P->req_host, 128, hipHostMallocMapped | hipHostMallocCoherent));
    P->req_host[0] = 0;
    P->req_host[16] = 0;
    TC_HIP_C(hipHostGetDevicePointer((void**)&P->req_dev, (void*)P->req_host, 0));
    P->exit_host = P->req_host + 16;
    P->exit_dev = P->req_dev + 16;
  }

  // Zero the workspace (gates start at zero, [TP] Gates and rounds; a
  // no-allocation workspace also still holds the previous plan's state),
  // then upload the descriptors once.  Both go over the plan's side stream,
  // which is non-blocking: the shared engine stream, or the legacy stream
  // that waits for it, may hold another plan's engine waiting on its gates.
  if ((rc = zero_device(P->ws, P->L.total, P->aux_stream))) return bail(rc);
  std::vector<uint32_t> writers(P->G);
  std::vector<uint64_t> wprefix(P->G + 1, 0);
  for (uint32_t g = 0; g < P->G; ++g) {
    writers[g] = P->chunks[g].writers;
    wprefix[g + 1] = wprefix[g] + writers[g];
  }
  P->total_writers = wprefix[P->G];
  if (!P->pieces.empty())
    TC_HIP_C(hipMemcpyAsync(P->ws + P->L.pieces, P->pieces.data(), P->pieces.size() * sizeof(PieceD),
                            hipMemcpyHostToDevice, P->aux_stream));
  if (P->G) {
    TC_HIP_C(hipMemcpyAsync(P->ws + P->L.chunks, P->chunks.data(), P->G * sizeof(ChunkD),
                            hipMemcpyHostToDevice, P->aux_stream));
    TC_HIP_C(hipMemcpyAsync(P->ws + P->L.writers, writers.data(), P->G * 4, hipMemcpyHostToDevice,
                            P->aux_stream));
  }
  TC_HIP_C(hipMemcpyAsync(P->ws + P->L.wprefix, wprefix.data(), wprefix.size() * 8,
                          hipMemcpyHostToDevice, P->aux_stream));
  TC_HIP_C(hipStreamSynchronize(P->aux_stream));  // the host arrays above are about to go

  // Longest byte range one writer of a contiguous chunk covers (the parallel
  // fill writes such a share with one write-through span when it fits).
  P->max_range_share = 0;
  for (const ChunkD& c : P->chunks) {
    if (!(c.flags & kChunkContiguous)) continue;
    for (uint32_t j = 0; j < c.writers; ++j) {
      const uint64_t lo = (uint64_t)j * c.npieces / c.writers;
      const uint64_t hi = (uint64_t)(j + 1) * c.npieces / c.writers;
      if (lo == hi) continue;
      const PieceD& a = P->pieces[c.first_piece + lo];
      const PieceD& b = P->pieces[c.first_piece + hi - 1];
      P->max_range_share = std::max(P->max_range_share, b.off + b.row_bytes - a.off);
    }
  }

  // One-shot fill table, when every chunk is one byte range: each writer's
  // share cut into kOneShotBlock blocks, every rank's chunk 0 first, then
  // chunk 1, ... (an empty share still gets one block, which issues its
  // writer's mark).
  bool all_ranges = P->G > 0;
  for (const ChunkD& c : P->chunks)
    if (!(c.flags & kChunkContiguous)) all_ranges = false;
  if (all_ranges) {
    std::vector<ShareD> sh;
    uint32_t maxc = 0;
    for (uint32_t p = 0; p < P->P; ++p) maxc = std::max(maxc, P->chunk_base[p + 1] - P->chunk_base[p]);
    uint64_t blocks = 0;
    for (uint32_t c = 0; c < maxc; ++c)
      for (uint32_t p = 0; p < P->P; ++p) {
        if (c >= P->chunk_base[p + 1] - P->chunk_base[p]) continue;
        const uint32_t g = P->chunk_base[p] + c;
        const ChunkD& cd = P->chunks[g];
        for (uint32_t j = 0; j < cd.writers; ++j) {
          const uint64_t lo = (uint64_t)j * cd.npieces / cd.writers;
          const uint64_t hi = (uint64_t)(j + 1) * cd.npieces / cd.writers;
          ShareD d{};
          d.first_block = blocks;
          d.g = g;
          d.j = j;
          if (lo < hi) {
            const PieceD& a = P->pieces[cd.first_piece + lo];
            const PieceD& b = P->pieces[cd.first_piece + hi - 1];
            d.off = a.off;
            d.bytes = b.off + b.row_bytes - a.off;
          }
          blocks += d.bytes ? (d.bytes + kOneShotBlock - 1) / kOneShotBlock : 1;
          sh.push_back(d);
        }
      }
    ShareD end{};
    end.first_block = blocks;
    sh.push_back(end);
    TC_HIP_C(hipMemcpyAsync(P->ws + P->L.shares, sh.data(), sh.size() * sizeof(ShareD),
                            hipMemcpyHostToDevice, P->aux_stream));
    TC_HIP_C(hipStreamSynchronize(P->aux_stream));
    P->oneshot_blocks = blocks;
  }

  // Default engine size: one worker wave per piece up to 256 (small rounds
  // are latency-bound: every piece in flight at once), otherwise one wave per
  // 150 KiB of delivered bytes per round, at most 16 per usable CU (the count
  // that saturates HBM).  A wave's work is what it writes: each piece it
  // reads goes to all P - 1 receivers.  Fewer waves leave the producer's CUs
  // quieter when a round moves little data; more copy a finished producer's
  // chunks sooner.  (Beside 4 GEMM producers delivering 96 MB a round: one
  // wave per 192 KiB, 122 CTAs, gave 127 us rounds at 3.8-4.0% producer
  // slowdown; per 150 KiB, 157 CTAs, 118-119 us at 4.1-5.6%; per 128 KiB,
  // 183 CTAs, 115.5 us at 4.9-5.2%.)  One more wave is the gate publisher,
  // which copies nothing.
  const uint32_t npieces = (uint32_t)P->pieces.size();
  uint64_t src_bytes = 0;
  for (const ChunkD& c : P->chunks) src_bytes += c.bytes;
  const uint64_t delivered = src_bytes * (P->P - 1);
  if (d->engine_ctas) {
    P->engine_ctas = d->engine_ctas;
  } else {
    const uint64_t waves = std::min<uint64_t>(
        16ull * usable,
        std::max<uint64_t>(std::min<uint64_t>(npieces, 256) + 1, delivered / (150u << 10)));
    P->engine_ctas = (uint32_t)((waves + 3) / 4);
  }
  P->engine_ctas = std::max<uint32_t>(
      1, std::min<uint32_t>(P->engine_ctas, (std::max<uint32_t>(npieces, 1) + 1 + 3) / 4));
  const uint64_t backstop_us = d->engine_backstop_us ? d->engine_backstop_us : 30ull * 1000 * 1000;
  P->backstop_ticks = backstop_us * 100;  // s_memrealtime runs at 100 MHz
  for (const ChunkD& c : P->chunks) {
    P->bytes_read += c.bytes;
    P->bytes_moved += c.bytes * (P->P - 1);
  }
  P->round = 1;
  P->state = TC_STATE_READY;
#undef TC_HIP_C
  {
    Registry& R = registry();
    std::lock_guard<std::mutex> lock(R.mu);
    R.live.push_back(P);
  }
  *out = P;
  return TC_OK;
}

int tc_plan_create(const tc_plan_desc* d, tc_plan** out) {
  if (!d) {
    if (out) *out = nullptr;
    return fail(TC_EINVAL, "desc is NULL");
  }
  return create_plan(d, (uint8_t*)d->workspace, d->workspace_bytes, nullptr, 0, out);
}

int tc_plan_create_noalloc(const tc_plan_desc* d, tc_plan** out) {
  if (!out) return fail(TC_EINVAL, "out is NULL");
  *out = nullptr;
  if (int rc = tc_plan_validate(d)) return rc;
  if (d->workspace || d->workspace_bytes)
    return fail(TC_EINVAL, "create_noalloc: the plan uses the library's own workspace; pass "
                           "workspace = NULL and workspace_bytes = 0");
  uint64_t need = 0;
  if (int rc = tc_plan_workspace_bytes(d->nranks, d->schedules, d->piece_bytes, &need)) return rc;
  if (need > TC_NOALLOC_WORKSPACE_BYTES)
    return fail(TC_ENOMEM, "create_noalloc: the plan needs a " + std::to_string(need) +
                               "-byte workspace; a no-allocation plan has at most " +
                               std::to_string(TC_NOALLOC_WORKSPACE_BYTES) +
                               " (use tc_plan_create with a workspace of its own)");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TC_EHIP, "create_noalloc: hipGetDevice failed");
  Registry& R = registry();
  uint8_t* ws = nullptr;
  hipStream_t aux = nullptr;
  {
    std::lock_guard<std::mutex> lock(R.mu);
    NoallocDevice& nd = R.noalloc[dev];
    if (nd.in_use)
      return fail(TC_ESTATE, "create_noalloc: a no-allocation plan is already open on device " +
                                 std::to_string(dev) + " (they share one workspace)");
    if (!nd.scratch) {
      // Once per device, with the device current: the array's address on
      // this device (the name itself is only a host-side stand-in).
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "create_noalloc: hipGetSymbolAddress(scratch)");
      nd.scratch = (uint8_t*)ptr;
    }
    if (!nd.aux) {
      const hipError_t e = hipStreamCreateWithFlags(&nd.aux, hipStreamNonBlocking);
      if (e != hipSuccess) return hip_fail(e, "create_noalloc: hipStreamCreateWithFlags");
    }
    nd.in_use = true;
    ws = nd.scratch;
    aux = nd.aux;
  }
  const int rc = create_plan(d, ws, TC_NOALLOC_WORKSPACE_BYTES, aux, dev, out);
  if (rc != TC_OK) {
    std::lock_guard<std::mutex> lock(R.mu);
    R.noalloc[dev].in_use = false;
  }
  return rc;
}

int tc_plan_start(tc_plan* P, void* stream, tc_handle* out) {
  if (!P || !out) return fail(TC_EINVAL, "start: NULL argument");
  if (P->state != TC_STATE_READY) return fail(TC_ESTATE, "start() needs a READY plan");
  hipStream_t ps = (hipStream_t)stream;
  if (ps == nullptr || ps == hipStreamLegacy)
    return fail(TC_EINVAL, "start: the legacy default stream waits for every blocking stream, "
                           "the copy engine's included; run the producer on another stream");
  // The copies of this round may overwrite the replicas: order the engine
  // after everything already queued on the producer's stream.
  if (int rc = order_engine_after(P, ps, P->ev_prod_start)) return rc;
  P->producer_stream = ps;
  P->launches_this_round = 0;
  P->need_relaunch = false;
  P->problems.clear();
  if (int rc = launch_engine(P)) return rc;
  P->state = TC_STATE_STARTED;
  fill_handle(P, out);
  return TC_OK;
}

int tc_plan_wait(tc_plan* P, uint64_t timeout_us) {
  if (!P) return fail(TC_EINVAL, "wait: NULL plan");
  if (P->state != TC_STATE_STARTED) return fail(TC_ESTATE, "wait() needs a STARTED plan");
  P->problems.clear();
  if (P->need_relaunch) {  // resume a round a timeout interrupted
    if (int rc = launch_engine(P)) return rc;
    P->need_relaunch = false;
  }
  const auto deadline = std::chrono::steady_clock::now() + std::chrono::microseconds(timeout_us);
  // The check must follow the producer's work too, so that extra marks issued
  // after a gate opened count.  Waiting here, on the host, for the producer's
  // work queued so far to finish lets the check follow the engine alone on
  // its stream; a device-side dependency on the other stream starts it about
  // 4 us later.  Past the deadline the dependency is put on the device after
  // all.  The host watches an event recorded behind that work: queried, it
  // reports completion sooner than a query of the stream (2-rank rounds
  // 42 us median against 51, p90 44 against 60-65).  The queries are spaced
  // 2 us apart: back to back, they slowed the kernels running meanwhile (GEMM
  // producers beside the engine) by about 2%.  After 1 ms the host sleeps 20
  // us between queries instead of spinning, so a long producer does not hold
  // a host core for the whole round.
  bool drained = false;
  {
    TC_HIP(hipEventRecord(P->ev_prod_end, P->producer_stream));
    const auto spin_until = std::chrono::steady_clock::now() + std::chrono::milliseconds(1);
    for (;;) {
      const hipError_t q = hipEventQuery(P->ev_prod_end);
      if (q == hipSuccess) {
        drained = true;
        break;
      }
      if (q != hipErrorNotReady) return hip_fail(q, "hipEventQuery(producer's work)");
      const auto now = std::chrono::steady_clock::now();
      if (now >= deadline) break;
      if (now >= spin_until) {
        std::this_thread::sleep_for(std::chrono::microseconds(20));
        continue;
      }
      const auto next = now + std::chrono::microseconds(2);
      while (std::chrono::steady_clock::now() < next) {
      }
    }
  }
  // The producer's work is done, so every mark it makes is counted: ask the
  // engine's publisher for the check (it runs once every chunk is
  // signalled), and fall back to the check kernel if the engine left
  // without it.  Past the deadline the check kernel, ordered after the
  // producer on the device, is the only way.
  int in_engine = 0;
  if (drained && P->engine_chk_seq && P->launch_id) {
    __atomic_store_n(P->req_host, P->engine_chk_seq, __ATOMIC_SEQ_CST);
    in_engine = engine_check_by(P, deadline);
  }
  P->engine_chk_seq = 0;
  P->checked_in_engine = in_engine == 1;
  bool timed_out = false;
  if (in_engine != 1) {
    if (int rc = queue_check(P)) return rc;
    const uint32_t seq = P->check_seq;
    const int first_check = check_done_by(P, seq, deadline);
    if (first_check < 0) return first_check;
    timed_out = first_check == 0;
  }
  if (timed_out) {
    const uint32_t seq = P->check_seq;
    // Stop this launch of the engine if it still runs (every poll loop
    // watches the abort word), then let the queued check finish.
    if (hipEventQuery(P->ev_engine_done) != hipSuccess)
      if (int rc = set_abort(P)) return rc;
    const auto drain = std::chrono::steady_clock::now() + std::chrono::seconds(10);
    const int finished = check_done_by(P, seq, drain);
    if (finished < 0) return finished;
    if (finished == 0) {
      P->need_relaunch = hipEventQuery(P->ev_engine_done) == hipSuccess;
      return fail(TC_ETIMEOUT, "wait: the copy engine or the producer did not finish within 10 s "
                               "of the deadline");
    }
  }
  P->engine_ms_pending = true;
  P->pending_pair = P->cur_launch_block;
  const uint32_t st = __atomic_load_n(P->status_host, __ATOMIC_ACQUIRE);
  if (st & (kStatusAborted | kStatusExpired)) P->need_relaunch = true;
  bool extra = false, corrupt = false, shortc = false;
  for (uint32_t g = 0; g < P->G; ++g) {
    const uint32_t f = __atomic_load_n(P->flags_host + g, __ATOMIC_ACQUIRE);
    if (f & kFlagExtra) extra = true;
    if (f & kFlagCorrupt) corrupt = true;
    if (f & (kFlagShortMarks | kFlagNotArrived)) shortc = true;
  }
  auto collect = [&](uint32_t mask) {
    for (uint32_t g = 0; g < P->G; ++g)
      if (P->flags_host[g] & mask) {
        P->problems.push_back(P->chunks[g].rank);
        P->problems.push_back(P->chunks[g].local);
      }
  };
  if (extra) {
    collect(kFlagExtra);
    P->state = TC_STATE_FAILED;
    return fail(TC_EEXTRA, "wait: chunks got more marks than their writers this round");
  }
  if (corrupt) {
    collect(kFlagCorrupt);
    P->state = TC_STATE_FAILED;
    return fail(TC_ECORRUPT, "wait: gate rows hold values no correct round produces");
  }
  if (shortc || timed_out || P->need_relaunch) {
    collect(kFlagShortMarks | kFlagNotArrived);
    if (!P->need_relaunch && shortc) P->need_relaunch = true;
    return fail(TC_ETIMEOUT, "wait: timed out with " + std::to_string(P->problems.size() / 2) +
                                 " chunk(s) still short");
  }
  P->state = TC_STATE_DONE;
  return TC_OK;
}

int tc_plan_handle(const tc_plan* P, tc_handle* out) {
  if (!P || !out) return fail(TC_EINVAL, "handle: NULL argument");
  if (P->state != TC_STATE_READY && P->state != TC_STATE_STARTED)
    return fail(TC_ESTATE, "handle: plan is neither READY nor STARTED");
  fill_handle(P, out);
  return TC_OK;
}

int tc_plan_next_round(tc_plan* P) {
  if (!P) return fail(TC_EINVAL, "next_round: NULL plan");
  if (P->state != TC_STATE_DONE) return fail(TC_ESTATE, "next_round() needs a DONE plan");
  if (P->round >= TC_ROUND_LIMIT) return fail(TC_EROUNDS, "round limit 2^32-1 reached");
  P->round++;
  P->state = TC_STATE_READY;
  return TC_OK;
}

int tc_plan_close(tc_plan* P, int* closing) {
  if (closing) *closing = 0;
  if (!P) return TC_OK;
  const auto deadline = [](int s) { return std::chrono::steady_clock::now() + std::chrono::seconds(s); };
  hipError_t err = hipSuccess;
  // Prepared copies are sent as the chunks stand ([TP] The kernel author's
  // contract: closing in the middle of a round, or before it starts): force
  // every gate of the plan open, and run the engine -- for a round prepared
  // but not started, or again when a timeout stopped it.  A DONE or FAILED
  // round has nothing left to send.
  const bool sends = P->state == TC_STATE_STARTED || P->state == TC_STATE_CLOSING ||
                     P->state == TC_STATE_READY;
  if (sends && !P->forced) {
    const uint32_t one = 1;
    TC_HIP(hipMemcpyAsync(P->ws + P->L.status + kForceOffset, &one, 4, hipMemcpyHostToDevice,
                          P->aux_stream));
    TC_HIP(hipStreamSynchronize(P->aux_stream));
    P->forced = true;
    if (P->state == TC_STATE_READY || P->need_relaunch) {
      if (P->state == TC_STATE_READY) {
        P->launches_this_round = 0;
        P->problems.clear();
      }
      if (int rc = launch_engine(P)) return rc;
      P->need_relaunch = false;
    }
  }
  if (P->launch_id) {
    if (closing) {
      // The engine stream may be shared with other plans, so this plan's
      // launch may be queued behind another plan's engine.  As long as that
      // engine can finish by itself (its gates are open, or forced), wait
      // for it; once it is waiting on shut gates, this plan cannot finish
      // first ([TP] The kernel author's contract): it stays CLOSING, and a
      // later close() frees it after the earlier plan is closed.
      const auto until = deadline(10);
      for (;;) {
        const hipError_t e = hipEventQuery(P->ev_engine_done);
        if (e == hipSuccess) break;
        if (e != hipErrorNotReady) return hip_fail(e, "close: hipEventQuery");
        if (hipEventQuery(P->ev_engine_start) != hipSuccess) {
          bool blocked = false;
          if (int rc = queued_behind_blocked_plan(P, &blocked)) return rc;
          if (blocked) {
            P->state = TC_STATE_CLOSING;
            *closing = 1;
            return TC_OK;
          }
        }
        if (std::chrono::steady_clock::now() >= until) break;
        std::this_thread::sleep_for(std::chrono::microseconds(100));
      }
    }
    int done = event_done_by(P->ev_engine_done, deadline(10), &err);
    if (done != 1) {  // the forced engine did not finish: stop it
      if (int rc = set_abort(P)) return rc;
      done = event_done_by(P->ev_engine_done, deadline(10), &err);
    }
    if (done != 1 || (P->check_queued && event_done_by(P->ev_check_done, deadline(10), &err) != 1)) {
      // Leak rather than free memory a kernel may still touch.
      return fail(TC_ETIMEOUT, "close: copy engine did not stop within 10 s");
    }
  }
  destroy(P);
  return TC_OK;
}

int tc_release(void) {
  Registry& R = registry();
  std::lock_guard<std::mutex> lock(R.mu);
  if (!R.live.empty())
    return fail(TC_ESTATE, "release: " + std::to_string(R.live.size()) + " plan(s) still open");
  int rc = TC_OK;
  for (auto& kv : R.streams) {
    const hipError_t e = hipStreamDestroy(kv.second);
    if (e != hipSuccess && rc == TC_OK) rc = hip_fail(e, "release: hipStreamDestroy (engine stream)");
  }
  R.streams.clear();
  for (auto& kv : R.noalloc) {
    if (!kv.second.aux) continue;
    const hipError_t e = hipStreamDestroy(kv.second.aux);
    if (e != hipSuccess && rc == TC_OK) rc = hip_fail(e, "release: hipStreamDestroy (side stream)");
    kv.second.aux = nullptr;
  }
  return rc;
}

int tc_plan_state(const tc_plan* P, int* state, uint32_t* round) {
  if (!P) return fail(TC_EINVAL, "state: NULL plan");
  if (state) *state = P->state;
  if (round) *round = P->round;
  return TC_OK;
}

int tc_plan_problems(const tc_plan* P, uint32_t* rank_chunk, uint32_t cap, uint32_t* n) {
  if (!P) return fail(TC_EINVAL, "problems: NULL plan");
  const uint32_t total = (uint32_t)(P->problems.size() / 2);
  if (n) *n = total;
  if (rank_chunk)
    for (uint32_t i = 0; i < std::min(cap, total); ++i) {
      rank_chunk[2 * i] = P->problems[2 * i];
      rank_chunk[2 * i + 1] = P->problems[2 * i + 1];
    }
  return TC_OK;
}

int tc_plan_read_gates(tc_plan* P, void* host, uint64_t bytes) {
  if (!P || !host) return fail(TC_EINVAL, "read_gates: NULL argument");
  const uint64_t need = (uint64_t)P->P * P->G * TC_GATE_ROW_BYTES;
  if (bytes < need) return fail(TC_EINVAL, "read_gates: need " + std::to_string(need) + " bytes");
  if (P->G == 0) return TC_OK;
  std::vector<uint64_t> marks((size_t)P->G * TC_MARK_STRIPES * (TC_MARK_STRIPE_BYTES / 8));
  for (uint32_t q = 0; q < P->P; ++q)
    TC_HIP(hipMemcpyAsync((uint8_t*)host + (uint64_t)q * P->G * TC_GATE_ROW_BYTES,
                          P->ws + P->L.gates + q * P->L.gate_stride,
                          (size_t)P->G * TC_GATE_ROW_BYTES, hipMemcpyDeviceToHost, P->aux_stream));
  TC_HIP(hipMemcpyAsync(marks.data(), P->ws + P->L.marks, marks.size() * 8, hipMemcpyDeviceToHost,
                        P->aux_stream));
  TC_HIP(hipStreamSynchronize(P->aux_stream));
  // The sender's row: `ready` and `arrival` are the device words as read;
  // the writer counter is kept striped on the device, and its value is the
  // stripes' sum.
  for (uint32_t g = 0; g < P->G; ++g) {
    const ChunkD& cd = P->chunks[g];
    uint64_t count = 0;
    for (uint32_t k = 0; k < TC_MARK_STRIPES; ++k)
      count += marks[((size_t)g * TC_MARK_STRIPES + k) * (TC_MARK_STRIPE_BYTES / 8)];
    auto* row = reinterpret_cast<tc_gate_row*>((uint8_t*)host +
                                               ((uint64_t)cd.rank * P->G + g) * TC_GATE_ROW_BYTES);
    row->writers = count;
  }
  return TC_OK;
}

int tc_plan_row_deps(const tc_plan* P, const tc_view* view, uint32_t tile_rows, uint32_t* start,
                     uint32_t* pairs, uint32_t pairs_cap, uint32_t* nblocks, uint32_t* npairs) {
  if (!P || !view || !nblocks || !npairs) return fail(TC_EINVAL, "row_deps: NULL argument");
  if (tile_rows == 0 || view->rows == 0 || view->cols == 0 || view->elem_bytes == 0 ||
      view->row_stride < view->cols)
    return fail(TC_EINVAL, "row_deps: bad view or tile_rows");
  const uint64_t pitch = view->row_stride * view->elem_bytes;
  const uint64_t base = view->byte_offset, end = base + view->rows * pitch;
  const uint64_t nb = (view->rows + tile_rows - 1) / tile_rows;
  if (nb >= (1ull << 31)) return fail(TC_EINVAL, "row_deps: too many row blocks");
  // Row blocks each chunk's pieces reach into (conservatively: every row
  // between a piece's first and last byte).
  std::vector<std::vector<uint32_t>> blk(nb);
  for (uint32_t g = 0; g < P->G; ++g) {
    const ChunkD& cd = P->chunks[g];
    for (uint32_t k = 0; k < cd.npieces; ++k) {
      const PieceD& pc = P->pieces[cd.first_piece + k];
      const uint64_t a = pc.off, b = pc.off + (pc.rows - 1) * pc.pitch + pc.row_bytes;  // [a, b)
      if (b <= base || a >= end) continue;
      const uint64_t r0 = (std::max(a, base) - base) / pitch;
      const uint64_t r1 = (std::min(b, end) - 1 - base) / pitch;
      for (uint64_t t = r0 / tile_rows; t <= r1 / tile_rows; ++t)
        if (blk[t].empty() || blk[t].back() != g) blk[t].push_back(g);
    }
  }
  uint64_t total = 0;
  for (auto& v : blk) {
    std::sort(v.begin(), v.end());
    v.erase(std::unique(v.begin(), v.end()), v.end());
    total += v.size();
  }
  if (total >= (1ull << 31)) return fail(TC_EINVAL, "row_deps: too many dependencies");
  *nblocks = (uint32_t)nb;
  *npairs = (uint32_t)total;
  if (!start && !pairs) return TC_OK;  // size query
  if (!start || !pairs || pairs_cap < total)
    return fail(TC_EINVAL, "row_deps: start needs nblocks + 1 entries and pairs 2 * npairs");
  uint32_t at = 0;
  for (uint64_t t = 0; t < nb; ++t) {
    start[t] = at;
    for (uint32_t g : blk[t]) {
      pairs[2 * at] = P->chunks[g].rank;
      pairs[2 * at + 1] = P->chunks[g].local;
      ++at;
    }
  }
  start[nb] = at;
  return TC_OK;
}

int tc_plan_read_cursors(tc_plan* P, uint32_t* host) {
  if (!P || !host) return fail(TC_EINVAL, "read_cursors: NULL argument");
  const uint8_t* blk = P->ws + P->L.round_blk[P->round & 1u];
  TC_HIP(hipMemcpyAsync(host, blk + (uint64_t)P->P * kTicketStride * 4, (size_t)P->P * P->P * 4,
                        hipMemcpyDeviceToHost, P->aux_stream));
  TC_HIP(hipStreamSynchronize(P->aux_stream));
  return TC_OK;
}

int tc_plan_stats(tc_plan* P, tc_stats* out) {
  if (!P || !out) return fail(TC_EINVAL, "stats: NULL argument");
  std::memset(out, 0, sizeof(*out));
  if (P->engine_ms_pending) {  // the launch that wait() saw through ends by itself
    const uint32_t pp = P->pending_pair;
    TC_HIP(hipEventSynchronize(P->ev_eng_done[pp]));
    TC_HIP(hipEventElapsedTime(&P->last_engine_ms, P->ev_eng_start[pp], P->ev_eng_done[pp]));
    P->engine_ms_pending = false;
  }
  out->engine_ms = P->last_engine_ms;
  out->launches = P->launches_this_round;
  out->engine_ctas = P->engine_ctas;
  out->bytes_moved = P->bytes_moved;
  out->bytes_read = P->bytes_read;
  out->pieces = P->pieces.size();
  out->G = P->G;
  out->engine_checked = P->checked_in_engine ? 1u : 0u;
  if (P->launch_seq) {
    uint32_t st[2] = {0, 0};
    const uint8_t* blk = P->ws + P->L.launch[P->cur_launch_block];
    TC_HIP(hipMemcpyAsync(st, blk + (uint64_t)P->P * kTicketStride * 4, sizeof(st),
                          hipMemcpyDeviceToHost, P->aux_stream));
    TC_HIP(hipStreamSynchronize(P->aux_stream));
    const uint32_t first = ~st[0];
    if (st[0] && st[1]) out->window_ticks = (uint32_t)(st[1] - first);  // modulo 2^32
  }
  return TC_OK;
}

int tc_plan_engine_stream(tc_plan* P, void** stream) {
  if (!P || !stream) return fail(TC_EINVAL, "engine_stream: NULL argument");
  *stream = (void*)P->engine_stream;
  return TC_OK;
}

int tc_plan_debug_set_round(tc_plan* P, uint32_t round) {
  if (!P) return fail(TC_EINVAL, "debug_set_round: NULL plan");
  if (P->state != TC_STATE_DONE || round == 0)
    return fail(TC_ESTATE, "debug_set_round: plan must be DONE and round >= 1");
  P->round = round;
  return TC_OK;
}

}  // extern "C"

void tc::fill_handle(const tc_plan* P, tc_handle* h) {
  std::memset(h, 0, sizeof(*h));
  h->gates = (uint64_t)(P->ws + P->L.gates);
  h->gate_stride = P->L.gate_stride;
  h->writers = (uint64_t)(P->ws + P->L.writers);
  h->marks = (uint64_t)(P->ws + P->L.marks);
  h->round = P->round;
  h->nranks = P->P;
  for (uint32_t p = 0; p <= P->P; ++p) h->chunk_base[p] = P->chunk_base[p];
  for (uint32_t p = P->P + 1; p <= TC_MAX_RANKS; ++p) h->chunk_base[p] = P->G;
}
