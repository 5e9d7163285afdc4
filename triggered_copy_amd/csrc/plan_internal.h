// The plan object and its workspace layout (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "internal.h"
#include "tc.h"

namespace tc {

constexpr uint32_t kTicketStride = 32;  // u32 words between hot counters: one 128-byte line each
constexpr uint32_t kStatsWords = 2;     // u64 words of per-launch timestamps

constexpr uint64_t kForceOffset = 128;  // byte offset of the force word in the status block

// The host-visible words of a no-allocation plan, in its workspace's hostio
// segment (other plans keep them in mapped host memory): byte offsets.
constexpr uint64_t kHostioAbort = 0;    // the engine's abort word
constexpr uint64_t kHostioStatus = 64;  // the engine status handed over by the check
constexpr uint64_t kHostioSeq = 128;    // the check's sequence word
constexpr uint64_t kHostioFlags = 256;  // the check's per-chunk flags, G words

constexpr uint32_t kStatusAborted = 1;  // engine stopped by the host's abort word
constexpr uint32_t kStatusExpired = 2;  // engine stopped by its wall-clock backstop

// Per-chunk flags written by the completion check.
constexpr uint32_t kFlagExtra = 1;       // mark count > round * writers
constexpr uint32_t kFlagShortMarks = 2;  // mark count < round * writers (gate not open)
constexpr uint32_t kFlagNotArrived = 8;  // some receiver's arrival < round
constexpr uint32_t kFlagCorrupt = 16;    // values no correct run produces

// Byte offsets into the caller's workspace.
struct Layout {
  uint64_t gates, gate_stride;
  uint64_t pieces, chunks, writers, marks, wprefix;
  uint64_t launch[2], launch_bytes;     // tickets | stats | stop | done, per launch parity
  uint64_t round_blk[2], round_bytes;   // sig | cursors, per round parity
  uint64_t status;
  uint64_t hostio;                      // host-visible words of a no-allocation plan
  uint64_t shares, share_ctr;           // one-shot fill: share table and per-share counters
  uint64_t total;
};

Layout compute_layout(uint32_t P, uint32_t G, uint64_t npieces, uint64_t nwriters);

}  // namespace tc

struct tc_plan {
  uint32_t P = 0, G = 0;
  uint64_t buffer_bytes = 0;
  uint8_t* rep[TC_MAX_RANKS] = {};
  uint8_t* ws = nullptr;
  uint64_t ws_bytes = 0;
  tc::Layout L{};
  std::vector<tc::PieceD> pieces;
  std::vector<tc::ChunkD> chunks;
  std::vector<uint32_t> piece_base, chunk_base;
  uint64_t total_writers = 0;
  uint64_t bytes_read = 0, bytes_moved = 0;
  uint64_t oneshot_blocks = 0;  // one-shot fill grid (0: some chunk is not one byte range)
  uint64_t max_range_share = 0; // longest byte range of one writer of a contiguous chunk

  int device = 0;
  hipStream_t engine_stream = nullptr;
  hipStream_t aux_stream = nullptr;
  hipStream_t producer_stream = nullptr;
  hipEvent_t ev_prod_start = nullptr, ev_prod_end = nullptr;
  hipEvent_t ev_eng_start[2] = {}, ev_eng_done[2] = {};  // alternating timing pairs
  hipEvent_t ev_engine_start = nullptr, ev_engine_done = nullptr;  // the newest launch's pair
  hipEvent_t ev_check_done = nullptr;
  volatile uint32_t* abort_host = nullptr;  // pinned, mapped
  uint32_t* abort_dev = nullptr;
  uint32_t* flags_host = nullptr;           // pinned, mapped: check-kernel output
  uint32_t* flags_dev = nullptr;
  uint32_t* status_host = nullptr;          // pinned, mapped: engine status of the last launch
  uint32_t* status_dev = nullptr;
  volatile uint32_t* seq_host = nullptr;    // pinned, mapped: the last check's sequence number
  uint32_t* seq_dev = nullptr;
  volatile uint32_t* req_host = nullptr;    // pinned, mapped: asks the engine for the check
  uint32_t* req_dev = nullptr;
  volatile uint32_t* exit_host = nullptr;   // pinned, mapped: the engine left without checking
  uint32_t* exit_dev = nullptr;
  uint32_t check_seq = 0;                   // last sequence number handed out
  uint32_t engine_chk_seq = 0;              // the running launch's check number (0: none)
  bool checked_in_engine = false;           // the last wait()'s check ran in the engine
  bool check_queued = false;                // a check kernel was ever queued (ev_check_done)
  bool noalloc = false;                     // workspace = the device's static array
  std::vector<uint32_t> flags_buf;          // no-allocation plan: the check's flags, copied back
  uint32_t status_word = 0;                 // no-allocation plan: the status word, copied back
  uint32_t abort_value = 0;                 // no-allocation plan: source of the abort copy

  uint32_t engine_ctas = 0;
  uint64_t backstop_ticks = 0;
  uint32_t round = 1;
  int state = TC_STATE_READY;
  uint32_t launch_id = 0;    // id of the newest engine launch (abort compares to it)
  uint64_t last_submit = 0;  // process-wide submission number of the newest engine launch
  uint32_t launch_seq = 0;   // launches so far; parity picks the launch block
  uint32_t cur_launch_block = 0;
  uint32_t launches_this_round = 0;
  bool need_relaunch = false;
  bool forced = false;       // close() has forced every gate open
  float last_engine_ms = 0.f;
  bool engine_ms_pending = false;  // last_engine_ms not yet read from the events
  uint32_t pending_pair = 0;        // the pair holding that unread launch
  std::vector<uint32_t> problems;  // (rank, chunk) pairs
};

namespace tc {
void fill_handle(const tc_plan* P, tc_handle* h);
int hip_fail(hipError_t e, const char* what);
int check_device_range(const void* p, uint64_t bytes, int device, const char* what);
}  // namespace tc
