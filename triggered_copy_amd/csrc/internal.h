// Internal declarations shared by the library's translation units.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "tc.h"

struct tc_schedule {
  std::vector<tc_chunk> chunks;
  std::vector<tc_region> regions;
};

namespace tc {

// Records a message for tc_last_error() and returns `code`.
int fail(int code, const std::string& msg);
void clear_error();

// Appends the normal-form, 1 GiB-cut regions of one (offset, rows, row_bytes,
// pitch) window to `out`.
void push_region(uint64_t off, uint64_t rows, uint64_t row_bytes, uint64_t pitch,
                 std::vector<tc_region>& out);

// Plan-creation checks on the host (bounds, own rows, cross-rank overlap,
// writers).  Returns TC_OK or an error code with the message set.
int validate_schedules(uint32_t nranks, const tc_schedule* const* sched, uint64_t buffer_bytes,
                       bool own_rows, uint64_t rows_per_rank_bytes);

// Device-side descriptors uploaded into the workspace at plan creation.
struct PieceD {          // one copy work unit: whole rows of one region
  uint64_t off;          // byte offset of the first row
  uint64_t pitch;        // bytes between rows (== row_bytes when rows == 1)
  uint32_t rows;
  uint32_t row_bytes;
  uint32_t chunk;        // global chunk id
  uint32_t pad;
};
static_assert(sizeof(PieceD) == 32, "piece descriptor is 32 bytes");

struct ChunkD {
  uint32_t rank;
  uint32_t local;        // index in its rank's schedule
  uint32_t first_piece;  // global piece index
  uint32_t npieces;
  uint64_t bytes;        // payload bytes of the chunk
  uint32_t writers;
  uint32_t flags;        // kChunkContiguous
};
static_assert(sizeof(ChunkD) == 32, "chunk descriptor is 32 bytes");

// The chunk's pieces are all one row and each starts where the one before
// ends: the chunk is one contiguous byte range.
constexpr uint32_t kChunkContiguous = 1;

// One-shot fill: a writer's share of a contiguous chunk is written by
// ceil(bytes / kOneShotBlock) one-block CTAs.  Shares are listed every
// rank's chunk 0 first, then chunk 1, ...; `first_block` is the prefix sum of
// the blocks of the shares before (the entry past the last holds the total).
constexpr uint64_t kOneShotBlock = 16384;
struct ShareD {
  uint64_t first_block;
  uint64_t off, bytes;   // the share's byte range in its rank's replica
  uint32_t g, j;         // global chunk, writer index
};
static_assert(sizeof(ShareD) == 32, "ShareD layout");

// Cuts every rank's regions into pieces of about piece_bytes (whole rows for
// 2-D regions; a linear region into piece_bytes ranges).
void build_pieces(uint32_t nranks, const tc_schedule* const* sched, uint64_t piece_bytes,
                  std::vector<PieceD>& pieces, std::vector<ChunkD>& chunks,
                  std::vector<uint32_t>& piece_base, std::vector<uint32_t>& chunk_base);

constexpr uint64_t kDefaultPieceBytes = 8ull << 10;

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

}  // namespace tc
