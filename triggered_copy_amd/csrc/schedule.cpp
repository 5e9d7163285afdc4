// Schedule builders and plan-creation checks (host only, no GPU needed).
//
// [TP] = "Triggered Plans" (Iris documentation).  Regions, chunks, writers and
// schedules: section Model.  The 1 GiB cut of linear copies: Model and
// Requirements and limits.  Cross-rank overlap and own rows: Requirements and
// limits, and the all-gather wrapper at the end of Model.
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"
#include "tc.h"
#include "tc_device.h"  // tc_tile_of, shared with the producer kernels

namespace {
thread_local std::string g_error;
}

namespace tc {

int fail(int code, const std::string& msg) {
  g_error = msg;
  return code;
}
void clear_error() { g_error.clear(); }

static void push_linear(uint64_t off, uint64_t n, std::vector<tc_region>& out) {
  for (uint64_t k = 0; k < n; k += TC_LINEAR_MAX_BYTES) {
    const uint64_t len = std::min<uint64_t>(TC_LINEAR_MAX_BYTES, n - k);
    out.push_back(tc_region{off + k, 1, len, len});
  }
}

void push_region(uint64_t off, uint64_t rows, uint64_t row_bytes, uint64_t pitch,
                 std::vector<tc_region>& out) {
  if (rows == 1 || row_bytes == pitch) {  // one row, or rows back to back
    push_linear(off, rows * row_bytes, out);
    return;
  }
  if (row_bytes > TC_LINEAR_MAX_BYTES) {  // each row alone is over the cap
    for (uint64_t i = 0; i < rows; ++i) push_linear(off + i * pitch, row_bytes, out);
    return;
  }
  const uint64_t per = TC_LINEAR_MAX_BYTES / row_bytes;  // whole rows per piece
  for (uint64_t i = 0; i < rows; i += per) {
    const uint64_t n = std::min(per, rows - i);
    if (n == 1)
      push_linear(off + i * pitch, row_bytes, out);
    else
      out.push_back(tc_region{off + i * pitch, n, row_bytes, pitch});
  }
}

}  // namespace tc

using tc::fail;

// One past the last byte of `rows` rows of `row_bytes` at `pitch` from
// `off`, or false when that does not fit in 62 bits (no buffer is that big,
// and no address computed from it can wrap).
static bool extent_end(uint64_t off, uint64_t rows, uint64_t row_bytes, uint64_t pitch,
                       uint64_t* end) {
  uint64_t span = 0, e = 0;
  if (__builtin_mul_overflow(rows - 1, pitch, &span) || __builtin_add_overflow(span, row_bytes, &e) ||
      __builtin_add_overflow(e, off, &e) || e >= (1ull << 62))
    return false;
  *end = e;
  return true;
}

static int check_view(const tc_view* v) {
  if (!v) return fail(TC_EINVAL, "view is NULL");
  if (v->rows == 0 || v->cols == 0 || v->elem_bytes == 0)
    return fail(TC_EINVAL, "view has a zero size");
  if (v->row_stride < v->cols) return fail(TC_EINVAL, "row_stride < cols");
  uint64_t pitch = 0, row_bytes = 0, end = 0;
  if (__builtin_mul_overflow(v->row_stride, (uint64_t)v->elem_bytes, &pitch) ||
      __builtin_mul_overflow(v->cols, (uint64_t)v->elem_bytes, &row_bytes) ||
      !extent_end(v->byte_offset, v->rows, row_bytes, pitch, &end))
    return fail(TC_EINVAL, "view spans more than 2^62 bytes");
  return TC_OK;
}

// Regions of rows [r0, r1) x cols [c0, c1) of the view.
static void window(const tc_view& v, uint64_t r0, uint64_t r1, uint64_t c0, uint64_t c1,
                   std::vector<tc_region>& out) {
  const uint64_t e = v.elem_bytes;
  tc::push_region(v.byte_offset + (r0 * v.row_stride + c0) * e, r1 - r0, (c1 - c0) * e,
                  v.row_stride * e, out);
}

static void add_chunk(tc_schedule* s, size_t first, uint32_t writers) {
  tc_chunk c{};
  c.first_region = (uint32_t)first;
  c.num_regions = (uint32_t)(s->regions.size() - first);
  c.writers = writers;
  s->chunks.push_back(c);
}

extern "C" {

const char* tc_last_error(void) { return g_error.c_str(); }
const char* tc_version(void) { return "triggered_copy_amd 0.1 (gfx950)"; }

int tc_schedule_whole(const tc_view* view, uint32_t writers, tc_schedule** out) {
  if (!out) return fail(TC_EINVAL, "out is NULL");
  *out = nullptr;
  if (int rc = check_view(view)) return rc;
  if (writers == 0) return fail(TC_EINVAL, "writers must be positive");
  auto* s = new tc_schedule;
  window(*view, 0, view->rows, 0, view->cols, s->regions);
  add_chunk(s, 0, writers);
  *out = s;
  return TC_OK;
}

int tc_schedule_chunks(const tc_view* view, uint32_t n, uint32_t writers, tc_schedule** out) {
  if (!out) return fail(TC_EINVAL, "out is NULL");
  *out = nullptr;
  if (int rc = check_view(view)) return rc;
  if (writers == 0) return fail(TC_EINVAL, "writers must be positive");
  if (n == 0 || n > view->rows) return fail(TC_EINVAL, "chunks: need 1 <= n <= rows");
  auto* s = new tc_schedule;
  const uint64_t base = view->rows / n, extra = view->rows % n;
  uint64_t r = 0;
  for (uint32_t k = 0; k < n; ++k) {
    const uint64_t len = base + (k < extra ? 1 : 0);
    const size_t first = s->regions.size();
    window(*view, r, r + len, 0, view->cols, s->regions);
    add_chunk(s, first, writers);
    r += len;
  }
  *out = s;
  return TC_OK;
}

int tc_schedule_tile_chunks(const tc_view* view, uint32_t bm, uint32_t bn,
                            uint32_t tiles_per_chunk, const uint32_t* order,
                            uint32_t order_len, tc_schedule** out) {
  if (!out) return fail(TC_EINVAL, "out is NULL");
  *out = nullptr;
  if (int rc = check_view(view)) return rc;
  if (bm == 0 || bn == 0 || tiles_per_chunk == 0)
    return fail(TC_EINVAL, "tile_chunks: zero tile or chunk size");
  const uint64_t tm = (view->rows + bm - 1) / bm, tn = (view->cols + bn - 1) / bn;
  const uint64_t nt = tm * tn;
  if (nt > 0xFFFFFFFFull) return fail(TC_EINVAL, "tile_chunks: too many tiles");
  if (order) {
    if (order_len != nt) return fail(TC_EINVAL, "tile_chunks: order length != tile count");
    std::vector<uint8_t> seen(nt, 0);
    for (uint64_t i = 0; i < nt; ++i) {
      if (order[i] >= nt || seen[order[i]])
        return fail(TC_EINVAL, "tile_chunks: order is not a permutation of the tiles");
      seen[order[i]] = 1;
    }
  }
  auto* s = new tc_schedule;
  for (uint64_t k = 0; k < nt; k += tiles_per_chunk) {
    const uint64_t end = std::min<uint64_t>(nt, k + tiles_per_chunk);
    const size_t first = s->regions.size();
    for (uint64_t step = k; step < end; ++step) {
      const uint64_t t = order ? order[step] : step;
      const uint64_t mi = t / tn, ni = t % tn;
      window(*view, mi * bm, std::min<uint64_t>(view->rows, (mi + 1) * bm), ni * bn,
             std::min<uint64_t>(view->cols, (ni + 1) * bn), s->regions);
    }
    add_chunk(s, first, (uint32_t)(end - k));
  }
  *out = s;
  return TC_OK;
}

int tc_schedule_from_arrays(const tc_chunk* chunks, uint32_t nchunks, const tc_region* regions,
                            uint32_t nregions, tc_schedule** out) {
  if (!out) return fail(TC_EINVAL, "out is NULL");
  *out = nullptr;
  if ((nchunks && !chunks) || (nregions && !regions))
    return fail(TC_EINVAL, "from_arrays: NULL table");
  uint64_t pos = 0;
  auto* s = new tc_schedule;
  for (uint32_t k = 0; k < nchunks; ++k) {
    const tc_chunk& c = chunks[k];
    if (c.first_region != pos || c.num_regions == 0 || c.writers == 0 ||
        (uint64_t)c.first_region + c.num_regions > nregions) {
      delete s;
      return fail(TC_EINVAL, "from_arrays: chunks must cover the regions back to back, "
                             "each with regions and writers");
    }
    const size_t first = s->regions.size();
    for (uint32_t i = c.first_region; i < c.first_region + c.num_regions; ++i) {
      const tc_region& r = regions[i];
      uint64_t end = 0;
      if (r.rows == 0 || r.row_bytes == 0 || (r.rows > 1 && r.pitch < r.row_bytes)) {
        delete s;
        return fail(TC_EINVAL, "from_arrays: region with zero size or pitch < row_bytes");
      }
      if (!extent_end(r.offset, r.rows, r.row_bytes, r.rows > 1 ? r.pitch : 0, &end)) {
        delete s;
        return fail(TC_EINVAL, "from_arrays: region spans more than 2^62 bytes");
      }
      tc::push_region(r.offset, r.rows, r.row_bytes, r.pitch, s->regions);
    }
    add_chunk(s, first, c.writers);
    pos += c.num_regions;
  }
  if (pos != nregions) {
    delete s;
    return fail(TC_EINVAL, "from_arrays: regions left over");
  }
  *out = s;
  return TC_OK;
}

int tc_schedule_append(tc_schedule* dst, const tc_schedule* src) {
  if (!dst || !src) return fail(TC_EINVAL, "append: NULL schedule");
  const uint32_t shift = (uint32_t)dst->regions.size();
  std::vector<tc_chunk> add = src->chunks;  // copy first: dst may equal src
  std::vector<tc_region> regs = src->regions;
  for (auto& c : add) c.first_region += shift;
  dst->regions.insert(dst->regions.end(), regs.begin(), regs.end());
  dst->chunks.insert(dst->chunks.end(), add.begin(), add.end());
  return TC_OK;
}

int tc_schedule_get(const tc_schedule* s, const tc_chunk** chunks, uint32_t* nchunks,
                    const tc_region** regions, uint32_t* nregions) {
  if (!s) return fail(TC_EINVAL, "get: NULL schedule");
  if (chunks) *chunks = s->chunks.empty() ? nullptr : s->chunks.data();
  if (nchunks) *nchunks = (uint32_t)s->chunks.size();
  if (regions) *regions = s->regions.empty() ? nullptr : s->regions.data();
  if (nregions) *nregions = (uint32_t)s->regions.size();
  return TC_OK;
}

void tc_schedule_free(tc_schedule* s) { delete s; }

int tc_order_grouped(uint32_t tm, uint32_t tn, uint32_t group_m, uint32_t* out) {
  if (!out || tm == 0 || tn == 0 || group_m == 0)
    return fail(TC_EINVAL, "order_grouped: zero size or NULL out");
  const uint64_t nt = (uint64_t)tm * tn;
  for (uint64_t s = 0; s < nt; ++s) out[s] = tc_tile_of((uint32_t)s, tm, tn, group_m);
  return TC_OK;
}

}  // extern "C"

// ------------------------------------------------------------ validation

namespace {
struct Interval {
  uint64_t lo, hi;  // [lo, hi)
  uint32_t rank;
};
}  // namespace

int tc::validate_schedules(uint32_t nranks, const tc_schedule* const* sched,
                           uint64_t buffer_bytes, bool own_rows, uint64_t rows_per_rank_bytes) {
  std::vector<Interval> iv;
  for (uint32_t p = 0; p < nranks; ++p) {
    const tc_schedule* s = sched ? sched[p] : nullptr;
    if (!s) continue;
    for (size_t k = 0; k < s->chunks.size(); ++k) {
      const tc_chunk& c = s->chunks[k];
      if (c.writers == 0 || c.num_regions == 0)
        return fail(TC_EINVAL, "rank " + std::to_string(p) + " chunk " + std::to_string(k) +
                                   ": no writers or no regions");
      if ((uint64_t)c.first_region + c.num_regions > s->regions.size())
        return fail(TC_EINVAL, "chunk table points past the region table");
      for (uint32_t i = c.first_region; i < c.first_region + c.num_regions; ++i) {
        const tc_region& r = s->regions[i];
        if (r.rows == 0 || r.row_bytes == 0 || (r.rows > 1 && r.pitch < r.row_bytes))
          return fail(TC_EINVAL, "rank " + std::to_string(p) + ": malformed region");
        const uint64_t end = r.offset + (r.rows - 1) * r.pitch + r.row_bytes;
        if (end > buffer_bytes || end < r.offset)
          return fail(TC_EBOUNDS, "rank " + std::to_string(p) + " chunk " + std::to_string(k) +
                                      ": region ends past the buffer");
        if (own_rows) {
          const uint64_t lo = (uint64_t)p * rows_per_rank_bytes, hi = lo + rows_per_rank_bytes;
          if (r.offset < lo || end > hi)
            return fail(TC_EBOUNDS, "rank " + std::to_string(p) + " chunk " + std::to_string(k) +
                                        ": region outside the rank's own rows");
        }
        for (uint64_t row = 0; row < r.rows; ++row) {
          const uint64_t a = r.offset + row * r.pitch;
          iv.push_back(Interval{a, a + r.row_bytes, p});
        }
      }
    }
  }
  // Sweep by start.  `best` holds the largest end seen so far and its rank;
  // `second` the largest end among the other ranks.  A new interval of rank
  // r overlaps an earlier one of another rank iff it starts before the
  // largest end among ranks != r.
  std::sort(iv.begin(), iv.end(), [](const Interval& a, const Interval& b) { return a.lo < b.lo; });
  uint64_t best_end = 0, second_end = 0;
  uint32_t best_rank = UINT32_MAX;
  for (const Interval& x : iv) {
    const uint64_t other_end = (x.rank == best_rank) ? second_end : best_end;
    if (x.lo < other_end) {
      return fail(TC_EOVERLAP, "ranks " + std::to_string(x.rank) + " and another rank send the "
                               "same bytes at offset " + std::to_string(x.lo));
    }
    if (x.rank == best_rank) {
      best_end = std::max(best_end, x.hi);
    } else if (x.hi > best_end) {
      second_end = best_end;
      best_end = x.hi;
      best_rank = x.rank;
    } else {
      second_end = std::max(second_end, x.hi);
    }
  }
  return TC_OK;
}

void tc::build_pieces(uint32_t nranks, const tc_schedule* const* sched, uint64_t piece_bytes,
                      std::vector<PieceD>& pieces, std::vector<ChunkD>& chunks,
                      std::vector<uint32_t>& piece_base, std::vector<uint32_t>& chunk_base) {
  pieces.clear();
  chunks.clear();
  piece_base.assign(nranks + 1, 0);
  chunk_base.assign(nranks + 1, 0);
  for (uint32_t p = 0; p < nranks; ++p) {
    piece_base[p] = (uint32_t)pieces.size();
    chunk_base[p] = (uint32_t)chunks.size();
    const tc_schedule* s = sched ? sched[p] : nullptr;
    if (!s) continue;
    for (size_t k = 0; k < s->chunks.size(); ++k) {
      const tc_chunk& c = s->chunks[k];
      const uint32_t g = (uint32_t)chunks.size();
      ChunkD cd{};
      cd.rank = p;
      cd.local = (uint32_t)k;
      cd.first_piece = (uint32_t)pieces.size();
      cd.writers = c.writers;
      for (uint32_t i = c.first_region; i < c.first_region + c.num_regions; ++i) {
        const tc_region& r = s->regions[i];
        cd.bytes += r.rows * r.row_bytes;
        auto linear = [&](uint64_t off, uint64_t n) {
          for (uint64_t a = 0; a < n; a += piece_bytes) {
            const uint64_t len = std::min(piece_bytes, n - a);
            pieces.push_back(PieceD{off + a, len, 1, (uint32_t)len, g, 0});
          }
        };
        if (r.rows == 1) {
          linear(r.offset, r.row_bytes);
        } else if (r.row_bytes >= piece_bytes) {
          for (uint64_t row = 0; row < r.rows; ++row) linear(r.offset + row * r.pitch, r.row_bytes);
        } else {
          // Whole rows per piece; the piece's extent stays below 2^31 bytes
          // (the engine addresses a piece with 32-bit buffer offsets).
          const uint64_t by_extent = ((1ull << 31) - 1 - r.row_bytes) / r.pitch + 1;
          const uint64_t per = std::max<uint64_t>(1, std::min(piece_bytes / r.row_bytes, by_extent));
          for (uint64_t row = 0; row < r.rows; row += per) {
            const uint64_t n = std::min(per, r.rows - row);
            pieces.push_back(PieceD{r.offset + row * r.pitch, r.pitch, (uint32_t)n,
                                    (uint32_t)r.row_bytes, g, 0});
          }
        }
      }
      cd.npieces = (uint32_t)pieces.size() - cd.first_piece;
      bool contiguous = cd.npieces > 0;
      for (uint32_t i = cd.first_piece; i < cd.first_piece + cd.npieces && contiguous; ++i)
        contiguous = pieces[i].rows == 1 &&
                     (i == cd.first_piece ||
                      pieces[i].off == pieces[i - 1].off + pieces[i - 1].row_bytes);
      if (contiguous) cd.flags |= kChunkContiguous;
      chunks.push_back(cd);
    }
  }
  piece_base[nranks] = (uint32_t)pieces.size();
  chunk_base[nranks] = (uint32_t)chunks.size();
}
