// Synthetic producers and the device-view consumer of a plan.
//
// [TP] = "Triggered Plans" (Iris documentation).  Producers write their part
// of the output and mark each chunk ready once per writer (section Model;
// The kernel author's contract: one mark per writer per round); mark_ready is the device function of
// section Memory ordering.  The consumer reads a chunk only after
// arrived/wait (section Memory ordering, consumer side).
//
// Values: element i of rank p's view in round r holds
//   h = mix64((p << 48) | (r << 32) | i) ^ mix64(seed)),
// mix64 being SplitMix64's output function (Steele, Lea & Flood, OOPSLA 2014);
// u32 = low 32 bits, u8 = low 8 bits, bf16 = high half of the fp32 value
// ((h >> 41) - 2^22) * 2^-22, which lies in [-1, 1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "internal.h"
#include "plan_internal.h"
#include "tc.h"
#include "tc_device.h"

using tc::fail;

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kFillThreads = 256;
// One-shot blocks: 16 KiB each, 128 threads (8 vectors a thread): 5.62-5.65 ms per
// all-gather step against 5.67-5.68 with 256 threads, 6.17-6.20 with 512.
constexpr int kOneShotThreads = 128;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct FillArgs {
  uint64_t rep[TC_MAX_RANKS];
  uint64_t view_off[TC_MAX_RANKS];     // byte offset of rank p's view
  uint64_t view_pitch[TC_MAX_RANKS];   // bytes per view row (row_stride * elem)
  uint64_t view_cols[TC_MAX_RANKS];
  const tc::PieceD* pieces;
  const tc::ChunkD* chunks;
  const uint64_t* wprefix;             // G + 1 prefix sums of writers
  const uint32_t* order;               // serial mode: [P][order_stride], or NULL
  tc_handle h;
  uint64_t seed_mix;
  uint32_t contiguous;                 // bit p: view p has row_stride == cols
  uint32_t kind, mark, elem;
  uint32_t order_stride, G, max_chunks, pad1;
  const tc::ShareD* shares;            // one-shot mode: nshares + 1 entries
  uint64_t* share_ctr;                 // one-shot mode: blocks done per share (8 per 64 B)
  uint64_t nshares;
};

// mix64(k ^ mix64(seed)) for k = (p << 48) | (round << 32) | idx, idx < 2^32.
// The high word of the key is the same for every element of a rank, so
// half of the first 64-bit product is too: with z = k ^ seed_mix split into
// words (zhi, zlo) and t = z ^ (z >> 30), t * C1 mod 2^64 needs only
// tlo * C1lo in full plus the low words of tlo * C1hi and thi * C1lo, the
// last a constant.  Same bits as mix64, one 32-bit multiply fewer.
struct KeyHash {
  uint32_t zhi, smlo, thi_c1lo;
};

__device__ inline KeyHash key_hash_setup(const FillArgs& a, uint32_t p) {
  KeyHash k;
  k.zhi = ((p << 16) | a.h.round) ^ (uint32_t)(a.seed_mix >> 32);
  k.smlo = (uint32_t)a.seed_mix;
  k.thi_c1lo = (k.zhi ^ (k.zhi >> 30)) * 0x1CE4E5B9u;
  return k;
}

__device__ inline uint64_t key_hash(const KeyHash& k, uint32_t idx) {
  const uint32_t lo = idx ^ k.smlo;
  const uint32_t tlo = lo ^ ((k.zhi << 2) | (lo >> 30));
  const uint64_t prod = (uint64_t)tlo * 0x1CE4E5B9u;
  const uint32_t z1hi = (uint32_t)(prod >> 32) + tlo * 0xBF58476Du + k.thi_c1lo;
  const uint64_t z1 = ((uint64_t)z1hi << 32) | (uint32_t)prod;
  const uint64_t z2 = (z1 ^ (z1 >> 27)) * 0x94D049BB133111EBull;
  return z2 ^ (z2 >> 31);
}

__device__ inline uint32_t bf16_of(uint64_t h) {
  const int32_t u = (int32_t)(h >> 41) - (1 << 22);
  const float f = (float)u * (1.0f / 4194304.0f);  // exact: |u| <= 2^22
  return __float_as_uint(f) >> 16;
}

// Element index (within rank p's view) of the element at byte `off`.
__device__ inline uint64_t index_at(const FillArgs& a, uint32_t p, uint64_t off) {
  const uint64_t rel = off - a.view_off[p];
  if (a.contiguous & (1u << p)) return rel / a.elem;
  const uint64_t r = rel / a.view_pitch[p];
  return r * a.view_cols[p] + (rel - r * a.view_pitch[p]) / a.elem;
}

// The fill is a producer: its waves take the highest issue priority over
// the copy engine's waves sharing their SIMDs (the engine waits for what the
// producer writes).  Fully triggered 4 x 1.5 GiB rounds (waves fill, 3 CTAs
// per CU): 5.67-5.71 ms against 5.75-5.79 without it; the small rounds and
// the deferred-mark all-gather are unchanged or slightly faster.
__device__ inline void producer_priority() { __builtin_amdgcn_s_setprio(3); }

// Byte `at` of a range starting at d: a plain store, or a write-through
// buffer store through `wt` (the same range's descriptor).
template <bool kWriteThrough>
__device__ inline void put_byte(uint8_t* d, __amdgpu_buffer_rsrc_t wt, uint32_t at, uint8_t v) {
  if (kWriteThrough)
    __builtin_amdgcn_raw_buffer_store_b8(v, wt, (int)at, 0, 17 /* sc0 sc1 */);
  else
    d[at] = v;
}

// Whole CTA: write the values of `len` bytes at `off` (within one view row,
// or anywhere in a contiguous view) of replica p; idx0 is the view element
// index of byte `off`.  With kWriteThrough the stores go through to memory
// at system scope (len < 2^31), so that once they complete the bytes are
// visible to every CU without an L2 write-back.  kIlp 4 computes four vectors
// per thread before storing them (for long spans), 1 one at a time; kThreads
// is the CTA's thread count.
template <bool kWriteThrough, int kIlp = 4, int kThreads = kFillThreads>
__device__ void fill_span(const FillArgs& a, uint32_t p, uint64_t off, uint64_t len, uint64_t idx0) {
  uint8_t* base = reinterpret_cast<uint8_t*>(a.rep[p]);
  const __amdgpu_buffer_rsrc_t wt =
      __builtin_amdgcn_make_buffer_rsrc(base + off, 0, kWriteThrough ? (int)len : 0, 0x00020000);
  const KeyHash kh = key_hash_setup(a, p);
  const uint32_t e = a.elem;
  if (((off | len) & 15) == 0) {
    const uint32_t per = 16 / e;  // elements per 16-byte vector
    const uint64_t nv = len / 16;
    u32x4* dst = reinterpret_cast<u32x4*>(base + off);
    auto value = [&](uint64_t v) {
      const uint64_t i0 = idx0 + v * per;
      u32x4 out;
      if (a.kind == TC_FILL_U32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = (uint32_t)key_hash(kh, (uint32_t)(i0 + k));
      } else if (a.kind == TC_FILL_BF16) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          out[k] = bf16_of(key_hash(kh, (uint32_t)(i0 + 2 * k))) |
                   (bf16_of(key_hash(kh, (uint32_t)(i0 + 2 * k + 1))) << 16);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t w = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) w |= ((uint32_t)key_hash(kh, (uint32_t)(i0 + 4 * k + b)) & 0xFF) << (8 * b);
          out[k] = w;
        }
      }
      return out;
    };
    auto put = [&](uint64_t v, const u32x4& out) {
      if (kWriteThrough)
        __builtin_amdgcn_raw_buffer_store_b128(out, wt, (int)(v * 16), 0, 17 /* sc0 sc1 */);
      else
        dst[v] = out;
    };
    // Four vectors per thread per pass: their hash chains are independent,
    // so one wave per SIMD keeps the arithmetic units busy (a CTA of more
    // waves might not fit beside a persistent copy engine that fills the
    // CU's other slots, and must run while it waits for the marks).  A
    // 16 KiB one-shot block stores each vector as soon as it is computed
    // (with 256 threads, four vectors each: 5.672 ms per all-gather step
    // against 5.697 with the four computed first).
    uint64_t v = threadIdx.x;
    if (kIlp == 4) {
      for (; v + 3 * kThreads < nv; v += 4 * kThreads) {
        const u32x4 o0 = value(v), o1 = value(v + kThreads), o2 = value(v + 2 * kThreads),
                    o3 = value(v + 3 * kThreads);
        put(v, o0);
        put(v + kThreads, o1);
        put(v + 2 * kThreads, o2);
        put(v + 3 * kThreads, o3);
      }
    }
    for (; v < nv; v += kThreads) put(v, value(v));
  } else {
    const uint64_t n = len / e;
    uint8_t* d = base + off;
    for (uint64_t i = threadIdx.x; i < n; i += kThreads) {
      const uint64_t h = key_hash(kh, (uint32_t)(idx0 + i));
      const uint32_t at = (uint32_t)(i * e);
      if (a.kind == TC_FILL_U32) {
        const uint32_t v = (uint32_t)h;
#pragma unroll
        for (uint32_t b = 0; b < 4; ++b) put_byte<kWriteThrough>(d, wt, at + b, (uint8_t)(v >> (8 * b)));
      } else if (a.kind == TC_FILL_BF16) {
        const uint32_t v = bf16_of(h);
        put_byte<kWriteThrough>(d, wt, at, (uint8_t)v);
        put_byte<kWriteThrough>(d, wt, at + 1, (uint8_t)(v >> 8));
      } else {
        put_byte<kWriteThrough>(d, wt, at, (uint8_t)h);
      }
    }
  }
}

template <bool kWriteThrough = false>
__device__ void fill_range(const FillArgs& a, uint32_t p, uint64_t off, uint64_t len) {
  fill_span<kWriteThrough>(a, p, off, len, index_at(a, p, off));
}

template <bool kWriteThrough = false>
__device__ void fill_piece(const FillArgs& a, uint32_t p, const tc::PieceD& pc) {
  for (uint32_t r = 0; r < pc.rows; ++r)
    fill_range<kWriteThrough>(a, p, pc.off + (uint64_t)r * pc.pitch, pc.row_bytes);
}

// Writer j of chunk g writes pieces [j*np/w, (j+1)*np/w) of the chunk: as
// one byte range when the chunk is contiguous in a contiguous view (no
// per-piece descriptor round trips), else piece by piece.
__device__ inline bool share_is_range(const FillArgs& a, const tc::ChunkD& cd) {
  return (cd.flags & tc::kChunkContiguous) && (a.contiguous & (1u << cd.rank));
}

template <bool kWriteThrough = false>
__device__ void fill_share(const FillArgs& a, uint32_t g, uint32_t j) {
  const tc::ChunkD cd = a.chunks[g];
  const uint64_t lo = (uint64_t)j * cd.npieces / cd.writers;
  const uint64_t hi = (uint64_t)(j + 1) * cd.npieces / cd.writers;
  if (lo == hi) return;
  if (share_is_range(a, cd)) {
    const tc::PieceD first = a.pieces[cd.first_piece + lo];
    const tc::PieceD last = a.pieces[cd.first_piece + hi - 1];
    fill_range<kWriteThrough>(a, cd.rank, first.off, last.off + last.row_bytes - first.off);
    return;
  }
  for (uint64_t k = lo; k < hi; ++k) fill_piece<kWriteThrough>(a, cd.rank, a.pieces[cd.first_piece + k]);
}

// Largest g with wprefix[g] <= slot (binary search over G + 1 entries).
__device__ inline uint32_t slot_chunk(const uint64_t* wprefix, uint32_t G, uint64_t slot) {
  uint32_t lo = 0, hi = G;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const uint32_t mid = (lo + hi) / 2;
    if (wprefix[mid] <= slot) lo = mid; else hi = mid;
  }
  return lo;
}

// One CTA per writer slot.  With kWriteThrough every store goes through to
// memory at system scope and the mark needs no L2 write-back: a write-back
// release flushes the whole of its XCD's L2, the other writers' dirty lines
// included (8 ranks of one 4 MiB chunk each, 8 writers a chunk: 97 us
// rounds against 105.5).  The buffer stores need every span under 2 GiB: a
// share written as one byte range must be, a piece's row is by construction.
template <bool kWriteThrough>
__device__ void fill_parallel(const FillArgs& a) {
  producer_priority();
  const uint64_t slot = blockIdx.x;
  const uint32_t g = slot_chunk(a.wprefix, a.G, slot);
  fill_share<kWriteThrough>(a, g, (uint32_t)(slot - a.wprefix[g]));
  if (a.mark == TC_MARK_INKERNEL) {
    const tc::ChunkD cd = a.chunks[g];
    if (kWriteThrough) tc_mark_ready_wt(a.h, cd.rank, cd.local);
    else tc_mark_ready(a.h, cd.rank, cd.local);
  }
}

__global__ __launch_bounds__(kFillThreads) void fill_parallel_kernel(FillArgs a) { fill_parallel<false>(a); }
__global__ __launch_bounds__(kFillThreads) void fill_parallel_wt_kernel(FillArgs a) { fill_parallel<true>(a); }

__global__ __launch_bounds__(kFillThreads) void fill_serial_kernel(FillArgs a) {
  producer_priority();
  const uint32_t p = blockIdx.x;
  const uint32_t n = a.h.chunk_base[p + 1] - a.h.chunk_base[p];
  for (uint32_t k = 0; k < n; ++k) {
    const uint32_t c = a.order ? a.order[(uint64_t)p * a.order_stride + k] : k;
    if (c >= n) continue;  // not a chunk of this rank: it gets no marks, wait() names it
    const uint32_t g = a.h.chunk_base[p] + c;
    const uint32_t w = a.chunks[g].writers;
    for (uint32_t j = 0; j < w; ++j) {
      fill_share(a, g, j);
      if (a.mark == TC_MARK_INKERNEL) tc_mark_ready(a.h, p, c);
    }
  }
}

// Persistent grid: writer slots in waves (every rank's chunk 0 writers,
// then every rank's chunk 1 writers, ...); CTA i takes slots i, i + ctas, ...
// All loop bounds and indices are uniform over the CTA.  kWriteThrough as in
// fill_parallel (fully triggered rounds of 4 x 1.5 GiB: 5.80-5.85 ms against
// 5.84-5.88 with write-back stores and marks).
template <bool kWriteThrough>
__device__ void fill_waves(const FillArgs& a) {
  producer_priority();
  uint64_t slot = 0;
  for (uint32_t c = 0; c < a.max_chunks; ++c) {
    for (uint32_t p = 0; p < a.h.nranks; ++p) {
      if (c >= a.h.chunk_base[p + 1] - a.h.chunk_base[p]) continue;
      const uint32_t g = a.h.chunk_base[p] + c;
      const uint32_t w = a.chunks[g].writers;
      // This CTA's slots among [slot, slot + w): j = first, first + grid, ...
      const uint64_t first = (blockIdx.x + gridDim.x - slot % gridDim.x) % gridDim.x;
      for (uint64_t j = first; j < w; j += gridDim.x) {
        fill_share<kWriteThrough>(a, g, (uint32_t)j);
        if (a.mark == TC_MARK_INKERNEL) {
          if (kWriteThrough) tc_mark_ready_wt(a.h, p, c);
          else tc_mark_ready(a.h, p, c);
        }
      }
      slot += w;
    }
  }
}

__global__ __launch_bounds__(kFillThreads) void fill_waves_kernel(FillArgs a) { fill_waves<false>(a); }
__global__ __launch_bounds__(kFillThreads) void fill_waves_wt_kernel(FillArgs a) { fill_waves<true>(a); }

// One-shot grid: CTA b writes block b of the share table (kOneShotBlock
// bytes of one writer's share of a contiguous chunk) with write-through
// stores.  The share's blocks count themselves on a wrapping counter; the
// block that completes the count issues the writer's mark, so each writer
// slot still marks its chunk exactly once per round.  Counting happens only
// when the fill marks: a deferred-mark fill leaves the counters at zero.
__global__ __launch_bounds__(kOneShotThreads) void fill_oneshot_kernel(FillArgs a) {
  producer_priority();
  const uint64_t b = blockIdx.x;
  uint64_t lo = 0, hi = a.nshares;  // largest s with shares[s].first_block <= b
  while (hi - lo > 1) {
    const uint64_t mid = (lo + hi) / 2;
    if (a.shares[mid].first_block <= b) lo = mid; else hi = mid;
  }
  const tc::ShareD sh = a.shares[lo];
  const uint64_t nb = a.shares[lo + 1].first_block - sh.first_block;
  const uint64_t at = (b - sh.first_block) * tc::kOneShotBlock;
  if (at < sh.bytes) {
    // Contiguous view: the element index is the byte distance over the element size.
    const uint32_t p = a.chunks[sh.g].rank;
    const uint64_t rel = sh.off + at - a.view_off[p];
    const uint64_t idx0 = a.elem == 4 ? rel >> 2 : a.elem == 2 ? rel >> 1 : rel;
    fill_span<true, 1, kOneShotThreads>(a, p, sh.off + at, min(tc::kOneShotBlock, sh.bytes - at), idx0);
  }
  if (a.mark != TC_MARK_INKERNEL) return;
  __shared__ uint32_t last;
  __builtin_amdgcn_s_waitcnt(TC_WAITCNT_VMCNT0);  // this wave's write-through stores are in memory
  __syncthreads();                                // ... and every other wave's
  if (tc_is_cta_leader()) {
    uint32_t* ctr = reinterpret_cast<uint32_t*>(a.share_ctr + lo * 8);
    const uint32_t old = __builtin_amdgcn_atomic_inc32(ctr, (uint32_t)nb - 1, __ATOMIC_RELAXED, "agent");
    last = old == (uint32_t)nb - 1;
  }
  __syncthreads();
  if (tc_uniform(last)) {
    const tc::ChunkD cd = a.chunks[sh.g];
    tc_mark_ready_wt(a.h, cd.rank, cd.local);
  }
}

struct MarkArgs {
  tc_handle h;
  const uint64_t* wprefix;
  const tc::ChunkD* chunks;
  uint32_t G, rank, chunk, all;
};

__global__ __launch_bounds__(64) void mark_kernel(MarkArgs a) {
  if (a.all) {
    const uint32_t g = slot_chunk(a.wprefix, a.G, blockIdx.x);
    const tc::ChunkD cd = a.chunks[g];
    tc_mark_ready(a.h, cd.rank, cd.local);
  } else {
    tc_mark_ready(a.h, a.rank, a.chunk);
  }
}

struct ConsumeArgs {
  tc_handle h;
  uint64_t rep_dst;
  uint8_t* out;
  const tc::PieceD* pieces;
  const tc::ChunkD* chunks;
  uint32_t* status;
  uint32_t dst, max_polls;
};

// One CTA per global chunk: wait for its arrival at rank dst, then copy its
// bytes from replica dst to out at the same offsets.
__global__ __launch_bounds__(256) void consume_kernel(ConsumeArgs a) {
  const uint32_t g = blockIdx.x;
  const tc::ChunkD cd = a.chunks[g];
  const bool ok = tc_wait(a.h, a.dst, cd.rank, cd.local, a.max_polls);
  if (ok) {
    const uint8_t* src = reinterpret_cast<const uint8_t*>(a.rep_dst);
    for (uint32_t k = 0; k < cd.npieces; ++k) {
      const tc::PieceD pc = a.pieces[cd.first_piece + k];
      const uint64_t n = (uint64_t)pc.rows * pc.row_bytes;
      for (uint64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const uint64_t r = i / pc.row_bytes, c = i - r * pc.row_bytes;
        const uint64_t b = pc.off + r * pc.pitch + c;
        a.out[b] = src[b];
      }
    }
  }
  if (tc_is_cta_leader()) a.status[g] = ok ? 1u : 2u;
}

}  // namespace

#define TC_HIP(call)                                       \
  do {                                                     \
    hipError_t e_ = (call);                                \
    if (e_ != hipSuccess) return tc::hip_fail(e_, #call);  \
  } while (0)

extern "C" {

// Whether the writer-CTA fills (parallel and waves) store write-through and
// mark without an L2 write-back: when every share is one byte range under
// 2 GiB (every chunk one range, every view contiguous).  Shares written row
// by row keep plain stores: tiles' rows share cache lines, and writing them
// through measured slower (8 ranks of 64 x 64 u32 tiles, 4 a chunk: 108-110
// us rounds against 90).
static bool shares_write_through(const tc_plan* P, const FillArgs& a) {
  if (P->oneshot_blocks == 0 || P->max_range_share >= (1ull << 31)) return false;
  for (uint32_t p = 0; p < P->P; ++p)
    if (P->chunk_base[p + 1] > P->chunk_base[p] && !(a.contiguous & (1u << p))) return false;
  return true;
}

int tc_produce_fill(tc_plan* P, const tc_handle* h, const tc_fill_desc* d, void* stream) {
  if (!P || !h || !d || !d->views) return fail(TC_EINVAL, "fill: NULL argument");
  const uint32_t elem = d->kind == TC_FILL_U32 ? 4 : d->kind == TC_FILL_BF16 ? 2 : d->kind == TC_FILL_U8 ? 1 : 0;
  if (!elem) return fail(TC_EINVAL, "fill: unknown kind");
  if (d->mark_mode > TC_MARK_NONE) return fail(TC_EINVAL, "fill: unknown mark mode");
  if (h->round >= (1u << 16)) return fail(TC_EINVAL, "fill: value keys hold rounds below 65536");
  const bool ready_ok = d->mark_mode == TC_MARK_NONE && P->state == TC_STATE_READY;
  if ((P->state != TC_STATE_STARTED && !ready_ok) || h->round != P->round)
    return fail(TC_ESTATE, "fill: the handle is not this plan's current round");
  FillArgs a{};
  for (uint32_t p = 0; p < P->P; ++p) {
    const tc_view& v = d->views[p];
    if (v.elem_bytes != elem) return fail(TC_EINVAL, "fill: view elem_bytes does not match kind");
    if (v.rows * v.cols >= (1ull << 32)) return fail(TC_EINVAL, "fill: value keys hold < 2^32 elements");
    a.rep[p] = (uint64_t)P->rep[p];
    a.view_off[p] = v.byte_offset;
    a.view_pitch[p] = v.row_stride * elem;
    a.view_cols[p] = v.cols;
    if (v.row_stride == v.cols) a.contiguous |= 1u << p;
  }
  a.pieces = reinterpret_cast<const tc::PieceD*>(P->ws + P->L.pieces);
  a.chunks = reinterpret_cast<const tc::ChunkD*>(P->ws + P->L.chunks);
  a.wprefix = reinterpret_cast<const uint64_t*>(P->ws + P->L.wprefix);
  a.order = d->order;
  a.order_stride = d->order_stride;
  a.h = *h;
  a.seed_mix = mix64(d->seed);
  a.kind = d->kind;
  a.mark = d->mark_mode;
  a.elem = elem;
  a.G = P->G;
  hipStream_t s = (hipStream_t)stream;
  if (d->mode != TC_FILL_WAVES && d->ctas) return fail(TC_EINVAL, "fill: ctas is for the waves mode");
  if (d->mode != TC_FILL_SERIAL && d->order) return fail(TC_EINVAL, "fill: an order needs serial mode");
  if (d->order) {  // the kernel reads order[p * order_stride + k] for k below rank p's chunk count
    uint32_t most = 0;
    for (uint32_t p = 0; p < P->P; ++p) most = std::max(most, P->chunk_base[p + 1] - P->chunk_base[p]);
    if (d->order_stride < most) return fail(TC_EINVAL, "fill: order_stride below a rank's chunk count");
    if (int rc = tc::check_device_range(d->order, (uint64_t)P->P * d->order_stride * 4, P->device,
                                        "fill: order"))
      return rc;
  }
  if (d->mode == TC_FILL_SERIAL) {
    hipLaunchKernelGGL(fill_serial_kernel, dim3(P->P), dim3(kFillThreads), 0, s, a);
  } else if (d->mode == TC_FILL_PARALLEL) {
    if (P->total_writers == 0) return TC_OK;
    if (P->total_writers > 0x7FFFFFFFull) return fail(TC_EINVAL, "fill: too many writers");
    if (shares_write_through(P, a))
      hipLaunchKernelGGL(fill_parallel_wt_kernel, dim3((uint32_t)P->total_writers), dim3(kFillThreads), 0, s, a);
    else
      hipLaunchKernelGGL(fill_parallel_kernel, dim3((uint32_t)P->total_writers), dim3(kFillThreads), 0, s, a);
  } else if (d->mode == TC_FILL_WAVES) {
    if (P->total_writers == 0) return TC_OK;
    uint32_t ctas = d->ctas;
    if (ctas == 0) {  // two 4-wave CTAs per CU: the measured optimum for the hash fill
      int cus = 0;
      TC_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, P->device));
      ctas = 2u * (uint32_t)cus;
    }
    for (uint32_t p = 0; p < P->P; ++p)
      a.max_chunks = std::max(a.max_chunks, P->chunk_base[p + 1] - P->chunk_base[p]);
    if (shares_write_through(P, a))
      hipLaunchKernelGGL(fill_waves_wt_kernel, dim3(ctas), dim3(kFillThreads), 0, s, a);
    else
      hipLaunchKernelGGL(fill_waves_kernel, dim3(ctas), dim3(kFillThreads), 0, s, a);
  } else if (d->mode == TC_FILL_ONESHOT) {
    if (P->total_writers == 0) return TC_OK;
    if (P->oneshot_blocks == 0) return fail(TC_EINVAL, "fill: one-shot mode needs every chunk to be one byte range");
    for (uint32_t p = 0; p < P->P; ++p)
      if (P->chunk_base[p + 1] > P->chunk_base[p] && !(a.contiguous & (1u << p)))
        return fail(TC_EINVAL, "fill: one-shot mode needs contiguous views");
    if (P->oneshot_blocks > 0x7FFFFFFFull) return fail(TC_EINVAL, "fill: too many one-shot blocks");
    a.shares = reinterpret_cast<const tc::ShareD*>(P->ws + P->L.shares);
    a.share_ctr = reinterpret_cast<uint64_t*>(P->ws + P->L.share_ctr);
    a.nshares = P->total_writers;
    hipLaunchKernelGGL(fill_oneshot_kernel, dim3((uint32_t)P->oneshot_blocks), dim3(kOneShotThreads), 0, s, a);
  } else {
    return fail(TC_EINVAL, "fill: unknown mode");
  }
  TC_HIP(hipGetLastError());
  return TC_OK;
}

int tc_mark_all(tc_plan* P, const tc_handle* h, void* stream) {
  if (!P || !h) return fail(TC_EINVAL, "mark_all: NULL argument");
  if ((P->state != TC_STATE_READY && P->state != TC_STATE_STARTED) || h->round != P->round)
    return fail(TC_ESTATE, "mark_all: the handle is not this plan's current round");
  if (P->total_writers == 0) return TC_OK;
  if (P->total_writers > 0x7FFFFFFFull) return fail(TC_EINVAL, "mark_all: too many writers");
  MarkArgs a{};
  a.h = *h;
  a.wprefix = reinterpret_cast<const uint64_t*>(P->ws + P->L.wprefix);
  a.chunks = reinterpret_cast<const tc::ChunkD*>(P->ws + P->L.chunks);
  a.G = P->G;
  a.all = 1;
  hipLaunchKernelGGL(mark_kernel, dim3((uint32_t)P->total_writers), dim3(64), 0, (hipStream_t)stream, a);
  TC_HIP(hipGetLastError());
  return TC_OK;
}

int tc_mark(tc_plan* P, const tc_handle* h, uint32_t rank, uint32_t chunk, uint32_t count,
            void* stream) {
  if (!P || !h) return fail(TC_EINVAL, "mark: NULL argument");
  if (rank >= P->P || chunk >= P->chunk_base[rank + 1] - P->chunk_base[rank])
    return fail(TC_EINVAL, "mark: no such (rank, chunk)");
  if (count == 0) return TC_OK;
  MarkArgs a{};
  a.h = *h;
  a.rank = rank;
  a.chunk = chunk;
  hipLaunchKernelGGL(mark_kernel, dim3(count), dim3(64), 0, (hipStream_t)stream, a);
  TC_HIP(hipGetLastError());
  return TC_OK;
}

int tc_consume_copy(tc_plan* P, const tc_handle* h, uint32_t dst, void* out_buf,
                    uint32_t max_polls, uint32_t* status, void* stream) {
  if (!P || !h || !out_buf || !status) return fail(TC_EINVAL, "consume: NULL argument");
  if (dst >= P->P) return fail(TC_EINVAL, "consume: dst out of range");
  if (P->G == 0) return TC_OK;
  if (int rc = tc::check_device_range(out_buf, P->buffer_bytes, P->device, "consume: out_buf"))
    return rc;
  if (int rc = tc::check_device_range(status, (uint64_t)P->G * 4, P->device, "consume: status"))
    return rc;
  ConsumeArgs a{};
  a.h = *h;
  a.rep_dst = (uint64_t)P->rep[dst];
  a.out = (uint8_t*)out_buf;
  a.pieces = reinterpret_cast<const tc::PieceD*>(P->ws + P->L.pieces);
  a.chunks = reinterpret_cast<const tc::ChunkD*>(P->ws + P->L.chunks);
  a.status = status;
  a.dst = dst;
  a.max_polls = max_polls;
  hipLaunchKernelGGL(consume_kernel, dim3(P->G), dim3(256), 0, (hipStream_t)stream, a);
  TC_HIP(hipGetLastError());
  return TC_OK;
}

}  // extern "C"
