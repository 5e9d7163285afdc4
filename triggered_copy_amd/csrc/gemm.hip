// Persistent bf16 GEMM producer with an in-kernel mark_ready.
//
// [TP] = "Triggered Plans" (Iris documentation), section Model: the example
// producer is a persistent tiled kernel: program p handles the steps
// congruent to p modulo the number of programs; each step computes the tile tile_of(step) picks, stores
// it, then marks chunk first_chunk + step / tiles_per_chunk ready.  The host
// builds the schedule with tile_chunks() from the same tile_of, so the two
// cannot disagree.
//
// C[M,N] = A[M,K] * B, with B given as Bt[N,K] (K contiguous, so both
// operands stream along K), bf16 inputs, fp32 accumulation on the matrix
// cores, bf16 output (round to nearest even).
//
// The same kernel is the in-kernel consumer of a gathered buffer ([TP]
// Memory ordering, consumer side): A is a rank's replica of the gathered
// rows, and before a step touches its 128-row block of A, the CTA waits
// (tc_wait) for every chunk whose regions reach into those rows.
//
// gfx950 mapping: a 256-thread CTA computes a 128 x 128 tile; its 4 waves
// form a 2 x 2 grid of 64 x 64 sub-tiles, each 4 x 4 blocks of the 16x16x32
// bf16 MFMA (v_mfma_f32_16x16x32_bf16), and every wave runs the whole K
// range, so no partial sums are exchanged.  Operands reach LDS without
// passing through registers: buffer_load_dwordx4 with the LDS bit writes
// each lane's 16 bytes to LDS at M0 + 16 * lane, and the 64-wide K slabs go
// round a ring of kStages LDS buffers, so the loads for slabs k + 2 and
// k + 3 are in flight while slab k + 1 waits its turn.  The lane -> global
// address map is chosen so that the slab lands XOR-swizzled (16-byte column
// c of row r at position c ^ (r % 8)), which spreads every fragment read
// over all banks.  Rows past M and columns past K read as zero through the
// buffer range check.  The first k step's fragments of the next slab are
// read while the second k step of this slab is multiplied, so the matrix
// cores see no gap at the slab barrier.  The finished tile is staged
// through LDS so the bf16 stores are 16-byte vectors along the row.
#include <hip/hip_runtime.h>

#include <string>

#include "internal.h"
#include "plan_internal.h"
#include "tc.h"
#include "tc_device.h"

using tc::fail;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;                  // 4 waves
constexpr int kStages = 4;                     // LDS ring depth, in K slabs
constexpr int kRowBytes = BK * 2;              // one slab row: 8 columns of 16 bytes
constexpr int kOpBytes = BM * kRowBytes;       // one operand's slab: 16 KiB
constexpr int kStageBytes = 2 * kOpBytes;      // A slab, then B slab
constexpr int kLoads = kOpBytes / (kThreads * 16);  // LDS-DMA loads per thread per operand
constexpr int LDC = BN + 8;                    // bf16 elements per staged C row
constexpr uint32_t kNoRead = 0x80000000u;      // a buffer offset past every range: reads 0

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* Bt;
  uint16_t* C;
  uint64_t lda, ldc;
  uint32_t M, N, K;
  uint32_t tm, tn, group_m;
  uint32_t tiles;
  uint32_t mark, rank, first_chunk, tiles_per_chunk;
  // Consumer mode (wait != 0): before a step, wait for the chunks listed for
  // its 128-row block of A: pairs (src, chunk) dep_pairs[2 d], d in
  // [dep_start[b], dep_start[b + 1]), as seen by rank dst.
  uint32_t wait, dst, max_polls, pad;
  const uint32_t* dep_start;
  const uint32_t* dep_pairs;
  uint32_t* status;  // per row block: 2 when a wait ran out of polls (may be NULL)
  tc_handle h;
};

__device__ inline uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int n>
__device__ inline void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte LDS-DMA load per lane: buffer_load_dwordx4 with the LDS bit
// reads rsrc at voff and writes lane l's 16 bytes to LDS at m0 + 16 l.  It
// is written out by hand so that the compiler, which cannot tell which ring
// buffer a DMA fills, does not wait for every DMA in flight before each LDS
// read; the kernel waits for them itself (vmcnt counts these loads).
__device__ inline void lds_dma16(u32x4 rsrc, uint32_t voff, uint32_t m0) {
  asm volatile(
      "s_nop 0\n\t"  // one wait state between the write of m0 and its use here
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "{m0}"(m0)
      : "memory");
}

// A raw buffer descriptor (stride 0) over [base, base + bytes).
__device__ inline u32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return u32x4{tc_uniform((uint32_t)p), tc_uniform((uint32_t)(p >> 32) & 0xFFFFu), tc_uniform(bytes),
               0x00020000u};
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
  static_assert(kStages * kStageBytes >= BM * LDC * 2, "C staging fits in the ring");
  static_assert(kOpBytes % (kThreads * 16) == 0 && kLoads * 4 * 64 * 16 == kOpBytes,
                "every wave loads whole 1 KiB blocks");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStageBytes];
  uint16_t* cst = reinterpret_cast<uint16_t*>(lds);
  // The GEMM's waves take the highest issue priority: they share every CU's
  // SIMDs with the copy engine's waves, which are latency-bound and lose
  // little by it.  Beside the engine, 4 GEMM producers were slowed by 5.9-6.1%
  // with it against 7.2-8.2% without (the same round time; the GEMMs alone
  // unchanged).
  __builtin_amdgcn_s_setprio(3);
  const uint32_t lds_base = tc_uniform((uint32_t)(uintptr_t)(lds_ptr_t)lds);

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t wave = tc_uniform(tid >> 6);
  const uint32_t wm = wave >> 1, wn = wave & 1;
  const uint32_t nk = (a.K + BK - 1) / BK;

  // Loads: wave w, load i of an operand fills the 1 KiB block of slab rows
  // 8 (kLoads w + i) .. +7; lane l lands at row + l / 8, position l % 8,
  // which holds the row's 16-byte column (l % 8) ^ (l / 8).
  const uint32_t lrow = lane >> 3, lcol = (lane & 7) ^ lrow;
  // Fragment reads: lane l of a 16x16x32 block holds row l % 16 and the 8 k
  // values of 16-byte column 4 h + l / 16 (k step h of the slab).
  const uint32_t fr = lane & 15, fq = lane >> 4;
  const uint32_t a_frag = (wm * 64 + fr) * kRowBytes, b_frag = kOpBytes + (wn * 64 + fr) * kRowBytes;
  const uint32_t xcol0 = ((0 + fq) ^ (fr & 7)) * 16, xcol1 = ((4 + fq) ^ (fr & 7)) * 16;

  // Workgroups are dealt to the 8 XCDs round-robin; program p of the
  // persistent grid is workgroup w(p) such that each XCD runs consecutive
  // programs, hence consecutive steps: a compact block of tiles in the
  // grouped order, whose A and B panels its L2 shares.  A bijection on
  // [0, gridDim.x); every step is still taken exactly once.
  const uint32_t first = gridDim.x % 8 == 0 ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8
                                            : blockIdx.x;
  for (uint32_t step = first; step < a.tiles; step += gridDim.x) {
    const uint32_t t = tc_tile_of(step, a.tm, a.tn, a.group_m);
    const uint32_t m0 = (t / a.tn) * BM, n0 = (t % a.tn) * BN;
    const uint32_t rows_in = a.M - m0 < (uint32_t)BM ? a.M - m0 : (uint32_t)BM;
    const uint32_t cols_in = a.N - n0 < (uint32_t)BN ? a.N - n0 : (uint32_t)BN;

    // Each operand's tile rows through a buffer resource whose range ends
    // with the last valid row's K elements: rows past M or N read as zero.
    const u32x4 ra = buffer_desc(a.A + (uint64_t)m0 * a.lda,
                                 (uint32_t)(((uint64_t)(rows_in - 1) * a.lda + a.K) * 2));
    const u32x4 rb = buffer_desc(a.Bt + (uint64_t)n0 * a.K, (uint32_t)((uint64_t)cols_in * a.K * 2));
    uint32_t offa[kLoads], offb[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const uint32_t r = 8 * (kLoads * wave + i) + lrow;
      offa[i] = (uint32_t)(r * a.lda * 2) + lcol * 16;
      offb[i] = (uint32_t)(r * a.K * 2) + lcol * 16;
    }
    // Part i of slab kt's loads into ring buffer b: load i of each operand.
    // Columns past K (a ragged last slab, or a slab past the end) read as
    // zero: every offset stays below 2^31 (a tile spans less than 2 GiB),
    // so setting bit 31 moves it past the range.
    auto issue_part = [&](uint32_t kt, uint32_t b, int i) {
      const uint32_t kmask = kt * BK + lcol * 8 < a.K ? 0u : kNoRead;
      const uint32_t kb = kt * kRowBytes;
      const uint32_t base = lds_base + b * kStageBytes + wave * kLoads * 1024 + i * 1024;
      lds_dma16(ra, (offa[i] + kb) | kmask, base);
      lds_dma16(rb, (offb[i] + kb) | kmask, base + kOpBytes);
    };
    // Group g of one k step's 8 fragment reads: the B fragments (output
    // columns 16 j.. of this wave's 64) in groups 0 and 1, the A fragments
    // (rows 16 i..) in groups 2 and 3.  A row of MFMAs needs all of B and
    // one A fragment, so rows 0 and 1 can start once group 2 has landed.
    auto read_group = [&](uint32_t b, uint32_t xcol, int g, bf16x8 (&fa)[4], bf16x8 (&fb)[4]) {
      const uint8_t* s = lds + b * kStageBytes;
      bf16x8* f = g < 2 ? fb : fa;
      const uint32_t base = g < 2 ? b_frag : a_frag;
      const int i0 = 2 * (g & 1);
      f[i0] = *reinterpret_cast<const bf16x8*>(s + base + i0 * 16 * kRowBytes + xcol);
      f[i0 + 1] = *reinterpret_cast<const bf16x8*>(s + base + (i0 + 1) * 16 * kRowBytes + xcol);
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Row i of the 4 x 4 blocks for one k step.  The B fragment goes first,
    // so each output block is C transposed.
    auto mfma_row = [&](int i, const bf16x8 (&fa)[4], const bf16x8 (&fb)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    };

    if (a.wait) {
      // Whole-CTA waits with uniform bounds: every wave takes every wait.
      const uint32_t b = m0 / BM;
      const uint32_t d0 = tc_uniform(a.dep_start[b]), d1 = tc_uniform(a.dep_start[b + 1]);
      bool ok = true;
      for (uint32_t d = d0; d < d1; ++d)
        if (!tc_wait(a.h, a.dst, tc_uniform(a.dep_pairs[2 * d]), tc_uniform(a.dep_pairs[2 * d + 1]),
                     a.max_polls))
          ok = false;
      if (!ok && a.status && tc_is_cta_leader()) a.status[b] = 2u;
    }
    __syncthreads();  // the previous tile's C staging is no longer read
    // The ring holds slabs kt - 1 .. kt + 2.  At the barrier in the middle
    // of iteration kt every wave is done with slab kt - 1, whose buffer then
    // takes slab kt + 3.  Every iteration issues one slab, past the end too
    // (those read as zero into a buffer no one reads), so when slab kt + 1
    // is waited for, exactly one slab follows it.  (Refilling slab kt's own
    // buffer at that barrier, one more slab in flight, measured slower.)
    static_assert(kStages == 4, "the waits below count one slab in flight behind the next");
    constexpr int kSlabLoads = 2 * kLoads;  // one slab's loads per wave
    for (uint32_t s = 0; s + 1 < kStages; ++s)
#pragma unroll
      for (int i = 0; i < kLoads; ++i) issue_part(s, s, i);
    wait_vmcnt<2 * kSlabLoads>();  // slab 0 has landed; slabs 1 and 2 may be in flight
    __syncthreads();

    // Each k step's MFMAs run while the next k step's fragments are read:
    // the first row of four MFMAs goes out, then all 8 reads for the next k
    // step, then the other three rows, so the reads have a whole k step to
    // land; after the slab barrier the next slab's loads follow the rows.
    // The scheduling barriers keep the compiler from regrouping them.
    bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) read_group(0, xcol0, g, fa0, fb0);
    uint32_t kt = 0;
    for (; kt + 1 < nk; ++kt) {
      const uint32_t cur = kt % kStages, nxt = (kt + 1) % kStages;
      const uint32_t fill = (kt + kStages - 1) % kStages;
      mfma_row(0, fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) read_group(cur, xcol1, g, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 1; i < 4; ++i) mfma_row(i, fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<kSlabLoads>();  // slab kt + 1 has landed for this wave
      __syncthreads();
      mfma_row(0, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 4; ++g) read_group(nxt, xcol0, g, fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        issue_part(kt + kStages - 1, fill, i);
        __builtin_amdgcn_sched_barrier(0);
        if (i < 3) mfma_row(i + 1, fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mfma_row(0, fa0, fb0);
#pragma unroll
    for (int g = 0; g < 4; ++g) read_group(kt % kStages, xcol1, g, fa1, fb1);
#pragma unroll
    for (int i = 1; i < 4; ++i) mfma_row(i, fa0, fb0);
#pragma unroll
    for (int i = 0; i < 4; ++i) mfma_row(i, fa1, fb1);
    wait_vmcnt<0>();  // the loads past the end, before the ring is reused
    __syncthreads();  // every wave is done with the ring

    // Stage the tile as bf16.  The MFMA output block is C transposed: lane l
    // holds row l % 16 and the 4 consecutive columns 4 * (l / 16) + e --
    // one 8-byte write per block.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t r = wm * 64 + i * 16 + fr;
        const uint32_t c = wn * 64 + j * 16 + 4 * fq;
        const uint32_t lo = f32_to_bf16_rne(acc[i][j][0]) | (f32_to_bf16_rne(acc[i][j][1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(acc[i][j][2]) | (f32_to_bf16_rne(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(cst + r * LDC + c) = make_uint2(lo, hi);
      }
    __syncthreads();
    // 128 rows x 16 vectors of 8 bf16: 8 vectors per thread, stored through
    // to memory at system scope, so that once they complete the tile is
    // visible everywhere and mark_ready needs no L2 write-back.  Lanes
    // outside the matrix get an offset past the buffer range and their
    // stores are dropped.
    const uint32_t extent = (uint32_t)(((uint64_t)(rows_in - 1) * a.ldc + cols_in) * 2);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        a.C + (uint64_t)m0 * a.ldc + n0, 0, (int)extent, 0x00020000);
#pragma unroll
    for (int s = 0; s < BM * BN / 8 / kThreads; ++s) {
      const uint32_t v = tid + kThreads * s;
      const uint32_t r = v >> 4, c = (v & 15) * 8;
      const bool in = r < rows_in && c < cols_in;
      const uint32_t off = in ? (uint32_t)(((uint64_t)r * a.ldc + c) * 2) : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(cst + r * LDC + c), rc,
                                             (int)off, 0, 17 /* sc0 sc1 */);
    }
    if (a.mark) tc_mark_ready_wt(a.h, a.rank, a.first_chunk + step / a.tiles_per_chunk);
  }
}

}  // namespace

static int check_gemm_shape(const void* A, const void* Bt, const void* C, uint32_t M, uint32_t N,
                            uint32_t K, uint64_t lda, uint64_t ldc, uint32_t programs,
                            uint32_t group_m) {
  if (!A || !Bt || !C) return fail(TC_EINVAL, "gemm: NULL operand");
  if (M == 0 || N == 0 || K == 0 || programs == 0 || group_m == 0)
    return fail(TC_EINVAL, "gemm: zero size");
  if (K % 8 || N % 8 || ldc % 8 || ldc < N || lda % 8 || lda < K)
    return fail(TC_EINVAL, "gemm: K, N, lda and ldc must be multiples of 8 (16-byte rows), "
                           "lda >= K, ldc >= N");
  if ((uint64_t)BM * ldc * 2 >= (1ull << 31) || (uint64_t)BM * lda * 2 >= (1ull << 31))
    return fail(TC_EINVAL, "gemm: a 128-row tile of A or C must span less than 2 GiB "
                           "(lda, ldc < 2^23)");
  if (((uintptr_t)A | (uintptr_t)Bt | (uintptr_t)C) & 15)
    return fail(TC_EINVAL, "gemm: operands must be 16-byte aligned");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(TC_EHIP, "gemm: hipGetDevice failed");
  if (int rc = tc::check_device_range(A, ((uint64_t)(M - 1) * lda + K) * 2, dev, "gemm: A")) return rc;
  if (int rc = tc::check_device_range(Bt, (uint64_t)N * K * 2, dev, "gemm: Bt")) return rc;
  if (int rc = tc::check_device_range(C, ((uint64_t)(M - 1) * ldc + N) * 2, dev, "gemm: C")) return rc;
  return TC_OK;
}

static void fill_shape(GemmArgs& a, const void* A, const void* Bt, void* C, uint32_t M, uint32_t N,
                       uint32_t K, uint64_t lda, uint64_t ldc, uint32_t group_m) {
  a.A = (const uint16_t*)A;
  a.Bt = (const uint16_t*)Bt;
  a.C = (uint16_t*)C;
  a.lda = lda;
  a.ldc = ldc;
  a.M = M;
  a.N = N;
  a.K = K;
  a.tm = (M + BM - 1) / BM;
  a.tn = (N + BN - 1) / BN;
  a.group_m = group_m;
  a.tiles = a.tm * a.tn;
}

static int launch(const GemmArgs& a, uint32_t programs, void* stream) {
  hipLaunchKernelGGL(gemm_kernel, dim3(programs), dim3(kThreads), 0, (hipStream_t)stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return tc::hip_fail(e, "gemm launch");
  return TC_OK;
}

extern "C" int tc_gemm_bf16(const void* A, const void* Bt, void* C, uint32_t M, uint32_t N,
                            uint32_t K, uint64_t ldc, uint32_t programs, uint32_t group_m,
                            const tc_handle* h, uint32_t rank, uint32_t first_chunk,
                            uint32_t tiles_per_chunk, void* stream) {
  if (int rc = check_gemm_shape(A, Bt, C, M, N, K, K, ldc, programs, group_m)) return rc;
  if (h && (tiles_per_chunk == 0 || rank >= h->nranks))
    return fail(TC_EINVAL, "gemm: bad rank or tiles_per_chunk");
  GemmArgs a{};
  fill_shape(a, A, Bt, C, M, N, K, K, ldc, group_m);
  if (h) {
    a.mark = 1;
    a.h = *h;
    a.rank = rank;
    a.first_chunk = first_chunk;
    a.tiles_per_chunk = tiles_per_chunk;
    const uint32_t nchunks = h->chunk_base[rank + 1] - h->chunk_base[rank];
    if (first_chunk + (a.tiles - 1) / tiles_per_chunk >= nchunks)
      return fail(TC_EINVAL, "gemm: the tiles map past the rank's chunks");
  }
  return launch(a, programs, stream);
}

extern "C" int tc_gemm_consume_bf16(const tc_handle* h, uint32_t dst, const uint32_t* dep_start,
                                    const uint32_t* dep_pairs, uint32_t max_polls,
                                    uint32_t* status, const void* X, uint64_t ldx, const void* Wt,
                                    void* Y, uint32_t M, uint32_t N, uint32_t K, uint64_t ldy,
                                    uint32_t programs, uint32_t group_m, void* stream) {
  if (!h || !dep_start || !dep_pairs) return fail(TC_EINVAL, "consume gemm: NULL argument");
  if (dst >= h->nranks) return fail(TC_EINVAL, "consume gemm: dst out of range");
  if (max_polls == 0) return fail(TC_EINVAL, "consume gemm: max_polls is 0");
  if (int rc = check_gemm_shape(X, Wt, Y, M, N, K, ldx, ldy, programs, group_m)) return rc;
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(TC_EHIP, "consume gemm: hipGetDevice failed");
    const uint64_t nb = (M + BM - 1) / BM;
    if (int rc = tc::check_device_range(dep_start, (nb + 1) * 4, dev, "consume gemm: dep_start"))
      return rc;
    if (status)
      if (int rc = tc::check_device_range(status, nb * 4, dev, "consume gemm: status")) return rc;
  }
  GemmArgs a{};
  fill_shape(a, X, Wt, Y, M, N, K, ldx, ldy, group_m);
  a.h = *h;
  a.wait = 1;
  a.dst = dst;
  a.max_polls = max_polls;
  a.dep_start = dep_start;
  a.dep_pairs = dep_pairs;
  a.status = status;
  return launch(a, programs, stream);
}
