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
// gfx950 mapping: a 512-thread CTA computes a 128 x 128 tile with two groups
// of 4 waves.  In each group the waves form a 2 x 2 grid of 64 x 64
// sub-tiles, each 4 x 4 blocks of the 16x16x32 bf16 MFMA
// (v_mfma_f32_16x16x32_bf16).  The groups split K: group g multiplies the
// 64-wide slabs g, g + 2, g + 4, ..., each through two LDS buffers of its
// own (slab k + 2 travels from global memory into registers and then into
// the other buffer while slab k is multiplied).  Two waves per SIMD, one of
// each group, so one wave's MFMAs cover the other's load and LDS latency.
// At the end group 1 hands its partial sums to group 0 through LDS.  LDS
// rows are padded by 16 bytes to spread the 16-byte fragment reads over the
// banks; the finished tile is staged through LDS so the bf16 stores are
// 16-byte vectors along the row.
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

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDA = BK + 8;            // bf16 elements per LDS row (16 bytes of padding)
constexpr int kThreads = 512;          // two groups of 4 waves
constexpr int kGroupThreads = 256;
constexpr int LDC = BN + 8;            // bf16 elements per staged C row

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

__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs a) {
  // LDS: slab (group g, buffer b, operand o) at (4 g + 2 b + o) * kSlab during
  // the K loop; afterwards group 1's partial sums (kRed floats) followed by
  // the staged C tile.
  constexpr int kSlab = BM * LDA;        // bf16 elements per operand slab
  constexpr int kVecPerRow = BK / 8;     // 16-byte vectors per slab row
  constexpr int kVec = BM * kVecPerRow / kGroupThreads;  // vectors per thread per operand
  constexpr int kRed = 4 * 64 * 64;      // floats: 4 waves x 64 lanes x 64 accumulators
  static_assert(BM == BN && BM * kVecPerRow % kGroupThreads == 0, "slab vectors split evenly");
  static_assert(8 * kSlab * 2 >= kRed * 4 + BM * LDC * 2, "reduction and C staging fit");
  __shared__ __attribute__((aligned(16))) uint16_t lds[8 * kSlab];
  float* red = reinterpret_cast<float*>(lds);
  uint16_t* cst = lds + kRed * 2;

  const uint32_t tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const uint32_t grp = tc_uniform(tid >> 8);           // K group, wave-uniform
  const uint32_t gw = tc_uniform((tid >> 6) & 3);      // wave within the group
  const uint32_t gtid = tid & (kGroupThreads - 1);
  const uint32_t wm = gw >> 1, wn = gw & 1;
  const uint32_t nk = (a.K + BK - 1) / BK;
  const uint32_t niter = (nk + 1) / 2;                 // slabs per group, rounded up

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

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Vector v = gtid + 256 * s of a slab covers row v / kVecPerRow, k
    // columns 8 * (v % kVecPerRow) .. +7; rows and k past the matrix read
    // as zero.
    u32x4 ra[kVec], rb[kVec];
    auto fetch = [&](uint32_t kt) {
      const uint32_t k0 = kt * BK;
#pragma unroll
      for (int s = 0; s < kVec; ++s) {
        const uint32_t v = gtid + kGroupThreads * s;
        const uint32_t r = v / kVecPerRow, kc = k0 + (v % kVecPerRow) * 8;
        const bool kin = kc < a.K;
        ra[s] = (m0 + r < a.M && kin)
                    ? *reinterpret_cast<const u32x4*>(a.A + (uint64_t)(m0 + r) * a.lda + kc)
                    : u32x4{0, 0, 0, 0};
        rb[s] = (n0 + r < a.N && kin)
                    ? *reinterpret_cast<const u32x4*>(a.Bt + (uint64_t)(n0 + r) * a.K + kc)
                    : u32x4{0, 0, 0, 0};
      }
    };
    auto slab = [&](uint32_t buf) { return lds + (4 * grp + 2 * buf) * kSlab; };
    auto stash = [&](uint32_t buf) {
      uint16_t* As = slab(buf);
      uint16_t* Bs = As + kSlab;
#pragma unroll
      for (int s = 0; s < kVec; ++s) {
        const uint32_t v = gtid + kGroupThreads * s;
        const uint32_t r = v / kVecPerRow, c = (v % kVecPerRow) * 8;
        *reinterpret_cast<u32x4*>(As + r * LDA + c) = ra[s];
        *reinterpret_cast<u32x4*>(Bs + r * LDA + c) = rb[s];
      }
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
    __syncthreads();  // the previous tile's partial sums and C staging are no longer read
    if (grp < nk) {
      fetch(grp);
      stash(0);
    }
    __syncthreads();
    // Every wave passes the same barriers: a group without a slab in some
    // iteration (odd slab counts) skips the work, not the barrier.
    for (uint32_t it = 0; it < niter; ++it) {
      const uint32_t kt = 2 * it + grp, cur = it & 1;
      if (kt + 2 < nk) fetch(kt + 2);  // in flight while this slab is multiplied
      if (kt < nk) {
        // Operand fragment of one 16x16x32 block: lane l holds row (l % 16)
        // and 8 consecutive k values starting at 8 * (l / 16).  Both 32-wide
        // k steps' fragments are read first, then the 32 MFMAs run (the
        // scheduling barrier keeps the compiler from interleaving them back
        // into read-wait-multiply pairs); the other wave of the SIMD covers
        // this wave's LDS latency.
        const uint16_t* As = slab(cur);
        const uint16_t* Bs = As + kSlab;
        const uint32_t fr = lane & 15, fq = 8 * (lane >> 4);
        bf16x8 fa[2][4], fb[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            fa[h][i] = *reinterpret_cast<const bf16x8*>(As + (wm * 64 + i * 16 + fr) * LDA + 32 * h + fq);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            fb[h][j] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 64 + j * 16 + fr) * LDA + 32 * h + fq);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[h][j], fa[h][i], acc[i][j], 0, 0, 0);
      }
      // The other buffer was last read in the previous iteration, which every
      // wave finished before that iteration's closing barrier.
      if (kt + 2 < nk) stash(cur ^ 1);
      __syncthreads();
    }

    // Group 1's partial sums to LDS, in the same fragment order group 0's
    // wave of the same (wm, wn) holds them.
    if (grp == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<f32x4*>(red + ((gw * 16 + i * 4 + j) * 64 + lane) * 4) = acc[i][j];
    }
    __syncthreads();
    // Group 0 adds them and stages the tile as bf16.  The MFMA takes the B
    // fragment as its first operand, so its output block is C transposed:
    // lane l holds row l % 16 and the 4 consecutive columns 4 * (l / 16) + e,
    // e = 0..3 -- one 8-byte write per block.
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 o = *reinterpret_cast<const f32x4*>(red + ((gw * 16 + i * 4 + j) * 64 + lane) * 4);
          const uint32_t r = wm * 64 + i * 16 + (lane & 15);
          const uint32_t c = wn * 64 + j * 16 + 4 * (lane >> 4);
          const uint32_t lo = f32_to_bf16_rne(acc[i][j][0] + o[0]) | (f32_to_bf16_rne(acc[i][j][1] + o[1]) << 16);
          const uint32_t hi = f32_to_bf16_rne(acc[i][j][2] + o[2]) | (f32_to_bf16_rne(acc[i][j][3] + o[3]) << 16);
          *reinterpret_cast<uint2*>(cst + r * LDC + c) = make_uint2(lo, hi);
        }
    }
    __syncthreads();
    // 128 rows x 16 vectors of 8 bf16: 4 vectors per thread, stored through
    // to memory at system scope, so that once they complete the tile is
    // visible everywhere and mark_ready needs no L2 write-back.  Lanes
    // outside the matrix get an offset past the buffer range and their
    // stores are dropped.
    const uint32_t rows_in = a.M - m0 < (uint32_t)BM ? a.M - m0 : (uint32_t)BM;
    const uint32_t cols_in = a.N - n0 < (uint32_t)BN ? a.N - n0 : (uint32_t)BN;
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
  if ((uint64_t)BM * ldc * 2 >= (1ull << 31))
    return fail(TC_EINVAL, "gemm: a 128-row tile of C must span less than 2 GiB (ldc < 2^23)");
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
