/*
 * tc.h -- C boundary of the triggered (gated) chunked all-gather for MI355X.
 *
 * One GPU stands in for P ranks: the P peers' buffers are P equal-sized
 * replica buffers in the GPU's HBM.  A producer kernel writes rank p's part
 * of replica p and marks each chunk of it ready; a copy-engine kernel on the
 * same GPU copies every ready chunk to the same offsets in every other
 * replica, in schedule order, and then adds 1 to that chunk's arrival
 * counter in the destination's gate table.
 *
 * Sources (page title -- section):
 *   [TP]  "Triggered Plans" (Iris documentation)
 *   [PR]  "Triggered SDMA Plans" (Iris pull request)
 *   [BAR] "Barrier: Signals Only" (pypto documentation)
 *
 * Conventions.
 *   - Every function returns int: TC_OK (0) or a negative TC_E* code.  After a
 *     failure, tc_last_error() returns a message for the calling thread.
 *   - "device" pointers are HIP device addresses; "host" pointers are ordinary
 *     process memory.  Streams are hipStream_t values passed as void*
 *     (NULL = the default stream).
 *   - All PODs are little-endian, with the layouts written below; the caller
 *     owns every buffer it passes in.
 *   - The library allocates no device memory of its own: the caller passes a
 *     workspace (sized by tc_plan_workspace_bytes).  A plan allocates only
 *     small pinned host words, its streams and its events.  The one
 *     exception is tc_plan_create_noalloc, whose workspace is a static
 *     device array of the library (for callers that cannot allocate).
 */
#ifndef TC_H
#define TC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TC_MAX_RANKS 16
#define TC_GATE_ROW_BYTES 64
/* A linear region moves at most 1 GiB; longer ranges are cut by the builders
 * ([TP] Model; Requirements and limits: the DMA packet that copies a byte
 * range holds its length in 30 bits). */
#define TC_LINEAR_MAX_BYTES (1ull << 30)
/* The first round is 1 and no gate is ever cleared, so one plan runs at most
 * 2^32 - 1 rounds ([TP] Gates and rounds). */
#define TC_ROUND_LIMIT 0xFFFFFFFFu

enum tc_status {
  TC_OK = 0,
  TC_EINVAL = -1,    /* bad argument: zero sizes, writers 0, n > rows, bad order */
  TC_EBOUNDS = -2,   /* a region outside the buffer, or outside its rank's rows */
  TC_EOVERLAP = -3,  /* two ranks send the same bytes ([TP] Requirements and limits) */
  TC_ENOMEM = -4,    /* workspace too small */
  TC_EHIP = -5,      /* a HIP runtime call failed (message names it) */
  TC_ESTATE = -6,    /* call out of order for the plan's state */
  TC_ETIMEOUT = -7,  /* wait() deadline passed; tc_plan_problems names the chunks */
  TC_EEXTRA = -8,    /* a chunk got more than writers marks this round */
  TC_EROUNDS = -9,   /* next_round() at round 2^32 - 1 */
  TC_ENODEV = -10,   /* no GPU visible */
  TC_ECORRUPT = -11  /* gate state no correct run can produce (arrival counts off) */
};

enum tc_plan_state_t {
  TC_STATE_READY = 0,   /* round r prepared, not started */
  TC_STATE_STARTED = 1, /* start() returned; marks and copies may be in flight */
  TC_STATE_DONE = 2,    /* wait() found every chunk delivered everywhere */
  TC_STATE_FAILED = 3,  /* extra marks or corrupt gates: only close() is allowed */
  TC_STATE_CLOSED = 4,
  TC_STATE_CLOSING = 5  /* close() found its copies queued behind another plan's */
};

/* Plan-creation flags. */
#define TC_CHECK_OWN_ROWS 1u   /* rank p's bytes must lie in [p*R, (p+1)*R), R = rows_per_rank_bytes */

/* ---------------------------------------------------------------- PODs */

/* A 2-D window of the base buffer ("base=out" in [TP] Model): rows x cols
 * elements of elem_bytes each, consecutive rows row_stride elements apart,
 * starting byte_offset bytes into every replica. */
typedef struct tc_view {
  uint64_t byte_offset;
  uint64_t rows;
  uint64_t cols;
  uint64_t row_stride;   /* elements; >= cols */
  uint32_t elem_bytes;
  uint32_t rsvd;
} tc_view;

/* One copy ([TP] Model: a byte range or a 2-D sub-window).  Normal form:
 * linear iff rows == 1, and then pitch == row_bytes <= 2^30; otherwise rows
 * rows of row_bytes bytes, pitch bytes apart (pitch > row_bytes). */
typedef struct tc_region {
  uint64_t offset;
  uint64_t rows;
  uint64_t row_bytes;
  uint64_t pitch;
} tc_region;

/* Regions delivered as one unit, in their order, with a single arrival per
 * peer, plus how many mark_ready calls finish it in a round ([TP] Model). */
typedef struct tc_chunk {
  uint32_t first_region;
  uint32_t num_regions;
  uint32_t writers;
  uint32_t rsvd;
} tc_chunk;

/* A 64-byte gate row ([TP] Gates and rounds: the fields ready, arrival and
 * the marks' count; the copy side opens on ready >= round).  As
 * reported by tc_plan_read_gates: in rank p's own table the row of its chunk
 * c holds ready (= the last round whose gate opened) and writers (cumulative
 * marks); in a peer q's table the same row holds arrival (= rounds delivered
 * to q).  Bytes 24..63 are zero.
 *
 * On the device the rows hold `ready` and `arrival`.  The writer count is
 * kept in TC_MARK_STRIPES counters per chunk, TC_MARK_STRIPE_BYTES apart, so
 * that the marks of many CTAs finishing together do not queue on one
 * address; a mark adds 1 to one of them.  The count is their sum and the
 * gate of round r is open when it reaches r * writers.  Nobody learns that
 * its mark was the last: the copy engine, which sums the stripes, stores r
 * into `ready` when it finds the gate open, before it signals the chunk.
 * tc_plan_read_gates reports the device words, with the writer counter as
 * the stripes' sum. */
typedef struct tc_gate_row {
  uint64_t ready;
  uint64_t arrival;
  uint64_t writers;
  uint64_t rsvd[5];
} tc_gate_row;

#define TC_MARK_STRIPES 8
#define TC_MARK_STRIPE_BYTES 128

/* What start() hands to kernels, by value ([TP] Model: handle = plan.start(),
 * passed to the producer).  Arrival row of rank src's chunk c in rank q's
 * table: gates + q*gate_stride + (chunk_base[src] + c) * 64.  Mark stripe s
 * of global chunk g: the uint64 at marks + (g*TC_MARK_STRIPES + s) *
 * TC_MARK_STRIPE_BYTES. */
typedef struct tc_handle {
  uint64_t gates;        /* device address of rank 0's gate table */
  uint64_t gate_stride;  /* bytes between consecutive ranks' gate tables */
  uint64_t writers;      /* device address of uint32 writers[G], by global chunk id */
  uint64_t marks;        /* device address of the mark stripes */
  uint32_t round;        /* this round, >= 1 */
  uint32_t nranks;       /* P */
  uint32_t chunk_base[TC_MAX_RANKS + 1]; /* [P] = total chunks G */
  uint32_t rsvd;
} tc_handle;

typedef struct tc_schedule tc_schedule;  /* opaque, host memory */
typedef struct tc_plan tc_plan;          /* opaque */

/* -------------------------------------------------------- schedules */

/* One chunk holding the whole view, completed by `writers` marks (one per
 * program that writes it, marked once each at its end) ([TP] Model: whole()).
 * Out: *out, freed with tc_schedule_free.  TC_EINVAL on a zero-size view,
 * row_stride < cols, a view whose last byte lies at 2^62 or beyond (every
 * builder checks its view so), or writers == 0. */
int tc_schedule_whole(const tc_view* view, uint32_t writers, tc_schedule** out);

/* n chunks, one per row block, completed in order ([TP] Model: chunks()).
 * Blocks follow the tensor_split rule: the first rows % n blocks hold one
 * extra row.  TC_EINVAL when n == 0, n > rows or writers == 0. */
int tc_schedule_chunks(const tc_view* view, uint32_t n, uint32_t writers, tc_schedule** out);

/* One region per bm x bn tile (clipped at the edges), consecutive producer
 * steps grouped tiles_per_chunk at a time; chunk k's writers = the number of
 * steps it holds ([TP] Model: tile_chunks()).  order[step] = the tile the
 * producer computes at that step (row-major tile index); NULL = row-major.
 * order_len must equal the tile count.  TC_EINVAL when order is not a
 * permutation, or on zero sizes. */
int tc_schedule_tile_chunks(const tc_view* view, uint32_t bm, uint32_t bn,
                            uint32_t tiles_per_chunk, const uint32_t* order,
                            uint32_t order_len, tc_schedule** out);

/* A hand-built schedule ([TP] Model: the builders are conveniences; a plan
 * accepts an arbitrary list of chunks).  chunks[k]
 * must cover regions[first_region .. first_region+num_regions) back to back
 * in order; regions are normalised and cut at 1 GiB like the builders'.
 * nchunks == 0 gives the empty schedule of a rank that sends nothing
 * ([TP] Requirements and limits).  TC_EINVAL on a malformed table or a
 * region whose last byte lies at 2^62 or beyond. */
int tc_schedule_from_arrays(const tc_chunk* chunks, uint32_t nchunks,
                            const tc_region* regions, uint32_t nregions, tc_schedule** out);

/* Appends src's chunks after dst's (the producer's first_chunk offset of
 * [TP] Model).  dst is modified in place. */
int tc_schedule_append(tc_schedule* dst, const tc_schedule* src);

/* Borrowed views of a schedule's tables, valid until it is modified or freed. */
int tc_schedule_get(const tc_schedule* s, const tc_chunk** chunks, uint32_t* nchunks,
                    const tc_region** regions, uint32_t* nregions);

void tc_schedule_free(tc_schedule* s);

/* The producer's step->tile map, for steps 0 .. tm*tn-1 into out[]: group_m
 * tile-rows are walked column by column before the next band (the grouped
 * order that [TP] Model's tile_of stands for; its body is elided there). */
int tc_order_grouped(uint32_t tm, uint32_t tn, uint32_t group_m, uint32_t* out);

/* ------------------------------------------------------------ plans */

typedef struct tc_plan_desc {
  uint32_t nranks;                     /* P, 1..TC_MAX_RANKS */
  uint32_t flags;                      /* TC_CHECK_OWN_ROWS */
  void* const* replicas;               /* P device pointers, 256-byte aligned */
  uint64_t buffer_bytes;               /* size of every replica */
  const tc_schedule* const* schedules; /* P entries; NULL = sends nothing */
  void* workspace;                     /* device memory, 256-byte aligned */
  uint64_t workspace_bytes;
  uint64_t rows_per_rank_bytes;        /* for TC_CHECK_OWN_ROWS */
  const uint32_t* cu_mask;             /* NULL = copy engine may use every CU */
  uint32_t cu_mask_words;
  uint32_t engine_ctas;                /* CTAs of 4 waves (the grid's last wave publishes the
                                          gates, the others copy); 0 = one wave per 150 KiB of
                                          delivered bytes per round (source bytes times the
                                          P - 1 receivers), at least one per piece up to 256
                                          plus the publisher, at most 16 waves per usable CU */
  uint64_t piece_bytes;                /* copy work unit, multiple of 256, <= 1 GiB; 0 = 8 KiB */
  uint64_t engine_backstop_us;         /* engine gives up after this long; 0 = 30 s */
} tc_plan_desc;

/* Workspace bytes a plan over these schedules needs (gate tables of P x G
 * rows of 64 B, descriptors, queue state).  piece_bytes as in the desc. */
int tc_plan_workspace_bytes(uint32_t nranks, const tc_schedule* const* schedules,
                            uint64_t piece_bytes, uint64_t* out_bytes);

/* The creation checks alone, on the host, with no GPU: region bounds, own
 * rows, cross-rank overlap ([TP] Requirements and limits: no byte may come
 * from two different ranks; a rank may list its own bytes twice), writers > 0. */
int tc_plan_validate(const tc_plan_desc* desc);

/* Creates a plan ([TP] Model: TriggeredPlan(ctx, out, schedule), with the
 * schedule-per-rank form of [PR] API).  Validates, lays out and zeroes the
 * workspace (gates start at zero), uploads the descriptors once (region sizes
 * are fixed at creation, [TP] The kernel author's contract), and creates the copy-engine
 * stream.  Round = 1, state READY.  The engine stream always has a hardware
 * queue of its own (it is created CU-masked: with cu_mask, or with every CU),
 * because the engine runs before the producer it waits for and streams that
 * share a hardware queue run their kernels in submission order.  For the same
 * reason a consumer kernel that waits on arrivals must be queued after the
 * producer work it depends on.
 * All-or-nothing ([TP] contract): on failure nothing is kept and *out = NULL.
 * The replicas and workspace must stay allocated, unmoved, until close.
 * Each replica (buffer_bytes) and the workspace (workspace_bytes) must lie in
 * one device allocation of the current device: a host pointer or a pointer of
 * another device gives TC_EINVAL, a size past the allocation's end TC_EBOUNDS.
 * Errors: TC_EINVAL, TC_EBOUNDS, TC_EOVERLAP, TC_ENOMEM, TC_EHIP, TC_ENODEV. */
int tc_plan_create(const tc_plan_desc* desc, tc_plan** out);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): tc_plan_create
 * without a caller-supplied workspace and without any allocation of device
 * or pinned host memory (no hipMalloc, hipHostMalloc or hipFree; the plan's
 * own bookkeeping lives on the C++ heap, and it creates its HIP events).
 * The workspace is a static device array of the library,
 * TC_NOALLOC_WORKSPACE_BYTES per device, that each device holds until the
 * process ends; the engine's abort word and the completion check's results
 * live in it too, and the host reads them back with copies.  desc is as for
 * tc_plan_create, with workspace = NULL and workspace_bytes = 0.  The array
 * keeps the previous plan's contents; the plan zeroes what it uses.  All
 * no-allocation plans of a device share the one array, so only one may be
 * open per device at a time: a second is refused (TC_ESTATE) rather than
 * left to race on it, and kernels still using a closed plan's handle race
 * with the next plan.  The plan is then used and closed like any other.
 * TC_ENOMEM when the plan's workspace (tc_plan_workspace_bytes) exceeds
 * TC_NOALLOC_WORKSPACE_BYTES; TC_EINVAL for a non-NULL workspace; otherwise
 * the errors of tc_plan_create. */
#define TC_NOALLOC_WORKSPACE_BYTES (32ull << 20)
int tc_plan_create_noalloc(const tc_plan_desc* desc, tc_plan** out);

/* Starts the round ([TP] Model: start()).  READY -> STARTED.  The copy
 * engine is launched on the plan's stream behind all work already queued on
 * `stream`, so reads of the previous round's data issued before start() are
 * not overwritten ([TP] The kernel author's contract: copies may overwrite a
 * peer's buffer once it has moved on to the next round); *out receives the
 * handle for producer and consumer kernels.
 * `stream` is the producer's stream; it may not be the legacy default stream
 * (NULL), which waits for every blocking stream and so for the engine.
 * Between start() and the launch of the producer nothing may wait for the
 * whole device (the engine is waiting for that producer).
 * TC_ESTATE unless READY; TC_EINVAL for the legacy default stream. */
int tc_plan_start(tc_plan* plan, void* stream, tc_handle* out);

/* The current round's handle without starting the round (state READY or
 * STARTED): for producers that write their data before start() and mark it
 * after (the deferred-mark mode of tc_produce_fill / tc_mark_all). */
int tc_plan_handle(const tc_plan* plan, tc_handle* out);

/* Blocks until every chunk is delivered everywhere ([TP] Model: wait()):
 * waits for the work queued so far on start()'s stream (the producers, so
 * that every mark is counted) and for the copy engine, then has the
 * completion check run ([TP] Gates and rounds): by the engine's last wave
 * when the request reaches it soon after the last chunk is signalled, else
 * by the check kernel.  Work queued on start()'s stream after the producers
 * (consumers, say) delays the check until it ends: queue such work on
 * another stream, behind an event recorded after the producers.
 *   TC_OK       STARTED -> DONE.
 *   TC_EEXTRA   a chunk got more than writers marks; state FAILED.
 *   TC_ETIMEOUT timeout_us passed; the copy engine is stopped, state stays
 *               STARTED, tc_plan_problems names the short chunks, and a
 *               later wait() (after the missing marks) resumes the round.
 *   TC_ECORRUPT arrival counts no correct run can produce; state FAILED.
 *   TC_ESTATE   not STARTED. */
int tc_plan_wait(tc_plan* plan, uint64_t timeout_us);

/* Tells the plan this round's data has been read ([TP] The kernel author's
 * contract: after next_round() peers may overwrite it).  DONE -> READY,
 * round + 1.  TC_ESTATE unless DONE; TC_EROUNDS at round 2^32 - 1. */
int tc_plan_next_round(tc_plan* plan);

/* Closes the plan ([TP] Model: close / leaving the with block; The kernel
 * author's contract: prepared copies cannot be withdrawn, so closing a plan
 * in the middle of a round, or before it starts, sends each rank's chunks as
 * they stand).  Safe in any state.  STARTED (or CLOSING) and READY: every
 * gate of the plan is forced open and the copy engine delivers every chunk
 * with whatever bytes it holds when its copy runs (the engine is launched
 * for a READY round, and run again after a timeout); DONE and FAILED: there
 * is nothing left to send.  Then its streams, events and host words are
 * freed; the caller's buffers keep what was delivered.
 * Plans with the same CU mask share one engine stream, so their rounds run
 * in start() order, and a plan whose engine is queued behind another plan's
 * waiting engine cannot finish first.  With closing != NULL, close() waits
 * for the engine as long as every earlier plan's unfinished engine on the
 * stream can finish by itself (all its gates open, or forced); once one
 * waits on shut gates, close() returns TC_OK with *closing = 1 and the plan
 * CLOSING (still valid): closing the earlier plan lets it finish, and a
 * later tc_plan_close frees it.  Otherwise (*closing = 0) the plan is freed.
 * With closing == NULL the call just waits for the engine.  TC_ETIMEOUT when
 * the engine does not stop within 10 s (the plan is then leaked, not
 * freed). */
int tc_plan_close(tc_plan* plan, int* closing);

/* The plan's state and current round ([TP] Model: a round is start(), the
 * producer's marks, wait(); Gates and rounds: rounds start at 1 and grow by
 * one per next_round(); The kernel author's contract: a plan with extra
 * marks is FAILED and only closes, and a close() queued behind an earlier
 * plan's waiting copies leaves the plan CLOSING).  Either output may be
 * NULL.  TC_EINVAL for a NULL plan. */
int tc_plan_state(const tc_plan* plan, int* state, uint32_t* round);

/* The chunks the last wait() found wrong ([TP] The kernel author's
 * contract, item 2: wait() raises when a chunk got extra marks, and a
 * timeout names the chunks still short).  After TC_EEXTRA: the chunks with
 * extra marks; after TC_ETIMEOUT: the chunks not marked by all their writers
 * or not yet arrived at every peer; after TC_ECORRUPT: the chunks whose rows
 * hold impossible counts; empty after TC_OK.  Up to cap (rank, chunk) pairs,
 * as rank_chunk[2i], rank_chunk[2i+1] (host, may be NULL with cap 0);
 * *n = the total number. */
int tc_plan_problems(const tc_plan* plan, uint32_t* rank_chunk, uint32_t cap, uint32_t* n);

/* Synchronous snapshot of all gate tables ([TP] Gates and rounds): P x G x
 * 64 bytes into host, rows as tc_gate_row describes (ready and arrival as
 * stored on the device, writers = the sum of the chunk's mark stripes).
 * TC_EINVAL when bytes < P * G * 64. */
int tc_plan_read_gates(tc_plan* plan, void* host, uint64_t bytes);

/* Synchronous snapshot of the queue cursors ([TP] The kernel author's
 * contract, item 1: a rank's copies to one peer share one queue and complete
 * strictly in schedule order, so how far a queue has got is one number):
 * host[p*P + q] = chunks of rank p delivered to rank q so far this round
 * (0 on the diagonal), P x P uint32 in host memory. */
int tc_plan_read_cursors(tc_plan* plan, uint32_t* host);

/* Per-round figures of the copy side, for benchmarks ([TP] opening
 * paragraph: the copy side moves each chunk to every peer and signals its
 * arrival there; Model: a round is one use of the plan).  Reads the last
 * engine launch's events and counters (synchronously, after wait()). */
typedef struct tc_stats {
  float engine_ms;         /* last copy-engine launch, HIP events on its stream */
  uint32_t launches;       /* copy-engine launches this round (1 + resumes) */
  uint32_t engine_ctas;
  uint64_t window_ticks;   /* first gate seen open -> last arrival, 100 MHz ticks */
  uint64_t bytes_moved;    /* bytes written to peers per round: sum over chunks of (P-1)*size */
  uint64_t bytes_read;     /* bytes the engine reads per round (each chunk once) */
  uint64_t pieces;         /* copy work units per round */
  uint32_t G;              /* total chunks */
  uint32_t engine_checked; /* 1: the last wait()'s completion check ran inside the copy
                              engine; 0: the check kernel ran it */
} tc_stats;

int tc_plan_stats(tc_plan* plan, tc_stats* out);

/* The copy engine's stream (hipStream_t), for timing kernels on it with
 * events: the engine is the plan's copy side ([TP] opening paragraph). */
int tc_plan_engine_stream(tc_plan* plan, void** stream);

/* Test hook: set the round of a DONE plan, to exercise the round limit
 * without 2^32 rounds ([TP] Gates and rounds: gates are never reset, so a
 * plan runs at most 2^32 - 1 rounds).  TC_ESTATE unless DONE or round 0. */
int tc_plan_debug_set_round(tc_plan* plan, uint32_t round);

/* ------------------------------------------------ synthetic producers */

/* Value kinds written by tc_produce_fill: element index i of rank p's view
 * in round r holds h = mix64((p<<48 | r<<32 | i) ^ mix64(seed)) (SplitMix64's
 * output function):  U32 = low 32 bits;  U8 = low 8 bits;  BF16 = uniform
 * [-1,1): u = h>>41, f = (u - 2^22) * 2^-22, the high 16 bits of f. */
enum { TC_FILL_U32 = 0, TC_FILL_BF16 = 1, TC_FILL_U8 = 2 };
/* Mark modes: INKERNEL marks each chunk after writing it ([TP] Memory
 * ordering: mark_ready); NONE writes only (deferred marks: tc_mark_all). */
enum { TC_MARK_INKERNEL = 0, TC_MARK_NONE = 1 };
/* Fill modes.  A writer slot is one (rank, chunk, writer j): its CTA writes
 * the j-th share of the chunk's bytes, then marks the chunk once.
 *   PARALLEL: one CTA per writer slot, chunks of a rank in schedule order.
 *   SERIAL:   one CTA per rank walks its chunks in order[] and, for each,
 *             writes its writers' shares one after another, marking after
 *             each.
 *   WAVES:    a persistent grid of `ctas` CTAs takes the writer slots in
 *             waves, every rank's chunk 0 first, then every rank's chunk 1,
 *             ...; CTA i takes slots i, i + ctas, ...  Chunks complete a few
 *             at a time, so the copy engine can deliver early chunks while
 *             later ones are still produced ([TP] Model: a schedule lists
 *             chunks in the order the producer completes them).
 *   ONESHOT:  one CTA per 16 KiB block of every writer's share, blocks in
 *             the WAVES order, stores written through to memory; the last
 *             block of a share to finish issues that writer's mark.  Only
 *             for plans whose every chunk is one byte range, with fewer
 *             than 2^31 blocks, and for contiguous views (else TC_EINVAL).
 *             A deferred-mark (TC_MARK_NONE) one-shot fill counts nothing. */
enum { TC_FILL_PARALLEL = 0, TC_FILL_SERIAL = 1, TC_FILL_WAVES = 2, TC_FILL_ONESHOT = 3 };

typedef struct tc_fill_desc {
  const tc_view* views;   /* host array of P views: rank p's part of the buffer */
  uint64_t seed;
  uint32_t kind;          /* TC_FILL_* ; elem_bytes of the views must match */
  uint32_t mark_mode;     /* TC_MARK_* */
  uint32_t mode;          /* TC_FILL_PARALLEL / SERIAL / WAVES / ONESHOT */
  uint32_t rsvd;
  const uint32_t* order;  /* device, [P][max_chunks] when SERIAL; NULL = schedule order */
  uint32_t order_stride;  /* entries per rank in order[], at least a rank's chunk count */
  uint32_t ctas;          /* WAVES: persistent grid size (0 = two CTAs per CU); else 0 */
} tc_fill_desc;

/* Hash-fill producer for every rank's chunks of `plan`, on `stream`.
 * Writes replica p only (rank p's regions).  With TC_MARK_INKERNEL the plan
 * must be STARTED; with TC_MARK_NONE it may also be READY (data written
 * before start(), marked after it).  TC_EINVAL on a kind / view / order
 * mismatch or an order array that is not device memory of the plan's
 * device; TC_EBOUNDS when P * order_stride words run past its allocation;
 * TC_ESTATE when h is not the plan's current round. */
int tc_produce_fill(tc_plan* plan, const tc_handle* h, const tc_fill_desc* d, void* stream);

/* Deferred marks: every chunk of every rank receives exactly its writers'
 * marks, one CTA per mark, on `stream`.  The plan may be READY or STARTED
 * (marks that precede start() simply find the engine's gates open). */
int tc_mark_all(tc_plan* plan, const tc_handle* h, void* stream);

/* `count` marks of rank `rank`'s chunk `chunk`, one CTA each, on `stream`
 * (stepped completion orders; misuse tests with extra marks). */
int tc_mark(tc_plan* plan, const tc_handle* h, uint32_t rank, uint32_t chunk,
            uint32_t count, void* stream);

/* Persistent bf16 GEMM producer ([TP] Model, the tiled-kernel example):
 * C[M,N] = A[M,K] * B with B given as Bt[N,K] (K contiguous), bf16 in, fp32
 * accumulate, bf16 out (round to nearest even), C row stride ldc elements.
 * 128x128 tiles; program p handles the steps s with s % programs == p; step s computes
 * tile tc_tile_of(s, tm, tn, group_m) and, when h != NULL, then marks chunk
 * first_chunk + s / tiles_per_chunk of rank `rank`.  When programs is a
 * multiple of 8, consecutive programs run on one XCD (workgroups are dealt
 * to the XCDs round-robin), so each XCD's L2 serves a compact block of
 * tiles.  A, Bt, C device.
 * C is stored with system-scope write-through stores, so its marks need no
 * L2 write-back (tc_mark_ready_wt).
 * TC_EINVAL unless K % 8 == 0, N % 8 == 0, ldc % 8 == 0, ldc < 2^23, pointers
 * 16-byte aligned, and A, Bt, C device memory of the current device;
 * TC_EBOUNDS when A ((M - 1) * K + K elements), Bt (N * K) or C
 * ((M - 1) * ldc + N) runs past the end of its allocation. */
int tc_gemm_bf16(const void* A, const void* Bt, void* C, uint32_t M, uint32_t N, uint32_t K,
                 uint64_t ldc, uint32_t programs, uint32_t group_m, const tc_handle* h,
                 uint32_t rank, uint32_t first_chunk, uint32_t tiles_per_chunk, void* stream);

/* Device-view consumer ([TP] Memory ordering, consumer side; contract item
 * 5): one CTA per chunk of every rank; each waits with tc_wait (dst = the
 * given rank, at most max_polls polls) and then copies the chunk's bytes from
 * replica dst into out_buf at the same offsets.  status[g] (device, one u32
 * per global chunk) = 1 when it arrived and was copied, 2 when polls ran out.
 * out_buf (buffer_bytes) and status (G words) must be device memory of the
 * plan's device within their allocations (TC_EINVAL, TC_EBOUNDS). */
int tc_consume_copy(tc_plan* plan, const tc_handle* h, uint32_t dst, void* out_buf,
                    uint32_t max_polls, uint32_t* status, void* stream);

/* Row dependencies of a consumer that reads the rows of `view` (relative to
 * the plan's buffer, in every replica) in blocks of tile_rows: for row block
 * b, the (src, chunk) pairs whose regions reach into rows [b * tile_rows,
 * (b + 1) * tile_rows), conservatively (every row between a piece's first
 * and last byte).  Host output, CSR: start[nblocks + 1] and pairs[2 * npairs]
 * = (src, local chunk), a rank's own chunks included.  With start == pairs
 * == NULL only *nblocks and *npairs are set (size query); otherwise
 * pairs_cap counts pairs.  TC_EINVAL on a bad view or short arrays. */
int tc_plan_row_deps(const tc_plan* plan, const tc_view* view, uint32_t tile_rows, uint32_t* start,
                     uint32_t* pairs, uint32_t pairs_cap, uint32_t* nblocks, uint32_t* npairs);

/* In-kernel consumer of the gathered rows ([TP] Memory ordering, consumer
 * side; the step after the gather): Y[M,N] = X[M,K] * W, W given as Wt[N,K],
 * bf16 in, fp32 accumulate, bf16 out, as tc_gemm_bf16.  X is rank dst's
 * replica of the gathered view (device, row stride ldx elements).  Before a
 * step reads its 128-row block b of X, the CTA waits (tc_wait: at most
 * max_polls polls per chunk) for the pairs dep_pairs[2 d], d in
 * [dep_start[b], dep_start[b + 1]) -- device copies of tc_plan_row_deps with
 * tile_rows = 128.  status (device, one u32 per row block, may be NULL) gets
 * 2 where a wait ran out of polls; the block is then computed from whatever
 * the rows hold.  Queue it behind its rank's producers on their stream (or
 * on any stream after they are queued): HIP maps streams onto a few hardware
 * queues, so a consumer queued ahead of its producer on another stream may
 * share that producer's hardware queue and block it until the polls run
 * out; and on one GPU the simulated ranks share the CUs, so waiting CTAs
 * hold CUs the producers need.
 * TC_EINVAL / TC_EBOUNDS as tc_gemm_bf16 (with X spanning (M - 1) * ldx + K
 * elements), and for dep_start (nblocks + 1 words) and status (nblocks
 * words) likewise; TC_EINVAL for dst >= nranks or max_polls == 0. */
int tc_gemm_consume_bf16(const tc_handle* h, uint32_t dst, const uint32_t* dep_start,
                         const uint32_t* dep_pairs, uint32_t max_polls, uint32_t* status,
                         const void* X, uint64_t ldx, const void* Wt, void* Y, uint32_t M,
                         uint32_t N, uint32_t K, uint64_t ldy, uint32_t programs,
                         uint32_t group_m, void* stream);

/* ------------------------------------------------------------ barrier */

/* Dedicated-row notify/wait barrier ([BAR] The idea; Walkthrough): one CTA
 * per simulated rank m (P <= TC_MAX_RANKS) runs generations g = first_gen ..
 * first_gen + n_gen - 1; in each it adds 1 to W[q][m] for every q != m
 * (release), then waits until W[m][s] >= g for every s != m (acquire),
 * polling at most max_polls times per cell.  W: device int32 [P][P], zeroed
 * by the caller before generation 1.  Optional device outputs (NULL = off):
 *   x    int32 [2][P]: rank m stages (g << 8) | m in x[g % 2][m] before its
 *        notifies;
 *   y    int32 [n_gen][P]: after the waits, y[g - first_gen][m] =
 *        x[g % 2][(m + 1) % P] (the data reveal: y[r] = x[(r+1) % N]);
 *   snap int32 [n_gen][P][P]: rank m's row W[m][*] right after its waits.
 * status: device u32, set to 1 + rank when a wait ran out of polls (the
 * kernel still exits).  Asynchronous on `stream`.  Every array given must be
 * device memory of the current device spanning its size (TC_EINVAL,
 * TC_EBOUNDS). */
int tc_barrier_run(int32_t* W, uint32_t P, uint32_t first_gen, uint32_t n_gen,
                   int32_t* x, int32_t* y, int32_t* snap, uint32_t max_polls,
                   uint32_t* status, void* stream);

/* ------------------------------------------------------------- misc */

/* Releases what the library keeps for the life of the process: the copy
 * engines' CU-masked streams (one per device and CU mask, shared by plans;
 * the plan's engine of [TP] Model and opening paragraph).  Call it after the
 * last plan is closed and before the HIP runtime shuts down (the Python
 * binding does so at interpreter exit), so that no stream outlives the
 * runtime's own teardown.  Later plans create streams again.  TC_ESTATE while
 * any plan is open (nothing is released then); TC_EHIP when a stream cannot
 * be destroyed. */
int tc_release(void);

const char* tc_last_error(void);
const char* tc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TC_H */
