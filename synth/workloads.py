"""The synthetic workloads, by shape (data only, no method arithmetic).

Every rank p owns rows [p*rows, (p+1)*rows) of an ``out`` buffer of
``P*rows`` rows; each of the P replicas is one copy of that buffer.  The
replicas start at the 0xA5 sentinel.

Geometry fields: ``P`` ranks; per-rank ``rows`` x ``cols`` elements of
``elem`` (value kind: "u32", "bf16", "u8"); ``stride`` (elements, default
cols); ``builder`` one of whole / chunks / tile_chunks with its arguments;
``writers`` per chunk (whole, chunks); ``rounds``.
"""

# Five named workloads at their full sizes.
FULL = {
    # P=2 bf16 [2*256, 256]; chunks() = 4 row blocks of 64 rows, 1 writer
    # each; 3 rounds with a per-round seed (stale-data check).
    "bf16_chunks_p2": dict(P=2, rows=256, cols=256, elem="bf16", builder="chunks",
                           n=4, writers=1, rounds=3),
    # P=4 bf16 GEMM producer M=N=2000, K=1024; 128x128 tiles, 256 programs,
    # GROUP_M=8 step order, tile_chunks with 256 tiles per chunk; 5 rounds.
    "gemm_tiles_p4": dict(P=4, rows=2000, cols=2000, elem="bf16", builder="tile_chunks",
                          bm=128, bn=128, tiles_per_chunk=256, group_m=8,
                          K=1024, programs=256, rounds=5),
    # P=8 whole(): one 4 MiB chunk of u32 per rank written by 8 CTAs; 10
    # rounds; in round 7 rank 3 marks its chunk once more than its writers.
    "u32_whole_p8": dict(P=8, rows=1, cols=1 << 20, elem="u32", builder="whole",
                         writers=8, rounds=10, extra_round=7, extra_rank=3),
    # P=4 large 1D: u32 [786432, 512] per rank (1.5 GiB) as chunks() of 3
    # blocks of 0.5 GiB, 64 writers each; 3 rounds.
    "u32_chunks_1p5g_p4": dict(P=4, rows=786432, cols=512, elem="u32", builder="chunks",
                               n=3, writers=64, rounds=3),
    # The same buffers as one whole() chunk split into 1 GiB + 0.5 GiB
    # regions, 192 writers; 3 rounds.
    "u32_whole_1p5g_p4": dict(P=4, rows=786432, cols=512, elem="u32", builder="whole",
                              writers=192, rounds=3),
    # P=8 2-D tiles completed in a shuffled (non-schedule) order: u32
    # [200, 300] per rank, 64x64 tiles (clipped), 4 tiles per chunk, one
    # producer CTA per rank; 3 rounds.
    "u32_tiles_shuffled_p8": dict(P=8, rows=200, cols=300, elem="u32", builder="tile_chunks",
                                  bm=64, bn=64, tiles_per_chunk=4, serial=True,
                                  shuffled=True, rounds=3),
    # P=8 signal-only barrier on an int32 [P, P] window, 1000 generations.
    "barrier_p8": dict(P=8, gens=1000),
}

# Small cases the oracle finishes in seconds: several tiles, ragged tails,
# unaligned pitches and offsets.
SMALL = {
    "u32_chunks_ragged_p3": dict(P=3, rows=37, cols=100, elem="u32", builder="chunks",
                                 n=5, writers=2, rounds=3),
    "bf16_tiles_ragged_p4": dict(P=4, rows=77, cols=90, elem="bf16", builder="tile_chunks",
                                 bm=32, bn=32, tiles_per_chunk=3, group_m=2, rounds=3),
    "u8_tiles_odd_p2": dict(P=2, rows=13, cols=29, stride=31, elem="u8", builder="tile_chunks",
                            bm=4, bn=8, tiles_per_chunk=2, rounds=2),
    "u32_whole_p5": dict(P=5, rows=64, cols=64, elem="u32", builder="whole",
                         writers=3, rounds=4),
    "u32_tiles_shuffled_p3": dict(P=3, rows=40, cols=50, elem="u32", builder="tile_chunks",
                                  bm=16, bn=16, tiles_per_chunk=2, serial=True,
                                  shuffled=True, rounds=3),
}

ALL = {**FULL, **SMALL}
