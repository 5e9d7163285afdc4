/*
 * Seeded values of the synthetic producers, oracle side, in plain C.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/ (and nothing in the product path)
 * to check every element of the largest workloads, whose blocks are too big
 * for the NumPy oracle to regenerate within a test's time.  It is the same
 * definition as oracle/values.py, written again here:
 *
 *   k = rank * 2^48 + round * 2^32 + index
 *   h = mix64(k XOR mix64(seed))
 *
 * mix64 is the output function of SplitMix64 (Steele, Lea & Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014; constants of
 * Vigna's public-domain splitmix64.c).  The u32 pattern is the low 32 bits
 * of h.  The pages fix no input data; their tests only ask that each round
 * writes values distinct from the round before ("Triggered SDMA Plans",
 * Testing: the stale-data check over several epochs).
 *
 * Pins (tests/test_oracle_pins.py): the generator reproduces the published
 * splitmix64.c output for seed 1234567, and the pattern equals the NumPy
 * oracle's on random indices.  Shares no code with the HIP library.
 */
#include <pthread.h>
#include <stdint.h>

static uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* The SplitMix64 generator: the state advances by the golden gamma, and
 * each output is mix64 of the new state. */
void oracle_splitmix64_stream(uint64_t seed, uint64_t n, uint64_t* out) {
  uint64_t state = seed;
  for (uint64_t i = 0; i < n; ++i) {
    state += 0x9E3779B97F4A7C15ull;
    out[i] = mix64(state);
  }
}

typedef struct {
  uint64_t salt, key0, n;
  uint32_t* out;
} span_t;

static void* fill_span(void* arg) {
  const span_t* s = (const span_t*)arg;
  for (uint64_t i = 0; i < s->n; ++i) s->out[i] = (uint32_t)mix64((s->key0 + i) ^ s->salt);
  return 0;
}

/* out[i] = the u32 pattern of element first + i of rank `rank`'s block in
 * round `rnd`, for i < n, computed by `threads` threads (at most 64) over
 * equal spans.  Returns 0, or -1 when the key layout cannot hold the
 * arguments (rank or round >= 2^16, index >= 2^32). */
int oracle_u32_pattern(uint64_t seed, uint32_t rank, uint32_t rnd, uint64_t first, uint64_t n,
                       uint32_t* out, uint32_t threads) {
  if (rank >= (1u << 16) || rnd >= (1u << 16) || first + n > (1ull << 32)) return -1;
  const uint64_t salt = mix64(seed);
  const uint64_t key0 = ((uint64_t)rank << 48) | ((uint64_t)rnd << 32) | first;
  if (threads < 1) threads = 1;
  if (threads > 64) threads = 64;
  span_t spans[64];
  pthread_t tid[64];
  uint32_t started = 0;
  for (uint32_t t = 0; t < threads; ++t) {
    const uint64_t lo = n * t / threads, hi = n * (t + 1) / threads;
    spans[t].salt = salt;
    spans[t].key0 = key0 + lo;
    spans[t].n = hi - lo;
    spans[t].out = out + lo;
    if (t + 1 < threads && pthread_create(&tid[t], 0, fill_span, &spans[t]) == 0) {
      ++started;
      continue;
    }
    if (t + 1 < threads) {  /* no thread: do the span here */
      fill_span(&spans[t]);
      tid[t] = 0;
      continue;
    }
    fill_span(&spans[t]);
  }
  for (uint32_t t = 0; t + 1 < threads; ++t)
    if (tid[t]) pthread_join(tid[t], 0);
  (void)started;
  return 0;
}
