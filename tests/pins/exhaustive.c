/*
 * Exhaustive pins of the CPU oracle, run by tests/test_oracle_pins.py.
 *
 * Each check compares the oracle with a formulation that shares nothing
 * with it:
 *   rne     oracle_bf16_rne(f) against the integer carry form
 *           (f + 0x7FFF + ((f >> 16) & 1)) >> 16 with a NaN branch, over all
 *           2^32 F32 patterns;
 *   sum     oracle_sum2_f32(a, b) against (float)((double)a + (double)b),
 *           over all 2^32 BF16 pairs.  Double rounding through binary64 is
 *           innocuous for a binary32 sum because 53 >= 2*24 + 2 (Figueroa,
 *           "When is double rounding innocuous?", SIGNUM 1995);
 *   comm    oracle_sum2_f32(a, b) == oracle_sum2_f32(b, a) bit for bit,
 *           over all 2^32 BF16 pairs.
 * Prints the mismatch count and the first mismatch.  Multi-threaded only to
 * keep the CPU suite short; each thread takes a contiguous share.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static int mode;
static int n_threads = 8;

typedef struct {
  uint64_t lo, hi;
  uint64_t bad;
  uint64_t first;
} job;

static uint16_t carry_rne(uint32_t f) {
  if ((f & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (uint16_t)((f + 0x7FFFu + ((f >> 16) & 1u)) >> 16);
}

static uint32_t double_sum(uint16_t a, uint16_t b) {
  uint32_t ab = (uint32_t)a << 16, bb = (uint32_t)b << 16;
  float fa, fb;
  memcpy(&fa, &ab, 4);
  memcpy(&fb, &bb, 4);
  float s = (float)((double)fa + (double)fb);
  uint32_t r;
  memcpy(&r, &s, 4);
  if ((r & 0x7FFFFFFFu) > 0x7F800000u) r = 0x7FC00000u;
  return r;
}

static void *run(void *arg) {
  job *j = (job *)arg;
  for (uint64_t x = j->lo; x < j->hi; ++x) {
    uint32_t v = (uint32_t)x;
    int ok;
    if (mode == 0) {
      ok = oracle_bf16_rne(v) == carry_rne(v);
    } else if (mode == 1) {
      ok = oracle_sum2_f32((uint16_t)(v >> 16), (uint16_t)v) == double_sum((uint16_t)(v >> 16), (uint16_t)v);
    } else {
      ok = oracle_sum2_f32((uint16_t)(v >> 16), (uint16_t)v) == oracle_sum2_f32((uint16_t)v, (uint16_t)(v >> 16));
    }
    if (!ok) {
      if (!j->bad) j->first = x;
      ++j->bad;
    }
  }
  return NULL;
}

int main(int argc, char **argv) {
  if (argc < 2) return 2;
  if (!strcmp(argv[1], "rne")) mode = 0;
  else if (!strcmp(argv[1], "sum")) mode = 1;
  else if (!strcmp(argv[1], "comm")) mode = 2;
  else return 2;
  if (argc > 2) n_threads = atoi(argv[2]);
  if (n_threads < 1 || n_threads > 64) return 2;
  const uint64_t total = 1ull << 32;
  pthread_t th[64];
  job jobs[64];
  for (int t = 0; t < n_threads; ++t) {
    jobs[t].lo = total * t / n_threads;
    jobs[t].hi = total * (t + 1) / n_threads;
    jobs[t].bad = 0;
    jobs[t].first = 0;
    pthread_create(&th[t], NULL, run, &jobs[t]);
  }
  uint64_t bad = 0, first = 0;
  for (int t = 0; t < n_threads; ++t) {
    pthread_join(th[t], NULL);
    if (jobs[t].bad && !bad) first = jobs[t].first;
    bad += jobs[t].bad;
  }
  printf("%s mismatches %llu first 0x%08llx\n", argv[1], (unsigned long long)bad, (unsigned long long)first);
  return bad ? 1 : 0;
}
