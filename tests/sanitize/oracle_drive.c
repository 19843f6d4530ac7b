/*
 * Drives every function of the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer, on seeded small inputs: the statuses are
 * checked where the oracle's header fixes them, plus invariants that hold
 * whatever the arithmetic (round trips, permutations, guard bytes around
 * every output left untouched).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "CHECK failed: %s (line %d)\n", #c, __LINE__);          \
      exit(1);                                                                \
    }                                                                         \
  } while (0)

static uint64_t g_s = 0x0A11CE5EEDull;
static uint64_t next(void) { /* SplitMix64 */
  uint64_t z = (g_s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static uint64_t below(uint64_t n) { return n ? next() % n : 0; }

enum { GUARD = 64 };
/* A buffer with GUARD bytes of 0xC3 on each side; returns the inside. */
static uint8_t *guarded(size_t n) {
  uint8_t *p = malloc(n + 2 * GUARD);
  CHECK(p);
  memset(p, 0xC3, n + 2 * GUARD);
  return p + GUARD;
}
static void check_guards(uint8_t *in, size_t n) {
  for (size_t k = 0; k < GUARD; ++k) CHECK(in[-1 - (long)k] == 0xC3 && in[n + k] == 0xC3);
}
static void release(uint8_t *in) { free(in - GUARD); }

static void numbers(void) {
  for (int it = 0; it < 200000; ++it) {
    const uint32_t f = (uint32_t)next(), g = (uint32_t)next();
    (void)oracle_bf16_rne(f);
    CHECK(oracle_sum2_f32((uint16_t)f, (uint16_t)g) == oracle_sum2_f32((uint16_t)g, (uint16_t)f) ||
          ((f & 0x7F80u) == 0x7F80u) || ((g & 0x7F80u) == 0x7F80u));
    (void)oracle_sum2_f32_f32(f, g);
  }
  for (int it = 0; it < 300; ++it) {
    const size_t n = below(3000);
    const size_t ce = 8 * (1 + below(40));
    const size_t R = 1 + below(4);
    const size_t n_chunks = n ? (n + ce - 1) / ce : 0;
    const size_t b = below(n_chunks + 1), e = b + below(R + 1);
    float *src = (float *)guarded(n * 4 + 4);
    for (size_t i = 0; i < n; ++i) ((uint32_t *)src)[i] = (uint32_t)next();
    uint16_t *ring = (uint16_t *)guarded(R * ce * 2);
    (void)oracle_pack(src, n, ring, R * ce, ce, b, e);
    check_guards((uint8_t *)ring, R * ce * 2);
    uint16_t *a = (uint16_t *)guarded(n * 2 + 2), *bb = (uint16_t *)guarded(n * 2 + 2);
    for (size_t i = 0; i < n; ++i) { a[i] = (uint16_t)next(); bb[i] = (uint16_t)next(); }
    uint8_t *out = guarded(n * 4 + 4);
    CHECK(oracle_combine2(a, bb, n, out, 0) == ORACLE_OK);
    check_guards(out, n * 4);
    CHECK(oracle_combine2(a, bb, n, out, 1) == ORACLE_OK);
    CHECK(oracle_combine2_f32(src, src, n, out, (int)below(2)) == ORACLE_OK);
    check_guards(out, n * 4);
    release((uint8_t *)src); release((uint8_t *)ring); release((uint8_t *)a); release((uint8_t *)bb); release(out);
  }
}

static void argmax(void) {
  for (int it = 0; it < 300; ++it) {
    const uint32_t rows = 1 + (uint32_t)below(12), n0 = 1 + (uint32_t)below(700), n1 = 1 + (uint32_t)below(700);
    const size_t ld = n0 + n1 + below(9);
    uint16_t *m = (uint16_t *)guarded((size_t)rows * ld * 2);
    for (size_t i = 0; i < (size_t)rows * ld; ++i) {
      uint16_t v = (uint16_t)next();
      if ((v & 0x7F80u) == 0x7F80u && (v & 0x7Fu)) v &= 0xBFFFu; /* no NaN */
      m[i] = v;
    }
    const oracle_shard s0 = {m, ld, rows, n0, 0}, s1 = {m + n0, ld, rows, n1, n0};
    const int mode = (int)below(2);
    uint8_t *out = guarded((size_t)rows * 16);
    CHECK(oracle_argmax_merge(&s0, &s1, mode, out) == ORACLE_OK);
    check_guards(out, (size_t)rows * (mode ? 16 : 8));
    if (mode == 0)
      for (uint32_t r = 0; r < rows; ++r) {
        const oracle_max_idx *rec = (const oracle_max_idx *)out + r;
        CHECK(rec->idx >= 0 && (uint32_t)rec->idx < n0 + n1);
      }
    m[(size_t)(rows - 1) * ld + below(n0)] = 0x7FC1; /* a NaN is refused */
    CHECK(oracle_argmax_merge(&s0, &s1, mode, out) == ORACLE_ENAN);
    release((uint8_t *)m);
    release(out);
  }
}

static void runs(void) {
  for (int it = 0; it < 300; ++it) {
    const uint32_t L = 1 + (uint32_t)below(20), B = 1 + (uint32_t)below(30);
    const uint64_t seg = 16 * (1 + below(8));
    const uint64_t slots = (uint64_t)L * B + below(6);
    uint8_t *src = guarded(slots * seg), *dst = guarded(slots * seg);
    for (uint64_t i = 0; i < slots * seg; ++i) src[i] = (uint8_t)next();
    const uint64_t sdev = 0x100000000ull, ddev = 0x900000000ull; /* device addresses of the two regions */
    uint64_t *perm = malloc(slots * 8), *addrs = malloc((size_t)L * B * 8), *back = malloc((size_t)L * B * 8);
    for (uint64_t i = 0; i < slots; ++i) perm[i] = i;
    for (uint64_t i = slots; i > 1; --i) { const uint64_t j = below(i), t = perm[i - 1]; perm[i - 1] = perm[j]; perm[j] = t; }
    const int kind = (int)below(3);
    for (uint32_t l = 0; l < L; ++l)
      for (uint32_t b = 0; b < B; ++b) {
        const uint64_t s = kind == 0 ? (uint64_t)b * L + l : kind == 1 ? (uint64_t)l * B + b : perm[(uint64_t)l * B + b];
        addrs[(size_t)l * B + b] = s * seg;
      }
    const uint64_t cap = (uint64_t)L * B;
    uint32_t *rpl = malloc(L * 4), *cnt = malloc(cap * 4);
    uint64_t *base = malloc(cap * 8);
    int64_t *stride = malloc(cap * 8);
    uint64_t n_runs = 0;
    /* source table: addresses in the source region */
    for (uint64_t i = 0; i < cap; ++i) addrs[i] += sdev;
    CHECK(oracle_runs_encode(addrs, L, B, rpl, base, stride, cnt, cap, &n_runs) == ORACLE_OK);
    CHECK(oracle_runs_decode(rpl, base, stride, cnt, n_runs, L, B, back) == ORACLE_OK);
    CHECK(memcmp(back, addrs, cap * 8) == 0);
    uint8_t *stg = guarded(cap * seg);
    oracle_region sr = {sdev, slots * seg, src}, dr = {ddev, slots * seg, dst};
    CHECK(oracle_gather(rpl, base, stride, cnt, n_runs, L, B, seg, &sr, 1, stg) == ORACLE_OK);
    check_guards(stg, cap * seg);
    for (uint32_t l = 0; l < L; ++l) /* every staged segment is the one the address names */
      for (uint32_t b = 0; b < B; ++b)
        CHECK(memcmp(stg + ((uint64_t)b * L + l) * seg, src + (addrs[(size_t)l * B + b] - sdev), seg) == 0);
    /* the fetch plan and its descriptors */
    const uint64_t rb = sdev, rbytes = slots * seg;
    uint64_t nd = 0, slab_bytes = 0;
    uint64_t *local = malloc(cap * 8);
    const uint64_t max_read = 16 * (1 + below(64));
    (void)oracle_groups_plan(rpl, base, stride, cnt, n_runs, L, B, seg, &rb, &rbytes, 1, max_read, NULL, 0, &nd,
                             &slab_bytes, local);
    oracle_desc *descs = malloc((nd + 1) * sizeof(oracle_desc));
    CHECK(oracle_groups_plan(rpl, base, stride, cnt, n_runs, L, B, seg, &rb, &rbytes, 1, max_read, descs, nd, &nd,
                             &slab_bytes, local) == ORACLE_OK);
    uint8_t *slab = guarded(slab_bytes);
    CHECK(oracle_copy_descs(descs, nd, &sr, 1, slab, slab_bytes) == ORACLE_OK);
    check_guards(slab, slab_bytes);
    for (uint64_t i = 0; i < cap; ++i) /* the slab holds every segment at its local offset */
      CHECK(memcmp(slab + local[i], src + (addrs[i] - sdev), seg) == 0);
    /* destination: a permutation scatter, then the gap bytes stay as they were */
    for (uint64_t i = 0; i < cap; ++i) addrs[i] = ddev + perm[i] * seg;
    CHECK(oracle_runs_encode(addrs, L, B, rpl, base, stride, cnt, cap, &n_runs) == ORACLE_OK);
    memset(dst, 0xA5, slots * seg);
    CHECK(oracle_scatter(rpl, base, stride, cnt, n_runs, L, B, seg, &dr, 1, stg) == ORACLE_OK);
    check_guards(dst, slots * seg);
    /* a table that leaves its region is refused */
    base[n_runs - 1] = ddev + slots * seg;
    CHECK(oracle_scatter(rpl, base, stride, cnt, n_runs, L, B, seg, &dr, 1, stg) != ORACLE_OK);
    cnt[0] = 0;
    CHECK(oracle_runs_decode(rpl, base, stride, cnt, n_runs, L, B, back) != ORACLE_OK);
    free(perm); free(addrs); free(back); free(rpl); free(cnt); free(base); free(stride); free(local); free(descs);
    release(src); release(dst); release(stg); release(slab);
  }
}

static void pages(void) {
  for (int it = 0; it < 300; ++it) {
    const uint64_t page_len = 16 * (1 + below(80)), stride = page_len + 16 * below(3);
    const uint64_t n = below(120), slots = n + 1 + below(8);
    uint8_t *src = guarded(slots * stride + 16), *dst = guarded(slots * stride + 16), *back = guarded(slots * stride + 16);
    for (uint64_t i = 0; i < slots * stride + 16; ++i) src[i] = (uint8_t)next();
    memset(dst, 0, slots * stride + 16);
    memcpy(back, src, slots * stride + 16);
    uint32_t *perm = malloc(slots * 4), *si = malloc((n + 1) * 4), *di = malloc((n + 1) * 4);
    for (uint64_t i = 0; i < slots; ++i) perm[i] = (uint32_t)i;
    for (uint64_t i = slots; i > 1; --i) { const uint64_t j = below(i); const uint32_t t = perm[i - 1]; perm[i - 1] = perm[j]; perm[j] = t; }
    for (uint64_t k = 0; k < n; ++k) { si[k] = (uint32_t)k; di[k] = perm[k]; }
    oracle_region s = {0, slots * stride + 16, src}, d = {0, slots * stride + 16, dst}, bk = {0, slots * stride + 16, back};
    const uint64_t off = 16 * below(2);
    CHECK(oracle_paged_copy(page_len, &s, si, stride, off, &d, di, stride, off, n) == ORACLE_OK);
    check_guards(dst, slots * stride + 16);
    /* copying back by the inverse lists restores the pages */
    memset(back, 0, slots * stride + 16);
    CHECK(oracle_paged_copy(page_len, &d, di, stride, off, &bk, si, stride, off, n) == ORACLE_OK);
    for (uint64_t k = 0; k < n; ++k) CHECK(memcmp(back + off + k * stride, src + off + k * stride, page_len) == 0);
    if (n) {
      si[n - 1] = (uint32_t)slots + 1; /* past the end of the region */
      CHECK(oracle_paged_copy(page_len, &s, si, stride, off, &d, di, stride, off, n) != ORACLE_OK);
    }
    free(perm); free(si); free(di);
    release(src); release(dst); release(back);
  }
}

int main(void) {
  numbers();
  argmax();
  runs();
  pages();
  printf("oracle under sanitizers: all checks passed\n");
  return 0;
}
