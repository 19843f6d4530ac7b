/*
 * Seeded synthetic inputs shared by the CPU oracle's tests, the GPU parity
 * tests and the benchmark.
 *
 * This file holds no step of the transfer method itself: no BF16 rounding,
 * no two-operand sum, no argmax fold, no run encoding or decoding, no
 * gather or scatter.  It only draws numbers and lays out addresses, so the
 * oracle and the HIP library can both consume its output without sharing
 * any of the arithmetic they are compared on.
 *
 * Generator: xoshiro256** (Blackman and Vigna, "Scrambled linear
 * pseudorandom number generators", 2018), its 256-bit state filled from the
 * 64-bit seed by SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", 2014).  Normal deviates come from the
 * Box-Muller transform evaluated in double and converted to float by C's
 * default conversion.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  uint64_t s[4];
} dg_rng;

static uint64_t splitmix64(uint64_t *x) {
  uint64_t z = (*x += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static void rng_seed(dg_rng *r, uint64_t seed) {
  uint64_t x = seed;
  for (int i = 0; i < 4; ++i) r->s[i] = splitmix64(&x);
}

static inline uint64_t rotl(uint64_t x, int k) { return (x << k) | (x >> (64 - k)); }

static inline uint64_t rng_next(dg_rng *r) {
  uint64_t *s = r->s;
  const uint64_t result = rotl(s[1] * 5, 7) * 9;
  const uint64_t t = s[1] << 17;
  s[2] ^= s[0];
  s[3] ^= s[1];
  s[1] ^= s[2];
  s[0] ^= s[3];
  s[2] ^= t;
  s[3] = rotl(s[3], 45);
  return result;
}

/* uniform in [0, 1) with 53 random bits */
static inline double rng_u01(dg_rng *r) { return (double)(rng_next(r) >> 11) * 0x1.0p-53; }

/* uniform integer in [0, n), n >= 1, by rejection (no modulo bias) */
static uint64_t rng_below(dg_rng *r, uint64_t n) {
  uint64_t limit = UINT64_MAX - (UINT64_MAX % n);
  uint64_t v;
  do v = rng_next(r);
  while (v >= limit);
  return v % n;
}

/* Fills out[0..n) with raw generator output (little-endian words). */
void dg_bytes(uint8_t *out, size_t n, uint64_t seed) {
  dg_rng r;
  rng_seed(&r, seed);
  size_t i = 0;
  for (; i + 8 <= n; i += 8) {
    uint64_t v = rng_next(&r);
    memcpy(out + i, &v, 8);
  }
  if (i < n) {
    uint64_t v = rng_next(&r);
    memcpy(out + i, &v, n - i);
  }
}

/* Raw 64-bit words, for tests that want random bit patterns. */
void dg_u64(uint64_t *out, size_t n, uint64_t seed) {
  dg_rng r;
  rng_seed(&r, seed);
  for (size_t i = 0; i < n; ++i) out[i] = rng_next(&r);
}

/* n deviates of N(0, sigma^2) (sigma is the standard deviation), each the
 * double Box-Muller value converted to float. */
void dg_normal_f32(float *out, size_t n, uint64_t seed, double sigma) {
  dg_rng r;
  rng_seed(&r, seed);
  const double two_pi = 6.283185307179586476925286766559;
  size_t i = 0;
  while (i < n) {
    double u1 = 1.0 - rng_u01(&r); /* (0, 1] so log() is finite */
    double u2 = rng_u01(&r);
    double rad = sqrt(-2.0 * log(u1));
    out[i++] = (float)(sigma * rad * cos(two_pi * u2));
    if (i < n) out[i++] = (float)(sigma * rad * sin(two_pi * u2));
  }
}

/* Multiplies exactly `count` distinct, uniformly drawn positions of x by
 * `factor` (the outliers of the prompt-batch workload).  Positions are drawn
 * without replacement by rejection against a bitmap.  Returns 0, or -1 if
 * count > n or memory runs out. */
int dg_outliers_f32(float *x, size_t n, uint64_t seed, size_t count, float factor) {
  if (count > n) return -1;
  if (count == 0) return 0;
  uint8_t *seen = (uint8_t *)calloc((n + 7) / 8, 1);
  if (!seen) return -1;
  dg_rng r;
  rng_seed(&r, seed);
  size_t placed = 0;
  while (placed < count) {
    uint64_t p = rng_below(&r, n);
    if (seen[p >> 3] & (1u << (p & 7))) continue;
    seen[p >> 3] |= (uint8_t)(1u << (p & 7));
    x[p] = x[p] * factor;
    ++placed;
  }
  free(seen);
  return 0;
}

/* BF16 bit patterns of N(0, sigma^2) deviates: each deviate is clamped to
 * [-clamp, clamp], converted to float, and its low 16 bits are dropped
 * (truncation, deliberately not the round-to-nearest-even under test). */
void dg_bf16_normal_trunc(uint16_t *out, size_t n, uint64_t seed, double sigma, double clamp) {
  dg_rng r;
  rng_seed(&r, seed);
  const double two_pi = 6.283185307179586476925286766559;
  size_t i = 0;
  while (i < n) {
    double u1 = 1.0 - rng_u01(&r);
    double u2 = rng_u01(&r);
    double rad = sqrt(-2.0 * log(u1));
    double z[2] = {sigma * rad * cos(two_pi * u2), sigma * rad * sin(two_pi * u2)};
    for (int k = 0; k < 2 && i < n; ++k) {
      double v = z[k];
      if (v > clamp) v = clamp;
      if (v < -clamp) v = -clamp;
      float f = (float)v;
      uint32_t bits;
      memcpy(&bits, &f, 4);
      out[i++] = (uint16_t)(bits >> 16);
    }
  }
}

/* Uniform random permutation of 0..n-1 (Fisher-Yates). */
void dg_perm_u32(uint32_t *out, uint32_t n, uint64_t seed) {
  dg_rng r;
  rng_seed(&r, seed);
  for (uint32_t i = 0; i < n; ++i) out[i] = i;
  for (uint32_t i = n; i > 1; --i) {
    uint32_t j = (uint32_t)rng_below(&r, i);
    uint32_t t = out[i - 1];
    out[i - 1] = out[j];
    out[j] = t;
  }
}

/* `count` distinct values from [0, n), in draw order. Returns 0 or -1. */
int dg_choose_u32(uint32_t *out, uint32_t count, uint32_t n, uint64_t seed) {
  if (count > n) return -1;
  uint8_t *seen = (uint8_t *)calloc(((size_t)n + 7) / 8, 1);
  if (!seen && n) return -1;
  dg_rng r;
  rng_seed(&r, seed);
  uint32_t k = 0;
  while (k < count) {
    uint32_t p = (uint32_t)rng_below(&r, n);
    if (seen[p >> 3] & (1u << (p & 7))) continue;
    seen[p >> 3] |= (uint8_t)(1u << (p & 7));
    out[k++] = p;
  }
  free(seen);
  return 0;
}

/*
 * Source addresses of a paged K/V cache whose blocks were bump-allocated.
 *
 * Lanes are l = 2*slot + kv (K of a slot, then its V).  Slots are split into
 * n_regions equal consecutive groups, one per memory region ("NUMA node").
 * Inside a region, every block owns one contiguous chunk holding, slot by
 * slot, the K then the V segment of each of that region's slots.  Block b's
 * chunk sits at chunk position pos[b] of the region (pos == NULL: pos[b] =
 * b, the fully sequential allocation).
 *
 * addrs is lane-major: addrs[l * n_blocks + b].  Returns 0, or -1 when the
 * slots do not split evenly.
 */
int dg_kv_src_addrs(uint64_t *addrs, uint32_t n_blocks, uint32_t n_slots, uint64_t seg_bytes,
                    const uint64_t *region_base, uint32_t n_regions, const uint32_t *pos) {
  if (n_regions == 0 || n_slots % n_regions) return -1;
  const uint64_t spr = n_slots / n_regions;
  const uint64_t chunk = spr * 2 * seg_bytes;
  const uint64_t n_lanes = 2ull * n_slots;
  for (uint64_t l = 0; l < n_lanes; ++l) {
    uint64_t s = l / 2, kv = l % 2;
    uint64_t reg = s / spr, within = s % spr;
    for (uint64_t b = 0; b < n_blocks; ++b) {
      uint64_t p = pos ? pos[b] : b;
      addrs[l * n_blocks + b] = region_base[reg] + p * chunk + (2 * within + kv) * seg_bytes;
    }
  }
  return 0;
}

/* Destination addresses laid out slot-major with its own slot stride:
 * daddr(2*slot + kv, b) = base + (b * n_slots + slot) * slot_stride + kv * seg_bytes.
 * Lane-major like dg_kv_src_addrs. */
void dg_kv_dst_addrs(uint64_t *addrs, uint32_t n_blocks, uint32_t n_slots, uint64_t seg_bytes,
                     uint64_t base, uint64_t slot_stride) {
  const uint64_t n_lanes = 2ull * n_slots;
  for (uint64_t l = 0; l < n_lanes; ++l) {
    uint64_t s = l / 2, kv = l % 2;
    for (uint64_t b = 0; b < n_blocks; ++b)
      addrs[l * n_blocks + b] = base + (b * n_slots + s) * slot_stride + kv * seg_bytes;
  }
}

/*
 * Stamps a 16-byte tag {0x5E6D7A61, lane, block, low 32 bits of seed} at the
 * start of every segment that lies wholly inside the host image `region`
 * of the device range [dev_base, dev_base + region_bytes).  The rest of
 * each segment is whatever the region already held (normally dg_bytes
 * output), so a segment copied to the wrong place identifies itself.
 */
void dg_tag_segments(uint8_t *region, uint64_t dev_base, uint64_t region_bytes, const uint64_t *addrs,
                     uint32_t n_lanes, uint32_t n_blocks, uint64_t seg_bytes, uint64_t seed) {
  if (seg_bytes < 16) return;
  for (uint64_t l = 0; l < n_lanes; ++l)
    for (uint64_t b = 0; b < n_blocks; ++b) {
      uint64_t a = addrs[l * n_blocks + b];
      if (a < dev_base || a - dev_base > region_bytes || region_bytes - (a - dev_base) < seg_bytes) continue;
      uint32_t tag[4] = {0x5E6D7A61u, (uint32_t)l, (uint32_t)b, (uint32_t)seed};
      memcpy(region + (a - dev_base), tag, 16);
    }
}
