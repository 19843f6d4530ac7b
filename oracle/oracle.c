/*
 * CPU oracle for the transfer staging / combine path.  TEST INFRASTRUCTURE
 * ONLY: see oracle.h for who may call it and for the page citations.
 *
 * Every function is written as the plain definition of its result, one
 * element (or one segment) at a time, with no blocking, vectorisation or
 * reordering.
 */
#include "oracle.h"

#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ BF16 */

static double f32_value(uint32_t bits) {
  float f;
  memcpy(&f, &bits, 4);
  return (double)f; /* exact: every float is a double */
}

/* Value of a non-negative BF16 magnitude pattern 0x0000..0x7F80, where
 * 0x7F80 stands for 2^128: the value one BF16 step above the largest finite
 * magnitude, which is where IEEE round-to-nearest places the overflow
 * threshold. */
static double bf16_magnitude(uint32_t mag) {
  if (mag == 0x7F80u) return 0x1p128;
  return f32_value(mag << 16);
}

/*
 * Round-to-nearest-even conversion of an F32 bit pattern to BF16, the wire
 * precision of [CE] "Change" (the F32 partials are converted to BF16 before
 * they are sent).
 *
 * Definition: of the two BF16 magnitudes that bracket |x| (the truncation
 * `lo` and the next one up `hi`), take the nearer; on an exact tie take the
 * one whose last significand bit is 0.  The sign is kept, subnormals are
 * rounded by the same rule.  Infinities are kept.  Any NaN becomes the
 * canonical quiet NaN 0x7FC0 (the pages fix no NaN encoding; this is the
 * reading that makes CPU and GPU agree bit for bit).
 */
uint16_t oracle_bf16_rne(uint32_t f) {
  const uint32_t sign = f & 0x80000000u;
  const uint32_t mag = f & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return 0x7FC0u;
  if (mag == 0x7F800000u) return (uint16_t)(f >> 16);
  const double x = f32_value(mag);
  const uint32_t lo = mag >> 16;
  const uint32_t hi = lo + 1;
  /* Both differences are exact in double: the operands share a grid of
   * spacing one F32 ulp of x and differ by less than one BF16 ulp. */
  const double d_lo = x - bf16_magnitude(lo);
  const double d_hi = bf16_magnitude(hi) - x;
  uint32_t r;
  if (d_lo < d_hi)
    r = lo;
  else if (d_hi < d_lo)
    r = hi;
  else
    r = (lo & 1u) ? hi : lo;
  return (uint16_t)(r | (sign >> 16));
}

void oracle_bf16_rne_array(const uint32_t *in, uint16_t *out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_bf16_rne(in[i]);
}

/* ------------------------------------------------------------------ pack */

/*
 * [CE] "Change": each rank converts its F32 part to BF16 in 512 KiB chunks,
 * and two slots alternate so the next chunk is converted while the previous
 * one is in flight.  Generalised to a ring of R = ring_elems / chunk_elems
 * slots: chunk c holds elements [c*CE, min((c+1)*CE, n)) and is written at
 * slot c mod R.  One call packs chunks [chunk_begin, chunk_end); a call may
 * not name more chunks than the ring has slots, and a chunk must hold at
 * least one element.
 */
int oracle_pack(const float *src, size_t n, uint16_t *ring, size_t ring_elems, size_t chunk_elems,
                size_t chunk_begin, size_t chunk_end) {
  if (chunk_elems == 0 || ring_elems == 0 || ring_elems % chunk_elems) return ORACLE_EARG;
  const size_t R = ring_elems / chunk_elems;
  if (chunk_begin > chunk_end || chunk_end - chunk_begin > R) return ORACLE_EARG;
  for (size_t c = chunk_begin; c < chunk_end; ++c) {
    const size_t start = c * chunk_elems;
    if (start >= n) return ORACLE_EARG;
    const size_t len = (n - start < chunk_elems) ? n - start : chunk_elems;
    const size_t slot = c % R;
    for (size_t j = 0; j < len; ++j) {
      uint32_t bits;
      memcpy(&bits, &src[start + j], 4);
      ring[slot * chunk_elems + j] = oracle_bf16_rne(bits);
    }
  }
  return ORACLE_OK;
}

/* --------------------------------------------------------------- combine */

/*
 * [CE] "Change" (sum kernel): the two BF16 values are added in F32, in the
 * same operand order on both ranks, so both get identical bits.  BF16 -> F32
 * is exact (the BF16 pattern is the top half of the F32 pattern).  The add
 * is one IEEE binary32 addition, round to nearest even, subnormals kept.
 * A NaN result is written as the canonical 0x7FC00000 (reading, as above).
 */
uint32_t oracle_sum2_f32(uint16_t a, uint16_t b) {
  uint32_t ab = (uint32_t)a << 16, bb = (uint32_t)b << 16;
  float fa, fb;
  memcpy(&fa, &ab, 4);
  memcpy(&fb, &bb, 4);
  float s = fa + fb;
  uint32_t r;
  memcpy(&r, &s, 4);
  if ((r & 0x7FFFFFFFu) > 0x7F800000u) r = 0x7FC00000u;
  return r;
}

/*
 * mode 0: out[i] = the F32 sum of [CE] "Change".
 * mode 1: out[i] = that F32 sum rounded to BF16 (RNE), the "fp32 sums
 *         rounded to bf16" of [TP2] "Layout".
 */
int oracle_combine2(const uint16_t *a, const uint16_t *b, size_t n, void *out, int mode) {
  if (mode != 0 && mode != 1) return ORACLE_EARG;
  for (size_t i = 0; i < n; ++i) {
    uint32_t s = oracle_sum2_f32(a[i], b[i]);
    if (mode == 0)
      memcpy((uint8_t *)out + 4 * i, &s, 4);
    else
      ((uint16_t *)out)[i] = oracle_bf16_rne(s);
  }
  return ORACLE_OK;
}

/*
 * [TP2] "Layout" and "Collectives": the drafter's all-reduce pushes the F32
 * partials themselves (no BF16 wire) and adds them in F32, rank 0's value
 * first on both ranks; the sum is then rounded to BF16 (or kept in F32, the
 * debug oracle's "optional BF16 rounding").  One IEEE binary32 addition,
 * round to nearest even, subnormals kept; a NaN sum is written as the
 * canonical 0x7FC00000, as for the BF16-wire sum.
 */
uint32_t oracle_sum2_f32_f32(uint32_t a_bits, uint32_t b_bits) {
  float fa, fb;
  memcpy(&fa, &a_bits, 4);
  memcpy(&fb, &b_bits, 4);
  float s = fa + fb;
  uint32_t r;
  memcpy(&r, &s, 4);
  if ((r & 0x7FFFFFFFu) > 0x7F800000u) r = 0x7FC00000u;
  return r;
}

/* mode 0: out[i] = the F32 sum; mode 1: that sum rounded to BF16 (RNE). */
int oracle_combine2_f32(const float *a, const float *b, size_t n, void *out, int mode) {
  if (mode != 0 && mode != 1) return ORACLE_EARG;
  for (size_t i = 0; i < n; ++i) {
    uint32_t ab, bb;
    memcpy(&ab, &a[i], 4);
    memcpy(&bb, &b[i], 4);
    const uint32_t s = oracle_sum2_f32_f32(ab, bb);
    if (mode == 0)
      memcpy((uint8_t *)out + 4 * i, &s, 4);
    else
      ((uint16_t *)out)[i] = oracle_bf16_rne(s);
  }
  return ORACLE_OK;
}

/* ---------------------------------------------------------------- argmax */

typedef struct {
  int has;
  uint16_t bits;
  double value;
  int64_t id;
} elem;

/* x comes strictly before y in the row order: larger value first (numeric
 * comparison, so -0 and +0 are equal), then the lower global id.  An absent
 * element comes after every present one. */
static int before(const elem *x, const elem *y) {
  if (!y->has) return x->has;
  if (!x->has) return 0;
  if (x->value != y->value) return x->value > y->value;
  return x->id < y->id;
}

typedef struct {
  elem top1, top2;
} shard_rec;

/* One shard's first and second element of a row under that order. */
static int shard_scan(const oracle_shard *s, uint32_t row, shard_rec *rec) {
  const uint16_t *p = s->ptr + (size_t)row * s->ld;
  rec->top1.has = rec->top2.has = 0;
  for (uint32_t j = 0; j < s->ncols; ++j) {
    elem e;
    e.has = 1;
    e.bits = p[j];
    if ((e.bits & 0x7FFFu) > 0x7F80u) return ORACLE_ENAN;
    e.value = f32_value((uint32_t)e.bits << 16);
    e.id = (int64_t)s->col_offset + j;
    if (before(&e, &rec->top1)) {
      rec->top2 = rec->top1;
      rec->top1 = e;
    } else if (before(&e, &rec->top2)) {
      rec->top2 = e;
    }
  }
  return ORACLE_OK;
}

/*
 * [TP2] "Layout": the vocabulary is split by columns between the ranks,
 * rank 0 holding the lower ids, so that a tie of the global argmax goes to
 * the lower id as on one card; per drafted position each rank's (shard max,
 * index) is exchanged and folded, or (top1, top2, index) when the margin is
 * wanted.
 *
 * The fold: global top1 = the earlier of the two shards' top1 in the row
 * order; global top2 = the earlier of the other shard's top1 and the
 * winning shard's top2.  Values are reported as the exact F32 of the chosen
 * BF16 elements.
 */
int oracle_argmax_merge(const oracle_shard *s0, const oracle_shard *s1, int mode, void *out) {
  if (mode != 0 && mode != 1) return ORACLE_EARG;
  if (s0->rows != s1->rows || s0->ncols == 0 || s1->ncols == 0) return ORACLE_EARG;
  const uint64_t a0 = s0->col_offset, a1 = a0 + s0->ncols;
  const uint64_t b0 = s1->col_offset, b1 = b0 + s1->ncols;
  if (!(a1 <= b0 || b1 <= a0)) return ORACLE_EARG; /* shards share ids */
  for (uint32_t r = 0; r < s0->rows; ++r) {
    shard_rec x, y;
    int rc = shard_scan(s0, r, &x);
    if (rc) return rc;
    rc = shard_scan(s1, r, &y);
    if (rc) return rc;
    const shard_rec *win = before(&x.top1, &y.top1) ? &x : &y;
    const shard_rec *lose = (win == &x) ? &y : &x;
    const elem *second = before(&lose->top1, &win->top2) ? &lose->top1 : &win->top2;
    const float v1 = (float)f32_value((uint32_t)win->top1.bits << 16);
    if (mode == 0) {
      oracle_max_idx *o = (oracle_max_idx *)out + r;
      o->max = v1;
      o->idx = (int32_t)win->top1.id;
    } else {
      oracle_top2 *o = (oracle_top2 *)out + r;
      o->top1 = v1;
      o->top2 = (float)f32_value((uint32_t)second->bits << 16);
      o->idx = (int32_t)win->top1.id;
      o->reserved = 0;
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------ run tables */

/* a_next - a_prev as a signed 64-bit delta; *ok = 0 if it does not fit. */
static int64_t signed_delta(uint64_t a_prev, uint64_t a_next, int *ok) {
  *ok = 1;
  if (a_next >= a_prev) {
    uint64_t d = a_next - a_prev;
    if (d > (uint64_t)INT64_MAX) {
      *ok = 0;
      return 0;
    }
    return (int64_t)d;
  }
  uint64_t d = a_prev - a_next;
  if (d > (uint64_t)INT64_MAX + 1u) {
    *ok = 0;
    return 0;
  }
  return (int64_t)(0 - d);
}

/*
 * [RUNS] "What this PR does": per lane (one slot's K or V across the
 * blocks) the holder feeds the segment addresses, block by block, into a
 * greedy run accumulator; the table is the parallel arrays runs_per_lane /
 * run_base / run_stride / run_count.  A run is an arithmetic sequence
 * base + i * stride, i < count ([RUNS] "Problem").
 *
 * Greedy rule (a run with one address takes the first non-zero delta as its
 * stride; a longer run extends while the delta equals its stride; any other
 * address starts a new run).  The stride of a one-address run is 0.
 */
int oracle_runs_encode(const uint64_t *addrs, uint32_t n_lanes, uint32_t n_blocks, uint32_t *runs_per_lane,
                       uint64_t *run_base, int64_t *run_stride, uint32_t *run_count, uint64_t cap_runs,
                       uint64_t *n_runs_out) {
  uint64_t nr = 0;
  for (uint32_t l = 0; l < n_lanes; ++l) {
    const uint64_t *a = addrs + (uint64_t)l * n_blocks;
    uint32_t lane_runs = 0;
    if (n_blocks == 0) {
      runs_per_lane[l] = 0;
      continue;
    }
    uint64_t base = a[0];
    int64_t stride = 0;
    uint32_t count = 1;
    for (uint32_t i = 1; i <= n_blocks; ++i) {
      int closes = (i == n_blocks);
      if (!closes) {
        int ok;
        int64_t d = signed_delta(a[i - 1], a[i], &ok);
        if (count == 1 && ok && d != 0) {
          stride = d;
          count = 2;
        } else if (count >= 2 && ok && d == stride) {
          count += 1;
        } else {
          closes = 1;
        }
      }
      if (closes) {
        if (nr >= cap_runs) return ORACLE_EARG;
        run_base[nr] = base;
        run_stride[nr] = (count == 1) ? 0 : stride;
        run_count[nr] = count;
        ++nr;
        ++lane_runs;
        if (i < n_blocks) {
          base = a[i];
          stride = 0;
          count = 1;
        }
      }
    }
    runs_per_lane[l] = lane_runs;
  }
  *n_runs_out = nr;
  return ORACLE_OK;
}

/* base + k * stride with every step checked for 64-bit overflow. */
static int run_addr(uint64_t base, int64_t stride, uint64_t k, uint64_t *out) {
  if (k > (uint64_t)INT64_MAX) return 0;
  int64_t prod;
  if (__builtin_mul_overflow((int64_t)k, stride, &prod)) return 0;
  if (prod >= 0) {
    if (base > UINT64_MAX - (uint64_t)prod) return 0;
    *out = base + (uint64_t)prod;
  } else {
    uint64_t m = (uint64_t)0 - (uint64_t)prod;
    if (base < m) return 0;
    *out = base - m;
  }
  return 1;
}

/*
 * [RUNS] "Problem": addr = base + i * stride along a lane.  Runs are stored
 * lane after lane; a lane's runs cover its blocks in order, so run r of a
 * lane covers blocks [start_r, start_r + count_r) with start_r the sum of
 * the counts of the lane's earlier runs.  A table whose counts do not cover
 * each lane's blocks exactly, that has a zero-count run, or whose arithmetic
 * overflows, is refused ([RUNS] "Trust boundary").
 */
int oracle_runs_decode(const uint32_t *runs_per_lane, const uint64_t *run_base, const int64_t *run_stride,
                       const uint32_t *run_count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                       uint64_t *addrs_out) {
  uint64_t r = 0;
  for (uint32_t l = 0; l < n_lanes; ++l) {
    uint64_t start = 0;
    for (uint32_t k = 0; k < runs_per_lane[l]; ++k, ++r) {
      if (r >= n_runs) return ORACLE_ETABLE;
      const uint32_t c = run_count[r];
      if (c == 0) return ORACLE_ETABLE;
      if (start + c > n_blocks) return ORACLE_ETABLE;
      for (uint32_t i = 0; i < c; ++i) {
        uint64_t a;
        if (!run_addr(run_base[r], run_stride[r], i, &a)) return ORACLE_ETABLE;
        addrs_out[(uint64_t)l * n_blocks + start + i] = a;
      }
      start += c;
    }
    if (start != n_blocks) return ORACLE_ETABLE;
  }
  if (r != n_runs) return ORACLE_ETABLE;
  return ORACLE_OK;
}

/* Host image of the seg_bytes at device address a, or NULL if no single
 * region holds all of them. */
static uint8_t *host_at(const oracle_region *regions, int n_regions, uint64_t a, uint64_t seg_bytes) {
  for (int i = 0; i < n_regions; ++i) {
    const oracle_region *g = &regions[i];
    if (a >= g->dev_base && a - g->dev_base <= g->bytes && g->bytes - (a - g->dev_base) >= seg_bytes)
      return g->host + (a - g->dev_base);
  }
  return NULL;
}

static uint64_t *decode_all(const uint32_t *rpl, const uint64_t *base, const int64_t *stride,
                            const uint32_t *count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                            int *rc) {
  uint64_t n = (uint64_t)n_lanes * n_blocks;
  uint64_t *addrs = (uint64_t *)malloc((n ? n : 1) * sizeof(uint64_t));
  if (!addrs) {
    *rc = ORACLE_EARG;
    return NULL;
  }
  *rc = oracle_runs_decode(rpl, base, stride, count, n_runs, n_lanes, n_blocks, addrs);
  if (*rc) {
    free(addrs);
    return NULL;
  }
  return addrs;
}

/*
 * Gather: decode the table, then copy each (lane l, block b) segment to
 * its place in the dense staging buffer, which is ordered block by block,
 * lane by lane within a block.  The data-movement counterpart of
 * [RUNS] "What this PR does" steps 2-4 (decode, then read every segment
 * into a dense local buffer).
 */
int oracle_gather(const uint32_t *runs_per_lane, const uint64_t *run_base, const int64_t *run_stride,
                  const uint32_t *run_count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                  uint64_t seg_bytes, const oracle_region *regions, int n_regions, uint8_t *staging) {
  int rc;
  uint64_t *addrs =
      decode_all(runs_per_lane, run_base, run_stride, run_count, n_runs, n_lanes, n_blocks, &rc);
  if (!addrs) return rc;
  for (uint64_t b = 0; b < n_blocks; ++b)
    for (uint64_t l = 0; l < n_lanes; ++l) {
      const uint8_t *from = host_at(regions, n_regions, addrs[l * n_blocks + b], seg_bytes);
      if (!from) {
        free(addrs);
        return ORACLE_ERANGE;
      }
      memcpy(staging + (b * n_lanes + l) * seg_bytes, from, seg_bytes);
    }
  free(addrs);
  return ORACLE_OK;
}

/*
 * Scatter: the inverse placement into a destination with its own table;
 * every destination segment (l, b) receives staging segment (b, l).  No
 * other destination byte is written.  The data-movement counterpart of
 * [RUNS] "What this PR does" step 5 (every block placed at its own local
 * address).
 */
int oracle_scatter(const uint32_t *runs_per_lane, const uint64_t *run_base, const int64_t *run_stride,
                   const uint32_t *run_count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                   uint64_t seg_bytes, const oracle_region *regions, int n_regions, const uint8_t *staging) {
  int rc;
  uint64_t *addrs =
      decode_all(runs_per_lane, run_base, run_stride, run_count, n_runs, n_lanes, n_blocks, &rc);
  if (!addrs) return rc;
  for (uint64_t b = 0; b < n_blocks; ++b)
    for (uint64_t l = 0; l < n_lanes; ++l) {
      uint8_t *to = host_at(regions, n_regions, addrs[l * n_blocks + b], seg_bytes);
      if (!to) {
        free(addrs);
        return ORACLE_ERANGE;
      }
      memcpy(to, staging + (b * n_lanes + l) * seg_bytes, seg_bytes);
    }
  free(addrs);
  return ORACLE_OK;
}

/* ------------------------------------------------- coalesced fetch planning */

typedef struct {
  uint64_t base;   /* remote address of block `start` */
  int64_t stride;  /* 0 for a one-block run */
  uint32_t lane, start, count, region;
  uint64_t index;
} run_info;

static int by_region_then_base(const void *pa, const void *pb) {
  const run_info *a = (const run_info *)pa, *b = (const run_info *)pb;
  if (a->region != b->region) return a->region < b->region ? -1 : 1;
  if (a->base != b->base) return a->base < b->base ? -1 : 1;
  return a->index < b->index ? -1 : (a->index > b->index);
}

static uint64_t abs64(int64_t s) { return s < 0 ? (uint64_t)0 - (uint64_t)s : (uint64_t)s; }

/*
 * [RUNS] "What this PR does", the requester's plan, step by step:
 *   2. decode the runs, bucket them per NUMA node (declared region), sort
 *      each bucket by remote base;
 *   3. group runs whose per-block chunks tile densely: same block range, same
 *      stride, base-adjacent, and the grown chunk still fits the stride;
 *   4. one slab carve and one coalesced read per dense group (chunks back to
 *      back); other groups are read block by block into a dense mirror;
 *      reads are split at max_read_bytes ("READ splitting");
 *   5. rebuild: local(b) = group_local + (remote(b) - group_remote).
 */
int oracle_groups_plan(const uint32_t *runs_per_lane, const uint64_t *run_base, const int64_t *run_stride,
                       const uint32_t *run_count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                       uint64_t seg_bytes, const uint64_t *region_base, const uint64_t *region_bytes, int n_regions,
                       uint64_t max_read_bytes, oracle_desc *descs, uint64_t cap, uint64_t *n_descs,
                       uint64_t *slab_bytes, uint64_t *local) {
  if (max_read_bytes == 0 || seg_bytes == 0) return ORACLE_EARG;
  run_info *runs = (run_info *)malloc((n_runs ? n_runs : 1) * sizeof(run_info));
  if (!runs) return ORACLE_EARG;
  /* step 2: decode */
  uint64_t r = 0;
  for (uint32_t l = 0; l < n_lanes; ++l) {
    uint32_t start = 0;
    for (uint32_t k = 0; k < runs_per_lane[l]; ++k, ++r) {
      if (r >= n_runs || run_count[r] == 0) {
        free(runs);
        return ORACLE_ETABLE;
      }
      run_info *x = &runs[r];
      x->base = run_base[r];
      x->count = run_count[r];
      x->stride = x->count > 1 ? run_stride[r] : 0;
      x->lane = l;
      x->start = start;
      x->index = r;
      uint64_t last;
      if (!run_addr(x->base, x->stride, x->count - 1, &last)) {
        free(runs);
        return ORACLE_ETABLE;
      }
      const uint64_t lo = x->base < last ? x->base : last;
      const uint64_t hi = (x->base > last ? x->base : last) + seg_bytes;
      int found = -1;
      for (int g = 0; g < n_regions && found < 0; ++g)
        if (lo >= region_base[g] && hi <= region_base[g] + region_bytes[g]) found = g;
      if (found < 0) {
        free(runs);
        return ORACLE_ERANGE;
      }
      x->region = (uint32_t)found;
      start += x->count;
    }
    if (start != n_blocks) {
      free(runs);
      return ORACLE_ETABLE;
    }
  }
  if (r != n_runs) {
    free(runs);
    return ORACLE_ETABLE;
  }
  /* bucket per region, sort by remote base */
  qsort(runs, n_runs, sizeof(run_info), by_region_then_base);

  uint64_t nd = 0, slab = 0;
  uint64_t i = 0;
  while (i < n_runs) {
    /* step 3: grow a group from runs[i] */
    const run_info *f = &runs[i];
    uint64_t j = i + 1, chunk = seg_bytes;
    while (j < n_runs) {
      const run_info *x = &runs[j];
      const int same_blocks = x->start == f->start && x->count == f->count;
      const int adjacent = x->region == f->region && x->base == f->base + chunk;
      const int fits = f->count == 1 || chunk + seg_bytes <= abs64(f->stride);
      if (!(same_blocks && x->stride == f->stride && adjacent && fits)) break;
      chunk += seg_bytes;
      ++j;
    }
    /* step 4: carve and read */
    const int dense = f->count == 1 || abs64(f->stride) == chunk;
    const uint64_t group_local = slab;
    uint64_t group_remote;
    if (dense) {
      const uint64_t span = f->count == 1 ? chunk : (uint64_t)f->count * abs64(f->stride);
      group_remote = f->stride >= 0 ? f->base : f->base - (uint64_t)(f->count - 1) * abs64(f->stride);
      for (uint64_t off = 0; off < span; off += max_read_bytes) {
        const uint64_t n = span - off < max_read_bytes ? span - off : max_read_bytes;
        if (nd < cap && descs) {
          descs[nd].src = group_remote + off;
          descs[nd].dst_off = group_local + off;
          descs[nd].bytes = n;
        }
        ++nd;
      }
      slab += span;
    } else {
      group_remote = f->base;
      for (uint32_t b = 0; b < f->count; ++b) {
        uint64_t block_remote = 0;
        run_addr(f->base, f->stride, b, &block_remote);
        for (uint64_t off = 0; off < chunk; off += max_read_bytes) {
          const uint64_t n = chunk - off < max_read_bytes ? chunk - off : max_read_bytes;
          if (nd < cap && descs) {
            descs[nd].src = block_remote + off;
            descs[nd].dst_off = group_local + (uint64_t)b * chunk + off;
            descs[nd].bytes = n;
          }
          ++nd;
        }
      }
      slab += (uint64_t)f->count * chunk;
    }
    /* step 5: rebuild every segment's local address */
    for (uint64_t k = i; k < j; ++k) {
      const run_info *x = &runs[k];
      for (uint32_t b = 0; b < x->count; ++b) {
        uint64_t remote = 0;
        run_addr(x->base, x->stride, b, &remote);
        uint64_t loc;
        if (dense) {
          loc = group_local + (remote - group_remote);
        } else {
          uint64_t block_remote = 0;
          run_addr(f->base, f->stride, b, &block_remote);
          loc = group_local + (uint64_t)b * chunk + (remote - block_remote);
        }
        local[(uint64_t)x->lane * n_blocks + x->start + b] = loc;
      }
    }
    i = j;
  }
  free(runs);
  *n_descs = nd;
  *slab_bytes = slab;
  return nd <= cap ? ORACLE_OK : ORACLE_EARG;
}

int oracle_copy_descs(const oracle_desc *descs, uint64_t n_descs, const oracle_region *regions, int n_regions,
                      uint8_t *slab, uint64_t slab_bytes) {
  for (uint64_t d = 0; d < n_descs; ++d) {
    const uint8_t *from = host_at(regions, n_regions, descs[d].src, descs[d].bytes);
    if (!from || descs[d].dst_off > slab_bytes || slab_bytes - descs[d].dst_off < descs[d].bytes)
      return ORACLE_ERANGE;
    memcpy(slab + descs[d].dst_off, from, descs[d].bytes);
  }
  return ORACLE_OK;
}

/* -------------------------------------------------------------- paged copy */

/* Byte offset of page idx of a list inside a region of region_bytes, or -1
 * if the page does not lie wholly inside it (checked arithmetic). */
static int page_offset(uint32_t idx, uint64_t stride, uint64_t offset, uint64_t page_len, uint64_t region_bytes,
                       uint64_t *out) {
  if (stride && idx > (UINT64_MAX - offset) / stride) return -1;
  const uint64_t at = offset + (uint64_t)idx * stride;
  if (at > region_bytes || region_bytes - at < page_len) return -1;
  *out = at;
  return 0;
}

static int cmp_u64(const void *x, const void *y) {
  const uint64_t a = *(const uint64_t *)x, b = *(const uint64_t *)y;
  return a < b ? -1 : a > b;
}

/*
 * [TE] the paged writes of the TransferEngine API: a page list is a set of
 * page indices with one stride and one offset inside a registered region;
 * page k of a list lies at region base + offset + indices[k] * stride, and
 * the k-th source page is written to the k-th destination page, page_len
 * bytes each (the page fixes only that pages are named by indices, a stride
 * and an offset; this is the plainest reading).  Done here as data movement
 * between two regions of one memory.  Every page must lie inside its region
 * (ORACLE_ERANGE); destination pages must not overlap (ORACLE_EARG), so the
 * order of the copies cannot matter.
 */
int oracle_paged_copy(uint64_t page_len, const oracle_region *src, const uint32_t *src_idx, uint64_t src_stride,
                      uint64_t src_offset, const oracle_region *dst, const uint32_t *dst_idx, uint64_t dst_stride,
                      uint64_t dst_offset, uint64_t n_pages) {
  if (page_len == 0 || !src || !dst) return ORACLE_EARG;
  if (n_pages == 0) return ORACLE_OK;
  uint64_t *starts = malloc(n_pages * sizeof(uint64_t));
  if (!starts) return ORACLE_EARG;
  int rc = ORACLE_OK;
  for (uint64_t k = 0; k < n_pages && rc == ORACLE_OK; ++k) {
    uint64_t s = 0, d = 0;
    if (page_offset(src_idx[k], src_stride, src_offset, page_len, src->bytes, &s) ||
        page_offset(dst_idx[k], dst_stride, dst_offset, page_len, dst->bytes, &d))
      rc = ORACLE_ERANGE;
    starts[k] = d;
  }
  if (rc == ORACLE_OK) {
    qsort(starts, n_pages, sizeof(uint64_t), cmp_u64);
    for (uint64_t k = 1; k < n_pages; ++k)
      if (starts[k] - starts[k - 1] < page_len) rc = ORACLE_EARG;
  }
  free(starts);
  if (rc != ORACLE_OK) return rc;
  for (uint64_t k = 0; k < n_pages; ++k) {
    uint64_t s = 0, d = 0;
    page_offset(src_idx[k], src_stride, src_offset, page_len, src->bytes, &s);
    page_offset(dst_idx[k], dst_stride, dst_offset, page_len, dst->bytes, &d);
    memcpy(dst->host + d, src->host + s, page_len);
  }
  return ORACLE_OK;
}
