/*
 * CPU oracle for the transfer staging / combine path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path
 * (the HIP library and its Python binding) never calls it, and the two
 * share no source, header, table or helper.
 *
 * Plain, slow, single-threaded C11.  Each function is the definition of
 * what the corresponding library call computes, written out directly, and
 * cites the page passage it follows.  Pages:
 *   [CE]   llama.cpp PR "Large all-reduces ... through the copy engines"
 *          (Piggidragon fork, PR 16), section "Change".
 *   [TP2]  "The two-card (TP = 2) DSpark worker" (TP2.md), sections
 *          "Layout" and "Collectives".
 *   [RUNS] pegaflow PR 350 "run-encode QueryBlocksForTransfer addresses",
 *          sections "Problem", "What this PR does", "Trust boundary".
 *
 * Parity status: every function below has at least one pin that does not
 * go through this file (see tests/test_oracle_pins.py); none is "parity
 * unpinned".
 *
 * Build: gcc -std=c11 -O2 -fno-fast-math -ffp-contract=off (x86-64 SSE
 * arithmetic, default MXCSR: no flush-to-zero, no denormals-are-zero).
 */
#ifndef XFER_ORACLE_H
#define XFER_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of the oracle (its own; unrelated to the library's). */
#define ORACLE_OK 0
#define ORACLE_EARG -1     /* arguments outside what the definition covers */
#define ORACLE_ENAN -2     /* NaN logit: outside the argmax contract       */
#define ORACLE_ETABLE -3   /* run table inconsistent or arithmetic overflow */
#define ORACLE_ERANGE -4   /* address outside every declared region         */

/* F32 bit pattern -> BF16 bit pattern, round to nearest, ties to even. */
uint16_t oracle_bf16_rne(uint32_t f32_bits);
void oracle_bf16_rne_array(const uint32_t *in, uint16_t *out, size_t n);

/* Pack the chunks [chunk_begin, chunk_end) of src[0..n) into the ring. */
int oracle_pack(const float *src, size_t n, uint16_t *ring, size_t ring_elems, size_t chunk_elems,
                size_t chunk_begin, size_t chunk_end);

/* Sum of two BF16 values in binary32, returned as F32 bits. */
uint32_t oracle_sum2_f32(uint16_t a_rank0, uint16_t b_rank1);

/* mode 0: out is float[n]; mode 1: out is BF16 bits uint16_t[n]. */
int oracle_combine2(const uint16_t *a_rank0, const uint16_t *b_rank1, size_t n, void *out, int mode);

/* F32-wire variant ([TP2]): sum of two F32 values in binary32 (F32 bits),
 * and its array form; mode 0 F32 out, mode 1 BF16 out. */
uint32_t oracle_sum2_f32_f32(uint32_t a_bits, uint32_t b_bits);
int oracle_combine2_f32(const float *a_rank0, const float *b_rank1, size_t n, void *out, int mode);

/* One shard's view of a row block of BF16 logits. */
typedef struct {
  const uint16_t *ptr;   /* element (0, 0) of the shard           */
  size_t ld;             /* elements between consecutive rows     */
  uint32_t rows;
  uint32_t ncols;
  uint32_t col_offset;   /* global id of the shard's column 0     */
} oracle_shard;

/* Output records.  mode 0: {max, idx}; mode 1: {top1, top2, idx, 0}. */
typedef struct {
  float max;
  int32_t idx;
} oracle_max_idx;
typedef struct {
  float top1, top2;
  int32_t idx, reserved;
} oracle_top2;

int oracle_argmax_merge(const oracle_shard *s0, const oracle_shard *s1, int mode, void *out);

/* Run tables (lane-major).  addrs is [n_lanes][n_blocks]. */
int oracle_runs_encode(const uint64_t *addrs, uint32_t n_lanes, uint32_t n_blocks, uint32_t *runs_per_lane,
                       uint64_t *run_base, int64_t *run_stride, uint32_t *run_count, uint64_t cap_runs,
                       uint64_t *n_runs_out);
int oracle_runs_decode(const uint32_t *runs_per_lane, const uint64_t *run_base, const int64_t *run_stride,
                       const uint32_t *run_count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                       uint64_t *addrs_out);

/* A device address range and the host image of its bytes. */
typedef struct {
  uint64_t dev_base;
  uint64_t bytes;
  uint8_t *host;
} oracle_region;

/* staging[(b * n_lanes + l) * seg_bytes + k] = src bytes at addr(l, b) + k */
int oracle_gather(const uint32_t *runs_per_lane, const uint64_t *run_base, const int64_t *run_stride,
                  const uint32_t *run_count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                  uint64_t seg_bytes, const oracle_region *regions, int n_regions, uint8_t *staging);
/* dst bytes at daddr(l, b) + k = staging[(b * n_lanes + l) * seg_bytes + k] */
int oracle_scatter(const uint32_t *runs_per_lane, const uint64_t *run_base, const int64_t *run_stride,
                   const uint32_t *run_count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                   uint64_t seg_bytes, const oracle_region *regions, int n_regions, const uint8_t *staging);

/* One contiguous read: bytes from device address src to slab offset dst_off. */
typedef struct {
  uint64_t src, dst_off, bytes;
} oracle_desc;

/* [RUNS] "What this PR does" steps 2-5 and "READ splitting": the descriptors
 * of the coalesced fetch, the slab size, and every segment's slab offset
 * (local[l * n_blocks + b]).  n_descs receives the count even when it
 * exceeds cap (then ORACLE_EARG). */
int oracle_groups_plan(const uint32_t *runs_per_lane, const uint64_t *run_base, const int64_t *run_stride,
                       const uint32_t *run_count, uint64_t n_runs, uint32_t n_lanes, uint32_t n_blocks,
                       uint64_t seg_bytes, const uint64_t *region_base, const uint64_t *region_bytes, int n_regions,
                       uint64_t max_read_bytes, oracle_desc *descs, uint64_t cap, uint64_t *n_descs,
                       uint64_t *slab_bytes, uint64_t *local);

/* slab[d.dst_off + k] = bytes at d.src + k for every descriptor. */
int oracle_copy_descs(const oracle_desc *descs, uint64_t n_descs, const oracle_region *regions, int n_regions,
                      uint8_t *slab, uint64_t slab_bytes);

/* [TE] paged writes: dst page dst_idx[k] <- src page src_idx[k], page_len
 * bytes, page i of a list at region start + offset + i * stride (offsets
 * relative to each region's host image). */
int oracle_paged_copy(uint64_t page_len, const oracle_region *src, const uint32_t *src_idx, uint64_t src_stride,
                      uint64_t src_offset, const oracle_region *dst, const uint32_t *dst_idx, uint64_t dst_stride,
                      uint64_t dst_offset, uint64_t n_pages);

#ifdef __cplusplus
}
#endif
#endif
