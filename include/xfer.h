/*
 * xfer.h - C ABI of libxfer, the staging and combine kernels around a
 * point-to-point tensor transfer, for AMD Instinct MI355X (gfx950).
 *
 * Pages the operations come from:
 *   [CE]   llama.cpp PR "Large all-reduces under -sm tensor now go through the
 *          copy engines" (Piggidragon fork, PR 16), section "Change".
 *   [TP2]  "The two-card (TP = 2) DSpark worker" (TP2.md), sections "Layout"
 *          and "Collectives".
 *   [RUNS] pegaflow PR 350 "run-encode QueryBlocksForTransfer addresses and
 *          coalesce RDMA READs", sections "Problem", "What this PR does" and
 *          "Trust boundary".
 *
 * Conventions shared by every call:
 *   - Pointers marked (device) are device addresses of the GPU that is current
 *     on the calling thread; pointers marked (host) are host memory.  The
 *     caller owns every buffer, including the run plans.  The library
 *     allocates no device memory itself; its only global state is the static
 *     partials array of xfer_argmax_merge_noalloc (one per GPU) and the cache
 *     of its addresses.  xfer_allreduce2_graph_create creates HIP graph
 *     objects, which the caller frees with xfer_allreduce2_graph_destroy.
 *   - Hot calls (pack, combine, argmax, gather, scatter, the descriptor and
 *     paged copies) only enqueue work on `stream`: they never allocate, never
 *     synchronise and never block.  The set-up calls that upload a plan
 *     (xfer_runs_prepare, xfer_descs_prepare, xfer_pages_prepare) block.
 *   - The set-up calls that sort or expand a table on the host
 *     (xfer_runs_validate, xfer_runs_prepare, xfer_groups_plan,
 *     xfer_descs_prepare, xfer_pages_prepare) use temporary host memory and
 *     return XFER_E_HOST_MEMORY when it cannot be allocated: no C++
 *     exception ever leaves the library.
 *   - Every call checks all its arguments on the host first.  On any status
 *     other than XFER_OK and XFER_E_DEVICE nothing has been enqueued and no
 *     output byte has been written.  XFER_E_DEVICE reports a launch or copy
 *     the HIP runtime refused; work enqueued before it may still run.  The
 *     outputs of a failed call must not be read.
 *   - Empty work (n == 0, rows == 0, an empty chunk range, an empty table) is
 *     XFER_OK with nothing enqueued; for xfer_pack_bf16 the chunk range is
 *     what counts (a chunk named with n == 0 starts at n, XFER_E_INVAL).
 *   - Every buffer a kernel streams through, and every row start and segment
 *     address, must be 16-byte aligned: the kernels move 64- and 128-bit
 *     vectors.  Element counts may be anything.
 *   - Results are deterministic and independent of launch shape: the same
 *     inputs give the same bits on every call and on every GPU.
 */
#ifndef XFER_H
#define XFER_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden visibility; only these calls are exported. */
#define XFER_API __attribute__((visibility("default")))

/* ------------------------------------------------------------ status codes */
enum {
  XFER_OK = 0,
  XFER_E_INVAL = 1,       /* bad pointer, size, alignment, mode or aliasing   */
  XFER_E_UNSUPPORTED = 2, /* valid request outside what the kernels handle    */
  XFER_E_TABLE = 3,       /* run table inconsistent                           */
  XFER_E_RANGE = 4,       /* a segment outside the declared regions, or an
                             address computation that overflows 64 bits       */
  XFER_E_OVERLAP = 5,     /* destination segments overlap each other          */
  XFER_E_DEVICE = 6,      /* the HIP runtime refused a launch or a copy       */
  XFER_E_HOST_MEMORY = 7  /* a set-up call could not allocate its host scratch
                             (no C++ exception ever leaves the library)       */
};

/* Static description of a status code (never NULL). */
XFER_API const char *xfer_status_str(int status);

/* -------------------------------------------------------------------- pack */

/*
 * xfer_pack_bf16 - [CE] "Change": a rank converts its F32 partial to BF16,
 * round to nearest with ties to even, into fixed-size chunks of a staging
 * ring; two slots alternate so one chunk can be converted while the previous
 * one is in flight.
 *
 *   src          (device) F32[n], the rank's partial.
 *   ring         (device) BF16 bit patterns, ring_bytes long, holding
 *                R = ring_bytes / chunk_bytes slots of chunk_bytes each.
 *   chunk_bytes  BF16 bytes per chunk (524288 = 512 KiB in [CE]); a multiple
 *                of 16.  CE = chunk_bytes / 2 elements per chunk.
 *   chunk_begin, chunk_end  the chunks this call packs.  Chunk c holds
 *                elements [c*CE, min((c+1)*CE, n)) and is written to slot
 *                c mod R: ring[(c mod R)*CE + j] = bf16_rne(src[c*CE + j]).
 *                Ring bytes past a short last chunk are not written.
 *
 * Rounding: IEEE round-to-nearest-even on the bit pattern, subnormals
 * rounded (not flushed), signs and infinities kept, every NaN written as the
 * canonical quiet NaN 0x7FC0.
 *
 * Errors: XFER_E_INVAL if a pointer is NULL or not 16-byte aligned, if
 * chunk_bytes is 0 or not a multiple of 16, if ring_bytes is not a non-zero
 * multiple of chunk_bytes, if chunk_end - chunk_begin > R (two chunks of one
 * call would share a slot), if a named chunk starts at or past n, or if src
 * and ring overlap; XFER_E_UNSUPPORTED if the call's range holds more than
 * (2^24 - 1) * 2048 elements (one launch).
 */
XFER_API int xfer_pack_bf16(const float *src, size_t n, uint16_t *ring, size_t ring_bytes, size_t chunk_bytes,
                   size_t chunk_begin, size_t chunk_end, hipStream_t stream);

/* ----------------------------------------------------------------- combine */

enum { XFER_OUT_F32 = 0, XFER_OUT_BF16 = 1 };

/*
 * xfer_combine2 - [CE] "Change" (the sum kernel) and [TP2] "Layout" (fp32
 * sums rounded to bf16): out[i] = f32(a[i]) + f32(b[i]), one IEEE binary32
 * addition with rank 0's value as the first operand on both ranks, so both
 * ranks get identical bits.
 *
 *   a_rank0, b_rank1  (device) BF16 bit patterns, n each.
 *   out               (device) F32[n] for XFER_OUT_F32, or BF16[n] for
 *                     XFER_OUT_BF16 (the F32 sum rounded to nearest even).
 *
 * Subnormals are kept.  A NaN result is written as 0x7FC00000 (F32) or
 * 0x7FC0 (BF16).
 *
 * Errors: XFER_E_INVAL for NULL or misaligned pointers, an unknown out_mode,
 * or an output that overlaps an input (except out == a_rank0 or
 * out == b_rank1 exactly in BF16 mode, which is computed in place);
 * XFER_E_UNSUPPORTED for n above (2^24 - 1) * 2048 (one launch).
 */
XFER_API int xfer_combine2(const uint16_t *a_rank0, const uint16_t *b_rank1, size_t n, void *out, int out_mode,
                  hipStream_t stream);

/*
 * xfer_combine2_f32 - the F32-wire all-reduce of [TP2] "Layout" and
 * "Collectives" (the drafter's partials are pushed as F32, not BF16):
 * out[i] = a[i] + b[i], one IEEE binary32 addition with rank 0's value first
 * (so both ranks get identical bits), written as F32 (XFER_OUT_F32) or as
 * that F32 sum rounded to BF16 with round to nearest even (XFER_OUT_BF16,
 * the page's "fp32 sums rounded to bf16": two roundings, in that order).
 *
 *   a_rank0, b_rank1  (device) F32[n] each.
 *   out               (device) F32[n] or BF16[n] bit patterns.
 *
 * Subnormals are kept; a NaN sum is written as 0x7FC00000 (F32) or 0x7FC0
 * (BF16).
 *
 * Errors: XFER_E_INVAL for NULL or misaligned (16-byte) pointers, an unknown
 * out_mode, or an output overlapping an input (except out == a_rank0 or
 * out == b_rank1 exactly in F32 mode, computed in place);
 * XFER_E_UNSUPPORTED for n above (2^24 - 1) * 2048 (one launch).
 */
XFER_API int xfer_combine2_f32(const float *a_rank0, const float *b_rank1, size_t n, void *out, int out_mode,
                               hipStream_t stream);

/* ------------------------------------------------------------ argmax merge */

enum { XFER_ARGMAX = 0, XFER_TOP2 = 1 };

/* One shard of a block of logit rows: BF16 bit patterns, row-major. */
typedef struct {
  const uint16_t *ptr; /* (device) element (0, 0) of the shard             */
  size_t ld;           /* elements between the starts of consecutive rows  */
  uint32_t rows;
  uint32_t ncols;      /* 1 .. 2,097,152                                   */
  uint32_t col_offset; /* global id of the shard's column 0                */
} xfer_shard;

typedef struct {
  float max;   /* exact F32 value of the winning BF16 element */
  int32_t idx; /* its global id                               */
} xfer_max_idx;  /* 8 bytes  */

typedef struct {
  float top1, top2; /* first and second element of the row's order    */
  int32_t idx;      /* global id of top1                               */
  int32_t reserved; /* written as 0                                    */
} xfer_top2;        /* 16 bytes */

/*
 * xfer_argmax_merge - [TP2] "Layout": the vocabulary is split by columns
 * between two ranks, rank 0 holding the lower ids so that a tie of the global
 * argmax goes to the lower id as on one card; each rank's (shard max, index),
 * or (top1, top2, index) when the margin is wanted, is exchanged and folded.
 *
 * Row order: larger value first (numeric, so -0 == +0), then the lower
 * global id.  Per row, each shard's first two elements are found, then
 * folded: global top1 is the earlier shard top1; global top2 is the earlier
 * of the other shard's top1 and the winner's top2.  Values are the exact F32
 * of the chosen BF16 elements (their own bits, so the sign of a zero is the
 * chosen element's).  NaN logits are outside the contract: the output for a
 * row holding a NaN is unspecified, but always a record of that row.
 *
 *   out        (device) xfer_max_idx[rows] (XFER_ARGMAX) or
 *              xfer_top2[rows] (XFER_TOP2).
 *   workspace  (device) at least xfer_argmax_workspace_bytes(rows, s0->ncols,
 *              s1->ncols) bytes, 16-byte aligned, any contents: the call writes
 *              per-slice partial records there and reads them back (it needs
 *              no initialisation and its contents afterwards are unspecified).
 *              Calls that may run concurrently must use different workspaces.
 *
 * Errors: XFER_E_INVAL for NULL or misaligned pointers (ptr and ld * 2 must
 * be multiples of 16), different row counts, ncols == 0, shards whose id
 * ranges overlap, col_offset + ncols > 2^31, an unknown mode, a small
 * workspace, or an output overlapping the logits or the workspace;
 * XFER_E_UNSUPPORTED for a shard wider than 2,097,152 columns (32 slices of
 * at most 65,536) or more than 2^23 - 1 rows.
 */
XFER_API size_t xfer_argmax_workspace_bytes(uint32_t rows, uint32_t ncols0, uint32_t ncols1);
XFER_API int xfer_argmax_merge(const xfer_shard *s0, const xfer_shard *s1, int mode, void *out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * xfer_argmax_merge_noalloc - xfer_argmax_merge for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It takes no workspace; the per-slice
 * partial records go to a static device array of the library,
 * XFER_ARGMAX_SCRATCH_BYTES bytes on each GPU the library runs on, held
 * until the process ends.  The array's address on a device is looked up
 * (hipGetSymbolAddress) on the first call made with that device current and
 * kept; the call allocates nothing and needs no initialised memory (every
 * partial record is written before it is read).
 *
 * Every call on one GPU shares that GPU's array and leaves its last
 * contents there: calls that may overlap in time on one GPU (on different
 * streams, or from different host threads without ordering) race, and their
 * outputs are then undefined.  Order such calls on one stream.
 *
 * Arguments, outputs and errors as xfer_argmax_merge without the workspace,
 * plus XFER_E_UNSUPPORTED when the partial records need more than
 * XFER_ARGMAX_SCRATCH_BYTES (xfer_argmax_workspace_bytes above it: with
 * shards of at most 65,536 columns, more than 4096 rows), and XFER_E_DEVICE
 * if the array's address cannot be obtained.
 */
#define XFER_ARGMAX_SCRATCH_BYTES 65536
XFER_API int xfer_argmax_merge_noalloc(const xfer_shard *s0, const xfer_shard *s1, int mode, void *out,
                                       hipStream_t stream);

/* ------------------------------------------------------------- run tables */

/*
 * A run-encoded address table, [RUNS] "What this PR does": parallel arrays
 * runs_per_lane / run_base / run_stride / run_count.  A lane is one slot's K
 * or V segment across the blocks; along a lane the addresses of consecutive
 * blocks form arithmetic runs addr = base + i * stride, i < count
 * ([RUNS] "Problem").  Runs are stored lane after lane and cover the lane's
 * blocks in order: run r of a lane covers blocks [start_r, start_r + count_r)
 * with start_r the sum of the counts of the lane's earlier runs.
 *
 * All array pointers are (host).  run_base values are device addresses.
 */
typedef struct {
  uint32_t n_lanes;
  uint32_t n_blocks;
  uint64_t seg_bytes; /* bytes per segment (4096 in [RUNS])            */
  uint64_t n_runs;
  const uint32_t *runs_per_lane; /* [n_lanes]                        */
  const uint64_t *run_base;      /* [n_runs]                         */
  const int64_t *run_stride;     /* [n_runs], ignored when count == 1 */
  const uint32_t *run_count;     /* [n_runs]                         */
} xfer_run_table;

/* A device address range that segments may occupy. */
typedef struct {
  uint64_t base;
  uint64_t bytes;
} xfer_region;

/*
 * xfer_runs_encode - the holder side of [RUNS] "What this PR does": feed the
 * segment addresses of each lane, block by block, into a greedy run
 * accumulator.  A run holding one address takes the next non-zero delta
 * (that fits a signed 64-bit stride) as its stride; a longer run grows while
 * the delta equals its stride; any other address starts a new run.  The
 * stride of a one-address run is written as 0.
 *
 *   addrs        (host) uint64[n_lanes][n_blocks], lane-major.
 *   max_count    0 for unlimited, else the longest run allowed (1 gives one
 *                run per segment, the unencoded worst case).
 *   out arrays   (host) runs_per_lane[n_lanes]; run_base, run_stride and
 *                run_count of capacity cap_runs each.
 *   *n_runs_out  receives the number of runs written.
 * Errors: XFER_E_INVAL for NULL pointers, XFER_E_RANGE if cap_runs is too
 * small.  Host only; usable without a GPU.
 */
XFER_API int xfer_runs_encode(const uint64_t *addrs, uint32_t n_lanes, uint32_t n_blocks, uint32_t max_count,
                     uint32_t *runs_per_lane, uint64_t *run_base, int64_t *run_stride, uint32_t *run_count,
                     uint64_t cap_runs, uint64_t *n_runs_out);

/*
 * xfer_runs_validate - [RUNS] "Trust boundary": the table is remote input and
 * is checked completely before any memory is touched.  Host only; usable
 * without a GPU.  Checks, in this order, each failure returning at once:
 *   XFER_E_INVAL  t or a needed array is NULL; n_regions < 0 or regions NULL
 *                 with n_regions > 0; seg_bytes is 0 ("no zero-size slots")
 *                 or not a multiple of 16; a region that wraps past 2^64;
 *   XFER_E_UNSUPPORTED  n_runs or n_lanes * n_blocks above 2^32 - 1, or
 *                 seg_bytes above 1 MiB;
 *   XFER_E_TABLE  the runs_per_lane sum differs from n_runs, a run has count
 *                 0, or a lane's counts do not sum to n_blocks;
 *   XFER_E_RANGE  a run's base, or its stride when count > 1, is not a
 *                 multiple of 16, or its address span [lowest address,
 *                 highest address + seg_bytes) overflows 64 bits or does not
 *                 lie inside one region;
 *   XFER_E_OVERLAP (is_dst != 0 only) two segments share a byte: the
 *                 result would depend on the order of the writes.
 */
XFER_API int xfer_runs_validate(const xfer_run_table *t, const xfer_region *regions, int n_regions, int is_dst);

/*
 * A validated table laid out for the kernels in a caller-owned device buffer.
 * Caller-held plain data: copy it freely; it stays valid while `dev` holds
 * what xfer_runs_prepare wrote there.  The remaining fields are private.
 */
typedef struct {
  void *dev;          /* (device) the plan buffer                   */
  uint64_t dev_bytes;
  uint32_t n_lanes, n_blocks;
  uint64_t seg_bytes;
  uint64_t n_runs;
  uint64_t span_lo, span_hi; /* byte range covering every segment      */
  uint32_t is_dst;
  uint32_t tile_blocks;      /* private from here on                   */
  uint32_t n_tiles;
  uint32_t group_blocks;
  uint32_t n_groups;
  uint32_t pieces;
  uint32_t magic;
  uint32_t lanes_per_wg;
  uint64_t off_group_run, off_run_start, off_run_base, off_run_stride;
  uint32_t n_spans, reserved;
  uint64_t spans[8];         /* up to 4 [lo, hi) pairs, see xfer_gather_runs */
} xfer_runs_plan;

/* Device bytes xfer_runs_prepare needs for table t (0 if t is NULL). */
XFER_API size_t xfer_runs_plan_bytes(const xfer_run_table *t);

/*
 * xfer_runs_prepare - validate t exactly as xfer_runs_validate does, then
 * write the kernels' form of it into dev (device, 16-byte aligned, at least
 * xfer_runs_plan_bytes(t) bytes) with a blocking host-to-device copy, and
 * fill *out.  Returns the validation status, XFER_E_INVAL for a small or
 * misaligned dev, XFER_E_UNSUPPORTED if the set needs more than 2^24 - 1
 * workgroups (about 8 KiB each: a set of more than ~128 GiB), or
 * XFER_E_DEVICE if the copy fails.
 */
XFER_API int xfer_runs_prepare(const xfer_run_table *t, const xfer_region *regions, int n_regions, int is_dst, void *dev,
                      size_t dev_bytes, xfer_runs_plan *out);

/*
 * xfer_gather_runs - the data movement of [RUNS] "What this PR does" steps
 * 2-4 (decode the runs and read every segment into a dense local buffer):
 *   staging[(b * n_lanes + l) * seg_bytes + k] = *(addr(l, b) + k)
 * for every lane l, block b and k < seg_bytes, with addr(l, b) decoded from
 * the run of lane l that covers block b.  Staging is block-major, lanes
 * inside a block.
 *
 *   staging  (device) at least n_lanes * n_blocks * seg_bytes bytes,
 *            16-byte aligned, and sharing no byte with the plan's segment
 *            spans: per declared region that holds segments, the range from
 *            its lowest to its highest segment byte.  A plan keeps at most
 *            four such ranges; beyond four, the two nearest are merged until
 *            four remain (so a buffer between two far-apart regions is
 *            accepted, one inside a region's segment range is not).
 * Errors: XFER_E_INVAL for a NULL / foreign / destination plan, a small,
 * misaligned or overlapping staging buffer.
 */
XFER_API int xfer_gather_runs(const xfer_runs_plan *src_plan, void *staging, size_t staging_bytes, hipStream_t stream);

/*
 * xfer_scatter_runs - the inverse placement, [RUNS] "What this PR does" step
 * 5 (every block placed at its own local address) done as data movement:
 *   *(daddr(l, b) + k) = staging[(b * n_lanes + l) * seg_bytes + k]
 * with daddr decoded from dst_plan (prepared with is_dst != 0, so its
 * segments are disjoint).  No other destination byte is written.
 * Errors: XFER_E_INVAL for a NULL / foreign / source plan, a small, misaligned
 * or overlapping staging buffer.
 */
XFER_API int xfer_scatter_runs(const void *staging, size_t staging_bytes, const xfer_runs_plan *dst_plan,
                      hipStream_t stream);

/* ------------------------------------------ coalesced fetch by dense group */

/* One contiguous copy: bytes from device address src to slab offset dst_off. */
typedef struct {
  uint64_t src;
  uint64_t dst_off;
  uint64_t bytes;
} xfer_desc;

/*
 * xfer_groups_plan - the requester's planning of [RUNS] "What this PR does"
 * steps 2-4 and "READ splitting", host only:
 *   1. runs are bucketed by the region that holds them and sorted by base;
 *   2. sweeping that order, a run joins the open group when it covers the
 *      same blocks, has the same stride, starts where the group's per-block
 *      chunk ends, and the grown chunk still fits the stride (|stride| >=
 *      chunk, any chunk for one-block runs); otherwise it opens a new group;
 *   3. a group whose per-block chunks are back to back (|stride| == chunk, or
 *      one block) is dense: one contiguous range, mirrored into the slab as
 *      is; any other group is read block by block into a dense local mirror;
 *   4. every range is split into descriptors of at most max_desc_bytes
 *      (32 MiB in [RUNS]).
 * Groups are laid out in the slab in that order.  The rebuilt local address
 * of every segment is arithmetic ([RUNS] step 5): local_base[r] and
 * local_stride[r] give run r's segments as slab offsets
 * (local = local_base[r] + i * local_stride[r]), so the table with these
 * arrays addresses the slab.
 *
 *   t, regions     as xfer_runs_validate (source table); validated first.
 *   descs          (host) capacity cap_descs; *n_descs receives the count.
 *   slab_bytes     receives the slab size (the sum of the descriptor bytes).
 *   local_base, local_stride  (host) n_runs each.
 *   n_groups, n_dense  receive the group counts (may be NULL).
 * Errors: those of xfer_runs_validate; XFER_E_INVAL for NULL outputs or a
 * max_desc_bytes that is 0 or not a multiple of 16; XFER_E_RANGE if
 * cap_descs is too small (then *n_descs holds the count needed; descs NULL
 * with cap_descs 0 asks for the count only).
 */
XFER_API int xfer_groups_plan(const xfer_run_table *t, const xfer_region *regions, int n_regions,
                              uint64_t max_desc_bytes, xfer_desc *descs, uint64_t cap_descs, uint64_t *n_descs,
                              uint64_t *slab_bytes, uint64_t *local_base, int64_t *local_stride, uint64_t *n_groups,
                              uint64_t *n_dense);

/* A validated descriptor list in a caller-owned device buffer (plain data). */
typedef struct {
  void *dev;
  uint64_t dev_bytes;
  uint64_t n_descs;
  uint64_t slab_bytes;
  uint64_t src_lo, src_hi;  /* byte range covering every source range */
  uint32_t max_pieces;      /* private from here on */
  uint32_t piece_bytes;
  uint32_t magic;
  uint32_t reserved;
  uint32_t n_spans, reserved2;
  uint64_t spans[8];        /* up to 4 [lo, hi) pairs, see xfer_copy_descs */
} xfer_descs_plan;

XFER_API size_t xfer_descs_plan_bytes(uint64_t n_descs);

/*
 * xfer_descs_prepare - check a descriptor list and upload it (blocking):
 * every descriptor has bytes > 0 and src, dst_off, bytes multiples of 16,
 * no source range wraps or leaves the declared regions (XFER_E_RANGE), the
 * destination ranges lie in [0, slab_bytes) and are pairwise disjoint
 * (XFER_E_OVERLAP).  dev: device, 16-byte aligned, xfer_descs_plan_bytes().
 * XFER_E_UNSUPPORTED if n_descs times the largest descriptor's workgroup
 * count (about one per 8 KiB) exceeds 2^24 - 1 (the kernel's grid).
 */
XFER_API int xfer_descs_prepare(const xfer_desc *descs, uint64_t n_descs, uint64_t slab_bytes,
                                const xfer_region *regions, int n_regions, void *dev, size_t dev_bytes,
                                xfer_descs_plan *out);

/*
 * xfer_copy_descs - execute the plan: slab[dst_off + k] = *(src + k) for every
 * descriptor, k < bytes.  slab (device) is slab_bytes long at least, 16-byte
 * aligned, and shares no byte with the plan's source spans: per declared
 * region that holds sources, the range from its lowest to its highest source
 * byte (at most four ranges; beyond four the two nearest are merged, as for
 * run plans).
 */
XFER_API int xfer_copy_descs(const xfer_descs_plan *plan, void *slab, size_t slab_bytes, hipStream_t stream);

/* ------------------------------------------------ paged copy (Pages lists) */

/*
 * A page list of [TE] (the Pages type of the TransferEngine API, which its
 * paged writes take for both ends): page k of the list lies at
 * region base + offset + indices[k] * stride.  The page names pages only by
 * indices, a stride and an offset; this is the plainest reading.
 */
typedef struct {
  const uint32_t *indices; /* (host) one index per page                        */
  uint64_t stride;         /* bytes per index step, multiple of 16             */
  uint64_t offset;         /* bytes from the region base to index 0, mult. 16  */
} xfer_pages;

/* Filled by xfer_pages_prepare; the caller owns dev. */
typedef struct {
  void *dev;
  size_t dev_bytes;
  uint64_t n_pages, page_len;
  uint64_t src_base, src_stride; /* region base + offset, and the stride */
  uint64_t dst_base, dst_stride;
  uint64_t off_src_idx, off_dst_idx; /* index arrays inside dev */
  uint32_t units_per_page;           /* ceil(page_len / 4096)    */
  uint32_t magic;
} xfer_pages_plan;

/* Device bytes xfer_pages_prepare needs for n_pages pages. */
XFER_API size_t xfer_pages_plan_bytes(uint64_t n_pages);

/*
 * xfer_pages_prepare - check two page lists of n_pages pages each and upload
 * their indices (blocking): source page k will be copied to destination page
 * k, page_len bytes.  src and dst are the regions the lists address (their
 * base is the device address of the region, 16-byte aligned).  Checks, in
 * this order:
 *   XFER_E_INVAL  NULL out, regions or page lists (with n_pages > 0), a
 *                 page_len that is 0 or not a multiple of 16, a stride,
 *                 offset or region base not a multiple of 16, or a region
 *                 that wraps past 2^64;
 *   XFER_E_UNSUPPORTED  more than 2^32 - 1 units of 4 KiB, or a grid above
 *                 2^24 - 1 workgroups;
 *   XFER_E_RANGE  a page (either list) not wholly inside its region, or
 *                 offset arithmetic that overflows 64 bits;
 *   XFER_E_OVERLAP  two destination pages that overlap, or (when the two
 *                 regions overlap or are one region, as for a copy within
 *                 one buffer) a destination page that shares a byte with a
 *                 source page;
 *   XFER_E_INVAL  dev NULL, misaligned or smaller than
 *                 xfer_pages_plan_bytes(n_pages);
 *   XFER_E_DEVICE  the upload failed.
 */
XFER_API int xfer_pages_prepare(uint64_t page_len, const xfer_region *src, const xfer_pages *src_pages,
                                const xfer_region *dst, const xfer_pages *dst_pages, uint64_t n_pages, void *dev,
                                size_t dev_bytes, xfer_pages_plan *out);

/*
 * xfer_paged_copy - [TE] paged writes done as data movement on one GPU: for
 * every k, the page_len bytes of source page k are copied to destination
 * page k.  A gather is a destination list of consecutive indices; a scatter
 * a source list of consecutive indices.
 * Errors: XFER_E_INVAL for a NULL or foreign plan.
 */
XFER_API int xfer_paged_copy(const xfer_pages_plan *plan, hipStream_t stream);

/* -------------------------------------------- streamed two-rank all-reduce */

/*
 * The copy-engine all-reduce of [CE] "Change", both ranks emulated on one GPU:
 * per chunk, each rank converts its F32 chunk to BF16 into a slot of its send
 * ring (xfer_pack_bf16), the chunk crosses the "wire" (a device-to-device copy
 * into the peer's receive ring, on the sending rank's wire stream), and each
 * rank sums its own and the peer's chunk in F32 with rank 0's value first
 * (xfer_combine2), so both ranks get identical bits.  R slots alternate
 * (R = 2 in [CE]); the streams are ordered by events only and the host never
 * waits.
 *
 * The schedule is a list of operations, each on one of four streams
 * (compute 0, compute 1, wire 0, wire 1):
 *   PACK r c       compute r: wait SENT[r][s] of chunk c - R (slot free); for c < R also
 *                             wait COMBINED[r][s] (the previous call's last reader of the slot,
 *                             maybe on other streams); pack; record PACKED[r][s]
 *   WIRE r c       wire r:    wait PACKED[r][s]; wait COMBINED[1-r][s] of chunk c - R (peer slot free);
 *                             copy send[r] slot s -> recv[1-r] slot s; record SENT[r][s]
 *   COMBINE r c    compute r: wait SENT[1-r][s]; combine; record COMBINED[r][s]
 * with s = c mod R.  The events are created already recorded and complete
 * (xfer_events_create), so the first R chunks of a call either proceed at
 * once or wait for the previous call that used the same events and rings.
 * With R >= 2, from chunk R on the slot-free waits (PACK's, WIRE's
 * COMBINED) are left out: stream order and the waits of chunk c - 1 already
 * order them (PACK r c follows COMBINE r c-1, which follows the peer's copy of
 * chunk c-1, which follows the peer's pack of chunk c-1 and so the peer's
 * earlier combines and copies).  Each operation keeps its record.  xfer_allreduce2_schedule returns the list (host
 * only, no GPU), so the ordering can be checked without running it.
 */
enum { XFER_OP_PACK = 0, XFER_OP_WIRE = 1, XFER_OP_COMBINE = 2 };
enum { XFER_EV_PACKED = 0, XFER_EV_SENT = 1, XFER_EV_COMBINED = 2 };

typedef struct {
  uint32_t kind;     /* XFER_OP_*                                                  */
  uint32_t rank;     /* 0 or 1                                                     */
  uint32_t chunk;
  uint32_t slot;     /* chunk mod R                                                */
  uint32_t stream;   /* 0, 1: compute stream of rank 0, 1; 2, 3: wire stream of 0, 1 */
  uint32_t n_waits;  /* 0..2                                                       */
  uint32_t wait_event[2]; /* event ids waited on before the operation              */
  uint32_t record_event;  /* event id recorded after it                            */
} xfer_op;

/* Event id of (kind, rank, slot): (kind * 2 + rank) * R + slot; 6 * R events. */
XFER_API uint32_t xfer_allreduce2_event_id(uint32_t kind, uint32_t rank, uint32_t slot, uint32_t R);

/*
 * xfer_allreduce2_schedule - the operation list for n_chunks chunks and R
 * slots, in issue order (3 operations per rank per chunk).  ops (host) has
 * capacity cap; *n_ops receives the count.
 * Errors: XFER_E_INVAL for R == 0 or NULL pointers, XFER_E_RANGE if cap is
 * too small.  Host only.
 */
XFER_API int xfer_allreduce2_schedule(uint32_t n_chunks, uint32_t R, xfer_op *ops, size_t cap, size_t *n_ops);

/* Create n events without timing, each recorded once on the null stream and
 * completed before returning; destroy them.  Host resources for the driver
 * (set-up calls: they may block and allocate runtime objects).  On
 * XFER_E_DEVICE from xfer_events_create every event it created has been
 * destroyed again and all n slots are NULL. */
XFER_API int xfer_events_create(hipEvent_t *events, int n);
XFER_API int xfer_events_destroy(hipEvent_t *events, int n);

typedef struct {
  const float *src[2];    /* (device) rank r's F32 partial, n elements                */
  uint16_t *send[2];      /* (device) rank r's send ring, ring_bytes                  */
  uint16_t *recv[2];      /* (device) rank r's receive ring, ring_bytes               */
  void *out[2];           /* (device) rank r's result: n F32 or n BF16 patterns       */
  size_t n;
  size_t chunk_bytes;     /* BF16 bytes per chunk, multiple of 16 (524288 in [CE])    */
  size_t ring_bytes;      /* R * chunk_bytes                                          */
  int out_mode;           /* XFER_OUT_F32 or XFER_OUT_BF16                            */
  hipStream_t compute[2]; /* rank r's conversion and sum stream                       */
  hipStream_t wire[2];    /* rank r's outgoing copy stream                            */
  hipEvent_t *events;     /* (host) n_events events from xfer_events_create           */
  size_t n_events;        /* entries of events; at least 6 * R                        */
} xfer_allreduce2_desc;

/*
 * xfer_allreduce2_streamed - enqueue the whole schedule; returns without
 * waiting.  out[0] and out[1] both receive combine2(pack(src[0]),
 * pack(src[1])) element by element.  The sources must be ready on the compute
 * streams; the outputs are complete when both compute streams have run past
 * this call.  A later call with the same rings and events is ordered after
 * this one by the events themselves.
 * Errors: XFER_E_INVAL for NULL or misaligned buffers, a bad chunk or ring
 * size, an unknown out_mode, any two of the eight buffers overlapping (the
 * two sources excepted: both are only read), events NULL or n_events below
 * 6 * R; XFER_E_DEVICE if the runtime refuses an enqueue (earlier chunks may
 * already be enqueued).
 */
XFER_API int xfer_allreduce2_streamed(const xfer_allreduce2_desc *d);

/*
 * xfer_allreduce2_graph_create - the same all-reduce built once as a HIP graph
 * over the descriptor's buffers, so that a whole all-reduce costs one launch
 * (the streamed call makes three to four runtime calls per operation and is
 * bound by them at 512 KiB chunks).  Every operation of the schedule becomes
 * a node: a pack or combine kernel node, or a device-to-device copy node for
 * the wire.  Its dependencies are the ones xfer_allreduce2_graph_deps lists:
 * the previous operation on its stream and, for each event it waits on, the
 * operation that last recorded that event earlier in the all-reduce.  There is
 * no stream capture: d->compute, d->wire, d->events and d->n_events are not
 * used (they may be NULL / 0).  The graph holds the buffer addresses; the
 * caller keeps the buffers alive and unmoved while the graph exists.
 * Launches on one stream run one after the other; launches on different
 * streams that share buffers must be ordered by the caller.
 * Errors: those of xfer_allreduce2_streamed's descriptor checks (XFER_E_INVAL,
 * a NULL exec included); XFER_E_DEVICE if the runtime refuses a node or the
 * instantiation; XFER_E_HOST_MEMORY if host scratch cannot be allocated.
 * n == 0: XFER_OK and *exec = NULL (nothing to launch).  Set-up call: it
 * allocates host memory and runtime objects.
 *
 * xfer_allreduce2_graph_launch - enqueue one all-reduce on stream (a NULL
 * exec is a no-op).  xfer_allreduce2_graph_destroy - release the graph (NULL
 * is a no-op).
 *
 * xfer_allreduce2_graph_deps - the graph form's dependency list for n_chunks
 * chunks and R slots, host only: dependency k says operation to[k] (an index
 * into xfer_allreduce2_schedule's list) runs after operation from[k].  from
 * and to (host) have capacity cap; *n_deps receives the count.  Errors:
 * XFER_E_INVAL for R == 0 or NULL n_deps, XFER_E_RANGE if cap is too small
 * (from and to may then be NULL with cap 0, to ask for the count).
 */
XFER_API int xfer_allreduce2_graph_deps(uint32_t n_chunks, uint32_t R, uint32_t *from, uint32_t *to, size_t cap,
                                        size_t *n_deps);
XFER_API int xfer_allreduce2_graph_create(const xfer_allreduce2_desc *d, hipGraphExec_t *exec);
XFER_API int xfer_allreduce2_graph_launch(hipGraphExec_t exec, hipStream_t stream);
XFER_API int xfer_allreduce2_graph_destroy(hipGraphExec_t exec);

#ifdef __cplusplus
}
#endif
#endif /* XFER_H */
