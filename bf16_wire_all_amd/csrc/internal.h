// Internal declarations shared by the host entry points and the kernel files
// of libxfer.  Nothing here is exported.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <new>
#include <stdexcept>
#include <type_traits>
#include <vector>

#include "xfer.h"

namespace xfer {

// Launch a kernel through hipLaunchKernel so the launch status is returned
// directly instead of being read back from the thread's sticky error slot.
template <typename... KArgs, typename... Args>
static inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                                Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  static_assert((std::is_same<KArgs, Args>::value && ...), "argument types must match the kernel exactly");
  void *argv[] = {(void *)&args...};
  return hipLaunchKernel((const void *)kernel, grid, block, argv, lds, stream);
}

// The same kernel and arguments as launch(), added as a node of graph g after
// the n_deps nodes in deps (the node copies the arguments).
template <typename... KArgs, typename... Args>
static inline hipError_t add_node(hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, hipGraphNode_t *node,
                                  void (*kernel)(KArgs...), dim3 grid, dim3 block, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  static_assert((std::is_same<KArgs, Args>::value && ...), "argument types must match the kernel exactly");
  void *argv[] = {(void *)&args...};
  hipKernelNodeParams p{};
  p.func = (void *)kernel;
  p.gridDim = grid;
  p.blockDim = block;
  p.sharedMemBytes = 0;
  p.kernelParams = argv;
  p.extra = nullptr;
  return hipGraphAddKernelNode(node, g, deps, n_deps, &p);
}

// Runs a set-up call's body and turns a failed host allocation into a status,
// so that no C++ exception crosses the C interface.
template <typename F>
inline int guarded(F &&body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc &) {
    return XFER_E_HOST_MEMORY;
  } catch (const std::length_error &) {
    return XFER_E_HOST_MEMORY;
  } catch (...) {
    return XFER_E_INVAL;
  }
}

// A dispatch holds at most 2^32 - 1 work-items along x (the packet's grid
// size is a 32-bit work-item count): 2^24 - 1 workgroups of 256 threads.
constexpr uint64_t kMaxGridBlocks = (1ull << 24) - 1;
// Pack and combine move 2048 elements per workgroup.
constexpr uint64_t kMaxStreamElems = kMaxGridBlocks * 2048;

// ---- paged copy (pages_copy.hip): 4 KiB units, two per workgroup
constexpr uint32_t kPageUnitBytes = 4096;
struct PagesView {
  const uint32_t *src_idx, *dst_idx;
  uint64_t src_base, src_stride, dst_base, dst_stride, page_len;
  uint32_t units_per_page, n_units;
  uint32_t span;    // a workgroup copies units c and c + span of a tile of 2 * span units
  uint32_t pieces;  // workgroups: ceil(n_units / (2 * span)) * span
};
hipError_t launch_paged_copy(const PagesView &v, hipStream_t stream);

// ---- host helpers shared by the entry points (api.cpp)
// Per declared region that holds segments, the [lo, hi) byte range of those
// segments (filled in region order when region_spans is not NULL).
struct Span {
  uint64_t lo, hi;
};
int validate_table(const xfer_run_table *t, const xfer_region *regions, int n_regions, int is_dst,
                   uint64_t *span_lo, uint64_t *span_hi, std::vector<Span> *region_spans);
// A plan keeps at most this many spans (xfer_runs_plan::spans,
// xfer_descs_plan::spans).
constexpr uint32_t kPlanSpans = 4;
// At most kPlanSpans ranges covering the given ones: sorted, overlapping or
// touching ranges joined, then the two with the smallest gap joined while
// there are more.
std::vector<Span> fold_spans(std::vector<Span> v);
// Whether [a, a + na) shares a byte with any of the n [lo, hi) pairs.
bool overlaps_spans(uintptr_t a, uint64_t na, const uint64_t *spans, uint32_t n);
// Plan-side check of a span list: at most kPlanSpans, each non-empty, and at
// least one when the plan has work.
bool spans_ok(const uint64_t *spans, uint32_t n, bool has_work);
bool run_addr(uint64_t base, int64_t stride, uint64_t k, uint64_t *out);

// ---- pack / combine (pack_combine.hip)
hipError_t launch_pack(const float *src, uint64_t n_elems, uint16_t *ring, uint64_t ring_elems,
                       uint64_t slot0_elem, hipStream_t stream);
hipError_t launch_combine(const uint16_t *a, const uint16_t *b, uint64_t n, void *out, int mode,
                          hipStream_t stream);
hipError_t launch_combine_f32(const float *a, const float *b, uint64_t n, void *out, int mode, hipStream_t stream);
// The same pack and combine launches as graph nodes (the graph form of the
// streamed all-reduce).
hipError_t node_pack(hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, hipGraphNode_t *node, const float *src,
                     uint64_t n_elems, uint16_t *ring, uint64_t ring_elems, uint64_t slot0_elem);
hipError_t node_combine(hipGraph_t g, const hipGraphNode_t *deps, size_t n_deps, hipGraphNode_t *node,
                        const uint16_t *a, const uint16_t *b, uint64_t n, void *out, int mode);

// ---- argmax (argmax.hip)
struct ArgmaxShard {
  const uint16_t *ptr;
  uint64_t ld;
  uint32_t ncols;
  uint32_t col_offset;
};
// Column slices per shard (the fold's wavefront holds 2 * splits partials) and
// the widest slice (a key carries a 16-bit column within its slice).
constexpr uint32_t kArgmaxMaxSplits = 32;
constexpr uint32_t kArgmaxMaxSliceCols = 65536;
constexpr uint64_t kArgmaxMaxShardCols = (uint64_t)kArgmaxMaxSplits * kArgmaxMaxSliceCols;
uint32_t argmax_splits(uint32_t rows, uint32_t ncols0, uint32_t ncols1);
uint64_t argmax_workspace_bytes(uint32_t rows, uint32_t splits);
hipError_t launch_argmax(ArgmaxShard s0, ArgmaxShard s1, uint32_t rows, int mode, void *out, void *workspace,
                         uint32_t splits, hipStream_t stream);
// The library's own argmax partials array (xfer_argmax_merge_noalloc): its
// device address on the current device, looked up on the first call made
// with that device current and kept per device.
constexpr uint64_t kArgmaxScratchBytes = XFER_ARGMAX_SCRATCH_BYTES;
hipError_t argmax_scratch(void **ptr);

// ---- run-table gather / scatter (runs_copy.hip)
struct PlanView {
  const uint32_t *group_run;  // [n_lanes][n_groups + 1]
  const uint32_t *run_start;  // [n_runs]
  const uint64_t *run_base;   // [n_runs]
  const int64_t *run_stride;  // [n_runs]
  uint32_t n_lanes, n_blocks;
  uint32_t lanes_per_wg;      // 1 or 2: a workgroup copies lanes l and l + lane_slots
  uint32_t lane_slots;        // ceil(n_lanes / lanes_per_wg)
  uint32_t tile_blocks;       // blocks per workgroup and lane; divides group_blocks
  uint32_t n_tiles;           // per lane
  uint32_t group_blocks;      // blocks per index entry
  uint32_t n_groups;          // per lane
  uint64_t seg_bytes;
  uint32_t vps;               // 16-byte vectors per segment, <= kMaxSegVectors
  uint32_t pieces;            // workgroups per segment (1, or vps / piece_vecs)
  uint32_t piece_vecs;        // vectors one workgroup copies per segment
  uint32_t piece_log2;        // log2(piece_vecs) if a power of two, else 32
};
constexpr uint32_t kMaxGroupBlocks = 32;
constexpr uint32_t kMaxTileBlocks = 32;
constexpr uint32_t kMaxLanesPerWorkgroup = 2;
constexpr uint32_t kMaxSegVectors = 1u << 16;  // 1 MiB segments
hipError_t launch_gather(const PlanView &p, void *staging, hipStream_t stream);
hipError_t launch_scatter(const PlanView &p, const void *staging, hipStream_t stream);

// ---- descriptor copies (descs_copy.hip) and paged copies (pages_copy.hip)
// Both cut their work into 4 KiB units and give a workgroup two units of a
// tile of 2T units, T apart: unit c and unit c + T of the tile, with
// T = min(kPairSpan, ceil(units / 2)).
constexpr uint32_t kDescPieceBytes = 8192;  // two units: the work of one workgroup
constexpr uint64_t kPairSpan = 576;         // units between a workgroup's two units (2.25 MiB)
__host__ __device__ inline uint64_t pair_span(uint64_t units) {
  const uint64_t half = (units + 1) / 2;
  return half < kPairSpan ? half : kPairSpan;
}
// Workgroups for a list of `units` units: ceil(units / 2T) tiles of T.
__host__ __device__ inline uint64_t paired_pieces(uint64_t units) {
  const uint64_t T = pair_span(units);
  return T ? (units + 2 * T - 1) / (2 * T) * T : 0;
}
hipError_t launch_copy_descs(const xfer_desc *descs, uint64_t n_descs, uint32_t max_pieces, void *slab,
                             hipStream_t stream);

}  // namespace xfer
