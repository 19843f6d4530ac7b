// Gather / scatter of fixed-size segments addressed by a run-encoded table.
//
// Work unit: one workgroup per (lane l, tile of tile_blocks consecutive
// blocks).  Consecutive workgroups take consecutive lanes of the same block
// tile, so at any moment the chip is reading and writing a few neighbouring
// address windows rather than scattered ones.  Tiles are small (2 blocks of
// 4 KiB by default): many short workgroups, each moving 8 KiB in one pass,
// kept HBM busier on MI355X than fewer long ones (measured 6.0-6.4 TB/s
// against 5.2-5.4 TB/s for 32-block tiles).
//
// Decode, staged in LDS (no per-segment address table exists anywhere):
//   1. the plan's group index (one entry per lane and group of 32 blocks)
//      gives the first run covering the workgroup's group and, via the next
//      entry, the last one: at most 33 runs, loaded in parallel into LDS;
//   2. each block of the tile finds its run by binary search over the LDS
//      run starts and computes addr = base + (b - start) * stride;
//   3. the segment copies read those addresses from LDS (a wave mostly reads
//      one entry: an LDS broadcast).
// Copy: each segment moves as 16-byte vectors, consecutive threads on
// consecutive vectors, up to UNROLL vectors loaded before the first store.
// Loads and stores carry the nontemporal hint: every byte is touched once, so
// keeping it in L2 / the Infinity Cache only evicts other data.  All offsets
// are 64-bit (the staging buffer of the paged K/V workload is 2.36 GB).
#include "internal.h"

namespace xfer {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

// Device addresses come from the plan as integers; naming the global address
// space lets the compiler emit global (not flat) loads and stores.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) v4u g_v4u;
__device__ __forceinline__ v4u load16(uint64_t a) {
  return __builtin_nontemporal_load(reinterpret_cast<const g_v4u *>(a));
}
__device__ __forceinline__ void store16(uint64_t a, v4u v) {
  __builtin_nontemporal_store(v, reinterpret_cast<g_v4u *>(a));
}

// Vector v of the workgroup's share (v < nb * w, w = piece_vecs) is vector
// v0 + v mod w of the tile's segment v / w.  Segments hold at most 2^16
// vectors (host check), so all tile-local indices fit 32 bits; POW2 replaces
// the division by a shift.
template <bool POW2>
__device__ __forceinline__ void split_index(uint32_t v, uint32_t w, uint32_t w_log2, uint32_t &j, uint32_t &o) {
  if (POW2) {
    j = v >> w_log2;
    o = v & (w - 1);
  } else {
    j = v / w;
    o = v - j * w;
  }
}

template <bool GATHER, bool POW2>
__global__ __launch_bounds__(kThreads) void runs_copy_kernel(PlanView p, uint8_t *staging_w,
                                                             const uint8_t *staging_r) {
  __shared__ uint32_t s_start[kMaxGroupBlocks + 1];
  __shared__ uint64_t s_base[kMaxGroupBlocks + 1];
  __shared__ int64_t s_stride[kMaxGroupBlocks + 1];
  __shared__ uint64_t s_addr[kMaxTileBlocks];

  // Workgroup -> (piece, lane, tile), pieces fastest: consecutive workgroups
  // stream consecutive pieces of one segment, then the next lane's.
  const uint32_t piece = blockIdx.x % p.pieces;
  const uint32_t rest = blockIdx.x / p.pieces;
  const uint32_t l = rest % p.n_lanes;
  const uint32_t t = rest / p.n_lanes;
  const uint32_t b0 = t * p.tile_blocks;
  const uint32_t nb = min(p.tile_blocks, p.n_blocks - b0);
  const uint32_t tid = threadIdx.x;

  // Runs covering the tile's group of blocks (the tile lies inside one group).
  const uint32_t g = b0 / p.group_blocks;
  const uint32_t *gr = p.group_run + (uint64_t)l * (p.n_groups + 1);
  const uint32_t r0 = gr[g];
  const uint32_t lane_end = gr[p.n_groups];
  const uint32_t r1 = min(gr[g + 1] + 1, lane_end);
  const uint32_t nr = r1 - r0;  // <= group_blocks + 1

  for (uint32_t i = tid; i < nr; i += kThreads) {
    s_start[i] = p.run_start[r0 + i];
    s_base[i] = p.run_base[r0 + i];
    s_stride[i] = p.run_stride[r0 + i];
  }
  __syncthreads();
  for (uint32_t j = tid; j < nb; j += kThreads) {
    const uint32_t b = b0 + j;
    // last run i with s_start[i] <= b; s_start[0] <= group start <= b
    uint32_t lo = 0, hi = nr;
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) / 2;
      if (s_start[mid] <= b)
        lo = mid;
      else
        hi = mid;
    }
    s_addr[j] = s_base[lo] + (uint64_t)(b - s_start[lo]) * (uint64_t)s_stride[lo];
  }
  __syncthreads();

  const uint32_t w = p.piece_vecs;
  const uint64_t v0 = (uint64_t)piece * w;  // first vector of this workgroup's piece
  const uint32_t total = nb * w;
  const uint64_t block_step = (uint64_t)p.n_lanes * p.seg_bytes;  // staging bytes between blocks
  const uint8_t *stage0 = (GATHER ? (const uint8_t *)staging_w : staging_r) +
                          ((uint64_t)b0 * p.n_lanes + l) * p.seg_bytes;

  // Address of vector v on the staging side and on the table side.
  auto stage_at = [&](uint32_t vv) {
    uint32_t j, o;
    split_index<POW2>(vv, w, p.piece_log2, j, o);
    return (uint64_t)stage0 + j * block_step + 16ull * (v0 + o);
  };
  auto table_at = [&](uint32_t vv) {
    uint32_t j, o;
    split_index<POW2>(vv, w, p.piece_log2, j, o);
    return s_addr[j] + 16ull * (v0 + o);
  };
  uint32_t v = tid;
  for (; v + (kUnroll - 1) * kThreads < total; v += kUnroll * kThreads) {
    v4u x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t vv = v + u * kThreads;
      x[u] = load16(GATHER ? table_at(vv) : stage_at(vv));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t vv = v + u * kThreads;
      store16(GATHER ? stage_at(vv) : table_at(vv), x[u]);
    }
  }
  for (; v < total; v += kThreads) store16(GATHER ? stage_at(v) : table_at(v), load16(GATHER ? table_at(v) : stage_at(v)));
}

}  // namespace

hipError_t launch_gather(const PlanView &p, void *staging, hipStream_t stream) {
  const dim3 grid(p.n_lanes * p.n_tiles * p.pieces);
  uint8_t *w = reinterpret_cast<uint8_t *>(staging);
  if (p.piece_log2 < 32)
    return launch(runs_copy_kernel<true, true>, grid, dim3(kThreads), 0, stream, p, w, (const uint8_t *)w);
  return launch(runs_copy_kernel<true, false>, grid, dim3(kThreads), 0, stream, p, w, (const uint8_t *)w);
}

hipError_t launch_scatter(const PlanView &p, const void *staging, hipStream_t stream) {
  const dim3 grid(p.n_lanes * p.n_tiles * p.pieces);
  const uint8_t *r = reinterpret_cast<const uint8_t *>(staging);
  if (p.piece_log2 < 32)
    return launch(runs_copy_kernel<false, true>, grid, dim3(kThreads), 0, stream, p, (uint8_t *)nullptr, r);
  return launch(runs_copy_kernel<false, false>, grid, dim3(kThreads), 0, stream, p, (uint8_t *)nullptr, r);
}

}  // namespace xfer
