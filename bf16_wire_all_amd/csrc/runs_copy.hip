// Gather / scatter of fixed-size segments addressed by a run-encoded table.
//
// Work unit: one workgroup per (lane slot, tile of tile_blocks consecutive
// blocks), about 8 KiB in all.  A slot is one lane, or (lanes_per_wg = 2, for
// tables whose lanes are broken into many runs) lane l and lane
// l + ceil(L/2), 4 KiB each.  Large segments are cut into pieces, one
// workgroup each; piece p of a segment of 2 * pieces 4 KiB units copies
// units p and p + pieces, two streams half a segment apart (on 64 KiB
// segments: gather 6.38 against 6.21 TB/s and scatter 6.24 against 6.00 for
// one contiguous 8 KiB piece).  Consecutive workgroups take consecutive slots of the same
// block tile, so the chip reads and writes a few neighbouring address windows
// at a time.  Measured on MI355X on the paged K/V set: many short workgroups
// moving 8 KiB in one pass beat longer ones (32-block tiles: 5.2-5.4 TB/s);
// the host picks one lane or two per workgroup by measurement (see the plan
// layout).
//
// Decode, staged in LDS (no per-segment address table exists anywhere):
//   1. per lane, the plan's group index (one entry per lane and group of 32
//      blocks) gives the first run covering the workgroup's group and, via the
//      next entry, the last one: at most 33 runs, loaded in parallel into LDS;
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

// SPLIT2: the workgroup copies one piece of two 4 KiB units of a split
// segment (one lane, two vectors per thread); both loads are issued before
// either store.  On 64 KiB segments that measured 2,321 against 2,399 us for
// the scatter and 2,338 against 2,348 us for the gather; on 4 KiB segments
// (two lanes or two blocks per workgroup) issuing the loads first was 5-6 %
// slower than each load followed by its store, so those keep the loop below.
template <bool GATHER, bool POW2, bool SPLIT2>
__global__ __launch_bounds__(kThreads) void runs_copy_kernel(PlanView p, uint8_t *staging_w,
                                                             const uint8_t *staging_r) {
  constexpr int LW = kMaxLanesPerWorkgroup;
  constexpr int NR = kMaxGroupBlocks + 1;
  __shared__ uint32_t s_start[LW][NR];
  __shared__ uint64_t s_base[LW][NR];
  __shared__ int64_t s_stride[LW][NR];
  __shared__ uint64_t s_addr[LW][kMaxTileBlocks];

  // Workgroup -> (piece, lane slot, tile), pieces fastest: consecutive
  // workgroups stream consecutive pieces of one segment, then the next slot's.
  const uint32_t piece = blockIdx.x % p.pieces;
  const uint32_t rest = blockIdx.x / p.pieces;
  const uint32_t slot = rest % p.lane_slots;
  const uint32_t t = rest / p.lane_slots;
  const uint32_t b0 = t * p.tile_blocks;
  const uint32_t nb = min(p.tile_blocks, p.n_blocks - b0);
  const uint32_t tid = threadIdx.x;
  // Lanes of this workgroup: slot, and slot + lane_slots when it exists.
  // slot < lane_slots <= n_lanes, so the first always does.
  static_assert(LW == 2, "the decode below handles one or two lanes");
  const uint32_t lane0 = slot, lane1 = slot + p.lane_slots;
  const uint32_t n_here = (p.lanes_per_wg == 2 && lane1 < p.n_lanes) ? 2 : 1;

  // Runs covering the tile's group of blocks, per lane (the tile lies inside
  // one group): at most group_blocks + 1 each.
  const uint32_t g = b0 / p.group_blocks;
  const uint32_t *gr0 = p.group_run + (uint64_t)lane0 * (p.n_groups + 1);
  const uint32_t ra = gr0[g];
  const uint32_t na = min(gr0[g + 1] + 1, gr0[p.n_groups]) - ra;
  uint32_t rb = 0, nbr = 0;
  if (n_here == 2) {
    const uint32_t *gr1 = p.group_run + (uint64_t)lane1 * (p.n_groups + 1);
    rb = gr1[g];
    nbr = min(gr1[g + 1] + 1, gr1[p.n_groups]) - rb;
  }
  for (uint32_t k = tid; k < na + nbr; k += kThreads) {
    const bool second = k >= na;
    const uint32_t m = second ? k - na : k;
    const uint32_t r = (second ? rb : ra) + m;
    const int i = second ? 1 : 0;
    s_start[i][m] = p.run_start[r];
    s_base[i][m] = p.run_base[r];
    s_stride[i][m] = p.run_stride[r];
  }
  __syncthreads();
  for (uint32_t k = tid; k < n_here * nb; k += kThreads) {
    const uint32_t i = k / nb, j = k - i * nb;
    const uint32_t b = b0 + j;
    // last run m with s_start[i][m] <= b; s_start[i][0] <= group start <= b
    uint32_t lo = 0, hi = i ? nbr : na;
    while (hi - lo > 1) {
      const uint32_t mid = (lo + hi) / 2;
      if (s_start[i][mid] <= b)
        lo = mid;
      else
        hi = mid;
    }
    s_addr[i][j] = s_base[i][lo] + (uint64_t)(b - s_start[i][lo]) * (uint64_t)s_stride[i][lo];
  }
  __syncthreads();

  const uint32_t w = p.piece_vecs;
  const uint64_t v0 = (uint64_t)piece * w;  // first vector of this workgroup's piece
  const uint32_t total = nb * w;
  const uint64_t block_step = (uint64_t)p.n_lanes * p.seg_bytes;  // staging bytes between blocks
  if (SPLIT2) {
    // One lane, one block (nb = 1), w = 2 * kThreads vectors: units piece and
    // piece + pieces of the lane's segment.
    const uint8_t *stage0 = (GATHER ? (const uint8_t *)staging_w : staging_r) +
                            ((uint64_t)b0 * p.n_lanes + lane0) * p.seg_bytes;
    uint64_t from[2], to[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t o = tid + k * kThreads;
      const uint64_t sv = ((uint64_t)(o >> 8) * p.pieces + piece) * 256 + (o & 255);
      const uint64_t st_a = (uint64_t)stage0 + 16ull * sv;
      const uint64_t tb_a = s_addr[0][0] + 16ull * sv;
      from[k] = GATHER ? tb_a : st_a;
      to[k] = GATHER ? st_a : tb_a;
    }
    const v4u x0 = load16(from[0]), x1 = load16(from[1]);
    store16(to[0], x0);
    store16(to[1], x1);
    return;
  }
  for (uint32_t i = 0; i < n_here; ++i) {
    const uint32_t l = i ? lane1 : lane0;
    const uint8_t *stage0 = (GATHER ? (const uint8_t *)staging_w : staging_r) +
                            ((uint64_t)b0 * p.n_lanes + l) * p.seg_bytes;
    const uint64_t *addr = s_addr[i];
    // Address of vector v on the staging side and on the table side.
    // A piece of a split segment takes w / 256 whole 4 KiB units (256
    // vectors), pieces units apart: unit (o / 256) * pieces + piece.  The
    // host splits only segments above a one-lane workgroup's 8 KiB share, so
    // w = 512 (two units); the plan check requires w to be a multiple of 256.
    auto seg_vec = [&](uint32_t o) -> uint64_t {
      return p.pieces > 1 ? ((uint64_t)(o >> 8) * p.pieces + piece) * 256 + (o & 255) : v0 + o;
    };
    auto stage_at = [&](uint32_t vv) {
      uint32_t j, o;
      split_index<POW2>(vv, w, p.piece_log2, j, o);
      return (uint64_t)stage0 + j * block_step + 16ull * seg_vec(o);
    };
    auto table_at = [&](uint32_t vv) {
      uint32_t j, o;
      split_index<POW2>(vv, w, p.piece_log2, j, o);
      return addr[j] + 16ull * seg_vec(o);
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
    for (; v < total; v += kThreads)
      store16(GATHER ? stage_at(v) : table_at(v), load16(GATHER ? table_at(v) : stage_at(v)));
  }
}

}  // namespace

namespace {

template <bool GATHER>
hipError_t launch_runs(const PlanView &p, uint8_t *w, const uint8_t *r, hipStream_t stream) {
  const dim3 grid(p.lane_slots * p.n_tiles * p.pieces);
  if (p.pieces > 1 && p.lanes_per_wg == 1 && p.tile_blocks == 1 && p.piece_vecs == 2 * kThreads)
    return launch(runs_copy_kernel<GATHER, true, true>, grid, dim3(kThreads), 0, stream, p, w, r);
  if (p.piece_log2 < 32)
    return launch(runs_copy_kernel<GATHER, true, false>, grid, dim3(kThreads), 0, stream, p, w, r);
  return launch(runs_copy_kernel<GATHER, false, false>, grid, dim3(kThreads), 0, stream, p, w, r);
}

}  // namespace

hipError_t launch_gather(const PlanView &p, void *staging, hipStream_t stream) {
  uint8_t *w = reinterpret_cast<uint8_t *>(staging);
  return launch_runs<true>(p, w, (const uint8_t *)w, stream);
}

hipError_t launch_scatter(const PlanView &p, const void *staging, hipStream_t stream) {
  return launch_runs<false>(p, (uint8_t *)nullptr, reinterpret_cast<const uint8_t *>(staging), stream);
}

}  // namespace xfer
