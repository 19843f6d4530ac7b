// Two-shard argmax / top-2 merge over BF16 logit rows.
//
// Two launches on the caller's stream:
//   1. scan: every (row, shard) is cut into `splits` column slices and each
//      slice gets one workgroup, so even 16 rows keep hundreds of CUs busy
//      (the per-element key arithmetic would make a one-workgroup-per-row
//      kernel ALU-bound on 16 CUs).  Each workgroup reduces its slice to the
//      slice's first two elements and writes them to the workspace.
//   2. fold: one wavefront per row folds the slices of each shard into the
//      shard's record, then the two shard records exactly as the exchange of
//      (top1, top2, index) records is folded on the two-card drafter, and
//      writes the row's output.
// The kernel boundary orders the two steps, so no atomics or device-scope
// fences are needed.  (A single kernel whose last workgroup per row folds,
// found through a per-row atomic counter, measured 2-3x slower on MI355X:
// the counter updates of a row's workgroups serialise, and an agent-scope
// release in every workgroup writes back L2.)
//
// Keys: an element is the 32-bit key
//     ord(value) << 16 | (0xFFFF - column)
// where ord maps BF16 bit patterns to 16-bit integers in numeric order with
// -0 and +0 equal (0x8000 +- magnitude), and the column counts from the shard
// start when the shard holds at most 65,536 columns.  A larger key is earlier
// in the row order (larger value, then lower id), and 0 (below every finite
// value and -inf) marks "no element".  A wider shard (up to 32 slices of at
// most 65,536 columns: 2,097,152) counts key columns from the slice start,
// and the fold widens each slice's keys to 64 bits, ord << 32 | (0xFFFFFFFF -
// column within the shard), before comparing keys of different slices.
// The first two elements of any set follow from the pairwise merge
//     top1 = max(x1, y1), top2 = max(min(x1, y1), max(x2, y2)).
// The wavefront reductions use DPP lane moves.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace xfer {

// Partial records of xfer_argmax_merge_noalloc: a static device array in
// place of the caller's workspace, one copy per GPU at its own address.  In
// host code `scratch` names a host-side stand-in, never the device memory:
// the device address comes from hipGetSymbolAddress, looked up once per
// device with that device current, and only that address reaches a kernel.
static __device__ __align__(256) uint64_t scratch[kArgmaxScratchBytes / sizeof(uint64_t)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t argmax_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr uint32_t kTargetWorkgroups = 1024;
constexpr uint32_t kMinSliceCols = 1024;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t ord16(uint32_t v) {
  const uint32_t mag = v & 0x7FFFu;
  return (v & 0x8000u) ? 0x8000u - mag : 0x8000u + mag;
}

__device__ __forceinline__ void take(uint32_t &t1, uint32_t &t2, uint32_t k) {
  t2 = max(t2, min(t1, k));
  t1 = max(t1, k);
}

__device__ __forceinline__ void merge(uint32_t &t1, uint32_t &t2, uint32_t o1, uint32_t o2) {
  const uint32_t n2 = max(max(t2, o2), min(t1, o1));
  t1 = max(t1, o1);
  t2 = n2;
}

// The 8 elements of a 16-byte vector whose first column (within the slice) is `col`.
__device__ __forceinline__ void take8(uint32_t &t1, uint32_t &t2, v4u w, uint32_t col) {
  const uint32_t id = 0xFFFFu - col;
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    take(t1, t2, (ord16(x[h] & 0xFFFFu) << 16) | (id - 2 * h));
    take(t1, t2, (ord16(x[h] >> 16) << 16) | (id - 2 * h - 1));
  }
}

// One DPP step: lanes whose source is outside the pattern, or whose row is
// masked off, read 0 (the identity of merge).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_merge(uint32_t &t1, uint32_t &t2) {
  const uint32_t o1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t1, CTRL, ROW_MASK, 0xF, false);
  const uint32_t o2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t2, CTRL, ROW_MASK, 0xF, false);
  merge(t1, t2, o1, o2);
}

// Wavefront reduction; the full result ends in lane 63.
__device__ __forceinline__ void wave_reduce(uint32_t &t1, uint32_t &t2) {
  dpp_merge<0xB1, 0xF>(t1, t2);   // quad_perm [1,0,3,2]
  dpp_merge<0x4E, 0xF>(t1, t2);   // quad_perm [2,3,0,1]: every lane holds its quad
  dpp_merge<0x114, 0xF>(t1, t2);  // row_shr:4
  dpp_merge<0x118, 0xF>(t1, t2);  // row_shr:8: lane 15 of each row holds the row
  dpp_merge<0x142, 0xA>(t1, t2);  // row_bcast:15 into rows 1 and 3
  dpp_merge<0x143, 0xC>(t1, t2);  // row_bcast:31 into rows 2 and 3: lane 63 holds all
}

// The same reduction on 64-bit keys (each DPP move is two 32-bit moves).
__device__ __forceinline__ void merge64(uint64_t &t1, uint64_t &t2, uint64_t o1, uint64_t o2) {
  const uint64_t n2 = max(max(t2, o2), min(t1, o1));
  t1 = max(t1, o1);
  t2 = n2;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_merge64(uint64_t &t1, uint64_t &t2) {
  const uint64_t o1 = dpp64<CTRL, ROW_MASK>(t1);
  const uint64_t o2 = dpp64<CTRL, ROW_MASK>(t2);
  merge64(t1, t2, o1, o2);
}

__device__ __forceinline__ void wave_reduce64(uint64_t &t1, uint64_t &t2) {
  dpp_merge64<0xB1, 0xF>(t1, t2);
  dpp_merge64<0x4E, 0xF>(t1, t2);
  dpp_merge64<0x114, 0xF>(t1, t2);
  dpp_merge64<0x118, 0xF>(t1, t2);
  dpp_merge64<0x142, 0xA>(t1, t2);
  dpp_merge64<0x143, 0xC>(t1, t2);
}

struct Shards {
  const uint16_t *ptr[2];
  uint64_t ld[2];
  uint32_t ncols[2];
  uint32_t off[2];
  uint32_t slice[2];  // columns per slice, a multiple of 8
};

// Workgroup (row, shard s, slice k) -> partials[blockIdx.x] = (top1 << 32 | top2).
// WIDE: a shard is wider than one 65,536-column slice, and key columns count
// from the slice start; otherwise from the shard start (keys of different
// slices then compare directly).
template <bool WIDE>
__global__ __launch_bounds__(kThreads) void argmax_scan_kernel(Shards sh, uint32_t splits, uint64_t *partials) {
  const uint32_t per_row = 2 * splits;
  const uint32_t row = blockIdx.x / per_row;
  const uint32_t rem = blockIdx.x % per_row;
  const uint32_t s = rem / splits;
  const uint32_t k = rem % splits;
  const uint32_t tid = threadIdx.x;

  const uint32_t ncols = sh.ncols[s];
  const uint32_t c0 = min(k * sh.slice[s], ncols);
  const uint32_t c1 = min(c0 + sh.slice[s], ncols);
  const uint16_t *rowp = sh.ptr[s] + (uint64_t)row * sh.ld[s];

  uint32_t t1 = 0, t2 = 0;
  // 16-byte vectors of 8 elements; c0 is a multiple of 8 and rows are 16-byte
  // aligned, so every vector is aligned.
  const uint32_t n_vec = (c1 - c0) / 8;
  const v4u *vp = reinterpret_cast<const v4u *>(rowp + c0);
  uint32_t v = tid;
  // Key columns count from `base` (c1 - base <= 65,536 either way).
  const uint32_t base = WIDE ? c0 : 0;
  for (; v + kThreads < n_vec; v += 2 * kThreads) {
    const v4u w0 = __builtin_nontemporal_load(&vp[v]);
    const v4u w1 = __builtin_nontemporal_load(&vp[v + kThreads]);
    take8(t1, t2, w0, c0 - base + 8 * v);
    take8(t1, t2, w1, c0 - base + 8 * (v + kThreads));
  }
  for (; v < n_vec; v += kThreads) take8(t1, t2, __builtin_nontemporal_load(&vp[v]), c0 - base + 8 * v);
  // Columns past the last whole vector (only in a shard's last slice).
  const uint32_t c_tail = c0 + 8 * n_vec;
  if (tid < c1 - c_tail) {
    const uint32_t c = c_tail + tid;
    take(t1, t2, (ord16(rowp[c]) << 16) | (0xFFFFu - (c - base)));
  }

  wave_reduce(t1, t2);
  __shared__ uint32_t lds1[kWaves], lds2[kWaves];
  const uint32_t wave = tid / 64, lane = tid % 64;
  if (lane == 63) {
    lds1[wave] = t1;
    lds2[wave] = t2;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t a1 = lds1[0], a2 = lds2[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) merge(a1, a2, lds1[w], lds2[w]);
    partials[blockIdx.x] = ((uint64_t)a1 << 32) | a2;
  }
}

// One wavefront per row: lane i holds partial i of the row; lanes
// [0, splits) are shard 0's slices, [splits, 2 * splits) shard 1's.  Each
// shard's top two end as 64-bit keys ord << 32 | (0xFFFFFFFF - column within
// the shard).
template <int MODE, bool WIDE>
__global__ __launch_bounds__(64) void argmax_fold_kernel(Shards sh, uint32_t splits, const uint64_t *partials,
                                                         void *out) {
  const uint32_t row = blockIdx.x, lane = threadIdx.x;
  const uint32_t per_row = 2 * splits;
  const uint64_t p = lane < per_row ? partials[(uint64_t)row * per_row + lane] : 0;
  const bool in0 = lane < splits;
  // A 32-bit key with its column counted from `c0` -> the 64-bit key.
  auto widen = [](uint32_t k, uint32_t c0) -> uint64_t {
    if (k == 0) return 0;
    const uint32_t col = c0 + (0xFFFFu - (k & 0xFFFFu));
    return ((uint64_t)(k >> 16) << 32) | (0xFFFFFFFFu - col);
  };
  uint64_t a1, a2, b1, b2;
  if (WIDE) {
    // keys of different slices compare only once widened with the slice start
    const uint32_t c0 = (in0 ? lane : lane - splits) * sh.slice[in0 ? 0 : 1];
    const uint64_t w1 = lane < per_row ? widen((uint32_t)(p >> 32), c0) : 0;
    const uint64_t w2 = lane < per_row ? widen((uint32_t)p, c0) : 0;
    a1 = in0 ? w1 : 0;
    a2 = in0 ? w2 : 0;
    b1 = in0 ? 0 : w1;
    b2 = in0 ? 0 : w2;
    wave_reduce64(a1, a2);
    wave_reduce64(b1, b2);
  } else {
    // shard-relative 32-bit keys compare directly; widen the shard's result
    uint32_t x1 = in0 ? (uint32_t)(p >> 32) : 0, x2 = in0 ? (uint32_t)p : 0;
    uint32_t y1 = in0 ? 0 : (uint32_t)(p >> 32), y2 = in0 ? 0 : (uint32_t)p;
    wave_reduce(x1, x2);
    wave_reduce(y1, y2);
    a1 = widen(x1, 0);
    a2 = widen(x2, 0);
    b1 = widen(y1, 0);
    b2 = widen(y2, 0);
  }
  if (lane != 63) return;

  // Shard records -> global order (ord desc, global id asc).
  struct Rec {
    uint32_t ord;
    uint32_t gid;
    uint32_t shard;
    uint32_t col;
    bool has;
  };
  auto rec = [&](uint64_t key, uint32_t shard) {
    Rec r;
    r.has = key != 0;
    r.ord = (uint32_t)(key >> 32);
    r.col = 0xFFFFFFFFu - (uint32_t)key;
    r.gid = sh.off[shard] + r.col;
    r.shard = shard;
    return r;
  };
  auto before = [](const Rec &x, const Rec &y) {
    if (!y.has) return x.has;
    if (!x.has) return false;
    if (x.ord != y.ord) return x.ord > y.ord;
    return x.gid < y.gid;
  };
  const Rec x1 = rec(a1, 0), x2 = rec(a2, 0), y1 = rec(b1, 1), y2 = rec(b2, 1);
  // Both shards hold at least one column, so both top1 records exist and the
  // chosen top2 (the loser's top1 if nothing beats it) always exists too.
  const bool x_wins = before(x1, y1);
  const Rec &top1 = x_wins ? x1 : y1;
  const Rec &lose1 = x_wins ? y1 : x1;
  const Rec &win2 = x_wins ? x2 : y2;
  const Rec &top2 = before(lose1, win2) ? lose1 : win2;
  // Exact bits of a chosen element: ord16 is one-to-one except that -0 and +0
  // share 0x8000, so only a zero is read back from the row for its sign.
  auto bits_of = [&](const Rec &r) -> uint32_t {
    if (r.ord > 0x8000u) return r.ord - 0x8000u;
    if (r.ord < 0x8000u) return 0x8000u | (0x8000u - r.ord);
    return sh.ptr[r.shard][(uint64_t)row * sh.ld[r.shard] + r.col];
  };
  const uint32_t v1 = bits_of(top1);
  if (MODE == XFER_ARGMAX) {
    xfer_max_idx r;
    r.max = __uint_as_float(v1 << 16);
    r.idx = (int32_t)top1.gid;
    reinterpret_cast<xfer_max_idx *>(out)[row] = r;
  } else {
    const uint32_t v2 = bits_of(top2);
    xfer_top2 r;
    r.top1 = __uint_as_float(v1 << 16);
    r.top2 = __uint_as_float(v2 << 16);
    r.idx = (int32_t)top1.gid;
    r.reserved = 0;
    reinterpret_cast<xfer_top2 *>(out)[row] = r;
  }
}

uint32_t round_up8(uint32_t x) { return (x + 7u) & ~7u; }

}  // namespace

uint32_t argmax_splits(uint32_t rows, uint32_t ncols0, uint32_t ncols1) {
  if (rows == 0) return 1;
  const uint32_t widest = ncols0 > ncols1 ? ncols0 : ncols1;
  uint64_t want = (kTargetWorkgroups + 2ull * rows - 1) / (2ull * rows);
  const uint64_t by_width = (widest + kMinSliceCols - 1) / kMinSliceCols;
  if (want > by_width) want = by_width;
  if (want > kArgmaxMaxSplits) want = kArgmaxMaxSplits;
  if (want < 1) want = 1;
  // no slice wider than kArgmaxMaxSliceCols (the 16-bit column of a key)
  const uint64_t need = ((uint64_t)widest + kArgmaxMaxSliceCols - 1) / kArgmaxMaxSliceCols;
  if (want < need) want = need;  // more than kArgmaxMaxSplits: the host refuses the call
  return (uint32_t)want;
}

// Layout: partials u64[rows][2][splits].
uint64_t argmax_workspace_bytes(uint32_t rows, uint32_t splits) { return (uint64_t)rows * 2 * splits * 8; }

hipError_t launch_argmax(ArgmaxShard s0, ArgmaxShard s1, uint32_t rows, int mode, void *out, void *workspace,
                         uint32_t splits, hipStream_t stream) {
  Shards sh;
  const ArgmaxShard in[2] = {s0, s1};
  for (int i = 0; i < 2; ++i) {
    sh.ptr[i] = in[i].ptr;
    sh.ld[i] = in[i].ld;
    sh.ncols[i] = in[i].ncols;
    sh.off[i] = in[i].col_offset;
    sh.slice[i] = round_up8((in[i].ncols + splits - 1) / splits);
  }
  uint64_t *partials = reinterpret_cast<uint64_t *>(workspace);
  const uint64_t *cp = partials;
  const dim3 scan_grid(rows * 2 * splits), fold_grid(rows);
  if (s0.ncols > kArgmaxMaxSliceCols || s1.ncols > kArgmaxMaxSliceCols) {
    hipError_t e = launch(argmax_scan_kernel<true>, scan_grid, dim3(kThreads), 0, stream, sh, splits, partials);
    if (e != hipSuccess) return e;
    if (mode == XFER_ARGMAX)
      return launch(argmax_fold_kernel<XFER_ARGMAX, true>, fold_grid, dim3(64), 0, stream, sh, splits, cp, out);
    return launch(argmax_fold_kernel<XFER_TOP2, true>, fold_grid, dim3(64), 0, stream, sh, splits, cp, out);
  }
  hipError_t e = launch(argmax_scan_kernel<false>, scan_grid, dim3(kThreads), 0, stream, sh, splits, partials);
  if (e != hipSuccess) return e;
  if (mode == XFER_ARGMAX)
    return launch(argmax_fold_kernel<XFER_ARGMAX, false>, fold_grid, dim3(64), 0, stream, sh, splits, cp, out);
  return launch(argmax_fold_kernel<XFER_TOP2, false>, fold_grid, dim3(64), 0, stream, sh, splits, cp, out);
}

}  // namespace xfer
