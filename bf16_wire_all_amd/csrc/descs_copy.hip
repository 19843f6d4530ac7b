// Execution of a descriptor list: every descriptor is one contiguous copy of
// `bytes` from a device address into the slab.  A descriptor is cut into
// 4 KiB units, grouped into tiles of 2T units (T = min(576, ceil(units / 2)));
// workgroup piece c of a tile copies unit c and unit c + T, each thread one
// 16-byte vector of each, every load followed by its store (nontemporal both
// ways).  On MI355X the two-stream shape measured 6.4-6.7 TB/s for a plain
// 2.36 GB copy, fastest with the streams about 1.2 MB apart, against 5.9 TB/s
// for one contiguous 8 KiB piece per workgroup with both loads issued first;
// on the 72-read fetch, tiles of 2 x 576 units beat pairing the two halves of
// each 32 MiB read by 4 % (6.52 against 6.27 TB/s; 2 x 288 units: 6.47).  The grid is
// n_descs x max_pieces (max_pieces from the largest descriptor); workgroups
// past a shorter descriptor's end exit at once.
#include "internal.h"

namespace xfer {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kUnitBytes = kDescPieceBytes / 2;  // 4 KiB: one 16-byte vector per thread

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) v4u g_v4u;

__device__ __forceinline__ void copy_unit(const xfer_desc &desc, uint8_t *slab, uint64_t unit) {
  const uint64_t off = unit * kUnitBytes + 16u * threadIdx.x;
  if (off >= desc.bytes) return;  // bytes is a multiple of 16: the whole vector is inside
  const g_v4u *src = reinterpret_cast<const g_v4u *>(desc.src + off);
  g_v4u *dst = reinterpret_cast<g_v4u *>((uint64_t)(slab + desc.dst_off + off));
  __builtin_nontemporal_store(__builtin_nontemporal_load(src), dst);
}

__global__ __launch_bounds__(kThreads) void copy_descs_kernel(const xfer_desc *descs, uint32_t max_pieces,
                                                              uint8_t *slab) {
  const uint32_t d = blockIdx.x / max_pieces;
  const uint32_t piece = blockIdx.x - d * max_pieces;
  const xfer_desc desc = descs[d];
  const uint64_t n_units = (desc.bytes + kUnitBytes - 1) / kUnitBytes;
  const uint64_t T = pair_span(n_units);  // >= 1: bytes > 0 (host check)
  const uint64_t t = piece / T, c = piece - t * T;
  const uint64_t u0 = t * 2 * T + c;
  if (u0 >= n_units) return;
  copy_unit(desc, slab, u0);
  if (u0 + T < n_units) copy_unit(desc, slab, u0 + T);
}

static_assert(kUnitBytes == 16 * kThreads, "one vector per thread per unit");

}  // namespace

hipError_t launch_copy_descs(const xfer_desc *descs, uint64_t n_descs, uint32_t max_pieces, void *slab,
                             hipStream_t stream) {
  const dim3 grid((uint32_t)(n_descs * max_pieces));
  return launch(copy_descs_kernel, grid, dim3(kThreads), 0, stream, descs, max_pieces,
                reinterpret_cast<uint8_t *>(slab));
}

}  // namespace xfer
