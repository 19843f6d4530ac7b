// Execution of a descriptor list: every descriptor is one contiguous copy of
// `bytes` from a device address into the slab.  Work unit: one 256-thread
// workgroup per 8 KiB piece of a descriptor (2 nontemporal 16-byte vectors
// per thread), pieces of one descriptor on consecutive workgroups so the chip
// streams contiguous ranges.  The grid is n_descs x max_pieces; workgroups
// past a short descriptor's end exit at once.  The same short-lived
// workgroup shape measured fastest for the segment gather.
#include "internal.h"

namespace xfer {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kVecsPerPiece = kDescPieceBytes / 16;  // 512

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) v4u g_v4u;

__global__ __launch_bounds__(kThreads) void copy_descs_kernel(const xfer_desc *descs, uint32_t max_pieces,
                                                              uint8_t *slab) {
  const uint64_t d = blockIdx.x / max_pieces;
  const uint32_t piece = blockIdx.x % max_pieces;
  const xfer_desc desc = descs[d];
  const uint64_t off = (uint64_t)piece * kDescPieceBytes;
  if (off >= desc.bytes) return;
  const uint64_t left = desc.bytes - off;
  const uint32_t nvec = (uint32_t)((left < kDescPieceBytes ? left : kDescPieceBytes) / 16);
  const g_v4u *src = reinterpret_cast<const g_v4u *>(desc.src + off);
  g_v4u *dst = reinterpret_cast<g_v4u *>((uint64_t)(slab + desc.dst_off + off));
  const uint32_t v = threadIdx.x;
  if (v + kThreads < nvec) {
    const v4u a = __builtin_nontemporal_load(&src[v]);
    const v4u b = __builtin_nontemporal_load(&src[v + kThreads]);
    __builtin_nontemporal_store(a, &dst[v]);
    __builtin_nontemporal_store(b, &dst[v + kThreads]);
  } else {
    for (uint32_t i = v; i < nvec; i += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
  }
}

static_assert(kVecsPerPiece == 2 * kThreads, "two vectors per thread per piece");

}  // namespace

hipError_t launch_copy_descs(const xfer_desc *descs, uint64_t n_descs, uint32_t max_pieces, void *slab,
                             hipStream_t stream) {
  const dim3 grid((uint32_t)(n_descs * max_pieces));
  return launch(copy_descs_kernel, grid, dim3(kThreads), 0, stream, descs, max_pieces,
                reinterpret_cast<uint8_t *>(slab));
}

}  // namespace xfer
