// Paged copy by two Pages lists (indices, stride, offset): source page k to
// destination page k.  Pages are cut into 4 KiB units (the last unit of a
// page may be shorter).  The units form tiles of 2 * span units, span =
// min(576, ceil(units / 2)); workgroup c of a tile copies its unit c and unit
// c + span, one 16-byte vector per thread each, every nontemporal load
// followed by its store: the two-stream shape that measured fastest for plain
// copies on MI355X.  On the 288,000-page gathers of 4 KiB pages, span 576 ran
// at 6.30 TB/s against 6.11 for the two halves of the list (the scatter of
// 576,000 pages: 6.14 against 6.12).  Unit u is page u / units_per_page,
// bytes from 4096 * (u mod units_per_page); the two page indices are uniform
// loads.
#include "internal.h"

namespace xfer {
namespace {

constexpr int kThreads = 256;
static_assert(kPageUnitBytes == 16 * kThreads, "one vector per thread per unit");

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) v4u g_v4u;

__device__ __forceinline__ void copy_unit(const PagesView &v, uint32_t u) {
  const uint32_t k = u / v.units_per_page;
  const uint32_t j = u - k * v.units_per_page;
  const uint64_t off = (uint64_t)j * kPageUnitBytes + 16u * threadIdx.x;
  if (off >= v.page_len) return;  // page_len is a multiple of 16: the vector is inside
  const uint64_t s = v.src_base + (uint64_t)v.src_idx[k] * v.src_stride + off;
  const uint64_t d = v.dst_base + (uint64_t)v.dst_idx[k] * v.dst_stride + off;
  __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const g_v4u *>(s)),
                              reinterpret_cast<g_v4u *>(d));
}

__global__ __launch_bounds__(kThreads) void paged_copy_kernel(PagesView v) {
  const uint32_t t = blockIdx.x / v.span, c = blockIdx.x - t * v.span;
  const uint64_t u0 = (uint64_t)t * 2 * v.span + c;
  if (u0 >= v.n_units) return;
  copy_unit(v, (uint32_t)u0);
  if (u0 + v.span < v.n_units) copy_unit(v, (uint32_t)(u0 + v.span));
}

}  // namespace

hipError_t launch_paged_copy(const PagesView &v, hipStream_t stream) {
  const dim3 grid(v.pieces);
  return launch(paged_copy_kernel, grid, dim3(kThreads), 0, stream, v);
}

}  // namespace xfer
