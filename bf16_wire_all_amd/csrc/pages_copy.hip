// Paged copy by two Pages lists (indices, stride, offset): source page k to
// destination page k.  Pages are cut into 4 KiB units (the last unit of a
// page may be shorter); workgroup c copies unit c and unit c + gridDim.x,
// one 16-byte vector per thread each, every nontemporal load followed by its
// store: the two-stream shape that measured fastest for plain copies on
// MI355X.  Unit u is page u / units_per_page, bytes from 4096 * (u mod
// units_per_page); the two page indices are uniform loads.
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
  copy_unit(v, blockIdx.x);  // blockIdx.x < ceil(n_units / 2) <= n_units
  const uint32_t u1 = blockIdx.x + gridDim.x;
  if (u1 < v.n_units) copy_unit(v, u1);
}

}  // namespace

hipError_t launch_paged_copy(const PagesView &v, hipStream_t stream) {
  const dim3 grid((uint32_t)(((uint64_t)v.n_units + 1) / 2));
  return launch(paged_copy_kernel, grid, dim3(kThreads), 0, stream, v);
}

}  // namespace xfer
