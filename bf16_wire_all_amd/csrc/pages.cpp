// Host side of the paged copy: checks of two Pages lists ([TE] paged
// writes), their upload, and the launch.
#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"

namespace {

constexpr uint32_t kPagesMagic = 0x45474150u;  // "PAGE"

bool aligned16(uint64_t x) { return (x & 15u) == 0; }
uint64_t up16(uint64_t x) { return (x + 15u) & ~15ull; }

// Byte offset of page idx inside a region of region_bytes, or false if the
// page is not wholly inside it (checked arithmetic).
bool page_at(uint32_t idx, const xfer_pages &p, uint64_t page_len, uint64_t region_bytes, uint64_t *out) {
  if (p.stride && idx > (UINT64_MAX - p.offset) / p.stride) return false;
  const uint64_t at = p.offset + (uint64_t)idx * p.stride;
  if (at > region_bytes || region_bytes - at < page_len) return false;
  *out = at;
  return true;
}

}  // namespace

extern "C" {

size_t xfer_pages_plan_bytes(uint64_t n_pages) { return (size_t)(2 * up16(n_pages * sizeof(uint32_t))); }

int xfer_pages_prepare(uint64_t page_len, const xfer_region *src, const xfer_pages *sp, const xfer_region *dst,
                       const xfer_pages *dp, uint64_t n_pages, void *dev, size_t dev_bytes, xfer_pages_plan *out) {
  return xfer::guarded([&]() -> int {
    if (!out || !src || !dst || !sp || !dp) return XFER_E_INVAL;
    if (n_pages && (!sp->indices || !dp->indices)) return XFER_E_INVAL;
    if (page_len == 0 || !aligned16(page_len)) return XFER_E_INVAL;
    if (!aligned16(sp->stride) || !aligned16(sp->offset) || !aligned16(dp->stride) || !aligned16(dp->offset))
      return XFER_E_INVAL;
    if (!aligned16(src->base) || !aligned16(dst->base)) return XFER_E_INVAL;
    if (src->base > UINT64_MAX - src->bytes || dst->base > UINT64_MAX - dst->bytes) return XFER_E_INVAL;
    const bool regions_overlap = src->base < dst->base + dst->bytes && dst->base < src->base + src->bytes;
    const uint64_t upp = (page_len + xfer::kPageUnitBytes - 1) / xfer::kPageUnitBytes;
    if (upp > UINT32_MAX || (n_pages && n_pages > UINT32_MAX / upp)) return XFER_E_UNSUPPORTED;
    const uint64_t n_units = n_pages * upp;
    if (xfer::paired_pieces(n_units) > xfer::kMaxGridBlocks) return XFER_E_UNSUPPORTED;
    // Page starts as device addresses (each region lies below 2^64, checked above).
    std::vector<uint64_t> starts(n_pages), src_starts(regions_overlap ? n_pages : 0);
    for (uint64_t k = 0; k < n_pages; ++k) {
      uint64_t s, d;
      if (!page_at(sp->indices[k], *sp, page_len, src->bytes, &s) ||
          !page_at(dp->indices[k], *dp, page_len, dst->bytes, &d))
        return XFER_E_RANGE;
      starts[k] = dst->base + d;
      if (regions_overlap) src_starts[k] = src->base + s;
    }
    std::sort(starts.begin(), starts.end());
    for (uint64_t k = 1; k < n_pages; ++k)
      if (starts[k] - starts[k - 1] < page_len) return XFER_E_OVERLAP;
    // The regions may overlap (or be one region): then no destination page may
    // share a byte with a source page, or the result would depend on the order
    // of the copies.  Both lists sorted; each destination page against its
    // nearest source pages below and above.
    if (regions_overlap) {
      std::sort(src_starts.begin(), src_starts.end());
      for (uint64_t d : starts) {
        const auto it = std::lower_bound(src_starts.begin(), src_starts.end(), d);
        if (it != src_starts.end() && *it - d < page_len) return XFER_E_OVERLAP;
        if (it != src_starts.begin() && d - *(it - 1) < page_len) return XFER_E_OVERLAP;
      }
    }
    const uint64_t need = xfer_pages_plan_bytes(n_pages);
    if (n_pages && (!dev || !aligned16((uintptr_t)dev) || dev_bytes < need)) return XFER_E_INVAL;
    const uint64_t half = up16(n_pages * sizeof(uint32_t));
    if (n_pages) {
      if (hipMemcpy(dev, sp->indices, n_pages * sizeof(uint32_t), hipMemcpyHostToDevice) != hipSuccess ||
          hipMemcpy((uint8_t *)dev + half, dp->indices, n_pages * sizeof(uint32_t), hipMemcpyHostToDevice) !=
              hipSuccess)
        return XFER_E_DEVICE;
    }
    xfer_pages_plan p;
    std::memset(&p, 0, sizeof(p));
    p.dev = dev;
    p.dev_bytes = dev_bytes;
    p.n_pages = n_pages;
    p.page_len = page_len;
    p.src_base = src->base + sp->offset;
    p.src_stride = sp->stride;
    p.dst_base = dst->base + dp->offset;
    p.dst_stride = dp->stride;
    p.off_src_idx = 0;
    p.off_dst_idx = half;
    p.units_per_page = (uint32_t)upp;
    p.magic = kPagesMagic;
    *out = p;
    return XFER_OK;
  });
}

int xfer_paged_copy(const xfer_pages_plan *plan, hipStream_t stream) {
  if (!plan || plan->magic != kPagesMagic) return XFER_E_INVAL;
  if (plan->n_pages == 0) return XFER_OK;
  if (!plan->dev || plan->units_per_page == 0 || plan->dev_bytes < xfer_pages_plan_bytes(plan->n_pages))
    return XFER_E_INVAL;
  xfer::PagesView v;
  v.src_idx = reinterpret_cast<const uint32_t *>((const uint8_t *)plan->dev + plan->off_src_idx);
  v.dst_idx = reinterpret_cast<const uint32_t *>((const uint8_t *)plan->dev + plan->off_dst_idx);
  v.src_base = plan->src_base;
  v.src_stride = plan->src_stride;
  v.dst_base = plan->dst_base;
  v.dst_stride = plan->dst_stride;
  v.page_len = plan->page_len;
  v.units_per_page = plan->units_per_page;
  v.n_units = (uint32_t)(plan->n_pages * plan->units_per_page);
  v.span = (uint32_t)xfer::pair_span(v.n_units);
  v.pieces = (uint32_t)xfer::paired_pieces(v.n_units);
  if (xfer::launch_paged_copy(v, stream) != hipSuccess) return XFER_E_DEVICE;
  return XFER_OK;
}

}  // extern "C"
