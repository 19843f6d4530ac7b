// Coalesced fetch by dense group: the requester's planning of the run-encoded
// transfer page ("What this PR does", steps 2-5, and "READ splitting"), and
// the checks and upload of the resulting descriptor list.
#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"

namespace {

constexpr uint32_t kDescMagic = 0x43534544u;  // "DESC"

bool aligned16(uint64_t x) { return (x & 15u) == 0; }
uint64_t up16(uint64_t x) { return (x + 15u) & ~15ull; }
uint64_t mag(int64_t s) { return s < 0 ? 0ull - (uint64_t)s : (uint64_t)s; }

struct RunRec {
  uint64_t base;
  int64_t stride;  // 0 for one-block runs
  uint32_t start, count;
  uint32_t region;
  uint64_t index;  // position in the table
};

struct Group {
  size_t first, n;  // range in the sorted run order
  uint64_t base;    // lowest run base (the first run's)
  uint64_t chunk;   // bytes per block: n * seg_bytes
};

}  // namespace

extern "C" {

int xfer_groups_plan(const xfer_run_table *t, const xfer_region *regions, int n_regions, uint64_t max_desc_bytes,
                     xfer_desc *descs, uint64_t cap_descs, uint64_t *n_descs, uint64_t *slab_bytes,
                     uint64_t *local_base, int64_t *local_stride, uint64_t *n_groups, uint64_t *n_dense) {
  return xfer::guarded([&]() -> int {
    const int st = xfer::validate_table(t, regions, n_regions, 0, nullptr, nullptr, nullptr);
    if (st != XFER_OK) return st;
    if (!n_descs || !slab_bytes || max_desc_bytes == 0 || max_desc_bytes % 16) return XFER_E_INVAL;
    if (t->n_runs && (!local_base || !local_stride)) return XFER_E_INVAL;
    const uint64_t seg = t->seg_bytes;

    // Step 2: decode the runs (their block ranges and regions), bucket per
    // region and sort by base.
    std::vector<RunRec> runs(t->n_runs);
    uint64_t r = 0;
    for (uint32_t l = 0; l < t->n_lanes; ++l) {
      uint32_t start = 0;
      for (uint32_t k = 0; k < t->runs_per_lane[l]; ++k, ++r) {
        RunRec &x = runs[r];
        x.base = t->run_base[r];
        x.count = t->run_count[r];
        x.stride = x.count > 1 ? t->run_stride[r] : 0;
        x.start = start;
        x.index = r;
        uint64_t last;
        xfer::run_addr(x.base, x.stride, x.count - 1, &last);  // checked by the validation
        const uint64_t lo = std::min(x.base, last), hi = std::max(x.base, last) + seg;
        x.region = 0;
        for (int g = 0; g < n_regions; ++g)
          if (lo >= regions[g].base && hi <= regions[g].base + regions[g].bytes) {
            x.region = (uint32_t)g;
            break;
          }
        start += x.count;
      }
    }
    std::sort(runs.begin(), runs.end(), [](const RunRec &a, const RunRec &b) {
      if (a.region != b.region) return a.region < b.region;
      if (a.base != b.base) return a.base < b.base;
      return a.index < b.index;
    });

    // Step 3: grow groups whose per-block chunks tile densely.
    std::vector<Group> groups;
    for (size_t i = 0; i < runs.size(); ++i) {
      const RunRec &x = runs[i];
      if (!groups.empty()) {
        Group &g = groups.back();
        const RunRec &f = runs[g.first];
        const bool joins = x.region == f.region && x.start == f.start && x.count == f.count && x.stride == f.stride &&
                           x.base == g.base + g.chunk && (f.count == 1 || g.chunk + seg <= mag(f.stride));
        if (joins) {
          g.n += 1;
          g.chunk += seg;
          continue;
        }
      }
      groups.push_back(Group{i, 1, x.base, seg});
    }

    // Step 4: one range per dense group, per-block ranges otherwise, each split
    // at max_desc_bytes; step 5: local addresses by the same offsets.
    uint64_t k = 0, cursor = 0, dense = 0;
    bool room = true;
    auto emit = [&](uint64_t src, uint64_t dst, uint64_t bytes) {
      while (bytes) {
        const uint64_t n = bytes < max_desc_bytes ? bytes : max_desc_bytes;
        if (k < cap_descs && descs) {
          descs[k] = xfer_desc{src, dst, n};
        } else {
          room = false;
        }
        ++k;
        src += n;
        dst += n;
        bytes -= n;
      }
    };
    for (const Group &g : groups) {
      const RunRec &f = runs[g.first];
      const bool is_dense = f.count == 1 || mag(f.stride) == g.chunk;
      const uint64_t local0 = cursor;
      if (is_dense) {
        ++dense;
        const uint64_t span = f.count == 1 ? g.chunk : (uint64_t)f.count * mag(f.stride);
        const uint64_t lo = f.stride >= 0 ? g.base : g.base - (uint64_t)(f.count - 1) * mag(f.stride);
        emit(lo, local0, span);
        cursor += span;
        for (size_t i = g.first; i < g.first + g.n; ++i) {
          local_base[runs[i].index] = local0 + (runs[i].base - lo);
          local_stride[runs[i].index] = f.stride;
        }
      } else {
        for (uint32_t b = 0; b < f.count; ++b) {
          uint64_t src;
          xfer::run_addr(g.base, f.stride, b, &src);
          emit(src, local0 + (uint64_t)b * g.chunk, g.chunk);
        }
        cursor += (uint64_t)f.count * g.chunk;
        for (size_t i = g.first; i < g.first + g.n; ++i) {
          local_base[runs[i].index] = local0 + (runs[i].base - g.base);
          local_stride[runs[i].index] = (int64_t)g.chunk;
        }
      }
    }
    *n_descs = k;
    *slab_bytes = cursor;
    if (n_groups) *n_groups = groups.size();
    if (n_dense) *n_dense = dense;
    return room ? XFER_OK : XFER_E_RANGE;
  });
}

size_t xfer_descs_plan_bytes(uint64_t n_descs) { return (size_t)up16(n_descs * sizeof(xfer_desc)); }

int xfer_descs_prepare(const xfer_desc *descs, uint64_t n_descs, uint64_t slab_bytes, const xfer_region *regions,
                       int n_regions, void *dev, size_t dev_bytes, xfer_descs_plan *out) {
  return xfer::guarded([&]() -> int {
    if (!out || (n_descs && !descs) || n_regions < 0 || (n_regions > 0 && !regions)) return XFER_E_INVAL;
    for (int i = 0; i < n_regions; ++i)
      if (regions[i].base > UINT64_MAX - regions[i].bytes) return XFER_E_INVAL;
    uint64_t lo_all = UINT64_MAX, hi_all = 0;
    std::vector<std::pair<uint64_t, uint64_t>> dst(n_descs);
    std::vector<xfer::Span> per_region((size_t)n_regions, xfer::Span{UINT64_MAX, 0});
    for (uint64_t i = 0; i < n_descs; ++i) {
      const xfer_desc &d = descs[i];
      if (d.bytes == 0 || !aligned16(d.src) || !aligned16(d.dst_off) || !aligned16(d.bytes)) return XFER_E_INVAL;
      if (d.src > UINT64_MAX - d.bytes) return XFER_E_RANGE;
      int g = 0;
      while (g < n_regions && !(d.src >= regions[g].base && d.src + d.bytes <= regions[g].base + regions[g].bytes))
        ++g;
      if (g == n_regions) return XFER_E_RANGE;
      if (d.dst_off > slab_bytes || slab_bytes - d.dst_off < d.bytes) return XFER_E_RANGE;
      dst[i] = {d.dst_off, d.bytes};
      lo_all = std::min(lo_all, d.src);
      hi_all = std::max(hi_all, d.src + d.bytes);
      per_region[g].lo = std::min(per_region[g].lo, d.src);
      per_region[g].hi = std::max(per_region[g].hi, d.src + d.bytes);
    }
    std::sort(dst.begin(), dst.end());
    for (size_t i = 1; i < dst.size(); ++i)
      if (dst[i].first < dst[i - 1].first + dst[i - 1].second) return XFER_E_OVERLAP;
    uint64_t pieces = 0;  // workgroups per descriptor slot of the grid: the largest descriptor's
    for (uint64_t i = 0; i < n_descs; ++i)
      pieces = std::max(pieces, xfer::paired_pieces((descs[i].bytes + 4095) / 4096));
    if (pieces > UINT32_MAX || (n_descs && pieces > xfer::kMaxGridBlocks / n_descs)) return XFER_E_UNSUPPORTED;
    const uint64_t need = xfer_descs_plan_bytes(n_descs);
    if (need && (!dev || ((uintptr_t)dev & 15u) || dev_bytes < need)) return XFER_E_INVAL;
    if (n_descs && hipMemcpy(dev, descs, n_descs * sizeof(xfer_desc), hipMemcpyHostToDevice) != hipSuccess)
      return XFER_E_DEVICE;
    xfer_descs_plan p;
    std::memset(&p, 0, sizeof(p));
    p.dev = dev;
    p.dev_bytes = dev_bytes;
    p.n_descs = n_descs;
    p.slab_bytes = slab_bytes;
    p.src_lo = n_descs ? lo_all : 0;
    p.src_hi = n_descs ? hi_all : 0;
    std::vector<xfer::Span> used;
    for (const xfer::Span &sp : per_region)
      if (sp.hi > sp.lo) used.push_back(sp);
    const std::vector<xfer::Span> spans = xfer::fold_spans(used);
    p.n_spans = (uint32_t)spans.size();
    for (size_t i = 0; i < spans.size(); ++i) {
      p.spans[2 * i] = spans[i].lo;
      p.spans[2 * i + 1] = spans[i].hi;
    }
    p.max_pieces = (uint32_t)pieces;
    p.piece_bytes = xfer::kDescPieceBytes;
    p.magic = kDescMagic;
    *out = p;
    return XFER_OK;
  });
}

int xfer_copy_descs(const xfer_descs_plan *plan, void *slab, size_t slab_bytes, hipStream_t stream) {
  if (!plan || plan->magic != kDescMagic) return XFER_E_INVAL;
  if (plan->n_descs == 0) return XFER_OK;
  if (!plan->dev || plan->dev_bytes < plan->n_descs * sizeof(xfer_desc)) return XFER_E_INVAL;
  if (!slab || ((uintptr_t)slab & 15u) || slab_bytes < plan->slab_bytes) return XFER_E_INVAL;
  if (!xfer::spans_ok(plan->spans, plan->n_spans, true)) return XFER_E_INVAL;
  if (xfer::overlaps_spans((uintptr_t)slab, plan->slab_bytes, plan->spans, plan->n_spans)) return XFER_E_INVAL;
  if (xfer::launch_copy_descs(reinterpret_cast<const xfer_desc *>(plan->dev), plan->n_descs, plan->max_pieces, slab,
                              stream) != hipSuccess)
    return XFER_E_DEVICE;
  return XFER_OK;
}

}  // extern "C"
