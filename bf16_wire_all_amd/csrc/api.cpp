// Exported C entry points of libxfer: argument checks, run-table validation,
// encoding and plan layout, then the kernel launches.
//
// Every check runs on the host before anything is enqueued, in the order the
// header documents; the first failure is returned and nothing is launched.
#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"

namespace {

using xfer::PlanView;

constexpr uint32_t kPlanMagic = 0x584E5552u;  // "RUNX"
constexpr uint64_t kTileBytes = 8192;         // segment bytes per gather/scatter workgroup (target)
constexpr uint32_t kLanesPerWorkgroup = 2;    // lanes l and l + ceil(L/2) share a workgroup
constexpr uint32_t kDefaultGroupBlocks = 32;  // blocks per run-index entry

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// [a, a + na) and [b, b + nb) share a byte (empty ranges share nothing).
bool overlaps(uintptr_t a, uint64_t na, uintptr_t b, uint64_t nb) {
  if (na == 0 || nb == 0) return false;
  return a < b + nb && b < a + na;
}

bool mul_ok(uint64_t a, uint64_t b, uint64_t *out) { return !__builtin_mul_overflow(a, b, out); }

}  // namespace

// base + k * stride, every step checked for 64-bit overflow.
bool xfer::run_addr(uint64_t base, int64_t stride, uint64_t k, uint64_t *out) {
  if (k > (uint64_t)INT64_MAX) return false;
  int64_t prod;
  if (__builtin_mul_overflow((int64_t)k, stride, &prod)) return false;
  if (prod >= 0) {
    if (base > UINT64_MAX - (uint64_t)prod) return false;
    *out = base + (uint64_t)prod;
  } else {
    const uint64_t m = 0ull - (uint64_t)prod;
    if (base < m) return false;
    *out = base - m;
  }
  return true;
}

namespace {
using xfer::run_addr;

// Byte layout of a plan inside its device buffer.
struct Layout {
  uint32_t lanes_per_wg, lane_slots, tile_blocks, n_tiles, group_blocks, n_groups, pieces;
  uint64_t off_group_run, off_run_start, off_run_base, off_run_stride, total;
};

uint64_t up16(uint64_t x) { return (x + 15u) & ~15ull; }

Layout layout_for(const xfer_run_table *t) {
  Layout L{};
  // Work per workgroup: about kTileBytes.  When the lanes are broken into
  // many runs (blocks scattered, more than two runs per lane on average) and
  // segments fit the per-lane share, a workgroup takes two lanes, l and
  // l + ceil(L/2), one share each: measured on MI355X on the shuffled paged
  // K/V set, 6.3 TB/s against 6.1 TB/s for two blocks of one lane, whose
  // addresses are then unrelated.  Bump-allocated lanes (consecutive blocks a
  // fixed stride apart) and large segments keep one lane per workgroup
  // (dense set 6.50 against 6.45 paired; 64 KiB segments 6.25 against 5.98).
  // Per lane, small segments: a power-of-two number of blocks (it must divide
  // the group size), e.g. two blocks of 4 KiB.  Large segments whose vector
  // count is a power of two: one block, split into pieces of the per-lane
  // share, one workgroup each (8 pieces of a 64 KiB segment).
  const bool scattered = t->n_runs > 2ull * t->n_lanes;
  const bool pair = t->n_lanes >= 2 && scattered && t->seg_bytes <= kTileBytes / kLanesPerWorkgroup;
  L.lanes_per_wg = pair ? kLanesPerWorkgroup : 1;
  L.lane_slots = (uint32_t)(((uint64_t)t->n_lanes + L.lanes_per_wg - 1) / L.lanes_per_wg);
  const uint64_t lane_bytes = kTileBytes / L.lanes_per_wg;
  uint32_t tb = 1;
  while (tb * 2 <= xfer::kMaxTileBlocks && (uint64_t)tb * 2 * t->seg_bytes <= lane_bytes) tb *= 2;
  L.tile_blocks = tb;
  const uint64_t vps = t->seg_bytes / 16;
  L.pieces = 1;
  if (t->seg_bytes > lane_bytes && (vps & (vps - 1)) == 0) L.pieces = (uint32_t)(t->seg_bytes / lane_bytes);
  L.group_blocks = kDefaultGroupBlocks;
  // Rounded up in 64 bits: n_blocks may be as large as 2^32 - 1.
  L.n_tiles = (uint32_t)(((uint64_t)t->n_blocks + L.tile_blocks - 1) / L.tile_blocks);
  L.n_groups = (uint32_t)(((uint64_t)t->n_blocks + L.group_blocks - 1) / L.group_blocks);
  L.off_group_run = 0;
  L.off_run_start = up16((uint64_t)t->n_lanes * (L.n_groups + 1) * 4);
  L.off_run_base = L.off_run_start + up16(t->n_runs * 4);
  L.off_run_stride = L.off_run_base + up16(t->n_runs * 8);
  L.total = L.off_run_stride + up16(t->n_runs * 8);
  return L;
}

}  // namespace

// The checks of xfer_runs_validate; on success also reports the byte span
// covering every segment.
int xfer::validate_table(const xfer_run_table *t, const xfer_region *regions, int n_regions, int is_dst,
                         uint64_t *span_lo, uint64_t *span_hi, std::vector<Span> *region_spans) {
  if (!t) return XFER_E_INVAL;
  if (n_regions < 0 || (n_regions > 0 && !regions)) return XFER_E_INVAL;
  if (t->n_lanes > 0 && !t->runs_per_lane) return XFER_E_INVAL;
  if (t->n_runs > 0 && (!t->run_base || !t->run_stride || !t->run_count)) return XFER_E_INVAL;
  if (t->seg_bytes == 0 || t->seg_bytes % 16) return XFER_E_INVAL;
  for (int i = 0; i < n_regions; ++i)
    if (regions[i].base > UINT64_MAX - regions[i].bytes) return XFER_E_INVAL;

  if (t->n_runs > UINT32_MAX) return XFER_E_UNSUPPORTED;
  if (t->seg_bytes / 16 > xfer::kMaxSegVectors) return XFER_E_UNSUPPORTED;
  if ((uint64_t)t->n_lanes * t->n_blocks > UINT32_MAX) return XFER_E_UNSUPPORTED;

  uint64_t sum = 0;
  for (uint32_t l = 0; l < t->n_lanes; ++l) sum += t->runs_per_lane[l];
  if (sum != t->n_runs) return XFER_E_TABLE;
  uint64_t r = 0;
  for (uint32_t l = 0; l < t->n_lanes; ++l) {
    uint64_t covered = 0;
    for (uint32_t k = 0; k < t->runs_per_lane[l]; ++k, ++r) {
      if (t->run_count[r] == 0) return XFER_E_TABLE;
      covered += t->run_count[r];
    }
    if (covered != t->n_blocks) return XFER_E_TABLE;
  }

  uint64_t lo_all = UINT64_MAX, hi_all = 0;
  std::vector<Span> per_region;
  if (region_spans) per_region.assign((size_t)n_regions, Span{UINT64_MAX, 0});
  for (uint64_t i = 0; i < t->n_runs; ++i) {
    const uint64_t base = t->run_base[i];
    const uint32_t count = t->run_count[i];
    const int64_t stride = count > 1 ? t->run_stride[i] : 0;
    if (base % 16 || (count > 1 && stride % 16)) return XFER_E_RANGE;
    uint64_t last;
    if (!run_addr(base, stride, count - 1, &last)) return XFER_E_RANGE;
    const uint64_t lo = std::min(base, last);
    const uint64_t top = std::max(base, last);
    if (top > UINT64_MAX - t->seg_bytes) return XFER_E_RANGE;
    const uint64_t hi = top + t->seg_bytes;
    int g = 0;
    while (g < n_regions && !(lo >= regions[g].base && hi <= regions[g].base + regions[g].bytes)) ++g;
    if (g == n_regions) return XFER_E_RANGE;
    lo_all = std::min(lo_all, lo);
    hi_all = std::max(hi_all, hi);
    if (region_spans) {
      per_region[g].lo = std::min(per_region[g].lo, lo);
      per_region[g].hi = std::max(per_region[g].hi, hi);
    }
  }

  if (is_dst && t->n_runs) {
    // Segments, not run spans: interleaved lanes have overlapping spans but
    // disjoint segments.
    std::vector<uint64_t> a;
    a.reserve((size_t)t->n_lanes * t->n_blocks);
    for (uint64_t i = 0; i < t->n_runs; ++i) {
      const int64_t stride = t->run_count[i] > 1 ? t->run_stride[i] : 0;
      for (uint32_t k = 0; k < t->run_count[i]; ++k) {
        uint64_t x;
        run_addr(t->run_base[i], stride, k, &x);  // checked above via the span
        a.push_back(x);
      }
    }
    std::sort(a.begin(), a.end());
    for (size_t i = 1; i < a.size(); ++i)
      if (a[i] - a[i - 1] < t->seg_bytes) return XFER_E_OVERLAP;
  }
  if (span_lo) *span_lo = t->n_runs ? lo_all : 0;
  if (span_hi) *span_hi = t->n_runs ? hi_all : 0;
  if (region_spans) {
    region_spans->clear();
    for (const Span &sp : per_region)
      if (sp.hi > sp.lo) region_spans->push_back(sp);
  }
  return XFER_OK;
}

namespace {
using xfer::validate_table;

bool plan_ok(const xfer_runs_plan *p) {
  if (!p || p->magic != kPlanMagic || !p->dev) return false;
  if (p->tile_blocks == 0 || p->tile_blocks > xfer::kMaxTileBlocks) return false;
  if (p->group_blocks == 0 || p->group_blocks > xfer::kMaxGroupBlocks || p->group_blocks % p->tile_blocks)
    return false;
  if (p->pieces == 0 || (p->seg_bytes / 16) % p->pieces || (p->pieces > 1 && p->tile_blocks != 1)) return false;
  // a split segment's piece is whole 4 KiB units (the kernel pairs units)
  if (p->pieces > 1 && (p->seg_bytes / 16 / p->pieces) % 256) return false;
  if (p->lanes_per_wg == 0 || p->lanes_per_wg > xfer::kMaxLanesPerWorkgroup) return false;
  if (p->off_run_stride + up16(p->n_runs * 8) > p->dev_bytes) return false;
  return xfer::spans_ok(p->spans, p->n_spans, p->n_runs != 0);
}

PlanView view_of(const xfer_runs_plan *p) {
  const uint8_t *d = reinterpret_cast<const uint8_t *>(p->dev);
  PlanView v;
  v.group_run = reinterpret_cast<const uint32_t *>(d + p->off_group_run);
  v.run_start = reinterpret_cast<const uint32_t *>(d + p->off_run_start);
  v.run_base = reinterpret_cast<const uint64_t *>(d + p->off_run_base);
  v.run_stride = reinterpret_cast<const int64_t *>(d + p->off_run_stride);
  v.n_lanes = p->n_lanes;
  v.n_blocks = p->n_blocks;
  v.lanes_per_wg = p->lanes_per_wg;
  v.lane_slots = (uint32_t)(((uint64_t)p->n_lanes + p->lanes_per_wg - 1) / p->lanes_per_wg);
  v.n_tiles = p->n_tiles;
  v.tile_blocks = p->tile_blocks;
  v.group_blocks = p->group_blocks;
  v.n_groups = p->n_groups;
  v.seg_bytes = p->seg_bytes;
  v.vps = (uint32_t)(p->seg_bytes / 16);
  v.pieces = p->pieces;
  v.piece_vecs = v.vps / p->pieces;
  v.piece_log2 = 32;
  if ((v.piece_vecs & (v.piece_vecs - 1)) == 0) v.piece_log2 = (uint32_t)__builtin_ctz(v.piece_vecs);
  return v;
}

int staging_check(const xfer_runs_plan *p, uintptr_t staging, size_t staging_bytes) {
  uint64_t need;
  if (!mul_ok((uint64_t)p->n_lanes * p->n_blocks, p->seg_bytes, &need)) return XFER_E_INVAL;
  if (!staging || !aligned16((const void *)staging) || staging_bytes < need) return XFER_E_INVAL;
  if (xfer::overlaps_spans(staging, need, p->spans, p->n_spans)) return XFER_E_INVAL;
  return XFER_OK;
}

}  // namespace

std::vector<xfer::Span> xfer::fold_spans(std::vector<Span> v) {
  std::sort(v.begin(), v.end(), [](const xfer::Span &a, const xfer::Span &b) { return a.lo < b.lo; });
  std::vector<xfer::Span> out;
  for (const xfer::Span &sp : v) {
    if (!out.empty() && sp.lo <= out.back().hi)
      out.back().hi = std::max(out.back().hi, sp.hi);
    else
      out.push_back(sp);
  }
  while (out.size() > xfer::kPlanSpans) {
    size_t best = 0;
    for (size_t i = 1; i + 1 < out.size(); ++i)
      if (out[i + 1].lo - out[i].hi < out[best + 1].lo - out[best].hi) best = i;
    out[best].hi = out[best + 1].hi;
    out.erase(out.begin() + (std::ptrdiff_t)best + 1);
  }
  return out;
}

bool xfer::overlaps_spans(uintptr_t a, uint64_t na, const uint64_t *spans, uint32_t n) {
  for (uint32_t i = 0; i < n; ++i)
    if (overlaps(a, na, spans[2 * i], spans[2 * i + 1] - spans[2 * i])) return true;
  return false;
}

bool xfer::spans_ok(const uint64_t *spans, uint32_t n, bool has_work) {
  if (n > kPlanSpans || (has_work && n == 0)) return false;
  for (uint32_t i = 0; i < n; ++i)
    if (spans[2 * i + 1] <= spans[2 * i]) return false;
  return true;
}

extern "C" {

const char *xfer_status_str(int status) {
  switch (status) {
    case XFER_OK: return "ok";
    case XFER_E_INVAL: return "invalid argument";
    case XFER_E_UNSUPPORTED: return "unsupported request";
    case XFER_E_TABLE: return "inconsistent run table";
    case XFER_E_RANGE: return "segment outside the declared regions or address overflow";
    case XFER_E_OVERLAP: return "destination segments overlap";
    case XFER_E_DEVICE: return "HIP runtime error";
    case XFER_E_HOST_MEMORY: return "host memory for set-up scratch could not be allocated";
    default: return "unknown status";
  }
}

int xfer_pack_bf16(const float *src, size_t n, uint16_t *ring, size_t ring_bytes, size_t chunk_bytes,
                   size_t chunk_begin, size_t chunk_end, hipStream_t stream) {
  if (chunk_bytes == 0 || chunk_bytes % 16) return XFER_E_INVAL;
  if (ring_bytes == 0 || ring_bytes % chunk_bytes) return XFER_E_INVAL;
  if (chunk_begin > chunk_end) return XFER_E_INVAL;
  const uint64_t R = ring_bytes / chunk_bytes;
  if (chunk_end - chunk_begin > R) return XFER_E_INVAL;
  if (chunk_begin == chunk_end) return XFER_OK;
  // n == 0 with a named chunk falls through: that chunk starts at or past n.
  if (!src || !ring || !aligned16(src) || !aligned16(ring)) return XFER_E_INVAL;
  const uint64_t ce = chunk_bytes / 2;
  const uint64_t n_chunks = n / ce + (n % ce != 0);
  if (chunk_end > n_chunks) return XFER_E_INVAL;
  if (n > SIZE_MAX / 4) return XFER_E_INVAL;
  if (std::min<uint64_t>(chunk_end * ce, n) - chunk_begin * ce > xfer::kMaxStreamElems) return XFER_E_UNSUPPORTED;
  if (overlaps((uintptr_t)src, (uint64_t)n * 4, (uintptr_t)ring, ring_bytes)) return XFER_E_INVAL;
  const uint64_t e0 = chunk_begin * ce;
  const uint64_t e1 = std::min<uint64_t>(chunk_end * ce, n);
  const uint64_t slot0 = (chunk_begin % R) * ce;
  if (xfer::launch_pack(src + e0, e1 - e0, ring, R * ce, slot0, stream) != hipSuccess) return XFER_E_DEVICE;
  return XFER_OK;
}

int xfer_combine2(const uint16_t *a, const uint16_t *b, size_t n, void *out, int out_mode, hipStream_t stream) {
  if (out_mode != XFER_OUT_F32 && out_mode != XFER_OUT_BF16) return XFER_E_INVAL;
  if (n == 0) return XFER_OK;
  if (!a || !b || !out || !aligned16(a) || !aligned16(b) || !aligned16(out)) return XFER_E_INVAL;
  if (n > SIZE_MAX / 4) return XFER_E_INVAL;
  if (n > xfer::kMaxStreamElems) return XFER_E_UNSUPPORTED;
  const uint64_t out_bytes = (uint64_t)n * (out_mode == XFER_OUT_F32 ? 4 : 2);
  const uintptr_t o = (uintptr_t)out;
  const bool in_place = out_mode == XFER_OUT_BF16 && (out == (const void *)a || out == (const void *)b);
  if (!in_place) {
    if (overlaps(o, out_bytes, (uintptr_t)a, (uint64_t)n * 2)) return XFER_E_INVAL;
    if (overlaps(o, out_bytes, (uintptr_t)b, (uint64_t)n * 2)) return XFER_E_INVAL;
  } else {
    // the other input must not overlap the output at all
    const void *other = (out == (const void *)a) ? (const void *)b : (const void *)a;
    if (other != out && overlaps(o, out_bytes, (uintptr_t)other, (uint64_t)n * 2)) return XFER_E_INVAL;
  }
  if (xfer::launch_combine(a, b, n, out, out_mode, stream) != hipSuccess) return XFER_E_DEVICE;
  return XFER_OK;
}

int xfer_combine2_f32(const float *a, const float *b, size_t n, void *out, int out_mode, hipStream_t stream) {
  if (out_mode != XFER_OUT_F32 && out_mode != XFER_OUT_BF16) return XFER_E_INVAL;
  if (n == 0) return XFER_OK;
  if (!a || !b || !out || !aligned16(a) || !aligned16(b) || !aligned16(out)) return XFER_E_INVAL;
  if (n > SIZE_MAX / 4) return XFER_E_INVAL;
  if (n > xfer::kMaxStreamElems) return XFER_E_UNSUPPORTED;
  const uint64_t in_bytes = (uint64_t)n * 4;
  const uint64_t out_bytes = (uint64_t)n * (out_mode == XFER_OUT_F32 ? 4 : 2);
  const uintptr_t o = (uintptr_t)out;
  for (const void *in : {(const void *)a, (const void *)b}) {
    if (out_mode == XFER_OUT_F32 && in == (const void *)out) continue;  // in place: same element, same width
    if (overlaps(o, out_bytes, (uintptr_t)in, in_bytes)) return XFER_E_INVAL;
  }
  if (xfer::launch_combine_f32(a, b, n, out, out_mode, stream) != hipSuccess) return XFER_E_DEVICE;
  return XFER_OK;
}

size_t xfer_argmax_workspace_bytes(uint32_t rows, uint32_t ncols0, uint32_t ncols1) {
  return (size_t)xfer::argmax_workspace_bytes(rows, xfer::argmax_splits(rows, ncols0, ncols1));
}

namespace {

// The checks xfer_argmax_merge and xfer_argmax_merge_noalloc share: shards,
// mode and output.  On XFER_OK with rows > 0, fills the launch arguments,
// the workspace bytes the call needs and the shards' byte spans.
struct ArgmaxCall {
  uint32_t rows = 0, splits = 0;
  uint64_t need = 0;
  uint64_t lo[2] = {0, 0}, span[2] = {0, 0};
  xfer::ArgmaxShard a{}, b{};
};

int argmax_checks(const xfer_shard *s0, const xfer_shard *s1, int mode, const void *out, ArgmaxCall *c) {
  if (!s0 || !s1) return XFER_E_INVAL;
  if (mode != XFER_ARGMAX && mode != XFER_TOP2) return XFER_E_INVAL;
  if (s0->rows != s1->rows) return XFER_E_INVAL;
  const uint32_t rows = s0->rows;
  c->rows = rows;
  if (rows == 0) return XFER_OK;
  const xfer_shard *s[2] = {s0, s1};
  for (int i = 0; i < 2; ++i) {
    if (s[i]->ncols == 0) return XFER_E_INVAL;
    if ((uint64_t)s[i]->col_offset + s[i]->ncols > (1ull << 31)) return XFER_E_INVAL;
  }
  {
    const uint64_t a0 = s0->col_offset, a1 = a0 + s0->ncols, b0 = s1->col_offset, b1 = b0 + s1->ncols;
    if (a0 < b1 && b0 < a1) return XFER_E_INVAL;
  }
  for (int i = 0; i < 2; ++i) {
    if (s[i]->ncols > xfer::kArgmaxMaxShardCols) return XFER_E_UNSUPPORTED;
    if (!s[i]->ptr || !aligned16(s[i]->ptr) || (s[i]->ld * 2) % 16) return XFER_E_INVAL;
    if (rows > 1 && s[i]->ld < s[i]->ncols) return XFER_E_INVAL;
    uint64_t last_row;
    if (!mul_ok((uint64_t)(rows - 1), s[i]->ld, &last_row)) return XFER_E_INVAL;
    c->lo[i] = (uintptr_t)s[i]->ptr;
    c->span[i] = (last_row + s[i]->ncols) * 2;
  }
  c->splits = xfer::argmax_splits(rows, s0->ncols, s1->ncols);
  if ((uint64_t)rows * 2 * c->splits > xfer::kMaxGridBlocks) return XFER_E_UNSUPPORTED;
  c->need = xfer::argmax_workspace_bytes(rows, c->splits);
  if (!out || !aligned16(out)) return XFER_E_INVAL;
  const uint64_t out_bytes = (uint64_t)rows * (mode == XFER_ARGMAX ? sizeof(xfer_max_idx) : sizeof(xfer_top2));
  for (int i = 0; i < 2; ++i)
    if (overlaps((uintptr_t)out, out_bytes, c->lo[i], c->span[i])) return XFER_E_INVAL;
  c->a = xfer::ArgmaxShard{s0->ptr, s0->ld, s0->ncols, s0->col_offset};
  c->b = xfer::ArgmaxShard{s1->ptr, s1->ld, s1->ncols, s1->col_offset};
  return XFER_OK;
}

}  // namespace

int xfer_argmax_merge(const xfer_shard *s0, const xfer_shard *s1, int mode, void *out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  ArgmaxCall c;
  const int st = argmax_checks(s0, s1, mode, out, &c);
  if (st != XFER_OK || c.rows == 0) return st;
  if (!workspace || !aligned16(workspace) || workspace_bytes < c.need) return XFER_E_INVAL;
  const uint64_t out_bytes = (uint64_t)c.rows * (mode == XFER_ARGMAX ? sizeof(xfer_max_idx) : sizeof(xfer_top2));
  for (int i = 0; i < 2; ++i)
    if (overlaps((uintptr_t)workspace, c.need, c.lo[i], c.span[i])) return XFER_E_INVAL;
  if (overlaps((uintptr_t)out, out_bytes, (uintptr_t)workspace, c.need)) return XFER_E_INVAL;
  if (xfer::launch_argmax(c.a, c.b, c.rows, mode, out, workspace, c.splits, stream) != hipSuccess)
    return XFER_E_DEVICE;
  return XFER_OK;
}

int xfer_argmax_merge_noalloc(const xfer_shard *s0, const xfer_shard *s1, int mode, void *out,
                              hipStream_t stream) {
  ArgmaxCall c;
  const int st = argmax_checks(s0, s1, mode, out, &c);
  if (st != XFER_OK || c.rows == 0) return st;
  if (c.need > xfer::kArgmaxScratchBytes) return XFER_E_UNSUPPORTED;
  void *scratch = nullptr;
  if (xfer::argmax_scratch(&scratch) != hipSuccess) return XFER_E_DEVICE;
  if (xfer::launch_argmax(c.a, c.b, c.rows, mode, out, scratch, c.splits, stream) != hipSuccess)
    return XFER_E_DEVICE;
  return XFER_OK;
}

int xfer_runs_encode(const uint64_t *addrs, uint32_t n_lanes, uint32_t n_blocks, uint32_t max_count,
                     uint32_t *runs_per_lane, uint64_t *run_base, int64_t *run_stride, uint32_t *run_count,
                     uint64_t cap_runs, uint64_t *n_runs_out) {
  if (!n_runs_out || (n_lanes && !runs_per_lane)) return XFER_E_INVAL;
  if (n_lanes && n_blocks && (!addrs || !run_base || !run_stride || !run_count)) return XFER_E_INVAL;
  const uint32_t limit = max_count ? max_count : UINT32_MAX;
  uint64_t out = 0;
  for (uint32_t l = 0; l < n_lanes; ++l) {
    const uint64_t *a = addrs + (uint64_t)l * n_blocks;
    uint32_t lane_runs = 0;
    uint32_t i = 0;
    while (i < n_blocks) {
      // open a run at block i, then grow it as far as the greedy rule allows
      const uint64_t base = a[i];
      int64_t stride = 0;
      uint32_t count = 1;
      while (i + count < n_blocks && count < limit) {
        const uint64_t prev = a[i + count - 1], next = a[i + count];
        // next - prev as a signed 64-bit delta, if it fits
        const uint64_t up = next - prev, down = prev - next;
        bool fits;
        int64_t d;
        if (next >= prev) {
          fits = up <= (uint64_t)INT64_MAX;
          d = (int64_t)up;
        } else {
          fits = down <= (uint64_t)INT64_MAX + 1;
          d = (int64_t)(0 - down);
        }
        if (!fits) break;
        if (count == 1) {
          if (d == 0) break;
          stride = d;
        } else if (d != stride) {
          break;
        }
        ++count;
      }
      if (out >= cap_runs) return XFER_E_RANGE;
      run_base[out] = base;
      run_stride[out] = count > 1 ? stride : 0;
      run_count[out] = count;
      ++out;
      ++lane_runs;
      i += count;
    }
    runs_per_lane[l] = lane_runs;
  }
  *n_runs_out = out;
  return XFER_OK;
}

int xfer_runs_validate(const xfer_run_table *t, const xfer_region *regions, int n_regions, int is_dst) {
  return xfer::guarded([&]() -> int {
    return validate_table(t, regions, n_regions, is_dst, nullptr, nullptr, nullptr);
  });
}

size_t xfer_runs_plan_bytes(const xfer_run_table *t) {
  if (!t) return 0;
  return (size_t)layout_for(t).total;
}

int xfer_runs_prepare(const xfer_run_table *t, const xfer_region *regions, int n_regions, int is_dst, void *dev,
                      size_t dev_bytes, xfer_runs_plan *out) {
  return xfer::guarded([&]() -> int {
    uint64_t span_lo = 0, span_hi = 0;
    std::vector<xfer::Span> region_spans;
    const int st = validate_table(t, regions, n_regions, is_dst, &span_lo, &span_hi, &region_spans);
    if (st != XFER_OK) return st;
    if (!out) return XFER_E_INVAL;
    const Layout L = layout_for(t);
    if ((uint64_t)L.lane_slots * L.n_tiles * L.pieces > xfer::kMaxGridBlocks) return XFER_E_UNSUPPORTED;
    if (L.total && (!dev || !aligned16(dev) || dev_bytes < L.total)) return XFER_E_INVAL;

    // Host image of the plan: per (lane, group of blocks) the run covering the
    // group's first block, then each lane's end; per run its first block
    // within its lane.
    std::vector<uint8_t> img(L.total, 0);
    uint32_t *group_run = reinterpret_cast<uint32_t *>(img.data() + L.off_group_run);
    uint32_t *run_start = reinterpret_cast<uint32_t *>(img.data() + L.off_run_start);
    uint64_t r = 0;
    for (uint32_t l = 0; l < t->n_lanes; ++l) {
      uint32_t *gr = group_run + (uint64_t)l * (L.n_groups + 1);
      uint32_t start = 0, group = 0;
      for (uint32_t k = 0; k < t->runs_per_lane[l]; ++k, ++r) {
        run_start[r] = start;
        const uint32_t end = start + t->run_count[r];
        // every group whose first block lies in [start, end) starts in run r
        while (group < L.n_groups && (uint64_t)group * L.group_blocks < end) gr[group++] = (uint32_t)r;
        start = end;
      }
      gr[L.n_groups] = (uint32_t)r;
    }
    if (t->n_runs) {
      std::memcpy(img.data() + L.off_run_base, t->run_base, t->n_runs * 8);
      int64_t *strides = reinterpret_cast<int64_t *>(img.data() + L.off_run_stride);
      for (uint64_t i = 0; i < t->n_runs; ++i) strides[i] = t->run_count[i] > 1 ? t->run_stride[i] : 0;
    }
    if (L.total && hipMemcpy(dev, img.data(), L.total, hipMemcpyHostToDevice) != hipSuccess) return XFER_E_DEVICE;

    xfer_runs_plan p;
    std::memset(&p, 0, sizeof(p));
    p.dev = dev;
    p.dev_bytes = dev_bytes;
    p.n_lanes = t->n_lanes;
    p.n_blocks = t->n_blocks;
    p.seg_bytes = t->seg_bytes;
    p.n_runs = t->n_runs;
    p.span_lo = span_lo;
    p.span_hi = span_hi;
    const std::vector<xfer::Span> spans = xfer::fold_spans(region_spans);
    p.n_spans = (uint32_t)spans.size();
    for (size_t i = 0; i < spans.size(); ++i) {
      p.spans[2 * i] = spans[i].lo;
      p.spans[2 * i + 1] = spans[i].hi;
    }
    p.is_dst = is_dst ? 1u : 0u;
    p.tile_blocks = L.tile_blocks;
    p.n_tiles = L.n_tiles;
    p.group_blocks = L.group_blocks;
    p.n_groups = L.n_groups;
    p.pieces = L.pieces;
    p.lanes_per_wg = L.lanes_per_wg;
    p.magic = kPlanMagic;
    p.off_group_run = L.off_group_run;
    p.off_run_start = L.off_run_start;
    p.off_run_base = L.off_run_base;
    p.off_run_stride = L.off_run_stride;
    *out = p;
    return XFER_OK;
  });
}

int xfer_gather_runs(const xfer_runs_plan *plan, void *staging, size_t staging_bytes, hipStream_t stream) {
  if (!plan || plan->magic != kPlanMagic || plan->is_dst) return XFER_E_INVAL;
  if ((uint64_t)plan->n_lanes * plan->n_blocks == 0) return XFER_OK;
  if (!plan_ok(plan)) return XFER_E_INVAL;
  const int st = staging_check(plan, (uintptr_t)staging, staging_bytes);
  if (st != XFER_OK) return st;
  if (((uint64_t)plan->n_lanes + plan->lanes_per_wg - 1) / plan->lanes_per_wg * plan->n_tiles * plan->pieces >
      xfer::kMaxGridBlocks) return XFER_E_UNSUPPORTED;
  if (xfer::launch_gather(view_of(plan), staging, stream) != hipSuccess) return XFER_E_DEVICE;
  return XFER_OK;
}

int xfer_scatter_runs(const void *staging, size_t staging_bytes, const xfer_runs_plan *plan, hipStream_t stream) {
  if (!plan || plan->magic != kPlanMagic || !plan->is_dst) return XFER_E_INVAL;
  if ((uint64_t)plan->n_lanes * plan->n_blocks == 0) return XFER_OK;
  if (!plan_ok(plan)) return XFER_E_INVAL;
  const int st = staging_check(plan, (uintptr_t)staging, staging_bytes);
  if (st != XFER_OK) return st;
  if (((uint64_t)plan->n_lanes + plan->lanes_per_wg - 1) / plan->lanes_per_wg * plan->n_tiles * plan->pieces >
      xfer::kMaxGridBlocks) return XFER_E_UNSUPPORTED;
  if (xfer::launch_scatter(view_of(plan), staging, stream) != hipSuccess) return XFER_E_DEVICE;
  return XFER_OK;
}

}  // extern "C"
