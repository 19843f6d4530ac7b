// Drives every exported call of libxfer's host code, built with the host
// compiler against the mock HIP runtime, under AddressSanitizer and
// UndefinedBehaviorSanitizer: valid and corrupted run tables, page lists,
// descriptor lists and stream arguments from a seeded generator, plus
// injected runtime failures.  The statuses are checked where the header
// fixes them; everywhere else the point is that no call reads or writes out
// of bounds, overflows a signed integer or leaks an event.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <vector>

#include "mock_hip.h"
#include "xfer.h"

#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      std::fprintf(stderr, "CHECK failed: %s (line %d)\n", #c, __LINE__);  \
      std::exit(1);                                                         \
    }                                                                       \
  } while (0)

namespace {

struct Rng {  // SplitMix64
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  uint64_t below(uint64_t n) { return n ? next() % n : 0; }
};

// A host buffer standing in for device memory, 256-byte aligned.
struct Buf {
  uint8_t *p = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) {
    const size_t cap = std::max<size_t>(256, (bytes + 255) / 256 * 256);
    p = static_cast<uint8_t *>(std::aligned_alloc(256, cap));
    std::memset(p, 0x5A, cap);
  }
  ~Buf() { std::free(p); }
  Buf(const Buf &) = delete;
  Buf &operator=(const Buf &) = delete;
  uint64_t addr() const { return (uint64_t)(uintptr_t)p; }
};

hipStream_t token(uintptr_t k) { return reinterpret_cast<hipStream_t>(k); }

void statuses() {
  for (int s = -3; s < 12; ++s) CHECK(xfer_status_str(s) != nullptr);
}

void pack_combine(Rng &g) {
  for (int it = 0; it < 400; ++it) {
    const size_t n = g.below(3000);
    const size_t chunk = 16 * (1 + g.below(8));
    const size_t R = 1 + g.below(4);
    Buf src(n * 4 + 16), ring(R * chunk);
    const size_t ce = chunk / 2, n_chunks = n ? (n + ce - 1) / ce : 0;
    const size_t b = g.below(n_chunks + 2), e = b + g.below(R + 2);
    const int st = xfer_pack_bf16((const float *)src.p, n, (uint16_t *)ring.p, R * chunk, chunk, b, e, token(1));
    if (n && b < e && e - b <= R && e <= n_chunks) CHECK(st == XFER_OK);
    if (e - b > R) CHECK(st == XFER_E_INVAL);
    // aliasing source and ring
    CHECK(xfer_pack_bf16((const float *)ring.p, R * chunk / 4, (uint16_t *)ring.p, R * chunk, chunk, 0, 1,
                         token(1)) == XFER_E_INVAL);
    const int mode = (int)g.below(2);
    Buf a(n * 2 + 16), bb(n * 2 + 16), out(n * 4 + 16), fa(n * 4 + 16), fb(n * 4 + 16);
    CHECK(xfer_combine2((const uint16_t *)a.p, (const uint16_t *)bb.p, n, out.p, mode, token(2)) == XFER_OK);
    if (mode == XFER_OUT_BF16)  // in place over rank 0's operand
      CHECK(xfer_combine2((const uint16_t *)a.p, (const uint16_t *)bb.p, n, a.p, mode, token(2)) == XFER_OK);
    CHECK(xfer_combine2_f32((const float *)fa.p, (const float *)fb.p, n, out.p, mode, token(2)) == XFER_OK);
    if (n > 8)
      CHECK(xfer_combine2((const uint16_t *)a.p, (const uint16_t *)bb.p, n, a.p + 16, mode, token(2)) ==
            XFER_E_INVAL);
    CHECK(xfer_combine2((const uint16_t *)a.p, (const uint16_t *)bb.p, n, out.p, 7, token(2)) == XFER_E_INVAL);
  }
}

void argmax(Rng &g) {
  for (int it = 0; it < 200; ++it) {
    const uint32_t rows = 1 + (uint32_t)g.below(40);
    const uint32_t n0 = 1 + (uint32_t)g.below(3000), n1 = 1 + (uint32_t)g.below(3000);
    const uint32_t n0a = (n0 + 7) / 8 * 8;
    const size_t ld = (n0a + n1 + g.below(4) * 8 + 7) / 8 * 8;
    Buf m((size_t)rows * ld * 2);
    xfer_shard s0{(const uint16_t *)m.p, ld, rows, n0, 0};
    xfer_shard s1{(const uint16_t *)m.p + n0a, ld, rows, n1, n0};
    const size_t wsb = xfer_argmax_workspace_bytes(rows, n0, n1);
    Buf ws(wsb), out((size_t)rows * 16);
    const int mode = (int)g.below(2);
    CHECK(xfer_argmax_merge(&s0, &s1, mode, out.p, ws.p, wsb, token(3)) == XFER_OK);
    CHECK(xfer_argmax_merge(&s0, &s1, mode, out.p, ws.p, wsb ? wsb - 1 : 0, token(3)) == XFER_E_INVAL);
    xfer_shard clash = s1;
    clash.col_offset = n0 - 1;  // overlaps shard 0's ids
    CHECK(xfer_argmax_merge(&s0, &clash, mode, out.p, ws.p, wsb, token(3)) == XFER_E_INVAL);
    CHECK(xfer_argmax_merge(&s0, &s1, mode, m.p, ws.p, wsb, token(3)) == XFER_E_INVAL);  // out over the logits
    // the form with the library's static partials array: same checks, no workspace
    CHECK(xfer_argmax_merge_noalloc(&s0, &s1, mode, out.p, token(3)) == XFER_OK);
    CHECK(mock::g_last.a == rows);
    CHECK(xfer_argmax_merge_noalloc(&s0, &clash, mode, out.p, token(3)) == XFER_E_INVAL);
    CHECK(xfer_argmax_merge_noalloc(&s0, &s1, mode, m.p, token(3)) == XFER_E_INVAL);
    CHECK(xfer_argmax_merge_noalloc(&s0, &s1, mode, nullptr, token(3)) == XFER_E_INVAL);
    CHECK(xfer_argmax_merge_noalloc(&s0, &s1, 5, out.p, token(3)) == XFER_E_INVAL);
  }
  // partial records beyond the static array: refused before any launch
  {
    const uint32_t ld = 16;
    for (uint32_t rows : {4096u, 4097u}) {
      Buf m((size_t)rows * ld * 2), out((size_t)rows * 16);
      xfer_shard s0{(const uint16_t *)m.p, ld, rows, 8, 0};
      xfer_shard s1{(const uint16_t *)m.p + 8, ld, rows, 8, 8};
      const bool fits = xfer_argmax_workspace_bytes(rows, 8, 8) <= XFER_ARGMAX_SCRATCH_BYTES;
      const long before = mock::g_launches;
      CHECK(xfer_argmax_merge_noalloc(&s0, &s1, XFER_TOP2, out.p, token(3)) ==
            (fits ? XFER_OK : XFER_E_UNSUPPORTED));
      CHECK(mock::g_launches == before + (fits ? 1 : 0));
      CHECK(fits == (rows <= 4096));
    }
    Buf m(64), out(16);
    xfer_shard s0{(const uint16_t *)m.p, 16, 1, 8, 0};
    xfer_shard s1{(const uint16_t *)m.p + 8, 16, 1, 8, 8};
    mock::fail_scratch(true);
    CHECK(xfer_argmax_merge_noalloc(&s0, &s1, XFER_ARGMAX, out.p, token(3)) == XFER_E_DEVICE);
    mock::reset_failures();
    xfer_shard e0 = s0, e1 = s1;
    e0.rows = e1.rows = 0;
    CHECK(xfer_argmax_merge_noalloc(&e0, &e1, XFER_ARGMAX, nullptr, token(3)) == XFER_OK);  // empty work
  }
}

// Segment addresses [n_lanes][n_blocks] inside [base, base + slots * seg).
std::vector<uint64_t> layout(Rng &g, uint32_t L, uint32_t B, uint64_t seg, uint64_t base, uint64_t slots,
                             int kind) {
  std::vector<uint64_t> a((size_t)L * B);
  std::vector<uint64_t> perm(slots);
  std::iota(perm.begin(), perm.end(), 0);
  for (uint64_t i = slots; i > 1; --i) std::swap(perm[i - 1], perm[g.below(i)]);
  for (uint32_t l = 0; l < L; ++l)
    for (uint32_t b = 0; b < B; ++b) {
      uint64_t s;
      if (kind == 0) s = (uint64_t)b * L + l;             // block-major, dense
      else if (kind == 1) s = (uint64_t)l * B + b;        // lane-major (one run per lane)
      else if (kind == 2) s = perm[(uint64_t)l * B + b];  // shuffled, no repeats
      else s = g.below(slots);                            // repeats allowed (sources only)
      a[(size_t)l * B + b] = base + s * seg;
    }
  return a;
}

struct Table {
  std::vector<uint32_t> rpl, count;
  std::vector<uint64_t> base;
  std::vector<int64_t> stride;
  xfer_run_table t{};
  void bind(uint32_t L, uint32_t B, uint64_t seg) {
    t.n_lanes = L;
    t.n_blocks = B;
    t.seg_bytes = seg;
    t.n_runs = base.size();
    t.runs_per_lane = rpl.data();
    t.run_base = base.data();
    t.run_stride = stride.data();
    t.run_count = count.data();
  }
};

Table encode(const std::vector<uint64_t> &a, uint32_t L, uint32_t B, uint64_t seg, uint32_t max_count) {
  Table T;
  T.rpl.resize(L);
  const uint64_t cap = (uint64_t)L * B;
  T.base.resize(cap);
  T.stride.resize(cap);
  T.count.resize(cap);
  uint64_t n = 0;
  CHECK(xfer_runs_encode(a.data(), L, B, max_count, T.rpl.data(), T.base.data(), T.stride.data(), T.count.data(),
                         cap, &n) == XFER_OK);
  if (n) {
    uint64_t small = 0;  // too little room is refused
    CHECK(xfer_runs_encode(a.data(), L, B, max_count, T.rpl.data(), T.base.data(), T.stride.data(),
                           T.count.data(), n - 1, &small) == XFER_E_RANGE);
  }
  T.base.resize(n);
  T.stride.resize(n);
  T.count.resize(n);
  T.bind(L, B, seg);
  return T;
}

void runs_and_groups(Rng &g) {
  for (int it = 0; it < 300; ++it) {
    const uint32_t L = 1 + (uint32_t)g.below(24), B = 1 + (uint32_t)g.below(40);
    const uint64_t segs[] = {16, 48, 4096, 8192, 65536};
    const uint64_t seg = segs[g.below(it % 7 == 0 ? 5 : 4)];
    const uint64_t slots = (uint64_t)L * B + g.below(8);
    Buf src(slots * seg), stg((uint64_t)L * B * seg), dst(slots * seg);
    const int kind = (int)g.below(4);
    const uint32_t max_count = (uint32_t)g.below(6);
    const xfer_region sreg{src.addr(), src.n}, dreg{dst.addr(), dst.n};

    Table S = encode(layout(g, L, B, seg, src.addr(), slots, kind), L, B, seg, max_count);
    CHECK(xfer_runs_validate(&S.t, &sreg, 1, 0) == XFER_OK);
    const size_t pb = xfer_runs_plan_bytes(&S.t);
    Buf plan_dev(pb);
    xfer_runs_plan sp;
    CHECK(xfer_runs_prepare(&S.t, &sreg, 1, 0, plan_dev.p, pb, &sp) == XFER_OK);
    CHECK(xfer_gather_runs(&sp, stg.p, stg.n, token(4)) == XFER_OK);
    CHECK(xfer_gather_runs(&sp, stg.p, stg.n - 16, token(4)) == XFER_E_INVAL);
    CHECK(xfer_scatter_runs(stg.p, stg.n, &sp, token(4)) == XFER_E_INVAL);  // a source plan
    if (sp.pieces > 1) {  // an edited plan whose pieces are not whole 4 KiB units is refused
      xfer_runs_plan bad = sp;
      bad.pieces = sp.pieces * 4;
      CHECK(xfer_gather_runs(&bad, stg.p, stg.n, token(4)) == XFER_E_INVAL);
      bad.pieces = sp.pieces * 2;  // one unit per piece: still whole units
      CHECK(xfer_gather_runs(&bad, stg.p, stg.n, token(4)) == XFER_OK);
    }

    Table D = encode(layout(g, L, B, seg, dst.addr(), slots, kind == 3 ? 2 : kind), L, B, seg, max_count);
    Buf dplan_dev(xfer_runs_plan_bytes(&D.t));
    xfer_runs_plan dp;
    CHECK(xfer_runs_prepare(&D.t, &dreg, 1, 1, dplan_dev.p, dplan_dev.n, &dp) == XFER_OK);
    CHECK(xfer_scatter_runs(stg.p, stg.n, &dp, token(4)) == XFER_OK);
    if (kind == 3 && (uint64_t)L * B > 1) {  // repeated slots as a destination
      Table R = encode(layout(g, L, B, seg, dst.addr(), 1, 3), L, B, seg, max_count);
      CHECK(xfer_runs_validate(&R.t, &dreg, 1, 1) == XFER_E_OVERLAP);
    }

    // the coalesced fetch of the source table
    uint64_t nd = 0, slab = 0, ng = 0, ndense = 0;
    std::vector<uint64_t> lb(S.t.n_runs + 1);
    std::vector<int64_t> ls(S.t.n_runs + 1);
    const uint64_t max_desc = 16 * (1 + g.below(4096));
    const int st0 = xfer_groups_plan(&S.t, &sreg, 1, max_desc, nullptr, 0, &nd, &slab, lb.data(), ls.data(), &ng,
                                     &ndense);
    CHECK(st0 == XFER_E_RANGE || (st0 == XFER_OK && nd == 0));
    std::vector<xfer_desc> descs(nd + 1);
    CHECK(xfer_groups_plan(&S.t, &sreg, 1, max_desc, descs.data(), nd, &nd, &slab, lb.data(), ls.data(), &ng,
                           &ndense) == XFER_OK);
    CHECK(slab == (uint64_t)L * B * seg || kind == 3);
    Buf ddev(xfer_descs_plan_bytes(nd)), slab_buf(slab);
    xfer_descs_plan dplan;
    CHECK(xfer_descs_prepare(descs.data(), nd, slab, &sreg, 1, ddev.p, ddev.n, &dplan) == XFER_OK);
    CHECK(xfer_copy_descs(&dplan, slab_buf.p, slab, token(5)) == XFER_OK);
    if (nd > 1) {
      std::vector<xfer_desc> bad(descs.begin(), descs.begin() + nd);
      bad[1].dst_off = bad[0].dst_off;  // two descriptors onto one slab range
      CHECK(xfer_descs_prepare(bad.data(), nd, slab, &sreg, 1, ddev.p, ddev.n, &dplan) == XFER_E_OVERLAP);
    }

    // corrupted copies of the source table: any status, no undefined behaviour
    for (int m = 0; m < 6; ++m) {
      Table C = S;
      C.bind(L, B, seg);
      const uint64_t r = g.below(C.t.n_runs);
      switch (m) {
        case 0: C.count[r] = 0; break;
        case 1: C.count[r] += 1; break;
        case 2: C.base[r] += 8; break;
        case 3: C.stride[r] = (int64_t)((g.next() & ~15ull) | 16u); break;
        case 4: C.base[r] = ~0ull - 15; break;
        case 5: C.rpl[g.below(L)] += 1; break;
      }
      if (m == 5) {  // the claimed run count must match the arrays' length
        C.base.resize(C.t.n_runs + 1, src.addr());
        C.stride.resize(C.t.n_runs + 1, 0);
        C.count.resize(C.t.n_runs + 1, 1);
        C.bind(L, B, seg);
      }
      const int v = xfer_runs_validate(&C.t, &sreg, 1, (int)(m & 1));
      CHECK(v != XFER_OK || m == 3 || m == 2);
      Buf cdev(xfer_runs_plan_bytes(&C.t));
      xfer_runs_plan cp;
      CHECK(xfer_runs_prepare(&C.t, &sreg, 1, 0, cdev.p, cdev.n, &cp) == v || m == 2 || m == 3);
      uint64_t cnd = 0, cslab = 0;
      std::vector<uint64_t> clb(C.t.n_runs + 1);
      std::vector<int64_t> cls(C.t.n_runs + 1);
      (void)xfer_groups_plan(&C.t, &sreg, 1, max_desc, nullptr, 0, &cnd, &cslab, clb.data(), cls.data(), nullptr,
                             nullptr);
    }
  }
}

void pages(Rng &g) {
  for (int it = 0; it < 300; ++it) {
    const uint64_t page_len = 16 * (1 + g.below(it % 5 == 0 ? 1400 : 300));
    const uint64_t n = g.below(it % 7 == 0 ? 3000 : 200);  // some lists span several groups of 128 workgroups
    const uint64_t stride = page_len + 16 * g.below(4);
    const uint64_t slots = n + g.below(16) + 1;
    Buf src(slots * stride + 64), dst(slots * stride + 64);
    std::vector<uint32_t> si(n + 1), di(n + 1);
    std::vector<uint32_t> perm(slots);
    std::iota(perm.begin(), perm.end(), 0u);
    for (uint64_t i = slots; i > 1; --i) std::swap(perm[i - 1], perm[g.below(i)]);
    for (uint64_t k = 0; k < n; ++k) {
      si[k] = (uint32_t)g.below(slots);
      di[k] = perm[k];
    }
    const int trouble = (int)g.below(5);  // 0: none, 1: dst repeat, 2: page out of range, 3: huge stride
    if (trouble == 1 && n > 1) di[1] = di[0];
    if (trouble == 2 && n) si[n - 1] = (uint32_t)slots + 8;  // past the 64 bytes of slack for any stride
    if (trouble == 3 && n) si[0] = 1;  // index 1 at a 2^62 stride lies outside the region
    const uint64_t sstride = trouble == 3 ? (1ull << 62) : stride;
    const xfer_region sr{src.addr(), src.n}, dr{dst.addr(), dst.n};
    const xfer_pages sp{si.data(), sstride, 16 * g.below(2)}, dp{di.data(), stride, 0};
    Buf dev(xfer_pages_plan_bytes(n));
    xfer_pages_plan plan;
    const int st = xfer_pages_prepare(page_len, &sr, &sp, &dr, &dp, n, dev.p, dev.n, &plan);
    if (n == 0) CHECK(st == XFER_OK);
    if (trouble == 1 && n > 1) CHECK(st == XFER_E_OVERLAP);
    if ((trouble == 2 || trouble == 3) && n) CHECK(st == XFER_E_RANGE);
    if (st == XFER_OK) CHECK(xfer_paged_copy(&plan, token(6)) == XFER_OK);
    if (trouble == 0 && n) {
      mock::fail_memcpy_at((int)g.below(2));
      CHECK(xfer_pages_prepare(page_len, &sr, &sp, &dr, &dp, n, dev.p, dev.n, &plan) == XFER_E_DEVICE);
      mock::reset_failures();
    }
  }
}

// A paged copy inside one buffer: accepted while no destination page shares a
// byte with a source page, refused (XFER_E_OVERLAP) once one does.
void pages_in_one_region(Rng &g) {
  const uint64_t page = 256, slots = 64;
  Buf buf(slots * page);
  const xfer_region r{buf.addr(), buf.n};
  for (int it = 0; it < 100; ++it) {
    const uint64_t n = 1 + g.below(slots / 2);
    std::vector<uint32_t> perm(slots);
    std::iota(perm.begin(), perm.end(), 0u);
    for (uint64_t i = slots; i > 1; --i) std::swap(perm[i - 1], perm[g.below(i)]);
    std::vector<uint32_t> si(perm.begin(), perm.begin() + n), di(perm.begin() + n, perm.begin() + 2 * n);
    const bool clash = g.below(2) == 1;
    if (clash) di[g.below(n)] = si[g.below(n)];  // one destination page is also a source page
    const xfer_pages sp{si.data(), page, 0}, dp{di.data(), page, 0};
    Buf dev(xfer_pages_plan_bytes(n));
    xfer_pages_plan plan;
    const int st = xfer_pages_prepare(page, &r, &sp, &r, &dp, n, dev.p, dev.n, &plan);
    CHECK(st == (clash ? XFER_E_OVERLAP : XFER_OK));
    if (st == XFER_OK) CHECK(xfer_paged_copy(&plan, token(6)) == XFER_OK);
    // the same lists shifted by a few bytes of offset: pages straddle, still disjoint or not
    const xfer_pages dp16{di.data(), page, 16};
    if (!clash && di.size() && *std::max_element(di.begin(), di.end()) < slots - 1) {
      bool touch = false;
      for (uint32_t a : si)
        for (uint32_t b : di) touch = touch || a == b + 1;  // page b shifted by 16 bytes runs into page b + 1
      CHECK(xfer_pages_prepare(page, &r, &sp, &r, &dp16, n, dev.p, dev.n, &plan) ==
            (touch ? XFER_E_OVERLAP : XFER_OK));
    }
  }
}

void streamed(Rng &g) {
  for (uint32_t R = 1; R <= 4; ++R)
    for (uint32_t nc = 0; nc < 10; ++nc) {
      std::vector<xfer_op> ops(6 * nc + 1);
      size_t n_ops = 0;
      CHECK(xfer_allreduce2_schedule(nc, R, ops.data(), ops.size(), &n_ops) == XFER_OK);
      CHECK(n_ops == 6ull * nc);
      for (size_t i = 0; i < n_ops; ++i) {
        CHECK(ops[i].n_waits <= 2 && ops[i].record_event < 6 * R);
        for (uint32_t w = 0; w < ops[i].n_waits; ++w) CHECK(ops[i].wait_event[w] < 6 * R);
      }
    }
  // event creation with a failure at every position: nothing leaks, nothing
  // that was not created is destroyed (the slots start as garbage)
  for (int n = 1; n <= 6; ++n)
    for (int k = 0; k < n; ++k) {
      for (int which = 0; which < 2; ++which) {
        std::vector<hipEvent_t> ev(n, reinterpret_cast<hipEvent_t>((uintptr_t)0xBAD0 + 16 * k));
        if (which == 0) mock::fail_event_create_at(k);
        else mock::fail_event_record_at(k);
        CHECK(xfer_events_create(ev.data(), n) == XFER_E_DEVICE);
        mock::reset_failures();
        CHECK(mock::live_events() == 0);
      }
    }
  for (int it = 0; it < 60; ++it) {
    const uint64_t chunk = 16 * (1 + g.below(8));
    const uint32_t R = 1 + (uint32_t)g.below(3);
    const uint64_t n = g.below(2000);
    const int mode = (int)g.below(2);
    Buf s0(n * 4 + 16), s1(n * 4 + 16), snd0(R * chunk), snd1(R * chunk), rcv0(R * chunk), rcv1(R * chunk);
    Buf o0(n * 4 + 16), o1(n * 4 + 16);
    std::vector<hipEvent_t> ev(6 * R);
    CHECK(xfer_events_create(ev.data(), (int)ev.size()) == XFER_OK);
    xfer_allreduce2_desc d{};
    d.src[0] = (const float *)s0.p;
    d.src[1] = (const float *)s1.p;
    d.send[0] = (uint16_t *)snd0.p;
    d.send[1] = (uint16_t *)snd1.p;
    d.recv[0] = (uint16_t *)rcv0.p;
    d.recv[1] = (uint16_t *)rcv1.p;
    d.out[0] = o0.p;
    d.out[1] = o1.p;
    d.n = n;
    d.chunk_bytes = chunk;
    d.ring_bytes = R * chunk;
    d.out_mode = mode;
    d.compute[0] = token(11);
    d.compute[1] = token(12);
    d.wire[0] = token(13);
    d.wire[1] = token(14);
    d.events = ev.data();
    d.n_events = ev.size() - 1;
    CHECK(xfer_allreduce2_streamed(&d) == (n ? XFER_E_INVAL : XFER_OK));  // one event short
    d.n_events = ev.size();
    CHECK(xfer_allreduce2_streamed(&d) == XFER_OK);
    CHECK(xfer_allreduce2_streamed(&d) == XFER_OK);  // a second call on the same rings and events
    // The graph form: built without the descriptor's streams and events.
    {
      xfer_allreduce2_desc gd = d;
      gd.events = nullptr;
      gd.n_events = 0;
      gd.compute[0] = gd.compute[1] = gd.wire[0] = gd.wire[1] = nullptr;
      hipGraphExec_t ex = reinterpret_cast<hipGraphExec_t>((uintptr_t)1);
      mock::g_last_graph.clear();
      CHECK(xfer_allreduce2_graph_create(&gd, &ex) == XFER_OK);
      CHECK((ex == nullptr) == (n == 0));
      CHECK(mock::g_live_graphs == 0);  // only the executable graph is kept
      if (n) {
        const uint64_t ce = chunk / 2, n_chunks = (n + ce - 1) / ce;
        std::vector<xfer_op> ops(6 * n_chunks);
        size_t n_ops = 0;
        CHECK(xfer_allreduce2_schedule((uint32_t)n_chunks, R, ops.data(), ops.size(), &n_ops) == XFER_OK);
        size_t n_deps = 0;
        CHECK(xfer_allreduce2_graph_deps((uint32_t)n_chunks, R, nullptr, nullptr, 0, &n_deps) ==
              (n_ops > 1 ? XFER_E_RANGE : XFER_OK));
        std::vector<uint32_t> from(n_deps + 1), to(n_deps + 1);
        CHECK(xfer_allreduce2_graph_deps((uint32_t)n_chunks, R, from.data(), to.data(), from.size(), &n_deps) ==
              XFER_OK);
        // one node per operation, of its kind and size, with exactly the listed dependencies
        const std::vector<mock::GraphNodeLog> &gl = mock::g_last_graph;
        CHECK(gl.size() == n_ops);
        std::vector<std::vector<uint32_t>> want(n_ops);
        for (size_t k = 0; k < n_deps; ++k) {
          CHECK(from[k] < to[k]);  // a dependency always points back in issue order
          want[to[k]].push_back(from[k]);
        }
        for (size_t i = 0; i < n_ops; ++i) {
          CHECK(gl[i].kind == (int)ops[i].kind);
          const uint64_t e0 = (uint64_t)ops[i].chunk * ce, len = std::min<uint64_t>(ce, n - e0);
          CHECK(gl[i].n == (ops[i].kind == XFER_OP_WIRE ? 2 * len : len));
          std::vector<uint32_t> a = gl[i].deps, b = want[i];
          std::sort(a.begin(), a.end());
          std::sort(b.begin(), b.end());
          CHECK(a == b);
        }
        const long launches = mock::g_graph_launches;
        CHECK(xfer_allreduce2_graph_launch(ex, token(15)) == XFER_OK);
        CHECK(mock::g_graph_launches == launches + 1);
        CHECK(xfer_allreduce2_graph_destroy(ex) == XFER_OK);
        // a refused node or instantiation: nothing is kept
        mock::fail_graph_node_at((int)g.below(n_ops));
        CHECK(xfer_allreduce2_graph_create(&gd, &ex) == XFER_E_DEVICE);
        CHECK(ex == nullptr);
        mock::reset_failures();
        mock::fail_instantiate(true);
        CHECK(xfer_allreduce2_graph_create(&gd, &ex) == XFER_E_DEVICE);
        CHECK(ex == nullptr);
        mock::reset_failures();
        // a host allocation failing at each point of the build in turn:
        // XFER_E_HOST_MEMORY, and the graph made so far is released
        static bool host_failures_done = false;
        if (!host_failures_done) {
          host_failures_done = true;
          long k = 0;
          for (;; ++k) {
            mock::fail_new_after(k);
            hipGraphExec_t e2 = reinterpret_cast<hipGraphExec_t>((uintptr_t)1);
            const int st = xfer_allreduce2_graph_create(&gd, &e2);
            const bool thrown = !mock::new_failure_pending();
            mock::fail_new_after(-1);
            if (!thrown) {
              CHECK(st == XFER_OK && e2 != nullptr);
              CHECK(xfer_allreduce2_graph_destroy(e2) == XFER_OK);
              break;
            }
            CHECK(st == XFER_E_HOST_MEMORY && e2 == nullptr);
            CHECK(mock::g_live_graphs == 0 && mock::g_live_execs == 0);
          }
          CHECK(k >= 2);  // the node list, and the last-recorder table after the graph exists
          for (k = 0;; ++k) {  // the same for the dependency list
            mock::fail_new_after(k);
            size_t nd2 = 0;
            const int st = xfer_allreduce2_graph_deps((uint32_t)n_chunks, R, from.data(), to.data(), from.size(), &nd2);
            const bool thrown = !mock::new_failure_pending();
            mock::fail_new_after(-1);
            if (!thrown) {
              CHECK(st == XFER_OK && nd2 == n_deps);
              break;
            }
            CHECK(st == XFER_E_HOST_MEMORY);
          }
          CHECK(k >= 1);
        }
      }
      CHECK(mock::g_live_graphs == 0 && mock::g_live_execs == 0);
      CHECK(xfer_allreduce2_graph_create(&gd, nullptr) == XFER_E_INVAL);
    }
    d.recv[1] = d.send[0];  // rings that alias
    CHECK(xfer_allreduce2_streamed(&d) == (n ? XFER_E_INVAL : XFER_OK));
    CHECK(xfer_events_destroy(ev.data(), (int)ev.size()) == XFER_OK);
    CHECK(mock::live_events() == 0);
  }
  CHECK(xfer_allreduce2_graph_launch(nullptr, token(1)) == XFER_OK);
  CHECK(xfer_allreduce2_graph_destroy(nullptr) == XFER_OK);
}

// A launch the runtime refuses comes back as XFER_E_DEVICE from every hot call.
// Staging (and the coalesced fetch's slab) checked against per-region spans:
// a buffer between two regions is accepted; one inside a region's segment
// range, or inside a gap that was merged away to keep four spans, is refused.  Six one-segment
// regions at offsets 0, 7, 20, 27, 60 and 67 segments; staging is six
// segments long.  The two smallest gaps ([1, 7) and [21, 27)) are merged.
void staging_spans() {
  const uint64_t U = 4096;
  const uint64_t off[6] = {0, 7, 20, 27, 60, 67};
  Buf arena(70 * U);
  const uint64_t a0 = arena.addr();
  std::vector<uint32_t> rpl(6, 1), cnt(6, 1);
  std::vector<uint64_t> base(6);
  std::vector<int64_t> stride(6, 0);
  std::vector<xfer_region> regs(6);
  for (int i = 0; i < 6; ++i) {
    base[i] = a0 + off[i] * U;
    regs[i] = xfer_region{base[i], U};
  }
  xfer_run_table t{6, 1, U, 6, rpl.data(), base.data(), stride.data(), cnt.data()};
  Buf dev(xfer_runs_plan_bytes(&t));
  for (int is_dst = 0; is_dst < 2; ++is_dst) {
    xfer_runs_plan p;
    CHECK(xfer_runs_prepare(&t, regs.data(), 6, is_dst, dev.p, dev.n, &p) == XFER_OK);
    CHECK(p.n_spans == 4);
    CHECK(p.spans[0] == a0 && p.spans[1] == a0 + 8 * U);            // [0, 8): the first gap merged
    CHECK(p.spans[2] == a0 + 20 * U && p.spans[3] == a0 + 28 * U);  // [20, 28): the third gap merged
    CHECK(p.spans[4] == a0 + 60 * U && p.spans[5] == a0 + 61 * U);
    CHECK(p.spans[6] == a0 + 67 * U && p.spans[7] == a0 + 68 * U);
    const struct {
      uint64_t at;
      int want;
    } cases[] = {{1, XFER_E_INVAL}, {8, XFER_OK}, {14, XFER_OK}, {15, XFER_E_INVAL}, {21, XFER_E_INVAL},
                 {28, XFER_OK}, {54, XFER_OK}, {55, XFER_E_INVAL}, {61, XFER_OK}, {62, XFER_E_INVAL}};
    for (const auto &c : cases) {
      uint8_t *stg = arena.p + c.at * U;
      const int st = is_dst ? xfer_scatter_runs(stg, 6 * U, &p, token(9)) : xfer_gather_runs(&p, stg, 6 * U, token(9));
      CHECK(st == c.want);
    }
    // an edited plan with no spans for its segments, or a reversed span, is refused
    xfer_runs_plan bad = p;
    bad.n_spans = 0;
    CHECK(xfer_gather_runs(&bad, arena.p + 8 * U, 6 * U, token(9)) == XFER_E_INVAL);
    bad = p;
    bad.n_spans = 5;
    CHECK(xfer_gather_runs(&bad, arena.p + 8 * U, 6 * U, token(9)) == XFER_E_INVAL);
    bad = p;
    std::swap(bad.spans[0], bad.spans[1]);
    CHECK(xfer_gather_runs(&bad, arena.p + 8 * U, 6 * U, token(9)) == XFER_E_INVAL);
  }
  // the coalesced fetch's slab, checked the same way against per-region source spans
  {
    std::vector<xfer_desc> d(6);
    for (int i = 0; i < 6; ++i) d[i] = xfer_desc{base[i], (uint64_t)i * U, U};
    Buf ddev(xfer_descs_plan_bytes(6));
    xfer_descs_plan p;
    CHECK(xfer_descs_prepare(d.data(), 6, 6 * U, regs.data(), 6, ddev.p, ddev.n, &p) == XFER_OK);
    CHECK(p.n_spans == 4 && p.src_lo == a0 && p.src_hi == a0 + 68 * U);
    CHECK(p.spans[0] == a0 && p.spans[1] == a0 + 8 * U && p.spans[2] == a0 + 20 * U && p.spans[3] == a0 + 28 * U);
    const struct {
      uint64_t at;
      int want;
    } cases[] = {{1, XFER_E_INVAL}, {8, XFER_OK}, {15, XFER_E_INVAL}, {28, XFER_OK}, {61, XFER_OK},
                 {62, XFER_E_INVAL}};
    for (const auto &c : cases) CHECK(xfer_copy_descs(&p, arena.p + c.at * U, 6 * U, token(9)) == c.want);
    xfer_descs_plan bad = p;
    bad.n_spans = 0;
    CHECK(xfer_copy_descs(&bad, arena.p + 8 * U, 6 * U, token(9)) == XFER_E_INVAL);
    bad = p;
    bad.spans[3] = bad.spans[2];
    CHECK(xfer_copy_descs(&bad, arena.p + 8 * U, 6 * U, token(9)) == XFER_E_INVAL);
  }
  // random region sets: at most four sorted, disjoint spans that cover every
  // segment byte, inside [span_lo, span_hi), each starting and ending on a segment
  {
    Rng g{0x5BA45ull};
    for (int it = 0; it < 200; ++it) {
      const uint32_t nr = 1 + (uint32_t)g.below(9), L = 1 + (uint32_t)g.below(12);
      std::vector<uint64_t> roff(nr);
      uint64_t at = 0;
      for (uint32_t r = 0; r < nr; ++r) {
        roff[r] = at;
        at += 4 + g.below(6) + g.below(2) * g.below(40);  // region of 4 units, then a gap of 0..50
      }
      Buf ar((at + 4) * 64);
      std::vector<xfer_region> rr(nr);
      for (uint32_t r = 0; r < nr; ++r) rr[r] = xfer_region{ar.addr() + roff[r] * 64, 4 * 64};
      std::vector<uint32_t> rp(L, 1), ct(L, 1);
      std::vector<uint64_t> bs(L);
      std::vector<int64_t> sd(L, 0);
      std::vector<bool> used(4 * nr, false);
      for (uint32_t l = 0; l < L; ++l) {  // one 64-byte segment per lane, in a random free slot
        uint64_t k;
        do k = g.below(4 * nr); while (used[k]);
        if ((uint64_t)std::count(used.begin(), used.end(), true) + 1 >= 4 * nr) break;
        used[k] = true;
        bs[l] = rr[k / 4].base + (k % 4) * 64;
      }
      const uint32_t Lu = (uint32_t)std::count(used.begin(), used.end(), true);
      if (Lu == 0) continue;
      bs.resize(Lu);
      xfer_run_table rt{Lu, 1, 64, Lu, rp.data(), bs.data(), sd.data(), ct.data()};
      Buf rdev(xfer_runs_plan_bytes(&rt));
      xfer_runs_plan pl;
      CHECK(xfer_runs_prepare(&rt, rr.data(), (int)nr, 0, rdev.p, rdev.n, &pl) == XFER_OK);
      CHECK(pl.n_spans >= 1 && pl.n_spans <= 4);
      for (uint32_t i = 0; i < pl.n_spans; ++i) {
        CHECK(pl.spans[2 * i] < pl.spans[2 * i + 1]);
        if (i) CHECK(pl.spans[2 * i - 1] < pl.spans[2 * i]);  // sorted, disjoint, not touching
      }
      CHECK(pl.spans[0] == pl.span_lo && pl.spans[2 * pl.n_spans - 1] == pl.span_hi);
      for (uint32_t l = 0; l < Lu; ++l) {  // every segment inside one span
        bool in = false;
        for (uint32_t i = 0; i < pl.n_spans && !in; ++i) in = bs[l] >= pl.spans[2 * i] && bs[l] + 64 <= pl.spans[2 * i + 1];
        CHECK(in);
      }
      for (uint32_t i = 0; i < pl.n_spans; ++i) {  // every span starts and ends on a segment
        bool lo = false, hi = false;
        for (uint32_t l = 0; l < Lu; ++l) {
          lo = lo || bs[l] == pl.spans[2 * i];
          hi = hi || bs[l] + 64 == pl.spans[2 * i + 1];
        }
        CHECK(lo && hi);
      }
    }
  }
  // two regions: the whole range between them is free for staging
  xfer_run_table t2{2, 1, U, 2, rpl.data(), base.data(), stride.data(), cnt.data()};
  Buf dev2(xfer_runs_plan_bytes(&t2));
  xfer_runs_plan p2;
  CHECK(xfer_runs_prepare(&t2, regs.data(), 6, 0, dev2.p, dev2.n, &p2) == XFER_OK);
  CHECK(p2.n_spans == 2 && p2.span_lo == a0 && p2.span_hi == a0 + 8 * U);
  CHECK(xfer_gather_runs(&p2, arena.p + 1 * U, 2 * U, token(9)) == XFER_OK);
  CHECK(xfer_gather_runs(&p2, arena.p + 6 * U, 2 * U, token(9)) == XFER_E_INVAL);
}

void refused_launches() {
  const size_t n = 1000;
  Buf src(n * 4), ring(2 * 64), a(n * 2), b(n * 2), out(n * 4);
  Buf m(16 * 64 * 2), ws(1 << 16), rec(16 * 16);
  const uint32_t L = 4, B = 8;
  const uint64_t seg = 64;
  Buf reg(L * B * seg), stg(L * B * seg), dst(L * B * seg);
  std::vector<uint64_t> addrs((size_t)L * B);
  for (uint32_t l = 0; l < L; ++l)
    for (uint32_t k = 0; k < B; ++k) addrs[(size_t)l * B + k] = reg.addr() + ((uint64_t)k * L + l) * seg;
  Table T = encode(addrs, L, B, seg, 0);
  const xfer_region sreg{reg.addr(), reg.n};
  Buf pdev(xfer_runs_plan_bytes(&T.t));
  xfer_runs_plan sp;
  CHECK(xfer_runs_prepare(&T.t, &sreg, 1, 0, pdev.p, pdev.n, &sp) == XFER_OK);
  for (auto &x : addrs) x = x - reg.addr() + dst.addr();
  Table D = encode(addrs, L, B, seg, 0);
  const xfer_region dreg{dst.addr(), dst.n};
  Buf ddev(xfer_runs_plan_bytes(&D.t));
  xfer_runs_plan dp;
  CHECK(xfer_runs_prepare(&D.t, &dreg, 1, 1, ddev.p, ddev.n, &dp) == XFER_OK);
  xfer_desc desc{reg.addr(), 0, reg.n};
  Buf descdev(xfer_descs_plan_bytes(1));
  xfer_descs_plan fp;
  CHECK(xfer_descs_prepare(&desc, 1, stg.n, &sreg, 1, descdev.p, descdev.n, &fp) == XFER_OK);
  std::vector<uint32_t> idx(L * B);
  std::iota(idx.begin(), idx.end(), 0u);
  const xfer_pages pl{idx.data(), seg, 0};
  Buf pgdev(xfer_pages_plan_bytes(idx.size()));
  xfer_pages_plan pp;
  CHECK(xfer_pages_prepare(seg, &sreg, &pl, &dreg, &pl, idx.size(), pgdev.p, pgdev.n, &pp) == XFER_OK);
  xfer_shard s0{(const uint16_t *)m.p, 64, 16, 32, 0}, s1{(const uint16_t *)m.p + 32, 64, 16, 32, 32};
  std::vector<hipEvent_t> ev(12);
  CHECK(xfer_events_create(ev.data(), 12) == XFER_OK);
  xfer_allreduce2_desc d{};
  Buf snd0(128), snd1(128), rcv0(128), rcv1(128), o0(n * 4), o1(n * 4), f1(n * 4);
  d.src[0] = (const float *)src.p;
  d.src[1] = (const float *)f1.p;
  d.send[0] = (uint16_t *)snd0.p;
  d.send[1] = (uint16_t *)snd1.p;
  d.recv[0] = (uint16_t *)rcv0.p;
  d.recv[1] = (uint16_t *)rcv1.p;
  d.out[0] = o0.p;
  d.out[1] = o1.p;
  d.n = n;
  d.chunk_bytes = 64;
  d.ring_bytes = 128;
  d.out_mode = XFER_OUT_F32;
  d.compute[0] = token(21);
  d.compute[1] = token(22);
  d.wire[0] = token(23);
  d.wire[1] = token(24);
  d.events = ev.data();
  d.n_events = 12;
  mock::fail_launches(true);
  CHECK(xfer_pack_bf16((const float *)src.p, n, (uint16_t *)ring.p, 128, 64, 0, 2, token(1)) == XFER_E_DEVICE);
  CHECK(xfer_combine2((const uint16_t *)a.p, (const uint16_t *)b.p, n, out.p, XFER_OUT_F32, token(1)) == XFER_E_DEVICE);
  CHECK(xfer_combine2_f32((const float *)src.p, (const float *)f1.p, n, out.p, XFER_OUT_BF16, token(1)) ==
        XFER_E_DEVICE);
  CHECK(xfer_argmax_merge(&s0, &s1, XFER_TOP2, rec.p, ws.p, ws.n, token(1)) == XFER_E_DEVICE);
  CHECK(xfer_argmax_merge_noalloc(&s0, &s1, XFER_TOP2, rec.p, token(1)) == XFER_E_DEVICE);
  CHECK(xfer_gather_runs(&sp, stg.p, stg.n, token(1)) == XFER_E_DEVICE);
  CHECK(xfer_scatter_runs(stg.p, stg.n, &dp, token(1)) == XFER_E_DEVICE);
  CHECK(xfer_copy_descs(&fp, stg.p, stg.n, token(1)) == XFER_E_DEVICE);
  CHECK(xfer_paged_copy(&pp, token(1)) == XFER_E_DEVICE);
  CHECK(xfer_allreduce2_streamed(&d) == XFER_E_DEVICE);
  mock::reset_failures();
  CHECK(xfer_allreduce2_streamed(&d) == XFER_OK);
  CHECK(xfer_events_destroy(ev.data(), 12) == XFER_OK);
  CHECK(mock::live_events() == 0);
}

void host_memory() {
  xfer_desc d{};
  xfer_descs_plan plan;
  CHECK(xfer_descs_prepare(&d, 1ull << 60, 1 << 20, nullptr, 0, nullptr, 0, &plan) == XFER_E_HOST_MEMORY);
}

}  // namespace

int main() {
  Rng g{0x5EED5A5Eull};
  statuses();
  pack_combine(g);
  staging_spans();
  pages_in_one_region(g);
  argmax(g);
  runs_and_groups(g);
  pages(g);
  streamed(g);
  refused_launches();
  host_memory();
  std::printf("host code under sanitizers: %ld launches recorded, all checks passed\n", mock::g_launches);
  return 0;
}
