"""GPU parity of xfer_gather_runs / xfer_scatter_runs against the CPU oracle,
byte for byte: small layouts of every shape class (segment sizes that are and
are not powers of two, tile-straddling runs, three encodings of one address
set), and the full paged-K/V set of 1000 blocks x 288 slots x 2 segments of
4 KiB, bump-allocated (one run per lane) and with a shuffled allocation order
(greedy runs, and one run per segment)."""
import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, say, up, zeros

pytestmark = pytest.mark.gpu


def _otable(t: x.RunTable) -> oracle.RunTable:
    return oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks)


def _split_runs(t: x.RunTable, seed: int) -> x.RunTable:
    """The same address set with every run cut at a random point."""
    w = dg.random_u64(t.n_runs + 1, seed)
    rpl, base, stride, count = [], [], [], []
    r = 0
    for l in range(t.n_lanes):
        k = 0
        for _ in range(int(t.runs_per_lane[l])):
            c = int(t.run_count[r])
            cut = int(w[r] % c) if c > 1 else 0
            for lo, hi in ([(0, cut), (cut, c)] if cut else [(0, c)]):
                base.append((int(t.run_base[r]) + lo * int(t.run_stride[r])) % 2**64)
                stride.append(int(t.run_stride[r]) if hi - lo > 1 else 0)
                count.append(hi - lo)
                k += 1
            r += 1
        rpl.append(k)
    return x.RunTable(np.array(rpl, np.uint32), np.array(base, np.uint64), np.array(stride, np.int64),
                      np.array(count, np.uint32), t.n_blocks, t.seg_bytes)


def _world(n_blocks, n_slots, seg, shuffle_seed, n_regions=2):
    rb = dg.region_bytes_for(n_blocks, n_slots, seg, n_regions)
    regs = [zeros(rb) for _ in range(n_regions)]
    bases = [r.data_ptr() for r in regs]
    pos = dg.permutation(n_blocks, shuffle_seed) if shuffle_seed is not None else None
    addrs = dg.kv_src_addrs(n_blocks, n_slots, seg, bases, pos=pos)
    hosts = []
    for i, r in enumerate(regs):
        h = np.empty(rb, np.uint8)
        dg.fill_region(h, bases[i], addrs, seg, 1000 + i + (shuffle_seed or 0))
        r.copy_(torch.from_numpy(h))
        hosts.append(h)
    return regs, hosts, addrs


def _plan(t, regions, is_dst):
    buf = zeros(max(16, x.runs_plan_bytes(t)))
    return x.runs_prepare(t, regions, is_dst, buf), buf


SMALL = [
    # (n_blocks, n_slots, seg_bytes, shuffle seed)
    (1, 1, 16, None),
    (5, 3, 64, 1),
    (33, 2, 48, 2),        # 3 vectors per segment, 2 tiles
    (64, 4, 4096, 3),
    (65, 4, 4096, None),   # one block past two whole tiles
    (100, 6, 80, 4),       # 5 vectors per segment
    (31, 10, 1024, 5),
    (7, 2, 65536, 6),      # 64 KiB segments
    (5, 2, 49168, 3),      # 3073 vectors: a large segment that is not a power of two
    (3, 2, 1 << 20, None),  # the largest segment the plan accepts: 1 MiB, 128 pieces
]


@pytest.mark.parametrize("n_blocks,n_slots,seg,shuffle", SMALL)
def test_gather_scatter_small(n_blocks, n_slots, seg, shuffle):
    say("runs small", n_blocks, n_slots, seg, shuffle)
    regs, hosts, addrs = _world(n_blocks, n_slots, seg, shuffle, n_regions=2 if n_slots % 2 == 0 else 1)
    regions = [(r.data_ptr(), r.numel()) for r in regs]
    oregions = [(r.data_ptr(), h) for r, h in zip(regs, hosts)]
    n_lanes = 2 * n_slots
    greedy = x.runs_encode(addrs, seg)
    want = oracle.gather(_otable(greedy), seg, oregions)
    # a sentinel tail after the staging area must survive
    staging = filled(n_lanes * n_blocks * seg + 256, 0x3C)
    for t in (greedy, x.runs_encode(addrs, seg, max_count=1), _split_runs(greedy, n_blocks)):
        plan, _buf = _plan(t, regions, False)
        staging.fill_(0x3C)
        x.gather_runs(plan, staging)
        got = down(staging)
        assert np.array_equal(got[:want.size], want)
        assert np.all(got[want.size:] == 0x3C)
    # scatter into a slot-major destination with a gap segment per slot
    dst = filled(n_blocks * n_slots * 3 * seg, 0xA5)
    daddrs = dg.kv_dst_addrs(n_blocks, n_slots, seg, dst.data_ptr(), 3 * seg)
    dwant = np.full(dst.numel(), 0xA5, np.uint8)
    oracle.scatter(_otable(x.runs_encode(daddrs, seg)), seg, [(dst.data_ptr(), dwant)], want)
    staging_exact = up(want)
    for t in (x.runs_encode(daddrs, seg), x.runs_encode(daddrs, seg, max_count=1)):
        dst.fill_(0xA5)
        plan, _buf = _plan(t, [(dst.data_ptr(), dst.numel())], True)
        x.scatter_runs(staging_exact, plan)
        assert np.array_equal(down(dst), dwant)


def test_descending_and_interleaved_runs():
    """Lanes whose addresses run backwards (negative strides) and lanes that
    interleave with each other, gathered and scattered back to a mirror."""
    n_blocks, n_lanes, seg = 50, 4, 64
    region = zeros(n_blocks * n_lanes * seg * 2)
    base = region.data_ptr()
    a = np.empty((n_lanes, n_blocks), np.uint64)
    for l in range(n_lanes):
        for b in range(n_blocks):
            if l % 2 == 0:
                a[l, b] = base + ((n_blocks - 1 - b) * n_lanes + l) * seg            # descending
            else:
                a[l, b] = base + (n_blocks * n_lanes + b * n_lanes + l) * seg        # interleaved
    host = np.empty(region.numel(), np.uint8)
    dg.fill_region(host, base, a, seg, 77)
    region.copy_(torch.from_numpy(host))
    t = x.runs_encode(a, seg)
    assert np.any(t.run_stride < 0)
    plan, _b = _plan(t, [(base, region.numel())], False)
    staging = zeros(n_lanes * n_blocks * seg)
    x.gather_runs(plan, staging)
    want = oracle.gather(_otable(t), seg, [(base, host)])
    assert np.array_equal(down(staging), want)
    # the same address set is a valid destination (segments disjoint)
    mirror = zeros(region.numel())
    ma = a - np.uint64(base) + np.uint64(mirror.data_ptr())
    mt = x.runs_encode(ma, seg)
    mplan, _mb = _plan(mt, [(mirror.data_ptr(), mirror.numel())], True)
    x.scatter_runs(staging, mplan)
    mwant = np.zeros(mirror.numel(), np.uint8)
    oracle.scatter(_otable(mt), seg, [(mirror.data_ptr(), mwant)], want)
    assert np.array_equal(down(mirror), mwant)


@pytest.mark.parametrize("layout", ["dense", "shuffled"])
def test_full_size_kv_gather_scatter(layout):
    B, S, SEG = dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES
    L = 2 * S
    say("full-size", layout, "regions")
    shuffle = dg.seed_for(5, 0, 1) if layout == "shuffled" else None
    regs, hosts, addrs = _world(B, S, SEG, shuffle)
    regions = [(r.data_ptr(), r.numel()) for r in regs]
    oregions = [(r.data_ptr(), h) for r, h in zip(regs, hosts)]
    greedy = x.runs_encode(addrs, SEG)
    if layout == "dense":
        assert greedy.n_runs == L
        encodings = [greedy]
    else:
        assert greedy.n_runs > 250_000
        encodings = [greedy, x.runs_encode(addrs, SEG, max_count=1)]
    say("oracle gather", layout)
    want = oracle.gather(_otable(greedy), SEG, oregions)
    staging = zeros(L * B * SEG)
    for t in encodings:
        say("gpu gather", layout, "runs", t.n_runs)
        plan, _buf = _plan(t, regions, False)
        x.gather_runs(plan, staging)
        got = down(staging)
        assert np.array_equal(got, want)
        del got
        staging.zero_()
    del regs
    torch.cuda.empty_cache()
    staging = up(want)
    say("scatter", layout)
    dst = filled(B * S * dg.DST_SLOT_STRIDE, 0xA5)
    daddrs = dg.kv_dst_addrs(B, S, SEG, dst.data_ptr(), dg.DST_SLOT_STRIDE)
    dt = x.runs_encode(daddrs, SEG)
    assert dt.n_runs == L
    dwant = np.full(dst.numel(), 0xA5, np.uint8)
    oracle.scatter(_otable(dt), SEG, [(dst.data_ptr(), dwant)], want)
    plan, _buf = _plan(dt, [(dst.data_ptr(), dst.numel())], True)
    x.scatter_runs(staging, plan)
    assert np.array_equal(down(dst), dwant)
    del dst, staging
    torch.cuda.empty_cache()


def test_full_size_64k_segments():
    """200 blocks x 288 slots x 2 segments of 64 KiB (7200 MiB per set), dense,
    and its scatter into a slot-major destination with a gap segment per slot."""
    B, S, SEG = 200, dg.N_SLOTS, 65536
    L = 2 * S
    say("64 KiB segments regions")
    regs, hosts, addrs = _world(B, S, SEG, None)
    regions = [(r.data_ptr(), r.numel()) for r in regs]
    oregions = [(r.data_ptr(), h) for r, h in zip(regs, hosts)]
    t = x.runs_encode(addrs, SEG)
    assert t.n_runs == L
    say("64 KiB oracle gather")
    want = oracle.gather(_otable(t), SEG, oregions)
    staging = zeros(L * B * SEG)
    plan, _buf = _plan(t, regions, False)
    say("64 KiB gpu gather")
    x.gather_runs(plan, staging)
    got = down(staging)
    assert np.array_equal(got, want)
    del got, regs, hosts
    torch.cuda.empty_cache()
    dst = filled(B * S * 3 * SEG, 0xA5)
    daddrs = dg.kv_dst_addrs(B, S, SEG, dst.data_ptr(), 3 * SEG)
    dt = x.runs_encode(daddrs, SEG)
    dwant = np.full(dst.numel(), 0xA5, np.uint8)
    say("64 KiB oracle scatter")
    oracle.scatter(_otable(dt), SEG, [(dst.data_ptr(), dwant)], want)
    dplan, _dbuf = _plan(dt, [(dst.data_ptr(), dst.numel())], True)
    say("64 KiB gpu scatter")
    x.scatter_runs(staging, dplan)
    assert np.array_equal(down(dst), dwant)
    del dst, staging
    torch.cuda.empty_cache()


def test_plan_misuse_refused():
    regs, hosts, addrs = _world(4, 2, 64, None, n_regions=1)
    t = x.runs_encode(addrs, 64)
    region = [(regs[0].data_ptr(), regs[0].numel())]
    plan, _b = _plan(t, region, False)
    staging = filled(4 * 4 * 64, 0x11)
    assert x.scatter_runs_raw(staging.data_ptr(), staging.numel(), plan) == x.E_INVAL   # source plan
    assert x.gather_runs_raw(plan, staging.data_ptr(), staging.numel() - 16) == x.E_INVAL  # small staging
    assert x.gather_runs_raw(plan, regs[0].data_ptr(), regs[0].numel()) == x.E_INVAL       # staging = source
    assert np.all(down(staging) == 0x11)


def test_odd_lane_count_scattered_table():
    """Five lanes of scattered single-segment runs (the host pairs lanes l and
    l + 3 per workgroup; the last slot holds one lane), gathered and
    scattered back to a mirror."""
    n_lanes, n_blocks, seg = 5, 37, 272
    region = zeros(n_lanes * n_blocks * seg + 4096)
    base = region.data_ptr()
    order = dg.permutation(n_lanes * n_blocks, 41)
    a = (np.uint64(base) + order.astype(np.uint64).reshape(n_lanes, n_blocks) * np.uint64(seg))
    host = np.empty(region.numel(), np.uint8)
    dg.fill_region(host, base, a, seg, 43)
    region.copy_(torch.from_numpy(host))
    t = x.runs_encode(a, seg)
    assert t.n_runs > 2 * n_lanes
    plan, _b = _plan(t, [(base, region.numel())], False)
    assert plan.lanes_per_wg == 2
    staging = filled(n_lanes * n_blocks * seg + 64, 0x3C)
    x.gather_runs(plan, staging)
    want = oracle.gather(_otable(t), seg, [(base, host)])
    got = down(staging)
    assert np.array_equal(got[:want.size], want) and np.all(got[want.size:] == 0x3C)
    mirror = filled(region.numel(), 0x5A)
    ma = a - np.uint64(base) + np.uint64(mirror.data_ptr())
    mt = x.runs_encode(ma, seg)
    mplan, _mb = _plan(mt, [(mirror.data_ptr(), mirror.numel())], True)
    assert mplan.lanes_per_wg == 2
    x.scatter_runs(up(want), mplan)
    mwant = np.full(mirror.numel(), 0x5A, np.uint8)
    oracle.scatter(_otable(mt), seg, [(mirror.data_ptr(), mwant)], want)
    assert np.array_equal(down(mirror), mwant)


def test_staging_between_the_two_regions():
    """One allocation holds region 0, then the staging buffer, then region 1:
    the staging shares no byte with either region's segments, so the gather
    into it and the scatter out of it (into a second allocation laid out the
    same way) are accepted and match the oracle; a staging buffer that runs
    one segment into region 1 is refused."""
    n_blocks, n_slots, seg = 40, 6, 4096
    rb = dg.region_bytes_for(n_blocks, n_slots, seg, 2)
    sb = 2 * n_slots * n_blocks * seg                          # = 2 * rb
    arena = zeros(rb + sb + rb)
    bases = [arena.data_ptr(), arena.data_ptr() + rb + sb]
    addrs = dg.kv_src_addrs(n_blocks, n_slots, seg, bases, pos=dg.permutation(n_blocks, 77))
    hosts = []
    for i in range(2):
        h = np.empty(rb, np.uint8)
        dg.fill_region(h, bases[i], addrs, seg, 2000 + i)
        hosts.append(h)
    arena[:rb].copy_(torch.from_numpy(hosts[0]))
    arena[rb + sb:].copy_(torch.from_numpy(hosts[1]))
    t = x.runs_encode(addrs, seg)
    plan, _b = _plan(t, [(bases[0], rb), (bases[1], rb)], False)
    assert plan.n_spans == 2
    staging = arena[rb:rb + sb]
    say("staging between the regions", n_blocks, n_slots)
    assert x.gather_runs_raw(plan, staging.data_ptr() + seg, sb) == x.E_INVAL     # one segment into region 1
    x.gather_runs(plan, staging)
    want = oracle.gather(_otable(t), seg, [(bases[0], hosts[0]), (bases[1], hosts[1])])
    assert np.array_equal(down(staging), want)
    assert np.array_equal(down(arena[:rb]), hosts[0]) and np.array_equal(down(arena[rb + sb:]), hosts[1])
    # scatter from a staging buffer between the two destination regions
    arena2 = filled(rb + sb + rb, 0x5A)
    dbases = [arena2.data_ptr(), arena2.data_ptr() + rb + sb]
    daddrs = dg.kv_src_addrs(n_blocks, n_slots, seg, dbases)
    dt = x.runs_encode(daddrs, seg)
    dplan, _db = _plan(dt, [(dbases[0], rb), (dbases[1], rb)], True)
    stg2 = arena2[rb:rb + sb]
    stg2.copy_(up(want))
    x.scatter_runs(stg2, dplan)
    dwant = [np.full(rb, 0x5A, np.uint8) for _ in range(2)]
    oracle.scatter(_otable(dt), seg, [(dbases[0], dwant[0]), (dbases[1], dwant[1])], want)
    assert np.array_equal(down(arena2[:rb]), dwant[0]) and np.array_equal(down(arena2[rb + sb:]), dwant[1])
    assert np.array_equal(down(stg2), want)
