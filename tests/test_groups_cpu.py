"""The coalesced-fetch planner (dense groups, 32 MiB reads), on the CPU.

Pins from the run-encoded transfer page: the 4 KiB shape (1000 blocks x 288
slots x 2) fetches with 72 descriptors and the 64 KiB shape (200 blocks) with
226 ("Results" table).  The oracle's plan is replayed by brute force: copy by
descriptors, then every (lane, block) segment must sit at its rebuilt slab
address with the source bytes (the page's plan-replay check).  The library's
planner must agree with the oracle's exactly.
"""
import numpy as np
import pytest

import bf16_wire_all_amd as x
import datagen as dg
import oracle

MiB = 1 << 20


def _kv(B, seg, shuffle=None, n_slots=dg.N_SLOTS, bases=(1 << 40, (1 << 40) + (1 << 36))):
    rb = dg.region_bytes_for(B, n_slots, seg)
    pos = dg.permutation(B, shuffle) if shuffle is not None else None
    a = dg.kv_src_addrs(B, n_slots, seg, list(bases), pos=pos)
    return a, [(b, rb) for b in bases]


def _otable(t):
    return oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks)


@pytest.mark.parametrize("B,seg,want", [(1000, 4096, 72), (200, 65536, 226)])
def test_page_descriptor_counts(B, seg, want):
    a, regions = _kv(B, seg)
    t = x.runs_encode(a, seg)
    g = x.groups_plan(t, regions)
    od, oslab, _ = oracle.groups_plan(_otable(t), seg, regions)
    assert len(g.descs) == want and len(od) == want
    assert g.slab_bytes == oslab == a.size * seg             # the whole set, no holes
    assert g.n_groups == 2 and g.n_dense == 2                 # one dense group per region
    assert np.all(g.descs["bytes"] <= 32 * MiB)
    per_region = a.size * seg // 2
    assert np.sum(g.descs["bytes"] == 32 * MiB) == 2 * (per_region // (32 * MiB))


def _replay(t, seg, regions_host, descs, slab_bytes, local):
    """Copy by descriptors, then check every segment at its slab offset."""
    slab = np.full(slab_bytes, 0xEE, np.uint8)
    oracle.copy_descs(descs, regions_host, slab)
    addrs = oracle.runs_decode(_otable(t))
    for l in range(t.n_lanes):
        for b in range(t.n_blocks):
            a = int(addrs[l, b])
            for base, host in regions_host:
                if base <= a and a + seg <= base + host.nbytes:
                    src = host[a - base:a - base + seg]
                    break
            o = int(local[l, b])
            assert np.array_equal(slab[o:o + seg], src), (l, b)
    # destination ranges are disjoint and cover the slab exactly
    d = np.sort(descs, order="dst_off")
    assert d["dst_off"][0] == 0
    assert np.all(d["dst_off"][1:] == d["dst_off"][:-1] + d["bytes"][:-1])
    assert int(d["dst_off"][-1] + d["bytes"][-1]) == slab_bytes
    return slab


def _tiny_world(B, n_slots, seg, shuffle, n_regions=2, descending=False):
    rb = dg.region_bytes_for(B, n_slots, seg, n_regions)
    bases = [0x100000 + i * (rb + 4096) for i in range(n_regions)]
    pos = dg.permutation(B, shuffle) if shuffle is not None else None
    if descending:
        pos = np.arange(B - 1, -1, -1, dtype=np.uint32)
    a = dg.kv_src_addrs(B, n_slots, seg, bases, pos=pos)
    hosts = []
    for i, b in enumerate(bases):
        h = np.empty(rb, np.uint8)
        dg.fill_region(h, b, a, seg, 50 + i)
        hosts.append((b, h))
    return a, [(b, rb) for b in bases], hosts


WORLDS = [
    (6, 4, 64, None, 2, False),
    (9, 4, 64, 3, 2, False),
    (12, 6, 48, 4, 2, False),
    (7, 3, 32, 5, 1, False),
    (10, 2, 64, None, 2, True),       # descending blocks: negative strides, dense
    (33, 2, 16, 6, 1, False),
]


@pytest.mark.parametrize("B,S,seg,shuffle,nreg,desc", WORLDS)
@pytest.mark.parametrize("max_read", [32 * MiB, 96, 256])
def test_oracle_plan_replays(B, S, seg, shuffle, nreg, desc, max_read):
    a, regions, hosts = _tiny_world(B, S, seg, shuffle, nreg, desc)
    for t in (x.runs_encode(a, seg), x.runs_encode(a, seg, max_count=1), x.runs_encode(a, seg, max_count=3)):
        od, slab_bytes, local = oracle.groups_plan(_otable(t), seg, regions, max_read)
        assert np.all(od["bytes"] <= max_read)
        _replay(t, seg, hosts, od, slab_bytes, local)


@pytest.mark.parametrize("B,S,seg,shuffle,nreg,desc", WORLDS)
@pytest.mark.parametrize("max_read", [32 * MiB, 96])
def test_library_plan_equals_oracle(B, S, seg, shuffle, nreg, desc, max_read):
    a, regions, _ = _tiny_world(B, S, seg, shuffle, nreg, desc)
    for t in (x.runs_encode(a, seg), x.runs_encode(a, seg, max_count=1), x.runs_encode(a, seg, max_count=3)):
        g = x.groups_plan(t, regions, max_read)
        od, oslab, oloc = oracle.groups_plan(_otable(t), seg, regions, max_read)
        assert g.slab_bytes == oslab
        assert np.array_equal(g.descs.view(np.uint64), od.view(np.uint64))
        lt = g.local_table(t, 0)
        assert np.array_equal(oracle.runs_decode(_otable(lt)), oloc)
        # the rebuilt table is a valid destination over the slab: no two segments overlap
        assert x.runs_validate_status(g.local_table(t, 1 << 30), [(1 << 30, g.slab_bytes)], True) == x.OK


@pytest.mark.parametrize("shuffle", [dg.seed_for(5, 0, 1), 77])
def test_full_size_shuffled_plans_agree(shuffle):
    a, regions = _kv(dg.N_BLOCKS, dg.SEG_BYTES, shuffle)
    for max_count in (0, 1):
        t = x.runs_encode(a, dg.SEG_BYTES, max_count=max_count)
        g = x.groups_plan(t, regions)
        od, oslab, oloc = oracle.groups_plan(_otable(t), dg.SEG_BYTES, regions)
        assert np.array_equal(g.descs.view(np.uint64), od.view(np.uint64))
        assert g.slab_bytes == oslab == a.size * dg.SEG_BYTES
        assert np.array_equal(oracle.runs_decode(_otable(g.local_table(t, 0))), oloc)
        # every block's region chunk is read whole: at most 2 reads per block per region
        assert len(g.descs) <= 2 * dg.N_BLOCKS


def test_descriptor_checks():
    R = [(0x100000, 0x10000)]
    ok = np.array([(0x100000, 0, 4096), (0x101000, 4096, 4096)], dtype=x.DESC)
    st, _ = x.descs_prepare_status(ok, 8192, R, 0, 0)
    assert st == x.E_INVAL                                   # no device buffer: refused after the checks
    cases = [
        (x.E_INVAL, np.array([(0x100000, 0, 0)], x.DESC), 8192),          # empty descriptor
        (x.E_INVAL, np.array([(0x100008, 0, 4096)], x.DESC), 8192),       # misaligned source
        (x.E_INVAL, np.array([(0x100000, 8, 4096)], x.DESC), 8192),       # misaligned offset
        (x.E_RANGE, np.array([(0x10F000, 0, 8192)], x.DESC), 8192),       # leaves the region
        (x.E_RANGE, np.array([(0x100000, 4096, 8192)], x.DESC), 8192),    # past the slab end
        (x.E_OVERLAP, np.array([(0x100000, 0, 4096), (0x102000, 2048, 4096)], x.DESC), 8192),
    ]
    for code, d, slab in cases:
        st, _ = x.descs_prepare_status(d, slab, R, 0x200000, 1 << 20)
        assert st == code, (code, d)


# Worked examples: tables built by hand, plans derived by hand from the page's
# grouping rules (same blocks, same stride, base-adjacent, grown chunk fits the
# stride; per region; dense groups read whole).  Segments of 64 bytes.
def _table(rows, n_blocks, seg=64):
    """rows: per lane a list of (base, stride, count)."""
    rpl = [len(r) for r in rows]
    flat = [run for r in rows for run in r]
    return x.RunTable(np.array(rpl, np.uint32), np.array([f[0] for f in flat], np.uint64),
                      np.array([f[1] for f in flat], np.int64), np.array([f[2] for f in flat], np.uint32),
                      n_blocks, seg)


WORKED = [
    # interleaved lanes whose grown chunk (128) would not fit the stride (64): two groups
    ("chunk must fit the stride", [[(0x1000, 64, 3)], [(0x1040, 64, 3)]], 3, [(0x1000, 0x1000)],
     [(0x1000, 0, 192), (0x1040, 192, 192)], [[0, 64, 128], [192, 256, 320]]),
    # adjacent bases but different strides: no merge, each read block by block
    ("same stride", [[(0x1000, 256, 2)], [(0x1040, 512, 2)]], 2, [(0x1000, 0x1000)],
     [(0x1000, 0, 64), (0x1100, 64, 64), (0x1040, 128, 64), (0x1240, 192, 64)], [[0, 64], [128, 192]]),
    # touching regions: runs are grouped per region, never across
    ("per region", [[(0x1000, 0, 1)], [(0x1040, 0, 1)], [(0x1080, 0, 1)], [(0x10C0, 0, 1)]], 1,
     [(0x1000, 0x80), (0x1080, 0x80)], [(0x1000, 0, 128), (0x1080, 128, 128)], [[0], [64], [128], [192]]),
    # back-to-back chunks (chunk == stride): one dense read
    ("dense merge", [[(0x1000, 128, 2)], [(0x1040, 128, 2)]], 2, [(0x1000, 0x1000)],
     [(0x1000, 0, 256)], [[0, 128], [64, 192]]),
    # descending blocks, dense: the read starts at the lowest block
    ("dense descending", [[(0x1080, -128, 2)], [(0x10C0, -128, 2)]], 2, [(0x1000, 0x1000)],
     [(0x1000, 0, 256)], [[128, 0], [192, 64]]),
    # different block ranges: lane 0 is one run of 2, lane 1 two runs of 1
    ("same blocks", [[(0x1000, 128, 2)], [(0x1040, 0, 1), (0x10C0, 0, 1)]], 2, [(0x1000, 0x1000)],
     [(0x1000, 0, 64), (0x1080, 64, 64), (0x1040, 128, 64), (0x10C0, 192, 64)], [[0, 64], [128, 192]]),
]


@pytest.mark.parametrize("name,rows,n_blocks,regions,want_descs,want_local", WORKED, ids=[w[0] for w in WORKED])
def test_worked_examples(name, rows, n_blocks, regions, want_descs, want_local):
    t = _table(rows, n_blocks)
    od, oslab, oloc = oracle.groups_plan(_otable(t), 64, regions, 32 * MiB)
    assert [tuple(int(v) for v in d) for d in od] == want_descs, name
    assert oloc.tolist() == want_local, name
    assert oslab == sum(d[2] for d in want_descs)
    g = x.groups_plan(t, regions)
    assert [tuple(int(v) for v in d) for d in g.descs] == want_descs, name
    assert oracle.runs_decode(_otable(g.local_table(t, 0))).tolist() == want_local, name


def test_descriptors_stay_inside_one_region():
    """Regions that touch: the plan never reads across a region boundary."""
    B, S, seg = 8, 4, 64
    rb = dg.region_bytes_for(B, S, seg)
    bases = [0x200000, 0x200000 + rb]                      # region 1 starts where region 0 ends
    a = dg.kv_src_addrs(B, S, seg, bases)
    regions = [(b, rb) for b in bases]
    for t in (x.runs_encode(a, seg), x.runs_encode(a, seg, max_count=1)):
        od, _, _ = oracle.groups_plan(_otable(t), seg, regions)
        for d in od:
            s, e = int(d["src"]), int(d["src"] + d["bytes"])
            assert any(b <= s and e <= b + n for b, n in regions), d
        assert len(x.groups_plan(t, regions).descs) == len(od)
