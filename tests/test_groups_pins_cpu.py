"""Pins of the coalescing planner's grouping that go through neither
oracle/oracle.c nor the library's planner (groups.cpp).

- tests/plan_reference.py restates the grouping of the run-encoded transfer
  page (pegaflow PR 350, "What this PR does" steps 2-5, "READ splitting")
  from the expanded segment list, organised by classes of runs instead of the
  implementations' single sorted sweep.  Both implementations must produce
  its descriptors, slab size and rebuilt local offsets exactly, on every
  small world, three encodings and three read sizes, and on the full
  paged K/V sets (dense, shuffled greedy, one run per segment).
- From the segments alone (no planner): the reads tile the segments exactly,
  i.e. no byte outside a segment is read ("tile densely") and every segment
  is read once.
- Hand examples, each derived by hand from the page's rules: negative strides
  (ascending and descending lanes side by side) and split runs (a lane whose
  blocks break into several runs next to lanes that do not).
"""
import numpy as np
import pytest

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests import plan_reference as ref

MiB = 1 << 20


def _otable(t):
    return oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks)


def _arrays(t):
    return t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks


def _as_list(descs):
    return [(int(d["src"]), int(d["dst_off"]), int(d["bytes"])) for d in descs]


def _check_against_reference(t, seg, regions, max_read):
    want, want_slab, want_local = ref.plan(*_arrays(t), seg, regions, max_read)
    addr, _ = ref.expand(*_arrays(t))
    assert ref.reads_only_segments(want, addr, seg)
    od, oslab, oloc = oracle.groups_plan(_otable(t), seg, regions, max_read)
    assert _as_list(od) == want
    assert oslab == want_slab
    assert np.array_equal(oloc, want_local)
    g = x.groups_plan(t, regions, max_read)
    assert _as_list(g.descs) == want
    assert g.slab_bytes == want_slab
    assert np.array_equal(oracle.runs_decode(_otable(g.local_table(t, 0))), want_local)
    return want


def _world(B, n_slots, seg, shuffle, n_regions=2, descending=False, gap=4096):
    rb = dg.region_bytes_for(B, n_slots, seg, n_regions)
    bases = [0x100000 + i * (rb + gap) for i in range(n_regions)]
    pos = dg.permutation(B, shuffle) if shuffle is not None else None
    if descending:
        pos = np.arange(B - 1, -1, -1, dtype=np.uint32)
    return dg.kv_src_addrs(B, n_slots, seg, bases, pos=pos), [(b, rb) for b in bases]


WORLDS = [
    (6, 4, 64, None, 2, False),
    (9, 4, 64, 3, 2, False),
    (12, 6, 48, 4, 2, False),
    (7, 3, 32, 5, 1, False),
    (10, 2, 64, None, 2, True),
    (33, 2, 16, 6, 1, False),
    (16, 5, 64, 8, 1, False),
    (20, 1, 32, None, 1, True),
]


@pytest.mark.parametrize("B,S,seg,shuffle,nreg,desc", WORLDS)
@pytest.mark.parametrize("max_read", [32 * MiB, 96, 256])
def test_plans_equal_the_reference(B, S, seg, shuffle, nreg, desc, max_read):
    a, regions = _world(B, S, seg, shuffle, nreg, desc)
    for mc in (0, 1, 2, 3):
        t = x.runs_encode(a, seg, max_count=mc)
        _check_against_reference(t, seg, regions, max_read)


def _gapped_world(B, n_slots, seg, gap, shuffle, n_regions=2):
    """Paged K/V layout whose lanes sit seg + gap bytes apart inside a block
    chunk (gap bytes between neighbouring segments): runs over the same
    blocks with the same stride that are not base-adjacent."""
    per = n_slots // n_regions
    pitch = seg + gap
    chunk = 2 * per * pitch
    rb = B * chunk
    bases = [0x400000 + i * (rb + 8192) for i in range(n_regions)]
    pos = dg.permutation(B, shuffle) if shuffle is not None else np.arange(B)
    a = np.zeros((2 * n_slots, B), np.uint64)
    for s in range(n_slots):
        g, j = divmod(s, per)
        for kv in range(2):
            a[2 * s + kv] = bases[g] + pos.astype(np.uint64) * chunk + (2 * j + kv) * pitch
    return a, [(b, rb) for b in bases]


@pytest.mark.parametrize("gap", [16, 64])
@pytest.mark.parametrize("shuffle", [None, 11])
def test_gapped_lanes_equal_the_reference(gap, shuffle):
    a, regions = _gapped_world(9, 4, 64, gap, shuffle)
    for mc in (0, 1, 2):
        want = _check_against_reference(x.runs_encode(a, 64, max_count=mc), 64, regions, 32 * MiB)
        assert all(n == 64 for _, _, n in want)       # no two segments are adjacent: one read each


@pytest.mark.parametrize("B", [8, 1])
def test_touching_regions_equal_the_reference(B):
    """Region 1 starts where region 0 ends: a dense region may not be read
    into its neighbour, even though the addresses continue (with one block,
    region 0's last segment ends exactly at region 1's first)."""
    S, seg = 4, 64
    rb = dg.region_bytes_for(B, S, seg)
    bases = [0x200000, 0x200000 + rb]
    a = dg.kv_src_addrs(B, S, seg, bases)
    for mc in (0, 1):
        want = _check_against_reference(x.runs_encode(a, seg, max_count=mc), seg, [(b, rb) for b in bases], 32 * MiB)
        for src, _, n in want:
            assert any(b <= src and src + n <= b + rb for b in bases)


@pytest.mark.parametrize("shuffle,max_count", [(None, 0), (dg.seed_for(5, 0, 1), 0), (dg.seed_for(5, 0, 1), 1)])
def test_full_size_sets_equal_the_reference(shuffle, max_count):
    """The 1000 x 288 x 2 x 4 KiB set: bump-allocated (72 reads), shuffled
    blocks by the greedy table and by one run per segment."""
    bases = (1 << 40, (1 << 40) + (1 << 36))
    rb = dg.region_bytes_for(dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES)
    pos = dg.permutation(dg.N_BLOCKS, shuffle) if shuffle is not None else None
    a = dg.kv_src_addrs(dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES, list(bases), pos=pos)
    t = x.runs_encode(a, dg.SEG_BYTES, max_count=max_count)
    want = _check_against_reference(t, dg.SEG_BYTES, [(b, rb) for b in bases], 32 * MiB)
    chunk = dg.N_SLOTS // 2 * 2 * dg.SEG_BYTES                  # one block's share of a region
    if shuffle is None:
        assert len(want) == 72
    elif max_count == 1:
        # one-block runs: each block's chunk of a region is one contiguous range, read whole
        assert len(want) == 2 * dg.N_BLOCKS and all(n == chunk for _, _, n in want)
    else:
        # greedy runs of two blocks whose positions happen to be adjacent tile densely and
        # are read as one range of two chunks; every other block chunk is read alone
        assert all(n in (chunk, 2 * chunk) for _, _, n in want)
        assert sum(n for _, _, n in want) == a.size * dg.SEG_BYTES


def _table(rows, n_blocks, seg=64):
    """rows: per lane a list of (base, stride, count)."""
    rpl = [len(r) for r in rows]
    flat = [run for r in rows for run in r]
    return x.RunTable(np.array(rpl, np.uint32), np.array([f[0] for f in flat], np.uint64),
                      np.array([f[1] for f in flat], np.int64), np.array([f[2] for f in flat], np.uint32),
                      n_blocks, seg)


# (name, lanes, n_blocks, regions, expected descriptors, expected local offsets); segments of 64 bytes.
HAND = [
    # Two descending lanes side by side (stride -256): K and V of a slot merge
    # (chunk 128 fits 256) but the blocks' chunks are 128 bytes apart, so the
    # group is read block by block, from block 0 (the highest addresses) down.
    ("descending, not dense", [[(0x1200, -256, 3)], [(0x1240, -256, 3)]], 3, [(0x1000, 0x1000)],
     [(0x1200, 0, 128), (0x1100, 128, 128), (0x1000, 256, 128)], [[0, 128, 256], [64, 192, 320]]),
    # An ascending and a descending lane with base-adjacent starts: different
    # strides, never one group; each lane alone is read block by block.
    ("ascending next to descending", [[(0x1000, 256, 2)], [(0x1040, -256, 2)]], 2, [(0x0F00, 0x1000)],
     [(0x1000, 0, 64), (0x1100, 64, 64), (0x1040, 128, 64), (0x0F40, 192, 64)], [[0, 64], [128, 192]]),
    # Four descending lanes filling the stride: dense, one read from the lowest block.
    ("descending, dense", [[(0x1100, -256, 2)], [(0x1140, -256, 2)], [(0x1180, -256, 2)], [(0x11C0, -256, 2)]],
     2, [(0x1000, 0x1000)], [(0x1000, 0, 512)], [[256, 0], [320, 64], [384, 128], [448, 192]]),
    # Lane 1 is split into two runs (blocks [0, 2) and [2, 4)); lane 0 is one
    # run over [0, 4).  Lane 1's first run starts right after lane 0's base
    # with the same stride, but covers other blocks: no merge.  Every run is
    # read block by block.
    ("split run, same stride", [[(0x1000, 256, 4)], [(0x1040, 256, 2), (0x2000, 256, 2)]], 4,
     [(0x1000, 0x2000)],
     [(0x1000, 0, 64), (0x1100, 64, 64), (0x1200, 128, 64), (0x1300, 192, 64),
      (0x1040, 256, 64), (0x1140, 320, 64), (0x2000, 384, 64), (0x2100, 448, 64)],
     [[0, 64, 128, 192], [256, 320, 384, 448]]),
    # Both lanes split the same way (blocks [0, 2) and [2, 4)): the runs over
    # the same blocks merge pairwise, and each pair is dense (stride 128 ==
    # chunk): two reads.
    ("split runs, pairwise merge", [[(0x1000, 128, 2), (0x2000, 128, 2)], [(0x1040, 128, 2), (0x2040, 128, 2)]], 4,
     [(0x1000, 0x2000)], [(0x1000, 0, 256), (0x2000, 256, 256)], [[0, 128, 256, 384], [64, 192, 320, 448]]),
    # Three lanes whose chunk (192 bytes) is shorter than the stride (256):
    # one group, read block by block.
    ("three lanes, short chunk", [[(0x1000, 256, 2)], [(0x1040, 256, 2)], [(0x1080, 256, 2)]], 2,
     [(0x1000, 0x1000)], [(0x1000, 0, 192), (0x1100, 192, 192)], [[0, 192], [64, 256], [128, 320]]),
    # Same blocks and stride, but 64 bytes between the lanes' bases: not
    # base-adjacent, two groups, each read block by block.
    ("gap between lanes", [[(0x1000, 256, 2)], [(0x1080, 256, 2)]], 2, [(0x1000, 0x1000)],
     [(0x1000, 0, 64), (0x1100, 64, 64), (0x1080, 128, 64), (0x1180, 192, 64)], [[0, 64], [128, 192]]),
    # One block, four lanes back to back across two touching regions: one
    # read per region, never one read across the boundary.
    ("touching regions, one block", [[(0x1000, 0, 1)], [(0x1040, 0, 1)], [(0x1080, 0, 1)], [(0x10C0, 0, 1)]], 1,
     [(0x1000, 0x80), (0x1080, 0x80)], [(0x1000, 0, 128), (0x1080, 128, 128)], [[0], [64], [128], [192]]),
]

# Source tables whose segments overlap (legal for a source: only destinations
# must be disjoint).  Only here can the chunk outgrow the stride; the plans are
# derived by hand and compared with both implementations directly.
OVERLAPPING = [
    # Three base-adjacent lanes, stride 128: the first two fill the stride
    # (dense, one read); the third would make the chunk 192 > 128 and starts
    # its own group, read block by block.
    ("chain cut where the chunk outgrows the stride", [[(0x1000, 128, 2)], [(0x1040, 128, 2)], [(0x1080, 128, 2)]],
     2, [(0x1000, 0x1000)], [(0x1000, 0, 256), (0x1080, 256, 64), (0x1100, 320, 64)],
     [[0, 128], [64, 192], [256, 320]]),
    # Interleaved lanes, stride 64 == seg: no two lanes fit one chunk.
    ("stride of one segment", [[(0x1000, 64, 3)], [(0x1040, 64, 3)]], 3, [(0x1000, 0x1000)],
     [(0x1000, 0, 192), (0x1040, 192, 192)], [[0, 64, 128], [192, 256, 320]]),
]


@pytest.mark.parametrize("name,rows,n_blocks,regions,want_descs,want_local", OVERLAPPING,
                         ids=[h[0] for h in OVERLAPPING])
def test_overlapping_sources_by_hand(name, rows, n_blocks, regions, want_descs, want_local):
    t = _table(rows, n_blocks)
    addr, _ = ref.expand(*_arrays(t))
    assert not ref.segments_disjoint(addr, 64)
    od, oslab, oloc = oracle.groups_plan(_otable(t), 64, regions, 32 * MiB)
    assert _as_list(od) == want_descs, name
    assert oloc.tolist() == want_local, name
    assert oslab == sum(d[2] for d in want_descs)
    g = x.groups_plan(t, regions)
    assert _as_list(g.descs) == want_descs, name
    assert oracle.runs_decode(_otable(g.local_table(t, 0))).tolist() == want_local, name


@pytest.mark.parametrize("name,rows,n_blocks,regions,want_descs,want_local", HAND, ids=[h[0] for h in HAND])
def test_hand_examples(name, rows, n_blocks, regions, want_descs, want_local):
    t = _table(rows, n_blocks)
    addr, _ = ref.expand(*_arrays(t))
    assert ref.reads_only_segments(want_descs, addr, 64), name       # the hand plan itself tiles the segments
    got = _check_against_reference(t, 64, regions, 32 * MiB)
    assert got == want_descs, name
    od, _, oloc = oracle.groups_plan(_otable(t), 64, regions, 32 * MiB)
    assert oloc.tolist() == want_local, name


def test_a_group_over_other_blocks_would_read_outside_the_segments():
    """The property the 'same blocks' rule protects: merging lane 1's first
    run (blocks [0, 2)) into lane 0's group (blocks [0, 4)) would read lane
    1's chunk at blocks 2 and 3 too, bytes that are not segments."""
    t = _table(HAND[3][1], 4)
    addr, _ = ref.expand(*_arrays(t))
    merged = [(0x1000 + b * 256, b * 128, 128) for b in range(4)] + [(0x2000, 512, 64), (0x2100, 576, 64)]
    assert not ref.reads_only_segments(merged, addr, 64)
