"""GPU parity of the coalesced fetch (xfer_groups_plan + xfer_copy_descs)
against the CPU oracle, byte for byte: the slab the descriptor kernel fills
must equal the oracle's copy by the same descriptors, and gathering from the
slab through the re-based ("local") table must give the staging that
gathering from the source gives.  Small layouts of every shape class, reads
split at odd sizes, and the full paged-K/V sets (4 KiB segments dense and
shuffled, 64 KiB segments dense)."""
import ctypes

import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, say, zeros

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


def _otable(t: x.RunTable) -> oracle.RunTable:
    return oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks)


def _world(n_blocks, n_slots, seg, shuffle_seed, n_regions=2, descending=False):
    rb = dg.region_bytes_for(n_blocks, n_slots, seg, n_regions)
    regs = [zeros(rb) for _ in range(n_regions)]
    bases = [r.data_ptr() for r in regs]
    pos = dg.permutation(n_blocks, shuffle_seed) if shuffle_seed is not None else None
    if descending:
        pos = np.arange(n_blocks - 1, -1, -1, dtype=np.uint32)
    addrs = dg.kv_src_addrs(n_blocks, n_slots, seg, bases, pos=pos)
    hosts = []
    for i, r in enumerate(regs):
        h = np.empty(rb, np.uint8)
        dg.fill_region(h, bases[i], addrs, seg, 3000 + i + (shuffle_seed or 0))
        r.copy_(torch.from_numpy(h))
        hosts.append(h)
    return regs, hosts, addrs


def _fetch(t, regions, max_read=x.MAX_READ_BYTES, tail=256):
    """Plan, upload and run the coalesced fetch; returns (plan, slab tensor)."""
    g = x.groups_plan(t, regions, max_read)
    dev = zeros(max(16, x.descs_plan_bytes(len(g.descs))))
    p = x.descs_prepare(g.descs, g.slab_bytes, regions, dev)
    slab = filled(g.slab_bytes + tail, SENTINEL)
    x.copy_descs(p, slab)
    return g, slab, dev


def _check_fetch(t, regs, hosts, seg, max_read=x.MAX_READ_BYTES):
    regions = [(r.data_ptr(), r.numel()) for r in regs]
    oregions = [(r.data_ptr(), h) for r, h in zip(regs, hosts)]
    g, slab, _dev = _fetch(t, regions, max_read)
    od, oslab_bytes, oloc = oracle.groups_plan(_otable(t), seg, regions, max_read)
    assert np.array_equal(g.descs.view(np.uint64), od.view(np.uint64))
    want = np.full(oslab_bytes, SENTINEL, np.uint8)
    oracle.copy_descs(od, oregions, want)
    got = down(slab)
    assert np.array_equal(got[:oslab_bytes], want)
    assert np.all(got[oslab_bytes:] == SENTINEL)
    return g, slab, oregions, oloc


SMALL = [
    # (n_blocks, n_slots, seg_bytes, shuffle seed, regions, descending)
    (1, 1, 16, None, 1, False),
    (6, 4, 64, None, 2, False),
    (9, 4, 64, 3, 2, False),
    (12, 6, 48, 4, 2, False),
    (10, 2, 64, None, 2, True),
    (33, 2, 4096, 6, 1, False),
    (65, 4, 4096, None, 2, False),
    (7, 2, 65536, 7, 2, False),
]


@pytest.mark.parametrize("n_blocks,n_slots,seg,shuffle,nreg,desc", SMALL)
def test_fetch_small(n_blocks, n_slots, seg, shuffle, nreg, desc):
    say("fetch small", n_blocks, n_slots, seg, shuffle, nreg, desc)
    regs, hosts, addrs = _world(n_blocks, n_slots, seg, shuffle, nreg, desc)
    for max_count in (0, 1, 3):
        t = x.runs_encode(addrs, seg, max_count=max_count)
        g, slab, oregions, oloc = _check_fetch(t, regs, hosts, seg)
        # gather from the slab through the re-based table == gather from the source
        lt = g.local_table(t, slab.data_ptr())
        assert np.array_equal(oracle.runs_decode(_otable(lt)) - np.uint64(slab.data_ptr()), oloc)
        buf = zeros(max(16, x.runs_plan_bytes(lt)))
        plan = x.runs_prepare(lt, [(slab.data_ptr(), g.slab_bytes)], False, buf)
        staging = zeros(t.n_lanes * t.n_blocks * seg)
        x.gather_runs(plan, staging)
        assert np.array_equal(down(staging), oracle.gather(_otable(t), seg, oregions))


@pytest.mark.parametrize("max_read", [16, 8192 + 16, 3 * 8192, 100 * 1024 + 48])
def test_fetch_split_reads(max_read):
    """Reads cut at sizes below, across and off the 8 KiB piece of one workgroup."""
    say("fetch split", max_read)
    regs, hosts, addrs = _world(40, 4, 1024, None, 2)
    _check_fetch(x.runs_encode(addrs, 1024), regs, hosts, 1024, max_read)


@pytest.mark.parametrize("layout", ["dense", "shuffled", "shuffled-per-segment"])
def test_full_size_fetch(layout):
    B, S, SEG = dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES
    say("full-size fetch", layout)
    shuffle = None if layout == "dense" else dg.seed_for(5, 0, 1)
    regs, hosts, addrs = _world(B, S, SEG, shuffle)
    t = x.runs_encode(addrs, SEG, max_count=1 if layout == "shuffled-per-segment" else 0)
    g, slab, _, _ = _check_fetch(t, regs, hosts, SEG)
    if layout == "dense":
        assert len(g.descs) == 72
    else:
        assert len(g.descs) <= 2 * B
    del slab, regs
    torch.cuda.empty_cache()


def test_full_size_fetch_64k():
    say("full-size fetch 64 KiB")
    regs, hosts, addrs = _world(200, dg.N_SLOTS, 65536, None)
    g, slab, _, _ = _check_fetch(x.runs_encode(addrs, 65536), regs, hosts, 65536)
    assert len(g.descs) == 226
    del slab, regs
    torch.cuda.empty_cache()


def test_fetch_misuse_refused():
    regs, hosts, addrs = _world(4, 2, 64, None, 1)
    region = [(regs[0].data_ptr(), regs[0].numel())]
    g = x.groups_plan(x.runs_encode(addrs, 64), region)
    dev = zeros(max(16, x.descs_plan_bytes(len(g.descs))))
    p = x.descs_prepare(g.descs, g.slab_bytes, region, dev)
    L = x.lib()
    slab = filled(g.slab_bytes, 0x11)
    assert L.xfer_copy_descs(ctypes.byref(p), slab.data_ptr(), g.slab_bytes - 16, None) == x.E_INVAL
    assert L.xfer_copy_descs(ctypes.byref(p), slab.data_ptr() + 8, g.slab_bytes, None) == x.E_INVAL
    assert L.xfer_copy_descs(ctypes.byref(p), regs[0].data_ptr(), g.slab_bytes, None) == x.E_INVAL  # slab = source
    assert np.all(down(slab) == 0x11)
    empty = x.descs_prepare(np.zeros(0, x.DESC), 0, region, dev)
    assert L.xfer_copy_descs(ctypes.byref(empty), slab.data_ptr(), 16, None) == x.OK
    assert np.all(down(slab) == 0x11)


def test_slab_between_the_two_regions():
    """One allocation holds region 0, then the slab, then region 1: the slab
    shares no byte with either region's sources, so the fetch into it is
    accepted and equals the oracle's copy; a slab reaching into region 1 is
    refused."""
    n_blocks, n_slots, seg = 30, 6, 4096
    rb = dg.region_bytes_for(n_blocks, n_slots, seg, 2)
    sb = 2 * rb
    arena = zeros(rb + sb + rb)
    bases = [arena.data_ptr(), arena.data_ptr() + rb + sb]
    addrs = dg.kv_src_addrs(n_blocks, n_slots, seg, bases, pos=dg.permutation(n_blocks, 91))
    hosts = []
    for i in range(2):
        h = np.empty(rb, np.uint8)
        dg.fill_region(h, bases[i], addrs, seg, 4000 + i)
        hosts.append(h)
    arena[:rb].copy_(torch.from_numpy(hosts[0]))
    arena[rb + sb:].copy_(torch.from_numpy(hosts[1]))
    t = x.runs_encode(addrs, seg)
    regions = [(bases[0], rb), (bases[1], rb)]
    g = x.groups_plan(t, regions)
    assert g.slab_bytes == sb
    dev = zeros(max(16, x.descs_plan_bytes(len(g.descs))))
    p = x.descs_prepare(g.descs, g.slab_bytes, regions, dev)
    assert p.n_spans == 2
    say("slab between the regions", n_blocks, n_slots)
    assert lib_copy(p, arena.data_ptr() + rb + seg, sb) == x.E_INVAL            # one segment into region 1
    slab = arena[rb:rb + sb]
    x.copy_descs(p, slab)
    want = np.zeros(sb, np.uint8)
    oracle.copy_descs(g.descs, [(bases[0], hosts[0]), (bases[1], hosts[1])], want)
    assert np.array_equal(down(slab), want)
    assert np.array_equal(down(arena[:rb]), hosts[0]) and np.array_equal(down(arena[rb + sb:]), hosts[1])


def lib_copy(plan, slab_ptr, slab_bytes):
    """The raw call (returns the status; the current stream)."""
    return x.lib().xfer_copy_descs(ctypes.byref(plan), slab_ptr, slab_bytes,
                                   torch.cuda.current_stream().cuda_stream)
