"""The C-ABI boundary on the CPU: the library loads, exports every call the
header declares, and its host-side logic (argument checks, run-table
validation and encoding, plan sizing) behaves as documented.  No call here
reaches a kernel launch: every argument set either fails a host check or is
empty work."""
import ctypes
import os
import re

import numpy as np
import pytest

import bf16_wire_all_amd as x
import datagen as dg
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
S0 = 0  # NULL stream: nothing here is enqueued


def _declared():
    with open(os.path.join(ROOT, "include", "xfer.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"XFER_API\s+[\w\s\*]*?\b(xfer_\w+)\s*\(", text)))


def test_library_exports_every_declared_call():
    names = _declared()
    assert len(names) == 29
    assert set(names) == set(x.EXPORTED)
    L = x.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(8):
        assert x.status_str(s) and x.status_str(s) != "unknown status"
    assert x.status_str(99) == "unknown status"


# -------------------------------------------------------------------- pack

def test_pack_argument_checks():
    f = lambda *a: x.pack_bf16_raw(*a, stream=S0)
    src, ring = 0x100000, 0x900000
    assert f(src, 100, ring, 64, 0, 0, 1) == x.E_INVAL            # chunk_bytes 0
    assert f(src, 100, ring, 64, 24, 0, 1) == x.E_INVAL           # not a multiple of 16
    assert f(src, 100, ring, 48, 32, 0, 1) == x.E_INVAL           # ring not a multiple of chunk
    assert f(src, 100, ring, 0, 32, 0, 1) == x.E_INVAL            # empty ring
    assert f(src, 100, ring, 64, 32, 2, 1) == x.E_INVAL           # begin > end
    assert f(src, 100, ring, 64, 32, 0, 3) == x.E_INVAL           # 3 chunks into 2 slots
    assert f(src, 0, ring, 64, 32, 0, 1) == x.E_INVAL             # n == 0: chunk 0 starts at n
    assert f(src, 0, ring, 64, 32, 0, 0) == x.OK                  # n == 0, no chunk: empty work
    assert f(0, 0, 0, 64, 32, 1, 1) == x.OK                       # empty range: nothing is read
    assert f(src, 100, ring, 64, 32, 1, 1) == x.OK                # empty chunk range
    assert f(0, 100, ring, 64, 32, 0, 1) == x.E_INVAL             # NULL src
    assert f(src + 4, 100, ring, 64, 32, 0, 1) == x.E_INVAL       # misaligned src
    assert f(src, 100, ring + 2, 64, 32, 0, 1) == x.E_INVAL       # misaligned ring
    assert f(src, 100, ring, 64, 32, 7, 8) == x.E_INVAL           # chunk 7 starts past n=100 (CE 16)
    assert f(src, 100, ring, 64, 32, 6, 8) == x.E_INVAL           # chunk 7 named
    assert f(src, 100, src + 128, 64, 32, 0, 1) == x.E_INVAL      # ring inside src


def test_combine_argument_checks():
    f = lambda *a: x.combine2_raw(*a, stream=S0)
    a, b, o = 0x100000, 0x200000, 0x300000
    assert f(a, b, 10, o, 2) == x.E_INVAL                         # unknown mode
    assert f(a, b, 0, o, 0) == x.OK                               # empty
    assert f(0, b, 10, o, 0) == x.E_INVAL
    assert f(a, b, 10, 0, 1) == x.E_INVAL
    assert f(a + 8, b, 10, o, 0) == x.E_INVAL                     # misaligned
    assert f(a, b, 10, a + 16, 0) == x.E_INVAL                    # F32 out overlaps a
    assert f(a, b, 10, a, 0) == x.E_INVAL                         # F32 out cannot alias a
    assert f(a, b, 1000, b - 16, 1) == x.E_INVAL                  # BF16 out overlaps b partly
    assert f(a, a + 16, 10, a, 1) == x.E_INVAL                    # in place, but b overlaps out


def test_combine_f32_argument_checks():
    f = lambda *a: x.combine2_f32_raw(*a, stream=S0)
    a, b, o = 0x100000, 0x200000, 0x300000
    assert f(a, b, 10, o, 2) == x.E_INVAL                         # unknown mode
    assert f(a, b, 0, o, 0) == x.OK                               # empty
    assert f(0, b, 10, o, 0) == x.E_INVAL
    assert f(a, b, 10, 0, 1) == x.E_INVAL
    assert f(a + 8, b, 10, o, 0) == x.E_INVAL                     # misaligned
    assert f(a, b, 10, a + 16, 0) == x.E_INVAL                    # F32 out overlaps a partly
    assert f(a, b, 10, a, 1) == x.E_INVAL                         # BF16 out cannot alias a (other width)
    assert f(a, b, 1000, b - 16, 0) == x.E_INVAL                  # overlaps b partly
    assert f(a, a + 16, 10, a, 0) == x.E_INVAL                    # in place, but b overlaps out
    assert f(a, b, ((1 << 24) - 1) * 2048 + 4, 1 << 40, 0) == x.E_UNSUPPORTED


# ------------------------------------------------------------------ argmax

def _sh(ptr=0x100000, ld=1024, rows=4, ncols=512, off=0):
    return x.shard(ptr, ld, rows, ncols, off)


def test_argmax_argument_checks():
    f = lambda s0, s1, mode=0, out=0x900000, ws=0xA00000, wsb=1 << 20: x.argmax_merge_raw(s0, s1, mode, out, ws,
                                                                                             wsb, stream=S0)
    s0 = _sh()
    s1 = _sh(ptr=0x100000 + 1024, ncols=512, off=512)
    assert f(s0, s1, mode=2) == x.E_INVAL                         # unknown mode
    assert f(s0, _sh(rows=3, off=512, ptr=0x100400)) == x.E_INVAL  # row counts differ
    assert f(_sh(rows=0), _sh(rows=0, off=512)) == x.OK           # no rows: empty work
    assert f(s0, _sh(ncols=0, off=512)) == x.E_INVAL              # empty shard
    assert f(s0, _sh(off=100, ptr=0x100400)) == x.E_INVAL         # id ranges overlap
    assert f(s0, _sh(off=(1 << 31) - 10, ptr=0x100400)) == x.E_INVAL  # ids past 2^31
    wide = 32 * 65536                                             # 32 slices of 65,536 columns
    assert f(_sh(ncols=wide + 1, ld=wide + 8), _sh(off=wide + 1, ptr=1 << 34), out=1 << 36, ws=1 << 37) \
        == x.E_UNSUPPORTED
    assert f(_sh(ncols=wide, ld=wide), _sh(off=wide, ptr=1 << 34), out=1 << 36, ws=1 << 37, wsb=16) \
        == x.E_INVAL                                              # the widest shard passes, then the workspace is short
    assert x.argmax_workspace_bytes(4, wide, 1) == 4 * 2 * 32 * 8  # 32 slices per shard
    assert x.argmax_workspace_bytes(4096, 65536, 1) == 4096 * 2 * 1 * 8  # many rows: one slice per shard
    assert x.argmax_workspace_bytes(4096, 65537, 1) == 4096 * 2 * 2 * 8  # a slice holds at most 65,536 columns
    assert f(_sh(ptr=0x100002), s1) == x.E_INVAL                  # misaligned shard
    assert f(_sh(ld=1001), s1) == x.E_INVAL                       # row stride not 16 B
    assert f(_sh(ld=256), s1) == x.E_INVAL                        # rows overlap (ld < ncols)
    assert f(s0, s1, out=0) == x.E_INVAL
    assert f(s0, s1, ws=0) == x.E_INVAL
    assert f(s0, s1, wsb=16) == x.E_INVAL                         # workspace too small
    assert f(s0, s1, out=0x100000 + 64) == x.E_INVAL              # out inside the logits
    assert f(s0, s1, ws=0x100000 + 64) == x.E_INVAL               # workspace inside the logits
    assert f(s0, s1, out=0xA00000 + 32) == x.E_INVAL              # out inside the workspace


def test_argmax_noalloc_argument_checks():
    """The no-allocation form runs the same checks, and refuses on the host
    (before any runtime call) partial records that need more than the
    library's static array: more than 4096 rows."""
    f = lambda s0, s1, mode=0, out=0x900000: x.argmax_merge_noalloc_raw(s0, s1, mode, out, stream=S0)
    s0 = _sh()
    s1 = _sh(ptr=0x100000 + 1024, ncols=512, off=512)
    assert f(s0, s1, mode=2) == x.E_INVAL
    assert f(s0, _sh(rows=3, off=512, ptr=0x100400)) == x.E_INVAL
    assert f(_sh(rows=0), _sh(rows=0, off=512), out=0) == x.OK    # no rows: empty work
    assert f(s0, _sh(off=100, ptr=0x100400)) == x.E_INVAL
    assert f(_sh(ncols=32 * 65536 + 1, ld=32 * 65536 + 8), _sh(off=32 * 65536 + 1, ptr=1 << 34),
             out=1 << 36) == x.E_UNSUPPORTED
    assert f(s0, s1, out=0) == x.E_INVAL
    assert f(s0, s1, out=0x900008) == x.E_INVAL                   # misaligned output
    assert f(s0, s1, out=0x100000 + 64) == x.E_INVAL              # out inside the logits
    ld = 64768 + 64512
    big = 4097
    assert x.argmax_workspace_bytes(4096, 64768, 64512) <= x.ARGMAX_SCRATCH_BYTES
    assert x.argmax_workspace_bytes(big, 64768, 64512) > x.ARGMAX_SCRATCH_BYTES
    b0 = x.shard(1 << 32, ld, big, 64768, 0)
    b1 = x.shard((1 << 32) + 2 * 64768, ld, big, 64512, 64768)
    assert f(b0, b1, out=1 << 40) == x.E_UNSUPPORTED              # beyond the static array


def test_argmax_workspace_size_is_monotone_and_small():
    sizes = [x.argmax_workspace_bytes(r, 64768, 64512) for r in (1, 4, 16, 256, 4096)]
    assert all(s > 0 for s in sizes)
    assert sizes[2] <= 16 * 1024                                   # 16 rows x 129280 vocab: a few KB
    assert sizes[-1] <= 4096 * 64


# -------------------------------------------------------------- run tables

def _dense_world(n_blocks=40, n_slots=6, seg=64):
    rb = dg.region_bytes_for(n_blocks, n_slots, seg)
    bases = [1 << 32, (1 << 32) + 4 * rb]
    a = dg.kv_src_addrs(n_blocks, n_slots, seg, bases)
    return a, [(bases[0], rb), (bases[1], rb)], seg


@pytest.mark.parametrize("kind", ["dense", "shuffled", "random", "adversarial", "full_size_dense",
                                  "full_size_shuffled"])
def test_library_encoder_matches_oracle(kind):
    if kind == "dense":
        a, _, _ = _dense_world()
    elif kind == "shuffled":
        a = dg.kv_src_addrs(50, 4, 64, [1 << 20, 1 << 30], pos=dg.permutation(50, 3))
    elif kind == "random":
        a = dg.random_u64(5 * 64, 42).reshape(5, 64)
    elif kind == "adversarial":
        a = np.tile(np.array([0, 2**63 + 16, 32, 2**64 - 16, 5, 5, 5, 10, 15, 20, 0, 2**63, 2**64 - 2**63],
                             dtype=np.uint64), (3, 1))
    elif kind == "full_size_dense":
        a = dg.kv_src_addrs(dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES, [1 << 40, (1 << 40) + (1 << 33)])
    else:
        a = dg.kv_src_addrs(dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES, [1 << 40, (1 << 40) + (1 << 33)],
                            pos=dg.permutation(dg.N_BLOCKS, dg.seed_for(5, 0, 1)))
    ours = x.runs_encode(a, 64)
    ref = oracle.runs_encode(a)
    assert np.array_equal(ours.runs_per_lane, ref.runs_per_lane)
    assert np.array_equal(ours.run_base, ref.run_base)
    assert np.array_equal(ours.run_stride, ref.run_stride)
    assert np.array_equal(ours.run_count, ref.run_count)


def test_encoder_max_count():
    a, _, _ = _dense_world()
    one = x.runs_encode(a, 64, max_count=1)
    assert one.n_runs == a.size and np.all(one.run_count == 1) and np.all(one.run_stride == 0)
    assert np.array_equal(one.run_base, a.reshape(-1))
    seven = x.runs_encode(a, 64, max_count=7)
    assert np.all(seven.run_count <= 7)
    t = oracle.RunTable(seven.runs_per_lane, seven.run_base, seven.run_stride, seven.run_count, a.shape[1])
    assert np.array_equal(oracle.runs_decode(t), a)


def _table(rpl, base, stride, count, n_blocks, seg=64):
    return x.RunTable(np.array(rpl, np.uint32), np.array(base, np.uint64), np.array(stride, np.int64),
                      np.array(count, np.uint32), n_blocks, seg)


def test_validation_accepts_good_tables():
    a, regions, seg = _dense_world()
    t = x.runs_encode(a, seg)
    assert x.runs_validate_status(t, regions, False) == x.OK
    assert x.runs_validate_status(x.runs_encode(a, seg, max_count=1), regions, False) == x.OK
    d = dg.kv_dst_addrs(40, 6, seg, 1 << 36, 3 * seg)
    assert x.runs_validate_status(x.runs_encode(d, seg), [(1 << 36, 40 * 6 * 3 * seg)], True) == x.OK


def test_validation_rejects_each_rule():
    R = [(0x10000, 0x10000)]
    ok = _table([1, 2], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 2, 2], 4)
    assert x.runs_validate_status(ok, R, True) == x.OK
    cases = [
        (x.E_INVAL, _table([1, 2], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 2, 2], 4, seg=0), R),
        (x.E_INVAL, _table([1, 2], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 2, 2], 4, seg=40), R),
        (x.E_INVAL, ok, [(2**64 - 16, 32)]),                                          # region wraps
        (x.E_UNSUPPORTED, _table([1, 2], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 2, 2], 4,
                                 seg=2 << 20), R),                                    # 2 MiB segments
        (x.E_TABLE, _table([1, 1], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 2, 2], 4), R),  # sum
        (x.E_TABLE, _table([1, 2], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 0, 4], 4), R),  # zero count
        (x.E_TABLE, _table([1, 2], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 2, 1], 4), R),  # short lane
        (x.E_TABLE, _table([1, 2], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 3, 2], 4), R),  # long lane
        (x.E_RANGE, _table([1, 2], [0x10008, 0x10400, 0x10800], [64, 64, 64], [4, 2, 2], 4), R),  # base align
        (x.E_RANGE, _table([1, 2], [0x10000, 0x10400, 0x10800], [72, 64, 64], [4, 2, 2], 4), R),  # stride align
        (x.E_RANGE, _table([1, 2], [0x10000, 0x1FFC0, 0x10800], [64, 64, 64], [4, 2, 2], 4), R),  # escapes
        (x.E_RANGE, _table([1, 2], [0x10000, 0x10400, 0x10000], [64, 64, -64], [4, 2, 2], 4), R),  # below
        (x.E_RANGE, _table([1, 2], [0x10000, 2**64 - 64, 0x10800], [64, 64, 64], [4, 2, 2], 4), R),  # wraps
        (x.E_RANGE, _table([1, 2], [0x10000, 0x10400, 0x10800], [2**62, 64, 64], [4, 2, 2], 4), R),  # mul ovf
        (x.E_RANGE, _table([1, 2], [0x10000, 0x107C0, 0x10900], [64, 64, 64], [4, 2, 2], 4),
         [(0x10000, 0x800), (0x10800, 0x800)]),                      # a run crosses two regions' seam
    ]
    for code, t, regions in cases:
        assert x.runs_validate_status(t, regions, False) == code, (code, t)
    # overlapping destination segments: lane 1's second run lands on lane 0's block 1
    ov = _table([1, 2], [0x10000, 0x10400, 0x10040], [64, 64, 64], [4, 2, 2], 4)
    assert x.runs_validate_status(ov, R, False) == x.OK
    assert x.runs_validate_status(ov, R, True) == x.E_OVERLAP
    # partial overlap (32 B) also refused; exactly adjacent segments accepted
    ov2 = _table([1, 1], [0x10000, 0x10020], [128, 128], [4, 4], 4)
    assert x.runs_validate_status(ov2, R, True) == x.E_OVERLAP
    adj = _table([1, 1], [0x10000, 0x10040], [128, 128], [4, 4], 4)
    assert x.runs_validate_status(adj, R, True) == x.OK


def test_prepare_checks_before_any_copy():
    R = [(0x10000, 0x10000)]
    bad = _table([1, 1], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 2, 2], 4)
    st, _ = x.runs_prepare_status(bad, R, False, 0x1000, 1 << 20)
    assert st == x.E_TABLE
    good = _table([1, 2], [0x10000, 0x10400, 0x10800], [64, 64, 64], [4, 2, 2], 4)
    need = x.runs_plan_bytes(good)
    assert need > 0 and need % 16 == 0
    st, _ = x.runs_prepare_status(good, R, False, 0x1000, need - 16)      # too small
    assert st == x.E_INVAL
    st, _ = x.runs_prepare_status(good, R, False, 0x1008, need)           # misaligned
    assert st == x.E_INVAL
    st, _ = x.runs_prepare_status(good, R, False, 0, need)                # NULL
    assert st == x.E_INVAL


def test_gather_scatter_refuse_foreign_plans():
    p = x.RunsPlan()
    assert x.gather_runs_raw(p, 0x1000, 1 << 20, stream=S0) == x.E_INVAL
    assert x.scatter_runs_raw(0x1000, 1 << 20, p, stream=S0) == x.E_INVAL


def test_plan_bytes_dense_config():
    a = dg.kv_src_addrs(dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES, [1 << 40, (1 << 40) + (1 << 33)])
    t = x.runs_encode(a, dg.SEG_BYTES)
    nb = x.runs_plan_bytes(t)
    # 576 runs * 20 B plus a tile index of 576 lanes * 33 entries * 4 B
    assert nb < 128 * 1024


def test_launch_size_limits():
    """Requests whose one launch would need more than 2^24 - 1 workgroups of
    256 threads (the dispatch's 32-bit work-item count) are refused on the
    host, before any device call."""
    big = 1 << 40
    max_stream = ((1 << 24) - 1) * 2048
    # pack: two 2^34-element chunks in one call
    assert x.pack_bf16_raw(0x100000, 1 << 36, big, 1 << 36, 1 << 35, 0, 2, stream=S0) == x.E_UNSUPPORTED
    assert x.combine2_raw(0x100000, big, max_stream + 4, 2 * big, 0, stream=S0) == x.E_UNSUPPORTED
    rows = 1 << 23
    s0 = x.shard(0x100000, 1024, rows, 512, 0)
    s1 = x.shard(0x100000 + 1024, 1024, rows, 512, 512)
    assert x.argmax_merge_raw(s0, s1, 0, big, 2 * big, 1 << 30, stream=S0) == x.E_UNSUPPORTED
    # gather: one lane of 2^25 blocks of 4 KiB (2^24 tiles of 2 blocks)
    t = _table([1], [big], [4096], [1 << 25], 1 << 25, seg=4096)
    st, _ = x.runs_prepare_status(t, [(big, 1 << 37)], False, 0x1000, 1 << 30)
    assert st == x.E_UNSUPPORTED
    # descriptors: 4 KiB units paired in tiles of 2 x 288, one workgroup per pair: the largest read that
    # fits 2^24 - 1 workgroups is 58,254 tiles of 576 units
    top = 58254 * 576 * 4096
    d = np.array([(big, 0, top + 4096)], x.DESC)                         # one unit more: a 58,255th tile
    st, _ = x.descs_prepare_status(d, 1 << 38, [(big, 1 << 38)], 0x1000, 1 << 20)
    assert st == x.E_UNSUPPORTED
    d = np.array([(big, 0, top)], x.DESC)
    st, _ = x.descs_prepare_status(d, 1 << 38, [(big, 1 << 38)], 0, 0)
    assert st == x.E_INVAL                                              # accepted up to the missing device buffer


def test_setup_scratch_failure_is_a_status():
    """A descriptor count whose host scratch cannot exist (2^60 entries of 16
    bytes is past what a vector may hold) comes back as XFER_E_HOST_MEMORY,
    before any descriptor is read; no C++ exception reaches the caller."""
    d = np.zeros(1, x.DESC)
    plan = x.DescsPlan()
    st = x.lib().xfer_descs_prepare(d.ctypes.data, 1 << 60, 1 << 20, None, 0, None, 0, ctypes.byref(plan))
    assert st == x.E_HOST_MEMORY
    assert x.status_str(st) != "unknown status"
