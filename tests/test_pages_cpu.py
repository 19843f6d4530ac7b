"""The Pages{indices, stride, offset} address format (TransferEngine paged
writes), on the CPU: the oracle pinned against the run-table gather (an
independently pinned formulation), a permutation round trip, a worked
example with literal byte positions, and its refusals; then the library's
host-side checks (no GPU needed)."""
import numpy as np
import pytest

import bf16_wire_all_amd as x
import datagen as dg
import oracle


def _kv_world(B, S, seg, shuffle):
    rb = dg.region_bytes_for(B, S, seg)
    bases = [0x100000, 0x100000 + rb + 4096]
    pos = dg.permutation(B, shuffle) if shuffle is not None else np.arange(B, dtype=np.uint32)
    a = dg.kv_src_addrs(B, S, seg, bases, pos=pos)
    hosts = []
    for i, b in enumerate(bases):
        h = np.empty(rb, np.uint8)
        dg.fill_region(h, b, a, seg, 70 + i)
        hosts.append(h)
    return a, bases, hosts, pos


def _kv_pages(B, S, pos, region):
    """Source page indices (inside the region) and staging page indices of the
    region's lanes, block-major as the run-table gather stages them."""
    L, half = 2 * S, S  # lanes per region: 2 * (S / 2)
    src, dst = [], []
    for b in range(B):
        for j in range(half):
            l = region * half + j
            src.append(int(pos[b]) * half + j)
            dst.append(b * L + l)
    return np.array(src, np.uint32), np.array(dst, np.uint32)


@pytest.mark.parametrize("B,S,seg,shuffle", [(6, 4, 64, None), (12, 6, 48, 5), (9, 2, 4096, 7)])
def test_paged_gather_equals_run_gather(B, S, seg, shuffle):
    a, bases, hosts, pos = _kv_world(B, S, seg, shuffle)
    t = x.runs_encode(a, seg)
    want = oracle.gather(oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks),
                         seg, list(zip(bases, hosts)))
    got = np.full(want.size, 0xEE, np.uint8)
    for r in range(2):
        si, di = _kv_pages(B, S, pos, r)
        oracle.paged_copy(seg, hosts[r], si, seg, 0, got, di, seg, 0)
    assert np.array_equal(got, want)


def test_permutation_round_trip_leaves_the_rest_untouched():
    n, page = 37, 80
    src = dg.random_u64(n * page // 8 + 1, 9).view(np.uint8)[: n * page].copy()
    perm = dg.permutation(n, 11)
    ident = np.arange(n, dtype=np.uint32)
    tmp = np.full(2 * n * page + 48, 0x77, np.uint8)
    # out: page k -> slot perm[k] of a stride-2*page layout starting at byte 48
    oracle.paged_copy(page, src, ident, page, 0, tmp, perm, 2 * page, 48)
    back = np.zeros_like(src)
    oracle.paged_copy(page, tmp, perm, 2 * page, 48, back, ident, page, 0)
    assert np.array_equal(back, src)
    gaps = np.ones(tmp.size, bool)
    for k in range(n):
        lo = 48 + int(perm[k]) * 2 * page
        gaps[lo:lo + page] = False
    assert np.all(tmp[gaps] == 0x77)


def test_worked_example():
    src = np.arange(64, dtype=np.uint8)
    dst = np.full(80, 0xFF, np.uint8)
    # pages of 16 bytes: source pages 3 and 0 (stride 16) go to destination pages 0 and 1 (stride 32, offset 16)
    oracle.paged_copy(16, src, [3, 0], 16, 0, dst, [0, 1], 32, 16)
    want = np.full(80, 0xFF, np.uint8)
    want[16:32] = np.arange(48, 64)
    want[48:64] = np.arange(0, 16)
    assert np.array_equal(dst, want)


def test_oracle_refusals():
    src = np.zeros(64, np.uint8)
    dst = np.zeros(64, np.uint8)
    with pytest.raises(oracle.OracleError) as e:
        oracle.paged_copy(16, src, [4], 16, 0, dst, [0], 16, 0)        # source page past the end
    assert e.value.code == oracle.ERANGE
    with pytest.raises(oracle.OracleError) as e:
        oracle.paged_copy(16, src, [0], 16, 0, dst, [0xFFFFFFFF], 1 << 40, 0)  # offset arithmetic overflows
    assert e.value.code == oracle.ERANGE
    with pytest.raises(oracle.OracleError) as e:
        oracle.paged_copy(16, src, [0, 1], 16, 0, dst, [0, 1], 8, 0)  # destination pages overlap
    assert e.value.code == oracle.EARG
    with pytest.raises(oracle.OracleError):
        oracle.paged_copy(0, src, [0], 16, 0, dst, [0], 16, 0)
    oracle.paged_copy(16, src, [], 16, 0, dst, [], 16, 0)              # no pages: nothing to do


def test_scatter_by_pages_places_every_page():
    """Staging pages (block-major) to a slot-major destination with a gap page
    per slot, expressed as Pages: every page lands at its slot, gaps keep
    their fill."""
    B, S, seg = 7, 4, 64
    L = 2 * S
    staging = dg.random_u64(B * L * seg // 8, 13).view(np.uint8).copy()
    dst = np.full(B * S * 3 * seg, 0xA5, np.uint8)
    si = np.arange(B * L, dtype=np.uint32)
    di = np.array([(b * S + l // 2) * 3 + l % 2 for b in range(B) for l in range(L)], np.uint32)
    oracle.paged_copy(seg, staging, si, seg, 0, dst, di, seg, 0)
    for b in range(B):
        for s in range(S):
            for kv in range(2):
                page = ((b * S + s) * 3 + kv) * seg
                k = b * L + 2 * s + kv
                assert np.array_equal(dst[page:page + seg], staging[k * seg:(k + 1) * seg])
            gap = ((b * S + s) * 3 + 2) * seg
            assert np.all(dst[gap:gap + seg] == 0xA5)


# ------------------------------------------------------ library host checks

SRC = (0x10000000, 1 << 20)
DST = (0x20000000, 1 << 20)


def _prep(page_len=4096, si=(0, 1), ss=4096, so=0, di=(0, 1), ds=4096, do=0, src=SRC, dst=DST, dev=0, dev_bytes=0):
    st, _ = x.pages_prepare_status(page_len, src, si, ss, so, dst, di, ds, do, dev, dev_bytes)
    return st


def test_library_checks_in_order():
    assert _prep(page_len=0) == x.E_INVAL
    assert _prep(page_len=24) == x.E_INVAL                                # not a multiple of 16
    assert _prep(ss=4104) == x.E_INVAL                                    # misaligned stride
    assert _prep(do=8) == x.E_INVAL                                       # misaligned offset
    assert _prep(src=(0x10000008, 1 << 20)) == x.E_INVAL                  # misaligned region
    # overlapping regions (or one region) are allowed as long as no destination page touches a source page
    assert _prep(dst=(0x10080000, 1 << 20)) == x.E_INVAL                  # disjoint pages: then no dev
    assert _prep(dst=SRC, di=(2, 3)) == x.E_INVAL                         # one region, disjoint pages: no dev
    assert _prep(dst=SRC, di=(1, 2)) == x.E_OVERLAP                       # page 1 is read and written
    assert _prep(dst=SRC, di=(2, 3), ds=2048) == x.E_OVERLAP              # destination bytes [4096, 8192) in a source page
    assert _prep(dst=SRC, si=(4, 5), di=(0, 1), do=64) == x.E_INVAL       # ends 64 bytes short of page 4: no dev
    assert _prep(dst=SRC, si=(4, 5), di=(3, 4), do=16) == x.E_OVERLAP     # 16 bytes into source page 4
    assert _prep(si=(0, 256)) == x.E_RANGE                                # source page past the end
    assert _prep(di=(255, 256)) == x.E_RANGE                              # destination page past the end
    assert _prep(si=(0, 0xFFFFFFFF), ss=1 << 40) == x.E_RANGE             # offset arithmetic overflows
    assert _prep(di=(0, 1), ds=2048) == x.E_OVERLAP                       # destination pages overlap
    assert _prep(di=(3, 3)) == x.E_OVERLAP                                # the same page twice
    assert _prep(si=(3, 3)) == x.E_INVAL                                  # same source page twice is fine: then no dev
    assert _prep() == x.E_INVAL                                           # valid lists, no device buffer
    assert _prep(si=(), di=()) == x.OK                                    # no pages: nothing to upload


def test_library_refuses_oversized_launches():
    n = 1 << 21                                                           # 2^21 pages of 64 KiB = 2^25 units
    idx = np.arange(n, dtype=np.uint32)
    big = (1 << 40, 1 << 38)
    assert _prep(page_len=65536, si=idx, ss=65536, di=idx, ds=65536, src=big, dst=(1 << 41, 1 << 38)) == \
        x.E_UNSUPPORTED
    assert _prep(page_len=1 << 28, si=np.arange(1 << 16 | 1, dtype=np.uint32), ss=1 << 28,
                 di=np.arange(1 << 16 | 1, dtype=np.uint32), ds=1 << 28, src=(1 << 44, 1 << 45),
                 dst=(1 << 46, 1 << 45)) == x.E_UNSUPPORTED             # more than 2^32 - 1 units


def test_launch_limit_boundary():
    """Workgroups pair units 576 apart in tiles of 1152 units, 576 workgroups a
    tile: 29127 tiles (33,554,304 units) fit under 2^24 - 1 workgroups, one
    unit more needs a 29128th tile and is refused."""
    n = 262143                                                            # 512 KiB pages: 128 units each
    idx = np.arange(n, dtype=np.uint32)
    assert _prep(page_len=1 << 19, si=idx, ss=1 << 19, di=idx, ds=1 << 19, src=(1 << 40, 1 << 38),
                 dst=(1 << 41, 1 << 38)) == x.E_INVAL                    # accepted; then no device buffer
    n = 33554305 // 5                                                     # 16400-byte pages: 5 units each
    idx = np.arange(n, dtype=np.uint32)
    assert _prep(page_len=16400, si=idx, ss=16400, di=idx, ds=16400, src=(1 << 40, 1 << 38),
                 dst=(1 << 41, 1 << 38)) == x.E_UNSUPPORTED


def test_library_agrees_with_oracle_on_what_is_refused():
    """The same lists, refused or accepted alike by the oracle and the library."""
    cases = [dict(si=(0, 256)), dict(di=(255, 256)), dict(di=(0, 1), ds=2048), dict(si=(0, 1))]
    for c in cases:
        st = _prep(**c)
        src = np.zeros(SRC[1], np.uint8)
        dst = np.zeros(DST[1], np.uint8)
        try:
            oracle.paged_copy(4096, src, c.get("si", (0, 1)), c.get("ss", 4096), 0, dst, c.get("di", (0, 1)),
                              c.get("ds", 4096), 0)
            ok = True
        except oracle.OracleError:
            ok = False
        assert ok == (st == x.E_INVAL), (c, st)   # accepted lists fail only for the missing device buffer


def test_paged_copy_refuses_foreign_plans():
    assert x.lib().xfer_paged_copy(x.ctypes.byref(x.PagesPlan()), None) == x.E_INVAL
