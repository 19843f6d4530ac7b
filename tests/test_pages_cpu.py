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
