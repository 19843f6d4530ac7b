"""GPU parity of the paged copy (xfer_pages_prepare + xfer_paged_copy, the
TransferEngine Pages format) against the CPU oracle, byte for byte: seeded
page permutations over page lengths from 16 B to 64 KiB (units of 4 KiB
split and unsplit), offsets and gapped strides, with the untouched
destination bytes checked; and the full paged K/V set gathered by pages
(two lists of 288,000 pages, one per region) and scattered by pages into the
12 KiB slot-stride destination."""
import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, say, up, zeros

pytestmark = pytest.mark.gpu


def _copy(page_len, src, si, ss, so, dst, di, ds, do):
    """Plan and run one paged copy between two uint8 CUDA tensors."""
    dev = zeros(max(16, x.pages_plan_bytes(len(si))))
    plan = x.pages_prepare(page_len, (src.data_ptr(), src.numel()), si, ss, so, (dst.data_ptr(), dst.numel()), di,
                           ds, do, dev)
    x.paged_copy(plan)
    torch.cuda.synchronize()


@pytest.mark.parametrize("page_len", [16, 48, 4096, 4112, 8192, 12288, 65536])
@pytest.mark.parametrize("n", [1, 2, 3, 33, 257])
def test_permutations(page_len, n):
    say("paged perm", page_len, n)
    ss, so = page_len + 32, 64            # gapped source pages after a 64-byte offset
    ds, do = 2 * page_len, 16             # every other destination page slot
    src_bytes = so + (n + 3) * ss
    dst_bytes = do + (n + 3) * ds
    src_h = dg.random_u64(src_bytes // 8 + 1, page_len * 31 + n).view(np.uint8)[:src_bytes].copy()
    si = dg.permutation(n + 3, n * 7 + 1)[:n]
    di = dg.permutation(n + 3, n * 7 + 2)[:n]
    src = up(src_h)
    dst = filled(dst_bytes, 0x3C)
    _copy(page_len, src, si, ss, so, dst, di, ds, do)
    want = np.full(dst_bytes, 0x3C, np.uint8)
    oracle.paged_copy(page_len, src_h, si, ss, so, want, di, ds, do)
    assert np.array_equal(down(dst), want)


def _kv(B, S, seg, shuffle):
    rb = dg.region_bytes_for(B, S, seg)
    regs = [zeros(rb) for _ in range(2)]
    bases = [r.data_ptr() for r in regs]
    pos = dg.permutation(B, shuffle) if shuffle is not None else np.arange(B, dtype=np.uint32)
    addrs = dg.kv_src_addrs(B, S, seg, bases, pos=pos)
    hosts = []
    for i, r in enumerate(regs):
        h = np.empty(rb, np.uint8)
        dg.fill_region(h, bases[i], addrs, seg, 4000 + i)
        r.copy_(torch.from_numpy(h))
        hosts.append(h)
    return regs, hosts, addrs, pos


def _kv_lists(B, S, pos, region):
    """Region pages of the region's lanes and their block-major staging pages."""
    L = 2 * S
    b = np.repeat(np.arange(B, dtype=np.int64), S)
    j = np.tile(np.arange(S, dtype=np.int64), B)
    src = pos.astype(np.int64)[b] * S + j
    dst = b * L + region * S + j
    return src.astype(np.uint32), dst.astype(np.uint32)


@pytest.mark.parametrize("B,S,seg,shuffle", [(6, 4, 64, None), (40, 6, 4096, 3), (1000, dg.N_SLOTS, 4096, None),
                                             (1000, dg.N_SLOTS, 4096, 9)])
def test_kv_gather_and_scatter_by_pages(B, S, seg, shuffle):
    say("paged kv", B, S, seg, shuffle)
    regs, hosts, addrs, pos = _kv(B, S, seg, shuffle)
    L = 2 * S
    t = x.runs_encode(addrs, seg)
    want = oracle.gather(oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks), seg,
                         [(r.data_ptr(), h) for r, h in zip(regs, hosts)])
    staging = filled(L * B * seg, 0xEE)
    for r in range(2):
        si, di = _kv_lists(B, S, pos, r)
        _copy(seg, regs[r], si, seg, 0, staging, di, seg, 0)
    got = down(staging)
    assert np.array_equal(got, want)
    del got, regs, hosts
    # scatter: staging page b * L + l -> destination slot (b * S + l / 2) * 3 + l % 2 (gap page per slot)
    dst = filled(B * S * 3 * seg, 0xA5)
    k = np.arange(B * L, dtype=np.int64)
    di = ((k // L) * S + (k % L) // 2) * 3 + (k % L) % 2
    si = k.astype(np.uint32)
    _copy(seg, staging, si, seg, 0, dst, di.astype(np.uint32), seg, 0)
    dwant = np.full(dst.numel(), 0xA5, np.uint8)
    oracle.paged_copy(seg, want, si, seg, 0, dwant, di.astype(np.uint32), seg, 0)
    assert np.array_equal(down(dst), dwant)
    del dst, staging
    torch.cuda.empty_cache()


def test_refused_prepare_writes_nothing():
    src = filled(1 << 16, 0x11)
    dst = filled(1 << 16, 0x22)
    dev = zeros(256)
    st, _ = x.pages_prepare_status(4096, (src.data_ptr(), src.numel()), [0, 16], 4096, 0,
                                   (dst.data_ptr(), dst.numel()), [0, 1], 4096, 0, dev.data_ptr(), 256)
    assert st == x.E_RANGE
    st, _ = x.pages_prepare_status(4096, (src.data_ptr(), src.numel()), [0, 1], 4096, 0,
                                   (dst.data_ptr(), dst.numel()), [1, 1], 4096, 0, dev.data_ptr(), 256)
    assert st == x.E_OVERLAP
    assert np.all(down(dst) == 0x22) and np.all(down(dev) == 0)


@pytest.mark.parametrize("page_len,n", [(4096, 300), (272, 41), (65536, 9)])
def test_copy_within_one_buffer(page_len, n):
    """Source and destination pages in one buffer (a compaction: scattered
    pages moved into a free area of the same allocation).  The prepare
    accepts it because no destination page shares a byte with a source page;
    every moved page, and every byte outside the destination pages, matches
    the oracle run on the same single image."""
    slots = 3 * n + 5
    nbytes = 32 + slots * page_len
    h = dg.random_u64(nbytes // 8 + 1, page_len + n).view(np.uint8)[:nbytes].copy()
    perm = dg.permutation(slots, 7 * n + page_len)
    si, di = perm[:n], perm[n:2 * n]
    buf = up(h)
    say("paged copy within one buffer", page_len, n)
    dev = zeros(max(16, x.pages_plan_bytes(n)))
    region = (buf.data_ptr(), buf.numel())
    plan = x.pages_prepare(page_len, region, si, page_len, 32, region, di, page_len, 32, dev)
    x.paged_copy(plan)
    want = h.copy()
    oracle.paged_copy(page_len, h, si, page_len, 32, want, di, page_len, 32)
    assert np.array_equal(down(buf), want)
    # a destination list that reuses one source page is refused, and nothing is written
    bad = di.copy()
    bad[n // 2] = si[0]
    st, _ = x.pages_prepare_status(page_len, region, si, page_len, 32, region, bad, page_len, 32, dev.data_ptr(),
                                   dev.numel())
    assert st == x.E_OVERLAP
    assert np.array_equal(down(buf), want)
