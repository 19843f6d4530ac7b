"""Seeded random sweeps of the copy and pack paths against the CPU oracle,
byte for byte, with guard bytes after every output:

- run-table gather and scatter over segment sizes from 16 B to 256 KiB
  (split and unsplit, powers of two and not), four layout classes and
  random run-length caps;
- paged copies with random page lengths, strides, offsets and lists;
- descriptor copies with random sizes, sources and slab gaps;
- pack over random sizes, chunk sizes, ring slots and chunk ranges.

Case shapes are drawn by numpy's seeded generator (test scaffolding); the
data come from the shared seeded generators."""
import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, say, up, zeros

pytestmark = pytest.mark.gpu

GUARD = 256
SEGS = [16, 32, 48, 96, 4096, 4112, 8192, 8208, 16384, 32768, 131072, 262144]


def _otable(t: x.RunTable) -> oracle.RunTable:
    return oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks)


def _addrs(rng, L, B, seg, base, slots, kind):
    perm = rng.permutation(slots)
    a = np.empty((L, B), np.uint64)
    for l in range(L):
        for b in range(B):
            if kind == 0:
                s = b * L + l
            elif kind == 1:
                s = l * B + b
            elif kind == 2:
                s = int(perm[l * B + b])
            else:
                s = int(rng.integers(slots))
            a[l, b] = base + s * seg
    return a


@pytest.mark.parametrize("case", range(36))
def test_runs_sweep(case):
    rng = np.random.default_rng(7000 + case)
    seg = SEGS[case % len(SEGS)]
    cap = max(1, (48 << 20) // seg)
    L = int(rng.integers(1, 24))
    B = int(rng.integers(1, max(2, min(40, cap // L))))
    kind = int(rng.integers(4))
    slots = L * B + int(rng.integers(4))
    say("sweep runs", case, "seg", seg, "L", L, "B", B, "kind", kind)
    src = zeros(slots * seg)
    host = dg.random_bytes(slots * seg, 9000 + case)
    src.copy_(torch.from_numpy(host))
    addrs = _addrs(rng, L, B, seg, src.data_ptr(), slots, kind)
    t = x.runs_encode(addrs, seg, max_count=int(rng.integers(0, 5)))
    buf = zeros(max(16, x.runs_plan_bytes(t)))
    plan = x.runs_prepare(t, [(src.data_ptr(), src.numel())], False, buf)
    n = L * B * seg
    staging = filled(n + GUARD, 0x3C)
    x.gather_runs_raw(plan, staging.data_ptr(), n)
    want = oracle.gather(_otable(t), seg, [(src.data_ptr(), host)])
    got = down(staging)
    assert np.array_equal(got[:n], want)
    assert np.all(got[n:] == 0x3C)
    # scatter the oracle's staging to a permutation of destination slots
    dst = filled(slots * seg + GUARD, 0xA5)
    dt = x.runs_encode(_addrs(rng, L, B, seg, dst.data_ptr(), slots, 2), seg, max_count=int(rng.integers(0, 5)))
    dbuf = zeros(max(16, x.runs_plan_bytes(dt)))
    dplan = x.runs_prepare(dt, [(dst.data_ptr(), slots * seg)], True, dbuf)
    staged = up(want)
    assert x.scatter_runs_raw(staged.data_ptr(), n, dplan) == x.OK
    dwant = np.full(slots * seg + GUARD, 0xA5, np.uint8)
    oracle.scatter(_otable(dt), seg, [(dst.data_ptr(), dwant[:slots * seg])], want)
    assert np.array_equal(down(dst), dwant)


@pytest.mark.parametrize("case", range(30))
def test_pages_sweep(case):
    rng = np.random.default_rng(8000 + case)
    page_len = 16 * int(rng.integers(1, 1300))
    n = int(rng.integers(0, 200))
    stride = page_len + 16 * int(rng.integers(0, 4))
    s_off, d_off = 16 * int(rng.integers(0, 3)), 16 * int(rng.integers(0, 3))
    slots = n + 1 + int(rng.integers(0, 8))
    rb = s_off + slots * stride + 16
    say("sweep pages", case, "page_len", page_len, "n", n)
    si = rng.integers(0, slots, n).astype(np.uint32)
    di = rng.permutation(slots)[:n].astype(np.uint32)
    src = zeros(rb)
    host = dg.random_bytes(rb, 9500 + case)
    src.copy_(torch.from_numpy(host))
    dst = filled(d_off + slots * stride + 16 + GUARD, 0x6B)
    drb = d_off + slots * stride + 16
    buf = zeros(max(16, x.pages_plan_bytes(n)))
    plan = x.pages_prepare(page_len, (src.data_ptr(), rb), si, stride, s_off, (dst.data_ptr(), drb), di, stride,
                           d_off, buf)
    x.paged_copy(plan)
    want = np.full(drb + GUARD, 0x6B, np.uint8)
    oracle.paged_copy(page_len, host, si, stride, s_off, want[:drb], di, stride, d_off)
    assert np.array_equal(down(dst), want)


@pytest.mark.parametrize("case", range(20))
def test_descs_sweep(case):
    rng = np.random.default_rng(8500 + case)
    n_d = int(rng.integers(1, 40))
    sizes = 16 * rng.integers(1, 20000, n_d)
    rb = int(sizes.max()) * 2 + 4096
    src = zeros(rb)
    host = dg.random_bytes(rb, 9800 + case)
    src.copy_(torch.from_numpy(host))
    descs = np.zeros(n_d, x.DESC)
    off = 0
    for k in range(n_d):
        descs["src"][k] = src.data_ptr() + 16 * int(rng.integers(0, (rb - int(sizes[k])) // 16))
        off += 16 * int(rng.integers(0, 3))
        descs["dst_off"][k] = off
        descs["bytes"][k] = int(sizes[k])
        off += int(sizes[k])
    order = rng.permutation(n_d)  # the list need not be in slab order
    descs = descs[order]
    slab_bytes = off
    say("sweep descs", case, "n", n_d, "slab", slab_bytes)
    slab = filled(slab_bytes + GUARD, 0x2D)
    dbuf = zeros(max(16, x.descs_plan_bytes(n_d)))
    plan = x.descs_prepare(descs, slab_bytes, [(src.data_ptr(), rb)], dbuf)
    x.copy_descs(plan, slab)
    want = np.full(slab_bytes + GUARD, 0x2D, np.uint8)
    oracle.copy_descs(descs, [(src.data_ptr(), host)], want[:slab_bytes])
    assert np.array_equal(down(slab), want)


@pytest.mark.parametrize("case", range(30))
def test_pack_sweep(case):
    rng = np.random.default_rng(8800 + case)
    n = int(rng.integers(1, 60000))
    chunk = 16 * int(rng.integers(1, 64))
    ce = chunk // 2
    R = int(rng.integers(1, 5))
    n_chunks = -(-n // ce)
    b = int(rng.integers(0, n_chunks))
    e = min(n_chunks, b + int(rng.integers(1, R + 1)))
    say("sweep pack", case, "n", n, "chunk", chunk, "R", R, "range", b, e)
    a = dg.random_u64((n + 1) // 2, 9900 + case).view(np.float32)[:n].copy()
    src = up(a)
    ring = filled(R * chunk + GUARD, 0xEE)
    assert x.pack_bf16_raw(src.data_ptr(), n, ring.data_ptr(), R * chunk, chunk, b, e) == x.OK
    want = np.full((R * chunk + GUARD) // 2, 0xEEEE, np.uint16)
    oracle.pack(a, R * ce, ce, b, e, ring=want[:R * ce])
    assert np.array_equal(down(ring, np.uint16), want)
