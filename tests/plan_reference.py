"""A test-side reading of the coalesced-fetch planning of the run-encoded
transfer page (pegaflow PR 350, "What this PR does", steps 2-5, and "READ
splitting"), written from the expanded segment list.  It shares nothing with
oracle/oracle.c or the library's planner, and is organised differently from
both: they sweep one (region, base)-sorted list of runs and grow a group
while the next run passes the merge test; here the runs are first split into
classes that may share a group at all, and each class is cut into groups
from its own segments.

The page's grouping, restated:
  - runs are bucketed by the region (NUMA node) that holds them;
  - runs that share a group cover the same blocks (same first block and
    count) with the same stride (a one-block run has none);
  - inside a class, a group is a chain of runs whose first segments lie back
    to back (each starts where the previous one ends: "base-adjacent"), so
    at every block the group's segments form one contiguous chunk;
  - a chain may grow only while the chunk still fits the stride (its blocks'
    chunks must not overlap), so chains are cut, from the lowest address up,
    into pieces of at most floor(|stride| / seg) runs (no limit for
    one-block runs);
  - a group whose blocks' chunks are back to back (|stride| == chunk, or one
    block) is dense and read as one range; any other is read block by block;
  - every read is cut into pieces of at most max_read bytes, in address
    order; groups take slab space in the order of their first run in
    (region, base, table position) order, and a dense group mirrors its range,
    a per-block group stores its chunks block after block.
Only valid for tables whose source segments are pairwise disjoint (then the
classes can be chained independently of one another); callers assert it.
"""
from __future__ import annotations

import numpy as np


def expand(runs_per_lane, run_base, run_stride, run_count, n_blocks: int):
    """Per segment (lane-major, block-minor): address and the run covering it."""
    n_lanes = len(runs_per_lane)
    addr = np.zeros((n_lanes, n_blocks), np.uint64)
    run_of = np.zeros((n_lanes, n_blocks), np.int64)
    r = 0
    for lane in range(n_lanes):
        b = 0
        for _ in range(int(runs_per_lane[lane])):
            c = int(run_count[r])
            st = int(run_stride[r]) if c > 1 else 0
            for i in range(c):
                addr[lane, b + i] = (int(run_base[r]) + i * st) % (1 << 64)
                run_of[lane, b + i] = r
            b += c
            r += 1
        assert b == n_blocks
    return addr, run_of


def segments_disjoint(addr: np.ndarray, seg: int) -> bool:
    a = np.sort(addr.reshape(-1))
    return bool(np.all(a[1:] - a[:-1] >= np.uint64(seg))) if a.size > 1 else True


def plan(runs_per_lane, run_base, run_stride, run_count, n_blocks: int, seg: int, regions, max_read: int):
    """Returns (descs as a list of (src, dst_off, bytes), slab_bytes,
    local offsets uint64[n_lanes, n_blocks])."""
    n_lanes = len(runs_per_lane)
    n_runs = len(run_base)
    addr, run_of = expand(runs_per_lane, run_base, run_stride, run_count, n_blocks)
    assert segments_disjoint(addr, seg), "the reference planner needs disjoint source segments"
    # per run: lane, first block, count, stride, base, region (from its segments)
    lane_of = np.repeat(np.arange(n_lanes), np.asarray(runs_per_lane, np.int64))
    first = np.zeros(n_runs, np.int64)
    r = 0
    for lane in range(n_lanes):
        b = 0
        for _ in range(int(runs_per_lane[lane])):
            first[r] = b
            b += int(run_count[r])
            r += 1
    count = np.asarray(run_count, np.int64)
    stride = np.where(count > 1, np.asarray(run_stride, np.int64), 0)
    base = np.asarray(run_base, np.uint64)
    region = np.full(n_runs, -1, np.int64)
    for k in range(n_runs):
        segs = addr[lane_of[k], first[k]:first[k] + count[k]]
        lo, hi = int(segs.min()), int(segs.max()) + seg
        for g, (rb, rn) in enumerate(regions):
            if rb <= lo and hi <= rb + rn:
                region[k] = g
                break
        assert region[k] >= 0, "a run outside every region"

    # classes of runs that may share a group
    classes: dict = {}
    for k in range(n_runs):
        classes.setdefault((int(region[k]), int(first[k]), int(count[k]), int(stride[k])), []).append(k)
    groups = []  # lists of run ids, lowest base first
    for (g, b0, c, st), members in classes.items():
        members.sort(key=lambda k: (int(base[k]), k))
        cap = abs(st) // seg if c > 1 else None
        chain = [members[0]]
        for k in members[1:]:
            if int(base[k]) == int(base[chain[-1]]) + seg:
                chain.append(k)
            else:
                groups += _cut(chain, cap)
                chain = [k]
        groups += _cut(chain, cap)
    groups.sort(key=lambda grp: (int(region[grp[0]]), int(base[grp[0]]), grp[0]))

    descs, local, slab = [], np.zeros((n_lanes, n_blocks), np.uint64), 0
    for grp in groups:
        f = grp[0]
        c, st = int(count[f]), int(stride[f])
        chunk = len(grp) * seg
        block_lo = [int(addr[lane_of[f], first[f] + i]) for i in range(c)]  # chunk start per block
        dense = c == 1 or abs(st) == chunk
        if dense:
            lo = min(block_lo)
            span = chunk if c == 1 else c * abs(st)
            descs += _split(lo, slab, span, max_read)
            for k in grp:
                for i in range(c):
                    local[lane_of[k], first[k] + i] = slab + int(addr[lane_of[k], first[k] + i]) - lo
            slab += span
        else:
            for i in range(c):
                descs += _split(block_lo[i], slab + i * chunk, chunk, max_read)
                for k in grp:
                    local[lane_of[k], first[k] + i] = slab + i * chunk + int(addr[lane_of[k], first[k] + i]) - block_lo[i]
            slab += c * chunk
    return descs, slab, local


def _cut(chain, cap):
    if cap is None:
        return [chain]
    cap = max(cap, 1)
    return [chain[i:i + cap] for i in range(0, len(chain), cap)]


def _split(src, dst, n, max_read):
    return [(src + o, dst + o, min(max_read, n - o)) for o in range(0, n, max_read)]


def reads_only_segments(descs, addr: np.ndarray, seg: int) -> bool:
    """Every byte the descriptors read belongs to a segment, no byte is read
    twice, and every segment is read (disjoint segments): the reads tile the
    segments exactly.  Pieces of one split read are joined first."""
    a = np.sort(addr.reshape(-1).astype(np.uint64))
    spans = sorted((int(src), int(src) + int(n)) for src, _, n in descs)
    merged = []
    for s0, e0 in spans:
        if merged and s0 < merged[-1][1]:
            return False                      # a byte read twice
        if merged and s0 == merged[-1][1]:
            merged[-1][1] = e0
        else:
            merged.append([s0, e0])
    total = 0
    for s0, e0 in merged:
        if (e0 - s0) % seg:
            return False
        k = (e0 - s0) // seg
        i0 = int(np.searchsorted(a, np.uint64(s0)))
        want = np.uint64(s0) + np.uint64(seg) * np.arange(k, dtype=np.uint64)
        if i0 + k > a.size or not np.array_equal(a[i0:i0 + k], want):
            return False
        total += k
    return total == a.size
