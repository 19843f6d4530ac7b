"""ctypes front end of the CPU oracle (``liboracle.so``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
It shares nothing with the HIP library.  The arithmetic lives in ``oracle.c``;
this module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

OK, EARG, ENAN, ETABLE, ERANGE = 0, -1, -2, -3, -4


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


class Shard(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("ld", ctypes.c_size_t), ("rows", ctypes.c_uint32),
                ("ncols", ctypes.c_uint32), ("col_offset", ctypes.c_uint32)]


class Region(ctypes.Structure):
    _fields_ = [("dev_base", ctypes.c_uint64), ("bytes", ctypes.c_uint64), ("host", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, S, U64, U32, U16, I = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_uint32,
                                  ctypes.c_uint16, ctypes.c_int)
        L.oracle_bf16_rne.argtypes = [U32]
        L.oracle_bf16_rne.restype = U16
        L.oracle_bf16_rne_array.argtypes = [P, P, S]
        L.oracle_pack.argtypes = [P, S, P, S, S, S, S]
        L.oracle_pack.restype = I
        L.oracle_sum2_f32.argtypes = [U16, U16]
        L.oracle_sum2_f32.restype = U32
        L.oracle_combine2.argtypes = [P, P, S, P, I]
        L.oracle_combine2.restype = I
        L.oracle_sum2_f32_f32.argtypes = [U32, U32]
        L.oracle_sum2_f32_f32.restype = U32
        L.oracle_combine2_f32.argtypes = [P, P, S, P, I]
        L.oracle_combine2_f32.restype = I
        L.oracle_argmax_merge.argtypes = [ctypes.POINTER(Shard), ctypes.POINTER(Shard), I, P]
        L.oracle_argmax_merge.restype = I
        L.oracle_runs_encode.argtypes = [P, U32, U32, P, P, P, P, U64, ctypes.POINTER(U64)]
        L.oracle_runs_encode.restype = I
        L.oracle_runs_decode.argtypes = [P, P, P, P, U64, U32, U32, P]
        L.oracle_runs_decode.restype = I
        L.oracle_gather.argtypes = [P, P, P, P, U64, U32, U32, U64, ctypes.POINTER(Region), I, P]
        L.oracle_gather.restype = I
        L.oracle_scatter.argtypes = [P, P, P, P, U64, U32, U32, U64, ctypes.POINTER(Region), I, P]
        L.oracle_scatter.restype = I
        L.oracle_groups_plan.argtypes = [P, P, P, P, U64, U32, U32, U64, P, P, I, U64, P, U64,
                                         ctypes.POINTER(U64), ctypes.POINTER(U64), P]
        L.oracle_groups_plan.restype = I
        L.oracle_copy_descs.argtypes = [P, U64, ctypes.POINTER(Region), I, P, U64]
        L.oracle_copy_descs.restype = I
        L.oracle_paged_copy.argtypes = [U64, ctypes.POINTER(Region), P, U64, U64, ctypes.POINTER(Region), P, U64, U64,
                                        U64]
        L.oracle_paged_copy.restype = I
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise OracleError(rc, what)


# ------------------------------------------------------------ arithmetic

def bf16_rne_scalar(bits: int) -> int:
    return int(lib().oracle_bf16_rne(bits))


def bf16_rne(f32_bits: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(f32_bits).view(np.uint32).reshape(-1)
    out = np.empty(x.size, dtype=np.uint16)
    if x.size:
        lib().oracle_bf16_rne_array(_p(x), _p(out), x.size)
    return out


def pack(src: np.ndarray, ring_elems: int, chunk_elems: int, chunk_begin: int, chunk_end: int,
         ring: np.ndarray | None = None) -> np.ndarray:
    s = np.ascontiguousarray(src, dtype=np.float32).reshape(-1)
    if ring is None:
        ring = np.zeros(ring_elems, dtype=np.uint16)
    assert ring.dtype == np.uint16 and ring.size == ring_elems
    _check(lib().oracle_pack(_p(s), s.size, _p(ring), ring_elems, chunk_elems, chunk_begin, chunk_end),
           "pack")
    return ring


def sum2_f32_scalar(a: int, b: int) -> int:
    return int(lib().oracle_sum2_f32(a, b))


def combine2(a: np.ndarray, b: np.ndarray, mode: int) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.uint16).reshape(-1)
    b = np.ascontiguousarray(b, dtype=np.uint16).reshape(-1)
    assert a.size == b.size
    out = np.empty(a.size, dtype=np.uint32 if mode == 0 else np.uint16)
    _check(lib().oracle_combine2(_p(a), _p(b), a.size, _p(out), mode), "combine2")
    return out


def sum2_f32_f32_scalar(a_bits: int, b_bits: int) -> int:
    return int(lib().oracle_sum2_f32_f32(a_bits, b_bits))


def combine2_f32(a: np.ndarray, b: np.ndarray, mode: int) -> np.ndarray:
    """F32-wire combine: a, b F32 values (or their uint32 bit patterns)."""
    a = np.ascontiguousarray(a).view(np.float32).reshape(-1)
    b = np.ascontiguousarray(b).view(np.float32).reshape(-1)
    assert a.size == b.size
    out = np.empty(a.size, dtype=np.uint32 if mode == 0 else np.uint16)
    _check(lib().oracle_combine2_f32(_p(a), _p(b), a.size, _p(out), mode), "combine2_f32")
    return out


MAX_IDX = np.dtype([("max", "<f4"), ("idx", "<i4")])
TOP2 = np.dtype([("top1", "<f4"), ("top2", "<f4"), ("idx", "<i4"), ("reserved", "<i4")])


def argmax_merge(logits: np.ndarray, split: int, mode: int, ncols1: int | None = None) -> np.ndarray:
    """Both shards are column ranges of one row-major BF16 matrix:
    shard 0 = columns [0, split), shard 1 = columns [split, split + ncols1)."""
    x = np.ascontiguousarray(logits, dtype=np.uint16)
    rows, cols = x.shape
    n1 = cols - split if ncols1 is None else ncols1
    s0 = Shard(x.ctypes.data, cols, rows, split, 0)
    s1 = Shard(x.ctypes.data + 2 * split, cols, rows, n1, split)
    out = np.zeros(rows, dtype=MAX_IDX if mode == 0 else TOP2)
    _check(lib().oracle_argmax_merge(ctypes.byref(s0), ctypes.byref(s1), mode, out.ctypes.data),
           "argmax_merge")
    return out


def argmax_merge_shards(s0: Shard, s1: Shard, mode: int) -> np.ndarray:
    out = np.zeros(s0.rows, dtype=MAX_IDX if mode == 0 else TOP2)
    _check(lib().oracle_argmax_merge(ctypes.byref(s0), ctypes.byref(s1), mode, out.ctypes.data),
           "argmax_merge")
    return out


# ------------------------------------------------------------ run tables

class RunTable:
    """Parallel arrays of a run-encoded address table (lane-major)."""

    def __init__(self, runs_per_lane, run_base, run_stride, run_count, n_blocks: int):
        self.runs_per_lane = np.ascontiguousarray(runs_per_lane, dtype=np.uint32)
        self.run_base = np.ascontiguousarray(run_base, dtype=np.uint64)
        self.run_stride = np.ascontiguousarray(run_stride, dtype=np.int64)
        self.run_count = np.ascontiguousarray(run_count, dtype=np.uint32)
        self.n_blocks = int(n_blocks)

    @property
    def n_lanes(self) -> int:
        return int(self.runs_per_lane.size)

    @property
    def n_runs(self) -> int:
        return int(self.run_base.size)

    def _args(self):
        return (_p(self.runs_per_lane), _p(self.run_base), _p(self.run_stride), _p(self.run_count),
                self.n_runs, self.n_lanes, self.n_blocks)


def runs_encode(addrs: np.ndarray) -> RunTable:
    a = np.ascontiguousarray(addrs, dtype=np.uint64)
    n_lanes, n_blocks = a.shape
    cap = max(1, n_lanes * n_blocks)
    rpl = np.zeros(n_lanes, dtype=np.uint32)
    base = np.zeros(cap, dtype=np.uint64)
    stride = np.zeros(cap, dtype=np.int64)
    count = np.zeros(cap, dtype=np.uint32)
    nr = ctypes.c_uint64(0)
    _check(lib().oracle_runs_encode(_p(a), n_lanes, n_blocks, _p(rpl), _p(base), _p(stride), _p(count),
                                    cap, ctypes.byref(nr)), "runs_encode")
    n = nr.value
    return RunTable(rpl, base[:n].copy(), stride[:n].copy(), count[:n].copy(), n_blocks)


def runs_decode(t: RunTable) -> np.ndarray:
    out = np.zeros((t.n_lanes, t.n_blocks), dtype=np.uint64)
    _check(lib().oracle_runs_decode(*t._args(), _p(out)), "runs_decode")
    return out


def _regions(regions):
    arr = (Region * max(1, len(regions)))()
    for i, (dev_base, host) in enumerate(regions):
        assert host.dtype == np.uint8 and host.flags.c_contiguous
        arr[i] = Region(dev_base, host.nbytes, host.ctypes.data)
    return arr


def gather(t: RunTable, seg_bytes: int, regions, staging: np.ndarray | None = None) -> np.ndarray:
    """regions: list of (device base address, host uint8 image)."""
    if staging is None:
        staging = np.empty(t.n_lanes * t.n_blocks * seg_bytes, dtype=np.uint8)
    reg = _regions(regions)
    _check(lib().oracle_gather(*t._args(), seg_bytes, reg, len(regions), _p(staging)), "gather")
    return staging


def scatter(t: RunTable, seg_bytes: int, regions, staging: np.ndarray) -> None:
    reg = _regions(regions)
    _check(lib().oracle_scatter(*t._args(), seg_bytes, reg, len(regions), _p(staging)), "scatter")


# ---------------------------------------------------------- coalesced fetch

DESC = np.dtype([("src", "<u8"), ("dst_off", "<u8"), ("bytes", "<u8")])


def groups_plan(t: RunTable, seg_bytes: int, regions, max_read_bytes: int = 32 << 20):
    """regions: list of (device base, bytes).  Returns (descs, slab_bytes,
    local offsets [n_lanes, n_blocks])."""
    rb = np.array([b for b, _ in regions], np.uint64)
    rs = np.array([n for _, n in regions], np.uint64)
    n = ctypes.c_uint64(0)
    slab = ctypes.c_uint64(0)
    local = np.zeros((t.n_lanes, t.n_blocks), np.uint64)
    rc = lib().oracle_groups_plan(*t._args(), seg_bytes, _p(rb), _p(rs), len(regions), max_read_bytes, None, 0,
                                  ctypes.byref(n), ctypes.byref(slab), _p(local))
    if rc not in (OK, EARG) or (rc == EARG and n.value == 0 and t.n_runs):
        _check(rc, "groups_plan")
    descs = np.zeros(max(1, n.value), DESC)
    _check(lib().oracle_groups_plan(*t._args(), seg_bytes, _p(rb), _p(rs), len(regions), max_read_bytes,
                                    _p(descs), n.value, ctypes.byref(n), ctypes.byref(slab), _p(local)),
           "groups_plan")
    return descs[:n.value].copy(), slab.value, local


def copy_descs(descs: np.ndarray, regions, slab: np.ndarray) -> None:
    """regions: list of (device base, host uint8 image)."""
    d = np.ascontiguousarray(descs, dtype=DESC)
    reg = _regions(regions)
    _check(lib().oracle_copy_descs(_p(d) if d.size else None, d.size, reg, len(regions), _p(slab), slab.nbytes),
           "copy_descs")


# -------------------------------------------------------------- paged copy

def paged_copy(page_len: int, src_host: np.ndarray, src_idx, src_stride: int, src_offset: int,
               dst_host: np.ndarray, dst_idx, dst_stride: int, dst_offset: int) -> None:
    """Copy page src_idx[k] of src_host to page dst_idx[k] of dst_host (in place
    on dst_host); page i of a list is at offset + i * stride."""
    si = np.ascontiguousarray(src_idx, dtype=np.uint32)
    di = np.ascontiguousarray(dst_idx, dtype=np.uint32)
    assert si.size == di.size
    assert src_host.dtype == np.uint8 and dst_host.dtype == np.uint8
    s = Region(0, src_host.nbytes, src_host.ctypes.data)
    d = Region(0, dst_host.nbytes, dst_host.ctypes.data)
    _check(lib().oracle_paged_copy(page_len, ctypes.byref(s), _p(si) if si.size else None, src_stride, src_offset,
                                   ctypes.byref(d), _p(di) if di.size else None, dst_stride, dst_offset, si.size),
           "paged_copy")
