"""Python binding of libxfer (include/xfer.h): argument marshalling only.

Every step of the path runs in the HIP library; this module turns torch
tensors and numpy arrays into pointers and sizes, passes the current torch
stream, and raises XferError on a non-OK status.  It has no fallback: if
libxfer.so is missing, importing the functions fails loudly.

Device buffers are torch CUDA tensors (PyTorch supplies memory and streams);
run tables and addresses are numpy arrays on the host.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libxfer.so")

OK, E_INVAL, E_UNSUPPORTED, E_TABLE, E_RANGE, E_OVERLAP, E_DEVICE, E_HOST_MEMORY = range(8)
OUT_F32, OUT_BF16 = 0, 1
ARGMAX, TOP2 = 0, 1

EXPORTED = [
    "xfer_status_str", "xfer_pack_bf16", "xfer_combine2", "xfer_combine2_f32", "xfer_argmax_workspace_bytes",
    "xfer_argmax_merge", "xfer_runs_encode", "xfer_runs_validate", "xfer_runs_plan_bytes",
    "xfer_runs_prepare", "xfer_gather_runs", "xfer_scatter_runs", "xfer_allreduce2_event_id",
    "xfer_allreduce2_schedule", "xfer_events_create", "xfer_events_destroy", "xfer_allreduce2_streamed",
    "xfer_groups_plan", "xfer_descs_plan_bytes", "xfer_descs_prepare", "xfer_copy_descs",
    "xfer_pages_plan_bytes", "xfer_pages_prepare", "xfer_paged_copy",
    "xfer_allreduce2_graph_create", "xfer_allreduce2_graph_launch", "xfer_allreduce2_graph_destroy",
    "xfer_argmax_merge_noalloc", "xfer_allreduce2_graph_deps",
]


class XferError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} (status {status})")
        self.status = status


class Shard(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("ld", ctypes.c_size_t), ("rows", ctypes.c_uint32),
                ("ncols", ctypes.c_uint32), ("col_offset", ctypes.c_uint32)]


class RunTableC(ctypes.Structure):
    _fields_ = [("n_lanes", ctypes.c_uint32), ("n_blocks", ctypes.c_uint32), ("seg_bytes", ctypes.c_uint64),
                ("n_runs", ctypes.c_uint64), ("runs_per_lane", ctypes.c_void_p), ("run_base", ctypes.c_void_p),
                ("run_stride", ctypes.c_void_p), ("run_count", ctypes.c_void_p)]


class Op(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_uint32), ("rank", ctypes.c_uint32), ("chunk", ctypes.c_uint32),
                ("slot", ctypes.c_uint32), ("stream", ctypes.c_uint32), ("n_waits", ctypes.c_uint32),
                ("wait_event", ctypes.c_uint32 * 2), ("record_event", ctypes.c_uint32)]


class AllReduce2Desc(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p * 2), ("send", ctypes.c_void_p * 2), ("recv", ctypes.c_void_p * 2),
                ("out", ctypes.c_void_p * 2), ("n", ctypes.c_size_t), ("chunk_bytes", ctypes.c_size_t),
                ("ring_bytes", ctypes.c_size_t), ("out_mode", ctypes.c_int), ("compute", ctypes.c_void_p * 2),
                ("wire", ctypes.c_void_p * 2), ("events", ctypes.c_void_p), ("n_events", ctypes.c_size_t)]


class DescsPlan(ctypes.Structure):
    _fields_ = [("dev", ctypes.c_void_p), ("dev_bytes", ctypes.c_uint64), ("n_descs", ctypes.c_uint64),
                ("slab_bytes", ctypes.c_uint64), ("src_lo", ctypes.c_uint64), ("src_hi", ctypes.c_uint64),
                ("max_pieces", ctypes.c_uint32), ("piece_bytes", ctypes.c_uint32), ("magic", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32), ("n_spans", ctypes.c_uint32), ("reserved2", ctypes.c_uint32),
                ("spans", ctypes.c_uint64 * 8)]


class PagesC(ctypes.Structure):
    _fields_ = [("indices", ctypes.c_void_p), ("stride", ctypes.c_uint64), ("offset", ctypes.c_uint64)]


class PagesPlan(ctypes.Structure):
    _fields_ = [("dev", ctypes.c_void_p), ("dev_bytes", ctypes.c_size_t), ("n_pages", ctypes.c_uint64),
                ("page_len", ctypes.c_uint64), ("src_base", ctypes.c_uint64), ("src_stride", ctypes.c_uint64),
                ("dst_base", ctypes.c_uint64), ("dst_stride", ctypes.c_uint64), ("off_src_idx", ctypes.c_uint64),
                ("off_dst_idx", ctypes.c_uint64), ("units_per_page", ctypes.c_uint32), ("magic", ctypes.c_uint32)]


class Region(ctypes.Structure):
    _fields_ = [("base", ctypes.c_uint64), ("bytes", ctypes.c_uint64)]


class RunsPlan(ctypes.Structure):
    _fields_ = [("dev", ctypes.c_void_p), ("dev_bytes", ctypes.c_uint64), ("n_lanes", ctypes.c_uint32),
                ("n_blocks", ctypes.c_uint32), ("seg_bytes", ctypes.c_uint64), ("n_runs", ctypes.c_uint64),
                ("span_lo", ctypes.c_uint64), ("span_hi", ctypes.c_uint64), ("is_dst", ctypes.c_uint32),
                ("tile_blocks", ctypes.c_uint32), ("n_tiles", ctypes.c_uint32), ("group_blocks", ctypes.c_uint32),
                ("n_groups", ctypes.c_uint32), ("pieces", ctypes.c_uint32), ("magic", ctypes.c_uint32),
                ("lanes_per_wg", ctypes.c_uint32), ("off_group_run", ctypes.c_uint64), ("off_run_start", ctypes.c_uint64),
                ("off_run_base", ctypes.c_uint64), ("off_run_stride", ctypes.c_uint64), ("n_spans", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32), ("spans", ctypes.c_uint64 * 8)]


_lib = None


def lib():
    """The loaded libxfer.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, S, U32, U64, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int
        L.xfer_status_str.argtypes = [I]
        L.xfer_status_str.restype = ctypes.c_char_p
        L.xfer_pack_bf16.argtypes = [P, S, P, S, S, S, S, P]
        L.xfer_pack_bf16.restype = I
        L.xfer_combine2.argtypes = [P, P, S, P, I, P]
        L.xfer_combine2.restype = I
        L.xfer_combine2_f32.argtypes = [P, P, S, P, I, P]
        L.xfer_combine2_f32.restype = I
        L.xfer_argmax_workspace_bytes.argtypes = [U32, U32, U32]
        L.xfer_argmax_workspace_bytes.restype = S
        L.xfer_argmax_merge.argtypes = [ctypes.POINTER(Shard), ctypes.POINTER(Shard), I, P, P, S, P]
        L.xfer_argmax_merge.restype = I
        L.xfer_argmax_merge_noalloc.argtypes = [ctypes.POINTER(Shard), ctypes.POINTER(Shard), I, P, P]
        L.xfer_argmax_merge_noalloc.restype = I
        L.xfer_runs_encode.argtypes = [P, U32, U32, U32, P, P, P, P, U64, ctypes.POINTER(U64)]
        L.xfer_runs_encode.restype = I
        L.xfer_runs_validate.argtypes = [ctypes.POINTER(RunTableC), ctypes.POINTER(Region), I, I]
        L.xfer_runs_validate.restype = I
        L.xfer_runs_plan_bytes.argtypes = [ctypes.POINTER(RunTableC)]
        L.xfer_runs_plan_bytes.restype = S
        L.xfer_runs_prepare.argtypes = [ctypes.POINTER(RunTableC), ctypes.POINTER(Region), I, I, P, S,
                                        ctypes.POINTER(RunsPlan)]
        L.xfer_runs_prepare.restype = I
        L.xfer_gather_runs.argtypes = [ctypes.POINTER(RunsPlan), P, S, P]
        L.xfer_gather_runs.restype = I
        L.xfer_scatter_runs.argtypes = [P, S, ctypes.POINTER(RunsPlan), P]
        L.xfer_scatter_runs.restype = I
        L.xfer_allreduce2_event_id.argtypes = [U32, U32, U32, U32]
        L.xfer_allreduce2_event_id.restype = U32
        L.xfer_allreduce2_schedule.argtypes = [U32, U32, ctypes.POINTER(Op), S, ctypes.POINTER(S)]
        L.xfer_allreduce2_schedule.restype = I
        L.xfer_events_create.argtypes = [P, I]
        L.xfer_events_create.restype = I
        L.xfer_events_destroy.argtypes = [P, I]
        L.xfer_events_destroy.restype = I
        L.xfer_allreduce2_streamed.argtypes = [ctypes.POINTER(AllReduce2Desc)]
        L.xfer_allreduce2_streamed.restype = I
        L.xfer_groups_plan.argtypes = [ctypes.POINTER(RunTableC), ctypes.POINTER(Region), I, U64, P, U64,
                                       ctypes.POINTER(U64), ctypes.POINTER(U64), P, P, ctypes.POINTER(U64),
                                       ctypes.POINTER(U64)]
        L.xfer_groups_plan.restype = I
        L.xfer_descs_plan_bytes.argtypes = [U64]
        L.xfer_descs_plan_bytes.restype = S
        L.xfer_descs_prepare.argtypes = [P, U64, U64, ctypes.POINTER(Region), I, P, S, ctypes.POINTER(DescsPlan)]
        L.xfer_descs_prepare.restype = I
        L.xfer_copy_descs.argtypes = [ctypes.POINTER(DescsPlan), P, S, P]
        L.xfer_copy_descs.restype = I
        L.xfer_allreduce2_graph_create.argtypes = [ctypes.POINTER(AllReduce2Desc), ctypes.POINTER(ctypes.c_void_p)]
        L.xfer_allreduce2_graph_create.restype = I
        L.xfer_allreduce2_graph_launch.argtypes = [P, P]
        L.xfer_allreduce2_graph_launch.restype = I
        L.xfer_allreduce2_graph_destroy.argtypes = [P]
        L.xfer_allreduce2_graph_destroy.restype = I
        L.xfer_allreduce2_graph_deps.argtypes = [U32, U32, P, P, S, ctypes.POINTER(S)]
        L.xfer_allreduce2_graph_deps.restype = I
        L.xfer_pages_plan_bytes.argtypes = [U64]
        L.xfer_pages_plan_bytes.restype = S
        L.xfer_pages_prepare.argtypes = [U64, ctypes.POINTER(Region), ctypes.POINTER(PagesC), ctypes.POINTER(Region),
                                         ctypes.POINTER(PagesC), U64, P, S, ctypes.POINTER(PagesPlan)]
        L.xfer_pages_prepare.restype = I
        L.xfer_paged_copy.argtypes = [ctypes.POINTER(PagesPlan), P]
        L.xfer_paged_copy.restype = I
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().xfer_status_str(status).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise XferError(status, what)


def _stream(stream):
    """A torch stream or a raw hipStream_t handle; None is torch's current stream."""
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dev(t) -> int:
    """Pointer of a CUDA tensor (None -> NULL)."""
    if t is None:
        return 0
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous CUDA tensor")
    return t.data_ptr()


# ------------------------------------------------------------ pack / combine

def pack_bf16(src, ring, chunk_bytes: int, chunk_begin: int, chunk_end: int, stream=None) -> None:
    """src: F32 CUDA tensor (n elements); ring: 2-byte CUDA tensor."""
    if src.element_size() != 4 or ring.element_size() != 2:
        raise ValueError("src must be 4-byte, ring 2-byte elements")
    _check(lib().xfer_pack_bf16(_dev(src), src.numel(), _dev(ring), ring.numel() * 2, chunk_bytes, chunk_begin,
                                chunk_end, _stream(stream)), "xfer_pack_bf16")


def pack_bf16_raw(src_ptr: int, n: int, ring_ptr: int, ring_bytes: int, chunk_bytes: int, chunk_begin: int,
                  chunk_end: int, stream=None) -> int:
    """Raw-pointer form; returns the status without raising."""
    return lib().xfer_pack_bf16(src_ptr, n, ring_ptr, ring_bytes, chunk_bytes, chunk_begin, chunk_end,
                                _stream(stream))


def combine2(a, b, out, mode: int, stream=None) -> None:
    """a, b: 2-byte CUDA tensors (BF16 patterns); out: F32 (mode 0) or 2-byte (mode 1)."""
    n = a.numel()
    if b.numel() != n or out.numel() != n:
        raise ValueError("size mismatch")
    if out.element_size() != (4 if mode == OUT_F32 else 2):
        raise ValueError("output element size does not match the mode")
    _check(lib().xfer_combine2(_dev(a), _dev(b), n, _dev(out), mode, _stream(stream)), "xfer_combine2")


def combine2_raw(a_ptr: int, b_ptr: int, n: int, out_ptr: int, mode: int, stream=None) -> int:
    return lib().xfer_combine2(a_ptr, b_ptr, n, out_ptr, mode, _stream(stream))


def combine2_f32(a, b, out, mode: int, stream=None) -> None:
    """F32-wire combine: a, b F32 CUDA tensors; out F32 (mode 0) or 2-byte (mode 1)."""
    n = a.numel()
    if b.numel() != n or out.numel() != n:
        raise ValueError("size mismatch")
    if a.element_size() != 4 or b.element_size() != 4:
        raise ValueError("inputs must be 4-byte elements (F32)")
    if out.element_size() != (4 if mode == OUT_F32 else 2):
        raise ValueError("output element size does not match the mode")
    _check(lib().xfer_combine2_f32(_dev(a), _dev(b), n, _dev(out), mode, _stream(stream)), "xfer_combine2_f32")


def combine2_f32_raw(a_ptr: int, b_ptr: int, n: int, out_ptr: int, mode: int, stream=None) -> int:
    return lib().xfer_combine2_f32(a_ptr, b_ptr, n, out_ptr, mode, _stream(stream))


# ------------------------------------------------------------------- argmax

MAX_IDX = np.dtype([("max", "<f4"), ("idx", "<i4")])
TOP2_REC = np.dtype([("top1", "<f4"), ("top2", "<f4"), ("idx", "<i4"), ("reserved", "<i4")])


def argmax_workspace_bytes(rows: int, ncols0: int, ncols1: int) -> int:
    return int(lib().xfer_argmax_workspace_bytes(rows, ncols0, ncols1))


def shard(ptr: int, ld: int, rows: int, ncols: int, col_offset: int) -> Shard:
    return Shard(ptr, ld, rows, ncols, col_offset)


def argmax_merge(s0: Shard, s1: Shard, mode: int, out, workspace, stream=None) -> None:
    """out: CUDA tensor of rows * 8 (ARGMAX) or rows * 16 (TOP2) bytes;
    workspace: CUDA tensor of at least argmax_workspace_bytes() bytes, any
    contents (the call fills and reads it)."""
    _check(lib().xfer_argmax_merge(ctypes.byref(s0), ctypes.byref(s1), mode, _dev(out), _dev(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "xfer_argmax_merge")


def argmax_merge_raw(s0: Shard, s1: Shard, mode: int, out_ptr: int, ws_ptr: int, ws_bytes: int,
                     stream=None) -> int:
    return lib().xfer_argmax_merge(ctypes.byref(s0), ctypes.byref(s1), mode, out_ptr, ws_ptr, ws_bytes,
                                   _stream(stream))


# Bytes of the library's static partials array on each GPU (include/xfer.h).
ARGMAX_SCRATCH_BYTES = 65536


def argmax_merge_noalloc(s0: Shard, s1: Shard, mode: int, out, stream=None) -> None:
    """argmax_merge without a workspace: the partial records go to the
    library's static device array (calls that overlap on one GPU race)."""
    _check(lib().xfer_argmax_merge_noalloc(ctypes.byref(s0), ctypes.byref(s1), mode, _dev(out), _stream(stream)),
           "xfer_argmax_merge_noalloc")


def argmax_merge_noalloc_raw(s0: Shard, s1: Shard, mode: int, out_ptr: int, stream=None) -> int:
    return lib().xfer_argmax_merge_noalloc(ctypes.byref(s0), ctypes.byref(s1), mode, out_ptr, _stream(stream))


# --------------------------------------------------------------- run tables

@dataclass
class RunTable:
    """Host arrays of a run-encoded table (lane-major)."""
    runs_per_lane: np.ndarray   # uint32[n_lanes]
    run_base: np.ndarray        # uint64[n_runs]
    run_stride: np.ndarray      # int64[n_runs]
    run_count: np.ndarray       # uint32[n_runs]
    n_blocks: int
    seg_bytes: int

    @property
    def n_lanes(self) -> int:
        return int(self.runs_per_lane.size)

    @property
    def n_runs(self) -> int:
        return int(self.run_base.size)

    def c(self) -> RunTableC:
        for name, dt in (("runs_per_lane", np.uint32), ("run_base", np.uint64), ("run_stride", np.int64),
                         ("run_count", np.uint32)):
            a = getattr(self, name)
            if a.dtype != dt or not a.flags.c_contiguous:
                setattr(self, name, np.ascontiguousarray(a, dtype=dt))
        return RunTableC(self.n_lanes, self.n_blocks, self.seg_bytes, self.n_runs,
                         self.runs_per_lane.ctypes.data, self.run_base.ctypes.data,
                         self.run_stride.ctypes.data, self.run_count.ctypes.data)


def runs_encode(addrs: np.ndarray, seg_bytes: int, max_count: int = 0) -> RunTable:
    """Greedy run encoding of lane-major addresses [n_lanes, n_blocks]."""
    a = np.ascontiguousarray(addrs, dtype=np.uint64)
    n_lanes, n_blocks = a.shape
    cap = max(1, n_lanes * n_blocks)
    rpl = np.zeros(n_lanes, np.uint32)
    base = np.zeros(cap, np.uint64)
    stride = np.zeros(cap, np.int64)
    count = np.zeros(cap, np.uint32)
    nr = ctypes.c_uint64(0)
    _check(lib().xfer_runs_encode(a.ctypes.data, n_lanes, n_blocks, max_count, rpl.ctypes.data, base.ctypes.data,
                                  stride.ctypes.data, count.ctypes.data, cap, ctypes.byref(nr)), "xfer_runs_encode")
    n = nr.value
    return RunTable(rpl, base[:n].copy(), stride[:n].copy(), count[:n].copy(), n_blocks, seg_bytes)


def _regions(regions):
    arr = (Region * max(1, len(regions)))()
    for i, (base, nbytes) in enumerate(regions):
        arr[i] = Region(base, nbytes)
    return arr


def runs_validate_status(t: RunTable, regions, is_dst: bool) -> int:
    tc = t.c()
    return lib().xfer_runs_validate(ctypes.byref(tc), _regions(regions), len(regions), int(is_dst))


def runs_plan_bytes(t: RunTable) -> int:
    tc = t.c()
    return int(lib().xfer_runs_plan_bytes(ctypes.byref(tc)))


def runs_prepare_status(t: RunTable, regions, is_dst: bool, dev_ptr: int, dev_bytes: int):
    tc = t.c()
    plan = RunsPlan()
    st = lib().xfer_runs_prepare(ctypes.byref(tc), _regions(regions), len(regions), int(is_dst), dev_ptr,
                                 dev_bytes, ctypes.byref(plan))
    return st, plan


def runs_prepare(t: RunTable, regions, is_dst: bool, dev) -> RunsPlan:
    """regions: list of (device base, bytes); dev: CUDA tensor holding the plan."""
    st, plan = runs_prepare_status(t, regions, is_dst, _dev(dev), dev.numel() * dev.element_size())
    _check(st, "xfer_runs_prepare")
    return plan


def gather_runs(plan: RunsPlan, staging, stream=None) -> None:
    _check(lib().xfer_gather_runs(ctypes.byref(plan), _dev(staging), staging.numel() * staging.element_size(),
                                  _stream(stream)), "xfer_gather_runs")


def scatter_runs(staging, plan: RunsPlan, stream=None) -> None:
    _check(lib().xfer_scatter_runs(_dev(staging), staging.numel() * staging.element_size(), ctypes.byref(plan),
                                   _stream(stream)), "xfer_scatter_runs")


def gather_runs_raw(plan: RunsPlan, staging_ptr: int, staging_bytes: int, stream=None) -> int:
    return lib().xfer_gather_runs(ctypes.byref(plan), staging_ptr, staging_bytes, _stream(stream))


def scatter_runs_raw(staging_ptr: int, staging_bytes: int, plan: RunsPlan, stream=None) -> int:
    return lib().xfer_scatter_runs(staging_ptr, staging_bytes, ctypes.byref(plan), _stream(stream))


# ------------------------------------------------ streamed two-rank all-reduce

OP_PACK, OP_WIRE, OP_COMBINE = 0, 1, 2
EV_PACKED, EV_SENT, EV_COMBINED = 0, 1, 2


def allreduce2_event_id(kind: int, rank: int, slot: int, R: int) -> int:
    return int(lib().xfer_allreduce2_event_id(kind, rank, slot, R))


def allreduce2_schedule(n_chunks: int, R: int):
    """The driver's operation list (host only) as a list of dicts."""
    cap = 6 * n_chunks
    ops = (Op * max(1, cap))()
    n = ctypes.c_size_t(0)
    _check(lib().xfer_allreduce2_schedule(n_chunks, R, ops, cap, ctypes.byref(n)), "xfer_allreduce2_schedule")
    return [{"kind": o.kind, "rank": o.rank, "chunk": o.chunk, "slot": o.slot, "stream": o.stream,
             "waits": list(o.wait_event[:o.n_waits]), "record": o.record_event} for o in ops[:n.value]]


class Events:
    """n HIP events for the streamed driver (created recorded and complete)."""

    def __init__(self, n: int):
        self.n = n
        self.array = (ctypes.c_void_p * max(1, n))()
        _check(lib().xfer_events_create(self.array, n), "xfer_events_create")

    def close(self):
        if self.array is not None:
            lib().xfer_events_destroy(self.array, self.n)
            self.array = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _allreduce2_desc(src, send, recv, out, chunk_bytes: int, mode: int, compute=None, wire=None, events=None,
                     ring_bytes: int | None = None) -> AllReduce2Desc:
    def h(s):
        if s is None:
            return None
        return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)
    d = AllReduce2Desc()
    for r in range(2):
        d.src[r] = _dev(src[r])
        d.send[r] = _dev(send[r])
        d.recv[r] = _dev(recv[r])
        d.out[r] = _dev(out[r])
        d.compute[r] = h(compute[r]) if compute is not None else None
        d.wire[r] = h(wire[r]) if wire is not None else None
    d.n = src[0].numel() * src[0].element_size() // 4     # F32 elements
    d.chunk_bytes = chunk_bytes
    d.ring_bytes = send[0].numel() * send[0].element_size() if ring_bytes is None else ring_bytes
    d.out_mode = mode
    d.events = ctypes.cast(events.array, ctypes.c_void_p) if events is not None else None
    d.n_events = events.n if events is not None else 0
    return d


def allreduce2_streamed(src, send, recv, out, chunk_bytes: int, mode: int, compute, wire, events: Events,
                        ring_bytes: int | None = None) -> int:
    """src, send, recv, out: pairs of CUDA tensors (rank 0, rank 1); compute,
    wire: pairs of torch streams (or raw stream handles).  Returns the status."""
    d = _allreduce2_desc(src, send, recv, out, chunk_bytes, mode, compute, wire, events, ring_bytes)
    return lib().xfer_allreduce2_streamed(ctypes.byref(d))


class AllReduce2Graph:
    """The streamed schedule built once as a HIP graph over fixed buffers
    (src, send, recv, out as in allreduce2_streamed; no streams or events)."""

    def __init__(self, src, send, recv, out, chunk_bytes: int, mode: int, ring_bytes: int | None = None):
        self._keep = (src, send, recv, out)       # the graph holds their addresses
        d = _allreduce2_desc(src, send, recv, out, chunk_bytes, mode, ring_bytes=ring_bytes)
        self.exec = ctypes.c_void_p(None)
        _check(lib().xfer_allreduce2_graph_create(ctypes.byref(d), ctypes.byref(self.exec)),
               "xfer_allreduce2_graph_create")

    def launch(self, stream=None) -> None:
        _check(lib().xfer_allreduce2_graph_launch(self.exec, _stream(stream)), "xfer_allreduce2_graph_launch")

    def close(self) -> None:
        if self.exec is not None:
            lib().xfer_allreduce2_graph_destroy(self.exec)
            self.exec = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def allreduce2_graph_deps(n_chunks: int, R: int):
    """The graph form's dependencies as a list of (from, to) operation indices."""
    n = ctypes.c_size_t(0)
    st = lib().xfer_allreduce2_graph_deps(n_chunks, R, None, None, 0, ctypes.byref(n))
    if st not in (OK, E_RANGE):
        _check(st, "xfer_allreduce2_graph_deps")
    frm = (ctypes.c_uint32 * max(1, n.value))()
    to = (ctypes.c_uint32 * max(1, n.value))()
    _check(lib().xfer_allreduce2_graph_deps(n_chunks, R, frm, to, n.value, ctypes.byref(n)),
           "xfer_allreduce2_graph_deps")
    return [(frm[k], to[k]) for k in range(n.value)]


def allreduce2_graph_create_status(d: AllReduce2Desc) -> int:
    exec_ = ctypes.c_void_p(None)
    st = lib().xfer_allreduce2_graph_create(ctypes.byref(d), ctypes.byref(exec_))
    if st == OK and exec_.value:
        lib().xfer_allreduce2_graph_destroy(exec_)
    return st


# ---------------------------------------------- coalesced fetch by dense group

DESC = np.dtype([("src", "<u8"), ("dst_off", "<u8"), ("bytes", "<u8")])
MAX_READ_BYTES = 32 << 20


@dataclass
class GroupsPlan:
    descs: np.ndarray          # DESC[n]
    slab_bytes: int
    local_base: np.ndarray     # uint64[n_runs], slab offsets
    local_stride: np.ndarray   # int64[n_runs]
    n_groups: int
    n_dense: int

    def local_table(self, t: RunTable, slab_base: int) -> RunTable:
        """The source table's runs re-based onto the slab at slab_base."""
        return RunTable(t.runs_per_lane.copy(), (self.local_base + np.uint64(slab_base)).astype(np.uint64),
                        self.local_stride.copy(), t.run_count.copy(), t.n_blocks, t.seg_bytes)


def groups_plan_status(t: RunTable, regions, max_desc_bytes: int = MAX_READ_BYTES):
    tc = t.c()
    regs = _regions(regions)
    n = ctypes.c_uint64(0)
    slab = ctypes.c_uint64(0)
    ng = ctypes.c_uint64(0)
    nd = ctypes.c_uint64(0)
    lb = np.zeros(max(1, t.n_runs), np.uint64)
    ls = np.zeros(max(1, t.n_runs), np.int64)
    st = lib().xfer_groups_plan(ctypes.byref(tc), regs, len(regions), max_desc_bytes, None, 0, ctypes.byref(n),
                                ctypes.byref(slab), lb.ctypes.data, ls.ctypes.data, ctypes.byref(ng),
                                ctypes.byref(nd))
    if st not in (OK, E_RANGE):
        return st, None
    descs = np.zeros(max(1, n.value), DESC)
    st = lib().xfer_groups_plan(ctypes.byref(tc), regs, len(regions), max_desc_bytes, descs.ctypes.data,
                                n.value, ctypes.byref(n), ctypes.byref(slab), lb.ctypes.data, ls.ctypes.data,
                                ctypes.byref(ng), ctypes.byref(nd))
    if st != OK:
        return st, None
    return OK, GroupsPlan(descs[:n.value].copy(), slab.value, lb[:t.n_runs].copy(), ls[:t.n_runs].copy(),
                          ng.value, nd.value)


def groups_plan(t: RunTable, regions, max_desc_bytes: int = MAX_READ_BYTES) -> GroupsPlan:
    """regions: list of (device base, bytes)."""
    st, plan = groups_plan_status(t, regions, max_desc_bytes)
    _check(st, "xfer_groups_plan")
    return plan


def descs_plan_bytes(n_descs: int) -> int:
    return int(lib().xfer_descs_plan_bytes(n_descs))


def descs_prepare_status(descs: np.ndarray, slab_bytes: int, regions, dev_ptr: int, dev_bytes: int):
    d = np.ascontiguousarray(descs, dtype=DESC)
    plan = DescsPlan()
    st = lib().xfer_descs_prepare(d.ctypes.data if d.size else None, d.size, slab_bytes, _regions(regions),
                                  len(regions), dev_ptr, dev_bytes, ctypes.byref(plan))
    return st, plan


def descs_prepare(descs: np.ndarray, slab_bytes: int, regions, dev) -> DescsPlan:
    st, plan = descs_prepare_status(descs, slab_bytes, regions, _dev(dev), dev.numel() * dev.element_size())
    _check(st, "xfer_descs_prepare")
    return plan


def copy_descs(plan: DescsPlan, slab, stream=None) -> None:
    _check(lib().xfer_copy_descs(ctypes.byref(plan), _dev(slab), slab.numel() * slab.element_size(),
                                 _stream(stream)), "xfer_copy_descs")


# ------------------------------------------------------ paged copy (Pages)

def pages_plan_bytes(n_pages: int) -> int:
    return int(lib().xfer_pages_plan_bytes(n_pages))


def pages_prepare_status(page_len: int, src_region, src_idx, src_stride: int, src_offset: int, dst_region, dst_idx,
                         dst_stride: int, dst_offset: int, dev_ptr: int, dev_bytes: int):
    """src_region, dst_region: (device base, bytes); *_idx: page indices (host)."""
    si = np.ascontiguousarray(src_idx, dtype=np.uint32)
    di = np.ascontiguousarray(dst_idx, dtype=np.uint32)
    if si.size != di.size:
        raise ValueError("page lists differ in length")
    sr, dr = Region(*src_region), Region(*dst_region)
    sp = PagesC(si.ctypes.data if si.size else None, src_stride, src_offset)
    dp = PagesC(di.ctypes.data if di.size else None, dst_stride, dst_offset)
    plan = PagesPlan()
    st = lib().xfer_pages_prepare(page_len, ctypes.byref(sr), ctypes.byref(sp), ctypes.byref(dr), ctypes.byref(dp),
                                  si.size, dev_ptr, dev_bytes, ctypes.byref(plan))
    return st, plan


def pages_prepare(page_len: int, src_region, src_idx, src_stride: int, src_offset: int, dst_region, dst_idx,
                  dst_stride: int, dst_offset: int, dev) -> PagesPlan:
    st, plan = pages_prepare_status(page_len, src_region, src_idx, src_stride, src_offset, dst_region, dst_idx,
                                    dst_stride, dst_offset, _dev(dev), dev.numel() * dev.element_size())
    _check(st, "xfer_pages_prepare")
    return plan


def paged_copy(plan: PagesPlan, stream=None) -> None:
    _check(lib().xfer_paged_copy(ctypes.byref(plan), _stream(stream)), "xfer_paged_copy")
