"""Hazard analysis of the streamed two-rank all-reduce schedule, on the CPU.

The copy-engine page's review traced every read-after-write and
write-after-read hazard across its streams by hand; here the library's own
operation list (xfer_allreduce2_schedule) is checked mechanically: build the
happens-before relation from stream order and event waits, then require every
pair of operations that touch the same slot, at least one of them writing, to
be ordered the way they were issued.  Removing a wait that carries a
read-after-write dependency must expose a hazard, and with one slot (R = 1)
every wait is needed.
"""
import itertools

import pytest

import bf16_wire_all_amd as x


def _accesses(op):
    """(buffer, is_write) pairs of one operation; buffers are (name, rank, slot)."""
    r, s = op["rank"], op["slot"]
    if op["kind"] == x.OP_PACK:
        return [(("send", r, s), True)]
    if op["kind"] == x.OP_WIRE:
        return [(("send", r, s), False), (("recv", 1 - r, s), True)]
    return [(("send", r, s), False), (("recv", r, s), False), (("out", r, op["chunk"]), True)]


def _direct_preds(ops):
    """preds[i] = the ops op i is directly ordered after: its stream's previous
    op and the last recorder of each event it waits on."""
    preds = [set() for _ in ops]
    last_on_stream = {}
    last_record = {}
    for i, op in enumerate(ops):
        if op["stream"] in last_on_stream:
            preds[i].add(last_on_stream[op["stream"]])
        for e in op["waits"]:
            if e in last_record:          # a wait on an event not recorded in this call is a no-op
                preds[i].add(last_record[e])
        last_on_stream[op["stream"]] = i
        last_record[op["record"]] = i
    return preds


def _closure(preds):
    """hb[i] = set of ops that happen before op i (transitively)."""
    n = len(preds)
    hb = []
    for i in range(n):
        s = set()
        for p in preds[i]:
            s.add(p)
            s |= hb[p]
        hb.append(s)
    return hb


def _happens_before(ops):
    return _closure(_direct_preds(ops))


def _hazards(ops, hb=None):
    hb = _happens_before(ops) if hb is None else hb
    acc = [_accesses(o) for o in ops]
    bad = []
    for j in range(len(ops)):
        for i in range(j):
            for (bi, wi), (bj, wj) in itertools.product(acc[i], acc[j]):
                if bi == bj and (wi or wj) and i not in hb[j]:
                    bad.append((i, j, bi))
    return bad


def _without_wait(ops, idx, event):
    out = [dict(o, waits=list(o["waits"])) for o in ops]
    out[idx]["waits"].remove(event)
    return out


@pytest.mark.parametrize("R", [1, 2, 3, 4])
@pytest.mark.parametrize("n_chunks", [1, 2, 3, 5, 9])
def test_schedule_has_no_unordered_conflicts(R, n_chunks):
    ops = x.allreduce2_schedule(n_chunks, R)
    assert len(ops) == 6 * n_chunks
    assert _hazards(ops) == []


@pytest.mark.parametrize("R", [1, 2, 3])
def test_read_after_write_waits_are_load_bearing(R):
    """Dropping the wire copy's wait for its packed chunk, or the combine's
    wait for the peer's copy, lets a read overtake its write."""
    ops = x.allreduce2_schedule(2 * R + 1, R)
    for idx, op in enumerate(ops):
        if op["kind"] == x.OP_WIRE:
            e = x.allreduce2_event_id(x.EV_PACKED, op["rank"], op["slot"], R)
        elif op["kind"] == x.OP_COMBINE:
            e = x.allreduce2_event_id(x.EV_SENT, 1 - op["rank"], op["slot"], R)
        else:
            continue
        assert _hazards(_without_wait(ops, idx, e)), (idx, op)


def test_with_one_slot_every_wait_is_needed():
    R = 1
    ops = x.allreduce2_schedule(4, R)
    recorded = set()
    checked = 0
    for idx, op in enumerate(ops):
        for e in op["waits"]:
            if e in recorded:                 # waits that create an edge within the call
                assert _hazards(_without_wait(ops, idx, e)), (idx, op, e)
                checked += 1
        recorded.add(op["record"])
    assert checked >= 15


def test_schedule_shape_and_events():
    R = 2
    ops = x.allreduce2_schedule(3, R)
    kinds = [(o["kind"], o["rank"]) for o in ops[:6]]
    assert kinds == [(0, 0), (0, 1), (1, 0), (1, 1), (2, 0), (2, 1)]
    assert {o["stream"] for o in ops if o["kind"] == x.OP_WIRE} == {2, 3}
    ids = {x.allreduce2_event_id(k, r, s, R) for k in range(3) for r in range(2) for s in range(R)}
    assert ids == set(range(6 * R))
    with pytest.raises(x.XferError):
        x.allreduce2_schedule(3, 0)


def test_streamed_argument_checks():
    """Refusals that happen before any runtime call (no GPU needed)."""
    d = x.AllReduce2Desc()
    base = 0x10000000
    for r in range(2):
        d.src[r] = base + r * 0x100000
        d.send[r] = base + 0x400000 + r * 0x10000
        d.recv[r] = base + 0x500000 + r * 0x10000
        d.out[r] = base + 0x600000 + r * 0x100000
    d.n, d.chunk_bytes, d.ring_bytes, d.out_mode = 1000, 64, 128, 0
    d.events, d.n_events = 0x1234, 12
    L = x.lib()
    import ctypes
    for field, value in (("out_mode", 5), ("chunk_bytes", 24), ("ring_bytes", 96)):
        bad = x.AllReduce2Desc.from_buffer_copy(d)
        setattr(bad, field, value)
        assert L.xfer_allreduce2_streamed(ctypes.byref(bad)) == x.E_INVAL
    bad = x.AllReduce2Desc.from_buffer_copy(d)
    bad.recv[1] = bad.send[0] + 64            # receive ring overlaps a send ring
    assert L.xfer_allreduce2_streamed(ctypes.byref(bad)) == x.E_INVAL
    bad = x.AllReduce2Desc.from_buffer_copy(d)
    bad.out[0] = base + 8                     # misaligned and overlapping
    assert L.xfer_allreduce2_streamed(ctypes.byref(bad)) == x.E_INVAL
    short = x.AllReduce2Desc.from_buffer_copy(d)
    short.n_events = 11                        # two slots name event ids 0..11
    assert L.xfer_allreduce2_streamed(ctypes.byref(short)) == x.E_INVAL
    three = x.AllReduce2Desc.from_buffer_copy(d)
    three.ring_bytes = 192                     # three slots need 18 events, not 12
    assert L.xfer_allreduce2_streamed(ctypes.byref(three)) == x.E_INVAL
    empty = x.AllReduce2Desc.from_buffer_copy(d)
    empty.n = 0
    assert L.xfer_allreduce2_streamed(ctypes.byref(empty)) == x.OK


def test_graph_builder_argument_checks():
    """The graph builder refuses what the streamed call refuses, before any
    runtime call; an empty all-reduce yields no graph (nothing to launch)."""
    import ctypes
    d = x.AllReduce2Desc()
    base = 0x10000000
    for r in range(2):
        d.src[r] = base + r * 0x100000
        d.send[r] = base + 0x400000 + r * 0x10000
        d.recv[r] = base + 0x500000 + r * 0x10000
        d.out[r] = base + 0x600000 + r * 0x100000
    d.n, d.chunk_bytes, d.ring_bytes, d.out_mode = 1000, 64, 128, 0
    for field, value in (("out_mode", 5), ("chunk_bytes", 24), ("ring_bytes", 96)):
        bad = x.AllReduce2Desc.from_buffer_copy(d)
        setattr(bad, field, value)
        assert x.allreduce2_graph_create_status(bad) == x.E_INVAL
    bad = x.AllReduce2Desc.from_buffer_copy(d)
    bad.out[1] = bad.recv[0] + 32             # an output overlaps a receive ring
    assert x.allreduce2_graph_create_status(bad) == x.E_INVAL
    empty = x.AllReduce2Desc.from_buffer_copy(d)
    empty.n = 0
    ex = ctypes.c_void_p(0x1)
    assert x.lib().xfer_allreduce2_graph_create(ctypes.byref(empty), ctypes.byref(ex)) == x.OK
    assert ex.value is None
    assert x.lib().xfer_allreduce2_graph_create(ctypes.byref(d), None) == x.E_INVAL
    assert x.lib().xfer_allreduce2_graph_launch(None, None) == x.OK
    assert x.lib().xfer_allreduce2_graph_destroy(None) == x.OK
    no_events = x.AllReduce2Desc.from_buffer_copy(d)
    no_events.events = None
    assert x.lib().xfer_allreduce2_streamed(ctypes.byref(no_events)) == x.E_INVAL


@pytest.mark.parametrize("R", [1, 2, 3, 4])
@pytest.mark.parametrize("n_chunks", [1, 2, 3, 5, 9])
def test_graph_dependencies_are_the_streams_orderings(R, n_chunks):
    """The graph form gives each operation exactly the edges its stream and
    event waits give it in the streamed call, so it runs no pair of
    conflicting operations unordered; and every edge points back in issue order."""
    ops = x.allreduce2_schedule(n_chunks, R)
    deps = x.allreduce2_graph_deps(n_chunks, R)
    assert len(deps) == len(set(deps))
    preds = [set() for _ in ops]
    for a, b in deps:
        assert 0 <= a < b < len(ops)
        preds[b].add(a)
    assert preds == _direct_preds(ops)
    assert _hazards(ops, _closure(preds)) == []


@pytest.mark.parametrize("R,n_chunks", [(2, 40), (5, 23), (8, 8), (8, 3), (3, 31)])
def test_graph_dependencies_larger_calls(R, n_chunks):
    """The same equality and hazard check on longer calls: the prompt batch's
    40 chunks through two slots, and slot counts near and above the chunk
    count."""
    ops = x.allreduce2_schedule(n_chunks, R)
    preds = [set() for _ in ops]
    for a, b in x.allreduce2_graph_deps(n_chunks, R):
        preds[b].add(a)
    assert preds == _direct_preds(ops)
    assert _hazards(ops, _closure(preds)) == []


def test_graph_dependency_edges_are_load_bearing():
    """With one slot, dropping any graph edge that stands for an event wait
    lets two conflicting operations run unordered (stream-order edges may be
    implied by the waits)."""
    R, n_chunks = 1, 4
    ops = x.allreduce2_schedule(n_chunks, R)
    deps = x.allreduce2_graph_deps(n_chunks, R)
    stream_prev = {}
    last_on_stream = {}
    for i, op in enumerate(ops):
        if op["stream"] in last_on_stream:
            stream_prev[i] = last_on_stream[op["stream"]]
        last_on_stream[op["stream"]] = i
    checked = 0
    for k, (a, b) in enumerate(deps):
        if stream_prev.get(b) == a:
            continue
        preds = [set() for _ in ops]
        for kk, (aa, bb) in enumerate(deps):
            if kk != k:
                preds[bb].add(aa)
        assert _hazards(ops, _closure(preds)), (a, b)
        checked += 1
    assert checked >= 15


def test_graph_deps_argument_checks():
    import ctypes
    n = ctypes.c_size_t(0)
    L = x.lib()
    assert L.xfer_allreduce2_graph_deps(3, 0, None, None, 0, ctypes.byref(n)) == x.E_INVAL
    assert L.xfer_allreduce2_graph_deps(3, 2, None, None, 0, None) == x.E_INVAL
    assert L.xfer_allreduce2_graph_deps(3, 2, None, None, 0, ctypes.byref(n)) == x.E_RANGE
    need = n.value
    assert need == len(x.allreduce2_graph_deps(3, 2))
    buf = (ctypes.c_uint32 * need)()
    assert L.xfer_allreduce2_graph_deps(3, 2, buf, None, need, ctypes.byref(n)) == x.E_INVAL
    assert L.xfer_allreduce2_graph_deps(0, 2, None, None, 0, ctypes.byref(n)) == x.OK and n.value == 0


def _accesses_call(op, call):
    """As _accesses, with each call writing its own outputs (rings are shared)."""
    out = []
    for (name, r, k), w in _accesses(op):
        out.append(((name, r, k, call) if name == "out" else (name, r, k), w))
    return out


def _two_calls(n1, n2, R, same_streams):
    """Two calls on the same rings and events, the second on the same four
    streams or on four others."""
    a = x.allreduce2_schedule(n1, R)
    b = x.allreduce2_schedule(n2, R)
    ops = [dict(o, call=0) for o in a]
    ops += [dict(o, call=1, stream=o["stream"] + (0 if same_streams else 4)) for o in b]
    return ops


def _hazards_calls(ops):
    hb = _happens_before(ops)
    acc = [_accesses_call(o, o["call"]) for o in ops]
    bad = []
    for j in range(len(ops)):
        for i in range(j):
            for (bi, wi), (bj, wj) in itertools.product(acc[i], acc[j]):
                if bi == bj and (wi or wj) and i not in hb[j]:
                    bad.append((i, j, bi))
    return bad


@pytest.mark.parametrize("R", [1, 2, 3])
@pytest.mark.parametrize("n1,n2", [(1, 1), (2, 3), (5, 4), (7, 7)])
@pytest.mark.parametrize("same_streams", [True, False])
def test_a_later_call_is_ordered_after_the_earlier_one(R, n1, n2, same_streams):
    """Rings and events shared by consecutive calls: every slot conflict
    between the two calls is ordered, also when the second call runs on other
    streams (then only the events order it)."""
    assert _hazards_calls(_two_calls(n1, n2, R, same_streams)) == []


@pytest.mark.parametrize("R", [1, 2, 3, 4])
def test_every_wait_inside_a_call_is_load_bearing(R):
    """No redundant waits: dropping any wait on an event recorded earlier in
    the same call exposes a conflict (each costs host time in the runtime)."""
    ops = x.allreduce2_schedule(3 * R + 2, R)
    recorded = set()
    checked = 0
    for idx, op in enumerate(ops):
        for e in op["waits"]:
            if e in recorded:
                assert _hazards(_without_wait(ops, idx, e)), (idx, op, e)
                checked += 1
        recorded.add(op["record"])
    assert checked >= 2 * (3 * R + 2) - 2


def test_waits_per_operation():
    """With two slots, from chunk 2 on: pack none, wire one, combine one."""
    R = 2
    ops = x.allreduce2_schedule(6, R)
    for o in ops:
        n = len(o["waits"])
        if o["chunk"] < R:
            assert n == {x.OP_PACK: 2, x.OP_WIRE: 2, x.OP_COMBINE: 1}[o["kind"]], o
        else:
            assert n == {x.OP_PACK: 0, x.OP_WIRE: 1, x.OP_COMBINE: 1}[o["kind"]], o
