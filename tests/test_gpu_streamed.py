"""GPU parity of the streamed two-rank all-reduce (xfer_allreduce2_streamed):
both emulated ranks end with combine2(pack(rank 0), pack(rank 1)) bit for
bit, equal to the oracle, whatever the relative speed of the four streams.
Streams are perturbed by spin kernels enqueued ahead of the call, and two
calls reusing the same rings and events are issued back to back with no host
synchronisation in between."""
import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, say, up, zeros

pytestmark = pytest.mark.gpu

SPIN = 2_000_000  # cycles of torch.cuda._sleep (about a millisecond)


def _want(a, b, mode):
    pa = oracle.bf16_rne(a.view(np.uint32))
    pb = oracle.bf16_rne(b.view(np.uint32))
    return oracle.combine2(pa, pb, mode)


class Pair:
    """Rings, outputs, streams and events of one emulated rank pair."""

    def __init__(self, n, chunk_bytes, R, mode):
        self.n, self.chunk_bytes, self.R, self.mode = n, chunk_bytes, R, mode
        self.esize = 4 if mode == x.OUT_F32 else 2
        self.send = [zeros(R * chunk_bytes) for _ in range(2)]
        self.recv = [zeros(R * chunk_bytes) for _ in range(2)]
        self.compute = [torch.cuda.Stream() for _ in range(2)]
        self.wire = [torch.cuda.Stream() for _ in range(2)]
        self.events = x.Events(6 * R)

    def run(self, a_dev, b_dev, outs, delays=()):
        cur = torch.cuda.current_stream()
        for s in self.compute + self.wire:
            s.wait_stream(cur)              # the inputs were written on the current stream
        for which in delays:
            s = {"c0": self.compute[0], "c1": self.compute[1], "w0": self.wire[0], "w1": self.wire[1]}[which]
            with torch.cuda.stream(s):
                torch.cuda._sleep(SPIN)
        st = x.allreduce2_streamed((a_dev, b_dev), self.send, self.recv, outs, self.chunk_bytes, self.mode,
                                   self.compute, self.wire, self.events)
        assert st == x.OK, x.status_str(st)
        for s in self.compute:
            cur.wait_stream(s)


@pytest.mark.parametrize("R", [1, 2, 3])
@pytest.mark.parametrize("mode", [x.OUT_F32, x.OUT_BF16])
def test_small_chunks_all_slot_counts(R, mode):
    n, chunk = 1001, 64                           # 32 elements per chunk, ragged last chunk
    a = dg.normal_f32(n, 100 + R, 1.0)
    b = dg.normal_f32(n, 200 + R, 1.0)
    a.view(np.uint32)[::97] = 0x7F800001          # NaNs, a tie and a subnormal sprinkled in
    b.view(np.uint32)[5::89] = 0x3F808000
    b.view(np.uint32)[7::101] = 0x00018000
    p = Pair(n, chunk, R, mode)
    outs = [zeros(n * p.esize) for _ in range(2)]
    p.run(up(a), up(b), outs)
    want = _want(a, b, mode)
    dt = np.uint32 if mode == x.OUT_F32 else np.uint16
    assert np.array_equal(down(outs[0], dt), want)
    assert np.array_equal(down(outs[1], dt), want)


@pytest.mark.parametrize("delays", [("w0",), ("w1",), ("c0",), ("c1",), ("c1", "w0"), ("c0", "w1"),
                                    ("w0", "w1")])
def test_delayed_streams_two_slots(delays):
    """One slow stream at a time (or two): a missing wait would let a slot be
    overwritten before its reader ran, or read before its writer."""
    n, chunk, R = 40 * 256 + 17, 512, 2          # 41 chunks of 256 elements
    a = dg.normal_f32(n, 7, 0.5)
    b = dg.normal_f32(n, 8, 0.5)
    p = Pair(n, chunk, R, x.OUT_F32)
    outs = [zeros(n * 4) for _ in range(2)]
    say("streamed delays", delays)
    p.run(up(a), up(b), outs, delays)
    want = _want(a, b, x.OUT_F32)
    assert np.array_equal(down(outs[0], np.uint32), want)
    assert np.array_equal(down(outs[1], np.uint32), want)


def test_back_to_back_calls_reuse_rings_and_events():
    n, chunk, R = 20 * 128 + 3, 256, 2
    p = Pair(n, chunk, R, x.OUT_BF16)
    inputs = [(dg.normal_f32(n, 30 + k, 1.0), dg.normal_f32(n, 40 + k, 1.0)) for k in range(3)]
    outs = [[zeros(n * 2) for _ in range(2)] for _ in range(3)]
    dev_in = [(up(a), up(b)) for a, b in inputs]
    torch.cuda.synchronize()
    for k, (da, db) in enumerate(dev_in):
        # a slow wire stream before the second call, a slow compute stream before the third
        p.run(da, db, outs[k], delays=[(), ("w1",), ("c0",)][k])
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(inputs):
        want = _want(a, b, x.OUT_BF16)
        assert np.array_equal(down(outs[k][0], np.uint16), want), k
        assert np.array_equal(down(outs[k][1], np.uint16), want), k


@pytest.mark.parametrize("R", [1, 2])
def test_later_call_on_other_streams_waits_for_the_earlier_readers(R):
    """Two calls share rings and events but not streams, and nothing else
    orders them.  The first is one chunk whose rank-1 wire stream starts with
    a spin, so its rank-0 combine reads send[0] slot 0 about a millisecond
    after its own copy out of that slot is done.  The second call's pack of
    chunk 0 must wait for that combine, not only for the copy, or the first
    call sums the second call's data."""
    n, chunk = 100, 256                           # 128 elements per chunk: one chunk
    first = Pair(n, chunk, R, x.OUT_F32)
    second = Pair(n, chunk, R, x.OUT_F32)
    second.send, second.recv, second.events = first.send, first.recv, first.events
    ins = [(dg.normal_f32(n, 500 + 10 * k + R, 1.0), dg.normal_f32(n, 600 + 10 * k + R, 1.0)) for k in range(2)]
    dev = [(up(a), up(b)) for a, b in ins]
    outs = [[zeros(n * 4) for _ in range(2)] for _ in range(2)]
    torch.cuda.synchronize()
    with torch.cuda.stream(first.wire[1]):
        torch.cuda._sleep(SPIN)
    say("streamed later call on other streams, R", R)
    for k, p in enumerate((first, second)):
        st = x.allreduce2_streamed(dev[k], p.send, p.recv, outs[k], chunk, x.OUT_F32, p.compute, p.wire, p.events)
        assert st == x.OK, x.status_str(st)
    torch.cuda.synchronize()
    for k, (a, b) in enumerate(ins):
        want = _want(a, b, x.OUT_F32)
        assert np.array_equal(down(outs[k][0], np.uint32), want), k
        assert np.array_equal(down(outs[k][1], np.uint32), want), k


def test_prompt_batch_2048x5120_two_512k_slots():
    n = 2048 * 5120
    a = dg.prompt_partial(n, dg.seed_for(2, 0, 2048))
    b = dg.prompt_partial(n, dg.seed_for(2, 1, 2048))
    p = Pair(n, 512 * 1024, 2, x.OUT_F32)
    outs = [zeros(n * 4) for _ in range(2)]
    say("streamed 2048 x 5120")
    p.run(up(a), up(b), outs)
    want = _want(a, b, x.OUT_F32)
    assert np.array_equal(down(outs[0], np.uint32), want)
    assert np.array_equal(down(outs[1], np.uint32), want)


@pytest.mark.parametrize("R", [1, 2, 3])
@pytest.mark.parametrize("mode", [x.OUT_F32, x.OUT_BF16])
def test_graph_small_chunks_repeated_launches(R, mode):
    """The schedule as one HIP graph over fixed buffers: three launches on the
    current stream, the inputs rewritten on that stream between launches and
    no host synchronisation until the end; then each launch checked after a
    synchronisation."""
    n, chunk = 1001, 64
    esize = 4 if mode == x.OUT_F32 else 2
    dt = np.uint32 if mode == x.OUT_F32 else np.uint16
    a_dev, b_dev = zeros(4 * n), zeros(4 * n)
    send = [zeros(R * chunk) for _ in range(2)]
    recv = [zeros(R * chunk) for _ in range(2)]
    outs = [zeros(n * esize) for _ in range(2)]
    g = x.AllReduce2Graph((a_dev, b_dev), send, recv, outs, chunk, mode)
    inputs = [(dg.normal_f32(n, 300 + 7 * k + R, 1.0), dg.normal_f32(n, 400 + 7 * k + R, 1.0)) for k in range(3)]
    keep = [zeros(n * esize) for _ in range(3)]
    say("graph streamed R", R, "mode", mode)
    for k, (a, b) in enumerate(inputs):
        a_dev.copy_(up(a))
        b_dev.copy_(up(b))
        g.launch()
        keep[k].copy_(outs[k % 2])          # alternate ranks' outputs, ordered on the same stream
    for k, (a, b) in enumerate(inputs):
        assert np.array_equal(down(keep[k], dt), _want(a, b, mode)), k
    assert np.array_equal(down(outs[0], dt), down(outs[1], dt))
    g.close()


@pytest.mark.parametrize("use_graph", [False, True])
def test_more_slots_than_chunks(use_graph):
    """Six slots per rank and four chunks (the last one ragged): each chunk
    takes slot c, the results match the oracle, and ring slots 4 and 5 are
    never written (their sentinel bytes survive)."""
    n, chunk, R = 3 * 32 + 13, 64, 6
    a = dg.normal_f32(n, 71, 1.0)
    b = dg.normal_f32(n, 72, 1.0)
    send = [filled(R * chunk, 0xC3) for _ in range(2)]
    recv = [filled(R * chunk, 0x3C) for _ in range(2)]
    outs = [zeros(n * 4) for _ in range(2)]
    da, db = up(a), up(b)
    say("streamed more slots than chunks, graph", use_graph)
    if use_graph:
        g = x.AllReduce2Graph((da, db), send, recv, outs, chunk, x.OUT_F32)
        g.launch()
        torch.cuda.synchronize()
        g.close()
    else:
        compute = [torch.cuda.Stream() for _ in range(2)]
        wire = [torch.cuda.Stream() for _ in range(2)]
        for s_ in compute + wire:
            s_.wait_stream(torch.cuda.current_stream())
        ev = x.Events(6 * R)
        st = x.allreduce2_streamed((da, db), send, recv, outs, chunk, x.OUT_F32, compute, wire, ev)
        assert st == x.OK, x.status_str(st)
        torch.cuda.synchronize()
        ev.close()
    want = _want(a, b, x.OUT_F32)
    assert np.array_equal(down(outs[0], np.uint32), want)
    assert np.array_equal(down(outs[1], np.uint32), want)
    for r in range(2):
        assert (down(send[r])[4 * chunk:] == 0xC3).all()
        assert (down(recv[r])[4 * chunk:] == 0x3C).all()


def test_graph_on_a_side_stream_bf16_four_slots():
    """The graph launched on a stream other than the current one, which waits
    for the inputs first: 512 x 5120 through four 512 KiB slots per rank,
    BF16 out, two launches with new inputs in between."""
    n, chunk, R = 512 * 5120, 512 * 1024, 4
    send = [zeros(R * chunk) for _ in range(2)]
    recv = [zeros(R * chunk) for _ in range(2)]
    outs = [zeros(2 * n) for _ in range(2)]
    da, db = zeros(4 * n), zeros(4 * n)
    g = x.AllReduce2Graph((da, db), send, recv, outs, chunk, x.OUT_BF16)
    side = torch.cuda.Stream()
    say("graph on a side stream, 512x5120, R", R)
    for k in range(2):
        a = dg.prompt_partial(n, dg.seed_for(2, 0, 512) + 7 * k)
        b = dg.prompt_partial(n, dg.seed_for(2, 1, 512) + 7 * k)
        da.copy_(up(a))
        db.copy_(up(b))
        side.wait_stream(torch.cuda.current_stream())
        g.launch(side)
        torch.cuda.current_stream().wait_stream(side)
        want = _want(a, b, x.OUT_BF16)
        assert np.array_equal(down(outs[0], np.uint16), want), k
        assert np.array_equal(down(outs[1], np.uint16), want), k
    g.close()


def test_graph_prompt_batch_2048x5120():
    n, chunk, R = 2048 * 5120, 512 * 1024, 2
    a = dg.prompt_partial(n, dg.seed_for(2, 0, 2048))
    b = dg.prompt_partial(n, dg.seed_for(2, 1, 2048))
    send = [zeros(R * chunk) for _ in range(2)]
    recv = [zeros(R * chunk) for _ in range(2)]
    outs = [zeros(4 * n) for _ in range(2)]
    da, db = up(a), up(b)
    g = x.AllReduce2Graph((da, db), send, recv, outs, chunk, x.OUT_F32)
    say("graph streamed 2048x5120")
    for _ in range(2):
        g.launch()
    want = _want(a, b, x.OUT_F32)
    assert np.array_equal(down(outs[0], np.uint32), want)
    assert np.array_equal(down(outs[1], np.uint32), want)
    g.close()
