"""Every hot call can be captured in a HIP graph: the calls only enqueue
kernels on the given stream (no allocation, no synchronisation, no memset).
A whole step (both packs, combine2 in both modes, combine2_f32, argmax_merge,
argmax_merge_noalloc (the form for callers that cannot allocate, e.g. under
capture), gather, scatter, the coalesced fetch and a paged copy) is captured once and
replayed three times, with the inputs rewritten by eager work between the
replays; after every replay each output must equal the oracle on that
replay's inputs, bit for bit."""
import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import DEV, down, say, up, zeros

pytestmark = pytest.mark.gpu

CHUNK = 512 * 1024


def test_captured_step_replays_bit_exact():
    n = 3 * (CHUNK // 2) + 1001                       # four chunks, the last one short, odd length
    B, S, seg = 40, 6, 1024
    rows, cols, split = 8, 6000, 2816
    L = 2 * S
    rb = dg.region_bytes_for(B, S, seg)

    # buffers, all allocated before the capture
    a, b = zeros(4 * n), zeros(4 * n)
    ring_a, ring_b = zeros(4 * CHUNK), zeros(4 * CHUNK)      # R = 4 slots = every chunk of the call
    sum_f32, sum_b16 = zeros(4 * n), zeros(2 * n)
    f32w_f32, f32w_b16 = zeros(4 * n), zeros(2 * n)
    logits = zeros(2 * rows * cols)
    ws = zeros(x.argmax_workspace_bytes(rows, split, cols - split))
    top2 = zeros(16 * rows)
    max_noalloc = zeros(8 * rows)
    regs = [zeros(rb) for _ in range(2)]
    bases = [r.data_ptr() for r in regs]
    regions = [(p, rb) for p in bases]
    addrs = dg.kv_src_addrs(B, S, seg, bases, pos=dg.permutation(B, 3))
    staging = zeros(L * B * seg)
    dst = zeros(B * S * 3 * seg)
    daddrs = dg.kv_dst_addrs(B, S, seg, dst.data_ptr(), 3 * seg)
    t, dt = x.runs_encode(addrs, seg), x.runs_encode(daddrs, seg)
    pbuf, dbuf = zeros(x.runs_plan_bytes(t)), zeros(x.runs_plan_bytes(dt))
    splan = x.runs_prepare(t, regions, False, pbuf)
    dplan = x.runs_prepare(dt, [(dst.data_ptr(), dst.numel())], True, dbuf)
    g = x.groups_plan(t, regions)
    gbuf = zeros(max(16, x.descs_plan_bytes(len(g.descs))))
    fplan = x.descs_prepare(g.descs, g.slab_bytes, regions, gbuf)
    slab = zeros(g.slab_bytes)
    pidx = ((addrs[:S] - np.uint64(bases[0])) // np.uint64(seg)).T.reshape(-1).astype(np.uint32)  # region 0 lanes
    page_dst = zeros(pidx.size * seg)
    pgbuf = zeros(x.pages_plan_bytes(pidx.size))
    pplan = x.pages_prepare(seg, regions[0], pidx, seg, 0, (page_dst.data_ptr(), page_dst.numel()),
                            np.arange(pidx.size, dtype=np.uint32), seg, 0, pgbuf)
    s0 = x.shard(logits.data_ptr(), cols, rows, split, 0)
    s1 = x.shard(logits.data_ptr() + 2 * split, cols, rows, cols - split, split)

    def step():
        fa, fb = a.view(torch.float32), b.view(torch.float32)
        x.pack_bf16(fa, ring_a.view(torch.int16), CHUNK, 0, 4)
        x.pack_bf16(fb, ring_b.view(torch.int16), CHUNK, 0, 4)
        ra, rb16 = ring_a.view(torch.int16)[:n], ring_b.view(torch.int16)[:n]
        x.combine2(ra, rb16, sum_f32.view(torch.float32), x.OUT_F32)
        x.combine2(ra, rb16, sum_b16.view(torch.int16), x.OUT_BF16)
        x.combine2_f32(fa, fb, f32w_f32.view(torch.float32), x.OUT_F32)
        x.combine2_f32(fa, fb, f32w_b16.view(torch.int16), x.OUT_BF16)
        x.argmax_merge(s0, s1, x.TOP2, top2, ws)
        x.argmax_merge_noalloc(s0, s1, x.ARGMAX, max_noalloc)
        x.gather_runs(splan, staging)
        x.scatter_runs(staging, dplan)
        x.copy_descs(fplan, slab)
        x.paged_copy(pplan)

    def load_inputs(k):
        """Eager writes of replay k's inputs (outside the graph)."""
        ha = dg.prompt_partial(n, dg.seed_for(7, 0, k))
        hb = dg.prompt_partial(n, dg.seed_for(7, 1, k))
        a.copy_(up(ha))
        b.copy_(up(hb))
        lg = dg.argmax_logits(rows, 100 + k, cols=cols, split=split).logits
        logits.copy_(up(lg))
        hosts = []
        for i, r in enumerate(regs):
            h = np.empty(rb, np.uint8)
            dg.fill_region(h, bases[i], addrs, seg, 500 + 10 * k + i)
            r.copy_(torch.from_numpy(h).to(DEV))
            hosts.append(h)
        dst.fill_(0xA5)
        torch.cuda.synchronize()
        return ha, hb, lg, hosts

    # warm up the calls once eagerly (first launches load the code objects), then capture
    load_inputs(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("capturing the step")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    ot = oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, B)
    odt = oracle.RunTable(dt.runs_per_lane, dt.run_base, dt.run_stride, dt.run_count, B)
    for k in range(1, 4):
        ha, hb, lg, hosts = load_inputs(k)
        say("replay", k)
        graph.replay()
        torch.cuda.synchronize()
        pa = oracle.pack(ha, 4 * (CHUNK // 2), CHUNK // 2, 0, 4)[:n]
        pb = oracle.pack(hb, 4 * (CHUNK // 2), CHUNK // 2, 0, 4)[:n]
        assert np.array_equal(down(ring_a, np.uint16)[:n], pa), k
        assert np.array_equal(down(ring_b, np.uint16)[:n], pb), k
        assert np.array_equal(down(sum_f32, np.uint32), oracle.combine2(pa, pb, 0)), k
        assert np.array_equal(down(sum_b16, np.uint16), oracle.combine2(pa, pb, 1)), k
        assert np.array_equal(down(f32w_f32, np.uint32), oracle.combine2_f32(ha, hb, 0)), k
        assert np.array_equal(down(f32w_b16, np.uint16), oracle.combine2_f32(ha, hb, 1)), k
        assert down(top2).tobytes() == oracle.argmax_merge(lg, split, x.TOP2).tobytes(), k
        assert down(max_noalloc).tobytes() == oracle.argmax_merge(lg, split, x.ARGMAX).tobytes(), k
        oregions = list(zip(bases, hosts))
        want_stage = oracle.gather(ot, seg, oregions)
        assert np.array_equal(down(staging), want_stage), k
        want_dst = np.full(dst.numel(), 0xA5, np.uint8)
        oracle.scatter(odt, seg, [(dst.data_ptr(), want_dst)], want_stage)
        assert np.array_equal(down(dst), want_dst), k
        want_slab = np.zeros(g.slab_bytes, np.uint8)
        oracle.copy_descs(g.descs, oregions, want_slab)
        assert np.array_equal(down(slab), want_slab), k
        want_pages = np.zeros(page_dst.numel(), np.uint8)
        oracle.paged_copy(seg, hosts[0], pidx, seg, 0, want_pages, np.arange(pidx.size, dtype=np.uint32), seg, 0)
        assert np.array_equal(down(page_dst), want_pages), k
    del graph
