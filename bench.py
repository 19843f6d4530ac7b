#!/usr/bin/env python3
"""Benchmark of the transfer staging / combine hot path on one MI355X.

One step is one pass of every hot-path kernel over one batch of synthetic,
HBM-resident input.  The default workload ("fragmented") is the largest
configuration that fits one GPU:
  pack_bf16 rank 0, pack_bf16 rank 1   16384 x 5120 F32 partials -> BF16, 512 KiB
                                       chunks (bulk: every chunk in one call)
  gather_runs (greedy table)           1000 blocks x 288 slots x 2 x 4 KiB from two
                                       regions whose blocks sit in a seeded shuffled
                                       order (288,000 runs) -> dense staging
  gather_runs (one run per segment)    the same set by 576,000 runs -> a second staging
  scatter_runs                         staging -> destination, 12 KiB slot stride
  argmax_merge (top1, top2, idx)       16 rows x 129280 BF16 logits, 2 shards
  combine2 (F32 out)                   the two packed partials summed in F32
combine runs last so its inputs, written by the packs, have been pushed out
of the caches by the gathers and the scatter: every kernel reads from HBM,
as in a cold pipeline.  `--workload step` is the smaller step (2048 x 5120
partials, bump-allocated blocks: one run per lane).

Prints ONE JSON line: value = algorithmic bytes of the whole step / wall
time of the step (GB/s, decimal).  The roofline kernel's duration comes from
HIP events recorded around it, on the stream it is launched on, in every
timed step.  The per-kernel breakdown ("kernels") comes from a separate,
untimed pass with events around every kernel; it also times kernels that are
not in the step (the 2048 x 5120 pack and combine, and combine's BF16
output mode).  After timing, every output of the last step and of the
breakdown pass is compared byte for byte with the CPU oracle on the same
inputs ("verified"); a mismatch makes the run exit with status 1.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
METRIC = "achieved HBM GB/s (and % of peak) for pack+combine and run-table segment gather"
CHUNK = 512 * 1024               # BF16 bytes per chunk
TOKENS, HIDDEN = 2048, 5120
ROWS, VOCAB, SPLIT = 16, 129280, 64768
N_BLOCKS, N_SLOTS, SEG, DST_SLOT_STRIDE = 1000, 288, 4096, 12288


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(tokens=TOKENS, extra_gathers=()):
    n = tokens * HIDDEN
    kv = N_BLOCKS * N_SLOTS * 2 * SEG
    ab = {
        "pack_rank0": 6 * n,                 # 4 B read + 2 B written per element
        "pack_rank1": 6 * n,
        "gather": 2 * kv,                    # every segment read once and written once
        "scatter": 2 * kv,
        "argmax_top2": ROWS * VOCAB * 2 + ROWS * 16,
        "combine_f32": 8 * n,                # 2 + 2 B read, 4 B written per element
    }
    for name in extra_gathers:
        ab[name] = 2 * kv
    return ab


def source_hash(name):
    with open(os.path.join(ROOT, "bf16_wire_all_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel_file, key):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it
    was taken on the kernel source as it is now (else None)."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    entry = data.get(key)
    if not entry or entry.get("source_sha256_16") != source_hash(kernel_file):
        return None
    return entry.get("traffic_bytes_per_launch")


# Set from the command line: added to every input seed, and the ring slots
# of the streamed all-reduce (two in the copy-engine design).
SEED_OFFSET = 0
SLOTS = 2
STREAM_CHUNK = CHUNK  # BF16 bytes per chunk of the streamed all-reduce


def _seed(dg, *args):
    return dg.seed_for(*args) + SEED_OFFSET


class Workload:
    """Device buffers of one step, filled from the seeded generators.

    tokens: rows of the F32 partials (x 5120); shuffled: blocks allocated in a
    seeded random order, so every lane breaks into many runs (the greedy
    table, and a second table with one run per segment, are both gathered)."""

    def __init__(self, dev, tokens=TOKENS, shuffled=False, n_blocks=N_BLOCKS, seg=SEG, coalesced=False,
                 streamed=False, f32wire=False, paged=False, extras=False, graph=False):
        import numpy as np
        import torch

        import bf16_wire_all_amd as x
        import datagen as dg

        self.x, self.torch, self.np = x, torch, np
        self.tokens, self.shuffled = tokens, shuffled
        self.n_blocks, self.seg = n_blocks, seg
        n = tokens * HIDDEN
        self.n = n
        self.n_chunks = -(-n // (CHUNK // 2))
        log("bench: generating inputs")
        cfg = 5 if shuffled else 2
        self.a_host = dg.prompt_partial(n, _seed(dg, cfg, 0, tokens))
        self.b_host = dg.prompt_partial(n, _seed(dg, cfg, 1, tokens))
        self.a = torch.from_numpy(self.a_host).to(dev)
        self.b = torch.from_numpy(self.b_host).to(dev)
        # BF16 bit patterns are held in int16 tensors (2-byte elements)
        self.ring_a = torch.zeros(self.n_chunks * CHUNK // 2, dtype=torch.int16, device=dev)
        self.ring_b = torch.zeros(self.n_chunks * CHUNK // 2, dtype=torch.int16, device=dev)
        self.sum = torch.zeros(n, dtype=torch.float32, device=dev)
        # kernels timed in the breakdown pass only: combine's BF16 output mode,
        # and the 2048 x 5120 pack and combine when the step's partials are larger
        self.extras = extras
        if extras:
            self.sum_bf16 = torch.zeros(n, dtype=torch.int16, device=dev)
            self.small = None
            if tokens != TOKENS:
                m = TOKENS * HIDDEN
                self.small_a_host = dg.prompt_partial(m, _seed(dg, 2, 0, TOKENS))
                self.small_b_host = dg.prompt_partial(m, _seed(dg, 2, 1, TOKENS))
                nc = -(-m // (CHUNK // 2))
                self.small = {
                    "n": m, "n_chunks": nc,
                    "a": torch.from_numpy(self.small_a_host).to(dev), "b": torch.from_numpy(self.small_b_host).to(dev),
                    "ring_a": torch.zeros(nc * CHUNK // 2, dtype=torch.int16, device=dev),
                    "ring_b": torch.zeros(nc * CHUNK // 2, dtype=torch.int16, device=dev),
                    "sum": torch.zeros(m, dtype=torch.float32, device=dev),
                    "sum_bf16": torch.zeros(m, dtype=torch.int16, device=dev),
                }

        inp = dg.argmax_logits(ROWS, _seed(dg, 3))
        self.logits_host = inp.logits
        self.logits = torch.from_numpy(inp.logits.view(np.int16).copy()).to(dev)
        p = self.logits.data_ptr()
        self.s0 = x.shard(p, VOCAB, ROWS, SPLIT, 0)
        self.s1 = x.shard(p + 2 * SPLIT, VOCAB, ROWS, VOCAB - SPLIT, SPLIT)
        self.ws = torch.zeros(x.argmax_workspace_bytes(ROWS, SPLIT, VOCAB - SPLIT), dtype=torch.uint8, device=dev)
        self.top2 = torch.zeros(ROWS * 16, dtype=torch.uint8, device=dev)

        B, SG = n_blocks, seg
        rb = dg.region_bytes_for(B, N_SLOTS, SG)
        self.regions = [torch.empty(rb, dtype=torch.uint8, device=dev) for _ in range(2)]
        bases = [r.data_ptr() for r in self.regions]
        pos = dg.permutation(B, _seed(dg, 5, 0, 1)) if shuffled else None
        self.src_addrs = dg.kv_src_addrs(B, N_SLOTS, SG, bases, pos=pos)
        self.region_hosts = []
        for i, r in enumerate(self.regions):
            h = np.empty(rb, np.uint8)
            dg.fill_region(h, bases[i], self.src_addrs, SG, _seed(dg, 4, 0, i))
            r.copy_(torch.from_numpy(h))
            self.region_hosts.append(h)
        self.src_table = x.runs_encode(self.src_addrs, SG)
        self.src_plan_buf = torch.zeros(x.runs_plan_bytes(self.src_table), dtype=torch.uint8, device=dev)
        self.src_plan = x.runs_prepare(self.src_table, [(b, rb) for b in bases], False, self.src_plan_buf)
        self.seg_plan = None
        if shuffled:
            # the unencoded worst case: one run per segment
            self.seg_table = x.runs_encode(self.src_addrs, SG, max_count=1)
            self.seg_plan_buf = torch.zeros(x.runs_plan_bytes(self.seg_table), dtype=torch.uint8, device=dev)
            self.seg_plan = x.runs_prepare(self.seg_table, [(b, rb) for b in bases], False, self.seg_plan_buf)
        self.staging = torch.empty(2 * N_SLOTS * B * SG, dtype=torch.uint8, device=dev)
        # the per-segment gather writes its own staging, so both gathers are checked
        self.staging_seg = torch.empty_like(self.staging) if shuffled else None
        self.fetch_plan = None
        if coalesced:
            # the whole source set read by dense-group descriptors into one slab
            self.groups = x.groups_plan(self.src_table, [(b, rb) for b in bases])
            self.desc_buf = torch.zeros(max(16, x.descs_plan_bytes(len(self.groups.descs))), dtype=torch.uint8,
                                        device=dev)
            self.fetch_plan = x.descs_prepare(self.groups.descs, self.groups.slab_bytes,
                                              [(b, rb) for b in bases], self.desc_buf)
            self.slab = torch.empty(self.groups.slab_bytes, dtype=torch.uint8, device=dev)
            log(f"bench: coalesced fetch with {len(self.groups.descs)} descriptors")
        slot_stride = 3 * SG  # K, V and a gap segment per slot
        self.dst = torch.full((B * N_SLOTS * slot_stride,), 0xA5, dtype=torch.uint8, device=dev)
        self.dst_addrs = dg.kv_dst_addrs(B, N_SLOTS, SG, self.dst.data_ptr(), slot_stride)
        self.dst_table = x.runs_encode(self.dst_addrs, SG)
        self.dst_plan_buf = torch.zeros(x.runs_plan_bytes(self.dst_table), dtype=torch.uint8, device=dev)
        self.dst_plan = x.runs_prepare(self.dst_table, [(self.dst.data_ptr(), self.dst.numel())], True,
                                       self.dst_plan_buf)
        self.paged = paged
        if paged:
            # the same set as Pages lists: per region, its lanes' pages -> block-major staging pages;
            # then staging pages -> the slot-major destination (gap page per slot)
            L, S = 2 * N_SLOTS, N_SLOTS // 2
            pos_ = pos if pos is not None else np.arange(B, dtype=np.uint32)
            bb = np.repeat(np.arange(B, dtype=np.int64), 2 * S)
            jj = np.tile(np.arange(2 * S, dtype=np.int64), B)
            self.page_plans, self.page_bufs, self.page_idx = [], [], []
            for r in range(2):
                si = (pos_.astype(np.int64)[bb] * 2 * S + jj).astype(np.uint32)
                di = (bb * L + r * 2 * S + jj).astype(np.uint32)
                buf = torch.zeros(x.pages_plan_bytes(si.size), dtype=torch.uint8, device=dev)
                self.page_plans.append(x.pages_prepare(SG, (bases[r], rb), si, SG, 0,
                                                       (self.staging.data_ptr(), self.staging.numel()), di, SG, 0,
                                                       buf))
                self.page_bufs.append(buf)
                self.page_idx.append((si, di))
            k = np.arange(B * L, dtype=np.int64)
            di = (((k // L) * N_SLOTS + (k % L) // 2) * 3 + (k % L) % 2).astype(np.uint32)
            buf = torch.zeros(x.pages_plan_bytes(k.size), dtype=torch.uint8, device=dev)
            self.page_scatter = x.pages_prepare(SG, (self.staging.data_ptr(), self.staging.numel()),
                                                k.astype(np.uint32), SG, 0, (self.dst.data_ptr(), self.dst.numel()),
                                                di, SG, 0, buf)
            self.page_bufs.append(buf)
            self.page_idx.append((k.astype(np.uint32), di))
        self.f32wire = f32wire
        if f32wire:
            # BF16 results of the F32-wire sum: the drafter's 20 rows, and the whole partials
            self.wire_rows = 20
            self.out_rows = torch.zeros(self.wire_rows * HIDDEN, dtype=torch.int16, device=dev)
            self.out_all = torch.zeros(n, dtype=torch.int16, device=dev)
        self.streamed = streamed
        if streamed:
            # both ranks' rings and results, and four default-priority streams
            self.send = [torch.zeros(SLOTS * STREAM_CHUNK // 2, dtype=torch.int16, device=dev) for _ in range(2)]
            self.recv = [torch.zeros(SLOTS * STREAM_CHUNK // 2, dtype=torch.int16, device=dev) for _ in range(2)]
            self.outs = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(2)]
            self.compute = [torch.cuda.Stream(device=dev) for _ in range(2)]
            self.wire = [torch.cuda.Stream(device=dev) for _ in range(2)]
            self.events = x.Events(6 * SLOTS)
        # graph: the same schedule built once as a HIP graph over these buffers,
        # launched on the current stream each step
        self.graph = x.AllReduce2Graph((self.a, self.b), self.send, self.recv, self.outs, STREAM_CHUNK,
                                       x.OUT_F32) if streamed and graph else None
        torch.cuda.synchronize()

    def _allreduce(self):
        """One streamed all-reduce, ordered after and before the current stream."""
        cur = self.torch.cuda.current_stream()
        for s in self.compute + self.wire:
            s.wait_stream(cur)
        st = self.x.allreduce2_streamed((self.a, self.b), self.send, self.recv, self.outs, STREAM_CHUNK, self.x.OUT_F32,
                                        self.compute, self.wire, self.events)
        if st != self.x.OK:
            raise RuntimeError(f"xfer_allreduce2_streamed: {self.x.status_str(st)}")
        for s in self.compute:
            cur.wait_stream(s)

    def kernels(self):
        """(name, callable) in step order; each callable enqueues one call."""
        x = self.x
        n, nc = self.n, self.n_chunks
        ra, rb = self.ring_a, self.ring_b
        if self.graph is not None:
            return [("allreduce2_graph", self.graph.launch)]
        if self.streamed:
            return [("allreduce2_streamed", self._allreduce)]
        if self.paged:
            return [("paged_gather_region0", lambda: x.paged_copy(self.page_plans[0])),
                    ("paged_gather_region1", lambda: x.paged_copy(self.page_plans[1])),
                    ("paged_scatter", lambda: x.paged_copy(self.page_scatter))]
        if self.f32wire:
            m = self.wire_rows * HIDDEN
            return [("combine_f32wire_20x5120", lambda: x.combine2_f32(self.a[:m], self.b[:m], self.out_rows,
                                                                      x.OUT_BF16)),
                    ("combine_f32wire_full", lambda: x.combine2_f32(self.a, self.b, self.out_all, x.OUT_BF16))]
        ks = [
            ("pack_rank0", lambda: x.pack_bf16(self.a, ra, CHUNK, 0, nc)),
            ("pack_rank1", lambda: x.pack_bf16(self.b, rb, CHUNK, 0, nc)),
            ("gather", lambda: x.gather_runs(self.src_plan, self.staging)),
        ]
        if self.seg_plan is not None:
            ks.append(("gather_per_segment", lambda: x.gather_runs(self.seg_plan, self.staging_seg)))
        if self.fetch_plan is not None:
            ks.append(("fetch_coalesced", lambda: x.copy_descs(self.fetch_plan, self.slab)))
        ks += [
            ("scatter", lambda: x.scatter_runs(self.staging, self.dst_plan)),
            ("argmax_top2", lambda: x.argmax_merge(self.s0, self.s1, x.TOP2, self.top2, self.ws)),
            ("combine_f32", lambda: x.combine2(ra[:n], rb[:n], self.sum, x.OUT_F32)),
        ]
        return ks

    def extra_kernels(self):
        """(name, callable) timed in the breakdown pass only, not in the step."""
        if not self.extras:
            return []
        x, n = self.x, self.n
        ks = [("combine_bf16", lambda: x.combine2(self.ring_a[:n], self.ring_b[:n], self.sum_bf16, x.OUT_BF16))]
        sm = self.small
        if sm is not None:
            m, nc = sm["n"], sm["n_chunks"]
            tag = f"{TOKENS}x{HIDDEN}"
            ks = [
                (f"pack_rank0_{tag}", lambda: x.pack_bf16(sm["a"], sm["ring_a"], CHUNK, 0, nc)),
                (f"pack_rank1_{tag}", lambda: x.pack_bf16(sm["b"], sm["ring_b"], CHUNK, 0, nc)),
                (f"combine_f32_{tag}", lambda: x.combine2(sm["ring_a"][:m], sm["ring_b"][:m], sm["sum"], x.OUT_F32)),
                (f"combine_bf16_{tag}", lambda: x.combine2(sm["ring_a"][:m], sm["ring_b"][:m], sm["sum_bf16"],
                                                           x.OUT_BF16)),
            ] + ks
        return ks

    def step_outputs(self):
        """Device buffers the step writes, by name (checked against the oracle)."""
        if self.streamed:
            return {"allreduce_rank0": self.outs[0], "allreduce_rank1": self.outs[1]}
        if self.f32wire:
            return {"combine_f32wire_20x5120": self.out_rows, "combine_f32wire_full": self.out_all}
        if self.paged:
            return {"paged_staging": self.staging, "paged_destination": self.dst}
        outs = {"ring_rank0": self.ring_a, "ring_rank1": self.ring_b, "gather_staging": self.staging,
                "scatter_destination": self.dst, "argmax_top2": self.top2, "combine_f32": self.sum}
        if self.staging_seg is not None:
            outs["gather_per_segment_staging"] = self.staging_seg
        if self.fetch_plan is not None:
            outs["fetch_slab"] = self.slab
        return outs

    def extra_outputs(self):
        """Device buffers the breakdown-only kernels write, by name."""
        if not self.extras:
            return {}
        outs = {"combine_bf16": self.sum_bf16}
        sm = self.small
        if sm is not None:
            tag = f"{TOKENS}x{HIDDEN}"
            outs.update({f"ring_rank0_{tag}": sm["ring_a"], f"ring_rank1_{tag}": sm["ring_b"],
                         f"combine_f32_{tag}": sm["sum"], f"combine_bf16_{tag}": sm["sum_bf16"]})
        return outs

    def extra_bytes(self):
        ab = {}
        for name, _ in self.extra_kernels():
            m = self.small["n"] if name.endswith(f"_{TOKENS}x{HIDDEN}") else self.n
            ab[name] = (6 if name.startswith(("pack", "combine_bf16")) else 8) * m
        return ab

    def algorithmic_bytes(self):
        if self.streamed:
            # per rank: pack 6 B, wire copy 2 B read + 2 B written, combine F32 8 B per element
            return {"allreduce2_graph" if self.graph is not None else "allreduce2_streamed": 2 * 18 * self.n}
        if self.paged:
            kv = self.n_blocks * N_SLOTS * 2 * self.seg
            return {"paged_gather_region0": kv, "paged_gather_region1": kv, "paged_scatter": 2 * kv}
        if self.f32wire:
            # 4 + 4 B read, 2 B written per element
            return {"combine_f32wire_20x5120": 10 * self.wire_rows * HIDDEN, "combine_f32wire_full": 10 * self.n}
        extra = (("gather_per_segment",) if self.seg_plan is not None else ()) + \
            (("fetch_coalesced",) if self.fetch_plan is not None else ())
        ab = algorithmic_bytes(self.tokens, extra)
        kv = self.n_blocks * N_SLOTS * 2 * self.seg
        for k in ("gather", "scatter", "gather_per_segment", "fetch_coalesced"):
            if k in ab:
                ab[k] = 2 * kv
        return ab


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def run_gpu(w, steps, warmup, roofline_kernel, expected):
    """Warm up, then time `steps` whole steps (wall clock, synchronised on both
    sides).  Inside the timed region only the roofline kernel is bracketed by
    HIP events (on the stream it is launched on), so the step's wall time
    carries one event pair per step, not one per kernel.  The outputs of the
    last timed step are then compared with the oracle's (`expected`).  A
    separate, untimed pass of up to 50 steps brackets every kernel for the
    breakdown, followed by the breakdown-only kernels, whose outputs are
    compared last."""
    import torch

    ks = w.kernels()
    rk = roofline_kernel
    log(f"bench: warmup {warmup} steps")
    for _ in range(warmup):
        for _, k in ks:
            k()
    torch.cuda.synchronize()
    live = []
    log(f"bench: timing {steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for name, k in ks:
            if name == rk:
                e0, e1 = _events()
                e0.record()
                k()
                e1.record()
                live.append((e0, e1))
            else:
                k()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    roofline_ms = sum(a.elapsed_time(b) for a, b in live) / len(live)
    log("bench: checking the last timed step against the oracle")
    checked = verify(w.step_outputs(), expected)
    log("bench: per-kernel breakdown pass")
    allk = ks + w.extra_kernels()
    events = {name: [] for name, _ in allk}
    for _ in range(min(steps, 50)):
        for name, k in allk:
            e0, e1 = _events()
            e0.record()
            k()
            e1.record()
            events[name].append((e0, e1))
    torch.cuda.synchronize()
    per_kernel_ms = {name: sum(a.elapsed_time(b) for a, b in ev) / len(ev) for name, ev in events.items()}
    checked.update(verify(w.extra_outputs(), expected))
    return elapsed, per_kernel_ms, roofline_ms, checked


def verify(outputs, expected, chunk=1 << 28):
    """Compare device buffers with the oracle's bytes, chunk by chunk.
    Returns {name: bytes compared}; raises Mismatch naming the first
    differing buffer and byte offset."""
    import numpy as np

    done = {}
    for name, t in outputs.items():
        want = expected[name].reshape(-1).view(np.uint8)
        got_t = t.reshape(-1).view(torch_uint8())
        if got_t.numel() != want.size:
            raise Mismatch(f"{name}: device {got_t.numel()} bytes, oracle {want.size} bytes")
        for off in range(0, want.size, chunk):
            got = got_t[off:off + chunk].cpu().numpy()
            ref = want[off:off + chunk]
            if not np.array_equal(got, ref):
                bad = off + int(np.flatnonzero(got != ref)[0])
                raise Mismatch(f"{name}: first differing byte at offset {bad}")
        done[name] = int(want.size)
    return done


class Mismatch(RuntimeError):
    pass


def torch_uint8():
    import torch
    return torch.uint8


WARM_SPIN_CYCLES = 200_000  # about 0.1 ms of GPU clock


def isolated(w, reps=20):
    """Each kernel of the workload on its own, cold two ways and warm, each
    kept as the median of `reps` event-timed repetitions:
      after_write:      before every repetition a 1 GiB scratch buffer is
                        written with ordinary stores (more than the 256 MB
                        Infinity Cache); the cache is then full of dirty
                        lines whose write-back shares HBM with the kernel;
      after_write_read: the same write, then a second 1 GiB buffer is read
                        (summed), which evicts those dirty lines first, so
                        the kernel starts on a cache full of clean,
                        unrelated data.
      warm:             no flush: the repetitions follow one another, so a
                        kernel whose bytes fit the 256 MB Infinity Cache may
                        find its inputs there (labelled, never the headline).
    In the step, by contrast, a short kernel that follows the gather or
    scatter shares HBM with their draining writes.

    Beside every kernel that moves at least 1 MB, the same cold protocol
    times two plain copies of the same algorithmic bytes (half read, half
    written): the HIP runtime's device-to-device copy, and the library's own
    128-bit copy (xfer_copy_descs over 32 MiB descriptors, the coalesced
    fetch's kernel).  They are the on-box ceiling at that size."""
    import numpy as np
    import torch

    import bf16_wire_all_amd as x

    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    other = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
    ab = w.algorithmic_bytes()
    calls = list(w.kernels())
    for name, _ in list(calls):
        half = ab[name] // 2 // 16 * 16
        if half < (1 << 19):
            continue
        src = torch.full((half,), 0x5A, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty(half, dtype=torch.uint8, device="cuda:0")
        n_d = -(-half // x.MAX_READ_BYTES)
        descs = np.zeros(n_d, x.DESC)
        descs["src"] = src.data_ptr() + np.arange(n_d, dtype=np.uint64) * x.MAX_READ_BYTES
        descs["dst_off"] = np.arange(n_d, dtype=np.uint64) * x.MAX_READ_BYTES
        descs["bytes"] = np.minimum(x.MAX_READ_BYTES, half - np.arange(n_d, dtype=np.int64) * x.MAX_READ_BYTES)
        buf = torch.zeros(x.descs_plan_bytes(n_d), dtype=torch.uint8, device="cuda:0")
        plan = x.descs_prepare(descs, half, [(src.data_ptr(), half)], buf)
        calls.append((f"ceiling_runtime_copy@{name}", lambda s=src, d=dst: d.copy_(s)))
        calls.append((f"ceiling_lib_copy@{name}", lambda p=plan, d=dst: x.copy_descs(p, d)))
        ab[f"ceiling_runtime_copy@{name}"] = ab[f"ceiling_lib_copy@{name}"] = 2 * half
        w._ceiling_keep = getattr(w, "_ceiling_keep", []) + [src, dst, buf]
    out = {"after_write": {}, "after_write_read": {}, "warm": {}}
    for mode in out:
        for name, k in calls:
            for _ in range(3):
                k()
            times = []
            for r in range(reps):
                if mode != "warm":
                    scratch.fill_(r & 0xFF)
                else:
                    # keep the GPU busy while the events and the kernel are
                    # enqueued, as the flush does in the cold states, so the
                    # host's launch latency stays outside the events
                    torch.cuda._sleep(WARM_SPIN_CYCLES)
                if mode == "after_write_read":
                    other.sum()
                e0, e1 = _events()
                e0.record()
                k()
                e1.record()
                e1.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = sorted(times)[len(times) // 2]
            gbs = ab[name] / (ms * 1e-3) / 1e9
            out[mode][name] = {"us": round(ms * 1e3, 2), "GBps": round(gbs, 1),
                               "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    del scratch, other
    w._ceiling_keep = []
    torch.cuda.empty_cache()
    return out


def oracle_step(w, bufs=None):
    """One step of the CPU oracle on the workload's host inputs, into `bufs`
    (allocated on the first call): the expected bytes of every output the
    step writes, by the names Workload.step_outputs uses."""
    import numpy as np

    import oracle

    n, ce = w.n, CHUNK // 2
    if bufs is None:
        bufs = {"ring_rank0": np.zeros(w.n_chunks * ce, np.uint16), "ring_rank1": np.zeros(w.n_chunks * ce, np.uint16),
                "gather_staging": np.zeros(2 * N_SLOTS * w.n_blocks * w.seg, np.uint8),
                "scatter_destination": np.full(w.dst.numel(), 0xA5, np.uint8)}
        if w.seg_plan is not None:
            bufs["gather_per_segment_staging"] = np.zeros_like(bufs["gather_staging"])
    regions = [(r.data_ptr(), h) for r, h in zip(w.regions, w.region_hosts)]
    oracle.pack(w.a_host, w.n_chunks * ce, ce, 0, w.n_chunks, ring=bufs["ring_rank0"])
    oracle.pack(w.b_host, w.n_chunks * ce, ce, 0, w.n_chunks, ring=bufs["ring_rank1"])
    oracle.gather(_oracle_table(w.src_table, w.n_blocks), w.seg, regions, staging=bufs["gather_staging"])
    if w.seg_plan is not None:
        oracle.gather(_oracle_table(w.seg_table, w.n_blocks), w.seg, regions,
                      staging=bufs["gather_per_segment_staging"])
    oracle.scatter(_oracle_table(w.dst_table, w.n_blocks), w.seg, [(w.dst.data_ptr(), bufs["scatter_destination"])],
                   bufs["gather_staging"])
    bufs["argmax_top2"] = oracle.argmax_merge(w.logits_host, SPLIT, 1)
    bufs["combine_f32"] = oracle.combine2(bufs["ring_rank0"][:n], bufs["ring_rank1"][:n], 0)
    if w.fetch_plan is not None:
        descs, _, _ = oracle.groups_plan(_oracle_table(w.src_table, w.n_blocks), w.seg,
                                         [(r.data_ptr(), r.numel()) for r in w.regions])
        slab = np.zeros(w.slab.numel(), np.uint8)
        oracle.copy_descs(descs, regions, slab)
        bufs["fetch_slab"] = slab
    return bufs


def _oracle_table(t, n_blocks):
    import oracle
    return oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, n_blocks)


def oracle_expected(w):
    """The oracle's bytes for every output the workload's kernels write
    (step and breakdown-only kernels), computed once, untimed."""
    import numpy as np

    import oracle

    if w.streamed:
        ce = CHUNK // 2
        nc = -(-w.n // ce)
        pa = oracle.pack(w.a_host, nc * ce, ce, 0, nc)[:w.n]
        pb = oracle.pack(w.b_host, nc * ce, ce, 0, nc)[:w.n]
        s = oracle.combine2(pa, pb, 0)
        return {"allreduce_rank0": s, "allreduce_rank1": s}
    if w.f32wire:
        m = w.wire_rows * HIDDEN
        return {"combine_f32wire_20x5120": oracle.combine2_f32(w.a_host[:m], w.b_host[:m], 1),
                "combine_f32wire_full": oracle.combine2_f32(w.a_host, w.b_host, 1)}
    if w.paged:
        staging = np.zeros(w.staging.numel(), np.uint8)
        for r in range(2):
            si, di = w.page_idx[r]
            oracle.paged_copy(w.seg, w.region_hosts[r], si, w.seg, 0, staging, di, w.seg, 0)
        dst = np.full(w.dst.numel(), 0xA5, np.uint8)
        si, di = w.page_idx[2]
        oracle.paged_copy(w.seg, staging, si, w.seg, 0, dst, di, w.seg, 0)
        return {"paged_staging": staging, "paged_destination": dst}
    return oracle_step(w)


def extra_expected(w, expected):
    """The oracle's bytes for the breakdown-only kernels; the step's packed
    partials are taken from `expected` (the oracle's step)."""
    import oracle

    out = {}
    if not w.extras:
        return out
    ce = CHUNK // 2
    pa, pb = expected["ring_rank0"][:w.n], expected["ring_rank1"][:w.n]
    out["combine_bf16"] = oracle.combine2(pa, pb, 1)
    sm = w.small
    if sm is not None:
        m, nc = sm["n"], sm["n_chunks"]
        tag = f"{TOKENS}x{HIDDEN}"
        ra = oracle.pack(w.small_a_host, nc * ce, ce, 0, nc)
        rb = oracle.pack(w.small_b_host, nc * ce, ce, 0, nc)
        out[f"ring_rank0_{tag}"], out[f"ring_rank1_{tag}"] = ra, rb
        out[f"combine_f32_{tag}"] = oracle.combine2(ra[:m], rb[:m], 0)
        out[f"combine_bf16_{tag}"] = oracle.combine2(ra[:m], rb[:m], 1)
    return out


def cpu_baseline(w, budget_s=12.0):
    """The oracle, as it is, on this host: the same step (same sizes, same
    inputs) repeated until about budget_s seconds of work (at least 3
    steps); buffers are allocated and touched before the clock starts.
    Returns the baseline record and the last step's outputs."""
    step_bytes = sum(w.algorithmic_bytes().values())
    bufs = oracle_step(w)
    reps, t_total, per_step = 0, 0.0, []
    while (t_total < budget_s or reps < 3) and reps < 50:
        t0 = time.perf_counter()
        oracle_step(w, bufs)
        per_step.append(time.perf_counter() - t0)
        t_total += per_step[-1]
        reps += 1
    med = sorted(per_step)[len(per_step) // 2]
    return {
        "value": round(step_bytes / med / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{reps} full steps of the same workload (same sizes and inputs), single-threaded C oracle, "
                  f"{t_total:.1f} s in all, median step {med * 1e3:.1f} ms (value from the median); host: "
                  f"{_cpu_model()}, {os.cpu_count()} logical CPUs",
    }, bufs


# hipDeviceAttribute_t values (ROCm 7.x hip_runtime_api.h): peak core clock,
# peak memory clock (both kHz) and compute-unit count.  The unit count is
# compared with torch's to confirm the numbering before the clocks are used.
_ATTR_CLOCK, _ATTR_BUS_WIDTH, _ATTR_MEM_CLOCK, _ATTR_CUS = 5, 59, 60, 63


def device_info():
    """Name, architecture, compute units, memory, peak clocks and memory bus
    width of cuda:0."""
    import ctypes

    import torch

    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2**30, 1), "l2_bytes": getattr(p, "L2_cache_size", None),
            "peak_clock_MHz": None, "peak_memory_clock_MHz": None, "memory_bus_bits": None}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)

        def attr(a):
            return v.value if hip.hipDeviceGetAttribute(ctypes.byref(v), a, 0) == 0 else None

        if attr(_ATTR_CUS) == p.multi_processor_count:
            clk, mem = attr(_ATTR_CLOCK), attr(_ATTR_MEM_CLOCK)
            info["peak_clock_MHz"] = clk // 1000 if clk else None
            info["peak_memory_clock_MHz"] = mem // 1000 if mem else None
            info["memory_bus_bits"] = attr(_ATTR_BUS_WIDTH)
    except OSError:
        pass
    return info


def _cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (or 'unknown')."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


WORKLOADS = {
    "step": {
        "args": {"tokens": TOKENS, "shuffled": False, "extras": True},
        "cpu_baseline": True,
        "describe": "transfer hot path: pack x2 + combine2 (2048x5120 F32 partials, 512 KiB BF16 chunks), "
                    "argmax merge (16x129280 BF16, split at 64768, top2), gather+scatter by run table "
                    "(1000 blocks x 288 slots x 2 x 4 KiB, one run per lane)",
        "roofline_kernel": ("gather", "gather_runs (paged K/V, 576 runs)", "runs_copy.hip", "gather_dense"),
    },
    "fragmented": {
        "args": {"tokens": 16384, "shuffled": True, "extras": True},
        "cpu_baseline": True,
        "describe": "fragmented transfer (the largest single-GPU configuration): pack x2 + combine2 (16384x5120 F32 "
                    "partials, 512 KiB BF16 chunks), argmax merge (16x129280 BF16, split at 64768, top2), gather of "
                    "1000 blocks x 288 slots x 2 x 4 KiB whose blocks sit in a seeded shuffled order, by the greedy "
                    "run table (288,000 runs) and by one run per segment (576,000 runs), scatter into a 12 KiB "
                    "slot-stride destination",
        "roofline_kernel": ("gather", "gather_runs (shuffled blocks, 288,000 runs)", "runs_copy.hip",
                            "gather_fragmented"),
    },
    "segments64k": {
        "args": {"tokens": TOKENS, "shuffled": False, "n_blocks": 200, "seg": 65536},
        "describe": "64 KiB segments: gather+scatter of 200 blocks x 288 slots x 2 x 64 KiB by run table (576 "
                    "runs, 7200 MiB per set), with the 2048x5120 pack/combine and the 16x129280 argmax",
        "roofline_kernel": ("gather", "gather_runs (64 KiB segments, 576 runs)", "runs_copy.hip", "gather_64k"),
    },
    "coalesced": {
        "args": {"tokens": TOKENS, "shuffled": False, "coalesced": True},
        "describe": "coalesced fetch: the step's kernels plus a read of the whole 1000 x 288 x 2 x 4 KiB source "
                    "set by 72 dense-group descriptors (at most 32 MiB each) into one slab",
        "roofline_kernel": ("fetch_coalesced", "copy_descs (72 dense-group reads)", "descs_copy.hip",
                            "fetch_dense"),
    },
    "paged": {
        "args": {"tokens": TOKENS, "shuffled": False, "paged": True},
        "describe": "paged copy by Pages lists (indices, stride, offset): the 1000 x 288 x 2 x 4 KiB set gathered by "
                    "two lists of 288,000 pages (one per region) into block-major staging, then scattered by one list "
                    "of 576,000 pages into the 12 KiB slot-stride destination",
        "roofline_kernel": ("paged_scatter", "paged_copy (576,000 pages of 4 KiB)", "pages_copy.hip",
                            "paged_scatter"),
    },
    "f32wire": {
        "args": {"tokens": 16384, "shuffled": False, "f32wire": True},
        "describe": "F32-wire all-reduce combine (two F32 partials summed in F32, rounded to BF16): the drafter's "
                    "20 x 5120 rows, and 16384 x 5120",
        "roofline_kernel": ("combine_f32wire_full", "combine2_f32 BF16 out (16384 x 5120)", "pack_combine.hip",
                            "combine_f32wire_16384x5120"),
    },
    "streamed": {
        "args": {"tokens": TOKENS, "shuffled": False, "streamed": True},
        "describe": "streamed two-rank all-reduce of two 2048x5120 F32 partials through BF16 chunks of "
                    "config.chunk_bytes (512 KiB unless --chunk-kib says otherwise) and config.slots ring slots "
                    "per rank (two unless --slots says otherwise): pack, "
                    "device-to-device wire copy, F32 combine for both ranks, ordered by events on four streams "
                    "(both ranks on one GPU)",
        "roofline_kernel": ("allreduce2_streamed", "allreduce2_streamed (40 chunks x 2 ranks x pack/copy/combine)",
                            None, None),
    },
    "streamed_graph": {
        "args": {"tokens": TOKENS, "shuffled": False, "streamed": True, "graph": True},
        "describe": "the streamed workload's all-reduce built once as a HIP graph (one kernel node per pack and "
                    "combine, one copy node per wire copy, the streams' orderings as explicit dependencies) and "
                    "launched on one stream each step",
        "roofline_kernel": ("allreduce2_graph", "allreduce2 graph (40 chunks x 2 ranks x pack/copy/combine)",
                            None, None),
    },
}


def calib_copy(gib=1, reps=5):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE readings to bytes."""
    import torch

    n = gib << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"calib: {reps} copies of {n} bytes")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="fragmented",
                    help="fragmented (default): the largest single-GPU configuration; step: the 2048 x 5120 / "
                         "bump-allocated step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true", help="run only the copy used to scale PMC readings")
    ap.add_argument("--isolated", action="store_true",
                    help="also time each kernel alone: cold (1 GiB written between repetitions, then also "
                         "read) and, labelled, warm")
    ap.add_argument("--seed-offset", type=int, default=0, help="added to every input seed (default 0)")
    ap.add_argument("--slots", type=int, default=2, help="ring slots of the streamed all-reduce (default 2)")
    ap.add_argument("--chunk-kib", type=int, default=CHUNK // 1024,
                    help="chunk size of the streamed all-reduce in KiB of BF16 (default 512)")
    args = ap.parse_args()
    global SEED_OFFSET, SLOTS, STREAM_CHUNK
    SEED_OFFSET, SLOTS, STREAM_CHUNK = args.seed_offset, args.slots, args.chunk_kib * 1024
    if SLOTS < 1:
        sys.exit("--slots must be >= 1")
    if args.chunk_kib < 1:
        sys.exit("--chunk-kib must be >= 1")
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the hot path here is single-GPU "
              "by design (both ranks are emulated in one HBM)", file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return
    if args.steps < 1:
        sys.exit("--steps must be >= 1")

    wl = WORKLOADS[args.workload]
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = Workload(dev, **wl["args"])
    baseline = None
    if not args.no_cpu_baseline and wl.get("cpu_baseline"):
        log("bench: cpu baseline (oracle); its last step is the expected output")
        baseline, expected = cpu_baseline(w)
    else:
        log("bench: oracle outputs (untimed)")
        expected = oracle_expected(w)
    expected.update(extra_expected(w, expected))
    rk, rk_label, rk_file, rk_key = wl["roofline_kernel"]
    verified, verify_error, checked = True, None, {}
    try:
        elapsed, kms, roofline_ms, checked = run_gpu(w, args.steps, args.warmup, rk, expected)
    except Mismatch as e:
        verified, verify_error = False, str(e)
        log(f"bench: OUTPUT MISMATCH against the oracle: {e}")
    if not verified:
        print(json.dumps({"metric": METRIC, "value": None, "verified": False, "verify_error": verify_error,
                          "config": {"workload": wl["describe"]}}), flush=True)
        sys.exit(1)
    ab = w.algorithmic_bytes()
    step_bytes = sum(ab.values())
    ab_all = dict(ab, **w.extra_bytes())
    ms_per_step = elapsed / args.steps * 1e3
    value = step_bytes * args.steps / elapsed / 1e9
    kernels = {}
    for name, ms in kms.items():
        gbs = ab_all[name] / (ms * 1e-3) / 1e9
        kernels[name] = {"us": round(ms * 1e3, 2), "bytes": ab_all[name], "GBps": round(gbs, 1),
                         "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4), "in_step": name in ab}

    def pack_combine(names):
        if not all(n in kms for n in names):
            return None
        return round(sum(ab_all[n] for n in names) / (sum(kms[n] for n in names) * 1e-3) / 1e9, 1)

    tag = f"{TOKENS}x{HIDDEN}"
    g_gbs = ab[rk] / (roofline_ms * 1e-3) / 1e9
    roofline = {"kernel": rk_label, "bound": "hbm", "achieved": round(g_gbs, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(g_gbs / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(rk_file, rk_key) if rk_file else None}
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl["describe"],
            "step_bytes": step_bytes,
            "parallelism": "single GPU; both ranks emulated in one HBM",
            "wire_dtype": "bf16",
            "inputs": "seeded synthetic: xoshiro256** seeded by SplitMix64, seed 0x5EED0000 + config "
                      f"+ (rank << 8) + (label << 16) + {SEED_OFFSET}",
            **({"slots": SLOTS, "chunk_bytes": STREAM_CHUNK} if args.workload.startswith("streamed") else {}),
        },
        "device": device_info(),
        "kernels": kernels,
        "pack_combine_GBps": pack_combine(("pack_rank0", "pack_rank1", "combine_f32")),
        f"pack_combine_{tag}_GBps": (pack_combine((f"pack_rank0_{tag}", f"pack_rank1_{tag}", f"combine_f32_{tag}"))
                                     or (pack_combine(("pack_rank0", "pack_rank1", "combine_f32"))
                                         if w.tokens == TOKENS else None)),
        "roofline": roofline,
        "verified": verified,
        "verified_outputs": checked,
        "cpu_baseline": baseline,
    }
    if args.isolated:
        log("bench: isolated pass (cold, then warm)")
        line["isolated"] = isolated(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
