"""Hot calls issued from several host threads at once, each thread on its own
default-priority stream and its own buffers: pack both partials, combine
them (F32 and BF16 out), and gather a small shuffled K/V set.  Every thread's
outputs equal the oracle's, bit for bit, so the hot calls keep no state
between calls that another thread could disturb."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, say, up, zeros

pytestmark = pytest.mark.gpu

THREADS = 6
SEG = 4096
CHUNK = 16 * 1024            # bytes of BF16 per chunk: 8192 elements
CE = CHUNK // 2


def _setup(k):
    n = 64 * 1024 + 37 * k + 3                   # ragged sizes, one per thread
    nc = -(-n // CE)
    a = dg.prompt_partial(n, dg.seed_for(2, 0, 40 + k))
    b = dg.prompt_partial(n, dg.seed_for(2, 1, 40 + k))
    B, n_slots = 24 + k, 8
    rb = dg.region_bytes_for(B, n_slots, SEG, 2)
    hosts = [dg.random_u64(rb // 8, dg.seed_for(4, r, 60 + k)).view(np.uint8) for r in range(2)]
    regions = [up(h) for h in hosts]
    bases = [regions[0].data_ptr(), regions[1].data_ptr()]
    addrs = dg.kv_src_addrs(B, n_slots, SEG, bases, pos=dg.permutation(B, 200 + k))
    t = x.runs_encode(addrs, SEG)
    plan_buf = zeros(x.runs_plan_bytes(t))
    plan = x.runs_prepare(t, [(bases[r], rb) for r in range(2)], False, plan_buf)
    return {"n": n, "nc": nc, "a": a, "b": b, "da": up(a).view(torch.float32), "db": up(b).view(torch.float32),
            "ring_a": torch.zeros(nc * CE, dtype=torch.int16, device="cuda"),
            "ring_b": torch.zeros(nc * CE, dtype=torch.int16, device="cuda"),
            "sum": torch.zeros(n, dtype=torch.float32, device="cuda"),
            "sum16": torch.zeros(n, dtype=torch.int16, device="cuda"),
            "staging": zeros(2 * n_slots * B * SEG), "t": t, "plan": plan, "plan_buf": plan_buf,
            "regions": regions, "hosts": hosts, "bases": bases, "stream": torch.cuda.Stream()}


def _issue(d, reps):
    """Everything this thread enqueues, on its own stream."""
    n, nc = d["n"], d["nc"]
    with torch.cuda.stream(d["stream"]):
        for _ in range(reps):
            x.pack_bf16(d["da"], d["ring_a"], CHUNK, 0, nc)
            x.pack_bf16(d["db"], d["ring_b"], CHUNK, 0, nc)
            x.combine2(d["ring_a"][:n], d["ring_b"][:n], d["sum"], x.OUT_F32)
            x.combine2(d["ring_a"][:n], d["ring_b"][:n], d["sum16"], x.OUT_BF16)
            x.gather_runs(d["plan"], d["staging"])
    return True


def test_hot_calls_from_several_threads():
    ds = [_setup(k) for k in range(THREADS)]
    torch.cuda.synchronize()
    say("hot calls from", THREADS, "threads")
    with ThreadPoolExecutor(max_workers=THREADS) as ex:
        assert all(ex.map(lambda d: _issue(d, 3), ds))
    torch.cuda.synchronize()
    for k, d in enumerate(ds):
        n, nc = d["n"], d["nc"]
        pa = oracle.pack(d["a"], nc * CE, CE, 0, nc)
        pb = oracle.pack(d["b"], nc * CE, CE, 0, nc)
        assert np.array_equal(down(d["ring_a"], np.uint16), pa), k
        assert np.array_equal(down(d["ring_b"], np.uint16), pb), k
        assert np.array_equal(down(d["sum"], np.uint32), oracle.combine2(pa[:n], pb[:n], x.OUT_F32)), k
        assert np.array_equal(down(d["sum16"], np.uint16), oracle.combine2(pa[:n], pb[:n], x.OUT_BF16)), k
        t = d["t"]
        ot = oracle.RunTable(t.runs_per_lane, t.run_base, t.run_stride, t.run_count, t.n_blocks)
        want = oracle.gather(ot, SEG, [(d["bases"][r], d["hosts"][r]) for r in range(2)])
        assert np.array_equal(down(d["staging"]), want), k
