"""The library's host-only calls are re-entrant: run from several host
threads at once (ctypes releases the interpreter lock during each call),
every call returns exactly what it returns when run alone.  Covers the greedy
encoder, table validation, the coalescing planner, the streamed schedule and
the graph form's dependency list; none of them may keep state between calls."""
from concurrent.futures import ThreadPoolExecutor


import bf16_wire_all_amd as x
import datagen as dg

SEG = 4096


def _world(B, shuffle):
    n_slots = 64
    rb = dg.region_bytes_for(B, n_slots, SEG, 2)
    bases = [0x100000 + i * (rb + 4096) for i in range(2)]
    pos = dg.permutation(B, shuffle) if shuffle is not None else None
    return dg.kv_src_addrs(B, n_slots, SEG, bases, pos=pos), [(b, rb) for b in bases]


def _job(k):
    """One mixed sequence of host calls; returns everything it computed."""
    B = 300 + 37 * (k % 5)
    addrs, regions = _world(B, None if k % 3 == 0 else 100 + k)
    t = x.runs_encode(addrs, SEG, max_count=k % 4)
    v = x.runs_validate_status(t, regions, False)
    plan = x.groups_plan(t, regions, (1 + k % 3) * 64 * 1024)
    R, n_chunks = 1 + k % 4, 30 + k % 11
    ops = x.allreduce2_schedule(n_chunks, R)
    deps = x.allreduce2_graph_deps(n_chunks, R)
    return (t.runs_per_lane.tobytes(), t.run_base.tobytes(), t.run_stride.tobytes(), t.run_count.tobytes(), v,
            plan.descs.tobytes(), plan.slab_bytes, plan.local_base.tobytes(), plan.local_stride.tobytes(),
            [tuple(sorted(o.items())) for o in ops], deps)


def test_host_calls_from_many_threads_match_the_serial_results():
    jobs = list(range(48))
    serial = [_job(k) for k in jobs]
    with ThreadPoolExecutor(max_workers=8) as ex:
        for _ in range(3):
            parallel = list(ex.map(_job, jobs))
            for k, (a, b) in enumerate(zip(serial, parallel)):
                assert a == b, f"job {k} differs when run concurrently"
