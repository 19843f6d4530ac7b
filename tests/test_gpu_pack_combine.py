"""GPU parity of xfer_pack_bf16 and xfer_combine2 against the CPU oracle:
bit-exact (0 ULP) on the tiny workload with planted edge pairs, on ragged
and degenerate shapes, on the prompt-batch all-reduce (512 and 2048 tokens
x 5120, streaming through two 512 KiB slots and in bulk) and on the large
16384 x 5120 combine."""
import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, random_bf16, random_f32_bits, say, up, zeros

pytestmark = pytest.mark.gpu

CHUNK = 512 * 1024           # bytes of BF16 per chunk, as on the copy-engine page
CE = CHUNK // 2              # elements per chunk


def _pack_ring(src_np, ring_bytes, chunk_bytes, calls, sentinel=0xEE):
    """Run the same sequence of pack calls on the GPU and in the oracle, from
    the same sentinel-filled ring; return (gpu ring, oracle ring) as uint16."""
    src = up(src_np)
    ring = filled(ring_bytes, sentinel)
    ref = np.full(ring_bytes // 2, sentinel * 0x0101, dtype=np.uint16)
    n = src_np.size
    for c0, c1 in calls:
        st = x.pack_bf16_raw(src.data_ptr(), n, ring.data_ptr(), ring_bytes, chunk_bytes, c0, c1)
        assert st == x.OK, x.status_str(st)
        oracle.pack(src_np.view(np.float32), ring_bytes // 2, chunk_bytes // 2, c0, c1, ring=ref)
    return down(ring, np.uint16), ref


def test_tiny_workload_pack_and_combine():
    """5120-element partials with the edge pairs planted: one partial chunk in
    a two-slot ring, then both combine modes; both emulated ranks get the same
    bits, and swapping the operands changes nothing."""
    a, b = dg.tiny_pair()
    say("tiny pack rank 0/1", a.size)
    ga, ra = _pack_ring(a, 2 * CHUNK, CHUNK, [(0, 1)])
    gb, rb = _pack_ring(b, 2 * CHUNK, CHUNK, [(0, 1)])
    assert np.array_equal(ga, ra) and np.array_equal(gb, rb)
    pa, pb = ra[:a.size], rb[:b.size]
    da, db = up(pa), up(pb)
    # rank 1 holds its own copies of both wire buffers
    da1, db1 = up(pa), up(pb)
    for mode, dt in ((x.OUT_F32, np.uint32), (x.OUT_BF16, np.uint16)):
        say("tiny combine mode", mode)
        nb = a.size * np.dtype(dt).itemsize
        o0, o1, osw = zeros(nb), zeros(nb), zeros(nb)
        assert x.combine2_raw(da.data_ptr(), db.data_ptr(), a.size, o0.data_ptr(), mode) == x.OK
        assert x.combine2_raw(da1.data_ptr(), db1.data_ptr(), a.size, o1.data_ptr(), mode) == x.OK
        assert x.combine2_raw(db.data_ptr(), da.data_ptr(), a.size, osw.data_ptr(), mode) == x.OK
        want = oracle.combine2(pa, pb, mode)
        g0 = down(o0, dt)
        assert np.array_equal(g0, want)
        assert np.array_equal(down(o1, dt), g0)
        assert np.array_equal(down(osw, dt), g0)


@pytest.mark.parametrize("chunk_bytes", [16, 64, 4096])
@pytest.mark.parametrize("slots", [1, 2, 3])
@pytest.mark.parametrize("n", [1, 3, 4, 5, 31, 32, 33, 100, 1001, 4099])
def test_pack_ragged_shapes_random_patterns(n, slots, chunk_bytes):
    """Random F32 bit patterns (NaNs and infinities included), every chunk
    packed in calls of up to R chunks; the whole ring, untouched bytes
    included, matches the oracle after the sequence."""
    ce = chunk_bytes // 2
    n_chunks = -(-n // ce)
    calls = []
    c = 0
    step = 0
    while c < n_chunks:
        k = 1 + (step % slots)
        calls.append((c, min(n_chunks, c + k)))
        c = calls[-1][1]
        step += 1
    src = random_f32_bits(n, 1000 * n + 10 * slots + chunk_bytes)
    g, r = _pack_ring(src, slots * chunk_bytes, chunk_bytes, calls)
    assert np.array_equal(g, r)


def test_pack_special_patterns():
    """Every F32 pattern whose low 16 bits are 0x7FFF, 0x8000 or 0x8001 for all
    high halves (the round-up / tie / round-down boundary of every BF16
    value), plus NaN payloads and subnormals."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    pats = np.concatenate([hi | 0x7FFF, hi | 0x8000, hi | 0x8001, hi, hi | 0xFFFF,
                           np.arange(1 << 16, dtype=np.uint32),                 # subnormals
                           np.arange(0x7F800000, 0x7F810000, dtype=np.uint32),   # NaN payloads
                           np.arange(0xFF800000, 0xFF810000, dtype=np.uint32)])
    n = pats.size
    say("pack special patterns", n)
    g, r = _pack_ring(pats, -(-n // 8) * 16, -(-n // 8) * 16, [(0, 1)])
    assert np.array_equal(g[:n], r[:n])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 9, 1023, 1025, 65537])
def test_combine_ragged_shapes_random_patterns(n):
    a = random_bf16(n, 7 * n + 1)
    b = random_bf16(n, 7 * n + 2)
    da, db = up(a), up(b)
    for mode, dt in ((x.OUT_F32, np.uint32), (x.OUT_BF16, np.uint16)):
        out = filled(n * np.dtype(dt).itemsize + 64, 0x5A)
        assert x.combine2_raw(da.data_ptr(), db.data_ptr(), n, out.data_ptr(), mode) == x.OK
        got = down(out)
        assert np.array_equal(got[:n * np.dtype(dt).itemsize].view(dt), oracle.combine2(a, b, mode))
        assert np.all(got[n * np.dtype(dt).itemsize:] == 0x5A)


def test_combine_bf16_in_place():
    n = 100003
    a = random_bf16(n, 11)
    b = random_bf16(n, 12)
    want = oracle.combine2(a, b, 1)
    for which in ("a", "b"):
        da, db = up(a), up(b)
        out = da if which == "a" else db
        assert x.combine2_raw(da.data_ptr(), db.data_ptr(), n, out.data_ptr(), x.OUT_BF16) == x.OK
        assert np.array_equal(down(out, np.uint16), want)


def test_combine_all_bf16_pairs_with_fixed_first_operand_rows():
    """All 65536 second operands against 70 first operands spread over the
    exponent range, with infinities, NaNs and the largest finite values
    (4.6 M pairs), both modes."""
    pos = [(e << 7) | (0x41 if (e // 8) % 2 else 0) for e in range(0, 256, 8)] + [0x7F80, 0x7FC0, 0x7F7F]
    firsts = np.array(pos, dtype=np.uint16)
    firsts = np.concatenate([firsts, firsts | 0x8000])
    a = np.repeat(firsts, 1 << 16)
    b = np.tile(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16), firsts.size)
    da, db = up(a), up(b)
    for mode, dt in ((x.OUT_F32, np.uint32), (x.OUT_BF16, np.uint16)):
        say("combine sweep mode", mode, a.size)
        out = zeros(a.size * np.dtype(dt).itemsize)
        assert x.combine2_raw(da.data_ptr(), db.data_ptr(), a.size, out.data_ptr(), mode) == x.OK
        assert np.array_equal(down(out, dt), oracle.combine2(a, b, mode))


@pytest.mark.parametrize("tokens", [512, 2048])
def test_prompt_batch_allreduce_streaming_and_bulk(tokens):
    """Two F32 partials of tokens x 5120 ~ N(0, 0.5) with 1 % outliers x50.
    Streaming: per chunk, pack rank 0, pack rank 1 into their two-slot rings,
    combine the slot into the output.  Bulk: one pack per rank over a ring
    holding every chunk, one combine.  Both equal the oracle bit for bit."""
    n = tokens * 5120
    a = dg.prompt_partial(n, dg.seed_for(2, 0, tokens))
    b = dg.prompt_partial(n, dg.seed_for(2, 1, tokens))
    n_chunks = -(-n // CE)
    pa = oracle.pack(a, n_chunks * CE, CE, 0, n_chunks)[:n]
    pb = oracle.pack(b, n_chunks * CE, CE, 0, n_chunks)[:n]
    want_f32 = oracle.combine2(pa, pb, 0)
    want_b16 = oracle.combine2(pa, pb, 1)
    da, db = up(a), up(b)

    say("streaming", tokens, "x 5120,", n_chunks, "chunks")
    ring_a, ring_b = zeros(2 * CHUNK), zeros(2 * CHUNK)
    out = zeros(n * 4)
    for c in range(n_chunks):
        for src, ring in ((da, ring_a), (db, ring_b)):
            assert x.pack_bf16_raw(src.data_ptr(), n, ring.data_ptr(), 2 * CHUNK, CHUNK, c, c + 1) == x.OK
        ln = min(CE, n - c * CE)
        off = (c % 2) * CHUNK
        assert x.combine2_raw(ring_a.data_ptr() + off, ring_b.data_ptr() + off, ln,
                              out.data_ptr() + c * CE * 4, x.OUT_F32) == x.OK
    assert np.array_equal(down(out, np.uint32), want_f32)

    say("bulk", tokens, "x 5120")
    bulk_a, bulk_b = zeros(n_chunks * CHUNK), zeros(n_chunks * CHUNK)
    for src, ring in ((da, bulk_a), (db, bulk_b)):
        assert x.pack_bf16_raw(src.data_ptr(), n, ring.data_ptr(), n_chunks * CHUNK, CHUNK, 0, n_chunks) == x.OK
    assert np.array_equal(down(bulk_a, np.uint16)[:n], pa)
    assert np.array_equal(down(bulk_b, np.uint16)[:n], pb)
    for mode, dt, want in ((x.OUT_F32, np.uint32, want_f32), (x.OUT_BF16, np.uint16, want_b16)):
        o = zeros(n * np.dtype(dt).itemsize)
        assert x.combine2_raw(bulk_a.data_ptr(), bulk_b.data_ptr(), n, o.data_ptr(), mode) == x.OK
        assert np.array_equal(down(o, dt), want)


def test_large_combine_16384x5120():
    """The 16384 x 5120 partials: bulk pack of both ranks, then combine in both
    modes, all compared element by element with the oracle."""
    n = 16384 * 5120
    a = dg.prompt_partial(n, dg.seed_for(5, 0, 2))
    b = dg.prompt_partial(n, dg.seed_for(5, 1, 2))
    n_chunks = n // CE
    say("large pack", n)
    da = up(a)
    ring_a = zeros(n * 2)
    assert x.pack_bf16_raw(da.data_ptr(), n, ring_a.data_ptr(), n * 2, CHUNK, 0, n_chunks) == x.OK
    del da
    db = up(b)
    ring_b = zeros(n * 2)
    assert x.pack_bf16_raw(db.data_ptr(), n, ring_b.data_ptr(), n * 2, CHUNK, 0, n_chunks) == x.OK
    del db
    pa = oracle.pack(a, n, CE, 0, n_chunks)
    pb = oracle.pack(b, n, CE, 0, n_chunks)
    assert np.array_equal(down(ring_a, np.uint16), pa)
    assert np.array_equal(down(ring_b, np.uint16), pb)
    for mode, dt in ((x.OUT_F32, np.uint32), (x.OUT_BF16, np.uint16)):
        say("large combine mode", mode)
        o = zeros(n * np.dtype(dt).itemsize)
        assert x.combine2_raw(ring_a.data_ptr(), ring_b.data_ptr(), n, o.data_ptr(), mode) == x.OK
        assert np.array_equal(down(o, dt), oracle.combine2(pa, pb, mode))
        del o
    torch.cuda.empty_cache()


def test_failed_calls_leave_outputs_untouched():
    n = 1000
    src = up(random_f32_bits(n, 5))
    ring = filled(2 * 64, 0x33)
    # three chunks into two slots: refused, nothing written
    assert x.pack_bf16_raw(src.data_ptr(), n, ring.data_ptr(), 128, 64, 0, 3) == x.E_INVAL
    out = filled(4 * n, 0x44)
    assert x.combine2_raw(src.data_ptr(), src.data_ptr() + 16, n, out.data_ptr(), 7) == x.E_INVAL
    assert np.all(down(ring) == 0x33) and np.all(down(out) == 0x44)
