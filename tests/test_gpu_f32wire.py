"""GPU parity of xfer_combine2_f32 (the F32-wire all-reduce of the two-card
worker page) against the CPU oracle, bit for bit: ragged sizes of random bit
patterns (NaN, infinities and subnormals included), the drafter's 5 / 10 /
15 / 20 rows x 5120 partials on both emulated ranks, a 4.6 M-pair sweep of
structured operands, in place, and the 16384 x 5120 partials."""
import numpy as np
import pytest
import torch

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, random_f32_bits, say, up, zeros

pytestmark = pytest.mark.gpu

MODES = ((x.OUT_F32, np.uint32), (x.OUT_BF16, np.uint16))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8, 9, 1023, 1025, 2047, 2049, 65537])
def test_ragged_shapes_random_patterns(n):
    a = random_f32_bits(n, 13 * n + 1)
    b = random_f32_bits(n, 13 * n + 2)
    da, db = up(a), up(b)
    for mode, dt in MODES:
        nb = n * np.dtype(dt).itemsize
        out = filled(nb + 64, 0x5A)
        assert x.combine2_f32_raw(da.data_ptr(), db.data_ptr(), n, out.data_ptr(), mode) == x.OK
        got = down(out)
        assert np.array_equal(got[:nb].view(dt), oracle.combine2_f32(a, b, mode))
        assert np.all(got[nb:] == 0x5A)


@pytest.mark.parametrize("rows", [5, 10, 15, 20])
def test_drafter_rows_both_ranks_identical(rows):
    n = rows * 5120
    a = dg.prompt_partial(n, dg.seed_for(6, 0, rows))
    b = dg.prompt_partial(n, dg.seed_for(6, 1, rows))
    da, db = up(a), up(b)
    for mode, dt in MODES:
        want = oracle.combine2_f32(a, b, mode)
        o0 = zeros(n * np.dtype(dt).itemsize)
        o1 = zeros(n * np.dtype(dt).itemsize)
        # rank 0 and rank 1 both put rank 0's partial first
        assert x.combine2_f32_raw(da.data_ptr(), db.data_ptr(), n, o0.data_ptr(), mode) == x.OK
        assert x.combine2_f32_raw(da.data_ptr(), db.data_ptr(), n, o1.data_ptr(), mode) == x.OK
        g0, g1 = down(o0, dt), down(o1, dt)
        assert np.array_equal(g0, want) and np.array_equal(g1, want)
        # the sum commutes: the swapped order gives the same bits
        assert x.combine2_f32_raw(db.data_ptr(), da.data_ptr(), n, o1.data_ptr(), mode) == x.OK
        assert np.array_equal(down(o1, dt), want)


def test_structured_operand_sweep():
    """70 first operands spread over the exponent range (with infinities, NaN,
    the largest finite value and subnormals) against 65536 second operands
    whose top 16 bits run through every value (low bits drawn)."""
    firsts = [(e << 23) | (0x2AAAAA if (e // 8) % 2 else 0x000001) for e in range(0, 256, 8)]
    firsts += [0x7F800000, 0x7FC00000, 0x7F7FFFFF]
    firsts = np.array(firsts, np.uint32)
    firsts = np.concatenate([firsts, firsts | 0x80000000])
    low = dg.random_u64(1 << 15, 0x5EC0).view(np.uint32)[: 1 << 16] & 0xFFFF
    seconds = (np.arange(1 << 16, dtype=np.uint32) << 16) | low
    a = np.repeat(firsts, 1 << 16)
    b = np.tile(seconds, firsts.size)
    da, db = up(a), up(b)
    for mode, dt in MODES:
        say("f32-wire sweep mode", mode, a.size)
        out = zeros(a.size * np.dtype(dt).itemsize)
        assert x.combine2_f32_raw(da.data_ptr(), db.data_ptr(), a.size, out.data_ptr(), mode) == x.OK
        assert np.array_equal(down(out, dt), oracle.combine2_f32(a, b, mode))


def test_in_place_f32():
    n = 100003
    a = random_f32_bits(n, 21)
    b = random_f32_bits(n, 22)
    want = oracle.combine2_f32(a, b, 0)
    for which in ("a", "b"):
        da, db = up(a), up(b)
        out = da if which == "a" else db
        assert x.combine2_f32_raw(da.data_ptr(), db.data_ptr(), n, out.data_ptr(), x.OUT_F32) == x.OK
        assert np.array_equal(down(out, np.uint32), want)


def test_large_16384x5120():
    n = 16384 * 5120
    a = dg.prompt_partial(n, dg.seed_for(6, 0, 16384))
    b = dg.prompt_partial(n, dg.seed_for(6, 1, 16384))
    da, db = up(a), up(b)
    for mode, dt in MODES:
        say("f32-wire large mode", mode)
        o = zeros(n * np.dtype(dt).itemsize)
        assert x.combine2_f32_raw(da.data_ptr(), db.data_ptr(), n, o.data_ptr(), mode) == x.OK
        assert np.array_equal(down(o, dt), oracle.combine2_f32(a, b, mode))
        del o
    del da, db
    torch.cuda.empty_cache()


def test_refused_calls_leave_output_untouched():
    n = 1000
    a = up(random_f32_bits(n, 31))
    out = filled(4 * n, 0x44)
    assert x.combine2_f32_raw(a.data_ptr(), out.data_ptr(), n, out.data_ptr(), x.OUT_BF16) == x.E_INVAL
    assert x.combine2_f32_raw(a.data_ptr(), a.data_ptr(), n, out.data_ptr(), 3) == x.E_INVAL
    assert np.all(down(out) == 0x44)
