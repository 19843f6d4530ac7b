"""xfer_argmax_merge_noalloc on the GPU: the form without a workspace (its
partial records live in the library's static device array) gives the same
records, byte for byte, as xfer_argmax_merge with a caller workspace, and as
the CPU oracle, on two calls in a row, the second with a smaller input; and
it refuses, with its outputs untouched, a call whose partials exceed the
array."""
import numpy as np
import pytest

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, say, up

pytestmark = pytest.mark.gpu

GUARD = 64
MODES = ((x.ARGMAX, x.MAX_IDX), (x.TOP2, x.TOP2_REC))


def _shards(dl, rows, cols, split):
    s0 = x.shard(dl.data_ptr(), cols, rows, split, 0)
    s1 = x.shard(dl.data_ptr() + 2 * split, cols, rows, cols - split, split)
    return s0, s1


def _records(call, rows, rec):
    """Run call(out_ptr) into a buffer with guard bands; return the records."""
    nb = rows * rec.itemsize
    out = filled(GUARD + nb + GUARD, 0x5A)
    st = call(out.data_ptr() + GUARD)
    assert st == x.OK, x.status_str(st)
    got = down(out)
    assert np.all(got[:GUARD] == 0x5A) and np.all(got[GUARD + nb:] == 0x5A), "write outside the records"
    return got[GUARD:GUARD + nb].copy().view(rec)


def _compare(logits, split):
    rows, cols = logits.shape
    dl = up(logits)
    s0, s1 = _shards(dl, rows, cols, split)
    ws_bytes = x.argmax_workspace_bytes(rows, split, cols - split)
    ws = filled(ws_bytes, 0xFF)
    for mode, rec in MODES:
        want = oracle.argmax_merge(logits, split, mode)
        with_ws = _records(lambda o: x.argmax_merge_raw(s0, s1, mode, o, ws.data_ptr(), ws_bytes), rows, rec)
        no_ws = _records(lambda o: x.argmax_merge_noalloc_raw(s0, s1, mode, o), rows, rec)
        assert no_ws.tobytes() == with_ws.tobytes(), (mode, np.nonzero(no_ws != with_ws)[0][:5])
        assert no_ws.tobytes() == want.tobytes(), mode


def test_noalloc_matches_workspace_form_twice_second_smaller():
    """16 x 129280 with planted cross-shard ties, then 3 rows of other logits:
    the second call leaves the first call's partials behind in the array."""
    first = dg.argmax_logits(16, dg.seed_for(3))
    say("noalloc argmax 16 x 129280")
    _compare(first.logits, dg.SPLIT)
    second = dg.argmax_logits(3, dg.seed_for(3, 0, 7))
    say("noalloc argmax 3 x 129280")
    _compare(second.logits, dg.SPLIT)


def test_noalloc_largest_then_small_odd_shape():
    """4096 rows, the most the static array holds (one slice per shard row),
    then 5 rows of a narrow, ragged vocabulary (several slices per shard)."""
    big = dg.argmax_logits(4096, dg.seed_for(3, 0, 8), cols=20000, split=9992)
    assert x.argmax_workspace_bytes(4096, 9992, 20000 - 9992) == x.ARGMAX_SCRATCH_BYTES
    say("noalloc argmax 4096 x 20000")
    _compare(big.logits, 9992)
    small = dg.argmax_logits(5, dg.seed_for(3, 0, 9), cols=7000, split=4104)
    say("noalloc argmax 5 x 7000")
    _compare(small.logits, 4104)


def test_noalloc_wide_shards_then_narrow():
    """Shards wider than one 65,536-column slice (100,000 and 140,000
    columns: the 64-bit fold), then a narrow call that reuses the array."""
    wide = dg.argmax_logits(8, dg.seed_for(3, 0, 10), cols=240000, split=100000)
    say("noalloc argmax 8 x 240000")
    _compare(wide.logits, 100000)
    narrow = dg.argmax_logits(4, dg.seed_for(3, 0, 11), cols=3000, split=1504)
    say("noalloc argmax 4 x 3000")
    _compare(narrow.logits, 1504)


def test_noalloc_refuses_more_than_the_array_holds():
    rows, cols, split = 4097, 64, 32
    logits = np.zeros((rows, cols), np.uint16)
    dl = up(logits)
    s0, s1 = _shards(dl, rows, cols, split)
    assert x.argmax_workspace_bytes(rows, split, cols - split) > x.ARGMAX_SCRATCH_BYTES
    out = filled(rows * 16, 0x33)
    say("noalloc argmax refusal, 4097 rows")
    assert x.argmax_merge_noalloc_raw(s0, s1, x.TOP2, out.data_ptr()) == x.E_UNSUPPORTED
    assert np.all(down(out) == 0x33)
