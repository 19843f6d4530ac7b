"""GPU parity of xfer_argmax_merge against the CPU oracle: records compared
byte for byte (value bits, id, reserved word) in both modes, on the sharded
16 x 129280 workload with planted cross-shard ties, on a wider coverage
block with the hand-made edge rows, and on odd shard shapes (narrow,
ragged, padded rows, shard 1 holding the lower ids)."""
import numpy as np
import pytest

import bf16_wire_all_amd as x
import datagen as dg
import oracle
from tests.gpu_util import down, filled, random_bf16, say, up, zeros

pytestmark = pytest.mark.gpu

MODES = ((x.ARGMAX, x.MAX_IDX), (x.TOP2, x.TOP2_REC))


GUARD = 64  # guard bytes before and after the records, and after the workspace


def _workspace(nbytes, value):
    """A workspace of nbytes followed by a guard band."""
    return filled(nbytes + GUARD, value), nbytes


def _run(dl, s0, s1, rows, ws, mode, rec):
    ws_buf, ws_bytes = ws
    ws_tail = down(ws_buf)[ws_bytes:].copy()
    nb = rows * rec.itemsize
    out = filled(GUARD + nb + GUARD, 0x5A)
    st = x.argmax_merge_raw(s0, s1, mode, out.data_ptr() + GUARD, ws_buf.data_ptr(), ws_bytes)
    assert st == x.OK, x.status_str(st)
    got = down(out)
    assert np.all(got[:GUARD] == 0x5A) and np.all(got[GUARD + nb:] == 0x5A), "write outside the records"
    assert np.array_equal(down(ws_buf)[ws_bytes:], ws_tail), "write past the workspace"
    return got[GUARD:GUARD + nb].copy().view(rec)


def _check_matrix(logits, split, n1=None, calls=2):
    """Shard 0 = columns [0, split), shard 1 = [split, split + n1) of a
    row-major matrix; compare both modes, `calls` times on one workspace."""
    rows, cols = logits.shape
    n1 = cols - split if n1 is None else n1
    dl = up(logits)
    s0 = x.shard(dl.data_ptr(), cols, rows, split, 0)
    s1 = x.shard(dl.data_ptr() + 2 * split, cols, rows, n1, split)
    # the workspace needs no initialisation: start it full of garbage
    ws = _workspace(x.argmax_workspace_bytes(rows, split, n1), 0xFF)
    for mode, rec in MODES:
        want = oracle.argmax_merge(logits, split, mode, ncols1=n1)
        for _ in range(calls):
            got = _run(dl, s0, s1, rows, ws, mode, rec)
            assert got.tobytes() == want.tobytes(), (mode, np.nonzero(got != want)[0][:5])
    return want


def test_sharded_argmax_16_rows():
    """4 requests x 4 drafted positions over the 129280 vocabulary split at
    64768; ties across the boundary go to the lower id."""
    inp = dg.argmax_logits(16, dg.seed_for(3))
    say("argmax 16 x 129280")
    want = _check_matrix(inp.logits, dg.SPLIT)
    for k, r in enumerate(inp.tie_rows):
        assert want[r]["idx"] == inp.tie_cols[k][0]


def test_coverage_rows_and_hand_rows():
    """1024 drawn rows (one workgroup per shard row) plus the hand rows."""
    inp = dg.argmax_logits(1024, dg.seed_for(3, 0, 1))
    m = np.concatenate([inp.logits, dg.argmax_hand_rows()])
    say("argmax coverage", m.shape)
    _check_matrix(m, dg.SPLIT)


@pytest.mark.parametrize("rows", [1, 3, 40, 129])
def test_hand_rows_alone_and_mixed(rows):
    h = dg.argmax_hand_rows()
    m = np.concatenate([h] * (rows // h.shape[0] + 1))[:rows]
    _check_matrix(np.ascontiguousarray(m), dg.SPLIT)


ODD = [
    # (rows, ncols0, ncols1, ld pad) - narrow, ragged, single-column and full-width shards
    (5, 1, 1, 8),
    (7, 1, 9, 0),
    (3, 7, 8, 16),
    (9, 8, 1, 0),
    (11, 255, 1025, 24),
    (4, 65536, 3, 0),
    (2, 3, 65536, 8),
    (33, 2049, 4095, 0),
    (64, 64768, 64512, 0),
    # shards wider than one 65,536-column slice: the slices' keys are widened in the fold
    (4, 75968, 75968, 0),
    (3, 70001, 131073, 8),
    (600, 65537, 9, 0),          # many rows: two slices of the wide shard, one of the narrow
    (1, 2097152, 5, 0),          # the widest shard: 32 slices of 65,536
]


@pytest.mark.parametrize("rows,n0,n1,pad", ODD)
@pytest.mark.parametrize("alphabet", [True, False])
def test_odd_shapes(rows, n0, n1, pad, alphabet):
    ld = -(-(n0 + n1 + pad) // 8) * 8  # row pitch a multiple of 16 bytes
    seed = rows * 131 + n0 * 7 + n1 + pad + int(alphabet)
    if alphabet:
        letters = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0x7F80, 0xFF80, 0x3F81, 0x0001, 0x8001],
                           np.uint16)
        w = dg.random_u64(rows * ld, seed)
        m = letters[(w % letters.size).astype(np.int64)].reshape(rows, ld)
    else:
        m = random_bf16(rows * ld, seed, allow_nan=False).reshape(rows, ld)
    # shard 0 on columns [0, n0); shard 1 on columns [ld - n1 ... ] would break
    # contiguity of ids, so shard 1 takes [n0_aligned, n0_aligned + n1) in memory
    # with ids continuing at n0.
    n0a = -(-n0 // 8) * 8
    if n0a + n1 > ld:
        ld = -(-(n0a + n1) // 8) * 8
        m = np.concatenate([m, np.zeros((rows, ld - m.shape[1]), np.uint16)], axis=1)
    dl = up(m)
    s0 = x.shard(dl.data_ptr(), ld, rows, n0, 0)
    s1 = x.shard(dl.data_ptr() + 2 * n0a, ld, rows, n1, n0)
    o0 = oracle.Shard(m.ctypes.data, ld, rows, n0, 0)
    o1 = oracle.Shard(m.ctypes.data + 2 * n0a, ld, rows, n1, n0)
    ws = _workspace(x.argmax_workspace_bytes(rows, n0, n1), 0)
    for mode, rec in MODES:
        want = oracle.argmax_merge_shards(o0, o1, mode)
        got = _run(dl, s0, s1, rows, ws, mode, rec)
        assert got.tobytes() == want.tobytes(), mode
        # swap the shards' roles: shard 1's memory holds the LOWER ids now
        s0b = x.shard(dl.data_ptr(), ld, rows, n0, n1)
        s1b = x.shard(dl.data_ptr() + 2 * n0a, ld, rows, n1, 0)
        o0b = oracle.Shard(m.ctypes.data, ld, rows, n0, n1)
        o1b = oracle.Shard(m.ctypes.data + 2 * n0a, ld, rows, n1, 0)
        want_b = oracle.argmax_merge_shards(o0b, o1b, mode)
        got_b = _run(dl, s0b, s1b, rows, ws, mode, rec)
        assert got_b.tobytes() == want_b.tobytes(), mode


def test_failed_call_leaves_output_untouched():
    rows, cols = 4, 1024
    m = random_bf16(rows * cols, 3, allow_nan=False)
    dl = up(m)
    s0 = x.shard(dl.data_ptr(), cols, rows, 512, 0)
    s1 = x.shard(dl.data_ptr() + 1024, cols, rows, 512, 100)  # ids overlap shard 0's
    out = zeros(rows * 16) + 7
    ws = zeros(4096)
    assert x.argmax_merge_raw(s0, s1, x.TOP2, out.data_ptr(), ws.data_ptr(), 4096) == x.E_INVAL
    assert np.all(down(out) == 7)


def test_every_value_wins_with_its_own_bits():
    """Every BF16 pattern but NaN is once a row's top1 (the rest of the row
    -inf) and once a row's top2 (under a planted +inf): both records carry the
    chosen element's exact bits, the sign of a zero included."""
    p = np.arange(1 << 16, dtype=np.uint32)
    pats = p[(p & 0x7FFF) <= 0x7F80].astype(np.uint16)
    n, cols, split = pats.size, 80, 40
    i = np.arange(n)
    m = np.full((2 * n, cols), 0xFF80, np.uint16)
    m[i, (i * 13) % cols] = pats                               # rows [0, n): pats[i] is top1
    c = (i * 29 + 5) % cols
    m[n + i, c] = pats                                         # rows [n, 2n): pats[i] is top2 ...
    m[n + i, (c + 1 + i % (cols - 1)) % cols] = 0x7F80          # ... under a +inf elsewhere in the row
    say(f"argmax: every value as winner, {2 * n} rows x {cols}")
    want = _check_matrix(m, split, calls=1)
    rec_v = want.view(x.TOP2_REC)
    assert np.array_equal(np.asarray(rec_v["top1"][:n]).view(np.uint32) >> 16, pats)
    assert np.array_equal(np.asarray(rec_v["top2"][n:]).view(np.uint32) >> 16, pats)
