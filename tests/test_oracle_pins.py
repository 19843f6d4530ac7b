"""Pins of the CPU oracle against what the pages and the mathematics fix.

No pin here re-types the oracle's own formula: each uses a different
formulation (integer carry form, exact rationals, binary64 closed form),
a library routine (torch / numpy), an invariant, a printed page figure, or
brute force on tiny inputs.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import datagen as dg
import oracle
from tests import exact

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ------------------------------------------------------------- exhaustive

@pytest.fixture(scope="module")
def exhaustive_bin(tmp_path_factory):
    d = tmp_path_factory.mktemp("pins")
    exe = str(d / "exhaustive")
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-pthread", "-o", exe,
                           os.path.join(ROOT, "tests", "pins", "exhaustive.c"),
                           os.path.join(ROOT, "oracle", "liboracle.so"),
                           "-Wl,-rpath," + os.path.join(ROOT, "oracle"), "-lm"])
    return exe


@pytest.mark.parametrize("what", ["rne", "sum", "comm"])
def test_exhaustive(exhaustive_bin, what):
    """rne: all 2^32 F32 patterns vs the carry form; sum: all 2^32 BF16 pairs
    vs the binary64 closed form; comm: commutativity over all pairs."""
    threads = str(min(8, os.cpu_count() or 1))
    r = subprocess.run([exhaustive_bin, what, threads], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout


# ---------------------------------------------------------------- BF16 RNE

def _edge_inputs():
    xs = set()
    for a, b in dg.EDGE_PAIRS:
        xs.add(a)
        xs.add(b)
    return sorted(xs)


def test_rne_exact_rationals_edge_values():
    for bits in _edge_inputs():
        assert oracle.bf16_rne_scalar(bits) == exact.rne_bf16_of_f32_bits(bits), hex(bits)


def test_rne_exact_rationals_ties_and_random():
    rng = dg.random_u64(4000, 0x1234)
    cands = []
    for v in rng:
        v = int(v) & 0xFFFFFFFF
        cands.append(v)
        cands.append((v & 0xFFFF0000) | 0x8000)        # exact tie
        cands.append((v & 0xFFFF0000) | 0x7FFF)        # just below a tie
        cands.append((v & 0xFFFF0000) | 0x8001)        # just above a tie
        cands.append(v & 0x807FFFFF)                   # subnormal / zero exponent
        cands.append((v & 0x80FFFFFF) | 0x7F000000)    # top binade
    for bits in cands:
        assert oracle.bf16_rne_scalar(bits) == exact.rne_bf16_of_f32_bits(bits), hex(bits)


def test_rne_special_values():
    # Readings: infinities kept; every NaN canonical 0x7FC0 (sign dropped);
    # zero and subnormals keep their sign; no flush.
    assert oracle.bf16_rne_scalar(0x7F800000) == 0x7F80
    assert oracle.bf16_rne_scalar(0xFF800000) == 0xFF80
    for nan in (0x7F800001, 0x7FC00000, 0xFFC00000, 0xFFFFFFFF, 0x7FBFFFFF, 0xFF800001):
        assert oracle.bf16_rne_scalar(nan) == 0x7FC0
    assert oracle.bf16_rne_scalar(0x80000000) == 0x8000
    assert oracle.bf16_rne_scalar(0x00000000) == 0x0000
    assert oracle.bf16_rne_scalar(0x00010000) == 0x0001     # smallest BF16 subnormal kept
    assert oracle.bf16_rne_scalar(0x80008000) == 0x8000     # tie between -0 and -min: even is -0
    assert oracle.bf16_rne_scalar(0x00018000) == 0x0002     # tie between 1 and 2 quanta: even is 2
    assert oracle.bf16_rne_scalar(0x7F7FFFFF) == 0x7F80     # FLT_MAX overflows
    assert oracle.bf16_rne_scalar(0x7F7F7FFF) == 0x7F7F     # just below the overflow midpoint
    assert oracle.bf16_rne_scalar(0x7F7F8000) == 0x7F80     # the midpoint itself: even is inf


def test_rne_matches_torch_on_random_patterns():
    """torch's CPU float->bfloat16 conversion is round-to-nearest-even; it
    disagrees only on NaN encodings, which are excluded."""
    bits = dg.random_u64(1 << 21, 0xBF16).astype(np.uint64)
    u = np.concatenate([(bits & 0xFFFFFFFF).astype(np.uint32),
                        (bits >> 32).astype(np.uint32) & np.uint32(0x807FFFFF)])  # + subnormals
    u = u[(u & 0x7FFFFFFF) <= 0x7F800000]
    ours = oracle.bf16_rne(u)
    t = torch.from_numpy(u.view(np.float32).copy()).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours, t.view(np.uint16))


# -------------------------------------------------------------------- pack

def test_pack_streaming_equals_bulk_equals_elementwise():
    ce = 64
    n = 5 * ce + 13                      # ragged tail chunk
    src = dg.normal_f32(n, 77, 2.0)
    n_chunks = -(-n // ce)
    bulk = oracle.pack(src, n_chunks * ce, ce, 0, n_chunks)
    # streaming: two alternating slots, one chunk per call
    ring = np.zeros(2 * ce, dtype=np.uint16)
    got = []
    for c in range(n_chunks):
        oracle.pack(src, 2 * ce, ce, c, c + 1, ring=ring)
        ln = min(ce, n - c * ce)
        got.append(ring[(c % 2) * ce:(c % 2) * ce + ln].copy())
    streamed = np.concatenate(got)
    # three slots, two chunks per call
    ring3 = np.zeros(3 * ce, dtype=np.uint16)
    got3 = []
    for c0 in range(0, n_chunks, 2):
        c1 = min(n_chunks, c0 + 2)
        oracle.pack(src, 3 * ce, ce, c0, c1, ring=ring3)
        for c in range(c0, c1):
            ln = min(ce, n - c * ce)
            got3.append(ring3[(c % 3) * ce:(c % 3) * ce + ln].copy())
    t = torch.from_numpy(src).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bulk[:n], t)
    assert np.array_equal(streamed, t)
    assert np.array_equal(np.concatenate(got3), t)


def test_pack_leaves_ring_beyond_tail_untouched():
    ce = 32
    src = dg.normal_f32(ce + 5, 3, 1.0)
    ring = np.full(2 * ce, 0xDEAD, dtype=np.uint16)
    oracle.pack(src, 2 * ce, ce, 1, 2, ring=ring)
    assert np.all(ring[:ce] == 0xDEAD)
    assert np.all(ring[ce + 5:] == 0xDEAD)
    assert not np.any(ring[ce:ce + 5] == 0xDEAD)


def test_pack_refuses_aliasing_ranges():
    src = np.zeros(100, dtype=np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.pack(src, 2 * 16, 16, 0, 3)        # three chunks into two slots
    with pytest.raises(oracle.OracleError):
        oracle.pack(src, 2 * 16, 16, 7, 8)        # chunk 7 starts past n


# ----------------------------------------------------------------- combine

def test_combine_edge_pairs_exact_rationals():
    a, b = dg.tiny_pair()
    pos = dg.edge_positions()
    ab = oracle.bf16_rne(a.view(np.uint32))
    bb = oracle.bf16_rne(b.view(np.uint32))
    f32 = oracle.combine2(ab, bb, 0)
    b16 = oracle.combine2(ab, bb, 1)
    for p in pos:
        x, y = int(ab[p]), int(bb[p])
        assert int(f32[p]) == exact.f32_bits_of_exact_sum_rounded(x, y), (p, hex(x), hex(y))
        assert int(b16[p]) == exact.rne_bf16_of_f32_bits(int(f32[p]))
        # one rounding of the exact sum gives the same BF16 (no double-rounding harm)
        assert int(b16[p]) == exact.bf16_bits_of_exact_sum(x, y), (p, hex(x), hex(y))


def test_combine_bf16_mode_is_the_correctly_rounded_exact_sum():
    w = dg.random_u64(3000, 0xC0B1)
    pairs = []
    for v in w:
        v = int(v)
        a, b = v & 0xFFFF, (v >> 16) & 0xFFFF
        pairs.append((a, b))
        # near-equal magnitudes and close exponents: where cancellation and ties live
        pairs.append((a, (a ^ 0x8000) + ((v >> 40) & 7) - 3 & 0xFFFF))
        pairs.append((a, ((a & 0xFF80) - 0x0400 * ((v >> 50) & 7) | (v >> 33) & 0x7F) & 0xFFFF))
    for a, b in pairs:
        if ((a & 0x7FFF) > 0x7F80) or ((b & 0x7FFF) > 0x7F80):
            continue
        assert int(oracle.combine2(np.array([a], np.uint16), np.array([b], np.uint16), 1)[0]) == \
            exact.bf16_bits_of_exact_sum(a, b), (hex(a), hex(b))


def test_combine_f32_matches_numpy_and_identities():
    w = dg.random_u64(1 << 18, 0x5A5A)
    a = (w & 0xFFFF).astype(np.uint16)
    b = ((w >> 16) & 0xFFFF).astype(np.uint16)
    keep = ((a & 0x7FFF) <= 0x7F80) & ((b & 0x7FFF) <= 0x7F80)
    a, b = a[keep], b[keep]
    fa = (a.astype(np.uint32) << 16).view(np.float32)
    fb = (b.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(all="ignore"):
        ref = (fa + fb).view(np.uint32).copy()
    nan = (ref & 0x7FFFFFFF) > 0x7F800000
    ref[nan] = 0x7FC00000
    assert np.array_equal(oracle.combine2(a, b, 0), ref)
    # x + (-0) == x for every non-NaN x (identity); the sign rules of zero sums
    xs = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    xs = xs[(xs & 0x7FFF) <= 0x7F80]
    negz = np.full(xs.size, 0x8000, np.uint16)
    assert np.array_equal(oracle.combine2(xs, negz, 0), xs.astype(np.uint32) << 16)
    assert oracle.sum2_f32_scalar(0x0000, 0x8000) == 0x00000000
    assert oracle.sum2_f32_scalar(0x8000, 0x8000) == 0x80000000
    assert oracle.sum2_f32_scalar(0x7F80, 0xFF80) == 0x7FC00000


# ---------------------------------------------------- F32-wire combine ([TP2])

def _f32_wire_pairs():
    """Structured F32 pairs: special values, ties of the binary32 grid,
    overflow, subnormal sums and cancellation, and random pairs of close
    exponents (where rounding happens)."""
    special = [0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001, 0xFFC12345,
               0x3F800000, 0xBF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00000001, 0x80000001, 0x00800000,
               0x807FFFFF, 0x007FFFFF, 0x33800000, 0xB3800000]
    pairs = [(x, y) for x in special for y in special]
    pairs += [
        (0x3F800000, 0x33800000),   # 1 + 2^-24: a tie, stays at the even 1
        (0x3F800001, 0x33800000),   # (1 + 2^-23) + 2^-24: a tie, goes up to the even 1 + 2^-22
        (0x3F800000, 0x33800001),   # just above the tie: rounds up
        (0x7F7FFFFF, 0x73000000),   # FLT_MAX + half its ulp: tie at the top, rounds to infinity
        (0x7F7FFFFF, 0x72FFFFFF),   # just below: stays FLT_MAX
        (0x00400000, 0x00400000),   # two subnormals sum to the smallest normal
        (0x00800001, 0x80800000),   # normal - normal = smallest subnormal
    ]
    w = dg.random_u64(12000, 0xF32F32)
    for v in w:
        v = int(v)
        a = v & 0xFFFFFFFF
        e = (a >> 23) & 0xFF
        de = (v >> 32) % 40
        e2 = max(0, min(254, e - de if (v >> 40) & 1 else e + de))
        b = ((v >> 41) & 1) << 31 | e2 << 23 | ((v >> 42) * 0x9E3779B1) & 0x7FFFFF
        pairs.append((a, b))
    return pairs


def test_f32_wire_sum_exact_rationals():
    pairs = _f32_wire_pairs()
    a = np.array([p[0] for p in pairs], np.uint32)
    b = np.array([p[1] for p in pairs], np.uint32)
    got = oracle.combine2_f32(a, b, 0)
    got16 = oracle.combine2_f32(a, b, 1)
    for i, (x, y) in enumerate(pairs):
        want = exact.f32_bits_of_exact_f32_sum(x, y)
        assert int(got[i]) == want, (hex(x), hex(y), hex(int(got[i])), hex(want))
        # the page's order: the F32 sum first, then its BF16 rounding
        assert int(got16[i]) == exact.rne_bf16_of_f32_bits(want), (hex(x), hex(y))


def test_f32_wire_rounds_twice_as_the_page_orders():
    """fp32 sum, then BF16: 1 + 2^-8 + 2^-30 is 1 + 2^-8 in binary32, a BF16
    tie that goes to the even 1.0; one rounding of the exact sum would give
    the next BF16 value up."""
    a, b = 0x3F808000, 0x30800000
    assert oracle.sum2_f32_f32_scalar(a, b) == 0x3F808000
    assert int(oracle.combine2_f32(np.array([a], np.uint32), np.array([b], np.uint32), 1)[0]) == 0x3F80


def test_f32_wire_matches_numpy_and_commutes():
    w = dg.random_u64(1 << 20, 0xF32A)
    a = (w & 0xFFFFFFFF).astype(np.uint32)
    b = (w >> 32).astype(np.uint32)
    with np.errstate(all="ignore"):
        ref = (a.view(np.float32) + b.view(np.float32)).view(np.uint32).copy()
    ref[(ref & 0x7FFFFFFF) > 0x7F800000] = 0x7FC00000
    assert np.array_equal(oracle.combine2_f32(a, b, 0), ref)
    assert np.array_equal(oracle.combine2_f32(b, a, 0), ref)


# ------------------------------------------------------------------ argmax

def _brute_top2(vals_bits):
    """Sort the whole row by (value descending, id ascending)."""
    v = [(float((np.uint32(x) << np.uint32(16)).view(np.float32)), i, int(x)) for i, x in enumerate(vals_bits)]
    order = sorted(v, key=lambda t: (-t[0], t[1]))
    return order[0], order[1]


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_argmax_brute_force_tiny(seed):
    w = dg.random_u64(64 * 40, seed)
    # values from a tiny alphabet so ties (inside a shard and across) are common
    alphabet = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0x7F80, 0xFF80, 0x3F81], np.uint16)
    x = alphabet[(w % alphabet.size).astype(np.int64)].reshape(64, 40)
    for split in (1, 17, 39):
        for mode in (0, 1):
            out = oracle.argmax_merge(x, split, mode)
            for r in range(x.shape[0]):
                t1, t2 = _brute_top2(x[r])
                if mode == 0:
                    assert out[r]["idx"] == t1[1]
                    assert out[r]["max"].view(np.uint32) == np.uint32(t1[2]) << 16
                else:
                    assert out[r]["idx"] == t1[1]
                    assert out[r]["top1"].view(np.uint32) == np.uint32(t1[2]) << 16
                    assert out[r]["top2"].view(np.uint32) == np.uint32(t2[2]) << 16


def test_argmax_full_rows_match_numpy():
    inp = dg.argmax_logits(16, dg.seed_for(3))
    x = inp.logits
    vals = (x.astype(np.uint32) << 16).view(np.float32)
    o1 = oracle.argmax_merge(x, dg.SPLIT, 1)
    o0 = oracle.argmax_merge(x, dg.SPLIT, 0)
    assert np.array_equal(o0["idx"], np.argmax(vals, axis=1))          # first occurrence
    assert np.array_equal(o1["idx"], o0["idx"])
    assert np.array_equal(o0["max"], vals.max(axis=1))
    srt = np.sort(vals, axis=1)
    assert np.array_equal(o1["top2"], srt[:, -2])                       # multiset second
    for k, r in enumerate(inp.tie_rows):
        assert o0[r]["idx"] == inp.tie_cols[k][0]                      # lower id wins
        assert o1[r]["top2"] == o1[r]["top1"]


def test_argmax_hand_rows():
    x = dg.argmax_hand_rows()
    s = dg.SPLIT
    o = oracle.argmax_merge(x, s, 1)
    b = lambda f: np.float32(f)
    assert o[0]["idx"] == s - 1 and o[0]["top1"] == 2.0 and o[0]["top2"] == 2.0
    assert o[1]["idx"] == 0 and o[1]["top1"] == 1.0 and o[1]["top2"] == 1.0
    assert o[2]["idx"] == 0 and o[2]["top1"] == 10.0 and o[2]["top2"] == -1.0
    assert o[3]["idx"] == dg.VOCAB - 1 and o[3]["top1"] == 10.0
    assert o[4]["idx"] == s + 7 and np.isinf(o[4]["top1"]) and o[4]["top2"] == b(3.3895314e38)
    # +0 at s+11 and -0 at 17: equal values, the lower id (17, the -0) wins
    assert o[5]["idx"] == 17 and o[5]["top1"].view(np.uint32) == 0x80000000
    assert o[5]["top2"].view(np.uint32) == 0x00000000
    assert o[6]["idx"] == s + 5 and o[6]["top1"].view(np.uint32) == 0x80000000 and o[6]["top2"] == -1.0
    assert o[7]["idx"] == dg.VOCAB - 2 and o[7]["top1"] == -1.0 and np.isneginf(o[7]["top2"])
    assert o[8]["idx"] == s + 50 and o[8]["top1"] == 128.0 and o[8]["top2"] == 128.0
    assert o[9]["idx"] == s + 3 and o[9]["top1"] == 128.0 and o[9]["top2"] == 127.0


def test_argmax_nan_is_refused():
    x = np.zeros((2, 10), np.uint16)
    x[1, 7] = 0x7FC1
    with pytest.raises(oracle.OracleError) as e:
        oracle.argmax_merge(x, 5, 0)
    assert e.value.code == oracle.ENAN


# -------------------------------------------------------------- run tables

def _geometry():
    g = {}
    with open(os.path.join(ROOT, "tests", "golden", "page_geometry.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0] if line.startswith("#") else line
            if "=" not in line:
                continue
            k, rest = line.split("=", 1)
            g[k.strip()] = float(rest.split("|", 1)[0])
    return g


def test_page_geometry_vocab_and_set():
    g = _geometry()
    assert dg.VOCAB == g["vocab_cols"] and dg.SPLIT == g["shard0_cols"]
    assert dg.SPLIT == 256 * g["shard0_tiles_of_256"]
    assert dg.VOCAB - dg.SPLIT == 256 * g["shard1_tiles_of_256"]
    assert dg.N_BLOCKS == g["kv_blocks"] and dg.N_SLOTS == g["kv_slots"]
    assert dg.N_BLOCKS * dg.N_SLOTS * 2 == g["kv_segments"]
    assert dg.SEG_BYTES == g["kv_segment_bytes"]
    assert dg.N_BLOCKS * dg.N_SLOTS * 2 * dg.SEG_BYTES == g["kv_set_mib"] * 2**20
    assert dg.region_bytes_for(dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES) == g["numa_region_mib"] * 2**20
    # 32 MiB splits of the two dense per-region groups: 2 * ceil(1125 / 32) descriptors
    assert 2 * -(-g["numa_region_mib"] // g["read_split_mib"]) == g["descs_4k"]
    # the 64 KiB shape: 200 blocks, 7200 MiB per set, 115,200 segments, 2 * ceil(3600 / 32)
    s64 = int(g["descs_64k_blocks"]) * dg.N_SLOTS * 2
    assert s64 == g["descs_64k_before"]
    assert s64 * 65536 == g["descs_64k_set_mib"] * 2**20
    assert 2 * -(-(g["descs_64k_set_mib"] / 2) // g["read_split_mib"]) == g["descs_64k"]
    # p4 payloads: 5..20 rows x 5120 fp32 = 100..400 KB (decimal, rounded)
    assert round(g["p4_rows_min"] * g["p4_hidden"] * 4 / 1024) == g["p4_kb_min"]
    assert round(g["p4_rows_max"] * g["p4_hidden"] * 4 / 1024) == g["p4_kb_max"]


def test_dense_layout_encodes_to_one_run_per_lane():
    """A fully bump-allocated holder collapses every lane to one run; the
    table is ~13 KB against ~4.6 MB for one address per segment."""
    g = _geometry()
    rb = dg.region_bytes_for(dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES)
    bases = [0x7F0000000000, 0x7F0000000000 + 2 * rb]
    a = dg.kv_src_addrs(dg.N_BLOCKS, dg.N_SLOTS, dg.SEG_BYTES, bases)
    t = oracle.runs_encode(a)
    assert t.n_lanes == 576 and t.n_runs == 576
    assert np.all(t.run_count == 1000) and np.all(t.runs_per_lane == 1)
    assert np.all(t.run_stride == dg.N_SLOTS // 2 * 2 * dg.SEG_BYTES)       # 1,179,648
    table_bytes = t.n_runs * (8 + 8 + 4) + t.n_lanes * 4
    assert round(table_bytes / 1024) == 13 or round(table_bytes / 1000) == 14
    assert abs(table_bytes / 1000 - g["new_response_kb"]) < 1.0
    assert round(a.size * 8 / 1e6, 1) == g["old_response_mb"]
    assert np.array_equal(oracle.runs_decode(t), a)


def test_shuffled_layout_round_trips_and_bounds_runs():
    B = dg.N_BLOCKS
    perm = dg.permutation(B, dg.seed_for(5, 0, 1))
    rb = dg.region_bytes_for(B, dg.N_SLOTS, dg.SEG_BYTES)
    a = dg.kv_src_addrs(B, dg.N_SLOTS, dg.SEG_BYTES, [1 << 40, (1 << 40) + rb], pos=perm)
    t = oracle.runs_encode(a)
    # every run but a lane's last has >= 2 addresses (distinct addresses)
    assert np.all(t.runs_per_lane <= -(-B // 2))
    assert t.n_runs > 576 * 300
    assert np.array_equal(oracle.runs_decode(t), a)


def test_runs_round_trip_random_and_adversarial():
    w = dg.random_u64(4 * 50, 99).reshape(4, 50)
    cases = [
        w,                                                              # random 64-bit addresses
        np.tile(np.arange(50, dtype=np.uint64) * np.uint64(16), (4, 1)),  # ascending
        np.tile((np.arange(50, dtype=np.uint64)[::-1] * np.uint64(32)).copy(), (4, 1)),  # descending
        np.full((4, 50), 4096, dtype=np.uint64),                       # repeated address
        np.tile(np.array([0, 2**63 + 16, 32, 2**64 - 16] * 12 + [0, 16], dtype=np.uint64), (4, 1)),
    ]
    for a in cases:
        t = oracle.runs_encode(a)
        assert np.array_equal(oracle.runs_decode(t), a)


def test_greedy_encoding_worked_example():
    # deltas: +16 +16 +32 -48 -48 -48 0 +16
    a = np.array([[100, 116, 132, 164, 116, 68, 20, 20, 36]], dtype=np.uint64)
    t = oracle.runs_encode(a)
    assert t.run_base.tolist() == [100, 164, 20]
    assert t.run_stride.tolist() == [16, -48, 16]
    assert t.run_count.tolist() == [3, 4, 2]


def test_decode_refuses_inconsistent_tables():
    good = oracle.RunTable([1, 2], [0, 64, 128], [16, 16, 16], [4, 2, 2], 4)
    assert oracle.runs_decode(good).shape == (2, 4)
    bad = [
        oracle.RunTable([1, 2], [0, 64, 128], [16, 16, 16], [4, 0, 4], 4),       # zero count
        oracle.RunTable([1, 2], [0, 64, 128], [16, 16, 16], [4, 2, 1], 4),       # lane 1 short
        oracle.RunTable([1, 2], [0, 64, 128], [16, 16, 16], [4, 3, 2], 4),       # lane 1 over
        oracle.RunTable([1, 1], [0, 64, 128], [16, 16, 16], [4, 4, 2], 4),       # n_runs mismatch
        oracle.RunTable([1, 1], [2**64 - 32, 0], [16, 16], [4, 4], 4),           # wraps past 2^64
        oracle.RunTable([1, 1], [32, 0], [-16, 16], [4, 4], 4),                  # below 0
    ]
    for t in bad:
        with pytest.raises(oracle.OracleError):
            oracle.runs_decode(t)


def _tiny_world(seed, n_blocks=5, n_slots=3, seg=64, shuffle=True):
    rb = dg.region_bytes_for(n_blocks, n_slots, seg, n_regions=1)
    base = 0x10000
    pos = dg.permutation(n_blocks, seed) if shuffle else None
    a = dg.kv_src_addrs(n_blocks, n_slots, seg, [base], pos=pos)
    host = np.empty(rb, dtype=np.uint8)
    dg.fill_region(host, base, a, seg, seed)
    return a, [(base, host)], seg


def _brute_gather(a, regions, seg):
    n_lanes, n_blocks = a.shape
    out = np.empty(n_lanes * n_blocks * seg, dtype=np.uint8)
    for b in range(n_blocks):
        for l in range(n_lanes):
            addr = int(a[l, b])
            for base, host in regions:
                if base <= addr and addr + seg <= base + host.nbytes:
                    o = (b * n_lanes + l) * seg
                    out[o:o + seg] = host[addr - base:addr - base + seg]
                    break
            else:
                raise AssertionError("address outside regions")
    return out


def _split_runs(t: oracle.RunTable, seed: int) -> oracle.RunTable:
    """Split runs at random points: the same address set, another encoding."""
    w = dg.random_u64(t.n_runs + 1, seed)
    rpl, base, stride, count = [], [], [], []
    r = 0
    for l in range(t.n_lanes):
        k = 0
        for _ in range(int(t.runs_per_lane[l])):
            c = int(t.run_count[r])
            cut = int(w[r] % c) if c > 1 else 0
            pieces = [(0, cut), (cut, c)] if cut else [(0, c)]
            for lo, hi in pieces:
                base.append((int(t.run_base[r]) + lo * int(t.run_stride[r])) % 2**64)
                stride.append(int(t.run_stride[r]) if hi - lo > 1 else 0)
                count.append(hi - lo)
                k += 1
            r += 1
        rpl.append(k)
    return oracle.RunTable(rpl, base, stride, count, t.n_blocks)


def _per_segment(a) -> oracle.RunTable:
    n_lanes, n_blocks = a.shape
    return oracle.RunTable([n_blocks] * n_lanes, a.reshape(-1), np.zeros(a.size, np.int64),
                           np.ones(a.size, np.uint32), n_blocks)


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_gather_brute_force_and_encoding_invariance(seed):
    a, regions, seg = _tiny_world(seed)
    ref = _brute_gather(a, regions, seg)
    t = oracle.runs_encode(a)
    for table in (t, _split_runs(t, seed), _per_segment(a)):
        assert np.array_equal(oracle.gather(table, seg, regions), ref)


@pytest.mark.parametrize("seed", [21, 22])
def test_scatter_places_every_segment_and_nothing_else(seed):
    a, regions, seg = _tiny_world(seed, n_blocks=6, n_slots=4)
    staging = oracle.gather(oracle.runs_encode(a), seg, regions)
    n_lanes, n_blocks = a.shape
    stride = 3 * seg                                           # K, V, one gap segment per slot
    dbase = 0x900000
    d = dg.kv_dst_addrs(n_blocks, n_lanes // 2, seg, dbase, stride)
    dst = np.full(n_blocks * (n_lanes // 2) * stride, 0xA5, dtype=np.uint8)
    oracle.scatter(oracle.runs_encode(d), seg, [(dbase, dst)], staging)
    written = np.zeros(dst.size, bool)
    for l in range(n_lanes):
        for b in range(n_blocks):
            o = int(d[l, b]) - dbase
            s = (b * n_lanes + l) * seg
            assert np.array_equal(dst[o:o + seg], staging[s:s + seg])
            # the tag names the source segment
            tag = dst[o:o + 16].view(np.uint32)
            assert tag[0] == 0x5E6D7A61 and tag[1] == l and tag[2] == b
            written[o:o + seg] = True
    assert np.all(dst[~written] == 0xA5)


def test_gather_refuses_addresses_outside_regions():
    a, regions, seg = _tiny_world(5)
    t = oracle.runs_encode(a)
    base, host = regions[0]
    with pytest.raises(oracle.OracleError) as e:
        oracle.gather(t, seg, [(base, host[:-seg])])
    assert e.value.code == oracle.ERANGE
