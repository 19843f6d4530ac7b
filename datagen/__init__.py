"""Seeded synthetic inputs for the transfer staging/combine path.

Shared by the oracle's tests, the GPU parity tests and ``bench.py``.  Nothing
here performs a step of the method under test (no BF16 rounding, no sum, no
argmax fold, no run encoding, no copy by address table): it only draws
numbers and lays out addresses.  The arithmetic lives in ``datagen.c``.

Workload shapes follow the pages:
  * hidden size 5120 and prompt batches of 512 / 2048 tokens: the large
    all-reduce page (llama.cpp copy-engine all-reduce, "Results");
  * vocabulary 129280 split at column 64768: the two-card drafter page
    ("Layout", head row);
  * 1000 blocks x 288 slots x 2 segments x 4 KiB: the run-encoded transfer
    page ("Problem").
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdatagen.so")

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, S, U64, U32, D, F, I = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint64,
                                   ctypes.c_uint32, ctypes.c_double, ctypes.c_float, ctypes.c_int)
        L.dg_bytes.argtypes = [P, S, U64]
        L.dg_u64.argtypes = [P, S, U64]
        L.dg_normal_f32.argtypes = [P, S, U64, D]
        L.dg_outliers_f32.argtypes = [P, S, U64, S, F]
        L.dg_outliers_f32.restype = I
        L.dg_bf16_normal_trunc.argtypes = [P, S, U64, D, D]
        L.dg_perm_u32.argtypes = [P, U32, U64]
        L.dg_choose_u32.argtypes = [P, U32, U32, U64]
        L.dg_choose_u32.restype = I
        L.dg_kv_src_addrs.argtypes = [P, U32, U32, U64, P, U32, P]
        L.dg_kv_src_addrs.restype = I
        L.dg_kv_dst_addrs.argtypes = [P, U32, U32, U64, U64, U64]
        L.dg_tag_segments.argtypes = [P, U64, U64, P, U32, U32, U64, U64]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def seed_for(config: int, rank: int = 0, label: int = 0) -> int:
    """Seed of sub-stream ``label`` of rank ``rank`` in workload ``config``."""
    return 0x5EED0000 + config + (rank << 8) + (label << 16)


# ---------------------------------------------------------------- raw draws

def random_bytes(n: int, seed: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint8)
    if n:
        lib().dg_bytes(_ptr(out), n, seed)
    return out


def fill_bytes(buf: np.ndarray, seed: int) -> None:
    """Fills a contiguous numpy buffer in place with generator bytes."""
    assert buf.flags.c_contiguous
    if buf.nbytes:
        lib().dg_bytes(_ptr(buf), buf.nbytes, seed)


def random_u64(n: int, seed: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    if n:
        lib().dg_u64(_ptr(out), n, seed)
    return out


def normal_f32(n: int, seed: int, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    if n:
        lib().dg_normal_f32(_ptr(out), n, seed, sigma)
    return out


def permutation(n: int, seed: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    if n:
        lib().dg_perm_u32(_ptr(out), n, seed)
    return out


def choose(count: int, n: int, seed: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint32)
    if lib().dg_choose_u32(_ptr(out), count, n, seed) != 0:
        raise ValueError("cannot choose that many")
    return out


# ------------------------------------------------ pack / combine workloads

# Hand-picked F32 input pairs (bit patterns) for the tiny combine workload:
# round-to-nearest-even ties in both directions, values just off a tie,
# overflow to infinity, subnormals, signed zeros, infinities and NaNs of
# several payloads and signs.  Inputs only: expected outputs are derived in
# the tests from exact rational arithmetic.
EDGE_PAIRS = [
    (0x3F808000, 0x00000000),  # tie, rounds down to even
    (0x3F818000, 0x80000000),  # tie, rounds up to even; plus -0
    (0x3F808001, 0x3F807FFF),  # just above / below a tie; sum is a BF16 tie
    (0x7F7FFFFF, 0x3F800000),  # FLT_MAX rounds to +inf
    (0x7F7F8000, 0xFF7F7FFF),  # tie at the BF16 maximum
    (0x7F7F7FFF, 0x7F7F7FFF),  # BF16 max + BF16 max overflows F32
    (0x00000001, 0x80000001),  # smallest subnormals round to +0 / -0
    (0x00010000, 0x00010000),  # smallest BF16 subnormal twice
    (0x00018000, 0x80008000),  # subnormal ties
    (0x007FFFFF, 0x807F0000),  # largest F32 subnormal rounds up to min normal
    (0x7F800000, 0xFF800000),  # +inf + -inf
    (0x7F800000, 0x3F800000),  # inf + finite
    (0x7FC00000, 0x3F800000),  # quiet NaN + finite
    (0x7F800001, 0x00000000),  # NaN with the lowest payload bit only
    (0xFFFFFFFF, 0xBF800000),  # all-ones NaN
    (0x80000000, 0x80000000),  # -0 + -0
    (0x40490FDB, 0xC0490FDB),  # x + (-x)
    (0x4B800000, 0x3F800000),  # 2^24 + 1
    (0x3F800000, 0x3B800000),  # 1 + 2^-8: sum is a BF16 tie, even below
    (0x3F810000, 0x3B800000),  # sum is a BF16 tie, even above
    (0x7F7F0000, 0x7B000000),  # finite F32 sum whose BF16 rounding overflows
    (0x00400000, 0x00400000),  # two subnormals summing to the min normal
    (0x47800000, 0xC77F0000),  # cancellation
    (0x42C80000, 0xC2C80000),  # outlier-scale cancellation
    (0x80000001, 0x80000001),  # both round to -0
    (0x00000000, 0x00000000),  # +0 + +0
    (0x7F7F0000, 0xFF7F0000),  # max - max
    (0xFF800000, 0xFF800000),  # -inf + -inf
    (0x7FC00000, 0x7F800000),  # NaN + inf
    (0xFFC00000, 0x7FC00000),  # negative NaN + positive NaN
    (0xBF808000, 0xBF818000),  # negative ties
    (0x3F7FFFFF, 0x3F7FFFFF),  # rounds up across a binade
]

TINY_N = 5120


def edge_positions() -> np.ndarray:
    """Positions p_k = 80 k + (k mod 8), k = 0..63, of the planted pairs."""
    k = np.arange(64)
    return (80 * k + (k % 8)).astype(np.int64)


def tiny_pair(seed0: int | None = None, seed1: int | None = None):
    """Two F32[5120] partials ~ N(0, 1) with the 32 edge pairs planted at
    positions p_0..p_31 as (a, b) and swapped at p_32..p_63."""
    a = normal_f32(TINY_N, seed_for(1, 0) if seed0 is None else seed0, 1.0)
    b = normal_f32(TINY_N, seed_for(1, 1) if seed1 is None else seed1, 1.0)
    ab, bb = a.view(np.uint32), b.view(np.uint32)
    pos = edge_positions()
    for k, (x, y) in enumerate(EDGE_PAIRS):
        ab[pos[k]], bb[pos[k]] = x, y
        ab[pos[32 + k]], bb[pos[32 + k]] = y, x
    return a, b


def prompt_partial(n: int, seed: int, sigma: float = 0.5, outlier_frac: float = 0.01,
                   factor: float = 50.0) -> np.ndarray:
    """F32[n] ~ N(0, sigma^2) with exactly n*outlier_frac distinct positions
    (rounded down) multiplied by ``factor``."""
    x = normal_f32(n, seed, sigma)
    count = int(n * outlier_frac)
    if count:
        if lib().dg_outliers_f32(_ptr(x), n, seed ^ 0xA5A5A5A5, count, factor) != 0:
            raise MemoryError("outlier placement failed")
    return x


# ------------------------------------------------------- argmax workload

VOCAB = 129280
SPLIT = 64768


@dataclass
class ArgmaxInput:
    logits: np.ndarray          # uint16 BF16 bits [rows, cols]
    split: int                  # first column of shard 1
    tie_rows: np.ndarray        # rows with a planted cross-shard tie
    tie_cols: np.ndarray        # [len(tie_rows), 2] the tied columns


def argmax_logits(rows: int, seed: int, cols: int = VOCAB, split: int = SPLIT, sigma: float = 3.0,
                  tie_frac: float = 0.05) -> ArgmaxInput:
    """BF16 logits of N(0, sigma^2) deviates (clamped to +-8 sigma and
    truncated to BF16).  max(1, round(tie_frac * rows)) rows get an exact tie
    across the shard boundary at a value above every drawn value: half of
    them (the even-numbered ones) at columns (split-1, split), the others at
    one random column of each shard."""
    x = np.empty(rows * cols, dtype=np.uint16)
    clamp = 8.0 * sigma
    if x.size:
        lib().dg_bf16_normal_trunc(_ptr(x), x.size, seed, sigma, clamp)
    x = x.reshape(rows, cols)
    n_tie = max(1, int(round(tie_frac * rows))) if rows else 0
    n_tie = min(n_tie, rows)
    tie_rows = choose(n_tie, rows, seed ^ 0x7E1E) if n_tie else np.empty(0, np.uint32)
    picks = random_u64(2 * n_tie, seed ^ 0xC01)
    # A value above the clamp: the smallest power of two above it, which is
    # exactly representable in BF16.
    tie_val = np.float32(2.0 ** int(np.ceil(np.log2(clamp * 1.01))))
    tie_bits = np.uint16(tie_val.view(np.uint32) >> 16)
    tie_cols = np.empty((n_tie, 2), dtype=np.int64)
    for k, r in enumerate(tie_rows):
        if k % 2 == 0:
            p0, p1 = split - 1, split
        else:
            p0 = int(picks[2 * k] % split)
            p1 = split + int(picks[2 * k + 1] % (cols - split))
        x[r, p0] = tie_bits
        x[r, p1] = tie_bits
        tie_cols[k] = (p0, p1)
    return ArgmaxInput(x, split, tie_rows.astype(np.int64), tie_cols)


def argmax_hand_rows(cols: int = VOCAB, split: int = SPLIT) -> np.ndarray:
    """Hand-made rows (BF16 bits) for the argmax edge cases:
      0 tie at columns (split-1, split) above everything else
      1 every element equal
      2 maximum only at column 0
      3 maximum only at the last column
      4 +inf maximum in shard 1
      5 all elements <= 0, maximum +0 at one column and -0 at an earlier one
      6 all elements <= 0, maximum -0 only
      7 -inf everywhere except one -1 in shard 1
      8 two equal maxima inside shard 1 only
      9 top1 in shard 1, top2 in shard 0 (the margin crosses the boundary)
    """
    base = np.full(cols, 0xBF80, dtype=np.uint16)  # -1.0
    rows = []
    r = base.copy(); r[split - 1] = r[split] = 0x4000; rows.append(r)
    rows.append(np.full(cols, 0x3F80, dtype=np.uint16))
    r = base.copy(); r[0] = 0x4120; rows.append(r)
    r = base.copy(); r[cols - 1] = 0x4120; rows.append(r)
    r = base.copy(); r[split + 7] = 0x7F80; r[3] = 0x7F7F; rows.append(r)
    r = base.copy(); r[split + 11] = 0x0000; r[17] = 0x8000; rows.append(r)
    r = base.copy(); r[split + 5] = 0x8000; rows.append(r)
    r = np.full(cols, 0xFF80, dtype=np.uint16); r[cols - 2] = 0xBF80; rows.append(r)
    r = base.copy(); r[split + 100] = r[split + 50] = 0x4300; rows.append(r)
    r = base.copy(); r[split + 3] = 0x4300; r[split - 2] = 0x42FE; rows.append(r)
    return np.stack(rows)


# ---------------------------------------------- paged K/V transfer layout

N_BLOCKS = 1000
N_SLOTS = 288
SEG_BYTES = 4096
DST_SLOT_STRIDE = 12288


def kv_src_addrs(n_blocks: int, n_slots: int, seg_bytes: int, region_bases, pos=None) -> np.ndarray:
    """Lane-major source addresses [2*n_slots, n_blocks] (see datagen.c)."""
    n_lanes = 2 * n_slots
    out = np.empty(n_lanes * n_blocks, dtype=np.uint64)
    rb = np.asarray(region_bases, dtype=np.uint64)
    p = None if pos is None else np.ascontiguousarray(pos, dtype=np.uint32)
    rc = lib().dg_kv_src_addrs(_ptr(out), n_blocks, n_slots, seg_bytes, _ptr(rb), len(rb),
                               None if p is None else _ptr(p))
    if rc:
        raise ValueError("slots do not split evenly over the regions")
    return out.reshape(n_lanes, n_blocks)


def kv_dst_addrs(n_blocks: int, n_slots: int, seg_bytes: int, base: int, slot_stride: int) -> np.ndarray:
    n_lanes = 2 * n_slots
    out = np.empty(n_lanes * n_blocks, dtype=np.uint64)
    lib().dg_kv_dst_addrs(_ptr(out), n_blocks, n_slots, seg_bytes, base, slot_stride)
    return out.reshape(n_lanes, n_blocks)


def region_bytes_for(n_blocks: int, n_slots: int, seg_bytes: int, n_regions: int = 2) -> int:
    return n_blocks * (n_slots // n_regions) * 2 * seg_bytes


def fill_region(host: np.ndarray, dev_base: int, addrs: np.ndarray, seg_bytes: int, seed: int) -> None:
    """Generator bytes over the whole region image, then a tag per segment."""
    fill_bytes(host, seed)
    a = np.ascontiguousarray(addrs, dtype=np.uint64)
    n_lanes, n_blocks = a.shape
    lib().dg_tag_segments(_ptr(host), dev_base, host.nbytes, _ptr(a), n_lanes, n_blocks, seg_bytes,
                          seed)
