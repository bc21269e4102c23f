"""Chunk checks for the exhaustive E4M3FN sweeps in test_oracle_fp8.py, in a
module of their own so that worker processes can import them without torch.

A chunk is a range [start, end) of fp32 bit patterns of positive values, in
increasing order of value.  The encoding is monotone there, so it is fully
described by the codes' step positions: `first_bits_above_code[c]` is the
first pattern whose code exceeds c."""
from __future__ import annotations

import numpy as np


def expected_steps(thresholds: np.ndarray, start: int, end: int):
    """(code of pattern `start`, patterns in (start, end) where the code steps up)."""
    first = int(np.searchsorted(thresholds, start, side="right"))
    steps = thresholds[(thresholds > start) & (thresholds < end)]
    return first, steps


def observed_steps(codes: np.ndarray, start: int):
    """(code of the first pattern, patterns where the code changes)."""
    changes = np.flatnonzero(codes[1:] != codes[:-1]) + 1 + start
    return int(codes[0]), changes


def oracle_chunk_ok(args) -> bool:
    """The oracle's encoder on every pattern of [start, end) against the
    thresholds.  Run in a worker process."""
    start, end, thresholds = args
    import oracle as O
    bits = np.arange(start, end, dtype=np.int64).astype(np.uint32)
    codes = O.e4m3_encode(bits.view(np.float32))
    got_first, got_steps = observed_steps(codes, start)
    want_first, want_steps = expected_steps(np.asarray(thresholds, dtype=np.int64), start, end)
    return got_first == want_first and np.array_equal(got_steps, want_steps)
