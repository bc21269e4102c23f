"""Write fp8_thresholds.json from the CPU oracle alone.

For each positive E4M3FN code c in 0..125, find by bisection over positive
fp32 bit patterns the smallest pattern that the oracle encodes to a code
greater than c.  Encoding is monotone in the bit pattern of a positive float,
so these 126 patterns describe the whole positive half of the encoder.

Run from the repository root:  python tests/golden/make_fp8_thresholds.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def code_of_bits(bits):
    b = np.asarray(bits, dtype=np.uint64).astype(np.uint32)
    return oracle.e4m3_encode(b.view(np.float32)).astype(np.int64)


def thresholds():
    lo = np.zeros(126, dtype=np.int64)                 # encodes to <= c
    hi = np.full(126, 0x43E00000, dtype=np.int64)      # bits of 448.0 -> code 126
    c = np.arange(126)
    while np.any(hi - lo > 1):
        mid = (lo + hi) // 2
        above = code_of_bits(mid) > c
        hi = np.where(above, mid, hi)
        lo = np.where(above, lo, mid)
    return hi


def main():
    th = thresholds()
    out = {
        "_source": "Written by tests/golden/make_fp8_thresholds.py from the CPU oracle's "
                   "E4M3FN encoder (round to nearest even, saturating at 448).",
        "first_bits_above_code": [int(x) for x in th],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_thresholds.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
