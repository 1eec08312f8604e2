"""Writes nf4_code_thresholds.txt from the CPU oracle alone.

For each i in 0..14 it finds, by bisection over the ordered binary32 values in
[-1, 1], the smallest normalised value n whose oracle code is at least i+1.
The file is what the exhaustive GPU test compares the kernel's code function
against. Run: python tests/golden/make_code_thresholds.py
"""
import os
import struct
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402


def ordinal(x):
    b = struct.unpack("<I", struct.pack("<f", x))[0]
    return b if b < 0x80000000 else -(b & 0x7FFFFFFF)


def from_ordinal(o):
    b = o if o >= 0 else (0x80000000 | (-o))
    return struct.unpack("<f", struct.pack("<I", b))[0]


def thresholds():
    lo0, hi0 = ordinal(-1.0), ordinal(1.0)
    out = []
    for i in range(15):
        lo, hi = lo0, hi0  # code(lo) <= i, code(hi) >= i+1
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if oracle.nearest_code(from_ordinal(mid)) >= i + 1:
                hi = mid
            else:
                lo = mid
        out.append(from_ordinal(hi))
    return out


def main():
    path = os.path.join(HERE, "nf4_code_thresholds.txt")
    with open(path, "w") as f:
        f.write("# Smallest binary32 n in [-1, 1] whose NF4 code is >= i+1, i = 0..14,\n")
        f.write("# found by bisection with the CPU oracle's nearest-level function\n")
        f.write("# (written by make_code_thresholds.py; do not edit by hand).\n")
        f.write("# columns: i | bits (hex) | value\n")
        for i, t in enumerate(thresholds()):
            bits = struct.unpack("<I", struct.pack("<f", t))[0]
            f.write(f"{i} | 0x{bits:08x} | {t!r}\n")
    print(path)


if __name__ == "__main__":
    main()
