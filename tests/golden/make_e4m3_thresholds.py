"""Write e4m3_thresholds.txt: for each code c = 1..126, the smallest positive
fp32 bit pattern whose oracle cast is >= c.  The cast is monotone in |x|, so
these 126 patterns describe the oracle's cast on every non-negative fp32 value
up to 448 (expected code = number of thresholds <= the pattern).

Calls only the oracle:  python tests/golden/make_e4m3_thresholds.py
"""

import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import e4m3  # noqa: E402

TOP = int(np.array([448.0], np.float32).view(np.uint32)[0])


def code_of(bits: int) -> int:
    return int(e4m3.encode(np.array([bits], np.uint32).view(np.float32))[0])


def first_at_least(c: int) -> int:
    lo, hi = 0, TOP            # code_of(hi) = 126 >= c
    while lo < hi:
        mid = (lo + hi) // 2
        if code_of(mid) >= c:
            hi = mid
        else:
            lo = mid + 1
    return lo


def main():
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "e4m3_thresholds.txt")
    with open(out, "w") as f:
        f.write("# code  first fp32 bit pattern cast to it (oracle cast; written by make_e4m3_thresholds.py)\n")
        for c in range(1, 127):
            f.write("%3d 0x%08x\n" % (c, first_at_least(c)))
    print(out)


if __name__ == "__main__":
    main()
