"""Write tests/golden/tiny_f32_oracle.txt: the oracle's output on the tiny fp32 workload.

Calls only oracle/ and the seeded input generator. The fixture is a regression
snapshot of the oracle and the generator together (1 row, 4 heads, head width
512, 256 cached positions, k = 64, seed 0): if either one changes its
arithmetic or its draw order, tests/test_golden.py fails.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402
import workloads as w  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_f32_oracle.txt")
COLS = (0, 1, 31, 32, 255, 256, 480, 511)


def main():
    c = w.tiny_f32()
    o = oracle.attention(c.dtype, c.q, c.k, c.v, c.idx, c.nsel, c.sinks, c.scale, c.shared_cache)
    with open(OUT, "w") as f:
        f.write("# oracle output on the tiny fp32 workload (seed 0); written by make_golden.py\n")
        f.write("idx " + " ".join(str(int(x)) for x in c.idx[0]) + "\n")
        f.write("sinks " + " ".join(repr(float(x)) for x in c.sinks) + "\n")
        for h in range(c.heads):
            f.write(f"head {h} sum {float(o[0, h].sum())!r} " +
                    " ".join(f"{j}:{float(o[0, h, j])!r}" for j in COLS) + "\n")
    print(OUT)


if __name__ == "__main__":
    main()
