"""The oracle and the input generator reproduce the stored tiny fp32 snapshot exactly."""
import os

import numpy as np

import oracle
import workloads as w

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_f32_oracle.txt")


def test_tiny_f32_snapshot():
    lines = [l.split() for l in open(GOLDEN) if not l.startswith("#")]
    c = w.tiny_f32()
    assert [int(x) for x in lines[0][1:]] == c.idx[0].tolist()
    assert [float(x) for x in lines[1][1:]] == c.sinks.astype(np.float64).tolist()
    o = oracle.attention(c.dtype, c.q, c.k, c.v, c.idx, c.nsel, c.sinks, c.scale, c.shared_cache)
    for h, row in enumerate(lines[2:]):
        assert int(row[1]) == h and float(row[3]) == float(o[0, h].sum())
        for item in row[4:]:
            j, val = item.split(":")
            assert float(val) == float(o[0, h, int(j)])
