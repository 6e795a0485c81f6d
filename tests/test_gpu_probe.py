"""sparse_attn_gather_probe (measurement only): the decode kernels' K and V gathers with no
compute and no output. It must run for both rows-in-flight settings over index lists that are
ragged (not a multiple of a workgroup's entries) and hold masked (-1) and out-of-range entries,
and it must leave every input as it was."""
import sys

import pytest
import torch

import workloads as w
from parity import to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("rif", [8, 16])
def test_probe_runs_and_reads_only(rif):
    import sparse_attention_attn_amd as sa
    c = w.decode_bf16(seed=340 + rif, batch=5, heads=64, n_ctx=1000, k=130)
    c.idx[1, 3] = -1
    c.idx[2, 7] = 1000            # out of range: reads nothing
    c.idx[3, 0] = 2 ** 31 - 1     # far out of range: reads nothing
    c.idx[4, 60:] = -1
    d = to_device(c, DEV)
    before = {key: d[key].clone() for key in ("k", "v", "idx")}
    say(f"gather probe rif={rif}: 5 rows, n_ctx 1000, kmax 130")
    for _ in range(3):
        sa.gather_probe(d["k"], d["v"], d["idx"], rif)
    torch.cuda.synchronize()
    for key, t in before.items():
        assert torch.equal(d[key], t), f"the probe changed {key}"
