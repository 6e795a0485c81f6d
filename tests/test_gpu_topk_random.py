"""Seeded random top-k cases, bit-exact against the oracle, across every launch shape: rows of
up to 4,096 (eight-wave rows when there are at most four rows per CU, four-wave rows beyond),
up to 16,384 and 32,768 (register kernels: sixteen waves per row when there is at most one row
per CU) and longer (the radix kernel); k below and above the
valid length; per-row valid lengths; N(0,1) scores, scores rounded to a coarse grid (many ties
at the threshold), and rows with planted +-0, NaN and +-inf.
"""
import sys

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def random_topk_case(seed: int):
    rng = np.random.default_rng(20_000 + seed)
    n = int(rng.choice([1, 63, 64, 65, 640, 4096, 4097, 16384, 16385, 32768, 40000, int(rng.integers(2, 5000))]))
    rows = int(rng.choice([1, 3, 37, 1024, 1025, 2048])) if n <= 4096 else int(rng.integers(1, 40))
    # The first seeds pin the launch-shape boundaries: the radix kernel (rows past 32,768), at
    # most vs more than four rows per CU (eight-wave vs four-wave rows) for rows of up to 4,096,
    # and at most vs more than one row per CU (sixteen-wave rows vs four- or eight-wave rows) for
    # rows of up to 16,384 and 32,768.
    n, rows = {0: (40000, 5), 1: (4096, 1024), 2: (4096, 1025), 3: (32769, 3), 4: (16384, 300),
               5: (32768, 257), 6: (16385, 256), 7: (4097, 2)}.get(seed, (n, rows))
    k = int(rng.choice([1, 2, 64, 640, 2048, int(rng.integers(1, n + 2))]))
    ld = n + int(rng.choice([0, 0, 3]))
    s = rng.standard_normal((rows, ld)).astype(np.float32)
    kind = rng.integers(0, 3)
    if kind == 1:
        s = np.round(s * 4) / 4                         # heavy ties
    elif kind == 2:
        for r in range(rows):
            for val in (0.0, -0.0, np.nan, np.inf, -np.inf):
                s[r, rng.integers(0, ld, size=3)] = val
    valid = None if rng.random() < 0.5 else rng.integers(0, n + 1, size=rows).astype(np.int32)
    return s, n, k, valid, f"seed {seed}: rows={rows} n={n} ld={ld} k={k} kind={kind} valid={'yes' if valid is not None else 'no'}"


@pytest.mark.parametrize("seed", range(20))
def test_random_topk_bit_exact(seed):
    import sparse_attention_attn_amd as sa
    s, n, k, valid, label = random_topk_case(seed)
    say(label)
    sd = torch.from_numpy(s).to(DEV)
    vl = None if valid is None else torch.from_numpy(valid).to(DEV)
    idx = torch.empty((s.shape[0], k), dtype=torch.int32, device=DEV)
    cnt = torch.empty((s.shape[0],), dtype=torch.int32, device=DEV)
    # a row of ld > n: the call sees only the first n columns of each row
    lib = sa.load()
    rc = lib.sparse_attn_topk(sd.data_ptr(), s.shape[0], n, s.shape[1], None if vl is None else vl.data_ptr(), k,
                              idx.data_ptr(), cnt.data_ptr(), None, 0, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    ref_i, ref_c = oracle.topk(np.ascontiguousarray(s[:, :n]), k, valid)
    np.testing.assert_array_equal(cnt.cpu().numpy(), ref_c)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_i)
