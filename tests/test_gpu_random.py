"""Seeded random shapes against the float64 oracle: decode or prefill (shared cache), separate
or aliased K/V, bf16 or fp32, head counts around the 16-head block sizes, small and odd cache
sizes, kmax above and below n_ctx, unsorted indices with duplicates, ragged per-row counts
(garbage past each count), sinks of -inf, and scales other than 1/sqrt(512). The oracle checks
a few sampled rows of every case, always including the first and the last.
"""
import sys

import numpy as np
import pytest

import workloads as w
from parity import BF16_TOL, F32_TOL, assert_parity, run_gpu, run_oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
HEADS = [1, 2, 3, 7, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 127, 128]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def random_case(seed: int) -> w.AttnCase:
    rng = np.random.default_rng(10_000 + seed)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    shared = rng.random() < 0.35
    alias = rng.random() < 0.3
    heads = int(rng.choice(HEADS))
    n_ctx = int(rng.choice([1, 5, 63, 64, 65])) if rng.random() < 0.35 else int(rng.integers(100, 3001))
    rows = int(rng.integers(1, 300 if shared else 24))
    kmax = int(rng.choice([1, 64, 65, 640])) if rng.random() < 0.4 else int(rng.integers(1, 801))
    normal = w._normal_bf16 if dtype == "bf16" else w._normal
    q = normal(rng, (rows, heads, w.D))
    caches = 1 if shared else rows
    k = normal(rng, (caches, n_ctx, w.D))
    v = k if alias else normal(rng, (caches, n_ctx, w.D))
    sinks = rng.standard_normal(heads).astype(np.float32)
    if rng.random() < 0.25:
        sinks[rng.integers(0, heads)] = -np.inf
    idx = rng.integers(0, n_ctx, size=(rows, kmax)).astype(np.int32)   # unsorted, with duplicates
    nsel = rng.integers(0, kmax + 1, size=rows).astype(np.int32)
    for r in range(rows):                                                 # past the count: never read
        idx[r, nsel[r]:] = rng.choice([-1, n_ctx, 2 ** 30])
    scale = w.SCALE if rng.random() < 0.6 else float(rng.uniform(0.01, 0.2))
    name = (f"random{seed} {dtype} {'prefill' if shared else 'decode'}{' aliased' if alias else ''} "
            f"R={rows} H={heads} N={n_ctx} kmax={kmax}")
    return w.AttnCase(name, dtype, q, k, v, idx, nsel, sinks, scale, shared)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_against_oracle(seed):
    case = random_case(seed)
    say(case.name)
    got = run_gpu(case, DEV)
    rows = sorted({0, case.rows // 3, case.rows // 2, case.rows - 1})
    ref = run_oracle(case, rows=rows)
    tol = BF16_TOL if case.dtype == "bf16" else F32_TOL
    st = assert_parity(got[rows], ref[rows], *tol, case.name)
    say(f"  ok {st}")
