"""GPU parity of the float32 path (sa_attn_f32.hip: one workgroup per row and 16-head group,
both products on v_mfma_f32_16x16x4_f32) against the float64 oracle, within the float32 bound:
|gpu - oracle| <= 1e-5 on finite elements, equal nonfinite classes."""
import sys

import numpy as np
import pytest
import torch

import workloads as w
from parity import F32_TOL, assert_parity, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    import sparse_attention_attn_amd as sa
    sa.load()


def check(case, rows=None, label=None):
    say(f"{label or case.name}: B={case.rows} H={case.heads} N={case.n_ctx} kmax={case.kmax} f32")
    got = run_gpu(case, DEV)
    ref = run_oracle(case, rows=rows)
    sel = slice(None) if rows is None else list(rows)
    st = assert_parity(got[sel], ref[sel], *F32_TOL, label or case.name)
    say(f"  ok {st}")
    return got, ref


def test_batched_decode_32k():
    """The batched decode shape in float32: 8 sequences of 32,768 positions, 64 heads, k = 640."""
    check(w.decode_f32(seed=6, batch=8, heads=64, n_ctx=32768, k=640), label="f32 batched 8 x 32K")


@pytest.mark.parametrize("heads", [1, 4, 16, 17, 48, 64, 100, 128])
def test_head_counts(heads):
    c = w.decode_f32(seed=600 + heads, batch=2, heads=heads, n_ctx=900, k=200)
    check(c, label=f"f32 H={heads}")


@pytest.mark.parametrize("k", [1, 31, 32, 33, 63, 64, 65, 639, 641])
def test_tile_boundaries(k):
    """32-key tiles: counts around 32 and 64, and ragged tails."""
    check(w.decode_f32(seed=700 + k, batch=2, heads=64, n_ctx=1500, k=k), label=f"f32 k={k}")


def test_ragged_counts_and_empty_row():
    c = w.decode_f32(seed=710, batch=4, heads=64, n_ctx=800, k=300)
    c.nsel[:] = [300, 137, 0, 33]
    c.idx[1, 137:] = -1
    c.idx[2, :] = -1
    c.idx[3, 33:] = -1
    got, _ = check(c, label="f32 nsel {300,137,0,33}")
    assert np.all(got[2] == 0)


def test_out_of_range_index_gives_nan_row():
    c = w.decode_f32(seed=711, batch=3, heads=64, n_ctx=500, k=100)
    c.idx[1, 50] = 500
    c.idx[2, 99] = -7
    got, _ = check(c, label="f32 out-of-range")
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2])) and np.all(np.isfinite(got[0]))


@pytest.mark.parametrize("which,val", [("k", np.nan), ("k", np.inf), ("k", -np.inf),
                                       ("v", np.nan), ("v", np.inf), ("v", -np.inf)])
def test_nonfinite_planted(which, val):
    c = w.decode_f32(seed=712, batch=2, heads=64, n_ctx=256, k=130)
    arr = c.k if which == "k" else c.v
    arr[0, c.idx[0, 70], 123] = val
    got, ref = check(c, label=f"f32 planted {which}={val}")
    assert not np.all(np.isfinite(ref[0]))


def test_nonfinite_sinks_and_far_scores():
    c = w.decode_f32(seed=713, batch=2, heads=64, n_ctx=300, k=130)
    c.sinks[3], c.sinks[5], c.sinks[7] = np.inf, -np.inf, np.nan
    got, _ = check(c, label="f32 nonfinite sinks")
    assert np.all(np.isnan(got[:, 3])) and np.all(np.isnan(got[:, 7])) and np.all(np.isfinite(got[:, 5]))
    c = w.decode_f32(seed=714, batch=2, heads=32, n_ctx=300, k=130)
    c.q[:] = 1.0
    c.k[:] = -0.5
    c.scale = 1.0
    c.sinks[:16] = -np.inf
    got, _ = check(c, label="f32 sink -inf, scores -256")
    assert np.all(np.isfinite(got))


def test_repeats_are_identical():
    import sparse_attention_attn_amd as sa
    c = w.decode_f32(seed=715, batch=3, heads=64, n_ctx=3000, k=640)
    d = to_device(c, DEV)
    outs = [sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"]) for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


@pytest.mark.parametrize("rows,heads,n_ctx,kmax", [(18, 65, 1, 452), (4, 16, 5, 788), (3, 64, 2, 1000), (20, 64, 3, 640)])
def test_heavily_duplicated_selections(rows, heads, n_ctx, kmax):
    """Hundreds of entries drawn from a cache of one to five positions (duplicates are summed):
    many equal weights, so the value sum's rounding must not grow with the number of entries.
    Both float32 paths: the split path (4 rows of 16 heads, 3 rows of 64) and attn_f32_kernel."""
    rng = np.random.default_rng(600 + n_ctx)
    q = w._normal(rng, (rows, heads, w.D))
    k = w._normal(rng, (rows, n_ctx, w.D))
    v = w._normal(rng, (rows, n_ctx, w.D))
    sinks = rng.standard_normal(heads).astype(np.float32)
    idx = rng.integers(0, n_ctx, size=(rows, kmax)).astype(np.int32)
    nsel = np.full(rows, kmax, dtype=np.int32)
    nsel[-1] = kmax // 2 + 1
    idx[-1, nsel[-1]:] = -1
    case = w.AttnCase(f"f32 duplicates R={rows} H={heads} N={n_ctx} kmax={kmax}", "f32", q, k, v, idx, nsel, sinks,
                      w.SCALE, False)
    check(case)
