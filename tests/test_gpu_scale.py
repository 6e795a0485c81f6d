"""GPU parity at softmax scales other than 1/sqrt(512).

The caller passes the scale that multiplies q.k (not the sinks). These cases take it to the
corners of the online softmax:
* 0: every score is 0, so every selected key weighs the same against the sink;
* -1/sqrt(512): the order of the weights is reversed;
* 1e-30: the scaled scores sit far below 1 but stay normal floats, so the weights are equal to
  within rounding;
* 0.25 and 1.0 (bf16 only): sharp weights. The exponent reference moves in most tiles, and one key
  carries nearly all the weight. Float32 storage stops at the first three: at these scales the
  float32 score sums' own conditioning exceeds the 1e-5 bar.

Each case runs a launch that takes the persistent kernel, compares sampled rows with the float64
oracle, and checks that the first two rows, launched alone (the split path), give the same bits.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as w
from parity import BF16_TOL, F32_TOL, assert_parity, run_oracle, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

BF16_SCALES = [0.0, -w.SCALE, 1e-30, 0.25, 1.0]
F32_SCALES = [0.0, -w.SCALE, 1e-30]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    import sparse_attention_attn_amd as sa
    sa.load()  # fails loudly if the HIP library is missing


def run_both(c, rows_full, tol, label):
    """The persistent launch (all rows) against the oracle on sampled rows, and rows 0..1 alone
    (the split path) against the same rows of it, bit for bit."""
    import sparse_attention_attn_amd as sa
    d = to_device(c, DEV)
    say(f"{label}: B={c.rows} H={c.heads} N={c.n_ctx} kmax={c.kmax} scale={c.scale!r}")
    full = sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"])
    part = sa.decode(d["q"][:2], d["k"][:2], d["v"][:2], d["idx"][:2], d["sinks"], c.scale, d["nsel"][:2])
    torch.cuda.synchronize()
    assert torch.equal(part.view(torch.int32), full[:2].view(torch.int32)), f"{label}: split path bits differ"
    ref = run_oracle(c, rows=rows_full)
    st = assert_parity(full.cpu().numpy()[rows_full], ref[rows_full], *tol, label)
    say(f"  ok {st}")
    return full


@pytest.mark.parametrize("alias", [False, True])
@pytest.mark.parametrize("scale", BF16_SCALES)
def test_bf16_scales(scale, alias):
    # 26 rows at 64 heads take the persistent kernel; 2 rows take the split path.
    c = w.decode_bf16(seed=1200 + BF16_SCALES.index(scale), batch=26, heads=64, n_ctx=1000, k=300)
    c.scale = float(scale)
    if alias:
        c.v = c.k
    out = run_both(c, [0, 1, 13, 25], BF16_TOL, f"bf16 scale {scale!r}{' aliased' if alias else ''}")
    assert np.all(np.isfinite(out.cpu().numpy()))


@pytest.mark.parametrize("scale", F32_SCALES)
def test_f32_scales(scale):
    # 20 rows at 64 heads take attn_f32_kernel; 2 rows with k = 200 take the float32 split path.
    c = w.decode_f32(seed=1300 + F32_SCALES.index(scale), batch=20, heads=64, n_ctx=600, k=200)
    c.scale = float(scale)
    out = run_both(c, [0, 1, 10, 19], F32_TOL, f"f32 scale {scale!r}")
    assert np.all(np.isfinite(out.cpu().numpy()))


def test_zero_scale_is_the_mean_against_the_sink():
    """At scale 0 every selected key weighs exp(0) = 1 against exp(sink): out = sum(v) / (n + e^sink).
    A closed form, checked on the GPU output directly (float64 on the host)."""
    import sparse_attention_attn_amd as sa
    c = w.decode_bf16(seed=1250, batch=3, heads=64, n_ctx=700, k=200)
    c.scale = 0.0
    d = to_device(c, DEV)
    out = sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], 0.0, d["nsel"])
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    v = w.bf16_to_f32(c.v).astype(np.float64)
    for r in range(c.rows):
        n = int(c.nsel[r])
        vs = v[r, c.idx[r, :n]].sum(axis=0)                     # [512]
        den = n + np.exp(c.sinks.astype(np.float64))              # [H]
        want = vs[None, :] / den[:, None]
        np.testing.assert_allclose(got[r], want, rtol=0, atol=BF16_TOL[0], err_msg=f"row {r}")
