"""GPU parity of the aliased-cache path: k_cache and v_cache are the same tensor (one
latent serving as keys and values), so each selected row is gathered once.

The aliased kernel runs the separate-cache kernel's arithmetic in the same order, so
on equal contents the two paths must agree bit for bit; both are also checked against
the float64 oracle evaluated with V = K.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as w
from parity import BF16_TOL, assert_parity, run_oracle, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def aliased(case):
    """V = K in the host case (the oracle then evaluates the same definition)."""
    case.v = case.k
    return case


def alias_and_separate(case):
    """Run the aliased path and the separate path on a copy of the same cache."""
    import sparse_attention_attn_amd as sa
    d = to_device(case, DEV)
    kk = d["k"]
    vv = kk.clone()
    fn = sa.prefill if case.shared_cache else sa.decode
    a = fn(d["q"], kk, kk, d["idx"], d["sinks"], case.scale, d["nsel"])
    s = fn(d["q"], kk, vv, d["idx"], d["sinks"], case.scale, d["nsel"])
    torch.cuda.synchronize()
    return a, s


@pytest.mark.parametrize("batch,heads,k", [
    (1, 64, 640),      # one unit, column slices of 64
    (8, 64, 640),
    (100, 64, 640),    # column slices of 128
    (300, 64, 640),    # more units than CUs: several units per workgroup
    (5, 16, 130),      # one head block, 16 real heads of 32
    (40, 32, 65),      # ragged tail tile
    (260, 48, 640),    # two head blocks, the second part-filled
    (60, 16, 640),     # persistent kernels, one 16-head group: score blocks shared by the waves
    (30, 32, 130),     # persistent kernels, two 16-head groups: the same
])
def test_alias_bits_equal_separate_and_oracle(batch, heads, k):
    case = aliased(w.decode_bf16(seed=80 + batch + heads, batch=batch, heads=heads,
                                 n_ctx=max(2 * k, 700), k=k, name="alias"))
    say(f"alias vs separate B={batch} H={heads} k={k}")
    a, s = alias_and_separate(case)
    assert torch.equal(a.view(torch.int32), s.view(torch.int32))
    rows = sorted({0, batch // 2, batch - 1})
    ref = run_oracle(case, rows=rows)
    st = assert_parity(a.cpu().numpy()[rows], ref[rows], *BF16_TOL, "alias")
    say(f"  ok {st}")


def test_alias_short_units_counts_and_bad_indices():
    """600 rows of at most one tile each, so a workgroup streams three units and the
    index lists it resolves run up to two units ahead; zero counts, a one-key row and
    out-of-range indices (inside the count: NaN row; beyond it: ignored) are mixed in."""
    rng = np.random.default_rng(90)
    case = aliased(w.decode_bf16(seed=90, batch=600, heads=64, n_ctx=200, k=50, name="alias short"))
    case.nsel[:] = rng.integers(0, 51, size=600).astype(np.int32)
    case.nsel[[0, 256, 512]] = [0, 1, 50]
    bad_rows = [3, 259, 515, 516, 599]
    for r in bad_rows:
        case.nsel[r] = max(case.nsel[r], 5)
        case.idx[r, case.nsel[r] - 1] = 200 + r  # out of range, inside the count
    case.idx[10, case.nsel[10]:] = 10_000_000    # out of range, beyond the count
    say("alias: 600 short rows, zero counts, out-of-range indices")
    a, s = alias_and_separate(case)
    assert torch.equal(a.view(torch.int32), s.view(torch.int32))
    got = a.cpu().numpy()
    nan_rows = [r for r in range(600) if np.isnan(got[r]).all()]
    assert nan_rows == bad_rows, nan_rows
    rows = [0, 1, 2, 4, 10, 255, 256, 257, 258, 260, 511, 512, 513, 514, 517, 598]
    ref = run_oracle(case, rows=rows)
    st = assert_parity(got[rows], ref[rows], *BF16_TOL, "alias short rows")
    say(f"  ok {st}")


def test_alias_prefill_shared_cache():
    """Prefill rows over one shared aliased cache."""
    case = aliased(w.prefill_bf16(seed=91, rows=48, first_pos=1000, heads=64, n_ctx=1100, k=640, row_stride=2))
    say("alias prefill 48 rows")
    a, s = alias_and_separate(case)
    assert torch.equal(a.view(torch.int32), s.view(torch.int32))
    rows = [0, 23, 47]
    ref = run_oracle(case, rows=rows)
    assert_parity(a.cpu().numpy()[rows], ref[rows], *BF16_TOL, "alias prefill")


def test_alias_nonfinite_rows():
    """Indexer top-k then decode on caches where about 1% of rows carry +inf/-inf/NaN,
    with the latent serving as both K and V."""
    import oracle
    import sparse_attention_attn_amd as sa
    scores, case, _, _ = w.indexer_then_decode(batch=4, n_ctx=8192)
    case = aliased(case)
    idx, cnt = oracle.topk(scores, 640)
    case.idx[:] = idx
    case.nsel[:] = cnt
    say("alias nonfinite rows")
    a, s = alias_and_separate(case)
    assert torch.equal(a.view(torch.int32), s.view(torch.int32))
    st = assert_parity(a.cpu().numpy(), run_oracle(case), *BF16_TOL, "alias nonfinite")
    say(f"  ok {st}")


def test_alias_determinism_and_guards():
    import sparse_attention_attn_amd as sa
    case = aliased(w.decode_bf16(seed=92, batch=3, heads=64, n_ctx=3000, k=640))
    d = to_device(case, DEV)
    n = case.rows * case.heads * w.D
    guard = 4096
    say("alias determinism x3 with guard regions")
    outs = []
    for _ in range(3):
        buf = torch.full((guard + n + guard,), 12345.0, dtype=torch.float32, device=DEV)
        out = buf[guard:guard + n].view(case.rows, case.heads, w.D)
        sa.decode(d["q"], d["k"], d["k"], d["idx"], d["sinks"], case.scale, d["nsel"], out=out)
        torch.cuda.synchronize()
        assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + n:] == 12345.0)
        outs.append(out.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


def test_alias_sustained_sampled():
    """The benchmarked shape with one cache as K and V: 1,024 sequences x 4,096 positions,
    64 heads, k = 640, device inputs; the oracle checks 12 sampled rows."""
    import sparse_attention_attn_amd as sa
    say("alias sustained decode B=1024 (device inputs, 12 sampled rows)")
    inp = w.device_decode_inputs(torch, DEV, batch=1024, heads=64, n_ctx=4096, k=640, seed=8)
    inp["v"] = inp["k"]
    out = sa.decode(inp["q"], inp["k"], inp["k"], inp["idx"], inp["sinks"], w.SCALE)
    torch.cuda.synchronize()
    for r in [0, 1, 255, 256, 511, 512, 767, 768, 1000, 1021, 1022, 1023]:
        case = w.host_case_from_device(inp, r)
        ref = run_oracle(case)
        assert_parity(out[r:r + 1].cpu().numpy(), ref, *BF16_TOL, f"alias sustained row {r}")
    del inp
    torch.cuda.empty_cache()


def test_alias_masked_slots_read_zeros_after_nonfinite_tile():
    """As for the separate path: row 0 (two tiles, both buffers) selects rows with +inf in
    column 7; row 256, on the same workgroup next, has 5 keys, and its tile reuses a buffer
    row 0 filled. The masked slots must read as zeros."""
    c = aliased(w.decode_bf16(seed=97, batch=300, heads=64, n_ctx=256, k=128, name="alias masked after inf"))
    c.k[0][c.idx[0, :128], 7] = 0x7F80
    c.nsel[256] = 5
    say("alias masked slots after an inf tile")
    a, s = alias_and_separate(c)
    assert torch.equal(a.view(torch.int32), s.view(torch.int32))
    rows = [0, 1, 256, 257, 299]
    ref = run_oracle(c, rows=rows)
    got = a.cpu().numpy()
    assert_parity(got[rows], ref[rows], *BF16_TOL, "alias masked after inf")
    assert np.isfinite(got[256]).all()
