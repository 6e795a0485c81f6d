"""The float32 split path for small batches (sa_attn_f32_split.hip: the scores of every 32-key
tile in their own workgroup, then the softmax and values per head group and column slice)
against attn_f32_kernel (sa_attn_f32.hip) and the float64 oracle.

A float32 launch with fewer than 24 rows per block of 64 heads and index lists of 129 to 1,024
entries takes the split path. The same rows padded with empty rows (nsel = 0, which read
nothing) to 24 per head block take attn_f32_kernel. Every real row must come out bit for bit
the same both ways, and within the float32 bound of the oracle: the split changes where the
work runs, never its arithmetic (the ds4 commit log for ds4_tp.c: a split that follows the
launch must not change the output bytes).
"""
import sys

import numpy as np
import pytest
import torch

import workloads as w
from parity import F32_TOL, assert_parity, run_oracle, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    import sparse_attention_attn_amd as sa
    sa.load()


def split_and_whole(case, alias=False):
    """(split output, attn_f32_kernel output) of the case's rows, both float32 host arrays."""
    import sparse_attention_attn_amd as sa
    from sparse_attention_attn_amd import _lib as L
    d = to_device(case, DEV)
    if alias:
        d["v"] = d["k"]
    rows, H = case.rows, case.heads
    n_hb = (H + 63) // 64
    assert rows * n_hb < 24 and 128 < case.kmax <= 1024, "not a split-path launch"
    fn = sa.prefill if case.shared_cache else sa.decode
    split = fn(d["q"], d["k"], d["v"], d["idx"], d["sinks"], case.scale, d["nsel"])
    P = 24 * n_hb
    op = L.SA_OP_PREFILL if case.shared_cache else L.SA_OP_DECODE
    assert sa.workspace_bytes(op, P, H, case.kmax, case.n_ctx) == 0, "not the whole-row path"
    q = torch.zeros((P, H, 512), dtype=d["q"].dtype, device=DEV)
    q[:rows] = d["q"]
    idx = torch.full((P, case.kmax), -1, dtype=torch.int32, device=DEV)
    idx[:rows] = d["idx"]
    nsel = torch.zeros((P,), dtype=torch.int32, device=DEV)
    nsel[:rows] = d["nsel"]
    if case.shared_cache:
        kc, vc = d["k"], d["v"]
    else:
        # Rows past the real ones select nothing, so their caches are never read.
        kc = torch.empty((P, case.n_ctx, 512), dtype=d["k"].dtype, device=DEV)
        kc[:rows] = d["k"]
        vc = kc if alias else torch.empty_like(kc)
        if not alias:
            vc[:rows] = d["v"]
    whole = fn(q, kc, vc, idx, d["sinks"], case.scale, nsel)
    torch.cuda.synchronize()
    out = split.cpu().numpy(), whole[:rows].cpu().numpy()
    del kc, vc, whole
    torch.cuda.empty_cache()
    return out


def check_both(case, label, alias=False, oracle_rows=None):
    say(f"{label}: B={case.rows} H={case.heads} N={case.n_ctx} kmax={case.kmax} f32{' aliased' if alias else ''}")
    split, whole = split_and_whole(case, alias)
    assert np.array_equal(split.view(np.int32), whole.view(np.int32)), f"{label}: split path differs"
    if alias:
        case.v = case.k
    ref = run_oracle(case, rows=oracle_rows)
    sel = slice(None) if oracle_rows is None else list(oracle_rows)
    st = assert_parity(split[sel], ref[sel], *F32_TOL, label)
    say(f"  ok (bit-equal to attn_f32_kernel) {st}")
    return split, ref


def test_batched_decode_32k():
    """The batched decode shape in float32: 8 sequences of 32,768 positions, 64 heads, k = 640."""
    check_both(w.decode_f32(seed=6, batch=8, heads=64, n_ctx=32768, k=640), "f32 split 8 x 32K")


@pytest.mark.parametrize("heads", [1, 16, 17, 48, 64, 100, 128])
def test_head_counts_ragged(heads):
    """Head counts off the 16-head groups and the 64-head blocks, with a full, an empty and a
    partial row (a masked tail)."""
    c = w.decode_f32(seed=800 + heads, batch=3, heads=heads, n_ctx=1000, k=300)
    c.nsel[:] = [300, 0, 161]
    c.idx[1, :] = -1
    c.idx[2, 161:] = -1
    got, _ = check_both(c, f"f32 split H={heads} nsel {{300,0,161}}")
    assert np.all(got[1] == 0)


@pytest.mark.parametrize("k", [129, 383, 384, 385, 640, 767, 1000, 1024])
def test_index_list_lengths(k):
    """Tile tails and the values kernel's rounds (twelve 32-key tiles per round: 385 and more
    take two, 769 and more three)."""
    check_both(w.decode_f32(seed=900 + k, batch=2, heads=64, n_ctx=2000, k=k), f"f32 split k={k}")


def test_out_of_range_and_garbage_beyond_count():
    c = w.decode_f32(seed=910, batch=4, heads=64, n_ctx=500, k=200)
    c.idx[1, 150] = 500          # inside the count: NaN row
    c.idx[2, 199] = -7           # inside the count: NaN row
    c.nsel[3] = 160
    c.idx[3, 160:] = 123456789   # beyond the count: never read
    got, _ = check_both(c, "f32 split out-of-range inside / garbage beyond the count")
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[3]))


@pytest.mark.parametrize("which,val", [("k", np.nan), ("k", np.inf), ("k", -np.inf),
                                       ("v", np.nan), ("v", np.inf), ("v", -np.inf)])
def test_nonfinite_planted(which, val):
    c = w.decode_f32(seed=912, batch=2, heads=64, n_ctx=256, k=200)
    arr = c.k if which == "k" else c.v
    arr[0, c.idx[0, 170], 123] = val
    check_both(c, f"f32 split planted {which}={val}")


def test_nonfinite_sinks_and_far_scores():
    c = w.decode_f32(seed=913, batch=2, heads=64, n_ctx=300, k=200)
    c.sinks[3], c.sinks[5], c.sinks[7] = np.inf, -np.inf, np.nan
    c.nsel[1] = 0
    c.idx[1, :] = -1
    check_both(c, "f32 split nonfinite sinks, an empty row")
    c = w.decode_f32(seed=914, batch=2, heads=32, n_ctx=300, k=200)
    c.q[:] = 1.0
    c.k[:] = -0.5
    c.scale = 1.0
    c.sinks[:16] = -np.inf
    got, _ = check_both(c, "f32 split sink -inf, scores -256")
    assert np.all(np.isfinite(got))


def test_aliased_latent():
    check_both(w.decode_f32(seed=915, batch=5, heads=64, n_ctx=3000, k=640), "f32 split K = V", alias=True)


def test_prefill_shared_cache():
    """Prefill rows over one shared cache, causal selections."""
    b = w.prefill_bf16(seed=916, rows=12, first_pos=980, heads=64, n_ctx=1000, k=640)
    c = w.AttnCase("prefill_f32", "f32", w.bf16_to_f32(b.q), w.bf16_to_f32(b.k), w.bf16_to_f32(b.v), b.idx, b.nsel,
                   b.sinks, b.scale, True, positions=b.positions)
    check_both(c, "f32 split prefill 12 rows")


def test_batch_sweep_bits():
    """One set of rows launched as batches of 1, 2, 8, 16 and 23 (split path) and 24, 40 and 60
    (attn_f32_kernel): every row's bits are the same in every launch."""
    import sparse_attention_attn_amd as sa
    c = w.decode_f32(seed=917, batch=60, heads=64, n_ctx=1024, k=640)
    d = to_device(c, DEV)
    say("f32 batch sweep: B in 1, 2, 8, 16, 23 | 24, 40, 60")
    full = sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"])
    for b in (1, 2, 8, 16, 23, 24, 40):
        part = sa.decode(d["q"][:b], d["k"][:b], d["v"][:b], d["idx"][:b], d["sinks"], c.scale, d["nsel"][:b])
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int32), full[:b].view(torch.int32)), f"B={b}"
    rows = [0, 22, 23, 59]
    assert_parity(full.cpu().numpy()[rows], run_oracle(c, rows=rows)[rows], *F32_TOL, "f32 batch sweep rows")


def test_repeats_and_guards():
    """Five repeats of a split launch are byte-identical and write nothing outside their output,
    with a workspace reused across the repeats (its old contents never matter)."""
    import sparse_attention_attn_amd as sa
    from sparse_attention_attn_amd import _lib as L
    c = w.decode_f32(seed=918, batch=3, heads=64, n_ctx=3000, k=640)
    d = to_device(c, DEV)
    n = c.rows * c.heads * 512
    guard = 4096
    need = sa.workspace_bytes(L.SA_OP_DECODE, c.rows, c.heads, c.kmax, c.n_ctx)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=DEV)
    say("f32 split path: 5 repeats with guards, reused workspace")
    outs = []
    for _ in range(5):
        buf = torch.full((guard + n + guard,), 12345.0, dtype=torch.float32, device=DEV)
        out = buf[guard:guard + n].view(c.rows, c.heads, 512)
        sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"], out=out, ws=ws)
        torch.cuda.synchronize()
        assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + n:] == 12345.0)
        outs.append(out.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
