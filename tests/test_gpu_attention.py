"""GPU parity of sparse_attn_decode / sparse_attn_prefill against the float64 oracle.

Every test calls the HIP kernels through the C ABI (via the thin binding) on
seeded inputs from `workloads` and compares with the oracle on the same inputs:
element by element at sizes the oracle finishes in seconds (several tiles and a
ragged tail), and on sampled rows at the full sizes the benchmark times.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as w
from parity import BF16_TOL, F32_TOL, assert_parity, run_gpu, run_oracle, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    import sparse_attention_attn_amd as sa
    sa.load()  # fails loudly if the HIP library is missing


def check_case(case, rows=None, label=None, with_nsel=True):
    say(f"{label or case.name}: B={case.rows} H={case.heads} N={case.n_ctx} kmax={case.kmax} dtype={case.dtype}")
    got = run_gpu(case, DEV, with_nsel=with_nsel)
    ref = run_oracle(case, rows=rows)
    sel = slice(None) if rows is None else list(rows)
    st = assert_parity(got[sel], ref[sel], *(BF16_TOL if case.dtype == "bf16" else F32_TOL), label or case.name)
    say(f"  ok {st}")
    return got, ref


def test_tiny_f32():
    """Tiny fp32 check: 1 row, 4 heads, 256 positions, k = 64, seed 0."""
    check_case(w.tiny_f32())


def test_tiny_f32_ragged_and_multi_tile():
    c = w.tiny_f32(seed=5, heads=3, n_ctx=300, k=150)
    check_case(c, label="f32 3 heads k=150 (3 tiles, ragged)")


@pytest.mark.parametrize("heads", [1, 4, 16, 32, 48, 64, 100, 128])
def test_bf16_head_counts(heads):
    """Head counts that are not a multiple of the 16-head MFMA block are padded internally (heads past H
    read a zero query and are not stored)."""
    c = w.decode_bf16(seed=20 + heads, batch=2, heads=heads, n_ctx=1000, k=200)
    check_case(c, label=f"bf16 H={heads} k=200")


def test_bf16_ragged_counts():
    """Rows with different counts, including 0 and a partial last tile; idx padded with -1."""
    c = w.decode_bf16(seed=30, batch=4, heads=64, n_ctx=2000, k=300)
    c.nsel[:] = [300, 137, 0, 65]
    c.idx[1, 137:] = -1
    c.idx[2, :] = -1
    c.idx[3, 65:] = -1
    got, _ = check_case(c, label="bf16 nsel {300,137,0,65}")
    # nsel = 0: o = 0 / exp(0) = 0 with finite sinks
    assert np.all(got[2] == 0)


def test_decode_single_row():
    """Decode: 1 row, 64 heads, 4,096 positions, k = 640, seed 1."""
    check_case(w.decode_bf16())


@pytest.fixture(scope="module")
def batched_case():
    return w.batched_decode_bf16()


def test_batched_decode(batched_case):
    """Batched decode: 8 sequences with 32,768 positions each, k = 640, seed 2."""
    check_case(batched_case)


@pytest.mark.parametrize("k", w.EDGE_K)
def test_batched_decode_edge_k(batched_case, k):
    """Tile boundaries: k in {1, 63, 64, 65, 639, 641} on the same 32K caches."""
    rng = np.random.default_rng(1000 + k)
    c = batched_case
    idx = np.stack([w.sorted_unique_indices(rng, c.n_ctx, k) for _ in range(c.rows)])
    ck = w.AttnCase(f"edge_k{k}", c.dtype, c.q, c.k, c.v, idx, np.full(c.rows, k, np.int32), c.sinks, c.scale, False)
    check_case(ck)
    check_case(ck, label=f"edge_k{k} nsel=NULL", with_nsel=False)


def test_prefill_sampled_rows():
    """Prefill segment: 2,048 rows at positions 2,048..4,095 over one 4,096-position cache.

    The full segment runs on the GPU; the oracle checks 16 sampled rows."""
    c = w.prefill_bf16()
    assert np.all(c.idx[np.arange(c.rows)[:, None], np.arange(c.kmax)[None]] <= c.positions[:, None])
    rows = [0, 1, 2, 63, 64, 511, 777, 1024, 1500, 1919, 2000, 2040, 2045, 2046, 2047, 1234]
    check_case(c, rows=rows, label="prefill 2048 rows (16 sampled)")


def test_prefill_padded_heads():
    """The whole 2,048-row prefill segment (positions 2,048..4,095) with 16 real heads zero-padded
    into a 32-head launch with zero sinks (TensorFold pull request 1206, "What changes"); only the
    real heads are compared. The real heads must equal an unpadded 16-head launch bit for bit on
    every row, and the oracle within tolerance on sampled rows."""
    import sparse_attention_attn_amd as sa
    c = w.prefill_bf16(seed=3, rows=2048, first_pos=2048, heads=16)
    d = to_device(c, DEV)
    say("prefill 2048 rows, 16 heads padded to 32")
    q_pad, s_pad = sa.pad_heads(d["q"], d["sinks"], 32)
    torch.cuda.synchronize()
    assert torch.equal(q_pad[:, 16:].float(), torch.zeros_like(q_pad[:, 16:].float()))
    assert torch.equal(s_pad[16:], torch.zeros(16, device=DEV)) and torch.equal(s_pad[:16], d["sinks"])
    out_pad = sa.prefill(q_pad, d["k"], d["v"], d["idx"], s_pad, c.scale, d["nsel"])
    real = sa.unpad_heads(out_pad, 16)
    plain = sa.prefill(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"])
    torch.cuda.synchronize()
    assert torch.equal(real, plain), "padded launch's real heads differ from the unpadded launch"
    assert torch.equal(real, out_pad[:, :16])
    rows = [0, 1, 2, 255, 256, 511, 777, 1023, 1024, 1500, 1919, 2040, 2045, 2046, 2047] + list(range(37, 2048, 173))
    ref = run_oracle(c, rows=rows)
    st = assert_parity(real.cpu().numpy()[rows], ref[rows], *BF16_TOL, "padded 16->32")
    say(f"  ok {st}")


def test_exact_sums_k640():
    """q = 0, sink = -inf, integer V: every sum is exact, so the GPU equals the oracle rounded to fp32."""
    rng = np.random.default_rng(12)
    c = w.decode_bf16(seed=40, batch=2, heads=64, n_ctx=4096, k=640)
    c.q[:] = 0
    c.v[:] = w.bf16_bits(rng.integers(-16, 17, size=c.v.shape).astype(np.float32))
    c.sinks[:] = -np.inf
    say("exact sums k=640")
    got = run_gpu(c, DEV)
    ref = run_oracle(c)
    assert np.array_equal(got, ref.astype(np.float32))


def test_out_of_range_index_gives_nan_row():
    c = w.decode_bf16(seed=41, batch=3, heads=64, n_ctx=500, k=100)
    c.idx[1, 50] = 500
    c.idx[2, 99] = -7
    got, _ = check_case(c, label="out-of-range index")
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2])) and np.all(np.isfinite(got[0]))


def test_out_of_range_beyond_count_is_ignored():
    c = w.decode_bf16(seed=42, batch=2, heads=64, n_ctx=500, k=100)
    c.nsel[:] = [60, 100]
    c.idx[0, 60:] = 123456789  # beyond the count: never read
    got, _ = check_case(c, label="garbage beyond nsel")
    assert np.all(np.isfinite(got))


def _planted(seed):
    return w.decode_bf16(seed=seed, batch=2, heads=64, n_ctx=256, k=130)


@pytest.mark.parametrize("which,cls", [("k", 0x7FC0), ("k", 0x7F80), ("k", 0xFF80),
                                       ("v", 0x7FC0), ("v", 0x7F80), ("v", 0xFF80)])
def test_nonfinite_planted(which, cls):
    """One selected cache row carries NaN / +inf / -inf in one column: classes follow the oracle."""
    c = _planted(50)
    arr = c.k if which == "k" else c.v
    i = c.idx[0, 70]
    arr[0, i, 123] = cls
    got, ref = check_case(c, label=f"planted {which}={cls:#x}")
    assert not np.all(np.isfinite(ref[0]))


def test_nonfinite_sinks():
    c = _planted(51)
    c.sinks[3] = np.inf
    c.sinks[5] = -np.inf
    c.sinks[7] = np.nan
    got, _ = check_case(c, label="nonfinite sinks")
    assert np.all(np.isnan(got[:, 3])) and np.all(np.isnan(got[:, 7])) and np.all(np.isfinite(got[:, 5]))


def test_sink_minus_inf_empty_row_is_nan():
    c = _planted(52)
    c.sinks[:] = -np.inf
    c.nsel[1] = 0
    got, _ = check_case(c, label="sink=-inf, nsel=0")
    assert np.all(np.isnan(got[1]))


@pytest.mark.parametrize("heads,alias", [(32, False), (64, False), (64, True)])
def test_sink_minus_inf_scores_far_below_zero(heads, alias):
    """Heads whose sink is -inf and whose every score lies near -250: the first tile moves the
    exponent reference from 0 down to the maximum, with nothing accumulated yet. The result
    is an ordinary weighted average (the oracle's), not inf * 0."""
    rng = np.random.default_rng(53)
    c = w.decode_bf16(seed=53, batch=3, heads=heads, n_ctx=300, k=130)
    c.q[:] = 0x3F80                                   # 1.0
    c.k[:] = rng.choice(np.array([0xBF00, 0xBE80, 0xBF40], dtype=np.uint16), size=c.k.shape)  # -0.5, -0.25, -0.75
    if alias:
        c.v = c.k
    c.scale = 1.0
    c.sinks[: heads // 2] = -np.inf
    got, ref = check_case(c, label=f"sink -inf, scores ~ -250, H={heads}{' aliased' if alias else ''}")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("alias", [False, True])
def test_largest_cache(alias):
    """Caches of 2^22 - 1 positions, the largest a bf16 cache may hold (4 GiB per sequence and
    tensor). Rows 0 and 1 select positions at both ends of the range (0, 1, 2^21, 2^22 - 3,
    2^22 - 2 and random others), so the gathers' 32-bit byte offsets and the buffer range are
    exercised at their limit. Row 2 also selects 2^22 - 1, one past the last position, inside its
    count: its output must be all NaN. The oracle evaluates the same selections on a compact
    copy that holds only the selected rows (nothing else in the caches is read)."""
    import sparse_attention_attn_amd as sa
    from sparse_attention_attn_amd import _lib
    N = _lib.SA_BF16_MAX_CTX
    rng = np.random.default_rng(96)
    small = w.decode_bf16(seed=96, batch=3, heads=64, n_ctx=640, k=640, name="largest cache")
    assert np.array_equal(small.idx, np.tile(np.arange(640, dtype=np.int32), (3, 1)))
    if alias:
        small.v = small.k
    fixed = np.array([0, 1, 1 << 21, N - 2, N - 1], dtype=np.int64)
    big_idx = np.empty((3, 640), dtype=np.int64)
    for r in range(3):
        others = rng.choice(np.arange(2, N - 2, dtype=np.int64), size=640 - len(fixed), replace=False)
        big_idx[r] = np.sort(np.concatenate([fixed, others]))
    big_idx[2, -1] = N  # one past the last position (the list stays sorted)
    say(f"largest cache N={N}{' aliased' if alias else ''}: 3 rows x 640, 64 heads")
    kd = torch.zeros((3, N, w.D), dtype=torch.bfloat16, device=DEV)
    vd = kd if alias else torch.zeros((3, N, w.D), dtype=torch.bfloat16, device=DEV)
    d = to_device(small, DEV)
    for r in range(3):
        pos = torch.from_numpy(big_idx[r][big_idx[r] < N]).to(DEV)
        kd[r, pos] = d["k"][r, : len(pos)]
        if not alias:
            vd[r, pos] = d["v"][r, : len(pos)]
    idx = torch.from_numpy(big_idx.astype(np.int32)).to(DEV)
    got = sa.decode(d["q"], kd, vd, idx, d["sinks"], small.scale).cpu().numpy()
    torch.cuda.synchronize()
    del kd, vd
    torch.cuda.empty_cache()
    ref = run_oracle(small, rows=[0, 1])
    st = assert_parity(got[:2], ref[:2], *BF16_TOL, "largest cache")
    assert np.isnan(got[2]).all()
    say(f"  ok {st}")


@pytest.mark.parametrize("dtype,rows,alias", [("bf16", 32, False), ("bf16", 32, True), ("f32", 32, False),
                                               ("f32", 4, False)])
def test_largest_shared_cache_with_masked_entries(dtype, rows, alias):
    """One shared cache of the largest size each storage type allows (2^22 - 1 bf16 positions,
    2^21 - 1 float32 positions: 4 GiB per tensor), read by a prefill launch that takes the
    persistent kernels (bf16, 32 rows; attn_f32_kernel, 32 rows) or the float32 split path
    (4 rows). Every row holds masked entries (-1) past a count below kmax, whose wrapped byte
    offsets sit at the 32-bit buffer range's end, next to selected positions at both ends of the
    cache (0, 1, 2^21 or 2^20, N - 2, N - 1). The oracle evaluates the same selections on a
    compact cache of the 640 positions used."""
    import sparse_attention_attn_amd as sa
    from sparse_attention_attn_amd import _lib
    N = _lib.SA_BF16_MAX_CTX if dtype == "bf16" else _lib.SA_F32_MAX_CTX
    rng = np.random.default_rng(97 + rows)
    kmax = 640
    normal = w._normal_bf16 if dtype == "bf16" else w._normal
    q = normal(rng, (rows, 64, w.D))
    kc = normal(rng, (1, kmax, w.D))
    vc = kc if alias else normal(rng, (1, kmax, w.D))
    sinks = rng.standard_normal(64).astype(np.float32)
    idx = np.empty((rows, kmax), dtype=np.int32)
    nsel = rng.integers(kmax // 2, kmax, size=rows).astype(np.int32)  # below kmax: masked tails
    for r in range(rows):
        idx[r, : nsel[r]] = rng.permutation(kmax)[: nsel[r]]
        idx[r, nsel[r]:] = -1
    small = w.AttnCase(f"largest shared cache {dtype}", dtype, q, kc, vc, idx, nsel, sinks, w.SCALE, True)
    # compact position i of the oracle's cache lives at big position pos[i]
    fixed = np.array([0, 1, (N + 1) // 2, N - 2, N - 1], dtype=np.int64)
    others = rng.choice(np.arange(2, N - 2, dtype=np.int64), size=kmax - len(fixed), replace=False)
    pos = np.sort(np.concatenate([fixed, others]))
    assert len(np.unique(pos)) == kmax
    say(f"largest shared cache N={N} {dtype}{' aliased' if alias else ''}: {rows} rows x {kmax}, 64 heads")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    d = to_device(small, DEV)
    kd = torch.zeros((N, w.D), dtype=tdt, device=DEV)
    vd = kd if alias else torch.zeros((N, w.D), dtype=tdt, device=DEV)
    pos_d = torch.from_numpy(pos).to(DEV)
    kd[pos_d] = d["k"]
    if not alias:
        vd[pos_d] = d["v"]
    big = np.where(idx >= 0, pos[np.maximum(idx, 0)], -1).astype(np.int32)
    got = sa.prefill(d["q"], kd, vd, torch.from_numpy(big).to(DEV), d["sinks"], small.scale, d["nsel"]).cpu().numpy()
    torch.cuda.synchronize()
    del kd, vd
    torch.cuda.empty_cache()
    sel = sorted({0, rows // 2, rows - 1})
    ref = run_oracle(small, rows=sel)
    st = assert_parity(got[sel], ref[sel], *(BF16_TOL if dtype == "bf16" else F32_TOL), small.name)
    say(f"  ok {st}")


def test_determinism_and_guards():
    """Five repeats are byte-identical and never write outside their output."""
    import sparse_attention_attn_amd as sa
    c = w.decode_bf16(seed=60, batch=3, heads=64, n_ctx=3000, k=640)
    d = to_device(c, DEV)
    n = c.rows * c.heads * w.D
    guard = 4096
    say("determinism x5 with guard regions")
    outs = []
    for _ in range(5):
        buf = torch.full((guard + n + guard,), 12345.0, dtype=torch.float32, device=DEV)
        out = buf[guard:guard + n].view(c.rows, c.heads, w.D)
        sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"], out=out)
        torch.cuda.synchronize()
        assert torch.all(buf[:guard] == 12345.0) and torch.all(buf[guard + n:] == 12345.0)
        outs.append(out.clone())
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))


@pytest.mark.parametrize("heads,alias", [(64, False), (32, False), (16, False), (64, True), (16, True)])
def test_batch_invariance_across_launch_shapes(heads, alias):
    """A row's bits do not depend on how many rows share the launch: B = 300, 200 and 100 run the
    persistent kernels with one or two column slices, which split heads and columns differently;
    B = 8 and 1 run the split path (every 64-key tile scored in its own workgroup, the scores
    folded in key order), which runs the same arithmetic."""
    import sparse_attention_attn_amd as sa
    c = w.decode_bf16(seed=61 + heads, batch=300, heads=heads, n_ctx=1024, k=640)
    d = to_device(c, DEV)
    vv = d["k"] if alias else d["v"]
    say(f"batch invariance H={heads}{' aliased' if alias else ''}, B in {{300, 200, 100, 8, 1}}")
    full = sa.decode(d["q"], d["k"], vv, d["idx"], d["sinks"], c.scale, d["nsel"])
    for b in (200, 100, 8, 1):
        part = sa.decode(d["q"][:b], d["k"][:b], vv[:b], d["idx"][:b], d["sinks"], c.scale, d["nsel"][:b])
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int32), full[:b].view(torch.int32)), f"B={b}"
    if alias:
        c.v = c.k
    ref = run_oracle(c, rows=[0, 150, 299])
    assert_parity(full.cpu().numpy()[[0, 150, 299]], ref[[0, 150, 299]], *BF16_TOL, "B=300 rows")


def test_empty_batch():
    import sparse_attention_attn_amd as sa
    c = w.decode_bf16(seed=62, batch=1, heads=64, n_ctx=100, k=10)
    d = to_device(c, DEV)
    out = sa.decode(d["q"][:0], d["k"][:0], d["v"][:0], d["idx"][:0], d["sinks"], c.scale)
    torch.cuda.synchronize()
    assert out.shape == (0, 64, 512)


def test_aliased_kv_and_prefill_equals_decode():
    """K and V may be one tensor; a shared cache through prefill equals decode on replicated caches."""
    import sparse_attention_attn_amd as sa
    c = w.prefill_bf16(seed=63, rows=4, first_pos=900, heads=64, n_ctx=1000, k=640)
    c.v = c.k  # aliased latent
    d = to_device(c, DEV)
    say("aliased K=V prefill vs decode")
    pre = sa.prefill(d["q"], d["k"], d["k"], d["idx"], d["sinks"], c.scale, d["nsel"])
    kk = d["k"].unsqueeze(0).expand(4, -1, -1).contiguous()
    dec = sa.decode(d["q"], kk, kk, d["idx"], d["sinks"], c.scale, d["nsel"])
    torch.cuda.synchronize()
    assert torch.equal(pre, dec)
    assert_parity(pre.cpu().numpy(), run_oracle(c), *BF16_TOL, "aliased")


@pytest.mark.parametrize("rows,heads", [(300, 64), (40, 64), (100, 32), (20, 16)])
def test_shared_cache_prefill_equals_decode_on_copies(rows, heads):
    """Prefill over one shared cache (whose kernel prefetches each next tile's rows into L2)
    equals decode over per-row copies of that cache (no prefetch) bit for bit, including
    NaN rows: ragged counts and masked tails, -1 and out-of-range indices inside a row's
    count (NaN row) and beyond it (ignored), over launch shapes with one to eight column
    slices (V rows prefetched whole or in part)."""
    import sparse_attention_attn_amd as sa
    n_ctx, k = 1000, 200
    c = w.prefill_bf16(seed=64 + rows + heads, rows=rows, first_pos=n_ctx - rows, heads=heads, n_ctx=n_ctx, k=k)
    rng = np.random.default_rng(rows * heads)
    c.nsel[:] = rng.integers(0, k + 1, size=rows)
    c.nsel[:4] = [k, 1, 0, 65]
    c.idx[1, 0] = -1                  # inside the count: NaN row
    c.idx[3, 64] = n_ctx + 5          # inside the count (65): NaN row
    c.idx[0, k - 1] = 2 ** 30         # inside the count (k): NaN row
    c.idx[5, c.nsel[5]:] = n_ctx * 7  # beyond the count: ignored
    c.idx[6, c.nsel[6]:] = -1
    d = to_device(c, DEV)
    say(f"shared-cache prefill vs decode on copies rows={rows} heads={heads}")
    pre = sa.prefill(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"])
    kk = d["k"].unsqueeze(0).expand(rows, -1, -1).contiguous()
    vv = d["v"].unsqueeze(0).expand(rows, -1, -1).contiguous()
    dec = sa.decode(d["q"], kk, vv, d["idx"], d["sinks"], c.scale, d["nsel"])
    torch.cuda.synchronize()
    assert torch.equal(pre.view(torch.int32), dec.view(torch.int32))
    got = pre.cpu().numpy()
    assert np.all(np.isnan(got[[0, 1, 3]])) and np.all(np.isfinite(got[[2, 5, 6]]))
    sample = [2, 4, 5, 6, rows // 2, rows - 1]
    st = assert_parity(got[sample], run_oracle(c, rows=sample)[sample], *BF16_TOL, "shared-cache prefill")
    say(f"  ok {st}")


def test_indexer_then_decode_nonfinite():
    """Indexer + attention: exact top-640 of 8 x 32,768 scores feeds decode on caches where
    about 1% of K and V rows carry +inf/-inf/NaN; classes and values follow the oracle."""
    import sparse_attention_attn_amd as sa
    scores, c, bad_k, bad_v = w.indexer_then_decode()
    say("indexer top-640 -> decode with nonfinite rows")
    s_dev = torch.from_numpy(scores).to(DEV)
    idx_dev, cnt_dev = sa.topk(s_dev, 640)
    torch.cuda.synchronize()
    ref_idx, ref_cnt = oracle.topk(scores, 640)
    assert np.array_equal(idx_dev.cpu().numpy(), ref_idx) and np.array_equal(cnt_dev.cpu().numpy(), ref_cnt)
    c.idx[:] = ref_idx
    c.nsel[:] = ref_cnt
    got, ref = check_case(c, label="indexer->decode nonfinite")
    say(f"  nonfinite outputs: {int((~np.isfinite(ref)).sum())} of {ref.size}")


def test_sustained_decode_sampled():
    """The benchmarked shape: 1,024 sequences x 4,096 positions, 64 heads, k = 640, inputs
    generated on the device; the oracle checks 16 sampled rows."""
    import sparse_attention_attn_amd as sa
    say("sustained decode B=1024 (device inputs, 16 sampled rows)")
    inp = w.device_decode_inputs(torch, DEV, batch=1024, heads=64, n_ctx=4096, k=640, seed=7)
    out = sa.decode(inp["q"], inp["k"], inp["v"], inp["idx"], inp["sinks"], w.SCALE)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 511, 512, 640, 700, 767, 768, 900, 1000, 1020, 1021, 1022, 1023]
    for r in rows:
        case = w.host_case_from_device(inp, r)
        ref = run_oracle(case)
        assert_parity(out[r:r + 1].cpu().numpy(), ref, *BF16_TOL, f"sustained row {r}")
    del inp
    torch.cuda.empty_cache()


def test_few_keys_precision():
    """Rows that select only a few keys of comparable weight: the value sum cancels
    towards zero while each term is large, so the weights p must enter the value product
    with more than bf16's 8 bits (they go in as a hi + lo pair of bf16 parts)."""
    rng = np.random.default_rng(95)
    c = w.decode_bf16(seed=95, batch=64, heads=64, n_ctx=300, k=40, name="few keys")
    c.nsel[:] = rng.integers(1, 41, size=64).astype(np.int32)
    got, ref = check_case(c, label="few keys")
    err = np.abs(got.astype(np.float64) - ref)
    say(f"  max abs error {err.max():.2e}")
    assert err.max() < 1e-4


def test_masked_slots_read_zeros_after_nonfinite_tile():
    """A workgroup's second unit (row 256 of 300) has 5 keys after its first unit (row 0)
    filled the tile buffers with value rows holding +inf: the 59 masked slots must read
    as zeros (a stale inf times the zero weight of a masked key would give NaN)."""
    c = w.decode_bf16(seed=96, batch=300, heads=64, n_ctx=256, k=128, name="masked after inf")
    c.v[0][c.idx[0, :128], 7] = 0x7F80  # +inf in column 7 of every row row 0 selects
    c.nsel[256] = 5
    got, ref = check_case(c, rows=[0, 1, 255, 256, 257, 299], label="masked slots after an inf tile")
    assert np.isinf(got[0][:, 7]).all() and np.isfinite(got[256]).all()
