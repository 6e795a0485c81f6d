"""The split path for small batches (sa_attn_split.hip, one launch: producer workgroups score
every 64-key tile, consumer workgroups wait for a row's scores and run the softmax and values per
head group and column slice) against the persistent kernels (sa_attn.hip) and the float64 oracle.

A launch with fewer than 24 rows per block of 64 heads (and index lists of at most 1,024
entries) takes the split path. The same rows padded with empty rows (nsel = 0, which read
nothing) to 64 per head block take the persistent kernels. Every real row must come out bit
for bit the same both ways, and within the tolerance of the oracle: the split changes where
the work runs, never its arithmetic (the ds4 commit log for ds4_tp.c: a split that follows the
launch must not change the output bytes).
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


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    import sparse_attention_attn_amd as sa
    sa.load()


def _lib():
    import sparse_attention_attn_amd as sa
    from sparse_attention_attn_amd import _lib as L
    return sa, L


def split_and_persistent(case, alias=False):
    """(split output, persistent output) of the case's rows, both float32 host arrays."""
    sa, L = _lib()
    d = to_device(case, DEV)
    if alias:
        d["v"] = d["k"]
    rows, H = case.rows, case.heads
    op = L.SA_OP_PREFILL if case.shared_cache else L.SA_OP_DECODE
    lib = sa.load()
    assert lib.sparse_attn_workspace_bytes(op, rows, H, 512, case.kmax, case.n_ctx) > 0, "not the split path"
    fn = sa.prefill if case.shared_cache else sa.decode
    split = fn(d["q"], d["k"], d["v"], d["idx"], d["sinks"], case.scale, d["nsel"])
    P = 64 * ((H + 63) // 64)
    assert lib.sparse_attn_workspace_bytes(op, P, H, 512, case.kmax, case.n_ctx) == 0, "not the persistent path"
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
    pers = fn(q, kc, vc, idx, d["sinks"], case.scale, nsel)
    torch.cuda.synchronize()
    out = split.cpu().numpy(), pers[:rows].cpu().numpy()
    del kc, vc, pers
    torch.cuda.empty_cache()
    return out


def check_both(case, label, alias=False, oracle_rows=None):
    say(f"{label}: B={case.rows} H={case.heads} N={case.n_ctx} kmax={case.kmax}{' aliased' if alias else ''}")
    split, pers = split_and_persistent(case, alias)
    assert np.array_equal(split.view(np.int32), pers.view(np.int32)), f"{label}: split path differs from persistent"
    if alias:
        case.v = case.k
    ref = run_oracle(case, rows=oracle_rows)
    sel = slice(None) if oracle_rows is None else list(oracle_rows)
    st = assert_parity(split[sel], ref[sel], *BF16_TOL, label)
    say(f"  ok (bit-equal to the persistent kernels) {st}")
    return split, ref


def test_decode_single_row_k640():
    """The decode shape, one row: 64 heads, 4,096 positions, k = 640 (ten tiles, one round)."""
    check_both(w.decode_bf16(), "decode 1 row")


@pytest.mark.parametrize("batch", [1, 3, 4, 5, 7])
def test_producer_block_widths(batch):
    """The decode shape at 1 to 7 rows: on a 256-CU part the launch scores with blocks of 16
    heads (1 and 3 rows), 32 heads (4 rows) and 64 heads (5 and 7 rows); every width gives the
    persistent kernels' bits."""
    c = w.decode_bf16(seed=400 + batch, batch=batch, heads=64, n_ctx=3000, k=640)
    c.nsel[-1] = 333
    c.idx[-1, 333:] = -1
    check_both(c, f"producer blocks, {batch} rows", oracle_rows=[0, batch - 1])


@pytest.mark.parametrize("heads", [1, 4, 16, 17, 32, 48, 64, 100, 128])
def test_head_counts_ragged(heads):
    """Head counts off the 16-head groups, with a full, an empty and a partial row (a masked tail)."""
    c = w.decode_bf16(seed=200 + heads, batch=3, heads=heads, n_ctx=1000, k=200)
    c.nsel[:] = [200, 0, 65]
    c.idx[1, :] = -1
    c.idx[2, 65:] = -1
    got, _ = check_both(c, f"H={heads} nsel {{200,0,65}}")
    assert np.all(got[1] == 0)


@pytest.mark.parametrize("k", [1, 63, 64, 65, 639, 640, 641, 704, 1023, 1024])
def test_index_list_lengths(k):
    """Tile boundaries and a consumer's rounds (ten tiles per round: 641 and more take two)."""
    c = w.decode_bf16(seed=300 + k, batch=2, heads=64, n_ctx=2000, k=k)
    check_both(c, f"k={k}")


def test_out_of_range_and_garbage_beyond_count():
    c = w.decode_bf16(seed=310, batch=4, heads=64, n_ctx=500, k=100)
    c.idx[1, 50] = 500           # inside the count: NaN row
    c.idx[2, 99] = -7            # inside the count: NaN row
    c.nsel[3] = 60
    c.idx[3, 60:] = 123456789    # beyond the count: never read
    got, _ = check_both(c, "out-of-range inside / garbage beyond the count")
    assert np.all(np.isnan(got[1])) and np.all(np.isnan(got[2]))
    assert np.all(np.isfinite(got[0])) and np.all(np.isfinite(got[3]))


@pytest.mark.parametrize("which,cls", [("k", 0x7FC0), ("k", 0x7F80), ("k", 0xFF80),
                                       ("v", 0x7FC0), ("v", 0x7F80), ("v", 0xFF80)])
def test_nonfinite_planted(which, cls):
    c = w.decode_bf16(seed=320, batch=2, heads=64, n_ctx=256, k=130)
    arr = c.k if which == "k" else c.v
    arr[0, c.idx[0, 70], 123] = cls
    check_both(c, f"planted {which}={cls:#x}")


def test_nonfinite_sinks():
    c = w.decode_bf16(seed=321, batch=2, heads=64, n_ctx=256, k=130)
    c.sinks[3], c.sinks[5], c.sinks[7] = np.inf, -np.inf, np.nan
    c.nsel[1] = 0
    c.idx[1, :] = -1
    check_both(c, "nonfinite sinks, an empty row")


@pytest.mark.parametrize("heads,alias", [(32, False), (64, False), (64, True)])
def test_reference_moves_from_far_below(heads, alias):
    """Sinks of -inf and every score near -250: the first tile moves the exponent reference with
    nothing accumulated yet (alpha = 0 path), and later tiles rescale."""
    rng = np.random.default_rng(322)
    c = w.decode_bf16(seed=322, batch=3, heads=heads, n_ctx=300, k=200)
    c.q[:] = 0x3F80
    c.k[:] = rng.choice(np.array([0xBF00, 0xBE80, 0xBF40], dtype=np.uint16), size=c.k.shape)
    c.scale = 1.0
    c.sinks[: heads // 2] = -np.inf
    got, _ = check_both(c, f"sink -inf, scores ~ -250, H={heads}", alias=alias)
    assert np.all(np.isfinite(got))


def test_aliased_latent():
    c = w.decode_bf16(seed=323, batch=5, heads=64, n_ctx=3000, k=640)
    check_both(c, "aliased K = V", alias=True)


@pytest.mark.parametrize("heads", [16, 64])
def test_prefill_shared_cache(heads):
    """Prefill rows over one shared cache, causal selections."""
    c = w.prefill_bf16(seed=324 + heads, rows=20, first_pos=980, heads=heads, n_ctx=1000, k=640)
    check_both(c, f"prefill 20 rows H={heads}")


def test_batched_decode_32k():
    """The batched decode shape: 8 sequences of 32,768 positions, k = 640."""
    check_both(w.batched_decode_bf16(), "batched decode 8 x 32K")


@pytest.mark.parametrize("alias", [False, True])
def test_batch_sweep_bits(alias):
    """One set of rows launched as batches of 1, 2, 8 and 23 (split path) and 24, 33, 63, 64, 100
    and 150 (persistent kernels with 8, 4, 2 and 1 column slices): every row's bits are the same in
    every launch."""
    sa, _ = _lib()
    c = w.decode_bf16(seed=330, batch=150, heads=64, n_ctx=1024, k=640)
    d = to_device(c, DEV)
    vv = d["k"] if alias else d["v"]
    say(f"batch sweep{' aliased' if alias else ''}: B in 1, 2, 8, 23 | 24, 33, 63, 64, 100, 150")
    full = sa.decode(d["q"], d["k"], vv, d["idx"], d["sinks"], c.scale, d["nsel"])
    for b in (1, 2, 8, 23, 24, 33, 63, 64, 100):
        part = sa.decode(d["q"][:b], d["k"][:b], vv[:b], d["idx"][:b], d["sinks"], c.scale, d["nsel"][:b])
        torch.cuda.synchronize()
        assert torch.equal(part.view(torch.int32), full[:b].view(torch.int32)), f"B={b}"
    if alias:
        c.v = c.k
    rows = [0, 62, 63, 149]
    assert_parity(full.cpu().numpy()[rows], run_oracle(c, rows=rows)[rows], *BF16_TOL, "batch sweep rows")


def test_split_repeats_and_guards():
    """Five repeats of a split launch are byte-identical and write nothing outside their output,
    with a workspace reused across the repeats (its old contents never matter)."""
    sa, L = _lib()
    c = w.decode_bf16(seed=331, batch=3, heads=64, n_ctx=3000, k=640)
    d = to_device(c, DEV)
    n = c.rows * c.heads * 512
    guard = 4096
    need = sa.load().sparse_attn_workspace_bytes(L.SA_OP_DECODE, c.rows, c.heads, 512, c.kmax, c.n_ctx)
    ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=DEV)
    say("split path: 5 repeats with guards, reused workspace")
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


@pytest.mark.parametrize("fill", ["zeros", "0xAB", "random"])
def test_workspace_contents_and_alternating_inputs(fill):
    """The split path passes scores between workgroups of one launch through the workspace, with
    per-tile ready words that depend on a sequence number the launch finds there. Whatever the
    workspace held before (zeros, a repeated byte, random bytes, what launches of other shapes
    left), every launch must wait for its own scores: calls that alternate between two input
    sets, with launches of other shapes in between, on one workspace, must each return their
    own inputs' result (a read of the previous call's scores would return the other set's)."""
    sa, L = _lib()
    shapes = [(3, 64, 2000, 640), (2, 128, 1500, 1000), (5, 16, 900, 700)]
    need = max(sa.load().sparse_attn_workspace_bytes(L.SA_OP_DECODE, b, h, 512, k, n) for b, h, n, k in shapes)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(333)
    if fill == "zeros":
        ws = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    elif fill == "0xAB":
        ws = torch.full((need,), 0xAB, dtype=torch.uint8, device=DEV)
    else:
        ws = torch.randint(0, 256, (need,), generator=gen, dtype=torch.uint8, device=DEV)
    sets = {}
    for si, (b, h, n, k) in enumerate(shapes):
        for v in range(2):
            c = w.decode_bf16(seed=340 + 2 * si + v, batch=b, heads=h, n_ctx=n, k=k)
            d = to_device(c, DEV)
            # The reference: the same call with a workspace of its own (fresh allocation).
            ref = sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"])
            sets[(si, v)] = (c, d, ref)
    torch.cuda.synchronize()
    say(f"workspace {fill}: 3 shapes x 2 input sets, alternating on one workspace")
    order = [(0, 0), (0, 1), (0, 0), (1, 0), (0, 1), (1, 1), (1, 0), (2, 0), (0, 0), (2, 1), (2, 0), (0, 1),
             (1, 1), (0, 0), (0, 1), (0, 0)]
    for i, key in enumerate(order):
        c, d, ref = sets[key]
        out = sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"], ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"call {i}: shape {key[0]} set {key[1]}"


def test_two_streams_at_once():
    """Split launches in flight at once on two streams, each with its own workspace, inputs and
    output (a consumer only ever waits for producers of its own launch): each call returns its own
    result, over several rounds."""
    sa, L = _lib()
    cases = [w.decode_bf16(seed=350 + i, batch=b, heads=64, n_ctx=3000, k=640) for i, b in enumerate((2, 8))]
    devs = [to_device(c, DEV) for c in cases]
    refs = [sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"]) for c, d in zip(cases, devs)]
    wss = [torch.empty((sa.load().sparse_attn_workspace_bytes(L.SA_OP_DECODE, c.rows, 64, 512, 640, 3000),),
                       dtype=torch.uint8, device=DEV) for c in cases]
    outs = [torch.empty_like(r) for r in refs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=DEV) for _ in cases]
    say("split path: two streams, 2 and 8 rows, 20 rounds")
    for rnd in range(20):
        for c, d, ws, o, st in zip(cases, devs, wss, outs, streams):
            with torch.cuda.stream(st):
                o.fill_(float("nan"))
                sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, d["nsel"], out=o, ws=ws)
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o.view(torch.int32), r.view(torch.int32)), f"round {rnd}: stream {i}"


def test_workspace_too_small_is_refused_before_launch():
    sa, L = _lib()
    c = w.decode_bf16(seed=332, batch=2, heads=64, n_ctx=500, k=100)
    d = to_device(c, DEV)
    need = sa.load().sparse_attn_workspace_bytes(L.SA_OP_DECODE, 2, 64, 512, 100, 500)
    out = torch.full((2, 64, 512), 7.0, device=DEV)
    with pytest.raises(sa.SparseAttnError):
        sa.decode(d["q"], d["k"], d["v"], d["idx"], d["sinks"], c.scale, out=out,
                  ws=torch.empty(need - 16, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
