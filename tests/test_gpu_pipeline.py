"""A step as a caller runs it: the indexer's top-k on the device, and its index and count outputs,
never copied to the host, fed straight into the attention call on the same stream (akol1/TensorFold
pull request 4, PR body: the indexer's merge and finish per row, "the same picks", ahead of the
attention). The oracle recomputes both stages from the same scores: its top-k must equal the
device's bit for bit, and its attention over its own selection must match the device's output.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as w
from parity import BF16_TOL, assert_parity, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib_loaded():
    import sparse_attention_attn_amd as sa
    sa.load()


def oracle_rows(case, scores, k, rows, valid_len=None):
    """Oracle top-k then attention for the sampled rows (each row on its own)."""
    outs, idxs, cnts = [], [], []
    for r in rows:
        vl = None if valid_len is None else valid_len[r:r + 1]
        idx, cnt = oracle.topk(scores[r:r + 1], k, vl)
        kc = case.k if case.shared_cache else case.k[r:r + 1]
        vc = case.v if case.shared_cache else case.v[r:r + 1]
        o = oracle.attention(case.dtype, case.q[r:r + 1], kc, vc, idx, cnt, case.sinks, case.scale,
                             case.shared_cache)
        outs.append(o[0])
        idxs.append(idx[0])
        cnts.append(cnt[0])
    return np.stack(outs), np.stack(idxs), np.array(cnts)


@pytest.mark.parametrize("heads", [64, 16])
def test_causal_topk_feeds_prefill(heads):
    """The prefill segment: 2,048 rows at positions 2,048..4,095 over one 4,096-position cache,
    causal top-640 over each row's 4,096 indexer scores (valid_len = pos + 1), then prefill
    attention on the device-resident selection."""
    import sparse_attention_attn_amd as sa
    T, N, K, first = 2048, 4096, 640, 2048
    c = w.prefill_bf16(seed=400 + heads, rows=T, first_pos=first, heads=heads, n_ctx=N, k=K)
    scores = w.indexer_scores(seed=410 + heads, rows=T, n=N)
    valid_len = np.arange(first + 1, first + T + 1, dtype=np.int32)
    d = to_device(c, DEV)
    say(f"causal top-{K} -> prefill, {T} rows, {heads} heads")
    s_dev = torch.from_numpy(scores).to(DEV)
    vl_dev = torch.from_numpy(valid_len).to(DEV)
    idx_dev, cnt_dev = sa.topk(s_dev, K, valid_len=vl_dev)
    out = sa.prefill(d["q"], d["k"], d["v"], idx_dev, d["sinks"], c.scale, cnt_dev)
    torch.cuda.synchronize()
    rows = [0, 1, 2, 511, 1024, 1500, 2046, 2047] + list(range(97, T, 331))
    ref, ref_idx, ref_cnt = oracle_rows(c, scores, K, rows, valid_len)
    assert np.array_equal(idx_dev.cpu().numpy()[rows], ref_idx)
    assert np.array_equal(cnt_dev.cpu().numpy()[rows], ref_cnt)
    assert np.all(idx_dev.cpu().numpy() <= (valid_len - 1)[:, None])  # causal
    st = assert_parity(out.cpu().numpy()[rows], ref, *BF16_TOL, f"top-k -> prefill H={heads}")
    say(f"  ok {st}")


@pytest.mark.parametrize("batch,n_ctx", [(8, 32768), (1, 4096), (1024, 4096)])
def test_topk_feeds_decode(batch, n_ctx):
    """Top-640 over each sequence's indexer scores feeding decode: the indexer shape (8 x 32,768,
    caches with about 1% of K and V rows carrying +inf/-inf/NaN), the single-row decode shape, and
    the benchmarked batch of 1,024 sequences (device-generated inputs, 16 sampled rows)."""
    import sparse_attention_attn_amd as sa
    K = 640
    if batch <= 8:
        scores, c, _, _ = w.indexer_then_decode(seed=420 + batch, batch=batch, n_ctx=n_ctx, k=K,
                                                p_bad=0.01 if batch == 8 else 0.0)
        d = to_device(c, DEV)
        q, kc, vc, sinks = d["q"], d["k"], d["v"], d["sinks"]
        rows = list(range(batch))
    else:
        inp = w.device_decode_inputs(torch, DEV, batch=batch, heads=64, n_ctx=n_ctx, k=K, seed=430)
        q, kc, vc, sinks = inp["q"], inp["k"], inp["v"], inp["sinks"]
        scores = w.indexer_scores(seed=431, rows=batch, n=n_ctx)
        rows = [0, 1, 255, 256, 511, 512, 700, 767, 768, 900, 1000, 1020, 1021, 1022, 1023, 333]
    say(f"top-{K} -> decode, {batch} x {n_ctx}")
    s_dev = torch.from_numpy(scores).to(DEV)
    idx_dev, cnt_dev = sa.topk(s_dev, K)
    out = sa.decode(q, kc, vc, idx_dev, sinks, w.SCALE, cnt_dev)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in rows:
        case = c if batch <= 8 else w.host_case_from_device(inp, r)
        rr = r if batch <= 8 else 0
        ref, ref_idx, ref_cnt = oracle_rows(case, scores[r:r + 1] if batch > 8 else scores, K,
                                            [rr])
        assert np.array_equal(idx_dev[r].cpu().numpy(), ref_idx[0]), f"row {r} indices"
        assert int(cnt_dev[r]) == ref_cnt[0]
        assert_parity(got[r:r + 1], ref, *BF16_TOL, f"top-k -> decode row {r}")
    say("  ok")
