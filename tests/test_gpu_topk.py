"""GPU parity of sparse_attn_topk: bit-exact against the oracle's exact selection."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as w

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def check(scores, k, valid_len=None, label=""):
    import sparse_attention_attn_amd as sa
    say(f"topk {label}: rows={scores.shape[0]} n={scores.shape[1]} k={k}")
    s = torch.from_numpy(np.ascontiguousarray(scores, np.float32)).to(DEV)
    vl = None if valid_len is None else torch.from_numpy(np.asarray(valid_len, np.int32)).to(DEV)
    idx, cnt = sa.topk(s, k, vl)
    torch.cuda.synchronize()
    ref_i, ref_c = oracle.topk(scores, k, valid_len)
    got_i, got_c = idx.cpu().numpy(), cnt.cpu().numpy()
    np.testing.assert_array_equal(got_c, ref_c)
    np.testing.assert_array_equal(got_i, ref_i)
    return got_i


def test_indexer_shape():
    """8 rows x 32,768 N(0,1) scores, exact top-640, seed 4."""
    check(w.indexer_scores(4), 640, label="indexer 8x32768")


def test_tie_stress():
    """Scores rounded to multiples of 1/16: thousands of ties at the threshold."""
    check(w.indexer_scores(4, tie_stress=True), 640, label="tie stress")
    check(np.full((3, 5000), 1.5, np.float32), 640, label="all equal")


def test_signed_zero_and_nan():
    rng = np.random.default_rng(70)
    s = rng.standard_normal((4, 3000)).astype(np.float32)
    s[0, ::3] = 0.0
    s[0, 1::3] = -0.0
    s[1, ::2] = np.nan
    s[2, :] = np.nan
    s[3, :1000] = -np.inf
    s[3, 1000:] = np.nan
    check(s, 640, label="+-0, NaN, -inf")


def test_causal_valid_lengths():
    """Prefill use: row t may select only positions <= 2048 + t (valid_len = pos + 1)."""
    rng = np.random.default_rng(71)
    s = rng.standard_normal((2048, 4096)).astype(np.float32)
    vl = (np.arange(2048) + 2049).astype(np.int32)
    got = check(s, 640, vl, label="causal 2048 rows")
    assert np.all(got <= (vl - 1)[:, None])


def test_short_rows_and_edges():
    rng = np.random.default_rng(72)
    s = rng.standard_normal((6, 1000)).astype(np.float32)
    check(s, 640, np.array([0, 1, 639, 640, 641, 1000], np.int32), label="valid_len edges")
    check(s, 1, label="k=1")
    check(s, 1000, label="k=n")
    check(s, 1500, label="k>n")


def test_long_rows_global_path():
    """Rows longer than the LDS-resident limit (32,768) are re-read from memory each pass."""
    rng = np.random.default_rng(73)
    s = rng.standard_normal((3, 50000)).astype(np.float32)
    s[1, 40000:] = 5.0  # ties beyond the LDS limit
    check(s, 640, label="n=50000")


def test_empty():
    import sparse_attention_attn_amd as sa
    s = torch.zeros((0, 100), device=DEV)
    idx, cnt = sa.topk(s, 10)
    torch.cuda.synchronize()
    assert idx.shape == (0, 10)


def test_mid_rows_four_waves():
    """Rows of 4,097..16,384 scores (four waves per row) with ragged valid lengths."""
    rng = np.random.default_rng(74)
    s = rng.standard_normal((5, 10000)).astype(np.float32)
    s[2, 5000:7000] = 0.25
    check(s, 640, np.array([10000, 4097, 6500, 700, 9999], np.int32), label="n=10000")
    check(np.round(s * 8) / 8, 1000, label="n=10000 ties")


def test_decode_shape():
    """The decode step's selection: 1,024 rows x 4,096 N(0,1) scores, top-640 (several
    waves per row), plus the same rows rounded to 1/8 (many ties at the threshold)."""
    rng = np.random.default_rng(75)
    s = rng.standard_normal((1024, 4096)).astype(np.float32)
    check(s, 640, label="decode 1024x4096")
    check(np.round(s * 8) / 8, 640, label="decode 1024x4096 ties")


def test_shared_upper_bits():
    """More than 256 keys agree in their upper 16 bits, so the bisection over every key
    continues into the lower half before the few remaining ones are singled out."""
    rng = np.random.default_rng(76)
    for rows, n in ((4, 4096), (1500, 4096), (2, 12000)):
        s = (1.0 + rng.integers(0, 1 << 14, size=(rows, n)) * 2.0 ** -22).astype(np.float32)
        check(s, 640, label=f"shared upper bits {rows}x{n}")


def test_large_k_unstaged():
    """k above 4,096: selected positions are written straight to memory."""
    rng = np.random.default_rng(77)
    s = rng.standard_normal((3, 20000)).astype(np.float32)
    s[1, ::7] = 0.5
    check(s, 5000, label="k=5000")
