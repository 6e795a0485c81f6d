"""Checks that pin the float64 oracle to facts outside itself.

Every check takes the loaded oracle library (so the mutation test can run the
same checks against deliberately broken copies) and raises AssertionError on a
mismatch. Each check states what fixes the expected value: a closed form of
softmax attention with a sink, a library routine on a special case, brute force
over an explicit mask, an invariant, or the IEEE class table.

The sink reading (one extra logit in the denominator with a zero value vector,
not scaled) comes from TensorFold pull request 1206, "What changes": padded
heads get zero sinks, and the problem statement's closed form "one selected key
returns its value scaled by the softmax weight against the sink".
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import workloads as w

SCALE = w.SCALE


def _att(lib, dtype, q, k, v, idx, nsel, sinks, shared=False, scale=SCALE):
    return oracle.attention(dtype, q, k, v, idx, nsel, sinks, scale, shared, lib=lib)


def _f64(dtype, a):
    return (w.bf16_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)).astype(np.float64)


def _rand_case(rng, dtype, rows=2, heads=3, n=40, k=7, shared=False):
    d = w.D
    f = (lambda s: w.bf16_bits(rng.standard_normal(s, dtype=np.float32))) if dtype == "bf16" \
        else (lambda s: rng.standard_normal(s, dtype=np.float32))
    q = f((rows, heads, d))
    kc = f((1 if shared else rows, n, d))
    vc = f((1 if shared else rows, n, d))
    sinks = rng.standard_normal(heads, dtype=np.float32)
    idx = np.stack([w.sorted_unique_indices(rng, n, k) for _ in range(rows)])
    nsel = np.full(rows, k, np.int32)
    return q, kc, vc, idx, nsel, sinks


def _sdpa_with_sink(q, kg, vg, sinks, scale):
    """torch float64 scaled_dot_product_attention with the sink as one extra key per head.

    q [H, D]; kg, vg [n, D] gathered rows. For head h the extra key is
    q_h * sink_h / (scale * |q_h|^2), whose scaled logit equals sink_h, with a zero value row.
    """
    qt = torch.from_numpy(q)  # [H, D]
    H, D = qt.shape
    keys = torch.from_numpy(kg).unsqueeze(0).expand(H, -1, -1)
    vals = torch.from_numpy(vg).unsqueeze(0).expand(H, -1, -1)
    s = torch.from_numpy(sinks.astype(np.float64))
    finite = torch.isfinite(s)
    extra_k = torch.where(finite[:, None], qt * (s / (scale * (qt * qt).sum(1)))[:, None], torch.zeros_like(qt))
    kk = torch.cat([keys, extra_k[:, None, :]], 1)
    vv = torch.cat([vals, torch.zeros(H, 1, D, dtype=torch.float64)], 1)
    mask = torch.zeros(H, 1, kk.shape[1], dtype=torch.float64)
    mask[~finite, :, -1] = -math.inf  # a -inf sink removes the extra key
    out = torch.nn.functional.scaled_dot_product_attention(qt[:, None, :], kk, vv, attn_mask=mask, scale=scale)
    return out[:, 0, :].numpy()


# ----------------------------------------------------------------------------- attention pins

def pin_single_key(lib):
    """k = 1: o = v * sigmoid(s - sink) (closed form), s from numpy's dot product."""
    rng = np.random.default_rng(10)
    for dtype in ("f32", "bf16"):
        q, kc, vc, idx, nsel, sinks = _rand_case(rng, dtype, rows=2, heads=4, n=20, k=1)
        sinks[1] = -np.inf
        out = _att(lib, dtype, q, kc, vc, idx, nsel, sinks)
        for r in range(2):
            krow = _f64(dtype, kc[r, idx[r, 0]])
            vrow = _f64(dtype, vc[r, idx[r, 0]])
            for h in range(4):
                s = SCALE * float(np.dot(_f64(dtype, q[r, h]), krow))
                wgt = 1.0 / (1.0 + math.exp(float(sinks[h]) - s))
                np.testing.assert_allclose(out[r, h], vrow * wgt, rtol=1e-12, atol=1e-13)


def pin_equal_scores(lib):
    """q = 0: every score is 0, so o = sum(V_sel) / (n + e^sink); with sink = -inf, the mean."""
    rng = np.random.default_rng(11)
    for dtype in ("f32", "bf16"):
        q, kc, vc, idx, nsel, sinks = _rand_case(rng, dtype, rows=2, heads=3, n=50, k=9)
        q[:] = 0
        sinks[2] = -np.inf
        out = _att(lib, dtype, q, kc, vc, idx, nsel, sinks)
        for r in range(2):
            vs = _f64(dtype, vc[r, idx[r]]).sum(0)
            for h in range(3):
                np.testing.assert_allclose(out[r, h], vs / (9 + math.exp(float(sinks[h]))), rtol=1e-12, atol=1e-14)


def pin_exact_sums_k640(lib):
    """q = 0, sink = -inf, integer V in [-16, 16]: every sum is exact, o == sum(V_sel) / 640 exactly.

    Mirrors the "exact sums at k 640" gate of akol1/TensorFold pull request 4 (second commit message).
    """
    rng = np.random.default_rng(12)
    n, k = 4096, 640
    q = np.zeros((1, 2, w.D), np.uint16)
    kc = w.bf16_bits(rng.standard_normal((1, n, w.D), dtype=np.float32))
    vc = w.bf16_bits(rng.integers(-16, 17, size=(1, n, w.D)).astype(np.float32))
    idx = w.sorted_unique_indices(rng, n, k)[None]
    sinks = np.full(2, -np.inf, np.float32)
    out = _att(lib, "bf16", q, kc, vc, idx, None, sinks)
    exact = _f64("bf16", vc[0, idx[0]]).sum(0) / 640.0
    for h in range(2):
        assert np.array_equal(out[0, h], exact)


def pin_sdpa_library(lib):
    """torch float64 scaled_dot_product_attention over the gathered rows, sink as an extra key."""
    rng = np.random.default_rng(13)
    for dtype in ("f32", "bf16"):
        q, kc, vc, idx, nsel, sinks = _rand_case(rng, dtype, rows=3, heads=5, n=64, k=17)
        sinks[0] = -np.inf
        sinks[3] = 0.0
        out = _att(lib, dtype, q, kc, vc, idx, nsel, sinks)
        for r in range(3):
            ref = _sdpa_with_sink(_f64(dtype, q[r]), _f64(dtype, kc[r, idx[r]]), _f64(dtype, vc[r, idx[r]]),
                                  sinks, SCALE)
            np.testing.assert_allclose(out[r], ref, rtol=1e-10, atol=1e-12)


def pin_dense_bruteforce(lib):
    """Dense attention over every cache position with an explicit -inf mask plus a sink column."""
    rng = np.random.default_rng(14)
    for dtype, shared in (("f32", False), ("bf16", False), ("bf16", True)):
        q, kc, vc, idx, nsel, sinks = _rand_case(rng, dtype, rows=3, heads=4, n=32, k=11, shared=shared)
        nsel[1] = 5
        out = _att(lib, dtype, q, kc, vc, idx, nsel, sinks, shared=shared)
        for r in range(3):
            c = 0 if shared else r
            K = _f64(dtype, kc[c])
            V = _f64(dtype, vc[c])
            logits = SCALE * (_f64(dtype, q[r]) @ K.T)  # [H, N]
            mask = np.full(K.shape[0], -np.inf)
            mask[idx[r, :nsel[r]]] = 0.0
            full = np.concatenate([logits + mask, sinks.astype(np.float64)[:, None]], 1)
            full -= full.max(1, keepdims=True)
            p = np.exp(full)
            p /= p.sum(1, keepdims=True)
            ref = p[:, :-1] @ V
            np.testing.assert_allclose(out[r], ref, rtol=1e-10, atol=1e-12)


def pin_permutation(lib):
    """Permuting a row's selected indices changes only rounding (invariance to 1e-12)."""
    rng = np.random.default_rng(15)
    q, kc, vc, idx, nsel, sinks = _rand_case(rng, "bf16", rows=2, heads=3, n=300, k=130)
    a = _att(lib, "bf16", q, kc, vc, idx, nsel, sinks)
    idx2 = np.stack([rng.permutation(x) for x in idx])
    b = _att(lib, "bf16", q, kc, vc, idx2, nsel, sinks)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    assert not np.array_equal(idx, idx2)


def pin_duplicates(lib):
    """A repeated index counts twice: idx [a, a] gives o = v_a / (1 + e^(sink - s_a) / 2)."""
    rng = np.random.default_rng(16)
    q, kc, vc, idx, nsel, sinks = _rand_case(rng, "f32", rows=1, heads=2, n=10, k=2)
    idx[0, 1] = idx[0, 0]
    out = _att(lib, "f32", q, kc, vc, idx, nsel, sinks)
    krow = _f64("f32", kc[0, idx[0, 0]])
    vrow = _f64("f32", vc[0, idx[0, 0]])
    for h in range(2):
        s = SCALE * float(np.dot(_f64("f32", q[0, h]), krow))
        np.testing.assert_allclose(out[0, h], vrow / (1.0 + math.exp(float(sinks[h]) - s) / 2.0), rtol=1e-12)


def pin_empty_selection(lib):
    """nsel = 0: o = 0 / e^0 = 0 for a finite sink; 0/0 = NaN when the sink is -inf."""
    rng = np.random.default_rng(17)
    q, kc, vc, idx, nsel, sinks = _rand_case(rng, "bf16", rows=2, heads=3, n=16, k=4)
    nsel[:] = [0, 4]
    sinks[1] = -np.inf
    out = _att(lib, "bf16", q, kc, vc, idx, nsel, sinks)
    assert np.all(out[0, 0] == 0) and np.all(out[0, 2] == 0)
    assert np.all(np.isnan(out[0, 1]))
    assert np.all(np.isfinite(out[1]))


def pin_shared_vs_replicated(lib):
    """A shared cache (prefill) equals the same cache replicated per row (decode)."""
    rng = np.random.default_rng(18)
    q, kc, vc, idx, nsel, sinks = _rand_case(rng, "bf16", rows=3, heads=2, n=40, k=6, shared=True)
    a = _att(lib, "bf16", q, kc, vc, idx, nsel, sinks, shared=True)
    b = _att(lib, "bf16", q, np.repeat(kc, 3, 0), np.repeat(vc, 3, 0), idx, nsel, sinks, shared=False)
    assert np.array_equal(a, b)


def pin_out_of_range_index(lib):
    """An index outside [0, n_ctx) makes that row's output NaN; other rows are untouched."""
    rng = np.random.default_rng(19)
    q, kc, vc, idx, nsel, sinks = _rand_case(rng, "bf16", rows=2, heads=2, n=16, k=4)
    idx[0, 2] = 16
    out = _att(lib, "bf16", q, kc, vc, idx, nsel, sinks)
    assert np.all(np.isnan(out[0])) and np.all(np.isfinite(out[1]))
    idx[0, 2] = -1
    out = _att(lib, "bf16", q, kc, vc, idx, nsel, sinks)
    assert np.all(np.isnan(out[0]))


def pin_nonfinite_classes(lib):
    """The IEEE class table for one planted bad entry among the selected rows.

    K[i,e] = NaN     -> every head entirely NaN.
    K[i,e] = +inf    -> heads with q[h,e] > 0 entirely NaN (inf - inf); q[h,e] < 0: key i gets
                        weight 0, equal to dropping key i; -inf mirrors this.
    V[i,e] = NaN     -> column e NaN in every head; other columns as with V[i,e] = 0.
    V[i,e] = +inf    -> column e +inf where key i has weight > 0, NaN where its weight is 0 (0 * inf).
    V[i,e] = +inf and V[j,e] = -inf (both weighted) -> column e NaN.
    sink = +inf      -> NaN (exp(inf - inf)) for that head.
    """
    rng = np.random.default_rng(20)
    H, n, k, e = 6, 24, 5, 37
    q, kc, vc, idx, nsel, sinks = _rand_case(rng, "f32", rows=1, heads=H, n=n, k=k)
    q[0, :3, e] = np.abs(q[0, :3, e]) + 0.5   # heads 0-2: q > 0 at column e
    q[0, 3:, e] = -np.abs(q[0, 3:, e]) - 0.5  # heads 3-5: q < 0
    i = idx[0, 2]
    base = _att(lib, "f32", q, kc, vc, idx, nsel, sinks)
    drop = np.delete(idx, 2, 1)
    dropped = _att(lib, "f32", q, kc, vc, drop, np.array([k - 1], np.int32), sinks)

    kk = kc.copy(); kk[0, i, e] = np.nan
    out = _att(lib, "f32", q, kk, vc, idx, nsel, sinks)
    assert np.all(np.isnan(out))

    kk = kc.copy(); kk[0, i, e] = np.inf
    out = _att(lib, "f32", q, kk, vc, idx, nsel, sinks)
    assert np.all(np.isnan(out[0, :3]))
    np.testing.assert_allclose(out[0, 3:], dropped[0, 3:], rtol=1e-12)

    kk = kc.copy(); kk[0, i, e] = -np.inf
    out = _att(lib, "f32", q, kk, vc, idx, nsel, sinks)
    assert np.all(np.isnan(out[0, 3:]))
    np.testing.assert_allclose(out[0, :3], dropped[0, :3], rtol=1e-12)

    qz = q.copy(); qz[0, 0, e] = 0.0
    kk = kc.copy(); kk[0, i, e] = np.inf
    out = _att(lib, "f32", qz, kk, vc, idx, nsel, sinks)
    assert np.all(np.isnan(out[0, 0]))  # 0 * inf

    vv = vc.copy(); vv[0, i, e] = np.nan
    out = _att(lib, "f32", q, kc, vv, idx, nsel, sinks)
    assert np.all(np.isnan(out[0, :, e]))
    v0 = vc.copy(); v0[0, i, e] = 0.0
    ref = _att(lib, "f32", q, kc, v0, idx, nsel, sinks)
    other = np.arange(w.D) != e
    np.testing.assert_array_equal(out[0][:, other], ref[0][:, other])

    # Key i at weight zero in heads 3-5 only: K[i, f] = +inf with q[h, f] < 0 there gives s = -inf.
    f = 101
    qq = q.copy(); qq[0, :3, f] = 0.25; qq[0, 3:, f] = -0.25
    kk = kc.copy(); kk[0, i, f] = np.inf
    vv = vc.copy(); vv[0, i, e] = np.inf
    out = _att(lib, "f32", qq, kk, vv, idx, nsel, sinks)
    assert np.all(np.isnan(out[0, :3]))               # s = +inf there: whole head NaN
    assert np.all(np.isnan(out[0, 3:, e]))             # weight 0 times inf
    assert np.all(np.isfinite(out[0, 3:][:, other]))

    vv = vc.copy(); vv[0, i, e] = np.inf
    out = _att(lib, "f32", q, kc, vv, idx, nsel, sinks)
    assert np.all(out[0, :, e] == np.inf)
    vv[0, idx[0, 4], e] = -np.inf
    out = _att(lib, "f32", q, kc, vv, idx, nsel, sinks)
    assert np.all(np.isnan(out[0, :, e]))

    s2 = sinks.copy(); s2[4] = np.inf
    out = _att(lib, "f32", q, kc, vc, idx, nsel, s2)
    assert np.all(np.isnan(out[0, 4]))
    np.testing.assert_array_equal(np.delete(out[0], 4, 0), np.delete(base[0], 4, 0))


ATTENTION_PINS = [pin_single_key, pin_equal_scores, pin_exact_sums_k640, pin_sdpa_library,
                  pin_dense_bruteforce, pin_permutation, pin_duplicates, pin_empty_selection,
                  pin_shared_vs_replicated, pin_out_of_range_index, pin_nonfinite_classes]


# ----------------------------------------------------------------------------- top-k pins

def lexsort_topk(scores: np.ndarray, k: int, valid_len=None):
    """Second, independent top-k: numpy lexsort on (NaN flag, -score, position)."""
    R, n = scores.shape
    idx = np.full((R, k), -1, np.int32)
    cnt = np.zeros(R, np.int32)
    for r in range(R):
        vl = n if valid_len is None else int(np.clip(valid_len[r], 0, n))
        s = scores[r, :vl].astype(np.float64)
        nan = np.isnan(s)
        neg = np.where(nan, 0.0, -s)  # -0.0 and +0.0 compare equal in lexsort
        order = np.lexsort((np.arange(vl), neg, nan))
        sel = np.sort(order[:min(k, vl)])
        idx[r, :len(sel)] = sel
        cnt[r] = len(sel)
    return idx, cnt


def _check_topk(lib, scores, k, valid_len=None):
    got_i, got_c = oracle.topk(scores, k, valid_len, lib=lib)
    ref_i, ref_c = lexsort_topk(scores, k, valid_len)
    np.testing.assert_array_equal(got_c, ref_c)
    np.testing.assert_array_equal(got_i, ref_i)
    return got_i, got_c


def pin_topk_random(lib):
    """Random N(0,1) rows at the indexer shape (8 x 32,768, k = 640) against lexsort."""
    _check_topk(lib, w.indexer_scores(4), 640)


def pin_topk_distinct_argsort(lib):
    """Distinct scores: the selected set is numpy's argsort top-k (library routine)."""
    rng = np.random.default_rng(21)
    s = rng.permutation(5000).astype(np.float32)[None] * 0.5
    got, cnt = oracle.topk(s, 100, lib=lib)
    assert cnt[0] == 100
    np.testing.assert_array_equal(got[0], np.sort(np.argsort(-s[0], kind="stable")[:100]))


def pin_topk_ties(lib):
    """Scores rounded to multiples of 1/16 (many threshold ties) and all-equal rows."""
    _check_topk(lib, w.indexer_scores(5, rows=4, n=4096, tie_stress=True), 640)
    eq, cnt = oracle.topk(np.full((2, 1000), 0.5, np.float32), 37, lib=lib)
    np.testing.assert_array_equal(eq, np.tile(np.arange(37, dtype=np.int32), (2, 1)))


def pin_topk_signed_zero_nan(lib):
    """-0 ties +0 (lower position wins); NaN ranks below -inf; NaNs among themselves by position."""
    s = np.array([[np.nan, -0.0, 1.0, 0.0, -np.inf, np.nan, -0.0]], np.float32)
    got, _ = oracle.topk(s, 3, lib=lib)
    np.testing.assert_array_equal(got[0], [1, 2, 3])
    got, _ = oracle.topk(s, 6, lib=lib)
    np.testing.assert_array_equal(got[0], [0, 1, 2, 3, 4, 6])
    got, _ = oracle.topk(-s, 2, lib=lib)  # +inf, then +0/-0 at position 1
    np.testing.assert_array_equal(got[0], [1, 4])


def pin_topk_valid_len(lib):
    """Causal valid lengths (prefill: valid_len = pos + 1), k > valid_len and valid_len = 0."""
    rng = np.random.default_rng(22)
    s = rng.standard_normal((6, 3000), dtype=np.float32)
    vl = np.array([0, 1, 639, 640, 641, 3000], np.int32)
    got, cnt = _check_topk(lib, s, 640, vl)
    np.testing.assert_array_equal(cnt, [0, 1, 639, 640, 640, 640])
    assert np.all(got[0] == -1) and got[1, 0] == 0 and np.all(got[1, 1:] == -1)
    np.testing.assert_array_equal(got[2, :639], np.arange(639))
    assert got[2, 639] == -1


TOPK_PINS = [pin_topk_random, pin_topk_distinct_argsort, pin_topk_ties, pin_topk_signed_zero_nan,
             pin_topk_valid_len]
