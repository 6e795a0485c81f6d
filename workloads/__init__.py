"""Seeded synthetic inputs shaped like the sparse-attention workloads on the pages.

This module is shared by the oracle-side tests and by the GPU path's tests and
benchmark. It holds no attention or selection arithmetic: only random draws,
the storage-type rounding of those draws to bfloat16, index sampling and
nonfinite planting. Every array it returns is plain numpy on the host.

Shapes follow the pages: a 512-wide head made of sixteen 32-wide output column
groups and 64 attention heads (akol1/TensorFold pull request 4, "sparse
attention on eight SIMD groups, the same bytes", first commit message;
TensorFold pull request 1206, "What changes"), k = 640 selected positions
("exact sums at k 640", pull request 4, second commit message), cache lengths
of 4,096 and 32,768 and prefill segments of 2,048 rows (pull request 1206).

Draw order inside one seeded generator is fixed: q, k, v, sinks, the index
list of each row in row order, then nonfinite masks.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

D = 512
SCALE = 1.0 / math.sqrt(D)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return the bit patterns.

    NaN inputs become quiet NaNs with the same sign; infinities stay infinite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """Standard normal float32 draws, generated in chunks to bound host memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def _normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = bf16_bits(rng.standard_normal(e - s, dtype=np.float32))
    return out.reshape(shape)


def sorted_unique_indices(rng: np.random.Generator, n_pool: int, k: int) -> np.ndarray:
    """k distinct positions drawn uniformly from [0, n_pool), ascending, int32."""
    if k > n_pool:
        raise ValueError("k exceeds the pool")
    return np.sort(rng.choice(n_pool, size=k, replace=False)).astype(np.int32)


@dataclasses.dataclass
class AttnCase:
    """One attention call's inputs (host copies).

    dtype: "bf16" (q, k, v hold uint16 bit patterns) or "f32" (float32 arrays).
    q: [R, H, D]. k, v: [C, N, D] with C = R (decode: one cache per row) or
    C = 1 (prefill: one cache shared by all rows). idx: [R, kmax] int32, with
    -1 padding beyond nsel[r]. sinks: [H] float32.
    """
    name: str
    dtype: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    idx: np.ndarray
    nsel: np.ndarray
    sinks: np.ndarray
    scale: float
    shared_cache: bool
    positions: Optional[np.ndarray] = None

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def heads(self) -> int:
        return self.q.shape[1]

    @property
    def n_ctx(self) -> int:
        return self.k.shape[1]

    @property
    def kmax(self) -> int:
        return self.idx.shape[1]


def _pack_idx(lists, kmax: Optional[int] = None):
    kmax = max(1, max(len(x) for x in lists)) if kmax is None else kmax
    idx = np.full((len(lists), kmax), -1, dtype=np.int32)
    nsel = np.zeros(len(lists), dtype=np.int32)
    for r, x in enumerate(lists):
        idx[r, :len(x)] = x
        nsel[r] = len(x)
    return idx, nsel


def tiny_f32(seed: int = 0, heads: int = 4, n_ctx: int = 256, k: int = 64) -> AttnCase:
    """Tiny fp32 check: 1 row, 4 heads, N = 256, k = 64 sorted unique, N(0,1) data, seed 0."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (1, heads, D))
    kc = _normal(rng, (1, n_ctx, D))
    vc = _normal(rng, (1, n_ctx, D))
    sinks = rng.standard_normal(heads, dtype=np.float32)
    idx, nsel = _pack_idx([sorted_unique_indices(rng, n_ctx, k)])
    return AttnCase("tiny_f32", "f32", q, kc, vc, idx, nsel, sinks, SCALE, False)


def decode_bf16(seed: int = 1, batch: int = 1, heads: int = 64, n_ctx: int = 4096, k: int = 640,
                name: str = "decode") -> AttnCase:
    """Decode: `batch` independent sequences, each with its own n_ctx-position bf16 K/V cache."""
    rng = np.random.default_rng(seed)
    q = _normal_bf16(rng, (batch, heads, D))
    kc = _normal_bf16(rng, (batch, n_ctx, D))
    vc = _normal_bf16(rng, (batch, n_ctx, D))
    sinks = rng.standard_normal(heads, dtype=np.float32)
    idx, nsel = _pack_idx([sorted_unique_indices(rng, n_ctx, min(k, n_ctx)) for _ in range(batch)])
    return AttnCase(name, "bf16", q, kc, vc, idx, nsel, sinks, SCALE, False)


def decode_f32(seed: int = 6, batch: int = 1, heads: int = 64, n_ctx: int = 4096, k: int = 640,
               name: str = "decode_f32") -> AttnCase:
    """Decode with float32 storage: `batch` sequences, each with its own n_ctx-position cache."""
    rng = np.random.default_rng(seed)
    q = _normal(rng, (batch, heads, D))
    kc = _normal(rng, (batch, n_ctx, D))
    vc = _normal(rng, (batch, n_ctx, D))
    sinks = rng.standard_normal(heads, dtype=np.float32)
    idx, nsel = _pack_idx([sorted_unique_indices(rng, n_ctx, min(k, n_ctx)) for _ in range(batch)])
    return AttnCase(name, "f32", q, kc, vc, idx, nsel, sinks, SCALE, False)


def batched_decode_bf16(seed: int = 2, batch: int = 8, heads: int = 64, n_ctx: int = 32768,
                        k: int = 640) -> AttnCase:
    """Batched decode: 8 sequences with 32,768 cached positions each, k = 640 (or an edge k)."""
    return decode_bf16(seed, batch, heads, n_ctx, k, name=f"batched_decode_k{k}")


def prefill_bf16(seed: int = 3, rows: int = 2048, first_pos: int = 2048, heads: int = 64,
                 n_ctx: int = 4096, k: int = 640, row_stride: int = 1) -> AttnCase:
    """Prefill segment: rows at positions first_pos + t (t < rows) over one shared cache.

    Row t selects min(k, pos + 1) distinct positions uniformly from [0, pos], so
    every index is causal (<= the row's own position); the row itself is eligible.
    `row_stride` > 1 keeps every row_stride-th row of the segment (for small tests).
    """
    rng = np.random.default_rng(seed)
    pos = np.arange(first_pos, first_pos + rows * row_stride, row_stride, dtype=np.int64)
    if pos[-1] >= n_ctx:
        raise ValueError("prefill positions exceed the cache")
    q = _normal_bf16(rng, (rows, heads, D))
    kc = _normal_bf16(rng, (1, n_ctx, D))
    vc = _normal_bf16(rng, (1, n_ctx, D))
    sinks = rng.standard_normal(heads, dtype=np.float32)
    lists = [sorted_unique_indices(rng, int(p) + 1, min(k, int(p) + 1)) for p in pos]
    idx, nsel = _pack_idx(lists, kmax=k)
    return AttnCase("prefill", "bf16", q, kc, vc, idx, nsel, sinks, SCALE, True, positions=pos)


def plant_nonfinite_rows(rng: np.random.Generator, cache_bits: np.ndarray, p: float = 0.01) -> np.ndarray:
    """In each cache row, with probability p, set one uniformly chosen element to +inf, -inf or NaN.

    cache_bits: [C, N, D] bf16 bit patterns, modified in place. Returns the
    boolean mask [C, N] of planted rows. The class is drawn uniformly from the three.
    """
    c, n, d = cache_bits.shape
    hit = rng.random((c, n)) < p
    cols = rng.integers(0, d, size=(c, n))
    cls = rng.integers(0, 3, size=(c, n))
    special = np.array([0x7F80, 0xFF80, 0x7FC0], dtype=np.uint16)  # +inf, -inf, NaN
    ci, ni = np.nonzero(hit)
    cache_bits[ci, ni, cols[ci, ni]] = special[cls[ci, ni]]
    return hit


def indexer_scores(seed: int = 4, rows: int = 8, n: int = 32768, tie_stress: bool = False) -> np.ndarray:
    """Indexer scores ~N(0,1) float32 [rows, n]; tie_stress rounds them to multiples of 1/16."""
    rng = np.random.default_rng(seed)
    s = rng.standard_normal((rows, n), dtype=np.float32)
    if tie_stress:
        s = (np.round(s * 16.0) / 16.0).astype(np.float32)
    return s


def indexer_then_decode(seed: int = 4, batch: int = 8, heads: int = 64, n_ctx: int = 32768,
                        k: int = 640, p_bad: float = 0.01):
    """Indexer + attention: scores [batch, n_ctx] and a decode case whose K/V carry nonfinite rows.

    Returns (scores, case, bad_k, bad_v). case.idx is left empty (nsel = 0):
    the caller fills it with the top-k selection of `scores`.
    """
    rng = np.random.default_rng(seed)
    scores = rng.standard_normal((batch, n_ctx), dtype=np.float32)
    q = _normal_bf16(rng, (batch, heads, D))
    kc = _normal_bf16(rng, (batch, n_ctx, D))
    vc = _normal_bf16(rng, (batch, n_ctx, D))
    sinks = rng.standard_normal(heads, dtype=np.float32)
    bad_k = plant_nonfinite_rows(rng, kc, p_bad)
    bad_v = plant_nonfinite_rows(rng, vc, p_bad)
    idx = np.full((batch, k), -1, dtype=np.int32)
    nsel = np.zeros(batch, dtype=np.int32)
    case = AttnCase("indexer_decode", "bf16", q, kc, vc, idx, nsel, sinks, SCALE, False)
    return scores, case, bad_k, bad_v


EDGE_K = (1, 63, 64, 65, 639, 641)


def device_decode_inputs(torch, device, batch: int, heads: int, n_ctx: int, k: int, seed: int,
                         chunk_rows: int = 32):
    """Decode inputs generated on the device with a seeded torch generator.

    For shapes too large to draw on the host (1,024 sequences x 4,096 positions
    x 512 is 4 GiB per cache in bf16). Values are N(0,1) float32 draws rounded
    to bf16; each row's k indices are distinct and uniform over the cache
    (the first k of a random permutation), sorted ascending.
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32, bf = torch.float32, torch.bfloat16
    q = torch.randn((batch, heads, D), generator=g, device=device, dtype=f32).to(bf)
    kc = torch.empty((batch, n_ctx, D), dtype=bf, device=device)
    vc = torch.empty((batch, n_ctx, D), dtype=bf, device=device)
    for cache in (kc, vc):
        for b0 in range(0, batch, chunk_rows):
            b1 = min(batch, b0 + chunk_rows)
            cache[b0:b1] = torch.randn((b1 - b0, n_ctx, D), generator=g, device=device, dtype=f32).to(bf)
    sinks = torch.randn((heads,), generator=g, device=device, dtype=f32)
    perm = torch.rand((batch, n_ctx), generator=g, device=device).argsort(dim=1)[:, :k]
    idx = perm.sort(dim=1).values.to(torch.int32).contiguous()
    return {"q": q, "k": kc, "v": vc, "idx": idx, "sinks": sinks, "nsel": None}


def host_case_from_device(inp, row: int, name: str = "device_row") -> AttnCase:
    """Copy one row of device decode inputs (its query, its cache, its indices) to the host."""
    import torch

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    q = bits(inp["q"][row:row + 1])
    kc = bits(inp["k"][row:row + 1])
    vc = bits(inp["v"][row:row + 1])
    idx = inp["idx"][row:row + 1].cpu().numpy().astype(np.int32)
    sinks = inp["sinks"].cpu().numpy().astype(np.float32)
    nsel = np.full(1, idx.shape[1], np.int32)
    return AttnCase(name, "bf16", q, kc, vc, idx, nsel, sinks, SCALE, False)
