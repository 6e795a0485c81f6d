"""Comparison of GPU outputs against the float64 oracle, and host<->device plumbing.

Bar: nonfinite classes (NaN, +inf, -inf, finite) must match element by element, and
every finite element must satisfy |gpu - oracle| <= atol: the maximum absolute error
is 2e-3 for bf16 inputs and 1e-5 for float32 inputs. For bf16 this also bounds the
relative error by 1e-2 wherever |oracle| >= 0.2; below that a relative bound is not
meaningful (outputs cancel towards zero), so max rel error is reported, not imposed.
"""
from __future__ import annotations

import numpy as np

BF16_TOL = (2e-3, 1e-2)
F32_TOL = (1e-5, 1e-5)


def tol_for(dtype: str):
    return BF16_TOL if dtype == "bf16" else F32_TOL


def classes(x: np.ndarray) -> np.ndarray:
    return np.where(np.isnan(x), 3, np.where(np.isposinf(x), 1, np.where(np.isneginf(x), 2, 0)))


def assert_parity(gpu, ref, atol: float, rtol: float, label: str = "") -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    cg, cr = classes(gpu), classes(ref)
    mism = cg != cr
    if mism.any():
        at = tuple(np.argwhere(mism)[0])
        raise AssertionError(f"{label}: {int(mism.sum())} nonfinite-class mismatches; first at {at}: "
                             f"gpu={gpu[at]!r} oracle={ref[at]!r}")
    fin = cr == 0
    g, o = gpu[fin], ref[fin]
    err = np.abs(g - o)
    stats = {"n": int(fin.sum()), "nonfinite": int((~fin).sum()),
             "max_abs": float(err.max()) if err.size else 0.0,
             "max_rel": float((err / np.maximum(np.abs(o), 1e-30)).max()) if err.size else 0.0}
    bad = err > atol
    big = np.abs(o) >= atol / rtol
    stats["max_rel_where_large"] = float((err[big] / np.abs(o[big])).max()) if big.any() else 0.0
    if bad.any():
        idx = np.flatnonzero(fin)[np.flatnonzero(bad)[0]]
        at = np.unravel_index(idx, gpu.shape)
        raise AssertionError(f"{label}: {int(bad.sum())} elements outside tolerance; first at {tuple(at)}: "
                             f"gpu={gpu[at]!r} oracle={ref[at]!r}; {stats}")
    return stats


def to_device(case, device):
    """Upload an AttnCase; returns dict of tensors (prefill caches are [N, D])."""
    import torch

    def t(a):
        if case.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    k = case.k[0] if case.shared_cache else case.k
    v = case.v[0] if case.shared_cache else case.v
    kt = t(k)
    # A case whose V is its K array runs on one device tensor (the aliased-cache path).
    vt = kt if case.v is case.k else t(v)
    return {"q": t(case.q), "k": kt, "v": vt,
            "idx": torch.from_numpy(np.ascontiguousarray(case.idx, dtype=np.int32)).to(device),
            "nsel": torch.from_numpy(np.ascontiguousarray(case.nsel, dtype=np.int32)).to(device),
            "sinks": torch.from_numpy(np.ascontiguousarray(case.sinks, dtype=np.float32)).to(device)}


def run_gpu(case, device="cuda:0", with_nsel=True):
    """Run decode (per-row caches) or prefill (shared cache) for an AttnCase; returns numpy float32."""
    import torch

    import sparse_attention_attn_amd as sa
    d = to_device(case, device)
    fn = sa.prefill if case.shared_cache else sa.decode
    out = fn(d["q"], d["k"], d["v"], d["idx"], d["sinks"], case.scale, d["nsel"] if with_nsel else None)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def run_oracle(case, rows=None, threads=0):
    import oracle
    return oracle.attention(case.dtype, case.q, case.k, case.v, case.idx, case.nsel, case.sinks, case.scale,
                            case.shared_cache, rows=rows, threads=threads)
