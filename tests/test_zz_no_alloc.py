"""sparse_attn_decode_noalloc (the decode call whose workspace is the library's static scratch, for
callers that cannot allocate) against sparse_attn_decode with a caller-allocated workspace, through
the C ABI: bit for bit on two calls in a row, the second with a smaller input, so the second call
runs on scratch that still holds the first call's contents, for the bf16 and the float32 split
paths. A large batch and a float32 call with a short index list (no workspace) go through it too."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import workloads as w
from parity import BF16_TOL, F32_TOL, assert_parity, run_oracle, to_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _call_both(case):
    import sparse_attention_attn_amd as sa
    from sparse_attention_attn_amd import _lib as L
    lib = L.load()
    d = to_device(case, DEV)
    code = L.SA_BF16 if case.dtype == "bf16" else L.SA_F32
    need = lib.sparse_attn_workspace_bytes(L.SA_OP_DECODE, case.rows, case.heads, 512, case.kmax, case.n_ctx)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ref = torch.full((case.rows, case.heads, 512), 7.0, device=DEV)
    got = torch.full((case.rows, case.heads, 512), 9.0, device=DEV)
    args = (code, d["q"].data_ptr(), d["k"].data_ptr(), d["v"].data_ptr(), case.n_ctx, d["idx"].data_ptr(),
            d["nsel"].data_ptr(), case.kmax, d["sinks"].data_ptr(), float(case.scale), case.rows, case.heads, 512)
    rc = lib.sparse_attn_decode(*args, ref.data_ptr(), ws.data_ptr() if need else None, need, stream)
    assert rc == L.SA_OK, lib.sparse_attn_last_error()
    rc = lib.sparse_attn_decode_noalloc(*args, got.data_ptr(), stream)
    assert rc == L.SA_OK, lib.sparse_attn_last_error()
    torch.cuda.synchronize()
    return need, ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("first,second", [
    # split path (scores through the workspace), then a smaller split launch
    (dict(seed=500, batch=8, heads=64, n_ctx=4096, k=640), dict(seed=501, batch=2, heads=48, n_ctx=1000, k=300)),
    (dict(seed=502, batch=23, heads=64, n_ctx=2000, k=1024), dict(seed=503, batch=1, heads=16, n_ctx=700, k=65)),
])
def test_noalloc_equals_decode_twice(first, second):
    for i, kw in enumerate((first, second)):
        case = w.decode_bf16(**kw)
        if i == 1:
            case.nsel[0] = kw["k"] // 2
            case.idx[0, kw["k"] // 2:] = -1
        say(f"call {i + 1}: B={case.rows} H={case.heads} N={case.n_ctx} k={case.kmax}")
        need, ref, got = _call_both(case)
        assert need > 0, "expected the split path (a workspace)"
        assert np.array_equal(ref.view(np.int32), got.view(np.int32)), f"call {i + 1}: noalloc differs from decode"
        rows = [0, case.rows - 1]
        st = assert_parity(got[rows], run_oracle(case, rows=rows)[rows], *BF16_TOL, f"noalloc call {i + 1}")
        say(f"  ok (bit-equal to sparse_attn_decode) {st}")


def test_noalloc_f32_split_twice():
    """The float32 split path (score tiles through the scratch), then a smaller float32 split launch."""
    for i, kw in enumerate((dict(seed=505, batch=8, heads=64, n_ctx=4096, k=640),
                            dict(seed=506, batch=2, heads=32, n_ctx=1000, k=300))):
        case = w.decode_f32(**kw)
        if i == 1:
            case.nsel[0] = kw["k"] // 2
            case.idx[0, kw["k"] // 2:] = -1
        say(f"f32 call {i + 1}: B={case.rows} H={case.heads} N={case.n_ctx} k={case.kmax}")
        need, ref, got = _call_both(case)
        assert np.array_equal(ref.view(np.int32), got.view(np.int32)), f"f32 call {i + 1}: noalloc differs"
        rows = [0, case.rows - 1]
        st = assert_parity(got[rows], run_oracle(case, rows=rows)[rows], *F32_TOL, f"noalloc f32 call {i + 1}")
        say(f"  ok (bit-equal to sparse_attn_decode) {st}")


def test_noalloc_without_workspace_paths():
    """Calls that need no workspace (a large batch on the persistent kernels, and float32 with a
    short index list) go through unchanged."""
    case = w.decode_bf16(seed=504, batch=64, heads=64, n_ctx=700, k=200)
    need, ref, got = _call_both(case)
    assert need == 0 and np.array_equal(ref.view(np.int32), got.view(np.int32))
    case = w.tiny_f32()
    need, ref, got = _call_both(case)
    assert np.array_equal(ref.view(np.int32), got.view(np.int32))
    assert_parity(got, run_oracle(case), *F32_TOL, "noalloc f32")
