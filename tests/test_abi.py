"""The C-ABI library loads without a GPU, exports every declared symbol, and rejects
invalid arguments on the host before anything is enqueued (no compute calls here)."""
import os
import re

import pytest

from sparse_attention_attn_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libsparse_attn.so not built")

A16 = 0x10000  # fake, 16-byte aligned device addresses: never dereferenced by these calls


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sparse_attn_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == sorted(L.SIGNATURES)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("SA_HEAD_DIM", "SA_MAX_HEADS", "SA_BF16_MAX_CTX", "SA_F32_MAX_CTX", "SA_ABI_VERSION"):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, text)
        assert m and int(m.group(1)) == getattr(L, name), name
    m = re.search(r"#define\s+SA_MAX_KMAX\s+\(1 << (\d+)\)", text)
    assert m and 1 << int(m.group(1)) == L.SA_MAX_KMAX
    m = re.search(r"#define\s+SA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == L.SA_NOALLOC_SCRATCH_BYTES


def test_every_declared_symbol_is_exported():
    lib = L.load()
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = L.load()
    assert lib.sparse_attn_abi_version() == L.SA_ABI_VERSION == 2
    for code in range(6):
        assert lib.sparse_attn_status_string(code)
    assert lib.sparse_attn_status_string(99) == b"unknown status"


SYNC = 24 * 32 * 8       # sync words: 32 of 8 bytes per (row, 64-head block), at most 24 pairs
TILE = 4096 + 128        # one score tile and its maxima


@pytest.mark.parametrize("op,rows,heads,kmax,expect", [
    # large batches: the persistent kernels, no workspace
    (L.SA_OP_DECODE, 1024, 64, 640, 0),
    (L.SA_OP_DECODE, 64, 64, 640, 0),
    (L.SA_OP_DECODE, 24, 64, 640, 0),
    (L.SA_OP_DECODE, 12, 128, 640, 0),
    (L.SA_OP_PREFILL, 2048, 16, 640, 0),
    # small batches: 6 KiB of sync words, then a 4 KiB score tile and 128 bytes of tile maxima
    # per (row, 64-key tile, 16-head group)
    (L.SA_OP_DECODE, 1, 64, 640, SYNC + 1 * 10 * 4 * TILE),
    (L.SA_OP_DECODE, 8, 64, 641, SYNC + 8 * 11 * 4 * TILE),
    (L.SA_OP_DECODE, 23, 64, 1, SYNC + 23 * 1 * 4 * TILE),
    (L.SA_OP_PREFILL, 11, 128, 64, SYNC + 11 * 1 * 8 * TILE),
    (L.SA_OP_DECODE, 2, 4, 64, SYNC + 2 * 1 * 1 * TILE),
    (L.SA_OP_DECODE, 2, 17, 1024, SYNC + 2 * 16 * 2 * TILE),
    # index lists longer than 1,024 entries stay on the persistent kernels
    (L.SA_OP_DECODE, 1, 64, 1025, 0),
    # top-k and invalid sizes: none
    (L.SA_OP_TOPK, 1, 64, 640, 0),
    (L.SA_OP_DECODE, 0, 64, 640, 0),
    (L.SA_OP_DECODE, 1, 0, 640, 0),
    (L.SA_OP_DECODE, 1, 64, 0, 0),
])
def test_workspace_bytes(op, rows, heads, kmax, expect):
    lib = L.load()
    assert lib.sparse_attn_workspace_bytes(op, rows, heads, 512, kmax, 4096) == expect


def _decode(lib, **kw):
    args = dict(dtype=L.SA_BF16, q=A16, k=A16, v=A16, n_ctx=4096, idx=A16, nsel=None, kmax=640, sinks=A16,
                scale=0.044, rows=1024, H=64, D=512, out=A16, ws=None, ws_bytes=0, stream=None)
    args.update(kw)
    return lib.sparse_attn_decode(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), L.SA_ERR_NULL),
    (dict(k=None), L.SA_ERR_NULL),
    (dict(out=None), L.SA_ERR_NULL),
    (dict(sinks=None), L.SA_ERR_NULL),
    (dict(idx=None), L.SA_ERR_NULL),
    (dict(D=256), L.SA_ERR_UNSUPPORTED),
    (dict(dtype=7), L.SA_ERR_UNSUPPORTED),
    (dict(H=0), L.SA_ERR_SHAPE),
    (dict(H=129), L.SA_ERR_SHAPE),
    (dict(rows=-1), L.SA_ERR_SHAPE),
    (dict(kmax=0), L.SA_ERR_SHAPE),
    (dict(kmax=L.SA_MAX_KMAX + 1), L.SA_ERR_SHAPE),
    (dict(kmax=2 ** 31 - 1), L.SA_ERR_SHAPE),
    (dict(rows=8, ws=A16, ws_bytes=SYNC + 8 * 10 * 4 * TILE - 1), L.SA_ERR_WORKSPACE),
    (dict(rows=8), L.SA_ERR_WORKSPACE),
    (dict(rows=8, ws=None, ws_bytes=SYNC + 8 * 10 * 4 * TILE), L.SA_ERR_NULL),
    (dict(rows=8, ws=A16 + 8, ws_bytes=SYNC + 8 * 10 * 4 * TILE), L.SA_ERR_UNSUPPORTED),
    (dict(n_ctx=0), L.SA_ERR_SHAPE),
    (dict(n_ctx=4194304), L.SA_ERR_UNSUPPORTED),  # bf16 caches: at most 2^22 - 1 positions
    (dict(dtype=L.SA_F32, n_ctx=2097152), L.SA_ERR_UNSUPPORTED),  # float32 caches: at most 2^21 - 1
    (dict(q=A16 + 8), L.SA_ERR_UNSUPPORTED),
    (dict(out=A16 + 4), L.SA_ERR_UNSUPPORTED),
    (dict(idx=A16 + 2), L.SA_ERR_UNSUPPORTED),
])
def test_decode_validation(kw, code):
    lib = L.load()
    assert _decode(lib, **kw) == code
    assert lib.sparse_attn_last_error()  # a message names the problem


def test_prefill_validation():
    lib = L.load()
    args = [L.SA_BF16, A16, A16, A16, 4096, A16, None, 640, A16, 0.04, 2048, 64, 512, A16, None, 0, None]
    bad = list(args); bad[12] = 128
    assert lib.sparse_attn_prefill(*bad) == L.SA_ERR_UNSUPPORTED
    bad = list(args); bad[1] = None
    assert lib.sparse_attn_prefill(*bad) == L.SA_ERR_NULL


def test_topk_validation():
    lib = L.load()
    ok = [A16, 8, 32768, 32768, None, 640, A16, A16, None, 0, None]
    for i, val, code in [(0, None, L.SA_ERR_NULL), (6, None, L.SA_ERR_NULL), (5, 0, L.SA_ERR_SHAPE),
                         (3, 100, L.SA_ERR_SHAPE), (1, -1, L.SA_ERR_SHAPE), (2, -5, L.SA_ERR_SHAPE),
                         (0, A16 + 2, L.SA_ERR_UNSUPPORTED)]:
        bad = list(ok); bad[i] = val
        assert lib.sparse_attn_topk(*bad) == code, (i, val)


def test_pad_validation():
    lib = L.load()
    assert lib.sparse_attn_pad_heads(L.SA_BF16, A16, 10, 16, 8, 512, A16, A16, A16, None) == L.SA_ERR_SHAPE
    assert lib.sparse_attn_pad_heads(L.SA_BF16, A16, 10, 16, 32, 500, A16, A16, A16, None) == L.SA_ERR_UNSUPPORTED
    assert lib.sparse_attn_pad_heads(L.SA_BF16, None, 10, 16, 32, 512, A16, A16, A16, None) == L.SA_ERR_NULL
    assert lib.sparse_attn_unpad_heads(A16, 10, 32, 33, 512, A16, None) == L.SA_ERR_SHAPE
    assert lib.sparse_attn_unpad_heads(A16, 10, 32, 16, 512, None, None) == L.SA_ERR_NULL


def test_python_binding_refuses_cpu_tensors():
    import torch
    import sparse_attention_attn_amd as sa
    q = torch.zeros(1, 4, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sa.decode(q, torch.zeros(1, 8, 512, dtype=torch.bfloat16), torch.zeros(1, 8, 512, dtype=torch.bfloat16),
                  torch.zeros(1, 4, dtype=torch.int32), torch.zeros(4), 0.04)


@pytest.fixture
def stub_library(monkeypatch):
    """The binding with a library object that fails the test if any entry point is reached:
    every refusal below must happen in argument checking, before a pointer is passed."""
    import sparse_attention_attn_amd as sa

    class Stub:
        def __getattr__(self, name):
            raise AssertionError(f"{name} was called for arguments the binding must refuse")

    monkeypatch.setattr(sa, "load", lambda *a, **k: Stub())
    return sa


def _attn_args(dev_of=None, **over):
    import torch
    t = {
        "q": torch.zeros(2, 4, 512, dtype=torch.bfloat16),
        "k_cache": torch.zeros(2, 8, 512, dtype=torch.bfloat16),
        "v_cache": torch.zeros(2, 8, 512, dtype=torch.bfloat16),
        "idx": torch.zeros(2, 4, dtype=torch.int32),
        "sinks": torch.zeros(4),
        "nsel": torch.zeros(2, dtype=torch.int32),
        "out": torch.zeros(2, 4, 512),
        "ws": torch.zeros(4096, dtype=torch.uint8),
    }
    if dev_of:
        t[dev_of] = t[dev_of].to("meta")
    t.update(over)
    return t


@pytest.mark.parametrize("name", ["k_cache", "v_cache", "idx", "sinks", "nsel", "out", "ws"])
def test_binding_refuses_a_tensor_on_another_device(stub_library, name):
    """A tensor on another device than q is refused before the library is reached, the outputs
    and the workspace included (a host pointer must never reach a kernel)."""
    sa = stub_library
    t = _attn_args(dev_of=name)
    with pytest.raises(ValueError, match=name):
        sa.decode(t["q"], t["k_cache"], t["v_cache"], t["idx"], t["sinks"], 0.04, nsel=t["nsel"], out=t["out"],
                  ws=t["ws"])


def test_binding_refuses_host_tensors_everywhere(stub_library):
    import torch
    sa = stub_library
    t = _attn_args()
    with pytest.raises(ValueError, match="HIP device"):
        sa.prefill(t["q"], t["k_cache"][0], t["v_cache"][0], t["idx"], t["sinks"], 0.04)
    s = torch.zeros(2, 100)
    with pytest.raises(ValueError, match="HIP device"):
        sa.topk(s, 10)
    for name, kw in (("valid_len", dict(valid_len=torch.zeros(2, dtype=torch.int32, device="meta"))),
                     ("idx_out", dict(idx_out=torch.zeros(2, 10, dtype=torch.int32, device="meta"))),
                     ("count_out", dict(count_out=torch.zeros(2, dtype=torch.int32, device="meta")))):
        with pytest.raises(ValueError, match=name):
            sa.topk(s, 10, **kw)
    for name, kw in (("sinks", dict(sinks=torch.zeros(4, device="meta"))),
                     ("q_pad", dict(q_pad=torch.zeros(2, 8, 512, dtype=torch.bfloat16, device="meta"))),
                     ("s_pad", dict(s_pad=torch.zeros(8, device="meta")))):
        args = dict(sinks=t["sinks"])
        args.update(kw)
        sinks = args.pop("sinks")
        with pytest.raises(ValueError, match=name):
            sa.pad_heads(t["q"], sinks, 8, **args)
    with pytest.raises(ValueError, match="HIP device"):
        sa.pad_heads(t["q"], t["sinks"], 8)
    with pytest.raises(ValueError, match="out"):
        sa.unpad_heads(torch.zeros(2, 8, 512), 4, out=torch.zeros(2, 4, 512, device="meta"))
    with pytest.raises(ValueError, match="HIP device"):
        sa.unpad_heads(torch.zeros(2, 8, 512), 4)


def test_noalloc_scratch_covers_every_split_launch():
    """The allocation-free decode's static scratch holds the workspace of every launch that takes
    the split path (at most 1,024 indices per row, fewer than 24 rows per block of 64 heads)."""
    lib = L.load()
    worst = max(lib.sparse_attn_workspace_bytes(L.SA_OP_DECODE, rows, heads, 512, 1024, 4096)
                for heads in range(1, L.SA_MAX_HEADS + 1) for rows in range(1, 64))
    assert 0 < worst <= L.SA_NOALLOC_SCRATCH_BYTES


def test_noalloc_validation():
    lib = L.load()
    args = [L.SA_BF16, A16, A16, A16, 4096, A16, None, 640, A16, 0.04, 1024, 64, 512, A16, None]
    bad = list(args); bad[12] = 256
    assert lib.sparse_attn_decode_noalloc(*bad) == L.SA_ERR_UNSUPPORTED
    bad = list(args); bad[1] = None
    assert lib.sparse_attn_decode_noalloc(*bad) == L.SA_ERR_NULL
    bad = list(args); bad[7] = 0
    assert lib.sparse_attn_decode_noalloc(*bad) == L.SA_ERR_SHAPE
    # Float32 at split-path sizes: the workspace is worked out only for valid sizes, so invalid
    # ones get their own status (nothing is launched for any of these).
    f32 = [L.SA_F32, A16, A16, A16, 4096, A16, None, 640, A16, 0.04, 8, 64, 512, A16, None]
    for i, val, code in [(10, -1, L.SA_ERR_SHAPE), (11, 0, L.SA_ERR_SHAPE), (7, 0, L.SA_ERR_SHAPE),
                         (1, None, L.SA_ERR_NULL), (12, 256, L.SA_ERR_UNSUPPORTED)]:
        bad = list(f32); bad[i] = val
        assert lib.sparse_attn_decode_noalloc(*bad) == code, (i, val)
    zero = list(f32); zero[10] = 0
    assert lib.sparse_attn_decode_noalloc(*zero) == L.SA_OK


def test_gather_probe_validation():
    lib = L.load()
    ok = [A16, A16, 4096, A16, 8, 640, 16, None]
    for i, val, code in [(0, None, L.SA_ERR_NULL), (3, None, L.SA_ERR_NULL), (6, 4, L.SA_ERR_UNSUPPORTED),
                         (5, 0, L.SA_ERR_SHAPE), (2, 0, L.SA_ERR_SHAPE), (4, -1, L.SA_ERR_SHAPE)]:
        bad = list(ok); bad[i] = val
        assert lib.sparse_attn_gather_probe(*bad) == code, (i, val)
    assert lib.sparse_attn_gather_probe(None, None, 4096, None, 0, 640, 8, None) == L.SA_OK


def test_zero_rows_is_a_noop_with_null_arrays():
    lib = L.load()
    assert _decode(lib, q=None, k=None, v=None, idx=None, out=None, rows=0) == L.SA_OK
    assert lib.sparse_attn_prefill(L.SA_BF16, None, A16, A16, 10, None, None, 4, A16, 0.1, 0, 64, 512,
                                   None, None, 0, None) == L.SA_OK
    assert lib.sparse_attn_topk(None, 0, 100, 100, None, 10, None, None, None, 0, None) == L.SA_OK
    assert _decode(lib, rows=0, D=256) == L.SA_ERR_UNSUPPORTED  # sizes are still checked
