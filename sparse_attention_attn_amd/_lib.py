"""ctypes loader for libsparse_attn.so (the C ABI in include/sparse_attn.h).

No fallback exists: if the library is missing or cannot be loaded, every call
raises. Build it with sparse_attention_attn_amd/build.py (or __graft_entry__.build()).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparse_attn.so")

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(6)
SA_F32, SA_BF16 = 0, 1
SA_OP_DECODE, SA_OP_PREFILL, SA_OP_TOPK = 0, 1, 2
SA_HEAD_DIM, SA_MAX_HEADS, SA_BF16_MAX_CTX, SA_MAX_KMAX = 512, 128, 4194303, 1 << 24
SA_F32_MAX_CTX = 2097151
SA_ABI_VERSION = 2
SA_NOALLOC_SCRATCH_BYTES = 8 << 20

_c = ctypes
_P = _c.c_void_p
_I32, _I64, _F, _SZ = _c.c_int32, _c.c_int64, _c.c_float, _c.c_size_t

# name -> (restype, argtypes); the same list the header declares.
SIGNATURES = {
    "sparse_attn_abi_version": (_c.c_int, []),
    "sparse_attn_status_string": (_c.c_char_p, [_c.c_int]),
    "sparse_attn_last_error": (_c.c_char_p, []),
    "sparse_attn_workspace_bytes": (_SZ, [_c.c_int, _I64, _I32, _I32, _I32, _I64]),
    "sparse_attn_decode": (_c.c_int, [_c.c_int, _P, _P, _P, _I64, _P, _P, _I32, _P, _F, _I32, _I32, _I32,
                                      _P, _P, _SZ, _P]),
    "sparse_attn_prefill": (_c.c_int, [_c.c_int, _P, _P, _P, _I64, _P, _P, _I32, _P, _F, _I32, _I32, _I32,
                                       _P, _P, _SZ, _P]),
    "sparse_attn_decode_noalloc": (_c.c_int, [_c.c_int, _P, _P, _P, _I64, _P, _P, _I32, _P, _F, _I32, _I32,
                                              _I32, _P, _P]),
    "sparse_attn_topk": (_c.c_int, [_P, _I64, _I64, _I64, _P, _I32, _P, _P, _P, _SZ, _P]),
    "sparse_attn_gather_probe": (_c.c_int, [_P, _P, _I64, _P, _I32, _I32, _I32, _P]),
    "sparse_attn_pad_heads": (_c.c_int, [_c.c_int, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _P]),
    "sparse_attn_unpad_heads": (_c.c_int, [_P, _I64, _I32, _I32, _I32, _P, _P]),
}

_lib = None


class SparseAttnError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        super().__init__(f"{where}: status {code} ({detail})")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once) and attach the C signatures; raises if it is missing."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run `python sparse_attention_attn_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.sparse_attn_abi_version() != SA_ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.sparse_attn_abi_version()}, this binding "
                           f"expects {SA_ABI_VERSION}; rebuild it")
    if path == LIB_PATH:
        _lib = lib
    return lib


def check(code: int, where: str, lib=None) -> None:
    if code != SA_OK:
        lib = lib or load()
        detail = lib.sparse_attn_last_error().decode() or lib.sparse_attn_status_string(code).decode()
        raise SparseAttnError(code, where, detail)
