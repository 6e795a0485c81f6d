"""Plausible mistakes planted in copies of the oracle must each fail at least one pin.

Each mutant is a one-line textual change to oracle.c (a dropped term, a wrong
sign, a wrong index, a wrong order), compiled on the CPU into its own library.
The real oracle passes every pin (tests/test_oracle_pins.py); a mutant that
passed them all would show a blind spot in the pins.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ATTENTION_PINS, TOPK_PINS

MUTANTS = {
    "sink_scaled": ("double sink = (double)sinks[h];", "double sink = scale * (double)sinks[h];"),
    "sink_dropped_from_Z": ("double z = exp(sink - m);", "double z = 0.0;"),
    "sink_sign": ("double z = exp(sink - m);", "double z = exp(-sink - m);"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "key_gather_first_index": ("const int64_t k_base = cache_base + (int64_t)idx[j] * D;",
                               "const int64_t k_base = cache_base + (int64_t)idx[0] * D;"),
    "value_not_gathered": ("widen(vc, dtype, cache_base + (int64_t)idx[j] * D + e)",
                           "widen(vc, dtype, cache_base + (int64_t)j * D + e)"),
    "q_head_transposed": ("const int64_t q_base = (r * H + h) * D;", "const int64_t q_base = (h * H + r) * D;"),
    "decode_cache_ignored": ("const int64_t cache_base = r * cache_rows_stride * D;",
                             "const int64_t cache_base = 0;"),
    "weight_sign": ("num += exp(s[j] - m) *", "num += exp(m - s[j]) *"),
    "max_ignores_sink": ("double m = sink;", "double m = -INFINITY;"),
    "oob_not_checked": ("if (idx[j] < 0 || (int64_t)idx[j] >= n_ctx) {", "if (0) {"),
    "topk_tie_high_index": ("return (a->j > b->j) - (a->j < b->j);", "return (a->j < b->j) - (a->j > b->j);"),
    "topk_nan_high": ("return an ? 1 : -1;", "return an ? -1 : 1;"),
    "topk_unsorted_output": ("qsort(sel, (size_t)cnt, sizeof(int32_t), int_cmp);", ";"),
    "topk_valid_len_off_by_one": ("int64_t vl = valid_len ? (int64_t)valid_len[r] : n;",
                                  "int64_t vl = valid_len ? (int64_t)valid_len[r] - 1 : n;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    lib_path = obuild.build(str(mpath), str(tmp_path / "libmutant.so"))
    lib = oracle.load(lib_path)
    failed = []
    for pin in ATTENTION_PINS + TOPK_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
