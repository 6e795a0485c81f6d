"""Host logic of bench.py: the kernel-code hash that decides whether the committed HBM-traffic
counters still apply (comments and blank lines do not count; code does)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return str(p)


def test_code_hash_ignores_comments_and_blank_lines(tmp_path):
    a = _write(tmp_path, "a.hip", "int f(int x) {\n    return x + 1;\n}\n")
    b = _write(tmp_path, "b.hip", "// a comment\nint f(int x) {  /* inline */\n\n    return x + 1;  // why\n}\n\n")
    assert bench.kernel_code_sha256([a]) == bench.kernel_code_sha256([b])


def test_code_hash_sees_code_changes_and_file_order(tmp_path):
    a = _write(tmp_path, "a.hip", "int f(int x) {\n    return x + 1;\n}\n")
    c = _write(tmp_path, "c.hip", "int f(int x) {\n    return x + 2;\n}\n")
    d = _write(tmp_path, "d.h", "#define K 64\n")
    assert bench.kernel_code_sha256([a]) != bench.kernel_code_sha256([c])
    assert bench.kernel_code_sha256([a, d]) != bench.kernel_code_sha256([d, a])


def test_traffic_only_for_the_recorded_workload():
    assert bench.measured_traffic(8, 64, 32768, 640) is None
    assert bench.measured_traffic(1024, 16, 4096, 640) is None
