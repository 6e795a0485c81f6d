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


class _StubSA:
    """workspace_bytes as the library plans it: the split path below 24 (row, 64-head block)
    pairs with at most 1,024 indices per row."""
    @staticmethod
    def workspace_bytes(op, rows, heads, k, n_ctx):
        return 1 if k <= 1024 and rows * -(-heads // 64) < 24 else 0


class _StubTorch:
    class cuda:
        @staticmethod
        def get_device_properties(dev):
            class P:
                multi_processor_count = 256
            return P()


def test_decode_kernel_label_follows_the_launch_plan():
    lab = lambda rows, heads, alias=False: bench.decode_kernel_label(_StubTorch, _StubSA, None, rows, heads, 640,
                                                                   4096, alias)
    assert lab(1024, 64) == "attn_bf16_kernel<4,1> (sparse_attn_decode)"
    assert lab(1024, 64, True) == "attn_bf16_alias_kernel<4,1> (sparse_attn_decode, K = V)"
    assert lab(1024, 32) == "attn_bf16_kernel<2,1> (sparse_attn_decode)"
    assert lab(1024, 16) == "attn_bf16_kernel<1,1> (sparse_attn_decode)"
    assert lab(64, 64) == "attn_bf16_kernel<4,4> (sparse_attn_decode)"
    assert lab(24, 64) == "attn_bf16_kernel<4,8> (sparse_attn_decode)"
    assert lab(8, 64).startswith("attn_split_kernel")


def test_f32_kernel_label_follows_the_launch_rule():
    """The float32 bench line names the kernels the library launches: the split path below 24
    (row, 64-head block) pairs with 129 <= k <= 1,024, attn_f32_kernel otherwise."""
    split = "attn_f32_split_scores_kernel"
    assert bench.f32_kernel_label(8, 64, 640).startswith(split)
    assert bench.f32_kernel_label(23, 64, 640).startswith(split)
    assert bench.f32_kernel_label(24, 64, 640).startswith("attn_f32_kernel")
    assert bench.f32_kernel_label(64, 64, 640).startswith("attn_f32_kernel")
    assert bench.f32_kernel_label(8, 64, 128).startswith("attn_f32_kernel")
    assert bench.f32_kernel_label(8, 64, 1025).startswith("attn_f32_kernel")
    assert bench.f32_kernel_label(11, 128, 640).startswith(split)
    assert bench.f32_kernel_label(12, 128, 640).startswith("attn_f32_kernel")
