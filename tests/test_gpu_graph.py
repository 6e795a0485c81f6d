"""The entry points only enqueue kernels on the caller's stream and allocate nothing (when the
caller passes the outputs), so a whole step, top-k then attention, can be captured in a HIP
graph and replayed. Each replay runs after new inputs are copied into the captured buffers
and after eager work (the same step on separate buffers) with synchronisations in between;
every replay must equal that eager result bit for bit."""
import sys

import pytest
import torch

import workloads as w

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("shared", [False, True], ids=["decode", "prefill"])
def test_captured_step_replays_equal_eager(shared):
    import sparse_attention_attn_amd as sa
    rows, H, N, K = (256, 64, 4096, 640) if shared else (64, 64, 2048, 640)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(17 + int(shared))
    cache_shape = (N, 512) if shared else (rows, N, 512)

    def draw():
        return {
            "q": torch.randn((rows, H, 512), generator=gen, device=DEV).to(torch.bfloat16),
            "k": torch.randn(cache_shape, generator=gen, device=DEV).to(torch.bfloat16),
            "v": torch.randn(cache_shape, generator=gen, device=DEV).to(torch.bfloat16),
            "sinks": torch.randn((H,), generator=gen, device=DEV),
            "scores": torch.randn((rows, N), generator=gen, device=DEV),
        }

    # Prefill rows sit at the last positions of the cache (causal valid lengths).
    valid_len = torch.arange(N - rows + 1, N + 1, dtype=torch.int32, device=DEV) if shared else None
    attend = sa.prefill if shared else sa.decode
    bufs = draw()
    idx = torch.empty((rows, K), dtype=torch.int32, device=DEV)
    cnt = torch.empty((rows,), dtype=torch.int32, device=DEV)
    out = torch.empty((rows, H, 512), dtype=torch.float32, device=DEV)

    def step():
        sa.topk(bufs["scores"], K, valid_len=valid_len, idx_out=idx, count_out=cnt)
        attend(bufs["q"], bufs["k"], bufs["v"], idx, bufs["sinks"], w.SCALE, cnt, out=out)

    def eager(inp):
        i2, c2 = sa.topk(inp["scores"], K, valid_len=valid_len)
        return i2, attend(inp["q"], inp["k"], inp["v"], i2, inp["sinks"], w.SCALE, c2)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        say(f"{'prefill' if shared else 'decode'} graph replay {r}")
        new = draw()
        for key, t in bufs.items():
            t.copy_(new[key])
        ref_idx, ref_out = eager(new)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"replay {r}: indices differ from eager"
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), f"replay {r}: outputs differ"


@pytest.mark.parametrize("entry", ["decode", "decode_noalloc"])
def test_captured_split_step_replays_equal_eager(entry):
    """Three sequences take the split path (score tiles through a workspace, then the values
    kernel). Captured with a workspace the caller allocated beforehand (sparse_attn_decode) or
    with the library's static scratch (sparse_attn_decode_noalloc, for callers that cannot
    allocate under capture); every replay must equal the eager result bit for bit."""
    import sparse_attention_attn_amd as sa
    from sparse_attention_attn_amd import _lib as L
    rows, H, N, K = 3, 64, 2048, 640
    assert sa.workspace_bytes(L.SA_OP_DECODE, rows, H, K, N) > 0, "not the split path"
    gen = torch.Generator(device=DEV)
    gen.manual_seed(19)

    def draw():
        return {
            "q": torch.randn((rows, H, 512), generator=gen, device=DEV).to(torch.bfloat16),
            "k": torch.randn((rows, N, 512), generator=gen, device=DEV).to(torch.bfloat16),
            "v": torch.randn((rows, N, 512), generator=gen, device=DEV).to(torch.bfloat16),
            "sinks": torch.randn((H,), generator=gen, device=DEV),
            "scores": torch.randn((rows, N), generator=gen, device=DEV),
        }

    bufs = draw()
    idx = torch.empty((rows, K), dtype=torch.int32, device=DEV)
    cnt = torch.empty((rows,), dtype=torch.int32, device=DEV)
    out = torch.empty((rows, H, 512), dtype=torch.float32, device=DEV)
    ws = torch.empty((sa.workspace_bytes(L.SA_OP_DECODE, rows, H, K, N),), dtype=torch.uint8, device=DEV)

    def step():
        sa.topk(bufs["scores"], K, idx_out=idx, count_out=cnt)
        if entry == "decode":
            sa.decode(bufs["q"], bufs["k"], bufs["v"], idx, bufs["sinks"], w.SCALE, cnt, out=out, ws=ws)
        else:
            sa.decode_noalloc(bufs["q"], bufs["k"], bufs["v"], idx, bufs["sinks"], w.SCALE, cnt, out=out)

    def eager(inp):
        i2, c2 = sa.topk(inp["scores"], K)
        return i2, sa.decode(inp["q"], inp["k"], inp["v"], i2, inp["sinks"], w.SCALE, c2)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        say(f"split-path {entry} graph replay {r}")
        new = draw()
        for key, t in bufs.items():
            t.copy_(new[key])
        ref_idx, ref_out = eager(new)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"replay {r}: indices differ from eager"
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), f"replay {r}: outputs differ"
