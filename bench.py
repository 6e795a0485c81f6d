"""Benchmark of the sparse-attention hot path on one MI355X.

One step = the whole hot path over one batch: exact indexer top-k (sparse_attn_topk)
over each row's scores, then gathered sparse attention with sinks
(sparse_attn_decode) over the selected cache rows. The default workload is the
decode shape (64 heads, head width 512, k = 640, 4,096 cached positions per
sequence) run over 1,024 independent sequences per step: a single row moves only
1.5 MB, less than one kernel launch's worth of time at HBM speed, so throughput
is measured on many rows at once. Inputs are synthetic (seeded, generated on the
device) and resident in HBM before timing starts; two input sets alternate so
that consecutive steps do not reuse cache contents (1.34 GB of distinct cache
rows are gathered per step, over five times the 256 MiB Infinity Cache).

Prints ONE JSON line: the metric (query-rows*heads per second for the whole
step), the step time, a roofline object for the dominant kernel (the attention
decode kernel: algorithmic bytes per launch over its HIP-event-timed average
duration, against 8 TB/s) and a cpu_baseline object (the float64 oracle timed
on this host's cores on a bounded sample of the same workload).

--workload selects other shapes of the same path (one JSON line each; the default
is the decode step above):
  decode-alias   the decode step with one latent tensor serving as K and V
                 (each selected row gathered once)
  prefill        2,048 query rows at positions 2,048..4,095 over one shared
                 4,096-position cache: causal top-640 (valid_len = pos + 1), then
                 prefill attention at 64 heads
  prefill-h16    the same with 16 real heads, launched as 16 (one 16-head block per
                 workgroup; its waves split the output columns four ways)
  prefill-pad16  the same 16 heads copied into a zero-padded 32-head buffer with
                 zero sinks, launched at 32 heads, real heads copied out
  decode-f32     float32 storage, the batched-decode shape (8 sequences x 32,768
                 positions, k = 640): top-k, then attention on the float32 matrix cores
  gather-ceiling the decode workload's K and V row gathers alone, no compute
                 (sparse_attn_gather_probe): the measured ceiling for this access
                 pattern, which the decode line also reports next to the HBM peak
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

EVENT_EVERY = 4  # timed steps per sampled attention launch (HIP events)
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(rows: int, heads: int, d: int, k: int, kv_tensors: int = 2) -> int:
    """Bytes the method itself moves per decode launch: bf16 q, the k gathered bf16 K and V
    rows (one gather when one tensor serves as both), the int32 index list and the fp32
    output of every row, plus the fp32 sinks."""
    per_row = 2 * heads * d + kv_tensors * 2 * d * k + 4 * k + 4 * heads * d
    return rows * per_row + 4 * heads


def algorithmic_flops(rows: int, heads: int, d: int, k: int) -> int:
    return rows * 4 * heads * d * k


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "attn_decode_b1024_h64_k640_hbm_traffic.md")
# The attention kernel's sources: the recorded counters apply while the sha256 of their code
# (kernel_code_sha256) is unchanged.
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_attention_attn_amd", "csrc", f) for f in ("sa_attn.hip", "sa_attn_common.h", "sa_device.h", "sa_internal.h")]


def kernel_code_sha256(files=None) -> str:
    """sha256 of the code of the given sources (KERNEL_SOURCES by default) in order, with
    comments, trailing blanks and blank lines removed: a change to a comment keeps the
    recorded counters, any change to the code does not."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        text = open(f).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update(("\n".join(lines) + "\n").encode())
    return h.hexdigest()


def measured_traffic(rows: int, heads: int, n_ctx: int, k: int):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary
    (copy-calibrated), or None when that summary was taken on another workload or on a kernel
    source that has changed since (its recorded sha256 no longer matches)."""
    if (rows, heads, n_ctx, k) != (1024, 64, 4096, 640) or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    for line in open(TRAFFIC_PROFILE):
        if ":" in line and not line.startswith(("|", " ", "#")):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_code_sha256") != kernel_code_sha256() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_baseline(inp, scores, out_gpu, idx_gpu, heads, k, budget_s: float, max_rows: int):
    """Time the float64 oracle (top-k then attention) on the host on a bounded sample of rows.

    The oracle's results for those rows are also compared with what the timed GPU
    launch produced for them (indices bit-exact; attention within the bf16 tolerance
    max |g - o| <= 2e-3 over finite elements, with equal nonfinite classes)."""
    import numpy as np

    import oracle
    import workloads as w
    threads = len(os.sched_getaffinity(0))
    lib = oracle.load()
    rows_done, t_total, max_err, ok = 0, 0.0, 0.0, True
    out_host = out_gpu.cpu().numpy()
    idx_host = idx_gpu.cpu().numpy()
    while rows_done < max_rows and t_total < budget_s:
        r = rows_done
        case = w.host_case_from_device(inp, r)
        s = scores[r:r + 1].cpu().numpy()
        t0 = time.perf_counter()
        idx, cnt = oracle.topk(s, k, lib=lib)
        case.idx, case.nsel = idx, cnt
        o = oracle.attention(case.dtype, case.q, case.k, case.v, case.idx, case.nsel, case.sinks, case.scale,
                             False, threads=threads, lib=lib)
        t_total += time.perf_counter() - t0
        g = out_host[r:r + 1].astype(np.float64)
        fin = np.isfinite(o)
        ok &= bool(np.array_equal(idx[0], idx_host[r]))
        ok &= bool(np.array_equal(np.isnan(g), np.isnan(o)) and np.array_equal(np.isinf(g), np.isinf(o)))
        err = np.abs(g[fin] - o[fin])
        ok &= bool(np.all(err <= 2e-3))
        max_err = max(max_err, float(err.max()) if err.size else 0.0)
        rows_done += 1
    value = rows_done * heads / t_total
    # The same oracle on one thread, over the first rows again (about 2 s of work).
    rows_1, t_1 = 0, 0.0
    while rows_1 < rows_done and t_1 < 2.0:
        case = w.host_case_from_device(inp, rows_1)
        s = scores[rows_1:rows_1 + 1].cpu().numpy()
        t0 = time.perf_counter()
        idx, cnt = oracle.topk(s, k, lib=lib)
        oracle.attention(case.dtype, case.q, case.k, case.v, idx, cnt, case.sinks, case.scale, False, threads=1,
                         lib=lib)
        t_1 += time.perf_counter() - t0
        rows_1 += 1
    base = {"value": value, "unit": "query-rows*heads/s", "cores": threads, "kind": "oracle",
            "sample": f"the first {rows_done} of the batch's {max_rows} rows (top-k over the row's scores, "
                      f"then {heads}-head attention), {t_total:.1f} s of float64 oracle work on "
                      f"{threads} OpenMP threads",
            "single_thread": {"value": rows_1 * heads / t_1, "cores": 1,
                              "sample": f"the first {rows_1} rows again, {t_1:.1f} s on one thread"}}
    parity = {"rows": rows_done, "indices_bit_exact_and_attention_within_tol": ok, "max_abs_err": max_err}
    return base, parity


def gather_ceiling(torch, sa, sets, rows: int, k: int, reps: int):
    """Time sparse_attn_gather_probe (the decode kernels' K and V gathers alone) over the given
    (inputs, idx) sets with HIP events on the current stream; returns the faster of 8 and 16 rows
    in flight per wave. Bytes per launch: the gathered bf16 K and V rows and the index list."""
    nbytes = rows * k * (2 * 2 * 512 + 4)
    best = None
    for rif in (8, 16):
        for i in range(10):
            inp, idx = sets[i % len(sets)]
            sa.gather_probe(inp["k"], inp["v"], idx, rif)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i in range(reps):
            inp, idx = sets[i % len(sets)]
            ev[i][0].record()
            sa.gather_probe(inp["k"], inp["v"], idx, rif)
            ev[i][1].record()
        torch.cuda.synchronize()
        ms = sum(a.elapsed_time(b) for a, b in ev) / reps
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["gbs"]:
            best = {"gbs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS, "rows_in_flight": rif, "kernel_ms": ms,
                    "bytes_per_launch": nbytes, "kernel": f"gather_probe_kernel<{rif}> (sparse_attn_gather_probe)"}
    return best


def copy_peak(torch, dev, mib: int = 1024, reps: int = 10):
    """A plain device-to-device copy of `mib` MiB (torch's copy kernel), timed with HIP events:
    bytes read plus bytes written per second, the streaming rate of this part as context for
    the gather ceiling."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"gbs": 2 * n / (ms * 1e-3) / 1e9, "bytes_moved_per_copy": 2 * n, "kernel_ms": ms}


def decode_kernel_label(torch, sa, dev, rows: int, heads: int, k: int, n_ctx: int, alias: bool) -> str:
    """Name of the kernel a bf16 decode launch of this shape runs, as the library's launch plan
    picks it (sa_attn.hip, plan_attn_bf16): the split path when the call needs a workspace, else
    the persistent kernel with 16 x HQ heads per workgroup and NS column slices."""
    if sa.workspace_bytes(0, rows, heads, k, n_ctx) > 0:
        return "attn_split_kernel (sparse_attn_decode, split path)"
    hq = 4 if heads > 32 else (2 if heads > 16 else 1)
    rows_hg = rows * -(-heads // (16 * hq))
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ns = 1
    while ns < 2 * hq and rows_hg * 2 * ns <= cus:
        ns *= 2
    if alias:
        return f"attn_bf16_alias_kernel<{hq},{ns}> (sparse_attn_decode, K = V)"
    return f"attn_bf16_kernel<{hq},{ns}> (sparse_attn_decode)"


def small_batch_latency(torch, sa, w, dev, n_ctx: int, k: int, heads: int, seed: int):
    """Attention call latency at 1 and 8 sequences (the split path): the median over 32 warm
    calls, each bracketed by HIP events on the launch stream with the device idle before it (a
    single warm call is how akol1/TensorFold pull request 4's PR body times attention), the
    median of 32 event pairs with nothing between them (the floor of that method), and the mean
    over 200 back-to-back calls between one pair of events."""
    res = {}
    for b in (1, 8):
        inp = w.device_decode_inputs(torch, dev, b, heads, n_ctx, k, seed=seed + b)
        out = torch.empty((b, heads, w.D), dtype=torch.float32, device=dev)
        need = sa.workspace_bytes(0, b, heads, k, n_ctx)
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)

        def call():
            sa.decode(inp["q"], inp["k"], inp["v"], inp["idx"], inp["sinks"], w.SCALE, out=out,
                      ws=ws if need else None)
        for _ in range(100):
            call()
        torch.cuda.synchronize()
        samples = []
        for _ in range(32):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            torch.cuda.synchronize()
            samples.append(e0.elapsed_time(e1) * 1e3)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(200):
            call()
        e1.record()
        torch.cuda.synchronize()
        back_to_back = e0.elapsed_time(e1) * 1e3 / 200
        samples.sort()
        floor = []
        for _ in range(32):
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            f0.record()
            f1.record()
            torch.cuda.synchronize()
            floor.append(f0.elapsed_time(f1) * 1e3)
        floor.sort()
        res[f"B{b}"] = {"call_us_median_of_32": (samples[15] + samples[16]) / 2,
                        "events_only_us_median_of_32": (floor[15] + floor[16]) / 2,
                        "call_us_back_to_back": back_to_back,
                        "path": "split" if need else "persistent"}
    return res


MFMA_F32_PEAK_TFLOPS = 157.3


def f32_kernel_label(rows, heads, k):
    """The float32 attention kernels of a decode launch, as the library picks them
    (f32_split_applies in csrc/sa_attn_f32_split.hip): the split path for fewer than 24
    (row, 64-head block) pairs and 129 <= k <= 1,024, else attn_f32_kernel. Both give the same bits."""
    n_hb = (heads + 63) // 64
    if 128 < k <= 1024 and rows * n_hb < 24:
        return "attn_f32_split_scores_kernel + attn_f32_split_values_kernel (sparse_attn_decode, SA_F32, split path)"
    return "attn_f32_kernel (sparse_attn_decode, SA_F32)"


def bench_decode_f32(args, torch, sa, w, dev) -> int:
    """Float32 decode step, batched-decode shape (8 sequences x 32,768 positions unless --batch /
    --n-ctx say otherwise): top-k over each row's scores, then float32 attention on the matrix
    cores. Roofline: float32 MFMA peak (the intensity, 32 FLOP/B at 64 heads, is above the float32
    ridge), with the HBM rate of the algorithmic bytes alongside."""
    B = args.batch if "--batch" in sys.argv else 8
    N = args.n_ctx if "--n-ctx" in sys.argv else 32768
    H, K, D = args.heads, args.k, w.D
    log(f"[bench] float32 decode: {B} sequences x {N} positions, {H} heads, k = {K}")
    sets = []
    for i in range(2):
        g = torch.Generator(device=dev)
        g.manual_seed(args.seed + 300 + i)
        st = {"q": torch.randn((B, H, D), generator=g, device=dev),
              "k": torch.randn((B, N, D), generator=g, device=dev),
              "v": torch.randn((B, N, D), generator=g, device=dev),
              "sinks": torch.randn((H,), generator=g, device=dev),
              "scores": torch.randn((B, N), generator=g, device=dev),
              "idx": torch.empty((B, K), dtype=torch.int32, device=dev),
              "cnt": torch.empty((B,), dtype=torch.int32, device=dev),
              "out": torch.empty((B, H, D), dtype=torch.float32, device=dev)}
        sets.append(st)
    torch.cuda.synchronize()

    # The split path's workspace (small batches), allocated once outside the timed steps.
    need = sa.workspace_bytes(0, B, H, K, N)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None

    def step(i, ev=None):
        st = sets[i % 2]
        sa.topk(st["scores"], K, idx_out=st["idx"], count_out=st["cnt"])
        if ev is not None:
            ev[0].record()
        sa.decode(st["q"], st["k"], st["v"], st["idx"], st["sinks"], w.SCALE, out=st["out"], ws=ws)
        if ev is not None:
            ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for i in range(0, args.steps, EVENT_EVERY)}
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events.get(i))
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    attn_ms = sum(a.elapsed_time(b) for a, b in events.values()) / len(events)
    flops = algorithmic_flops(B, H, D, K)
    nbytes = B * (4 * H * D + 2 * 4 * D * K + 4 * K + 4 * H * D) + 4 * H
    tflops = flops / (attn_ms * 1e-3) / 1e12
    gbs = nbytes / (attn_ms * 1e-3) / 1e9
    log(f"[bench] step {ms_per_step:.3f} ms, attention {attn_ms * 1e3:.1f} us: {tflops:.1f} TFLOP/s float32 "
        f"({tflops / MFMA_F32_PEAK_TFLOPS:.1%} of the float32 MFMA peak), {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of HBM)")
    result = {
        "metric": f"float32 decode query-rows*heads/s ({H} heads, d=512, k={K})",
        "value": B * H / (ms_per_step * 1e-3), "unit": "query-rows*heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded, generated on the device)",
        "config": {"workload": f"float32 decode: {B} sequences x {N} positions, indexer top-{K}, then attention "
                               f"with per-head sinks at {H} heads on the float32 matrix cores",
                   "batch_rows": B, "heads": H, "head_dim": D, "n_ctx": N, "k": K},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / MFMA_F32_PEAK_TFLOPS, "traffic": None,
                     "kernel": f32_kernel_label(B, H, K), "kernel_ms": attn_ms,
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": nbytes,
                     "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_gather_ceiling(args, torch, sa, w, dev) -> int:
    """The gather probe alone over the decode workload's inputs (one JSON line)."""
    B, H, N, K = args.batch, args.heads, args.n_ctx, args.k
    sets = [(w.device_decode_inputs(torch, dev, B, H, N, K, seed=args.seed + i), None) for i in range(2)]
    sets = [(inp, inp["idx"]) for inp, _ in sets]
    torch.cuda.synchronize()
    c = gather_ceiling(torch, sa, sets, B, K, reps=args.steps)
    print(json.dumps({"metric": "gathered K and V rows, GB/s (no compute)", "value": c["gbs"], "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "higher_is_better": True, "data": "synthetic",
                      "config": {"workload": f"gather probe: {B} sequences x {K} selected 1 KiB rows of K and of V "
                                             f"from {N}-position caches", "batch_rows": B, "n_ctx": N, "k": K},
                      "gather_ceiling": c}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # The part reaches its steady clocks only after tens of milliseconds of this load: with 5
    # warm-up steps the timed steps ran 5 % slower than after 200 (about 54 ms of work).
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--batch", type=int, default=1024, help="independent sequences per step")
    ap.add_argument("--heads", type=int, default=64)
    ap.add_argument("--n-ctx", type=int, default=4096)
    ap.add_argument("--k", type=int, default=640)
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attn-only", action="store_true", help="time only the attention kernel (profiling)")
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "decode-alias", "decode-f32", "prefill", "prefill-h16", "prefill-pad16",
                             "gather-ceiling"])
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, --steps times "
                         "(calibrates the HBM byte counters against a known size)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the path has no multi-GPU mode (rows and heads would "
              "shard without communication, one process per GPU); use --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import sparse_attention_attn_amd as sa
    import workloads as w

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / args.steps
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms": dt * 1e3,
                          "gbs_read_plus_write": 2 * n / dt / 1e9}), flush=True)
        return 0
    sa.load()
    if args.workload.startswith("prefill"):
        return bench_prefill(args, torch, sa, w, dev)
    if args.workload == "gather-ceiling":
        return bench_gather_ceiling(args, torch, sa, w, dev)
    if args.workload == "decode-f32":
        return bench_decode_f32(args, torch, sa, w, dev)
    B, H, N, K = args.batch, args.heads, args.n_ctx, args.k
    alias = args.workload == "decode-alias"

    log(f"[bench] generating 2 input sets: {B} sequences x {N} positions x {w.D} bf16 K and V each")
    sets = []
    for i in range(2):
        inp = w.device_decode_inputs(torch, dev, B, H, N, K, seed=args.seed + i)
        if alias:  # one latent tensor as K and V
            inp["v"] = inp["k"]
        g = torch.Generator(device=dev)
        g.manual_seed(args.seed + 100 + i)
        scores = torch.randn((B, N), generator=g, device=dev, dtype=torch.float32)
        idx = torch.empty((B, K), dtype=torch.int32, device=dev)
        cnt = torch.empty((B,), dtype=torch.int32, device=dev)
        out = torch.empty((B, H, w.D), dtype=torch.float32, device=dev)
        sets.append((inp, scores, idx, cnt, out))
    torch.cuda.synchronize()
    # The split path's workspace (small batches; none at 1,024 rows), allocated once outside the
    # timed steps.
    need = sa.workspace_bytes(0, B, H, K, N)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev) if need else None

    def step(i, ev=None):
        inp, scores, idx, cnt, out = sets[i % 2]
        if not args.attn_only:
            sa.topk(scores, K, idx_out=idx, count_out=cnt)
        else:
            idx = inp["idx"]
        if ev is not None:
            ev[0].record()
        sa.decode(inp["q"], inp["k"], inp["v"], idx, inp["sinks"], w.SCALE, out=out, ws=ws)
        if ev is not None:
            ev[1].record()

    # The gather ceiling: the same index-driven K and V row gathers with no compute
    # (sparse_attn_gather_probe), timed live over the same two input sets and their top-k index
    # lists, with 8 and 16 rows in flight per wave; the faster one is the ceiling the attention
    # kernel is compared with. It runs right before the warm-up steps with a fixed number of
    # launches (about 100 ms of gathers), after the plain copy measured as context: attention
    # launches that follow the gathers settle sooner than ones that follow the copy.
    ceiling = None
    if not alias:
        cpeak = copy_peak(torch, dev)
        for st in sets:
            if not args.attn_only:
                sa.topk(st[1], K, idx_out=st[2], count_out=st[3])
        ceiling = gather_ceiling(torch, sa, [(st[0], st[2] if not args.attn_only else st[0]["idx"]) for st in sets],
                                 B, K, reps=250)
        ceiling["copy_peak"] = cpeak

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # HIP events bracket the attention launch of every EVENT_EVERY-th timed step: each pair
    # of timing events costs about 4 us of the step, so sampling keeps the step close to what
    # it is without them, and the kernel's duration is still measured live in this region.
    events = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for i in range(0, args.steps, EVENT_EVERY)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = sum(a.elapsed_time(b) for a, b in events.values()) / len(events)
    ms_per_step = wall * 1e3 / args.steps

    nbytes = algorithmic_bytes(B, H, w.D, K, kv_tensors=1 if alias else 2)
    flops = algorithmic_flops(B, H, w.D, K)
    achieved_gbs = nbytes / (attn_ms * 1e-3) / 1e9
    log(f"[bench] step {ms_per_step:.3f} ms, attention kernel {attn_ms:.3f} ms: {achieved_gbs:.0f} GB/s "
        f"algorithmic ({achieved_gbs / HBM_PEAK_GBS:.1%} of 8 TB/s), "
        f"{flops / (attn_ms * 1e-3) / 1e12:.0f} TFLOP/s bf16 ({flops / (attn_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS:.1%} of MFMA peak)")

    if ceiling is not None:
        log(f"[bench] gather ceiling {ceiling['gbs']:.0f} GB/s ({ceiling['rows_in_flight']} rows in flight per wave, "
            f"{ceiling['kernel_ms'] * 1e3:.1f} us per launch): attention at {achieved_gbs / ceiling['gbs']:.1%} of it; "
            f"a 1 GiB device copy moves {ceiling['copy_peak']['gbs']:.0f} GB/s")

    small = None
    if not alias and not args.attn_only and (B, H, N, K) == (1024, 64, 4096, 640):
        small = small_batch_latency(torch, sa, w, dev, N, K, H, args.seed + 200)
        log("[bench] attention call latency: " + ", ".join(
            f"{b} {v['call_us_median_of_32']:.1f} us (median of 32 warm calls), {v['call_us_back_to_back']:.1f} us "
            f"back to back" for b, v in small.items()))

    inp, scores, idx, cnt, out = sets[(args.steps - 1) % 2]  # the last timed step's set
    result = {
        "metric": f"decode query-rows*heads/s ({H} heads, d=512, k={K})",
        "value": B * H / (ms_per_step * 1e-3),
        "unit": "query-rows*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, generated on the device)",
        "config": {
            "workload": f"decode: {B} independent sequences per step, {H} heads, head width {w.D}, "
                        f"{N} cached positions per sequence, indexer top-{K} over {N} fp32 scores per row, "
                        f"then sparse attention with per-head sinks over the {K} selected rows"
                        + (" of one latent tensor serving as K and V" if alias else "")
                        + (" (attention only)" if args.attn_only else ""),
            "batch_rows": B, "heads": H, "head_dim": w.D, "n_ctx": N, "k": K,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": None if alias else measured_traffic(B, H, N, K),
            "kernel": decode_kernel_label(torch, sa, dev, B, H, K, N, alias),
            "kernel_ms": attn_ms,
            "algorithmic_bytes_per_launch": nbytes,
            "mfma_tflops": flops / (attn_ms * 1e-3) / 1e12,
            "gather_ceiling": ceiling,
            "frac_of_gather_ceiling": None if ceiling is None else achieved_gbs / ceiling["gbs"],
        },
        "cpu_baseline": None,
    }
    if small is not None:
        result["small_batch"] = small
    if not args.no_cpu_baseline and not args.attn_only:
        log("[bench] timing the float64 oracle on the host")
        result["cpu_baseline"], result["parity_sampled"] = cpu_baseline(
            inp, scores, out, inp["idx"] if args.attn_only else idx, H, K, args.cpu_budget, max_rows=B)
    print(json.dumps(result), flush=True)
    return 0


def prefill_cpu_baseline(q, kc, vc, sinks, scores, valid_len, out_gpu, idx_gpu, k, budget_s: float, max_rows: int):
    """The float64 oracle (causal top-k over the row's scores, then attention over the
    shared cache) on the host on a bounded sample of prefill rows, compared with the GPU."""
    import numpy as np

    import torch

    import oracle
    import workloads as w
    threads = len(os.sched_getaffinity(0))
    lib = oracle.load()

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    kh, vh = bits(kc)[None], bits(vc)[None]
    s_h = sinks.cpu().numpy().astype(np.float32)
    out_host = out_gpu.cpu().numpy()
    idx_host = idx_gpu.cpu().numpy()
    vl_host = valid_len.cpu().numpy()
    rows_done, t_total, max_err, ok = 0, 0.0, 0.0, True
    while rows_done < max_rows and t_total < budget_s:
        r = rows_done
        qh = bits(q[r:r + 1])
        sr = scores[r:r + 1].cpu().numpy()
        t0 = time.perf_counter()
        idx, cnt = oracle.topk(sr, k, vl_host[r:r + 1], lib=lib)
        o = oracle.attention("bf16", qh, kh, vh, idx, cnt, s_h, w.SCALE, True, threads=threads, lib=lib)
        t_total += time.perf_counter() - t0
        g = out_host[r:r + 1].astype(np.float64)
        fin = np.isfinite(o)
        ok &= bool(np.array_equal(idx[0], idx_host[r]))
        ok &= bool(np.array_equal(np.isnan(g), np.isnan(o)) and np.array_equal(np.isinf(g), np.isinf(o)))
        err = np.abs(g[fin] - o[fin])
        ok &= bool(np.all(err <= 2e-3))
        max_err = max(max_err, float(err.max()) if err.size else 0.0)
        rows_done += 1
    heads = q.shape[1]
    base = {"value": rows_done * heads / t_total, "unit": "query-rows*heads/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the first {rows_done} of the segment's {q.shape[0]} rows (causal top-k over the row's "
                      f"scores, then {heads}-head attention over the shared cache), {t_total:.1f} s of float64 "
                      f"oracle work on {threads} OpenMP threads"}
    parity = {"rows": rows_done, "indices_bit_exact_and_attention_within_tol": ok, "max_abs_err": max_err}
    return base, parity


def bench_prefill(args, torch, sa, w, dev) -> int:
    """Prefill segment: T rows at positions first..first+T-1 over one shared cache; a step is
    the causal top-k (valid_len = pos + 1) then prefill attention (with explicit 16 -> 32
    head padding and copy-out for prefill-pad16)."""
    T, N, K, first = 2048, 4096, 640, 2048
    h_real = 16 if args.workload in ("prefill-h16", "prefill-pad16") else args.heads
    pad = args.workload == "prefill-pad16"
    h_launch = 32 if pad else h_real
    D = w.D
    log(f"[bench] prefill: {T} rows, {h_real} real heads (launch {h_launch}), shared cache of {N} positions")
    sets = []
    for i in range(2):
        g = torch.Generator(device=dev)
        g.manual_seed(args.seed + 200 + i)
        st = {
            "q": torch.randn((T, h_real, D), generator=g, device=dev).to(torch.bfloat16),
            "k": torch.randn((N, D), generator=g, device=dev).to(torch.bfloat16),
            "v": torch.randn((N, D), generator=g, device=dev).to(torch.bfloat16),
            "sinks": torch.randn((h_real,), generator=g, device=dev),
            "scores": torch.randn((T, N), generator=g, device=dev),
            "valid_len": torch.arange(first + 1, first + T + 1, dtype=torch.int32, device=dev),
            "idx": torch.empty((T, K), dtype=torch.int32, device=dev),
            "cnt": torch.empty((T,), dtype=torch.int32, device=dev),
            "out": torch.empty((T, h_real, D), dtype=torch.float32, device=dev),
        }
        if pad:
            st["q_pad"] = torch.empty((T, h_launch, D), dtype=torch.bfloat16, device=dev)
            st["s_pad"] = torch.empty((h_launch,), dtype=torch.float32, device=dev)
            st["out_pad"] = torch.empty((T, h_launch, D), dtype=torch.float32, device=dev)
        sets.append(st)
    torch.cuda.synchronize()

    def step(i, ev=None):
        st = sets[i % 2]
        sa.topk(st["scores"], K, valid_len=st["valid_len"], idx_out=st["idx"], count_out=st["cnt"])
        if pad:
            sa.pad_heads(st["q"], st["sinks"], h_launch, q_pad=st["q_pad"], s_pad=st["s_pad"])
            q, sinks, out = st["q_pad"], st["s_pad"], st["out_pad"]
        else:
            q, sinks, out = st["q"], st["sinks"], st["out"]
        if ev is not None:
            ev[0].record()
        sa.prefill(q, st["k"], st["v"], st["idx"], sinks, w.SCALE, st["cnt"], out=out)
        if ev is not None:
            ev[1].record()
        if pad:
            sa.unpad_heads(st["out_pad"], h_real, out=st["out"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for i in range(0, args.steps, EVENT_EVERY)}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_ms = sum(a.elapsed_time(b) for a, b in events.values()) / len(events)
    ms_per_step = wall * 1e3 / args.steps
    flops = T * 4 * h_real * D * K                 # useful work: the real heads
    gathered = T * 2 * 2 * D * K                   # K and V rows staged from L2/MALL into LDS
    unique = T * (2 * h_launch * D + 4 * K + 4 * h_launch * D) + 2 * 2 * N * D + 4 * h_launch
    tflops = flops / (attn_ms * 1e-3) / 1e12
    log(f"[bench] step {ms_per_step:.3f} ms, prefill kernel {attn_ms:.3f} ms: {tflops:.0f} TFLOP/s of real-head "
        f"bf16 work ({tflops / MFMA_BF16_PEAK_TFLOPS:.1%} of MFMA peak), gathered {gathered / (attn_ms * 1e-3) / 1e9:.0f} GB/s")
    st = sets[(args.steps - 1) % 2]
    result = {
        "metric": f"prefill query-rows*heads/s ({h_real} heads, d=512, k=640)",
        "value": T * h_real / (ms_per_step * 1e-3),
        "unit": "query-rows*heads/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded, generated on the device)",
        "config": {
            "workload": f"prefill: {T} query rows at positions {first}..{first + T - 1} over one shared "
                        f"{N}-position cache, causal indexer top-{K} (valid_len = pos + 1), then sparse "
                        f"attention with per-head sinks at {h_real} real heads"
                        + (" padded to 32 with zero sinks and copied out" if pad else
                           (" (launched as 16: one 16-head block per workgroup)" if h_real == 16 else "")),
            "rows": T, "heads": h_real, "launch_heads": h_launch, "head_dim": D, "n_ctx": N, "k": K,
        },
        "roofline": {
            "bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
            "kernel": f"attn_bf16_kernel<{4 if h_launch > 32 else (2 if h_launch > 16 else 1)},1> (sparse_attn_prefill)",
            "kernel_ms": attn_ms, "algorithmic_flops_per_launch": flops,
            "gathered_bytes_per_launch": gathered, "gathered_gbs": gathered / (attn_ms * 1e-3) / 1e9,
            "unique_hbm_bytes_per_launch": unique,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the float64 oracle on the host")
        result["cpu_baseline"], result["parity_sampled"] = prefill_cpu_baseline(
            st["q"], st["k"], st["v"], st["sinks"], st["scores"], st["valid_len"], st["out"], st["idx"], K,
            args.cpu_budget, max_rows=T)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
