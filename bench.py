"""Benchmark of libfa's attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload (the headline configuration): B=4, H=16, N=4096, d=128, bf16
inputs/outputs with fp32 softmax and accumulation, Q/K/V iid N(0,1) from a
fixed seed, scale = 1/sqrt(d). One step is one non-causal forward followed by
one causal forward on the same resident inputs, so a step covers every stage
of the path including the causal tile skip.

FLOPs follow the pages' convention, 4*B*H*N^2*d per forward, halved for
causal. ``value`` is the step's FLOPs over the step's wall time (HIP events
around the K timed steps). Per-kernel durations come from HIP events recorded
around every launch on the launch stream; the roofline entry uses the
non-causal kernel's average duration.

After the timed region (never inside it) the default run also samples board power and clock
with amd-smi while the step loops, times a plain hipBLASLt bf16 GEMM on random operands as
context for the roofline, and times the fp64 oracle on the host (cpu_baseline).

Other modes (used to collect counters; each runs a few launches only):
    --profile-kernels   a few launches of each kernel of --profile-set (d128: the
                        headline, the default; d64; long: the long-context causal
                        configuration with and without q x 4; small: the two
                        smallest configurations), nothing else
    --profile-timed     the same workloads after a warmup (for kernel traces)
    --copy-calibration  a plain device-to-device copy of a known size
    --profile-decode    the split-key decode path (one query x 16384 keys, B=1 H=32)
    --profile-masked    the padding and sliding-window workloads of the sweep
    --profile-variants  head dims 96 and 32 and fp32 inputs at the headline shape
    --profile-bwd       backward calls at the headline shape (both causal flags)
    --sweep             medians of 50 for every configuration of the workload
                        list, with each configuration's own peak memory and
                        the fp64 oracle's rate on a row sample of it (one
                        extra JSON object); the masked rows count exactly the
                        visible (query, key) pairs (fa_plan_masked)
"""

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 FLOP/clk/CU x 2.4 GHz, dense (no sparsity)
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "tiled_attention_forward_fwd_amd", "csrc", f)
                  for f in ("fa_fwd_kernel.h", "fa_fwd_kernel.hip", "fa_device.h", "fa_tiles.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fa_fwd_bf16_d128_N4096.txt")

HEADLINE = dict(B=4, H=16, N=4096, d=128, dtype="bf16", seed=7)


def kernel_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the non-causal headline kernel, from the
    committed rocprofv3 counter summary, if it was taken on this kernel source."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m_hash = re.search(r"^kernel_source_sha256_16:\s*(\w+)", text, re.M)
    m_bytes = re.search(r"^hbm_bytes_per_launch_noncausal:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def make_inputs(cfg, device):
    from fa_inputs import make_qkv
    q, k, v = make_qkv(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["dtype"], cfg["seed"],
                       q_scale=cfg.get("q_scale", 1.0))
    return q, k, v, q.to(device), k.to(device), v.to(device)


def timed_launches(fn, n, stream):
    """Run fn n times, each bracketed by HIP events on `stream`; returns ms list."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def warm(fn, min_calls, min_seconds):
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or time.perf_counter() - t0 < min_seconds:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def power_and_clock(step, seconds=2.0):
    """Socket power (W) and mean graphics clock (MHz) read once with amd-smi
    while `step` runs back to back; outside the timed region. None if amd-smi
    is unavailable. Under sustained attention load the MI355X runs at its
    board power limit, and the clock it holds sets the MFMA rate reached."""
    import subprocess
    import threading
    import torch
    result = {}

    def sample():
        time.sleep(seconds / 2)
        try:
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"],
                               capture_output=True, text=True, timeout=30)
            j = json.loads(r.stdout)
            g = j["gpu_data"][0] if isinstance(j, dict) else j[0]
            clks = [c["clk"]["value"] for name, c in g["clock"].items()
                    if name.startswith("gfx_") and isinstance(c, dict)
                    and isinstance(c.get("clk"), dict) and isinstance(c["clk"].get("value"), (int, float))]
            result["socket_power_w"] = g["power"]["socket_power"]["value"]
            result["gfx_clock_mhz"] = round(sum(clks) / len(clks)) if clks else None
        except Exception as e:  # telemetry is context only
            result["error"] = str(e)[:200]

    th = threading.Thread(target=sample)
    t0 = time.perf_counter()
    th.start()
    while th.is_alive() or time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    th.join()
    return result if "socket_power_w" in result else None


def time_backward(cfg, reps=10):
    """fa.bwd (its three kernels) back to back between HIP events on one configuration,
    non-causal and causal, with TFLOP/s in the FlashAttention-2 convention (2.5x the forward's
    4*B*H*N*N*d, halved for causal; d is the tensors' head dim)."""
    import torch
    import tiled_attention_forward_fwd_amd as fa
    dev = torch.device("cuda:0")
    _, _, _, qd, kd, vd = make_inputs(cfg, dev)
    from fa_inputs import make_qkv
    dout = make_qkv(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["dtype"], cfg["seed"] + 100)[0].to(dev)
    res = {}
    for causal in (False, True):
        o, lse = fa.fwd(qd, kd, vd, causal=causal)
        f = lambda: fa.bwd(qd, kd, vd, o, lse, dout, causal=causal)  # noqa: E731
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        flops = 2.5 * 4.0 * cfg["B"] * cfg["H"] * cfg["N"] ** 2 * cfg["d"] * (0.5 if causal else 1.0)
        res["causal" if causal else "noncausal"] = {
            "ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
            "frac_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    return res


def backward_leg(reps=10):
    """The backward pass after the timed region: the headline shape, and the same shape at head
    dim 96 (the d = 128 tiles computing 96 dims; FLOPs counted at d = 96)."""
    res = time_backward(HEADLINE, reps)
    res["what"] = ("fa.bwd (delta, dK/dV, dQ kernels) at B=4 H=16 N=4096 d=128 bf16, FLOPs = 2.5x "
                   "the forward's; the kernels execute 1.4x that (S and dP are recomputed for dQ)")
    res["d96"] = time_backward(dict(HEADLINE, d=96), reps)
    return res


def gemm_ceiling(seconds=1.0):
    """Context for the roofline: TFLOP/s of a plain 8192^3 bf16 GEMM (hipBLASLt through
    torch.matmul) on seeded N(0,1) operands, run back to back after the timed region. The
    dense peak assumes 2.4 GHz; under sustained random-operand MFMA load the board power limit
    holds the clock lower, and this measures what a vendor GEMM reaches under the same limit."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(11)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
    ts = timed_launches(lambda: torch.matmul(a, b, out=c), 20, torch.cuda.current_stream())
    med = statistics.median(ts)
    return {"value": 2.0 * n ** 3 / (med * 1e-3) / 1e12, "unit": "TFLOP/s",
            "what": "bf16 8192x8192x8192 GEMM, torch.matmul (hipBLASLt), N(0,1) operands, median of 20"}


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_rate(cfg, q, k, v, causal, flop_budget=4.0e10):
    """The fp64 oracle on a row sample of one sweep configuration: every
    stride-th query row (all heads), the stride chosen so that the sample
    holds about `flop_budget` visited-key FLOPs. Returns the rate over the
    sample's exact visited-key FLOPs and what the sample was."""
    import oracle
    import tiled_attention_forward_fwd_amd as fa
    B, H, Nk, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    Nq = q.shape[2]
    wl, wr, kls = cfg.get("wl", -1), cfg.get("wr", -1), cfg.get("key_lens")

    def keys_seen(i, kl):
        hi = min(i + 1, Nk) if causal else (min(i + wr + 1, Nk) if wr >= 0 else Nk)
        hi = min(hi, kl)
        lo = max(0, i - wl) if wl >= 0 else 0
        return max(0, hi - lo)

    lens = kls if kls is not None else [Nk] * B
    total = 4.0 * H * d * sum(keys_seen(i, kl) for kl in lens for i in range(Nq))
    stride = max(1, int(-(-total // flop_budget)))
    rows = list(range(0, Nq, stride))
    flops = 4.0 * H * d * sum(keys_seen(i, kl) for kl in lens for i in rows)
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.attention_fwd(q, k, v, causal, fa.default_scale(d), rows=rows, nthreads=threads,
                         window_left=wl, window_right=wr, key_lens=kls)
    dt = time.perf_counter() - t0
    return {"gflops": flops / dt / 1e9, "seconds": dt, "threads": threads,
            "sample": ("all query rows" if stride == 1 else f"every {stride}th query row")
                      + f" ({len(rows)} of {Nq}, all heads), {flops / 1e9:.2f} G visited-key FLOPs"}


def cpu_baseline(cfg, q, k, v, stride):
    """The fp64 oracle on a bounded row sample of the workload (host cores)."""
    import oracle
    import tiled_attention_forward_fwd_amd as fa
    N = cfg["N"]
    rows = list(range(0, N, stride))
    scale = fa.default_scale(cfg["d"])
    threads = oracle.default_threads()
    flops = 0.0
    t0 = time.perf_counter()
    for causal in (False, True):
        oracle.attention_fwd(q, k, v, causal, scale, rows=rows, nthreads=threads)
        keys = sum((r + 1) if causal else N for r in rows)
        flops += 4.0 * cfg["B"] * cfg["H"] * keys * cfg["d"]
    dt = time.perf_counter() - t0
    # the same convention as the GPU: the causal pass counts half of the full rows' keys
    conv = 4.0 * cfg["B"] * cfg["H"] * len(rows) * N * cfg["d"] * 1.5
    return {"value": conv / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": (f"B={cfg['B']} H={cfg['H']} N={N} d={cfg['d']} {cfg['dtype']}: "
                       + ("all query rows" if stride == 1 else f"every {stride}th query row")
                       + f" ({len(rows)} rows per head, all heads), one "
                       f"non-causal and one causal pass, fp64 two-pass; {dt:.1f} s wall; FLOPs "
                       f"counted like the GPU step (causal = half the rows' full key count); "
                       f"exact visited-key FLOPs {flops / 1e9:.1f} G"),
            "seconds": dt}


def headline(args):
    import torch
    import tiled_attention_forward_fwd_amd as fa
    cfg = HEADLINE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, qd, kd, vd = make_inputs(cfg, dev)
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)
    plan_nc = fa.fa_plan(B, H, N, d, 0, fa.FA_DTYPE_BF16)
    plan_c = fa.fa_plan(B, H, N, d, 1, fa.FA_DTYPE_BF16)

    def nc():
        fa.fwd(qd, kd, vd, causal=False, out=o, lse=lse)

    def c():
        fa.fwd(qd, kd, vd, causal=True, out=o, lse=lse)

    def step():
        nc()
        c()

    # warmup: W steps plus at least one second of back-to-back launches
    warm(step, args.warmup, 1.0)
    torch.cuda.reset_peak_memory_stats(dev)

    ev_nc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    ev_c = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        ev_nc[i][0].record(stream)
        nc()
        ev_nc[i][1].record(stream)
        ev_c[i][0].record(stream)
        c()
        ev_c[i][1].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    t_nc = [a.elapsed_time(b) for a, b in ev_nc]
    t_c = [a.elapsed_time(b) for a, b in ev_c]
    peak_mem = torch.cuda.max_memory_allocated(dev)

    flops_step = plan_nc["algo_flops"] + plan_c["algo_flops"]
    ms_step = total_ms / args.steps
    value = flops_step / (ms_step * 1e-3) / 1e12

    def kstats(ts, plan):
        avg, med = sum(ts) / len(ts), statistics.median(ts)
        return {"avg_ms": avg, "median_ms": med, "min_ms": min(ts), "max_ms": max(ts),
                "tflops_median": plan["algo_flops"] / (med * 1e-3) / 1e12,
                "frac_peak_median": plan["algo_flops"] / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "mfma_flops_executed": plan["mfma_flops"], "algo_flops": plan["algo_flops"],
                "workgroups": plan["workgroups"]}

    k_nc, k_c = kstats(t_nc, plan_nc), kstats(t_c, plan_c)
    achieved = plan_nc["algo_flops"] / (k_nc["avg_ms"] * 1e-3) / 1e12
    traffic = measured_traffic()
    out = {
        "metric": "attention fwd TFLOP/s at N=4096 bf16 (causal/non-causal); % of MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) Q/K/V, rounded to bf16)",
        "config": {"workload": "attention forward B=4 H=16 N=4096 d=128 bf16, one non-causal + "
                               "one causal pass per step",
                   "B": B, "H": H, "N": N, "d": d, "scale": fa.default_scale(d),
                   "parallelism": "single GPU"},
        "frac_peak": value / PEAK_BF16_TFLOPS,
        "kernels": {"noncausal": k_nc, "causal": k_c},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic, "kernel": "non-causal d=128 bf16",
                     "algorithmic_flops_per_launch": plan_nc["algo_flops"],
                     "algorithmic_bytes_per_launch": plan_nc["algo_bytes"],
                     "hbm_gbs_compulsory": plan_nc["algo_bytes"] / (k_nc["avg_ms"] * 1e-3) / 1e9},
        "peak_mem_bytes": peak_mem,
        "telemetry_during_step_loop": power_and_clock(step) if args.telemetry else None,
        "wall_s_timed": wall,
        "kernel_source_sha256_16": kernel_hash(),
        "device": torch.cuda.get_device_name(dev),
    }
    return out, (q, k, v)


def c_call(fa, qd, kd, vd, out, lse, causal, splits, ws, ws_bytes, kl_ptr, wl, wr, code, stream):
    """One forward call bound straight to its C entry point (pointers, sizes and stream fixed
    beforehand), so that timing it measures the launch and the kernels rather than the Python
    binding's argument checks: the call fa.fwd would make for the same arguments."""
    lib = fa.load_library()
    B, H, Nq, d = qd.shape
    Nk = kd.shape[2]
    scale = fa.default_scale(d)
    p = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), lse.data_ptr())
    masked = kl_ptr is not None or wl != -1 or wr != -1
    if qd.dtype.itemsize == 4:
        f, a = lib.fa_fwd_f32, p + (B, H, Nq, Nk, d, int(causal), scale, ws, ws_bytes, stream)
    elif masked and splits == 1:
        f, a = lib.fa_fwd_masked, p + (B, H, Nq, Nk, d, int(causal), wl, wr, kl_ptr, scale, code, stream)
    elif masked:
        f, a = lib.fa_fwd_split_masked, p + (B, H, Nq, Nk, d, int(causal), wl, wr, kl_ptr, scale, code, splits,
                                             ws, ws_bytes, stream)
    elif splits == 1:
        f, a = lib.fa_fwd_qk, p + (B, H, Nq, Nk, d, int(causal), scale, code, stream)
    else:
        f, a = lib.fa_fwd_split_qk, p + (B, H, Nq, Nk, d, int(causal), scale, code, splits, ws, ws_bytes, stream)
    rc = f(*a)
    if rc != fa.FA_OK:
        raise RuntimeError(f"forward call failed: {fa.fa_status_string(rc)}")
    return lambda: f(*a)


def back_to_back(fn, n, stream):
    """Mean ms per call of n calls enqueued back to back between two HIP events on `stream`."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / n


def sweep(args):
    """Medians of 50 (after a separate warmup) for each configuration, with peak memory and
    the fp64 oracle's rate on the host for the same configuration. Calls go straight to the C
    entry points (c_call); median_ms brackets each call with its own events (the launch
    latency included), b2b_ms is the mean of 50 calls enqueued back to back.

    peak_mem_bytes is the peak device allocation during the configuration's timed calls
    (statistics reset after its warmup) minus what was allocated before its inputs were
    created, i.e. its own inputs, outputs and workspace."""
    import torch
    import tiled_attention_forward_fwd_amd as fa
    dev = torch.device("cuda:0")
    rows = []
    configs = [
        dict(B=1, H=1, N=128, d=64, dtype="fp16", seed=1, flags=(0, 1)),
        dict(B=2, H=4, N=1000, d=64, dtype="bf16", seed=2, flags=(0, 1)),
        dict(B=2, H=4, N=1000, d=64, dtype="fp16", seed=2, flags=(0, 1)),
        dict(B=4, H=16, N=512, d=64, dtype="fp16", seed=3, flags=(0, 1)),
        dict(B=4, H=16, N=2048, d=64, dtype="fp16", seed=4, flags=(0, 1)),
        dict(B=4, H=16, N=8192, d=64, dtype="fp16", seed=5, flags=(0, 1)),
        dict(B=4, H=16, N=4096, d=64, dtype="bf16", seed=6, flags=(0, 1)),
        dict(B=4, H=16, N=4096, d=128, dtype="bf16", seed=7, flags=(0, 1)),
        dict(B=1, H=32, N=16384, d=128, dtype="bf16", seed=8, flags=(1,)),
        dict(B=1, H=32, N=16384, d=128, dtype="bf16", seed=9, q_scale=4.0, flags=(1,)),
        # fewer queries than keys: KV-cache decode (split-key path) and a long-key prefill
        dict(B=1, H=32, Nq=1, N=16384, d=128, dtype="bf16", seed=10, flags=(0,)),
        dict(B=4, H=32, Nq=1, N=16384, d=128, dtype="bf16", seed=11, flags=(0,)),
        dict(B=1, H=32, Nq=4096, N=16384, d=128, dtype="bf16", seed=12, flags=(1,)),
        # head dims other than 64 and 128 (run by the d = 128 / d = 64 kernels, padded)
        dict(B=4, H=16, N=4096, d=96, dtype="bf16", seed=17, flags=(0, 1)),
        dict(B=4, H=16, N=4096, d=32, dtype="fp16", seed=18, flags=(0, 1)),
        # fp32 inputs and outputs (split-bf16 products; FLOPs counted as for any dtype)
        dict(B=4, H=16, N=4096, d=128, dtype="fp32", seed=19, flags=(0, 1)),
        dict(B=4, H=16, N=4096, d=64, dtype="fp32", seed=20, flags=(0, 1)),
    ] + MASKED_WORKLOADS
    for cfg in configs:
        torch.cuda.synchronize()
        base_mem = torch.cuda.memory_allocated(dev)  # what earlier configurations still hold
        qh, kh, vh, qd, kd, vd = make_inputs(cfg, dev)
        B, H, Nk, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
        Nq = cfg.get("Nq", Nk)
        qd = qd[:, :, :Nq].contiguous()
        qh = qh[:, :, :Nq].contiguous()
        code = fa.FA_DTYPE_BF16 if cfg["dtype"] == "bf16" else fa.FA_DTYPE_F16
        wl, wr, kls = cfg.get("wl", -1), cfg.get("wr", -1), cfg.get("key_lens")
        masked = wl != -1 or wr != -1 or kls is not None
        kl_dev = None if kls is None else torch.tensor(kls, dtype=torch.int32, device=dev)
        for causal in cfg["flags"]:
            splits = 1 if cfg["dtype"] == "fp32" else fa.fa_split_count(B, H, Nq, Nk, d, causal)
            out = torch.empty_like(qd)
            lse = torch.empty((B, H, Nq), device=dev, dtype=torch.float32)
            ws_bytes = (fa.fa_f32_workspace_bytes(B, H, Nk, d) if cfg["dtype"] == "fp32" else
                        fa.fa_split_workspace_bytes(B, H, Nq, d, splits) if splits > 1 else 0)
            ws = torch.empty(max(ws_bytes, 16) // 4, device=dev, dtype=torch.float32) if ws_bytes else None
            stream = torch.cuda.current_stream(dev)
            fn = c_call(fa, qd, kd, vd, out, lse, causal, splits, None if ws is None else ws.data_ptr(),
                        ws_bytes, None if kl_dev is None else kl_dev.data_ptr(), wl, wr, code, stream.cuda_stream)
            warm(fn, 20, 0.5)
            torch.cuda.reset_peak_memory_stats(dev)
            ts = timed_launches(fn, 50, stream)
            b2b = back_to_back(fn, 50, stream)
            if masked:
                plan = fa.fa_plan_masked(B, H, Nq, Nk, d, causal, wl, wr, kls, code)
            else:
                plan = fa.fa_plan_qk(B, H, Nq, Nk, d, causal, code)
            peak = torch.cuda.max_memory_allocated(dev) - base_mem
            med = statistics.median(ts)
            cpu = oracle_rate(cfg, qh, kh, vh, bool(causal)) if args.sweep_oracle else None
            rows.append({"B": B, "H": H, "Nq": Nq, "N": Nk, "d": d,
                         "dtype": cfg["dtype"], "q_scale": cfg.get("q_scale", 1.0),
                         **({"window_left": wl, "window_right": wr, "key_lens": kls} if masked else {}),
                         "causal": bool(causal), "splits": splits,
                         "launch": ("split" if splits > 1 else
                                    "key-split" if (plan["block_m"], plan["block_n"]) == (32, 32) else "direct"),
                         "workgroups": plan["workgroups"], "median_ms": med,
                         "min_ms": min(ts), "max_ms": max(ts), "b2b_ms": b2b,
                         "tflops": plan["algo_flops"] / (med * 1e-3) / 1e12,
                         "frac_peak": plan["algo_flops"] / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "hbm_gbs_compulsory": plan["algo_bytes"] / (med * 1e-3) / 1e9,
                         "frac_hbm": plan["algo_bytes"] / (med * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "peak_mem_bytes": peak,
                         "cpu_oracle": cpu,
                         "gpu_over_oracle": (None if cpu is None else
                                             plan["algo_flops"] / (med * 1e-3) / (cpu["gflops"] * 1e9))})
            print(json.dumps({"sweep_row": rows[-1]}), flush=True)
        del qd, kd, vd, out, lse, ws, fn
        torch.cuda.empty_cache()
    return rows


# Padding and sliding-window workloads (sweep rows and --profile-masked):
# a padded batch at the headline shape, the headline problem through the
# masked kernel with a window that hides nothing (the cost of the masked
# launch itself), a 4096-key sliding window over a 16384-token causal
# sequence, the same at d = 64, and decode over four caches of different
# lengths (split-key path).
MASKED_WORKLOADS = [
    dict(B=4, H=16, N=4096, d=128, dtype="bf16", seed=13, key_lens=[4096, 3072, 2048, 1024], flags=(0, 1)),
    dict(B=4, H=16, N=4096, d=128, dtype="bf16", seed=7, wl=4096, flags=(0, 1)),
    dict(B=1, H=32, N=16384, d=128, dtype="bf16", seed=14, wl=4095, flags=(1,)),
    dict(B=4, H=16, N=8192, d=64, dtype="fp16", seed=15, wl=1023, flags=(1,)),
    dict(B=4, H=32, Nq=1, N=16384, d=128, dtype="bf16", seed=16, key_lens=[16384, 12000, 8000, 4000],
         flags=(0,)),
]


# Head dims other than 64 / 128 and fp32 inputs (--profile-variants).
VARIANT_WORKLOADS = [
    dict(B=4, H=16, N=4096, d=96, dtype="bf16", seed=17, flags=(0, 1)),
    dict(B=4, H=16, N=4096, d=32, dtype="fp16", seed=18, flags=(0, 1)),
    dict(B=4, H=16, N=4096, d=128, dtype="fp32", seed=19, flags=(0, 1)),
]


def profile_workloads(args, workloads, label):
    """Each workload (in order, each causal flag): untimed calls for at least half a second (the
    clock ramps up under load), then `steps` calls; the JSON line lists the (untimed, counted)
    call numbers in launch order."""
    import torch
    import tiled_attention_forward_fwd_amd as fa
    dev = torch.device("cuda:0")
    calls = []
    for cfg in workloads:
        _, _, _, qd, kd, vd = make_inputs(cfg, dev)
        Nq = cfg.get("Nq", cfg["N"])
        qd = qd[:, :, :Nq].contiguous()
        kl = None if cfg.get("key_lens") is None else torch.tensor(cfg["key_lens"], dtype=torch.int32,
                                                                   device=dev)
        for causal in cfg["flags"]:
            def fn(causal=causal):
                fa.fwd(qd, kd, vd, causal=bool(causal), window_left=cfg.get("wl", -1),
                       window_right=cfg.get("wr", -1), key_lens=kl)
            n_warm, t0 = 0, time.perf_counter()
            while n_warm < 5 or time.perf_counter() - t0 < 0.5:
                fn()
                n_warm += 1
                if n_warm % 16 == 0:
                    torch.cuda.synchronize()
            for _ in range(args.steps):
                fn()
            torch.cuda.synchronize()
            calls.append([n_warm, args.steps])
        del qd, kd, vd
    print(json.dumps({"profiled": label, "workloads": workloads, "calls": calls}))


# Workload sets of --profile-kernels / --profile-set: the headline (d=128), the
# headline at d=64, the long-context causal configuration with and without the
# heavy-tailed q, and the two smallest configurations.
PROFILE_SETS = {
    "d128": [HEADLINE],
    "d64": [dict(B=4, H=16, N=4096, d=64, dtype="bf16", seed=6)],
    "long": [dict(B=1, H=32, N=16384, d=128, dtype="bf16", seed=8, flags=(1,)),
             dict(B=1, H=32, N=16384, d=128, dtype="bf16", seed=9, q_scale=4.0, flags=(1,))],
    # the two smallest configurations (key-split launches)
    "small": [dict(B=1, H=1, N=128, d=64, dtype="fp16", seed=1),
              dict(B=2, H=4, N=1000, d=64, dtype="bf16", seed=2)],
}


def profile_kernels(args):
    """A few launches of each kernel of a profile set, nothing else (for rocprofv3
    counter passes): each workload and causal flag in order, `steps` launches."""
    import torch
    import tiled_attention_forward_fwd_amd as fa
    dev = torch.device("cuda:0")
    for cfg in PROFILE_SETS[args.profile_set]:
        _, _, _, qd, kd, vd = make_inputs(cfg, dev)
        for causal in cfg.get("flags", (False, True)):
            for _ in range(args.steps):
                fa.fwd(qd, kd, vd, causal=bool(causal))
        torch.cuda.synchronize()
        del qd, kd, vd
    print(json.dumps({"profiled": args.profile_set, "workloads": PROFILE_SETS[args.profile_set],
                      "launches_each": args.steps}))


def profile_bwd(args):
    """The backward pass at the headline shape, for rocprofv3: per causal flag one forward for O
    and lse, then `steps` fa.bwd calls (delta, dK/dV and dQ kernels each)."""
    import torch
    import tiled_attention_forward_fwd_amd as fa
    from fa_inputs import make_qkv
    dev = torch.device("cuda:0")
    cfg = HEADLINE
    _, _, _, qd, kd, vd = make_inputs(cfg, dev)
    dout = make_qkv(cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["dtype"], cfg["seed"] + 100)[0].to(dev)
    for causal in (False, True):
        o, lse = fa.fwd(qd, kd, vd, causal=causal)
        for _ in range(args.steps):
            fa.bwd(qd, kd, vd, o, lse, dout, causal=causal)
        torch.cuda.synchronize()
    print(json.dumps({"profiled": "backward", "workload": cfg, "calls_each": args.steps}))


DECODE = dict(B=1, H=32, Nq=1, N=16384, d=128, dtype="bf16", seed=10)


def profile_decode(args):
    """KV-cache decode (one query row per head against 16384 keys, B=1 H=32 d=128 bf16, non-causal)
    on the split-key path: `steps` calls back to back after 20 untimed ones, then one JSON line with
    the event-timed average per call and its compulsory HBM rate (for rocprofv3 passes)."""
    import torch
    import tiled_attention_forward_fwd_amd as fa
    dev = torch.device("cuda:0")
    cfg = DECODE
    _, _, _, qd, kd, vd = make_inputs(cfg, dev)
    B, H, Nq, Nk, d = cfg["B"], cfg["H"], cfg["Nq"], cfg["N"], cfg["d"]
    qd = qd[:, :, :Nq].contiguous()
    splits = fa.fa_split_count(B, H, Nq, Nk, d, 0)
    out = torch.empty_like(qd)
    lse = torch.empty((B, H, Nq), device=dev, dtype=torch.float32)
    ws = torch.empty(fa.fa_split_workspace_bytes(B, H, Nq, d, splits) // 4, device=dev,
                     dtype=torch.float32)

    def call():
        fa.fwd(qd, kd, vd, out=out, lse=lse, splits=splits, workspace=ws)
    for _ in range(20):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    plan = fa.fa_plan_qk(B, H, Nq, Nk, d, 0, fa.FA_DTYPE_BF16)
    print(json.dumps({"profiled": f"decode B={B} H={H} Nq={Nq} Nk={Nk} d={d} bf16, {splits} key chunks",
                      "calls": args.steps, "avg_ms_per_call_back_to_back": ms,
                      "algorithmic_bytes": plan["algo_bytes"],
                      "hbm_gbs_compulsory": plan["algo_bytes"] / (ms * 1e-3) / 1e9}))


def copy_calibration(args):
    """A plain copy of a known size, to scale the HBM byte counters."""
    import torch
    dev = torch.device("cuda:0")
    nbytes = 1 << 30
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).normal_()
    dst = torch.empty_like(src)
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                      "launches": args.steps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-stride", type=int, default=1,
                    help="oracle baseline evaluates every Nth query row")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-telemetry", dest="telemetry", action="store_false",
                    help="skip the amd-smi power/clock sample (taken outside the timed region)")
    ap.add_argument("--no-backward", dest="backward", action="store_false",
                    help="skip the backward-pass leg (timed after the headline region)")
    ap.add_argument("--no-gemm-ceiling", dest="gemm_ceiling", action="store_false",
                    help="skip the hipBLASLt GEMM reference run (context for the roofline)")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--no-sweep-oracle", dest="sweep_oracle", action="store_false",
                    help="skip the per-configuration oracle timing of --sweep")
    ap.add_argument("--profile-kernels", action="store_true",
                    help="`steps` launches of each kernel of --profile-set, nothing else")
    ap.add_argument("--profile-set", default="d128", choices=sorted(PROFILE_SETS),
                    help="workloads of --profile-kernels and --profile-timed")
    ap.add_argument("--profile-timed", action="store_true",
                    help="the --profile-set workloads with a warmup before the counted calls (kernel traces)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--profile-decode", action="store_true",
                    help="split-key decode calls only (one query x 16384 keys), for rocprofv3")
    ap.add_argument("--profile-masked", action="store_true",
                    help="padding and sliding-window workloads only, for rocprofv3")
    ap.add_argument("--profile-variants", action="store_true",
                    help="head dims 96 / 32 and fp32 inputs at B4 H16 N4096, for rocprofv3")
    ap.add_argument("--profile-bwd", action="store_true",
                    help="`steps` backward calls at the headline shape per causal flag, for rocprofv3")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this attention forward is built and measured on a "
              "single MI355X (heads shard across GPUs with no exchange, so N>1 adds nothing to "
              "measure here). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import tiled_attention_forward_fwd_amd as fa
    fa.load_library()  # fails loudly if the HIP library is missing

    if args.profile_kernels:
        return profile_kernels(args)
    if args.copy_calibration:
        return copy_calibration(args)
    if args.profile_decode:
        return profile_decode(args)
    if args.profile_masked:
        return profile_workloads(args, MASKED_WORKLOADS, "masked workloads")
    if args.profile_variants:
        return profile_workloads(args, VARIANT_WORKLOADS, "head-dim and fp32 workloads")
    if args.profile_bwd:
        return profile_bwd(args)
    if args.profile_timed:
        return profile_workloads(args, [dict(w, flags=w.get("flags", (0, 1))) for w in PROFILE_SETS[args.profile_set]],
                                 f"profile set {args.profile_set}")

    out, (q, k, v) = headline(args)
    if args.backward:
        out["backward"] = backward_leg()
    if args.gemm_ceiling:
        ceil = gemm_ceiling()
        ceil["attention_noncausal_fraction"] = out["roofline"]["achieved"] / ceil["value"]
        out["gemm_ceiling"] = ceil
    if args.sweep:
        out["sweep"] = sweep(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(HEADLINE, q, k, v, args.cpu_stride)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
