"""Benchmark of the MoE expert combine on one MI355X.

A step is one combine over one batch of synthetic inputs already resident in
HBM. Several identical copies of the inputs and outputs are rotated from step
to step, so no launch finds its payload in the 256 MB Infinity Cache or L2
left by the previous one. Two HIP events on the launch stream bracket the K
launches of the timed region; elapsed / K is the kernel duration used for the
roofline. ``value`` is tokens per second of wall-clock time over the
timed region.

Default workload: T=4096, hidden=7168, top_k=8, 256 experts over 8 simulated
ranks, bf16 output. Other workloads (--workload): skewed, rmsnorm,
rmsnorm_mxfp8, mxfp8, mxfp4, dense8 (the local reduce), dispatch (placement
+ row scatter, both kernels per step) and tiny.

The CPU baseline is the oracle (C, OpenMP), timed on the host cores on the
same host arrays: the median of three batches of whole-workload runs (about
ten seconds together) with every OpenMP thread, and the median of three
single-threaded runs; the record names the CPU model, the OS core count and
the threads used.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "combined tokens/s + achieved HBM GB/s (% peak), T=4096 H=7168 top_k=8"
PEAK_GBPS = 8000.0          # MI355X HBM3E, published peak

KIND = {"dsv3": "bf16", "skewed": "bf16", "tiny": "bf16", "rmsnorm": "rmsnorm",
        "mxfp8": "mxfp8", "rmsnorm_mxfp8": "rmsnorm_mxfp8", "mxfp4": "mxfp4",
        "dense8": "dense", "dispatch": "dispatch"}
# workloads that reuse another workload's inputs
INPUTS = {"rmsnorm_mxfp8": "rmsnorm", "mxfp4": "mxfp8"}
DESCR = {
    "dsv3": "moe combine T=4096 H=7168 top_k=8 E=256 ep=8, bf16 out",
    "skewed": "moe combine T=8192 H=4096 top_k=8 E=128 ep=8 zipf1.2, 10% drops + capacity, shared expert, bf16 out",
    "rmsnorm": "moe combine + residual + RMSNorm T=2048 H=7168 top_k=8 E=256 ep=8, weight_bias=1",
    "mxfp8": "moe combine T=16384 H=7168 top_k=8 E=256 ep=8, MXFP8 e4m3 out + UE8M0/32 scales",
    "tiny": "moe combine T=64 H=1024 top_k=2 E=8 ep=1, bf16 out",
    "mxfp4": "moe combine T=16384 H=7168 top_k=8 E=256 ep=8, MXFP4 e2m1 out + UE8M0/32 scales",
    "dense8": "local reduce of 8 partial sums [4096, 7168] bf16 (skip_a2a), bf16 out",
    "dispatch": "moe dispatch (inverse scatter) T=4096 H=7168 top_k=8 E=256 ep=8 capacity 4224, bf16",
    "rmsnorm_mxfp8": "moe combine + residual + RMSNorm T=2048 H=7168 top_k=8 E=256 ep=8, weight_bias=1, normalised row as MXFP8 e4m3 + UE8M0/32",
}



def strip_comments(src):
    """C/C++ source text without comments and with whitespace runs collapsed,
    so that the hash below changes with the code, not with its comments."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":                                   # string or char literal
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


KERNEL_SOURCES = ("combine_kernels.h", "dispatch_kernels.h", "moe_combine.hip")


def kernel_source_hash():
    """sha256 over the device code and the launch planning (what decides the
    bytes a launch moves), comments left out; byte counters taken from other
    kernel code are not reported."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_expert_combine_amd", "csrc")
    files = [os.path.join(csrc, f) for f in KERNEL_SOURCES]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(strip_comments(fh.read()).encode())
    return h.hexdigest()


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def time_cpu_oracle(run, T, algo_bytes, seconds, oracle):
    """The oracle as it stands, on the host cores, over the whole workload.

    Multi-threaded (OpenMP, the threads the process is allowed): three timed
    batches, each repeating the whole workload until it has run for about
    seconds / 3; value = the median batch rate. Single-threaded: three runs of
    the whole workload, median. Returns the cpu_baseline record."""
    import statistics
    threads = oracle.max_threads()
    run()                                              # warm caches and pages

    def batch(min_s):
        reps, t0 = 0, time.perf_counter()
        while True:
            run()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_s:
                return T * reps / dt, reps, dt
    multi = [batch(seconds / 3.0) for _ in range(3)]
    rates = [m[0] for m in multi]
    oracle.set_threads(1)
    try:
        single = [batch(0.0)[0] for _ in range(3)]
    finally:
        oracle.set_threads(threads)
    med = statistics.median(rates)
    return {"value": med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"whole workload ({T} tokens): median of 3 batches of "
                       f"{'/'.join(str(m[1]) for m in multi)} runs "
                       f"({sum(m[2] for m in multi):.1f} s) on {threads} OpenMP threads"),
            "gbps": med * algo_bytes / T / 1e9,
            "batch_tokens_per_s": rates,
            "single_thread": {"value": statistics.median(single), "unit": "tokens/s",
                              "runs_tokens_per_s": single,
                              "sample": f"whole workload ({T} tokens), median of 3 runs"},
            "omp_threads": threads, "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model()}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3", choices=sorted(KIND))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sets", type=int, default=0,
                    help="input copies rotated per step (0: enough for >= 1.5 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="about how long the multi-threaded oracle batches run in total")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="after timing, run 5 device copies of MIB MiB (a plain copy kernel "
                         "of known size, to calibrate profiler byte counters)")
    ap.add_argument("--traffic", default=None,
                    help="JSON with measured HBM bytes per launch (default: "
                         "profiles/traffic_<workload>.json)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported "
              "(the combine and dispatch have no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gen
    import moe_expert_combine_amd as mc

    kind = KIND[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating {args.workload} seed={args.seed}", file=sys.stderr, flush=True)

    def d16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    if kind == "dispatch":
        inp = gen.make_inputs(dict(gen.CONFIGS["dsv3"], H=8), args.seed)   # routing only
        T, k, ep, mtpr, E = inp.T, inp.k, inp.ep, inp.mtpr, inp.meta["E"]
        H = gen.CONFIGS["dsv3"]["H"]
        xs = gen.normal_bf16((T, H), args.seed, 9)
        kept = inp.meta["kept_slots"]
        algo_bytes = T * H * 2 + kept * 2 * H + T * k * (4 + 8)
        ws_bytes = mc.dispatch_workspace_size(T, k, E, ep, mtpr)
        base = dict(payload=d16(xs), src=torch.from_numpy(inp.topk_ids).to(dev), w=None,
                    shared=None)
    elif kind == "dense":
        inp = gen.make_dense_inputs(args.workload, args.seed)
        T, H, k, ep, mtpr = inp.T, inp.H, inp.n_in, inp.n_in, inp.T
        algo_bytes = gen.dense_algorithmic_bytes(inp)
        base = dict(payload=d16(inp.x), src=None, w=None, shared=None)
        kept = T * k
    else:
        inp = gen.make_inputs(INPUTS.get(args.workload, args.workload), args.seed)
        T, H, k, ep, mtpr = inp.T, inp.H, inp.k, inp.ep, inp.mtpr
        algo_bytes = gen.algorithmic_bytes(inp, kind)
        base = dict(payload=d16(inp.payload), src=torch.from_numpy(inp.src_info).to(dev),
                    w=torch.from_numpy(inp.weights).to(dev),
                    shared=None if inp.shared is None else d16(inp.shared))
        kept = inp.meta["kept_slots"]
    if kind in ("rmsnorm", "rmsnorm_mxfp8"):
        base["res"] = d16(inp.residual)
        base["gamma"] = d16(inp.gamma)
    per_set = sum(t.numel() * t.element_size() for t in base.values() if t is not None)
    nsets = args.sets or min(16, max(1, -(-int(1.5 * 2 ** 30) // max(per_set, 1))))
    sets = []
    for i in range(nsets):
        s = {kk: (None if v is None else (v if i == 0 else v.clone())) for kk, v in base.items()}
        if kind == "dispatch":
            s["pay"] = torch.empty((ep, mtpr, H), dtype=torch.bfloat16, device=dev)
            s["si"] = torch.empty((T, k, 2), dtype=torch.int32, device=dev)
            s["ws"] = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        elif kind in ("bf16", "dense"):
            s["out"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        elif kind == "rmsnorm":
            s["ro"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            s["no"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        elif kind == "mxfp4":
            s["codes"] = torch.empty((T, H // 2), dtype=torch.uint8, device=dev)
            s["scales"] = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        elif kind == "rmsnorm_mxfp8":
            s["ro"] = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
            s["codes"] = torch.empty((T, H), dtype=torch.uint8, device=dev)
            s["scales"] = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        else:
            s["codes"] = torch.empty((T, H), dtype=torch.uint8, device=dev)
            s["scales"] = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
        sets.append(s)
    torch.cuda.synchronize()

    L = mc.lib()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    P = lambda t: None if t is None else t.data_ptr()
    calls = []
    for s in sets:
        if kind == "dispatch":
            a = (P(s["payload"]), P(s["src"]), T, H, k, E, ep, mtpr, P(s["pay"]), P(s["si"]), None,
                 P(s["ws"]), ws_bytes, sptr)
            calls.append((L.moe_dispatch, a))
        elif kind == "dense":
            a = (P(s["payload"]), k, None, None, P(s["out"]), T, H, sptr)
            calls.append((L.moe_reduce_dense, a))
        elif kind == "bf16":
            a = (P(s["payload"]), P(s["src"]), P(s["w"]), P(s["shared"]), P(s["out"]),
                 T, H, k, ep, mtpr, sptr)
            calls.append((L.moe_combine, a))
        elif kind == "rmsnorm":
            a = (P(s["payload"]), P(s["src"]), P(s["w"]), P(s["shared"]), P(s["res"]),
                 P(s["gamma"]), inp.eps, 1.0, P(s["ro"]), P(s["no"]), T, H, k, ep, mtpr, sptr)
            calls.append((L.moe_combine_residual_rmsnorm, a))
        elif kind == "rmsnorm_mxfp8":
            a = (P(s["payload"]), P(s["src"]), P(s["w"]), P(s["shared"]), P(s["res"]),
                 P(s["gamma"]), inp.eps, 1.0, P(s["ro"]), None, P(s["codes"]), P(s["scales"]),
                 T, H, k, ep, mtpr, sptr)
            calls.append((L.moe_combine_residual_rmsnorm_mxfp8, a))
        elif kind == "mxfp4":
            a = (P(s["payload"]), P(s["src"]), P(s["w"]), P(s["shared"]), P(s["codes"]),
                 P(s["scales"]), T, H, k, ep, mtpr, sptr)
            calls.append((L.moe_combine_mxfp4, a))
        else:
            a = (P(s["payload"]), P(s["src"]), P(s["w"]), P(s["shared"]), P(s["codes"]),
                 P(s["scales"]), T, H, k, ep, mtpr, sptr)
            calls.append((L.moe_combine_mxfp8, a))

    def step(i):
        fn, a = calls[i % len(calls)]
        st = fn(*a)
        if st != 0:
            raise RuntimeError(L.moe_combine_last_error().decode())

    print(f"[bench] warmup {args.warmup} steps ({nsets} input sets)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    K = args.steps
    # timed region: K back-to-back launches between two events on the launch
    # stream; their mean is the kernel duration the roofline uses
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = e0.elapsed_time(e1) / K
    ms_per_step = wall * 1e3 / K
    tokens_per_s = T * K / wall
    achieved = algo_bytes / (kernel_ms * 1e-3) / 1e9
    # spread only: a short pass with an event pair around every launch (the
    # extra event packets add a few microseconds to each sample)
    n_sp = min(K, 100)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_sp)]
    for i in range(n_sp):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    kms = np.array([a.elapsed_time(b) for a, b in ev])
    print(f"[bench] kernel mean {kernel_ms * 1e3:.1f} us over the timed region; per-launch "
          f"median {np.median(kms) * 1e3:.1f} p10 {np.percentile(kms, 10) * 1e3:.1f} "
          f"p90 {np.percentile(kms, 90) * 1e3:.1f} us; "
          f"{achieved:.0f} GB/s", file=sys.stderr, flush=True)

    if args.copy_probe:
        src_t = torch.empty(args.copy_probe << 19, dtype=torch.int16, device=dev).fill_(3)
        dst_t = torch.empty_like(src_t)
        for _ in range(5):
            dst_t.copy_(src_t)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: 5 x {args.copy_probe} MiB device copies", file=sys.stderr, flush=True)
        del src_t, dst_t

    traffic = None
    tpath = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            tr = json.load(f)
        if (tr.get("workload") == args.workload
                and tr.get("kernel_source_sha256") == kernel_source_hash()):
            traffic = tr.get("bytes_per_launch")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        if kind == "dispatch":
            run = lambda: oracle.dispatch(xs, inp.topk_ids, E, ep, mtpr)
        elif kind == "dense":
            run = lambda: oracle.reduce_dense(inp.x)
        elif kind == "bf16":
            run = lambda: oracle.combine(inp.payload, inp.src_info, inp.weights, inp.shared, checked=False)
        elif kind == "rmsnorm":
            run = lambda: oracle.combine_residual_rmsnorm(inp.payload, inp.src_info, inp.weights,
                                                          inp.shared, inp.residual, inp.gamma,
                                                          inp.eps, 1.0, checked=False)
        elif kind == "mxfp4":
            run = lambda: oracle.combine_mxfp4(inp.payload, inp.src_info, inp.weights, inp.shared,
                                               checked=False)
        elif kind == "rmsnorm_mxfp8":
            run = lambda: oracle.combine_residual_rmsnorm_mxfp8(
                inp.payload, inp.src_info, inp.weights, inp.shared, inp.residual, inp.gamma,
                inp.eps, 1.0, checked=False)
        else:
            run = lambda: oracle.combine_mxfp8(inp.payload, inp.src_info, inp.weights, inp.shared,
                                               checked=False)
        cpu = time_cpu_oracle(run, T, algo_bytes, args.cpu_seconds, oracle)

    rec = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",   # fp32 arithmetic; inputs and outputs are bf16 (io_dtype)
        "config": {"workload": DESCR[args.workload], "num_tokens": T, "hidden": H,
                   "top_k": k, "ep_size": ep, "max_tokens_per_rank": mtpr,
                   "kept_slots": kept, "io_dtype": "bf16",
                   "seed": args.seed, "input_sets": nsets,
                   "launch": mc.describe_launch({"bf16": 0, "dense": 0, "rmsnorm": 1, "mxfp8": 2,
                                                 "rmsnorm_mxfp8": 3, "mxfp4": 4,
                                                 "dispatch": 5}[kind], T, H, k)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "kernel_us_mean": kernel_ms * 1e3,
                     "kernel_us_median_per_launch_events": float(np.median(kms) * 1e3),
                     "kernel_us_p10_p90_per_launch_events": [float(np.percentile(kms, 10) * 1e3),
                                                             float(np.percentile(kms, 90) * 1e3)]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
