"""Throughput of the batch-invariant W8A16 decode projection on one MI355X.

One step = one call of the projection on the 6144x5120 workload (int8 G32
weights, fp16 scales, bf16 activations) at the fixed width T_pad = 32 with
t = 32 real columns -- the whole hot path for this workload.  The weights are
held in the packed layout (w8_pack, prepared once when the weights are loaded,
outside the timed region) and the step is w8_linear_invariant_packed; the same
is measured on the plain row-major layout (w8_linear_invariant) and reported
beside it.  Both give the same bits.  The weights rotate over enough device
copies (>= 1 GiB) that the 256 MB Infinity Cache cannot serve them, steps are
replayed from HIP graphs, and the time of the timed steps is taken with HIP
events on the stream they run on.  The same is measured at t = 1.  Prints one
JSON line.

  python bench.py [--steps K] [--warmup W] [--no-cpu] [--gpus 1] [--layout packed|plain] [--pmc-pass] [--all]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weight GB/s and TFLOP/s at t=1 and t=T_pad (% roofline); t-invariance pass"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=3300)
    p.add_argument("--warmup", type=int, default=330)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--all", action="store_true",
                   help="instead of the bench line: one JSON line per workload (every configured projection and "
                        "the chain's, at t=1 and t=T_pad, and the head's logprob), with the CPU oracle on a row sample")
    p.add_argument("--only", default="",
                   help="with --all: only the workloads whose name contains this text")
    p.add_argument("--layout", choices=("packed", "plain"), default="packed",
                   help="weight layout of the headline step (the other one is reported beside it)")
    p.add_argument("--pmc-pass", action="store_true",
                   help="for rocprofv3 --pmc: a few plain launches at t=T_pad and t=1, then a plain 512 MiB "
                        "device copy (the calibration for the HBM byte counters); prints one short JSON line")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the projection shards by output rows "
              "with no reduction across GPUs, so per-GPU throughput is the one-GPU number.", file=sys.stderr)
        sys.exit(2)

    import torch

    import invariant_quantized_decode_amd as w8
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.all:
        run_all(torch, w8, synth, dev, args)
        return
    case = synth.LINEAR_6144
    N, K, T_pad = case.N, case.K, case.T_pad
    d = synth.linear_6144_permuted()
    q, s, pool = d["q"], d["s"], d["pool"]
    wbytes = case.weight_bytes

    W0 = torch.from_numpy(q).to(dev)
    S0 = torch.from_numpy(s.view(np.int16)).to(dev)
    copies = max(1, math.ceil((1 << 30) / wbytes))
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    Ss = [S0] + [S0.clone() for _ in range(copies - 1)]
    Ps = [w8.w8_pack(Ws[i], Ss[i]) for i in range(copies)]  # the packed layout, once per copy
    X = torch.from_numpy(pool.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((T_pad, N), dtype=torch.bfloat16, device=dev)

    def step(layout: str, c: int, Xt, t: int, y):
        if layout == "packed":
            return w8.w8_linear_invariant_packed(Ps[c][0], Ps[c][1], Xt, t, T_pad, N, y=y)
        return w8.w8_linear_invariant(Ws[c], Ss[c], Xt, t, T_pad, y=y)

    def kernel_of(layout: str) -> str:
        if layout == "packed":
            return w8.w8_linear_invariant_packed_kernel(N, K, T_pad)
        return w8.w8_linear_invariant_kernel(N, K, T_pad, S0)

    layout, other = args.layout, ("plain" if args.layout == "packed" else "packed")
    kernel = kernel_of(layout)
    if args.pmc_pass:
        for t in (T_pad, 1):
            for i in range(3):
                step(layout, i % copies, X[:t], t, Y)
        torch.cuda.synchronize()
        a = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": case.name, "layout": layout, "kernel": kernel, "launches_per_t": 3,
                          "t": [T_pad, 1], "copy_bytes": a.numel(),
                          "alg_bytes_t_pad": wbytes + 2 * T_pad * (K + N)}), flush=True)
        return

    # ---- t-invariance on this workload: every pool column keeps its bits for t = 1..32, on both
    # layouts, and the two layouts agree bit for bit
    base = step("plain", 0, X, T_pad, None).clone()
    inv_ok = True
    for t in range(1, T_pad + 1):
        cols = torch.from_numpy(d["perms"][t]).to(dev)
        for lay in ("plain", "packed"):
            y = step(lay, 0, X[cols].contiguous(), t, None)
            inv_ok &= bool(torch.equal(y.view(torch.int16), base[cols].view(torch.int16)))
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(device=dev)

    def capture(lay: str, t: int, count: int, start: int):
        g = torch.cuda.CUDAGraph()
        Xt = X[:t]
        with torch.cuda.stream(stream):
            step(lay, 0, Xt, t, Y)  # warm the launch path
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                for i in range(count):
                    step(lay, (start + i) % copies, Xt, t, Y)
        return g

    def measure(lay: str, t: int, steps: int, warmup: int):
        R = copies
        g_full = capture(lay, t, R, 0)
        rem = steps % R
        g_rem = capture(lay, t, rem, 0) if rem else None
        with torch.cuda.stream(stream):
            for _ in range(max(1, math.ceil(warmup / R))):
                g_full.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            wall0 = time.perf_counter()
            e0.record(stream)
            for _ in range(steps // R):
                g_full.replay()
            if g_rem is not None:
                g_rem.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            wall = time.perf_counter() - wall0
        ms = e0.elapsed_time(e1)
        sec_per_step = ms / 1e3 / steps
        alg_bytes = wbytes + 2 * t * K + 2 * t * N
        return dict(
            t=t,
            ms_per_step=ms / steps,
            weight_gbs=wbytes / sec_per_step / 1e9,
            alg_gbs=alg_bytes / sec_per_step / 1e9,
            tflops_useful=2.0 * N * K * t / sec_per_step / 1e12,
            tflops_executed=2.0 * N * K * T_pad / sec_per_step / 1e12,
            wall_s=wall,
            alg_bytes=alg_bytes,
        )

    full = measure(layout, T_pad, args.steps, args.warmup)
    one = measure(layout, 1, args.steps, args.warmup)
    alt_steps = max(copies, args.steps // 3)
    alt_full = measure(other, T_pad, alt_steps, args.warmup // 3)
    alt_one = measure(other, 1, alt_steps, args.warmup // 3)

    # context: a plain device-to-device copy of 1 GiB (read + write bytes / time)
    a = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    with torch.cuda.stream(stream):
        b.copy_(a)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(5):
            b.copy_(a)
        c1.record(stream)
        torch.cuda.synchronize()
    copy_gbs = 5 * 2 * a.numel() / (c0.elapsed_time(c1) / 1e3) / 1e9
    del a, b
    # context: the practical read ceiling of one launch over the same bytes, and the dense bf16
    # matrix-core rate (calibration kernels of libw8calib.so)
    from invariant_quantized_decode_amd import calib
    read_gbs = calib.stream_read_gbs(wbytes)
    mfma_tflops = calib.mfma_bf16_tflops()

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        from invariant_quantized_decode_amd import kernel_source_digest
        rec = json.load(open(tpath))
        if rec.get("kernel_digest") == kernel_source_digest() and rec.get("workload") == case.name \
                and rec.get("kernel") == kernel:
            traffic = rec.get("bytes_per_launch")

    roof = dict(bound="hbm", achieved=round(full["alg_gbs"], 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(full["alg_gbs"] / HBM_PEAK_GBS, 4), traffic=traffic,
                kernel=kernel, bytes_per_launch=full["alg_bytes"],
                avg_launch_us=round(full["ms_per_step"] * 1e3, 3))

    cpu = None
    if not args.no_cpu:
        import oracle
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.w8_linear(q, s, pool)
            reps += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        cpu = dict(value=round(reps * wbytes / el / 1e9, 4), unit="GB/s", cores=oracle.max_threads(),
                   kind="oracle",
                   sample=f"fp64 oracle on the full {N}x{K} projection at t={T_pad}, {reps} repetitions "
                          f"in {el:.1f} s",
                   host_cpus=len(os.sched_getaffinity(0)), cpu_model=cpu_model())

    def r(v, n=3):
        return round(v, n)

    line = {
        "metric": METRIC,
        "value": r(full["weight_gbs"], 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r(full["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.name, "N": N, "K": K, "T_pad": T_pad, "t": T_pad,
                   "weight_bytes": wbytes, "rotating_weight_copies": copies, "launch": "hipGraph replay",
                   "layout": layout + (" (w8_pack, prepared once outside the timed region)" if layout == "packed"
                                       else " (row-major codes and scales as given)")},
        "hbm_frac_t_pad": r(full["weight_gbs"] / HBM_PEAK_GBS, 4),
        "tflops_t_pad": {"useful": r(full["tflops_useful"]), "executed": r(full["tflops_executed"]),
                         "mfma_frac_executed": r(full["tflops_executed"] / BF16_PEAK_TFLOPS, 4)},
        "t1": {"value": r(one["weight_gbs"], 1), "unit": "GB/s", "ms_per_step": r(one["ms_per_step"], 5),
               "hbm_frac": r(one["weight_gbs"] / HBM_PEAK_GBS, 4), "tflops_useful": r(one["tflops_useful"]),
               "tflops_executed": r(one["tflops_executed"])},
        other + "_layout": {"kernel": kernel_of(other), "t_pad": {"value": r(alt_full["weight_gbs"], 1),
                                                                 "ms_per_step": r(alt_full["ms_per_step"], 5),
                                                                 "hbm_frac": r(alt_full["weight_gbs"] / HBM_PEAK_GBS, 4)},
                            "t1": {"value": r(alt_one["weight_gbs"], 1), "ms_per_step": r(alt_one["ms_per_step"], 5),
                                   "hbm_frac": r(alt_one["weight_gbs"] / HBM_PEAK_GBS, 4)}},
        "t_invariance": inv_ok,
        "device_copy_gbs": r(copy_gbs, 1),
        "context": {
            "stream_read_gbs": {str(k): r(v, 1) for k, v in read_gbs.items()},
            "stream_read_note": f"bare nontemporal read of the {wbytes} weight+scale bytes in one launch, by "
                                "workgroup count (the projection uses " + str((N + 31) // 32) + ")",
            "value_vs_best_read": r(full["weight_gbs"] / max(read_gbs.values()), 3),
            "t1_vs_best_read": r(one["weight_gbs"] / max(read_gbs.values()), 3),
            "mfma_bf16_tflops_measured": r(mfma_tflops, 1),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "inputs_sha256": {"codes": sha256_16(q), "scales": sha256_16(s), "activations": sha256_16(pool)},
    }
    print(json.dumps(line), flush=True)


def sha256_16(a) -> str:
    """First 16 hex digits of the SHA-256 of an array's bytes (C order): identifies the synthetic inputs."""
    import hashlib
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def run_all(torch, w8, synth, dev, args):
    """Per-workload figures (context for the bench line): synthetic inputs with the configured value
    distributions drawn on the device, weights rotating over >= 1 GiB of copies, graph-replayed
    launches timed with HIP events on their stream."""
    import oracle

    chain = [("chain qkv 7168x5120", 7168, 5120), ("chain o 5120x6144", 5120, 6144),
             ("chain gate+up 34816x5120", 34816, 5120), ("chain down 5120x17408", 5120, 17408)]
    work = [(c.name, c.N, c.K, c.T_pad, c.scale_eps, "linear") for c in
            (synth.LINEAR_1024, synth.LINEAR_6144, synth.MLP_GATE_UP, synth.MLP_DOWN, synth.HEAD)]
    work += [(n, N, K, synth.CHAIN_T_PAD, 0.0, "linear") for n, N, K in chain]
    # the same projections over the packed layout (w8_pack, prepared once per weight copy)
    work += [(n, N, K, T, e, "packed") for n, N, K, T, e, _ in list(work)]
    # the chain's projections with their glue fused into the epilogue
    work += [("chain o + residual (fused) 5120x6144", 5120, 6144, synth.CHAIN_T_PAD, 0.0, "add"),
             ("chain gate+up + SwiGLU (fused) 34816x5120", 34816, 5120, synth.CHAIN_T_PAD, 0.0, "swiglu"),
             ("chain down + residual (fused) 5120x17408", 5120, 17408, synth.CHAIN_T_PAD, 0.0, "add")]
    work += [(n, N, K, T, e, op + "_packed") for n, N, K, T, e, op in list(work) if op in ("add", "swiglu")]
    def want(workload: str) -> bool:
        return not args.only or args.only in workload

    g = torch.Generator(device=dev)
    g.manual_seed(0)
    stream = torch.cuda.Stream(device=dev)
    for name, N, K, T_pad, eps, op in work:
        if not want(name + (" [packed]" if op.endswith("packed") else "")):
            continue
        wbytes = N * K + 2 * N * (K // 32)
        copies = max(1, math.ceil((1 << 30) / wbytes))
        Ws = [torch.randint(-127, 128, (N, K), generator=g, dtype=torch.int8, device=dev) for _ in range(copies)]
        Ss = [(torch.randn(N, K // 32, generator=g, device=dev).abs_() * 0.02 + eps).half() for _ in range(copies)]
        X = torch.randn(T_pad, K, generator=g, device=dev).to(torch.bfloat16)
        R = torch.randn(T_pad, N, generator=g, device=dev).to(torch.bfloat16)
        Y = torch.empty((T_pad, N // 2 if op.startswith("swiglu") else N), dtype=torch.bfloat16, device=dev)
        if op.endswith("packed"):
            Ps = [w8.w8_pack(Ws[i], Ss[i]) for i in range(copies)]
        # the width the kernels run at: T_pad 48 / 64 calls with t <= 32 run the T_pad 32 kernel
        width = lambda t: T_pad if T_pad <= 32 or t > 32 else 32  # noqa: E731
        if op == "linear":
            kernel = lambda t: w8.w8_linear_invariant_kernel(N, K, width(t), Ss[0])  # noqa: E731
            call = lambda i, t: w8.w8_linear_invariant(Ws[i], Ss[i], X[:t], t, T_pad, y=Y)  # noqa: E731
        elif op == "packed":
            kernel = lambda t: w8.w8_linear_invariant_packed_kernel(N, K, width(t))  # noqa: E731
            call = lambda i, t: w8.w8_linear_invariant_packed(Ps[i][0], Ps[i][1], X[:t], t, T_pad, N, y=Y)  # noqa
        elif op == "add":
            kernel = "gemm_w8g32_split_lds, residual-add epilogue"
            call = lambda i, t: w8.w8_linear_add_invariant(Ws[i], Ss[i], X[:t], R[:t], t, T_pad, y=Y)  # noqa: E731
        elif op == "swiglu":
            kernel = "gemm_w8g32_split_lds, SwiGLU epilogue"
            call = lambda i, t: w8.w8_linear_swiglu_invariant(Ws[i], Ss[i], X[:t], t, T_pad, y=Y)  # noqa: E731
        elif op == "add_packed":
            kernel = "gemm_w8g32_split_lds, residual-add epilogue, packed layout"
            call = lambda i, t: w8.w8_linear_add_invariant_packed(  # noqa: E731
                Ps[i][0], Ps[i][1], X[:t], R[:t], t, T_pad, N, y=Y)
        else:
            kernel = "gemm_w8g32_split_lds, SwiGLU epilogue, packed layout"
            call = lambda i, t: w8.w8_linear_swiglu_invariant_packed(  # noqa: E731
                Ps[i][0], Ps[i][1], X[:t], t, T_pad, N // 2, y=Y)
        for t in (1, T_pad):
            reps = max(2, math.ceil(20000 / copies))  # about 20000 launches, fewer for the largest
            reps = min(reps, max(2, int(2e10 // (wbytes * copies))))
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                call(0, t)
                torch.cuda.synchronize()
                with torch.cuda.graph(graph, stream=stream):
                    for i in range(copies):
                        call(i, t)
                graph.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    graph.replay()
                e1.record(stream)
                torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / 1e3 / (reps * copies)
            # algorithmic bytes: weights and scales, x, y (and the residual read)
            alg = wbytes + 2 * t * K + 2 * t * Y.shape[1] + (2 * t * N if op.startswith("add") else 0)
            # CPU oracle on a 64-row sample of the same projection
            rows = np.arange(0, N, max(1, N // 64))[:64]
            qh = Ws[0][rows].cpu().numpy()
            sh = Ss[0][rows].view(torch.int16).cpu().numpy().view(np.uint16)
            xh = X[:t].view(torch.int16).cpu().numpy().view(np.uint16)
            c0 = time.perf_counter()
            oracle.w8_linear(qh, sh, xh)
            csec = time.perf_counter() - c0
            print(json.dumps({"workload": name + (" [packed]" if op.endswith("packed") else ""), "kernel": kernel(t) if callable(kernel) else kernel, "t": t, "T_pad": T_pad, "us": round(sec * 1e6, 2),
                              "weight_gbs": round(wbytes / sec / 1e9, 1),
                              "roofline_frac": round(alg / sec / 1e9 / HBM_PEAK_GBS, 4),
                              "tflops_useful": round(2.0 * N * K * t / sec / 1e12, 3),
                              "cpu_oracle_gbs": round(len(rows) * K * 1.0625 / csec / 1e9, 4),
                              "cpu_sample": f"{len(rows)} rows, {oracle.max_threads()} threads"}), flush=True)
        del Ws, Ss
        Ps = None
        torch.cuda.empty_cache()
    # the chain's column-local glue at T_pad columns (graph-replayed; bytes = reads + writes)
    H, F, tg = synth.CHAIN_HIDDEN, synth.CHAIN_FFN, synth.CHAIN_T_PAD
    xg = torch.randn(tg, H, generator=g, device=dev).to(torch.bfloat16)
    gu = (torch.randn(tg, 2 * F, generator=g, device=dev) * 30).to(torch.bfloat16)
    yh, yf = torch.empty_like(xg), torch.empty((tg, F), dtype=torch.bfloat16, device=dev)
    for gname, fn, nbytes in (("rmsnorm", lambda: w8.w8i_rmsnorm(xg, 1e-6, y=yh), 2 * 2 * tg * H),
                              ("swiglu", lambda: w8.w8i_swiglu(gu, y=yf), 3 * 2 * tg * F),
                              ("residual add", lambda: w8.w8i_residual_add(xg, xg, y=yh), 3 * 2 * tg * H)):
        if not want(f"glue {gname} t={tg} H={H} F={F}"):
            continue
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            fn()
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=stream):
                for _ in range(50):
                    fn()
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(20):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / 1000
        print(json.dumps({"workload": f"glue {gname} t={tg} H={H} F={F}", "us": round(sec * 1e6, 2),
                          "alg_gbs": round(nbytes / sec / 1e9, 1),
                          "roofline_frac": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
    # the head's logprob epilogue
    V, block = synth.HEAD.N, synth.HEAD_BLOCK
    vocab = (f"vocab block logprob V={V} block={block}", f"vocab greedy argmax V={V}",
             f"vocab block logprob, blockwise-direct V={V}")
    for t in (1, synth.HEAD.T_pad) if any(want(n) for n in vocab) else ():
        logits = (torch.randn(t, V, generator=g, device=dev) * 105).to(torch.bfloat16)
        targets = torch.randint(0, V, (t,), generator=g, device=dev, dtype=torch.int64)
        ws = torch.empty(w8.vocab_block_logprob_workspace_bytes(t, V, block), dtype=torch.uint8, device=dev)
        out = torch.empty(t, dtype=torch.float32, device=dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            w8.vocab_block_logprob(logits, targets, block, out=out, workspace=ws)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=stream):
                for _ in range(20):
                    w8.vocab_block_logprob(logits, targets, block, out=out, workspace=ws)
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(50):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / 1000
        nb = (V + block - 1) // block
        alg = 2 * (2 * t * V) + 8 * t * nb
        lh = logits.view(torch.int16).cpu().numpy().view(np.uint16)
        c0 = time.perf_counter()
        oracle.block_logprob(lh, targets.cpu().numpy(), block)
        csec = time.perf_counter() - c0
        print(json.dumps({"workload": f"vocab block logprob V={V} block={block}", "kernel": "lp_block_max/sumexp/fold",
                          "t": t, "us": round(sec * 1e6, 2), "alg_gbs": round(alg / sec / 1e9, 1),
                          "roofline_frac": round(alg / sec / 1e9 / HBM_PEAK_GBS, 4),
                          "cpu_oracle_us": round(csec * 1e6, 1)}), flush=True)
        # the other head epilogues on the same logits: canonical greedy argmax (one pass over the
        # logits) and the blockwise-direct logprob form
        aws = torch.empty(max(16, w8.vocab_argmax_workspace_bytes(t, V)), dtype=torch.uint8, device=dev)
        aout = torch.empty(t, dtype=torch.int64, device=dev)
        for ename, efn, ebytes, okind in (
                ("greedy argmax", lambda: w8.vocab_argmax(logits, out=aout, workspace=aws), 2 * t * V, "argmax"),
                ("block logprob, blockwise-direct",
                 lambda: w8.vocab_block_logprob_direct(logits, targets, block, out=out, workspace=ws), alg, "direct")):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                efn()
                torch.cuda.synchronize()
                with torch.cuda.graph(graph, stream=stream):
                    for _ in range(20):
                        efn()
                graph.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(50):
                    graph.replay()
                e1.record(stream)
                torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / 1e3 / 1000
            c0 = time.perf_counter()
            if okind == "argmax":
                oracle.argmax(lh)
            else:
                oracle.block_logprob(lh, targets.cpu().numpy(), block, direct=True)
            csec = time.perf_counter() - c0
            print(json.dumps({"workload": f"vocab {ename} V={V}", "t": t, "us": round(sec * 1e6, 2),
                              "alg_gbs": round(ebytes / sec / 1e9, 1),
                              "roofline_frac": round(ebytes / sec / 1e9 / HBM_PEAK_GBS, 4),
                              "cpu_oracle_us": round(csec * 1e6, 1)}), flush=True)


if __name__ == "__main__":
    main()
