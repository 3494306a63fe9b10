"""Throughput of the batch-invariant W8A16 decode path on one MI355X.

One step = the whole hot path on the largest single-GPU workload: the 248320x5120 vocabulary head
(int8 G32 weights, fp16 scales, bf16 hidden states) at the fixed width T_pad = 32 with t = 32 real
columns, then the blockwise target logprob of every column over 4096-wide vocabulary blocks.  The
head's weights are held in the packed layout (w8_pack, prepared once when the weights are loaded,
outside the timed region), so a step is w8_linear_invariant_packed followed by vocab_block_logprob;
the plain row-major layout (w8_linear_invariant) is measured beside it (same bits).  The same step
is measured at t = 1.

Timing: steps are replayed from HIP graphs in batches of at least 20 ms, with HIP events on the
stream they run on between batches; every figure is the median over at least 10 batches (spread
given beside it).  The K steps of --steps form the timed region of the contract (a barrier and a
device synchronisation on both sides); when they hold fewer than 10 whole batches, further batches
follow it.  Weights (1.35 GB) exceed the 256 MB Infinity Cache; the logits buffers rotate over
>= 1 GiB.  The dominant kernel (the head projection) and the logprob's kernels are also timed on
their own, the same way, for the roofline.  The 6144x5120 projection at T_pad 32 is reported as a
sub-record.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--no-cpu] [--gpus 1] [--all [--only TEXT]]
                  [--pmc-pass {head,linear6144,mlp_gate_up}]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "weight GB/s and TFLOP/s at t=1 and t=T_pad (% roofline); t-invariance pass"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
GIB = 1 << 30


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=640)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--batch-ms", type=float, default=20.0, help="minimum length of one timed batch")
    p.add_argument("--min-batches", type=int, default=10, help="batches behind every median")
    p.add_argument("--all", action="store_true",
                   help="instead of the bench line: one JSON line per workload (every configured projection and "
                        "the chain's, at t=1 and t=T_pad, and the head's logprob), with the CPU oracle on a row sample")
    p.add_argument("--only", default="",
                   help="with --all: only the workloads whose name contains this text")
    p.add_argument("--pmc-pass", choices=("head", "linear6144", "mlp_gate_up"), default=None,
                   help="for rocprofv3 --pmc: 3 launches of the workload's projection kernel at t=T_pad and 3 at "
                        "t=1, then a plain 512 MiB device copy 3 times (the calibration for the HBM byte "
                        "counters); prints one short JSON line")
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
    if args.pmc_pass:
        pmc_pass(torch, w8, synth, dev, args.pmc_pass)
        return
    headline(torch, w8, synth, dev, args)


# ------------------------------------------------------------------ timing
class Timer:
    """Graph-replayed batches on one stream, HIP events between them."""

    def __init__(self, torch, stream, batch_ms: float, min_batches: int):
        self.torch, self.stream = torch, stream
        self.batch_ms, self.min_batches = batch_ms, min_batches
        # per measure: (label, calls run on the GPU in launch order, how many of the last ones are timed),
        # printed to stderr so that a kernel trace of this run can be split by phase
        self.log = []

    def graph(self, calls):
        """One HIP graph of the zero-argument callables `calls` (each launch path warmed eagerly first)."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            calls[0]()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=self.stream):
                for c in calls:
                    c()
        return g

    def replay_timed(self, graph, n: int):
        """Replay `graph` n times back to back, an event before and after each; durations in ms."""
        torch = self.torch
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        with torch.cuda.stream(self.stream):
            ev[0].record(self.stream)
            for i in range(n):
                graph.replay()
                ev[i + 1].record(self.stream)
        torch.cuda.synchronize()
        return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]

    def per_call_ms(self, make_call, count: int):
        """Eager estimate of one call's time (ms): `count` distinct calls after one warm-up round."""
        torch = self.torch
        calls = [make_call(i) for i in range(count)]
        with torch.cuda.stream(self.stream):
            for c in calls:
                c()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            for c in calls:
                c()
            e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / count

    def measure(self, make_call, steps: int | None = None, warmup: int = 0, est_count: int = 4, label: str = ""):
        """Median time of one call: make_call(i) is the i-th call (rotating buffers by i).  Batches of B
        calls (B from an eager estimate so that a batch lasts >= batch_ms) are captured once and
        replayed; with `steps`, exactly that many calls form one timed region (a synchronisation on
        both sides; the last batch is a graph of the remainder), and whole batches follow it until
        min_batches whole batches are timed.  Returns a dict of per-call figures in microseconds."""
        torch = self.torch
        est = self.per_call_ms(make_call, est_count)
        B = max(1, math.ceil(self.batch_ms / max(est, 1e-4)))
        g = self.graph([make_call(i) for i in range(B)])
        n_warm = max(1, math.ceil(warmup / B))
        for _ in range(n_warm):
            g.replay()
        torch.cuda.synchronize()
        region_ms, batches, rem = None, [], 0
        if steps is not None:
            rem = steps % B
            g_rem = self.graph([make_call(i) for i in range(rem)]) if rem else None
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps // B + 1)]
            with torch.cuda.stream(self.stream):
                e0.record(self.stream)
                ev[0].record(self.stream)
                for i in range(steps // B):
                    g.replay()
                    ev[i + 1].record(self.stream)
                if g_rem is not None:
                    g_rem.replay()
                e1.record(self.stream)
            torch.cuda.synchronize()
            region_ms = e0.elapsed_time(e1)
            batches = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps // B)]
        extra = max(0, self.min_batches - len(batches))
        if extra:
            batches += self.replay_timed(g, extra)
        timed = (steps // B * B + rem if steps is not None else 0) + extra * B
        self.log.append((label, 2 * est_count + 1 + n_warm * B + (1 if rem else 0) + timed, timed))
        per = sorted(b / B * 1e3 for b in batches)
        q = statistics.quantiles(per, n=4) if len(per) >= 2 else [per[0]] * 3
        return dict(us=statistics.median(per), min_us=per[0], max_us=per[-1], q1_us=q[0], q3_us=q[2],
                    batch=B, batches=len(per), batch_ms=statistics.median(batches),
                    region_ms=region_ms, region_steps=steps)


def spread(m: dict) -> dict:
    return {"median_us": round(m["us"], 3), "min_us": round(m["min_us"], 3), "max_us": round(m["max_us"], 3),
            "iqr_us": [round(m["q1_us"], 3), round(m["q3_us"], 3)], "batches": m["batches"],
            "calls_per_batch": m["batch"], "median_batch_ms": round(m["batch_ms"], 3)}


def r(v, n=3):
    return None if v is None else round(v, n)


# ------------------------------------------------------------------ headline
def headline(torch, w8, synth, dev, args):
    """The bench line: head + logprob steps at t = 32 and t = 1 (see the module docstring)."""
    case = synth.HEAD
    N, K, T_pad, block = case.N, case.K, case.T_pad, synth.HEAD_BLOCK
    d = synth.head_logprob()
    q, s, pool, targets = d["q"], d["s"], d["pool"], d["targets"]
    wbytes = case.weight_bytes
    nb = (N + block - 1) // block

    W0 = torch.from_numpy(q).to(dev)
    S0 = torch.from_numpy(s.view(np.int16)).to(dev)
    Wp, Sp = w8.w8_pack(W0, S0)  # the packed layout, once (load time)
    X = torch.from_numpy(pool.view(np.int16)).to(dev).view(torch.bfloat16)
    Tg = torch.from_numpy(targets).to(dev)
    n_logits = max(1, math.ceil(GIB / (T_pad * N * 2)))  # logits buffers rotating over >= 1 GiB
    Ls = [torch.empty((T_pad, N), dtype=torch.bfloat16, device=dev) for _ in range(n_logits)]
    ws = torch.empty(w8.vocab_block_logprob_workspace_bytes(T_pad, N, block), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(w8.w8_head_logprob_workspace_bytes(T_pad, N, block), dtype=torch.uint8, device=dev)
    out = torch.empty(T_pad, dtype=torch.float32, device=dev)
    kernel = w8.w8_linear_invariant_packed_kernel(N, K, T_pad)
    kernel_plain = w8.w8_linear_invariant_kernel(N, K, T_pad, S0)

    def project(layout, Xt, t, y):
        if layout == "packed":
            return w8.w8_linear_invariant_packed(Wp, Sp, Xt, t, T_pad, N, y=y)
        return w8.w8_linear_invariant(W0, S0, Xt, t, T_pad, y=y)

    def logprob(lg, tg, t):
        return w8.vocab_block_logprob(lg, tg, block, out=out, t=t, workspace=ws)

    def fused(Xt, tg, t, lg):
        # the head projection with the logprob's row-max pass fused into it, then the logprob's
        # block partials and fold (w8_head_logprob_invariant_packed): the same bits as project + logprob
        return w8.w8_head_logprob_invariant_packed(Wp, Sp, Xt, tg, t, T_pad, block, N, logits=lg, out=out,
                                                   workspace=ws_f)

    # ---- t-invariance on this workload, before any timing: for t = 1..32 a random ordered subset of the
    # 32 pool columns keeps the logits bits and the logprob bits it has in the identity-order t = 32 run,
    # on both layouts (the plain layout at t = 32 and at every fourth t)
    base = project("packed", X, T_pad, None).clone()
    base_lp = w8.vocab_block_logprob(base, Tg, block).clone()
    inv = {"logits": True, "logprob": True, "plain_layout": True, "fused": True}
    for t in range(1, T_pad + 1):
        cols = torch.from_numpy(d["perms"][t]).to(dev)
        Xc = X[cols].contiguous()
        y = project("packed", Xc, t, None)
        inv["logits"] &= bool(torch.equal(y.view(torch.int16), base[cols].view(torch.int16)))
        lp = w8.vocab_block_logprob(y, Tg[cols].contiguous(), block)
        inv["logprob"] &= bool(torch.equal(lp.view(torch.int32), base_lp[cols].view(torch.int32)))
        if t % 4 == 0 or t == 1:
            yp = project("plain", Xc, t, None)
            inv["plain_layout"] &= bool(torch.equal(yp.view(torch.int16), base[cols].view(torch.int16)))
        fl, fo = w8.w8_head_logprob_invariant_packed(Wp, Sp, Xc, Tg[cols].contiguous(), t, T_pad, block, N)
        inv["fused"] &= bool(torch.equal(fl.view(torch.int16), base[cols].view(torch.int16))) and \
            bool(torch.equal(fo.view(torch.int32), base_lp[cols].view(torch.int32)))
    torch.cuda.synchronize()
    inv_ok = all(inv.values())

    stream = torch.cuda.Stream(device=dev)
    timer = Timer(torch, stream, args.batch_ms, args.min_batches)

    def step_call(t):
        def make(i):
            lg = Ls[i % n_logits]
            return lambda: (project("packed", X[:t], t, lg), logprob(lg, Tg, t))
        return make

    def fused_call(t):
        def make(i):
            lg = Ls[i % n_logits]
            return lambda: fused(X[:t], Tg, t, lg)
        return make

    def gemm_call(layout, t):
        def make(i):
            lg = Ls[i % n_logits]
            return lambda: project(layout, X[:t], t, lg)
        return make

    def lp_call(t):
        def make(i):
            lg = Ls[i % n_logits]
            return lambda: logprob(lg, Tg, t)
        return make

    timer.log.append(("t-invariance (packed; plain: 9)", T_pad + 1, 0))
    # the contract's timed region: exactly --steps steps at t = T_pad (warm-up before it)
    step = {T_pad: timer.measure(step_call(T_pad), steps=args.steps, warmup=args.warmup, label=f"step t={T_pad}")}
    step[1] = timer.measure(step_call(1), warmup=args.warmup, label="step t=1")
    fstep = {t: timer.measure(fused_call(t), warmup=args.warmup, label=f"fused step t={t}") for t in (T_pad, 1)}
    gemm = {t: timer.measure(gemm_call("packed", t), warmup=args.warmup, label=f"projection t={t}")
            for t in (T_pad, 1)}
    # every logits buffer holds a full projection before the logprob is timed on its own (cold: the
    # buffers rotate over >= 1 GiB, past the Infinity Cache)
    for lg in Ls:
        project("packed", X, T_pad, lg)
    timer.log.append(("logits fill", n_logits, 0))
    lpk = {t: timer.measure(lp_call(t), warmup=args.warmup, label=f"logprob t={t}") for t in (T_pad, 1)}
    plain = {t: timer.measure(gemm_call("plain", t), warmup=args.warmup // 4, label=f"plain projection t={t}")
             for t in (T_pad, 1)}
    print(json.dumps({"launch_log": timer.log, "kernel": kernel, "kernel_plain": kernel_plain}), file=sys.stderr,
          flush=True)

    def alg_gemm(t):  # weights + scales, x, y
        return wbytes + 2 * t * K + 2 * t * N

    def alg_lp(t):  # two passes over the logits, block maxima and partials written and read, targets, out
        return 2 * (2 * t * N) + 4 * (4 * t * nb) + 12 * t

    def gbs(nbytes, us):
        return nbytes / (us * 1e-6) / 1e9

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tpath):
        from invariant_quantized_decode_amd import kernel_source_digest
        rec = json.load(open(tpath))
        if rec.get("kernel_digest") == kernel_source_digest() and rec.get("workload") == case.name \
                and rec.get("kernel") == kernel:
            traffic = rec.get("bytes_per_launch")

    g32, g1 = gemm[T_pad]["us"], gemm[1]["us"]
    roof = dict(bound="hbm", achieved=r(gbs(alg_gemm(T_pad), g32), 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=r(gbs(alg_gemm(T_pad), g32) / HBM_PEAK_GBS, 4), traffic=traffic,
                kernel=kernel, bytes_per_launch=alg_gemm(T_pad), avg_launch_us=r(g32),
                launch_us_spread=spread(gemm[T_pad]),
                t1={"achieved": r(gbs(alg_gemm(1), g1), 1), "frac": r(gbs(alg_gemm(1), g1) / HBM_PEAK_GBS, 4),
                    "bytes_per_launch": alg_gemm(1), "avg_launch_us": r(g1), "launch_us_spread": spread(gemm[1])})
    st32, st1 = step[T_pad]["us"], step[1]["us"]
    step_rec = {t: {"us": r(step[t]["us"]), "weight_gbs": r(gbs(wbytes, step[t]["us"]), 1),
                    "hbm_frac_weights": r(gbs(wbytes, step[t]["us"]) / HBM_PEAK_GBS, 4),
                    "alg_bytes": alg_gemm(t) + alg_lp(t),
                    "alg_frac": r(gbs(alg_gemm(t) + alg_lp(t), step[t]["us"]) / HBM_PEAK_GBS, 4),
                    "spread": spread(step[t])} for t in (T_pad, 1)}
    lp_rec = {t: {"us": r(lpk[t]["us"]), "alg_bytes": alg_lp(t),
                  "alg_frac": r(gbs(alg_lp(t), lpk[t]["us"]) / HBM_PEAK_GBS, 4),
                  "note": "cold: logits rotate over >= 1 GiB", "spread": spread(lpk[t])} for t in (T_pad, 1)}
    targets_met = {"t1_hbm_frac_ge_0.70": bool(gbs(wbytes, st1) / HBM_PEAK_GBS >= 0.70),
                   "t_pad_hbm_frac_ge_0.50": bool(gbs(wbytes, st32) / HBM_PEAK_GBS >= 0.50),
                   "kernel_t1_frac_ge_0.70": bool(roof["t1"]["frac"] >= 0.70),
                   "kernel_t_pad_frac_ge_0.50": bool(roof["frac"] >= 0.50)}

    # free the head's buffers before the sub-record and the calibration
    del Ls, W0, S0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    sub = linear6144_record(torch, w8, synth, dev, timer, args)

    # context: a plain device-to-device copy of 1 GiB (read + write bytes / time), and the practical read
    # ceiling of one launch over the head's weight bytes plus the dense bf16 matrix-core rate
    # (calibration kernels of libw8calib.so)
    a = torch.zeros(GIB, dtype=torch.uint8, device=dev)
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
    torch.cuda.empty_cache()
    from invariant_quantized_decode_amd import calib
    read_gbs = calib.stream_read_gbs(wbytes, workgroups=(256, 512, 1024, 2048), replays=4)
    strip_gbs = calib.strip_read_gbs(N, K, workgroups=256, replays=4)
    best_read = max(max(read_gbs.values()), strip_gbs)
    mfma_tflops = calib.mfma_bf16_tflops()

    cpu, parity = None, None
    if not args.no_cpu:
        cpu, parity = cpu_baseline(torch, q, s, pool, targets, block, base, base_lp, wbytes, args)

    line = {
        "metric": METRIC,
        "value": r(gbs(wbytes, st32), 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r(st32 / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{case.name} + block-{block} logprob", "N": N, "K": K, "T_pad": T_pad, "t": T_pad,
                   "vocab_block": block, "weight_bytes": wbytes, "step": "w8_linear_invariant_packed + "
                   "vocab_block_logprob", "logits_buffers": n_logits, "launch": "hipGraph replay",
                   "layout": "packed (w8_pack, prepared once outside the timed region)",
                   "value_is": "weight bytes of the head / median step time"},
        "timing": {"timed_region": {"steps": args.steps, "ms": r(step[T_pad]["region_ms"], 3),
                                    "ms_per_step": r(step[T_pad]["region_ms"] / args.steps, 5)},
                   "median_of": step[T_pad]["batches"], "steps_per_batch": step[T_pad]["batch"],
                   "step_us_spread": spread(step[T_pad])},
        "hbm_frac_t_pad": step_rec[T_pad]["hbm_frac_weights"],
        "tflops_t_pad": {"useful": r(2.0 * N * K * T_pad / (st32 * 1e-6) / 1e12),
                         "executed": r(2.0 * N * K * T_pad / (st32 * 1e-6) / 1e12),
                         "mfma_frac_executed": r(2.0 * N * K * T_pad / (st32 * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "t1": {"value": step_rec[1]["weight_gbs"], "unit": "GB/s", "ms_per_step": r(st1 / 1e3, 5),
               "hbm_frac": step_rec[1]["hbm_frac_weights"],
               "tflops_useful": r(2.0 * N * K / (st1 * 1e-6) / 1e12),
               "tflops_executed": r(2.0 * N * K * T_pad / (st1 * 1e-6) / 1e12), "spread": spread(step[1])},
        "step": {"t_pad": step_rec[T_pad], "t1": step_rec[1]},
        "fused_step": {"call": "w8_head_logprob_invariant_packed (head projection with the row-max pass fused, "
                               "then block partials and fold; the same bits)",
                       "t_pad": {"us": r(fstep[T_pad]["us"]), "weight_gbs": r(gbs(wbytes, fstep[T_pad]["us"]), 1),
                                 "spread": spread(fstep[T_pad])},
                       "t1": {"us": r(fstep[1]["us"]), "weight_gbs": r(gbs(wbytes, fstep[1]["us"]), 1),
                              "spread": spread(fstep[1])}},
        "kernels": {"head_projection": {"kernel": kernel, "t_pad_us": r(g32), "t1_us": r(g1)},
                    "logprob": {"kernels": "lp_block_max + lp_block_sumexp + lp_fold", "t_pad": lp_rec[T_pad],
                                "t1": lp_rec[1]}},
        "plain_layout": {"kernel": kernel_plain,
                         "t_pad": {"us": r(plain[T_pad]["us"]), "weight_gbs": r(gbs(wbytes, plain[T_pad]["us"]), 1),
                                   "alg_frac": r(gbs(alg_gemm(T_pad), plain[T_pad]["us"]) / HBM_PEAK_GBS, 4)},
                         "t1": {"us": r(plain[1]["us"]), "weight_gbs": r(gbs(wbytes, plain[1]["us"]), 1),
                                "alg_frac": r(gbs(alg_gemm(1), plain[1]["us"]) / HBM_PEAK_GBS, 4)}},
        "targets_met": targets_met,
        "t_invariance": inv_ok,
        "t_invariance_detail": inv,
        "parity_vs_oracle": parity,
        "linear_6144x5120": sub,
        "device_copy_gbs": r(copy_gbs, 1),
        "context": {
            "stream_read_gbs": {str(k): r(v, 1) for k, v in read_gbs.items()},
            "stream_read_note": f"bare nontemporal read of the head's {wbytes} weight+scale bytes in one launch, "
                                "by workgroup count (the projection runs one persistent workgroup per CU)",
            "strip_read_gbs": r(strip_gbs, 1),
            "strip_read_note": "the head's packed codes and scales read the way the persistent projection "
                               "streams them: 256 workgroups x 8 waves, one strip per wave, its 2 KB blocks "
                               "and 128-byte scale lines in order, 8 blocks in flight per wave",
            "value_vs_best_read": r(gbs(wbytes, st32) / best_read, 3),
            "t1_vs_best_read": r(gbs(wbytes, st1) / best_read, 3),
            "kernel_vs_strip_read": {"t_pad": r(gbs(wbytes, g32) / strip_gbs, 3),
                                     "t1": r(gbs(wbytes, g1) / strip_gbs, 3)},
            "mfma_bf16_tflops_measured": r(mfma_tflops, 1),
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "inputs_sha256": {"codes": sha256_16(q), "scales": sha256_16(s), "activations": sha256_16(pool),
                          "targets": sha256_16(targets)},
    }
    print(json.dumps(line), flush=True)


def linear6144_record(torch, w8, synth, dev, timer, args):
    """Sub-record: the 6144x5120 projection at T_pad 32 (t = 32 and t = 1), packed and plain layouts,
    weights rotating over >= 1 GiB of copies, with its own t-invariance check."""
    case = synth.LINEAR_6144
    N, K, T_pad = case.N, case.K, case.T_pad
    d = synth.linear_6144_permuted()
    q, s, pool = d["q"], d["s"], d["pool"]
    wbytes = case.weight_bytes
    W0 = torch.from_numpy(q).to(dev)
    S0 = torch.from_numpy(s.view(np.int16)).to(dev)
    copies = max(1, math.ceil(GIB / wbytes))
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    Ss = [S0] + [S0.clone() for _ in range(copies - 1)]
    Ps = [w8.w8_pack(Ws[i], Ss[i]) for i in range(copies)]
    X = torch.from_numpy(pool.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((T_pad, N), dtype=torch.bfloat16, device=dev)

    def call(layout, t):
        def make(i):
            c = i % copies
            if layout == "packed":
                return lambda: w8.w8_linear_invariant_packed(Ps[c][0], Ps[c][1], X[:t], t, T_pad, N, y=Y)
            return lambda: w8.w8_linear_invariant(Ws[c], Ss[c], X[:t], t, T_pad, y=Y)
        return make

    base = w8.w8_linear_invariant(W0, S0, X, T_pad, T_pad).clone()
    inv_ok = True
    for t in range(1, T_pad + 1):
        cols = torch.from_numpy(d["perms"][t]).to(dev)
        Xc = X[cols].contiguous()
        for y in (w8.w8_linear_invariant(W0, S0, Xc, t, T_pad), w8.w8_linear_invariant_packed(*Ps[0], Xc, t, T_pad, N)):
            inv_ok &= bool(torch.equal(y.view(torch.int16), base[cols].view(torch.int16)))
    torch.cuda.synchronize()
    res = {}
    for layout in ("packed", "plain"):
        for t in (T_pad, 1):
            m = timer.measure(call(layout, t), warmup=args.warmup, label=f"6144x5120 {layout} t={t}")
            alg = wbytes + 2 * t * (K + N)
            res[f"{layout}_t{t}"] = {"us": r(m["us"]), "weight_gbs": r(wbytes / (m["us"] * 1e-6) / 1e9, 1),
                                     "alg_frac": r(alg / (m["us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                     "spread": spread(m)}
    rec = {"workload": case.name, "T_pad": T_pad, "rotating_weight_copies": copies,
           "kernel_packed": w8.w8_linear_invariant_packed_kernel(N, K, T_pad),
           "kernel_plain": w8.w8_linear_invariant_kernel(N, K, T_pad, S0), "t_invariance": inv_ok, **res}
    del Ws, Ss, Ps, W0, S0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(torch, q, s, pool, targets, block, base_logits, base_lp, wbytes, args):
    """The CPU oracle on the same step (fp64 head projection of all 32 columns, then the fixed-order fp32
    logprob of its bf16-rounded logits), repeated for >= --cpu-seconds on the host's cores.  Its first
    repetition also checks the GPU step against it: every logit within 2 bf16 ulps of the fp64 value and
    the logprob of the GPU's logits equal to the oracle's (1e-5 bar; bits counted)."""
    import oracle
    yg = base_logits.view(torch.int16).cpu().numpy().view(np.uint16)
    reps, t0, lp_ref = 0, time.perf_counter(), None
    while True:
        oracle.w8_linear(q, s, pool)
        lp = oracle.block_logprob(yg, targets, block)
        if lp_ref is None:
            lp_ref = lp
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    cpu = dict(value=round(reps * wbytes / el / 1e9, 4), unit="GB/s", cores=oracle.max_threads(), kind="oracle",
               sample=f"the whole step on the host: fp64 oracle projection of the full {q.shape[0]}x{q.shape[1]} "
                      f"head at t={pool.shape[0]} plus the fp32 fixed-order block-{block} logprob, {reps} "
                      f"repetitions in {el:.1f} s",
               host_cpus=len(os.sched_getaffinity(0)), cpu_model=cpu_model())
    # parity of the GPU step (untimed): every logit against the fp64 value -- within 2 bf16 ulps, or, where
    # the exact value has cancelled below what fp32 accumulation resolves, within one fp32 rounding of
    # sum |q s x| (counted as misses of 2 ulps) -- and the logprob against the fixed-order fp32 oracle
    y_ref, mass = oracle.w8_linear(q, s, pool, mass=True)
    yv = (yg.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.abs(y_ref)
    e = np.maximum(np.frexp(np.where(a > 0, a, 1.0))[1] - 1, -126)
    ulp = np.where(a > 0, np.ldexp(1.0, e - 7), 2.0 ** -133)
    d = np.abs(yv - y_ref)
    err = d / ulp
    in_ulps = err <= 2.0
    floor_ok = d <= 2.0 ** -24 * mass
    lpg = base_lp.cpu().numpy()
    parity = {"logits_outputs": int(err.size), "logits_within_2_ulp": int(np.sum(in_ulps)),
              "logits_misses_within_fp32_floor": int(np.sum(~in_ulps & floor_ok)),
              "logits_outside_bar": int(np.sum(~in_ulps & ~floor_ok)),
              "logits_max_err_bf16_ulp_within_bar": round(float(err[in_ulps].max()), 3),
              "logprob_max_abs_diff": float(np.max(np.abs(lpg.astype(np.float64) - lp_ref))),
              "logprob_not_bitwise": int(np.sum(lpg.view(np.uint32) != lp_ref.view(np.uint32)))}
    return cpu, parity


def pmc_pass(torch, w8, synth, dev, which: str):
    """For rocprofv3 --pmc runs: 3 launches of the workload's projection kernel (packed layout) at
    t = T_pad and 3 at t = 1, then a plain 512 MiB device copy 3 times (the counters' calibration)."""
    case = {"head": synth.HEAD, "linear6144": synth.LINEAR_6144, "mlp_gate_up": synth.MLP_GATE_UP}[which]
    N, K, T_pad = case.N, case.K, case.T_pad
    rng = np.random.default_rng(case.seed)
    q = synth.draw_codes(rng, N, K)
    s = synth.draw_scales(rng, N, K, case.scale_eps)
    x = synth.draw_acts(rng, T_pad, K)
    W0 = torch.from_numpy(q).to(dev)
    S0 = torch.from_numpy(s.view(np.int16)).to(dev)
    copies = 3 if which == "head" else 6  # distinct weights per launch: none is served from a cache
    Ps = [w8.w8_pack(W0, S0)] + ([] if which == "head" else [w8.w8_pack(W0.clone(), S0.clone()) for _ in range(copies - 1)])
    del W0, S0
    X = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    Y = torch.empty((T_pad, N), dtype=torch.bfloat16, device=dev)
    for t in (T_pad, 1):
        for i in range(3):
            P = Ps[i % len(Ps)]
            w8.w8_linear_invariant_packed(P[0], P[1], X[:t], t, T_pad, N, y=Y)
    torch.cuda.synchronize()
    a = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_pass": case.name, "layout": "packed", "kernel": w8.w8_linear_invariant_packed_kernel(N, K, T_pad),
                      "launches_per_t": 3, "t": [T_pad, 1], "copy_bytes": a.numel(),
                      "alg_bytes_t_pad": case.weight_bytes + 2 * T_pad * (K + N),
                      "alg_bytes_t1": case.weight_bytes + 2 * (K + N)}), flush=True)


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
    # where a workspace lets small N run the K-slice kernels and their fold launch, that path beside
    # the default one-launch kernel
    work += [(n, N, K, T, e, op + "_ks") for n, N, K, T, e, op in list(work)
             if w8.w8_linear_invariant_workspace_bytes(N, K, T) > 0]
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
    def label(name: str, op: str) -> str:
        return name + (" [packed]" if "packed" in op else "") + (" [K-slice + fold]" if op.endswith("_ks") else "")

    for name, N, K, T_pad, eps, op in work:
        if not want(label(name, op)):
            continue
        wbytes = N * K + 2 * N * (K // 32)
        copies = max(1, math.ceil((1 << 30) / wbytes))
        Ws = [torch.randint(-127, 128, (N, K), generator=g, dtype=torch.int8, device=dev) for _ in range(copies)]
        Ss = [(torch.randn(N, K // 32, generator=g, device=dev).abs_() * 0.02 + eps).half() for _ in range(copies)]
        X = torch.randn(T_pad, K, generator=g, device=dev).to(torch.bfloat16)
        R = torch.randn(T_pad, N, generator=g, device=dev).to(torch.bfloat16)
        Y = torch.empty((T_pad, N // 2 if op.startswith("swiglu") else N), dtype=torch.bfloat16, device=dev)
        if op.endswith("packed") or op == "packed_ks":
            Ps = [w8.w8_pack(Ws[i], Ss[i]) for i in range(copies)]
        # the width the kernels run at: T_pad 48 / 64 calls with t <= 32 run the T_pad 32 kernel
        width = lambda t: T_pad if T_pad <= 32 or t > 32 else 32  # noqa: E731
        if op == "linear":
            kernel = lambda t: w8.w8_linear_invariant_kernel(N, K, width(t), Ss[0])  # noqa: E731
            call = lambda i, t: w8.w8_linear_invariant(Ws[i], Ss[i], X[:t], t, T_pad, y=Y)  # noqa: E731
        elif op == "packed":
            kernel = lambda t: w8.w8_linear_invariant_packed_kernel(N, K, width(t))  # noqa: E731
            call = lambda i, t: w8.w8_linear_invariant_packed(Ps[i][0], Ps[i][1], X[:t], t, T_pad, N, y=Y)  # noqa
        elif op == "linear_ks":
            kernel = lambda t: f"gemm_w8g32_kslice<{width(t) // 16}, false> + kslice_fold"  # noqa: E731
            call = lambda i, t: w8.w8_linear_invariant(Ws[i], Ss[i], X[:t], t, T_pad, y=Y, workspace="auto")  # noqa
        elif op == "packed_ks":
            kernel = lambda t: f"gemm_w8g32_kslice<{width(t) // 16}, true> + kslice_fold"  # noqa: E731
            call = lambda i, t: w8.w8_linear_invariant_packed(Ps[i][0], Ps[i][1], X[:t], t, T_pad, N, y=Y,  # noqa
                                                              workspace="auto")
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
            print(json.dumps({"workload": label(name, op), "kernel": kernel(t) if callable(kernel) else kernel, "t": t, "T_pad": T_pad, "us": round(sec * 1e6, 2),
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
    # the head's logprob epilogues, cold: the logits rotate over >= 1 GiB of buffers (past the 256 MB
    # Infinity Cache), one graph replay walks all of them once
    V, block = synth.HEAD.N, synth.HEAD_BLOCK
    vocab = (f"vocab block logprob V={V} block={block}", f"vocab greedy argmax V={V}",
             f"vocab block logprob, blockwise-direct V={V}")
    for t in (1, synth.HEAD.T_pad) if any(want(n) for n in vocab) else ():
        nl = max(1, math.ceil(GIB / (t * V * 2)))
        Ls = [(torch.randn(t, V, generator=g, device=dev) * 105).to(torch.bfloat16) for _ in range(nl)]
        targets = torch.randint(0, V, (t,), generator=g, device=dev, dtype=torch.int64)
        ws = torch.empty(w8.vocab_block_logprob_workspace_bytes(t, V, block), dtype=torch.uint8, device=dev)
        out = torch.empty(t, dtype=torch.float32, device=dev)
        aws = torch.empty(max(16, w8.vocab_argmax_workspace_bytes(t, V)), dtype=torch.uint8, device=dev)
        aout = torch.empty(t, dtype=torch.int64, device=dev)
        nb = (V + block - 1) // block
        alg = 2 * (2 * t * V) + 4 * (4 * t * nb) + 12 * t
        lh = Ls[0].view(torch.int16).cpu().numpy().view(np.uint16)
        th = targets.cpu().numpy()
        for name, fn, ebytes, okind in (
                (f"vocab block logprob V={V} block={block}",
                 lambda L: w8.vocab_block_logprob(L, targets, block, out=out, workspace=ws), alg, "logprob"),
                (f"vocab greedy argmax V={V}", lambda L: w8.vocab_argmax(L, out=aout, workspace=aws),
                 2 * t * V + 8 * t, "argmax"),
                (f"vocab block logprob, blockwise-direct V={V}",
                 lambda L: w8.vocab_block_logprob_direct(L, targets, block, out=out, workspace=ws), alg, "direct")):
            if not want(name):
                continue
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(stream):
                fn(Ls[0])
                torch.cuda.synchronize()
                with torch.cuda.graph(graph, stream=stream):
                    for L in Ls:
                        fn(L)
                graph.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(10):
                    graph.replay()
                e1.record(stream)
                torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / 1e3 / (10 * nl)
            c0 = time.perf_counter()
            if okind == "argmax":
                oracle.argmax(lh)
            else:
                oracle.block_logprob(lh, th, block, direct=okind == "direct")
            csec = time.perf_counter() - c0
            print(json.dumps({"workload": name, "t": t, "us": round(sec * 1e6, 2), "cache": "cold (logits rotate "
                              f"over {nl} buffers, >= 1 GiB)", "alg_gbs": round(ebytes / sec / 1e9, 1),
                              "roofline_frac": round(ebytes / sec / 1e9 / HBM_PEAK_GBS, 4),
                              "cpu_oracle_us": round(csec * 1e6, 1)}), flush=True)
        del Ls
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
