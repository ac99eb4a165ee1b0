"""Benchmark: int8 TOPS of the fused grouped MoE GEMM + finalize-routing on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config prefill]
                    [--combine auto|atomic|ordered] [--no-cpu-baseline]

A step is one library call (seed, grouped int8 GEMM with fused dequant, combine
by rowIndex) over the whole workload, inputs resident in HBM.  The default
workload is the prefill-shaped one (m = 131072 rows from 16384 tokens x top-8,
e = 32, k = 2048, n = 7168, bf16 scale, sharedInput (8192, 7168) at offset
4096), synthetic and seeded.  Prints one JSON line.

ops per step = 2 * M_eff * k * n (multiply and add of the covered rows).
The roofline entry is the grouped GEMM kernel alone, timed with HIP events
recorded on the launch stream right around it, against the dense int8 MFMA
peak (5.0 POP/s).  The cpu_baseline entry times the CPU oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0       # MI355X dense int8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, GB/s
KERNEL_SRC = os.path.join(ROOT, "quantized_moe_grouped_amd", "csrc", "gmmfr_kernels.hip")
QP_SRC = os.path.join(ROOT, "quantized_moe_grouped_amd", "csrc", "quant_permute.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="prefill",
                    choices=["tiny", "decode", "skewed", "prefill", "int4", "mxa8w4", "fp8", "dispatch", "layer"])
    ap.add_argument("--combine", default="auto", choices=["auto", "atomic", "ordered"])
    ap.add_argument("--quant", default="int8", choices=["int8", "fp8", "mx"],
                    help="dispatch workload: x1 encoding of the producer step")
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--tile-m", type=int, default=0, choices=[0, 32, 64, 128, 256],
                    help="force the GEMM tile height (0 = the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--transpose-x2", action="store_true",
                    help="int8 or FP8 weights given transposed, (e,n,k) (the operator's transposed-x2 form)")
    ap.add_argument("--cpu-sample-rows", type=int, default=0, help="rows in the oracle sample (0 = auto)")
    ap.add_argument("--timing-detail", action="store_true",
                    help="after the timed steps, add a 'timing' object: per-call median/min/p90 with warm caches "
                         "and with 1 GiB written before each call (L2 and MALL evicted), and both combine modes")
    ap.add_argument("--zero-operands", action="store_true",
                    help="power study: x1 and x2 all zero (int8 workloads; the matrix cores then draw little "
                         "power); the line is marked, carries no CPU baseline, and is never the headline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (torch copy_) 5 times: the reference kernel whose "
                         "FETCH_SIZE / WRITE_SIZE counters scale the HBM traffic figures")
    return ap.parse_args()


class Hip:
    """The HIP runtime already loaded in this process (torch's), for events."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ev, ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b):
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


def _stats(ms):
    t = sorted(ms)
    return {"median": round(t[len(t) // 2], 5), "min": round(t[0], 5), "p90": round(t[int(0.9 * (len(t) - 1))], 5),
            "calls": len(t)}


def timing_detail(p, d, args, stream, hip, chosen, calls=20):
    """Whole-call times from events around each call: warm (back to back) and
    cold (a 1 GiB buffer written before each call, which evicts the L2s and
    the 256 MB MALL), for the combine mode the library chose and the other."""
    import torch
    from quantized_moe_grouped_amd import binding as B
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    out = {}
    for mode in ("atomic", "ordered"):
        cargs, keep = B.make_args(d["x1"], d["x2"], d["gl"], d["out"], scale=d["scale"], pertoken_scale=d["pts"],
                                  logit=d["logit"], row_index=d["ri"], shared_input=d["shared"],
                                  shared_input_offset=p.shared_input_offset, group_list_type=p.group_list_type,
                                  combine=mode, transpose_x2=p.x2_transposed)
        ws = torch.empty(max(B.workspace_size(cargs), 1), dtype=torch.uint8, device="cuda")
        for _ in range(args.warmup):
            B.run(cargs, ws, stream)
        res = {}
        for kind in ("warm", "cold"):
            evs = [(hip.event(), hip.event()) for _ in range(calls)]
            for i, (a, b) in enumerate(evs):
                if kind == "cold":
                    flush.fill_(float(i))
                hip.record(a, stream)
                B.run(cargs, ws, stream)
                hip.record(b, stream)
            torch.cuda.synchronize()
            res[kind + "_ms"] = _stats([hip.elapsed_ms(a, b) for a, b in evs])
        out[mode] = res
        del ws, keep
    out["chosen"] = chosen
    return out


def algorithmic_bytes(p):
    """Each input read once, the output written once (no atomics, no y)."""
    if getattr(p, "fp8", False):  # fp8 x1 and weights, per-channel scale (bf16 here) and per-token scale
        return (p.covered_rows * p.k + p.nonempty_experts * p.n * (p.k + 2) + p.m * (4 + 4 + 8) + p.e * 8
                + p.bsdp * p.n * 2 + p.output_bs * p.n * 4)
    if getattr(p, "mx", False):  # fp8 x1, fp4 weights, one E8M0 per 32 k of each row and column
        return (p.covered_rows * (p.k + p.k // 32) + p.nonempty_experts * p.n * (p.k // 2 + p.k // 32)
                + p.m * (4 + 8) + p.e * 8 + p.bsdp * p.n * 2 + p.output_bs * p.n * 4)
    wbytes = p.k * p.n // 2 if p.x2_int4 else p.k * p.n
    sbytes = 0 if p.scale is None else (2 if p.scale_bf16 else 4) * p.n
    return (p.covered_rows * p.k + p.nonempty_experts * (wbytes + sbytes) + p.m * (4 + 4 + p.row_index.itemsize)
            + p.e * 8 + p.bsdp * p.n * 2 + p.output_bs * p.n * 4)


def host_cpu() -> str:
    """The host CPU's model name and logical CPU count, as the kernel reports them."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"


def cpu_baseline(p, rows_wanted: int):
    """Time the oracle (whole computation) on a sample: the first rows of every
    expert group, all k and n, same destinations and output size."""
    import numpy as np
    import oracle
    from quantized_moe_grouped_amd import workloads as W

    counts = np.diff(np.concatenate([[0], np.cumsum(p.counts)]))
    frac = rows_wanted / max(p.covered_rows, 1)
    take = np.minimum(counts, np.ceil(counts * frac).astype(np.int64))
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    idx = np.concatenate([np.arange(s, s + t) for s, t in zip(starts, take)]) if take.sum() else np.zeros(0, np.int64)
    q = W.Problem(p.name + "-sample", int(idx.size), p.k, p.n, p.e, p.x1[idx], p.x2, p.x2_int4, p.scale,
                  p.scale_bf16, None if p.pertoken_scale is None else p.pertoken_scale[idx],
                  None if p.logit is None else p.logit[idx], np.cumsum(take).astype(np.int64), 0,
                  None if p.row_index is None else p.row_index[idx], p.shared_input, p.shared_input_offset,
                  p.output_bs, p.seed, take, x2_transposed=getattr(p, "x2_transposed", False),
                  fp8=getattr(p, "fp8", False), mx=getattr(p, "mx", False))
    if q.mx or q.fp8:
        from oracle import mx as omx
        t0 = time.perf_counter()
        omx.run(q)
        dt = time.perf_counter() - t0
    else:
        oracle.load()
        t0 = time.perf_counter()
        oracle.run(q, want_acc=False)
        dt = time.perf_counter() - t0
    ops = 2.0 * q.m * q.k * q.n
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle", "host": host_cpu(),
            "sample": f"{q.m} of {p.covered_rows} rows (first rows of each of the {p.e} experts), full k={p.k}, "
                      f"n={p.n}, seed + combine into outputBS={p.output_bs}; {dt:.2f} s wall",
            "seconds": dt}


def traffic_from_profiles(kernel_name: str, workload: str, prefix: str = "gmm_kernel", src: str = KERNEL_SRC):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{prefix}_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        src_hash = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") != src_hash or rec.get("kernel") != kernel_name:
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def dispatch_bytes(rp):
    """Algorithmic bytes of the producer step, each array moved once: (step,
    quantisation kernel).  The kernel reads the hidden rows and the entry -> row
    map and writes x1 and pertokenScale; the step adds the router outputs read
    and rowIndex, logit and groupList written."""
    m = rp.T * rp.K
    sbytes = m * (rp.k // 32) if getattr(rp, "mode", "int8") == "mx" else m * 4  # pertokenScale written
    kern = rp.T * rp.k * 2 + m * 4 + m * rp.k + sbytes
    step = (rp.T * rp.k * 2 + m * rp.expert_ids.itemsize + (0 if rp.topk_weights is None else m * 4)
            + m * rp.k + sbytes + (0 if rp.topk_weights is None else m * 4) + m * 8 + rp.e * 8)
    return step, kern


def bench_dispatch(args):
    """The producer step (per-token int8 quantisation of bf16 hidden states and
    the routing permute) at the prefill workload's shape; HBM-bound, reported
    in GB/s of algorithmic bytes."""
    import numpy as np
    import torch
    from quantized_moe_grouped_amd import binding as B
    from quantized_moe_grouped_amd import workloads as W

    rp = W.make_route_config("dispatch", args.seed)
    rp.mode = args.quant
    dev = "cuda"
    hidden = torch.from_numpy(rp.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(rp.expert_ids).to(dev)
    w = torch.from_numpy(rp.topk_weights).to(dev)
    m = rp.T * rp.K
    x1 = torch.empty((m, rp.k), dtype=torch.int8 if rp.mode == "int8" else torch.float8_e4m3fn, device=dev)
    if rp.mode == "mx":
        pts = torch.empty((m, rp.k // 64, 2), dtype=torch.float8_e8m0fnu, device=dev)
    else:
        pts = torch.empty(m, dtype=torch.float32, device=dev)
    logit = torch.empty(m, dtype=torch.float32, device=dev)
    ri = torch.empty(m, dtype=torch.int64, device=dev)
    gl = torch.empty(rp.e, dtype=torch.int64, device=dev)
    cargs, keep = B.make_qp_args(hidden, ids, x1, pts, ri, gl, topk_weights=w, logit=logit,
                                 group_list_type=rp.group_list_type)
    ws = torch.empty(max(B.qp_workspace_size(cargs), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()
    ev_all = (hip.event(), hip.event())
    ev_q = [(hip.event(), hip.event()) for _ in range(args.steps)]

    def call(evs=(None, None)):
        st = B.lib().gmm_quant_permute_profiled(ctypes.byref(cargs), ctypes.c_void_p(ws.data_ptr()),
                                                ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream), evs[0], evs[1])
        if st != 0:
            raise B.GmmfrError(st, "gmm_quant_permute_profiled")

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    hip.record(ev_all[0], stream)
    for s in range(args.steps):
        call(ev_q[s])
    hip.record(ev_all[1], stream)
    torch.cuda.synchronize()
    ms_step = hip.elapsed_ms(*ev_all) / args.steps
    q_ms = [hip.elapsed_ms(a, b) for a, b in ev_q]
    q_avg = sum(q_ms) / len(q_ms)
    step_bytes, kern_bytes = dispatch_bytes(rp)
    print(f"[bench] step {ms_step:.4f} ms, quant kernel {q_avg:.4f} ms", file=sys.stderr, flush=True)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    kgbs = kern_bytes / (q_avg * 1e-3) / 1e9
    res = {
        "metric": "GB/s (and % of HBM roofline) of per-token int8 quantisation + routing permute at 1 GPU",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"int8": "bf16->int8", "fp8": "bf16->fp8", "mx": "bf16->fp8+e8m0"}[rp.mode],
        "data": "synthetic (seeded generator; bf16 hidden states, top-8 of 32 router choices with softmax weights)",
        "config": {"workload": "dispatch" if rp.mode == "int8" else "dispatch-" + rp.mode, "tokens": rp.T,
                   "k": rp.k, "top_k": rp.K, "e": rp.e, "m": m, "quant": rp.mode,
                   "ids": str(rp.expert_ids.dtype), "group_list_type": rp.group_list_type, "seed": args.seed,
                   "algorithmic_bytes_per_step": step_bytes,
                   "path_roofline_frac": round(gbs / PEAK_HBM_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": "quant_rows_kernel", "achieved": round(kgbs, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(kgbs / PEAK_HBM_GBS, 4),
                     "launch_ms": round(q_avg, 5), "bytes_per_launch": kern_bytes,
                     "traffic": traffic_from_profiles("quant_rows_kernel", "dispatch", "quant_rows_kernel", QP_SRC)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle import quant as Q
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 10.0:
            Q.run(rp)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        res["cpu_baseline"] = {"value": round(step_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "host": host_cpu(),
                               "sample": f"the whole workload ({rp.T} tokens), {reps} runs, {dt:.2f} s each"}
    print(json.dumps(res), flush=True)
    del keep


def bench_layer(args):
    """Both entry points in sequence at the prefill shape: bf16 hidden states of
    16384 tokens and their top-8 of 32 router choices -> quantise and permute
    -> grouped int8 GEMM with dequant and the combine by token.  int8 TOPS of
    the whole layer (the GEMM's 2*m*k*n over the time of both calls)."""
    import numpy as np
    import torch
    from quantized_moe_grouped_amd import binding as B
    from quantized_moe_grouped_amd import workloads as W

    rp = W.make_route_config("dispatch", args.seed)
    pw = W.make_config("prefill", args.seed)  # weights, scales and sharedInput of the prefill workload
    dev = "cuda"
    m, n = rp.T * rp.K, pw.n
    hidden = torch.from_numpy(rp.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
    ids = torch.from_numpy(rp.expert_ids).to(dev)
    w = torch.from_numpy(rp.topk_weights).to(dev)
    x1 = torch.empty((m, rp.k), dtype=torch.int8, device=dev)
    pts = torch.empty(m, dtype=torch.float32, device=dev)
    logit = torch.empty(m, dtype=torch.float32, device=dev)
    ri = torch.empty(m, dtype=torch.int64, device=dev)
    gl = torch.empty(rp.e, dtype=torch.int64, device=dev)
    qargs, qkeep = B.make_qp_args(hidden, ids, x1, pts, ri, gl, topk_weights=w, logit=logit, group_list_type=1)
    qws = torch.empty(max(B.qp_workspace_size(qargs), 1), dtype=torch.uint8, device=dev)
    x2 = torch.from_numpy(pw.x2).to(dev)
    scale = torch.from_numpy(np.ascontiguousarray(pw.scale).view(np.int16)).to(dev).view(torch.bfloat16)
    shared = torch.from_numpy(np.ascontiguousarray(pw.shared_input).view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((rp.T, n), dtype=torch.float32, device=dev)
    gargs, gkeep = B.make_args(x1, x2, gl, out, scale=scale, pertoken_scale=pts, logit=logit, row_index=ri,
                               shared_input=shared, shared_input_offset=pw.shared_input_offset, group_list_type=1,
                               deterministic=args.deterministic, combine=args.combine,
                               tuning_config=[m // rp.e])  # expected rows per expert (the tiling hint)
    plan = B.plan(gargs)
    gws = torch.empty(max(B.workspace_size(gargs), 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()
    ev = (hip.event(), hip.event())

    def step():
        st = B.lib().gmm_quant_permute(ctypes.byref(qargs), ctypes.c_void_p(qws.data_ptr()),
                                       ctypes.c_size_t(qws.numel()), ctypes.c_void_p(stream))
        if st != 0:
            raise B.GmmfrError(st, "gmm_quant_permute")
        B.run(gargs, gws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hip.record(ev[0], stream)
    for _ in range(args.steps):
        step()
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(*ev) / args.steps
    ops = 2.0 * m * rp.k * n
    res = {
        "metric": "int8 TOPS of a whole MoE expert layer (quantise + permute + GMM + finalize-routing) at 1 GPU",
        "value": round(ops / (ms * 1e-3) / 1e12, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8",
        "data": "synthetic (seeded bf16 hidden states and top-8 router choices; the prefill workload's weights)",
        "config": {"workload": "layer", "tokens": rp.T, "top_k": rp.K, "m": m, "e": rp.e, "k": rp.k, "n": n,
                   "combine": plan["combine"], "gemm_kernel": plan["gemm_kernel"], "seed": args.seed,
                   "ops_per_step": ops},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)
    del qkeep, gkeep


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path runs on one GPU's share: expert-parallel ranks would each run it on their local "
              "experts' rows between two all-to-all exchanges).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from quantized_moe_grouped_amd import binding as B
    from quantized_moe_grouped_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / 5
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30,
                          "copy_GBps_read_plus_write": round(2 * (1 << 30) / dt / 1e9, 1)}), flush=True)
        return
    if args.config == "dispatch":
        bench_dispatch(args)
        return
    if args.config == "layer":
        bench_layer(args)
        return
    print(f"[bench] generating {args.config} seed {args.seed}", file=sys.stderr, flush=True)
    if args.config == "mxa8w4":
        p = W.make_mx_config(args.config, args.seed)
    elif args.config == "fp8":
        p = W.make_fp8_config(args.config, args.seed)
    else:
        p = W.make_config(args.config, args.seed)
    if args.transpose_x2:
        p = W.with_transposed_weights(p)
    dev = "cuda"

    def T(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def bf16(a):
        return None if a is None else T(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)

    if p.mx:
        x1, x2 = T(p.x1).view(torch.float8_e4m3fn), T(p.x2).view(torch.float4_e2m1fn_x2)
        scale, pts = T(p.scale).view(torch.float8_e8m0fnu), T(p.pertoken_scale).view(torch.float8_e8m0fnu)
    elif p.fp8:
        x1, x2 = T(p.x1).view(torch.float8_e4m3fn), T(p.x2).view(torch.float8_e4m3fn)
        scale = None if p.scale is None else (bf16(p.scale) if p.scale_bf16 else T(p.scale))
        pts = T(p.pertoken_scale)
    else:
        x1, x2 = T(p.x1), T(p.x2)
        scale = None if p.scale is None else (bf16(p.scale) if p.scale_bf16 else T(p.scale))
        pts = T(p.pertoken_scale)
    if args.zero_operands:
        if p.mx or p.fp8:
            print("--zero-operands applies to the int8 workloads", file=sys.stderr)
            sys.exit(2)
        x1.zero_()
        x2.zero_()
        args.no_cpu_baseline = True
    logit, gl, ri = T(p.logit), T(p.group_list), T(p.row_index)
    shared = bf16(p.shared_input)
    out = torch.empty((p.output_bs, p.n), dtype=torch.float32, device=dev)
    cargs, keep = B.make_args(x1, x2, gl, out, scale=scale, pertoken_scale=pts, logit=logit, row_index=ri,
                              shared_input=shared, shared_input_offset=p.shared_input_offset,
                              group_list_type=p.group_list_type, deterministic=args.deterministic,
                              combine=args.combine, tuning_config=[0, args.tile_m] if args.tile_m else None,
                              transpose_x2=p.x2_transposed)
    plan = B.plan(cargs)
    ws_bytes = B.workspace_size(cargs)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    hip = Hip()
    ev_all = (hip.event(), hip.event())
    ev_g = [(hip.event(), hip.event()) for _ in range(args.steps)]
    print(f"[bench] plan {plan}", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        B.run(cargs, ws, stream)
    torch.cuda.synchronize()
    hip.record(ev_all[0], stream)
    for s in range(args.steps):
        st = B.lib().gmm_finalize_routing_profiled(ctypes.byref(cargs), ctypes.c_void_p(ws.data_ptr()),
                                                    ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream),
                                                    ev_g[s][0], ev_g[s][1])
        if st != 0:
            raise B.GmmfrError(st, "gmm_finalize_routing_profiled")
    hip.record(ev_all[1], stream)
    torch.cuda.synchronize()
    total_ms = hip.elapsed_ms(ev_all[0], ev_all[1])
    gemm_ms = [hip.elapsed_ms(a, b) for a, b in ev_g]
    ms_step = total_ms / args.steps
    gemm_avg = sum(gemm_ms) / len(gemm_ms)
    print(f"[bench] step {ms_step:.4f} ms, gemm kernel {gemm_avg:.4f} ms "
          f"(min {min(gemm_ms):.4f}, max {max(gemm_ms):.4f})", file=sys.stderr, flush=True)

    # the same calls with cold caches: before each, 1 GiB is written (the L2s
    # and the 256 MB MALL evicted); events around the call alone
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    ev_c = [(hip.event(), hip.event(), hip.event(), hip.event()) for _ in range(args.steps)]
    for s, (a, g0, g1, b) in enumerate(ev_c):
        flush.fill_(float(s))
        hip.record(a, stream)
        st = B.lib().gmm_finalize_routing_profiled(ctypes.byref(cargs), ctypes.c_void_p(ws.data_ptr()),
                                                    ctypes.c_size_t(ws.numel()), ctypes.c_void_p(stream), g0, g1)
        if st != 0:
            raise B.GmmfrError(st, "gmm_finalize_routing_profiled")
        hip.record(b, stream)
    torch.cuda.synchronize()
    cold_step = sorted(hip.elapsed_ms(a, b) for a, _, _, b in ev_c)
    cold_gemm = sorted(hip.elapsed_ms(g0, g1) for _, g0, g1, _ in ev_c)
    del flush
    cold = {"ms_per_step_median": round(cold_step[len(cold_step) // 2], 5),
            "gemm_ms_median": round(cold_gemm[len(cold_gemm) // 2], 5), "calls": args.steps,
            "flush": "1 GiB written before each call (L2s and MALL evicted); events around the call only"}
    print(f"[bench] cold: step {cold['ms_per_step_median']:.4f} ms, gemm kernel {cold['gemm_ms_median']:.4f} ms "
          f"(medians)", file=sys.stderr, flush=True)

    ops = 2.0 * p.covered_rows * p.k * p.n
    tops = ops / (ms_step * 1e-3) / 1e12
    gemm_tops = ops / (gemm_avg * 1e-3) / 1e12
    abytes = algorithmic_bytes(p)
    t_roof_ms = max(ops / (PEAK_INT8_TOPS * 1e12), abytes / (PEAK_HBM_GBS * 1e9)) * 1e3
    kname = plan["gemm_kernel"]
    # the GEMM kernel against whichever roof bounds the workload: the dense
    # MFMA peak (int8 5.0 POP/s; FP8, and FP8 x FP4 which issues at the FP8
    # rate, 5.0 PFLOP/s) or HBM (8 TB/s) when its bytes take longer
    floating = p.mx or p.fp8
    if abytes / (PEAK_HBM_GBS * 1e9) > ops / (PEAK_INT8_TOPS * 1e12):
        gbs = abytes / (gemm_avg * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "launch_ms": round(gemm_avg, 5),
                    "traffic": traffic_from_profiles(kname, p.name)}
    else:
        roofline = {"bound": "mfma", "kernel": kname, "achieved": round(gemm_tops, 2), "peak": PEAK_INT8_TOPS,
                    "unit": "TFLOP/s" if floating else "TOP/s", "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
                    "launch_ms": round(gemm_avg, 5), "traffic": traffic_from_profiles(kname, p.name)}
    res = {
        "metric": ("FP8 TFLOPS" if floating else "int8 TOPS") + " (and % of MFMA/HBM roofline) for GMM+finalize-routing at 1 GPU",
        "value": round(tops, 2),
        "unit": "TFLOPS" if floating else "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4" if p.mx else ("fp8" if p.fp8 else "int8"),
        "data": ("synthetic, x1 and x2 all zero (power study, not the workload's data); routing and scales seeded"
                 if args.zero_operands else
                 "synthetic (seeded generator; random int8 weights/activations, routing and scales of the stated shapes)"),
        "config": {"workload": p.name, "tokens": p.output_bs, "top_k": p.m // max(p.output_bs, 1), "m": p.m,
                   "e": p.e, "k": p.k, "n": p.n,
                   "weights": "fp4 e2m1, e8m0 per 32 k" if p.mx else
                   ("fp8 e4m3" if p.fp8 else ("int4" if p.x2_int4 else "int8")),
                   "weights_layout": "(e,n,k)" if p.x2_transposed else "(e,k,n)",
                   "output_bs": p.output_bs, "shared_rows": p.bsdp, "combine": plan["combine"],
                   "deterministic": bool(args.deterministic), "seed": args.seed,
                   "ops_per_step": ops, "algorithmic_bytes_per_step": abytes,
                   "path_roofline_frac": round(t_roof_ms / ms_step, 4)},
        "roofline": roofline,
        "cpu_baseline": None,
        "cold": cold,
    }
    if args.timing_detail:
        res["timing"] = timing_detail(p, dict(x1=x1, x2=x2, gl=gl, out=out, scale=scale, pts=pts, logit=logit, ri=ri,
                                              shared=shared), args, stream, hip, plan["combine"])
    if not args.no_cpu_baseline:
        rows = args.cpu_sample_rows
        if not rows:
            # size the sample for about 20 s of oracle time from a short calibration run
            cal = cpu_baseline(p, min(p.covered_rows, 256))
            rate_rows = min(p.covered_rows, 256) / max(cal["seconds"], 1e-3)
            rows = int(max(256, min(p.covered_rows, 20.0 * rate_rows)))
        print(f"[bench] cpu oracle on a {rows}-row sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(p, rows)
        cb.pop("seconds")
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)
    del keep


if __name__ == "__main__":
    main()
