#!/usr/bin/env python3
"""Benchmark of the OPQ W4A16 hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input.  By
default the workload is the DiT FFN pair, the largest configuration that runs
all three kernels on one GPU:

    up/gate: opq_quantize(W 20480x3840 bf16) -> opq_dequantize -> opq_linear(x [4096, 3840])
    down:    opq_quantize(W 3840x10240 bf16) -> opq_dequantize -> opq_linear(x [4096, 10240])

(weights N(0, 0.02^2) with 1% Laplace(0, 0.02) tails, alpha 0.73).
--workload skinny|qkv|tiny|ffn_up|ffn_down selects one of the other shapes.

Prints ONE JSON line.  `value` is the step's fraction of the MI355X roofline
in percent: the sum of each kernel's ideal time (algorithmic bytes / 8 TB/s,
or flops / 2.5 PFLOP/s for the MFMA-bound linear) over the measured step time.
The timed region is exactly --steps steps between two HIP events.  Per-kernel
durations (under "kernels", with absolute GB/s and TFLOP/s) come from a second
pass: 7 batches of --steps back-to-back launches of one kernel on the same
stream, median batch; the "roofline" object is the slowest kernel's (the
up/gate linear layer by default).  Inputs are resident in HBM before timing
starts; every launch rotates to another set of input/output buffers so that
the 256 MB Infinity Cache cannot serve repeats.  The default run also times
the whole-model quantize/dequantize pass ("model_pass") and the CPU oracle on
the same workload ("cpu_baseline").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "opq_linear TFLOP/s + quantize/dequant GB/s, as % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
SKINNY_MAX_M = 64              # opq_linear switches to the tiled MFMA kernel above this
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "w4a16_linear_amd", "csrc")
KERNEL_SOURCE = {"quantize": "quantize.hip", "dequantize": "dequantize.hip",
                 "linear": "linear.hip"}
WORKLOADS = ["ffn", "skinny", "qkv", "ffn_up", "ffn_down", "tiny", "model"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ffn", choices=WORKLOADS)
    ap.add_argument("--alpha", type=float, default=0.73)
    ap.add_argument("--group", type=int, default=0, choices=[0, 32, 64, 128, 256],
                    help="0: one float32 max per row; else the group-wise form (float16 max "
                         "per this many weights along k)")
    ap.add_argument("--bits", type=int, default=4, choices=[3, 4, 5, 6],
                    help="code width; other than 4 the linear layer decodes into a workspace "
                         "and multiplies the bfloat16 weights")
    ap.add_argument("--rotate", type=int, default=0, help="buffer sets (0: enough for > 768 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-model-pass", action="store_true",
                    help="leave out the whole-model quantize/dequantize pass")
    ap.add_argument("--no-copy", action="store_true", help="leave out the same-bytes copies")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, 5 plain device copies of this many MiB (counter scaling)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each timed step (and each per-kernel batch) as a HIP graph")
    return ap.parse_args()


# ------------------------------------------------------------------ workload

def workload_layers(name):
    """[(tag, Layer)]: the layers one step runs, tagged as the counter
    summaries in profiles/ are named."""
    from w4a16_linear_amd import workloads as WL
    if name == "ffn":
        up, down = WL.config("ffn").layers
        return [("ffn_up", up), ("ffn_down", down)]
    if name == "ffn_up":
        return [("ffn_up", WL.config("ffn").layers[0])]
    if name == "ffn_down":
        return [("ffn_down", WL.config("ffn").layers[1])]
    return [(name, WL.config(name).layers[0])]


def workload_title(name):
    from w4a16_linear_amd import workloads as WL
    return {"ffn": WL.config("ffn").title, "skinny": WL.config("skinny").title,
            "qkv": WL.config("qkv").title, "tiny": WL.config("tiny").title,
            "ffn_up": "FFN up/gate: x bf16 [4096, 3840] x W 20480x3840",
            "ffn_down": "FFN down: x bf16 [4096, 10240] x W 3840x10240"}[name]


def algorithmic(m, n, k, w_bytes, group=0, bits=4):
    """Per-launch algorithmic bytes / flops (what the method must move).  The
    scales are 4 B per row, or 2 B per group of `group` weights; codes take
    bits/8 B and signs 1/8 B per weight."""
    sc = 2 * n * (k // group) if group else 4 * n
    st = (bits + 1) / 8.0
    # "read": the bytes a launch reads, which is what a cache could serve on a
    # repeat (the kernels' outputs are nontemporal stores and do not fill it)
    quant = {"bytes": n * k * (w_bytes + st) + sc, "flops": 0, "read": n * k * w_bytes}
    dequant = {"bytes": n * k * (st + 2) + sc, "flops": 0, "read": n * k * st + sc}
    lin = {"bytes": st * n * k + sc + 2 * m * k + 4 * m * n, "flops": 2 * m * n * k,
           "read": st * n * k + sc + 2 * m * k}
    return {"quantize": quant, "dequantize": dequant, "linear": lin}


def ideal_us(kind, alg, m):
    if kind == "linear" and m > SKINNY_MAX_M:
        return alg["flops"] / (BF16_PEAK_TFLOPS * 1e12) * 1e6, "mfma"
    return alg["bytes"] / (HBM_PEAK_GBS * 1e9) * 1e6, "hbm"


def source_hash(kind):
    """Hash of the kernel's source file and every shared device header."""
    h = hashlib.sha256()
    headers = sorted(f for f in os.listdir(CSRC) if f.endswith(".hpp"))
    for f in [KERNEL_SOURCE[kind]] + headers:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kind, tag):
    """HBM bytes per launch from the committed counter summary
    profiles/<kernel>_<tag>_traffic.txt, or None when there is none or the
    kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"{kind}_{tag}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, v = line.split(":", 1)
            vals[key.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash(kind):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ streaming ceiling

def ceiling_lib():
    """libopq_ceiling.so: plain row streaming of given bytes (built with libopq)."""
    import ctypes
    from w4a16_linear_amd import build as B
    if not os.path.exists(B.CEILING_LIB):
        raise RuntimeError(f"{B.CEILING_LIB} not built: run `python -m w4a16_linear_amd.build`")
    lib = ctypes.CDLL(B.CEILING_LIB)
    lib.opq_ceiling_stream_rows.restype = ctypes.c_int
    lib.opq_ceiling_stream_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
    return lib


def row_bytes(kind, k, w_bytes, group=0, bits=4):
    """(read, written) bytes per weight row of quantize or dequantize, each
    rounded up to 16: the weights, the codes and signs, the row's scales."""
    sc = 2 * (k // group) if group else 4
    st = k * (bits + 1) // 8 + sc
    up = lambda b: (b + 15) // 16 * 16
    return (up(k * w_bytes), up(st)) if kind == "quantize" else (up(st), up(2 * k))


def stream_ceiling_us(dev, stream, rows, rd, wr, reps, graph=False):
    """Microseconds per call of the streaming kernel over rows x (rd read, wr
    written) bytes, rotating over enough buffer pairs that more than 800 MB
    is read before a pair comes back (its stores are nontemporal and leave the
    cache to the reads).  graph: each batch recorded as a graph and replayed,
    as the kernels it is compared with."""
    import numpy as np
    import torch
    lib = ceiling_lib()
    per = rows * max(rd, 16)
    pairs = max(2, int(np.ceil(800e6 / per)))
    bufs = [(torch.zeros(max(rows * rd, 16), dtype=torch.uint8, device=dev),
             torch.zeros(max(rows * wr, 16), dtype=torch.uint8, device=dev)) for _ in range(pairs)]
    def call(i):
        a, b = bufs[i % pairs]
        h = torch.cuda.current_stream(dev).cuda_stream  # the capture stream inside a graph
        if lib.opq_ceiling_stream_rows(a.data_ptr(), b.data_ptr(), rows, rd, wr, h) != 0:
            raise RuntimeError("opq_ceiling_stream_rows failed")
    for i in range(3):
        call(i)
    res = []
    for b in range(7):
        g = None
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(reps):
                    call(b * reps + i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if g is not None:
            g.replay()
        else:
            for i in range(reps):
                call(b * reps + i)
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / reps * 1e3)
        del g
    del bufs
    return float(np.median(res))


# ------------------------------------------------------------------ host description

def host_description():
    """CPU model, thread count, numpy and BLAS of the host the oracle runs on."""
    import numpy as np
    from threadpoolctl import threadpool_info
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [{"api": d.get("internal_api"), "version": d.get("version"),
             "threads": d.get("num_threads")}
            for d in threadpool_info() if d.get("user_api") == "blas"]
    return {"cpu_model": model, "nproc": os.cpu_count(), "numpy": np.__version__,
            "blas": blas}


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(layers, alpha, ideal_total_us, group=0, threads=1, x_rows=512):
    """The oracle, as it stands, on the same workload.  Per layer: quantize and
    dequantize of the whole weight, and the linear layer on a seeded subset of
    `x_rows` activation rows (all rows when there are fewer), scaled to the
    full row count.  threads = 1: one thread, BLAS limited to one; threads >
    1: the weight's rows split into that many blocks run by a thread pool
    (NumPy releases the GIL), each block's BLAS limited to one thread."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O
    from w4a16_linear_amd import workloads as WL

    t_step = 0.0
    parts = []
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=threads) as pool:
        for tag, L in layers:
            w32 = L.make_w()
            if L.w_dtype == "bf16":
                w_vals = O.bf16_bits_to_f32(WL.bf16_bits(WL.to_bf16(w32)))
            else:
                w_vals = np.ascontiguousarray(w32, np.float32)
            del w32
            rows_x = np.sort(np.random.default_rng(L.m + L.k).choice(L.m, min(x_rows, L.m),
                                                                     replace=False))
            xb = WL.bf16_bits(WL.to_bf16(L.make_x()))[rows_x]

            def block(rows):
                w = w_vals[rows]
                t0 = time.perf_counter()
                if group:
                    p, s, m = O.quantize_grouped(w, alpha, group)
                    d = O.dequantize_grouped(p, s, m, alpha, group)
                else:
                    p, s, m = O.quantize(w, alpha)
                    d = O.dequantize(p, s, m, alpha)
                t1 = time.perf_counter()
                O.linear(xb, d)
                return t1 - t0, time.perf_counter() - t1

            blocks = [sl for sl in np.array_split(np.arange(L.n), threads) if len(sl)]
            t0 = time.perf_counter()
            res = list(pool.map(block, blocks))
            wall = time.perf_counter() - t0
            # wall time of the pool, split between the two phases in the
            # proportion the blocks measured, the linear part scaled to every x row
            qd = sum(r[0] for r in res)
            lin = sum(r[1] for r in res)
            frac_lin = lin / (qd + lin) if qd + lin > 0 else 0.0
            scale_x = L.m / len(rows_x)
            t_layer = wall * (1.0 - frac_lin) + wall * frac_lin * scale_x
            t_step += t_layer
            parts.append(f"{tag}: quantize+dequantize of all {L.n}x{L.k} weights, linear on "
                         f"{len(rows_x)} of {L.m} x rows (x{scale_x:g}), {wall:.1f} s measured")
    how = "one thread" if threads == 1 else f"{threads} threads over row blocks"
    return {
        "value": round(100.0 * ideal_total_us * 1e-6 / t_step, 6),
        "unit": "% of MI355X roofline",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{how}; " + "; ".join(parts) + f"; {t_step:.1f} s per step",
        "ms_per_step": round(t_step * 1e3, 1),
        "host": host_description(),
    }


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the OPQ hot path here has no multi-GPU "
              "path (its rows would shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from w4a16_linear_amd import opq
    from w4a16_linear_amd import workloads as WL

    opq.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "model":
        out = model_pass(args, dev)
        out.update({"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                    "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                    "dtype": "bf16", "cpu_baseline": None, "env": run_env(dev)})
        print(json.dumps(out), flush=True)
        return

    alpha = args.alpha
    group, bits = args.group, args.bits
    if group and bits != 4:
        print("--group and --bits other than 4 do not combine", file=sys.stderr)
        sys.exit(2)
    layers = workload_layers(args.workload)
    kinds = ["quantize", "dequantize", "linear"]
    stream = torch.cuda.current_stream(dev)

    # Per layer: host tensors once, then `rot` device sets of every buffer.
    plan = []
    for tag, L in layers:
        m, n, k = L.m, L.n, L.k
        if group and k % group:
            print(f"--group {group} does not divide k={k}", file=sys.stderr)
            sys.exit(2)
        w32 = L.make_w()
        if L.w_dtype == "bf16":
            w_host, w_bytes = WL.to_bf16(w32), 2
        else:
            w_host, w_bytes = torch.from_numpy(w32), 4
        del w32
        x_host = WL.to_bf16(L.make_x())
        alg = algorithmic(m, n, k, w_bytes, group, bits)
        # enough sets that every kernel reads more than 800 MB (three times the
        # 256 MB Infinity Cache) before it sees a set again: counted in bytes
        # read, since the nontemporal outputs do not evict the inputs
        least = min(alg["quantize"]["read"], alg["dequantize"]["read"],
                    alg["linear"]["read"])
        rot = args.rotate or max(2, int(np.ceil(800e6 / least)))
        # outputs are allocated zero-filled, so that a fill kernel and not a
        # measured kernel meets each freshly allocated buffer first
        sets = []
        for _ in range(rot):
            w = w_host.to(dev)
            if bits != 4:
                qw = opq.BitsWeight(torch.zeros((n, k * bits // 32), dtype=torch.int32, device=dev),
                                    torch.zeros((n, k // 32), dtype=torch.int32, device=dev),
                                    torch.zeros((n,), dtype=torch.float32, device=dev), bits)
            elif group:
                qw = opq.GroupedWeight(torch.zeros((n, k // 8), dtype=torch.int32, device=dev),
                                       torch.zeros((n, k // 32), dtype=torch.int32, device=dev),
                                       torch.zeros((n, k // group), dtype=torch.float16,
                                                   device=dev), group)
            else:
                qw = opq.QuantizedWeight(torch.zeros((n, k // 8), dtype=torch.int32, device=dev),
                                         torch.zeros((n, k // 32), dtype=torch.int32, device=dev),
                                         torch.zeros((n,), dtype=torch.float32, device=dev))
            d = torch.zeros((n, k), dtype=torch.bfloat16, device=dev)
            x = x_host.to(dev)
            y = torch.zeros((m, n), dtype=torch.float32, device=dev)
            sets.append((w, qw, d, x, y))
        plan.append({"tag": tag, "L": L, "alg": alg, "rot": rot, "sets": sets,
                     "w_bytes": w_bytes})
    torch.cuda.synchronize()

    def launch(p, kind, i):
        w, qw, d, x, y = p["sets"][i % p["rot"]]
        if kind == "quantize":
            if bits != 4:
                opq.quantize_bits(w, alpha, bits, out=qw)
            elif group:
                opq.quantize_grouped(w, alpha, group, out=qw)
            else:
                opq.quantize(w, alpha, out=qw)
        elif kind == "dequantize":
            opq.dequantize(qw, alpha, out=d)
        else:
            opq.linear(x, qw, alpha, out=y)

    def step(i):
        for p in plan:
            for kind in kinds:
                launch(p, kind, i)

    # Every buffer set once through each kernel before the warmup steps: the
    # first pass over freshly allocated buffers runs several times slower than
    # the passes after it (4.9 against 0.94 ms per FFN step), which is not the
    # kernels' own work, and the warmup steps alone reach only the first sets.
    for p in plan:
        for s in range(p["rot"]):
            for kind in kinds:
                launch(p, kind, s)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def capture(fn):
        """fn() recorded as a HIP graph (the library enqueues kernels only)."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        return g

    # --graph: each timed step recorded once, before the timed region, as a
    # graph of its kernels on its own buffer set; the timed region replays them.
    graphs = None
    if args.graph:
        graphs = [capture(lambda i=i: step(args.warmup + i)) for i in range(args.steps)]
        torch.cuda.synchronize()

    # Timed region: exactly K steps, events only at its two ends.
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if graphs:
            graphs[i].replay()
        else:
            step(args.warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / args.steps
    del graphs

    def timed(fn, reps):
        """Median over 7 batches of `reps` back-to-back calls, microseconds per call
        (--graph: each batch recorded as one graph and replayed)."""
        per = []
        for b in range(7):
            g = capture(lambda b=b: [fn(b * reps + i) for i in range(reps)]) if args.graph else None
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if g is not None:
                g.replay()
            else:
                for i in range(reps):
                    fn(b * reps + i)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) / reps * 1e3)
            del g
        return float(np.median(per))

    # Per-kernel duration: batches of K back-to-back launches of one kernel
    # (same rotation of buffers), median over 7 batches.
    kern = {}
    ideal_total = 0.0
    single = len(plan) == 1
    for p in plan:
        L = p["L"]
        for kind in kinds:
            us = timed(lambda i, p=p, kind=kind: launch(p, kind, i), args.steps)
            ideal, bound = ideal_us(kind, p["alg"][kind], L.m)
            ideal_total += ideal
            a = p["alg"][kind]
            rec = {"us": round(us, 3), "bound": bound, "ideal_us": round(ideal, 3),
                   "frac": round(ideal / us, 4),
                   "GBps": round(a["bytes"] / (us * 1e-6) / 1e9, 1),
                   "algorithmic_bytes": int(a["bytes"]), "shape": [L.m, L.n, L.k]}
            if a["flops"]:
                rec["TFLOPs"] = round(a["flops"] / (us * 1e-6) / 1e12, 2)
                rec["algorithmic_flops"] = int(a["flops"])
            rec["tag"] = p["tag"]
            kern[kind if single else f"{p['tag']}.{kind}"] = rec

    # The practical ceiling at each HBM-bound kernel's size: a plain device copy
    # that reads and writes the kernel's algorithmic bytes, over enough buffer
    # pairs to defeat the 256 MB cache, timed the same way.  Left out of counter
    # runs (--copy-mib), whose only copies calibrate the byte counters.
    if not (args.copy_mib or args.no_copy):
        for name, rec in kern.items():
            if rec["bound"] != "hbm":
                continue
            half = rec["algorithmic_bytes"] // 2
            pairs = max(2, int(np.ceil(800e6 / half)))  # > 800 MB read between repeats
            bufs = [(torch.zeros(half, dtype=torch.uint8, device=dev),
                     torch.zeros(half, dtype=torch.uint8, device=dev)) for _ in range(pairs)]

            def cp(i):
                dst, src = bufs[i % pairs]
                dst.copy_(src)
            rec["same_bytes_copy_us"] = round(timed(cp, args.steps), 3)
            del bufs
        torch.cuda.synchronize()

        # The repo's own streaming kernel on the same rows and bytes: what a
        # quantizer or dequantizer without arithmetic would take.
        for name, rec in kern.items():
            kind = name.split(".")[-1]
            if kind not in ("quantize", "dequantize"):
                continue
            p = next(q for q in plan if q["tag"] == rec["tag"])
            rd, wr = row_bytes(kind, p["L"].k, p["w_bytes"], group, bits)
            c = stream_ceiling_us(dev, stream, p["L"].n, rd, wr, args.steps, args.graph)
            rec["stream_ceiling_us"] = round(c, 3)
            rec["frac_of_stream_ceiling"] = round(c / rec["us"], 4)
        torch.cuda.synchronize()

    if args.copy_mib:
        # A plain device copy of known size, for scaling the HBM byte counters.
        src = torch.zeros(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.zeros_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    dom = max(kern, key=lambda kk: kern[kk]["us"])
    dk = kern[dom]
    if dk["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": dk["TFLOPs"], "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dk["TFLOPs"] / BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": dk["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dk["GBps"] / HBM_PEAK_GBS, 4)}
    kind_dom = dom.split(".")[-1]
    roof["kernel"] = f"{dk['tag']}.{kind_dom}"
    suffix = f"_g{group}" if group else (f"_b{bits}" if bits != 4 else "")
    roof["traffic"] = measured_traffic(kind_dom, dk["tag"] + suffix)
    roof["per_launch"] = ({"flops": dk.get("algorithmic_flops"), "us": dk["us"]}
                          if dk["bound"] == "mfma" else
                          {"bytes": dk["algorithmic_bytes"], "us": dk["us"]})

    value = 100.0 * (ideal_total * 1e-3) / ms_step
    shapes = {p["tag"]: {"m": p["L"].m, "n": p["L"].n, "k": p["L"].k, "w_dtype": p["L"].w_dtype,
                         "rotating_sets": p["rot"]} for p in plan}
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "% of MI355X roofline",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {workload_title(args.workload)}",
                   "layers": shapes, "alpha": alpha,
                   "scales": (f"float16 per group of {group}" if group else "float32 per row"),
                   "bits": bits,
                   "step": "per layer: quantize -> dequantize -> linear",
                   "launch": "one HIP graph per step" if args.graph else "stream launches"},
        "roofline": roof,
        "kernels": kern,
        "kernels_sum_us": round(sum(kk["us"] for kk in kern.values()), 3),
        "wall_s": round(wall, 3),
        "env": run_env(dev),
    }
    default_run = not (args.no_cpu_baseline or args.copy_mib)
    if default_run:
        # with the CPU baseline (the default run; profiled runs skip both)
        out["env"]["gfx_clock_under_load"] = gfx_clock_under_load(step)
    del plan
    torch.cuda.empty_cache()
    if not (args.no_model_pass or args.copy_mib) and group == 0 and bits == 4:
        out["model_pass"] = model_pass(args, dev)
        torch.cuda.empty_cache()
    if default_run and bits == 4:
        out["cpu_baseline"] = cpu_baseline(layers, alpha, ideal_total, group)
        threads = min(os.cpu_count() or 1, 16)
        if threads > 1:
            out["cpu_baseline_pool"] = cpu_baseline(layers, alpha, ideal_total, group, threads)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


# ------------------------------------------------------------------ whole-model pass

def model_pass(args, dev):
    """One pass = quantize + dequantize of every layer of 30 synthetic DiT
    blocks (QKV 11520x3840, O 3840x3840, FFN 20480x3840 and 3840x10240): 5.308 B
    bf16 weights, drawn on the device per layer seed.  Also SNR(alpha) - SNR(1)
    over the whole model, an alpha sweep of the error sums, and SNR by code
    width.  Returns a dict (reporting, not the headline)."""
    import numpy as np
    import torch
    from w4a16_linear_amd import opq
    from w4a16_linear_amd import workloads as WL

    alpha = args.alpha
    shapes = [(f"block{b}.{nm}", WL.model_seed(b, i), n, k)
              for b in range(WL.BLOCKS) for i, (nm, n, k) in enumerate(WL.BLOCK_LAYERS)]
    weights, qws, outs = [], [], {}
    for _, seed, n, k in shapes:
        weights.append(WL.student_t_device(seed, (n, k), dev))
        qws.append(opq.QuantizedWeight(torch.zeros((n, k // 8), dtype=torch.int32, device=dev),
                                       torch.zeros((n, k // 32), dtype=torch.int32, device=dev),
                                       torch.zeros((n,), dtype=torch.float32, device=dev)))
        if (n, k) not in outs:  # one bf16 output per shape: the pass rewrites it per layer
            outs[(n, k)] = torch.zeros((n, k), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    nweights = sum(n * k for _, _, n, k in shapes)
    alg_q = sum(n * k * 2.625 + 4 * n for _, _, n, k in shapes)
    alg_d = alg_q
    stream = torch.cuda.current_stream(dev)

    def quant_all(a):
        for w, qw in zip(weights, qws):
            opq.quantize(w, a, out=qw)

    def dequant_all(a):
        for qw, (_, _, n, k) in zip(qws, shapes):
            opq.dequantize(qw, a, out=outs[(n, k)])

    reps = max(1, min(args.steps, 10))
    for _ in range(max(1, min(args.warmup, 3))):
        quant_all(alpha)
        dequant_all(alpha)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        quant_all(alpha)
        dequant_all(alpha)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_pass = start.elapsed_time(stop) / reps

    kern = {}
    for name, fn, alg in (("quantize", quant_all, alg_q), ("dequantize", dequant_all, alg_d)):
        per = []
        for _ in range(5):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(alpha)
            e1.record(stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3)
        us = float(np.median(per))
        ideal = alg / (HBM_PEAK_GBS * 1e9) * 1e6
        kern[name] = {"us": round(us, 1), "bound": "hbm", "ideal_us": round(ideal, 1),
                      "frac": round(ideal / us, 4), "GBps": round(alg / (us * 1e-6) / 1e9, 1),
                      "algorithmic_bytes": int(alg), "launches": len(shapes)}
    ideal_total = sum(v["ideal_us"] for v in kern.values())

    # The streaming kernel on every layer's rows and bytes (each distinct shape
    # timed once, counted once per layer).
    counts = {}
    for _, _, n, k in shapes:
        counts[(n, k)] = counts.get((n, k), 0) + 1
    for name in ("quantize", "dequantize"):
        c = sum(cnt * stream_ceiling_us(dev, stream, n, *row_bytes(name, k, 2), 5)
                for (n, k), cnt in counts.items())
        kern[name]["stream_ceiling_us"] = round(c, 1)
        kern[name]["frac_of_stream_ceiling"] = round(c / kern[name]["us"], 4)

    # SNR(alpha) - SNR(1) over the whole model (reporting only, not timed)
    def snr_db(a):
        num = den = 0.0
        for w, qw, (_, _, n, k) in zip(weights, qws, shapes):
            opq.quantize(w, a, out=qw)
            d = opq.dequantize(qw, a, out=outs[(n, k)])
            wf = w.float()
            num += float(wf.double().square().sum())
            den += float((wf - d.float()).double().square().sum())
        return 10.0 * np.log10(num / den)
    snr = {a: snr_db(a) for a in (0.45, 0.73, 1.0)}

    # the card's own stored form (a float16 max per 128 weights), same weights
    def snr_grouped_db(a, gs=128):
        num = den = 0.0
        for w, (_, _, n, k) in zip(weights, shapes):
            d = opq.dequantize(opq.quantize_grouped(w, a, gs), a, out=outs[(n, k)])
            wf = w.float()
            num += float(wf.double().square().sum())
            den += float((wf - d.float()).double().square().sum())
        return 10.0 * np.log10(num / den)
    snr_g128 = {a: snr_grouped_db(a) for a in (0.45, 0.73, 1.0)}

    # alpha sweep: per-row error sums straight from the weights (nothing stored),
    # every layer at each alpha of the grid; timed per alpha.
    grid = [round(0.30 + 0.05 * i, 2) for i in range(15)]
    sums = [torch.empty((n, 2), dtype=torch.float64, device=dev) for _, _, n, _ in shapes]
    alg_e = sum(n * k * 2 + 16 * n for _, _, n, k in shapes)

    def sweep_one(a):
        for w, s in zip(weights, sums):
            opq.error_sums(w, a, out=s)

    sweep_one(grid[0])
    torch.cuda.synchronize()
    sweep_snr, sweep_us = [], []
    for a in grid:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sweep_one(a)
        e1.record(stream)
        tot = torch.stack([s.sum(dim=0) for s in sums]).sum(dim=0).cpu()
        sweep_us.append(e0.elapsed_time(e1) * 1e3)
        sweep_snr.append(10.0 * float(np.log10(float(tot[0]) / float(tot[1]))))
    sweep_med = float(np.median(sweep_us))
    best = int(np.argmax(sweep_snr))
    sweep = {"alphas": grid, "snr_db": [round(v, 3) for v in sweep_snr],
             "best_alpha": grid[best], "us_per_alpha": round(sweep_med, 1),
             "GBps": round(alg_e / (sweep_med * 1e-6) / 1e9, 1),
             "frac": round(alg_e / (sweep_med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
             "algorithmic_bytes": int(alg_e), "launches": len(shapes),
             "stored_form_agrees_db": max(abs(sweep_snr[grid.index(a)] - snr[a])
                                          for a in (0.45, 1.0))}
    # SNR per code width (3..6 bits) at three alphas, whole model, nothing stored
    widths = {}
    for b in (3, 4, 5, 6):
        row = {}
        for a in (0.45, 0.73, 1.0):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for w, s_ in zip(weights, sums):
                opq.error_sums(w, a, out=s_, bits=b)
            e1.record(stream)
            tot = torch.stack([s_.sum(dim=0) for s_ in sums]).sum(dim=0).cpu()
            row[str(a)] = {"snr_db": round(10.0 * float(np.log10(float(tot[0]) / float(tot[1]))), 3),
                           "us": round(e0.elapsed_time(e1) * 1e3, 1)}
        widths[str(b)] = row
    dom = max(kern, key=lambda kk: kern[kk]["us"])
    del weights, qws, outs, sums
    return {
        "value": round(100.0 * (ideal_total * 1e-3) / ms_pass, 3),
        "unit": "% of MI355X roofline",
        "ms_per_step": round(ms_pass, 4),
        "data": "synthetic (drawn on the GPU)",
        "config": {"workload": "model: 30 DiT blocks (QKV 11520x3840, O 3840x3840, FFN "
                               "20480x3840 + 3840x10240), Student-t(4) std 0.02",
                   "weights": nweights, "layers": len(shapes), "alpha": alpha,
                   "step": "quantize every layer -> dequantize every layer",
                   "passes_timed": reps},
        "roofline": {"bound": "hbm", "achieved": kern[dom]["GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kern[dom]["GBps"] / HBM_PEAK_GBS, 4),
                     "kernel": dom, "traffic": None},
        "kernels": kern,
        "snr_db": {str(a): round(v, 3) for a, v in snr.items()},
        "snr_gain_vs_alpha1_db": {str(a): round(v - snr[1.0], 3) for a, v in snr.items()},
        "snr_db_groups_of_128": {str(a): round(v, 3) for a, v in snr_g128.items()},
        "snr_gain_vs_alpha1_db_groups_of_128": {str(a): round(v - snr_g128[1.0], 3)
                                                for a, v in snr_g128.items()},
        "alpha_sweep": sweep,
        "snr_by_width": widths,
    }


def gfx_clock_under_load(step, seconds=1.0):
    """Shader clock while the step repeats: the per-XCD gfx clocks from
    `amd-smi metric --clock` (else rocm-smi's sclk), sampled once the load has
    run for half the time.  None when neither tool answers."""
    import subprocess
    import threading

    import torch
    done = threading.Event()

    def spin():
        i = 0
        while not done.is_set():
            for _ in range(8):
                step(i)
                i += 1
            torch.cuda.synchronize()

    t = threading.Thread(target=spin, daemon=True)
    t.start()
    time.sleep(seconds / 2)
    res = None
    try:
        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True,
                           text=True, timeout=30)
        d = json.loads(r.stdout)
        d = d["gpu_data"] if isinstance(d, dict) else d
        mhz = [v["clk"]["value"] for kk, v in d[0]["clock"].items() if kk.startswith("gfx_")]
        if mhz:
            res = {"tool": "amd-smi", "gfx_mhz_mean": round(sum(mhz) / len(mhz), 1),
                   "gfx_mhz_min": min(mhz), "gfx_mhz_max": max(mhz), "domains": len(mhz)}
    except Exception:  # noqa: BLE001 - a missing or changed tool only loses this field
        res = None
    if res is None:
        try:
            r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                               text=True, timeout=30)
            card = next(iter(json.loads(r.stdout).values()))
            v = card.get("sclk clock speed:", "")
            res = {"tool": "rocm-smi", "sclk_mhz": float(v.strip("()Mhz"))}
        except Exception:  # noqa: BLE001
            res = None
    done.set()
    t.join()
    return res


def run_env(dev):
    """What the numbers were measured on."""
    import torch
    prop = torch.cuda.get_device_properties(dev)
    env = {"gpu": prop.name, "gcn_arch": getattr(prop, "gcnArchName", None),
           "compute_units": prop.multi_processor_count,
           "hip": torch.version.hip, "torch": torch.__version__}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    return env


if __name__ == "__main__":
    main()
