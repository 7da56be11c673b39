"""Benchmark: one MoE layer, forward + backward, on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: router GEMM
+ softmax + top-K, capacity drop and maps, permute, grouped SwiGLU expert FFN (gate/up
and down), gate-weighted un-permute, then the backward duals (un-permute backward,
down dgrad + SwiGLU backward, the two wgrads, gate/up dgrad, router backward, permute
backward).  The workload is the Mixtral-8x22B-shaped layer: T = 4096 tokens (one
4096-token sub-sequence), d = 6144, E = 8, top-2, SwiGLU ffn 16384, capacity factor
1.0, bf16 with fp32 accumulation, seeded synthetic inputs already resident in HBM.

The timed steps issue the step's launches one by one (`--graph` replays the step
captured once in a HIP graph instead: the same time, the launches being asynchronous and
the kernels long); `value` is T over the wall time per step.  Prints one JSON line.  `roofline` is for the grouped GEMM (the six launches of the
matrix-core GEMM kernel per step, 18 * n_kept * d * f FLOPs), timed with HIP events
on the stream the kernels run on, with the HBM traffic of those launches taken from
the hardware-counter summary under profiles/ while the GEMM source is unchanged;
`hbm_kernels` gives the same for the row-movement calls with cold caches (a 1 GiB read
before each call; `hbm_kernels_warm` back to back), `cold` the whole step after a 1 GiB
read; `cpu_baseline` times the CPU oracle on the whole workload (about 30 s on 16
cores for the Mixtral shape).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec fwd+bwd on 1 MI355X; grouped-GEMM % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Timer:
    """HIP events around the ABI calls of one step, on the current stream.  With `flush`
    set, a 1 GiB buffer is read before each call (outside its events), so the call starts
    with cold caches: the 256 MB last-level cache and the L2s hold none of its operands."""

    def __init__(self, torch, flush=None):
        self.torch = torch
        self.acc = {}
        self.on = False
        self.flush = flush

    def __call__(self, name, fn, *a, **kw):
        if not self.on:
            return fn(*a, **kw)
        t = self.torch
        if self.flush is not None:
            self.flush()
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        fn(*a, **kw)
        e.record()
        self.acc.setdefault(name, []).append((s, e))

    def means_ms(self):
        self.torch.cuda.synchronize()
        return {k: sum(s.elapsed_time(e) for s, e in v) / len(v) for k, v in self.acc.items()}


FLUSH_BYTES = 1 << 30


def make_flush(torch):
    """Reads FLUSH_BYTES (four times the 256 MB last-level cache) on the current stream, so
    that the caches hold only clean lines of this buffer: the next call finds none of its
    operands cached and inherits no dirty lines to write back (a write-flush would charge
    the write-back of up to 256 MB of someone else's data to the timed call)."""
    buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")

    def flush():
        buf.sum()
    return flush


def run_step(lay, inp, L, tm):
    """The layer's ABI calls in order, each bracketed by the timer."""
    b, rt = lay.buf, lay.rt
    tm("route", L.moe_route, lay.desc, inp["x"], inp["w_router"], inp.get("bias"),
       inp.get("w_sg"), b["logits"], b["sg_logit"], lay.routing, lay.ws_route)
    tm("permute", L.moe_permute, lay.desc, inp["x"], lay.routing, b["xp"])
    tm("ffn_fwd", L.moe_expert_ffn_fwd, lay.desc, b["xp"], inp["w_gate"], inp["w_up"],
       inp["w_down"], rt["offsets"], b["a"], b["b"], b["h"], b["o"], None)
    if lay.fs:
        tm("shared_fwd", L.moe_expert_ffn_fwd, lay.sdesc, inp["x"], inp["ws_gate"], inp["ws_up"],
           inp["ws_down"], b["shared_offsets"], b["sa"], b["sb"], b["sh"], b["shared"], None)
    tm("unpermute", L.moe_unpermute, lay.desc, b["o"], lay.routing, b.get("shared"),
       b["sg_logit"], b["y"])
    tm("unpermute_bwd", L.moe_unpermute_bwd, lay.desc, inp["dy"], b["o"], lay.routing,
       b.get("shared"), b["sg_logit"], b["d_o"], b["dgate"], b.get("dshared"), b.get("dz"))
    tm("ffn_bwd", L.moe_expert_ffn_bwd, lay.desc, b["xp"], b["a"], b["b"], b["h"],
       inp["w_gate"], inp["w_up"], inp["w_down"], rt["offsets"], b["d_o"], b["dxp"],
       b["dw_gate"], b["dw_up"], b["dw_down"], lay.ws_ffn)
    if lay.fs:
        tm("shared_bwd", L.moe_expert_ffn_bwd, lay.sdesc, inp["x"], b["sa"], b["sb"], b["sh"],
           inp["ws_gate"], inp["ws_up"], inp["ws_down"], b["shared_offsets"], b["dshared"],
           b["dx_shared"], b["dws_gate"], b["dws_up"], b["dws_down"], lay.ws_ffn)
    tm("route_bwd", L.moe_route_bwd, lay.desc, inp["x"], lay.routing, b["dgate"], b.get("dz"),
       b["dlogits"], b["dw_router"], b.get("dw_sg"), lay.ws_route_bwd)
    tm("permute_bwd", L.moe_permute_bwd, lay.desc, b["dxp"], lay.routing, b["dlogits"],
       inp["w_router"], b.get("dz"), inp.get("w_sg"), b.get("dx_shared"), b["dx"],
       lay.ws_permute_bwd)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_threads():
    """Threads for the oracle: the CPUs this process may run on, capped by OMP_NUM_THREADS
    when it is set (the share of the host a one-GPU job gets)."""
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return n


def cpu_baseline(shape, inp, lay, cap):
    """Time the CPU oracle, as it stands, on the whole workload: routing of all T tokens
    (on the GPU's logits, as the parity tests do), permutation, every expert's SwiGLU FFN
    forward and backward, un-permutation and its backward, the router backward and the
    permute backward (oracle.layer_fwd_bwd; numpy float64 with the device's bf16 storage
    points).  The inputs are copied to host memory before the clock starts."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    n = cpu_threads()
    host = {}
    for k, v in inp.items():
        if v is None:
            host[k] = None
        else:
            host[k] = v.float().cpu().numpy()
    logits = lay.buf["logits"].cpu().numpy()
    with threadpool_limits(limits=n):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        t0 = time.perf_counter()
        ref = oracle.layer_fwd_bwd(host, shape.K, shape.sub_seq, cap,
                                   "bf16" if shape.dtype == "bf16" else "f32", logits=logits)
        total = time.perf_counter() - t0
    # the oracle's own output is checked against the GPU's on the way (y and dx)
    err = {}
    for k in ("y", "dx"):
        got = lay.buf[k].float().cpu().numpy().astype(np.float64)
        exp = np.asarray(ref[k], np.float64)
        err[k] = float(np.max(np.abs(got - exp)) / max(float(np.max(np.abs(exp))), 1e-30))
    del ref, host
    return {"value": round(shape.T / total, 2), "unit": "tokens/s", "cores": int(used),
            "kind": "oracle",
            "sample": (f"the whole workload: one forward + backward of the layer, all {shape.T} "
                       f"tokens and all {shape.E} experts (oracle.layer_fwd_bwd, numpy float64 "
                       f"with bf16 storage points, routing in C)"),
            "seconds": round(total, 3), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": cpu_model(), "gpu_vs_oracle_max_abs_rel": err}


def input_sha256(inp):
    """SHA-256 of each input tensor's raw bytes (bf16 or fp32 as stored on the device)."""
    import hashlib
    import torch
    out = {}
    for k, v in inp.items():
        if v is None:
            continue
        h = hashlib.sha256()
        flat = v.reshape(-1)
        step = 1 << 26
        for i in range(0, flat.numel(), step):
            c = flat[i:i + step]
            if c.dtype == torch.bfloat16:
                c = c.view(torch.int16)
            h.update(c.cpu().numpy().tobytes())
        out[k] = h.hexdigest()
    return out


def gpu_info(torch):
    import ctypes
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_GiB": round(p.total_memory / 2 ** 30, 1)}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, torch.cuda.current_device()) == 0:
            info["clock_peak_MHz"] = v.value // 1000   # hipDeviceAttributeClockRate (kHz)
    except OSError:
        pass
    info["torch"] = torch.__version__
    info["hip"] = getattr(torch.version, "hip", None)
    return info


def gemm_traffic(workload):
    """HBM bytes per step of the six grouped-GEMM launches, from the two hardware-counter
    passes summarised under profiles/ (FETCH_SIZE and WRITE_SIZE, scaled by what the
    same counters read for a 1 GiB copy).  None when no summary covers this workload or
    the GEMM source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gemm_mfma_{workload}_hbm_traffic.md")
    src = os.path.join(ROOT, "token_dispatch_expert_router_amd", "csrc", "gemm_mfma.hip")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("machine-readable:"):
            rec = json.loads(line.split(":", 1)[1])
    if not rec:
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if sha != rec.get("kernel_source_sha256"):
        return None
    return rec


def gemm_passes(workload):
    """Per-pass averages of the six grouped-GEMM launches from the kernel-trace summary under
    profiles/ (rocprofv3 --kernel-trace of this bench), while the GEMM source is unchanged."""
    import hashlib
    name = "moe_layer_mixtral_8x22b" if workload == "mixtral_8x22b" else workload
    path = os.path.join(ROOT, "profiles", f"{name}_kernel_trace.md")
    src = os.path.join(ROOT, "token_dispatch_expert_router_amd", "csrc", "gemm_mfma.hip")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        if line.startswith("machine-readable:"):
            rec = json.loads(line.split(":", 1)[1])
    if not rec or rec.get("kernel_source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
        return None
    return rec["passes"]


def bench_shard(args):
    """One GPU's expert-side share of the layer spread over G GPUs: the expert FFN
    forward + backward (six grouped-GEMM launches) on the rows its experts receive, with
    fp32 partial o and dxp under expert-tensor parallelism.  Routing and permutation of
    the G sources' tokens run once, untimed, to produce those rows."""
    import torch
    import moe_synth
    from token_dispatch_expert_router_amd import _lib as L
    from token_dispatch_expert_router_amd.layer import Dispatch, ExpertShard, expert_rows

    L.load()
    s = moe_synth.shard_by_name(args.shard)
    src = s.layer
    cap = L.moe_capacity(src.T, src.K, src.E, src.cf) if src.cf is not None else -1
    log(f"bench: shard {s.name}: routing {s.G} x {src.T} tokens on the GPU")
    tok = moe_synth.make_source_tokens(src, s.G, device="cuda")
    dp = Dispatch(s.G * src.T, src.d, src.E, src.K, src.T, cap, src.torch_dtype, device="cuda")
    dp.run(tok["x"], tok["w_router"], tok["bias"])
    xp, loc = expert_rows(dp, s.e0, s.e1)
    rows = xp.shape[0]
    del tok
    w = moe_synth.make_shard_weights(s, device="cuda")
    d_o = moe_synth.make_shard_grad(s, rows, device="cuda")
    sh = ExpertShard(rows, src.d, s.E_local, s.f_local, src.torch_dtype, partial=s.etp > 1,
                     device="cuda")
    tm = Timer(torch)

    def step():
        tm("ffn_fwd", sh.forward, xp, w, loc)
        tm("ffn_bwd", sh.backward, xp, w, loc, d_o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tm.on = True
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    calls = tm.means_ms()
    gemm_ms = calls["ffn_fwd"] + calls["ffn_bwd"]
    flops = 18.0 * rows * src.d * s.f_local
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    log(f"bench: {args.steps} timed steps, {ms:.3f} ms/step; per call (ms): "
        + ", ".join(f"{k} {v:.3f}" for k, v in calls.items()))
    rec = {
        "metric": "expert-shard grouped-GEMM TFLOP/s fwd+bwd on 1 MI355X",
        "value": round(flops / (ms * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": s.name, "source": src.name, "sources": s.G,
                   "experts": [s.e0, s.e1], "etp": s.etp, "rows": rows, "d": src.d,
                   "ffn_local": s.f_local, "rows_per_expert": host_list(loc),
                   "partial_fp32": s.etp > 1,
                   "parallelism": f"one GPU's share of ep{src.E // s.E_local} x etp{s.etp}"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None,
                     "kernel": "gg_mfma_kernel (6 launches per step)",
                     "flops_per_step": flops, "ms_per_step": round(gemm_ms, 4)},
        "calls_ms": {k: round(v, 4) for k, v in calls.items()},
    }
    print(json.dumps(rec), flush=True)


def bench_route_sweep(args):
    """Routing alone (moe_route_from_logits: softmax, top-K, drop, maps) on seeded logits of
    T tokens, with the drop taken per 4096-token sub-sequence or over the whole sequence
    (the selection over a gathered-logits tensor of several GPUs' tokens); one JSON line
    per case."""
    import torch
    from token_dispatch_expert_router_amd import _lib as L
    from token_dispatch_expert_router_amd.layer import Dispatch

    L.load()
    E, K, cf = 8, 2, 1.0
    for T in (4096, 16384, 32768, 65536):
        for S in sorted({4096, T}):
            g = torch.Generator(device="cuda").manual_seed(T + S)
            logits = torch.randn((T, E), generator=g, device="cuda") * 2.0
            cap = L.moe_capacity(S, K, E, cf)
            dp = Dispatch(T, 64, E, K, S, cap, torch.float32, device="cuda")
            for _ in range(3):
                L.moe_route_from_logits(dp.desc, logits, dp.routing, dp.ws)
            torch.cuda.synchronize()
            times = []
            for _ in range(20):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                L.moe_route_from_logits(dp.desc, logits, dp.routing, dp.ws)
                b.record()
                b.synchronize()
                times.append(a.elapsed_time(b))
            times.sort()
            ms = times[len(times) // 2]
            print(json.dumps({"metric": "routing time (softmax, top-K, capacity drop, maps)",
                              "value": round(ms * 1000.0, 2), "unit": "us", "T": T, "E": E,
                              "K": K, "sub_seq": S, "capacity": cap,
                              "n_kept": int(dp.rt["n_kept"].item()),
                              "higher_is_better": False, "data": "synthetic"}), flush=True)


def host_list(t):
    c = t.cpu().tolist()
    return [b - a for a, b in zip(c[:-1], c[1:])]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_8x22b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache leg (a 1 GiB read before each timed call)")
    ap.add_argument("--no-hash", action="store_true", help="skip the inputs' SHA-256")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph instead of the "
                         "launches issued one by one")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many MiB "
                         "(a known-size reference for hardware byte counters)")
    ap.add_argument("--shard", default=None,
                    help="time one GPU's expert-side share of a multi-GPU layer instead "
                         "(mixtral_ep8, mixtral_ep4_etp2, mixtral_etp8)")
    ap.add_argument("--route-sweep", action="store_true",
                    help="time the routing alone over 4096..65536 tokens, dropped per "
                         "4096-token sub-sequence or over the whole sequence")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's MoE layer; --gpus {args.gpus} is not supported "
              "(the cross-GPU exchanges are outside this library)", file=sys.stderr)
        sys.exit(2)

    if args.shard:
        bench_shard(args)
        return
    if args.route_sweep:
        bench_route_sweep(args)
        return

    import torch
    import moe_synth
    from token_dispatch_expert_router_amd import _lib as L
    from token_dispatch_expert_router_amd.layer import MoELayer

    L.load()
    shape = moe_synth.shape_by_name(args.workload)
    cap = L.moe_capacity(shape.sub_seq, shape.K, shape.E, shape.cf) if shape.cf is not None else -1
    log(f"bench: workload {shape.name}, drawing inputs on the GPU")
    inp = moe_synth.make_inputs(shape, device="cuda")
    lay = MoELayer(shape.T, shape.d, shape.E, shape.K, shape.f, shape.sub_seq, cap,
                   shape.torch_dtype, fs=shape.fs, device="cuda")
    tm = Timer(torch)
    for i in range(args.warmup):
        run_step(lay, inp, L, tm)
    torch.cuda.synchronize()
    log(f"bench: {args.warmup} warmup steps done")
    n_kept = int(lay.rt["n_kept"].item())

    # --graph: the step's launches are captured once in a HIP graph and the timed steps are
    # graph replays (the ABI calls allocate nothing and never synchronise, so a step is
    # capturable).
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step(lay, inp, L, tm)
        graph.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            run_step(lay, inp, L, tm)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1000.0 / args.steps
    # per-call HIP events: the same number of steps again, launched one by one
    tm.on = True
    for i in range(args.steps):
        run_step(lay, inp, L, tm)
    calls = tm.means_ms()
    log(f"bench: {args.steps} timed steps ({'HIP graph replays' if graph else 'eager'}), "
        f"{ms:.3f} ms/step; per call (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in calls.items()))

    # cold caches: the same steps again with a 1 GiB read before every call (per-call
    # figures) and before every step (whole-step figure)
    calls_cold, ms_cold = None, None
    if not args.no_cold:
        flush = make_flush(torch)
        tmc = Timer(torch, flush=flush)
        tmc.on = True
        for i in range(args.steps):
            run_step(lay, inp, L, tmc)
        calls_cold = tmc.means_ms()
        off = Timer(torch)
        pairs = []
        for i in range(args.steps):
            flush()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            run_step(lay, inp, L, off)
            z.record()
            pairs.append((a, z))
        torch.cuda.synchronize()
        ms_cold = sum(a.elapsed_time(z) for a, z in pairs) / len(pairs)
        log(f"bench: cold caches, {ms_cold:.3f} ms/step; per call (ms): "
            + ", ".join(f"{k} {v:.3f}" for k, v in calls_cold.items()))

    T, d, E, K, f, fs = shape.T, shape.d, shape.E, shape.K, shape.f, shape.fs
    gemm_flops = 18.0 * n_kept * d * f + (18.0 * T * d * fs if fs else 0.0)
    router_flops = 6.0 * T * d * E

    def gemm_ms_of(c):
        return c["ffn_fwd"] + c["ffn_bwd"] + c.get("shared_fwd", 0) + c.get("shared_bwd", 0)

    gemm_ms = gemm_ms_of(calls)
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    traffic = gemm_traffic(shape.name)
    s = 2 if shape.dtype == "bf16" else 4  # bytes per element
    hbm_bytes = {
        "permute": (T + n_kept) * d * s + 4 * n_kept,
        "unpermute": (n_kept + T) * d * s + 8 * T * K + (T * d * s if fs else 0),
        "unpermute_bwd": (T + 2 * n_kept) * d * s + 12 * T * K,
        "permute_bwd": (n_kept + T) * d * s + 4 * T * K,
    }

    def hbm_of(c, label):
        per = {k: {"bytes": v, "ms": round(c[k], 4),
                   "GBs": round(v / (c[k] * 1e-3) / 1e9, 1),
                   "frac": round(v / (c[k] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
               for k, v in hbm_bytes.items()}
        tot = sum(hbm_bytes.values())
        t_ms = sum(c[k] for k in hbm_bytes)
        return {"caches": label, "bytes": tot, "ms": round(t_ms, 4),
                "GBs": round(tot / (t_ms * 1e-3) / 1e9, 1),
                "frac": round(tot / (t_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "calls": per}

    kept = host_list(lay.rt["offsets"])
    rec = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic",
        "timing": "HIP graph replay of the whole step" if graph is not None else "eager launches",
        "config": {"workload": shape.name, "T": T, "d": d, "E": E, "K": K, "ffn": f,
                   "shared_ffn": fs, "sub_seq": shape.sub_seq, "capacity_factor": shape.cf,
                   "capacity": cap, "n_kept": n_kept, "kept_per_expert": kept,
                   "parallelism": "none (1 GPU)"},
        "tflops": round((gemm_flops + router_flops) / (ms * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic["traffic_bytes_per_step"] if traffic else None,
                     "traffic_unit": "HBM bytes per step (six launches), hardware counters",
                     "algorithmic_bytes_per_step": (traffic or {}).get("algorithmic_bytes_per_step"),
                     "kernel": "gg_mfma_kernel (6 launches per step: fwd gate/up, fwd down, "
                               "dgrad down, wgrad down, wgrad gate/up, dgrad gate/up)",
                     "flops_per_step": gemm_flops, "ms_per_step": round(gemm_ms, 4),
                     "passes_from_kernel_trace": gemm_passes(shape.name)},
        "calls_ms": {k: round(v, 4) for k, v in calls.items()},
    }
    if calls_cold is not None:
        gc = gemm_ms_of(calls_cold)
        rec["roofline"]["frac_cold"] = round(gemm_flops / (gc * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        rec["hbm_kernels"] = hbm_of(calls_cold, "cold: 1 GiB read before each call")
        rec["hbm_kernels_warm"] = hbm_of(calls, "warm: calls back to back")
        rec["cold"] = {"ms_per_step": round(ms_cold, 4),
                       "tokens_per_s": round(T / (ms_cold * 1e-3), 1),
                       "how": "1 GiB read before each step, HIP events around the step",
                       "calls_ms": {k: round(v, 4) for k, v in calls_cold.items()}}
    else:
        rec["hbm_kernels"] = hbm_of(calls, "warm: calls back to back")
    rec["gpu"] = gpu_info(torch)
    rec["host"] = {"cpu_model": cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0))}
    if not args.no_hash:
        rec["inputs_sha256"] = input_sha256(inp)
    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["calib_copy_bytes"] = n * 4
        del src, dst
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle on the whole workload")
        cb = cpu_baseline(shape, inp, lay, cap)
        # the same algorithmic FLOPs as the GPU's `tflops` (grouped GEMMs + router)
        cb["gflops"] = round((gemm_flops + router_flops) / cb["seconds"] / 1e9, 2)
        rec["cpu_baseline"] = cb
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
