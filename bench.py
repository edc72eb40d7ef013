"""MoE-layer forward benchmark on one MI355X.

One step = one moe_layer_forward (route -> dispatch -> expert FFN -> combine)
over one batch of seeded synthetic input, inputs resident in HBM.  Default
workload: the prefill-shaped Mixtral-style bf16 layer (T=16384 tokens,
d=4096, 8 SwiGLU experts with h=14336, top-2, softmax renormalised, skewed
logit offsets, no drops), the largest of the five workloads by flops and
bytes; ``--config i`` selects another.  Without ``--config``, the line also
carries the other four workloads under ``other_workloads`` (tokens/s and the
first expert GEMM against its roofline, timed the same way on fewer steps).

Prints one JSON line: tokens/s over the timed steps (back to back), the
roofline of the dominant kernel (the first expert GEMM) from HIP events
recorded around it on the stream it runs on, per-stage times from further
steps with an event at every stage boundary and the 256 MB Infinity Cache
flushed before each of them, and the fp64 CPU oracle timed on the host on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
import types

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # dense fp32 matrix
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
# rocprofv3 FETCH_SIZE/WRITE_SIZE records of each workload's first expert
# GEMM (per launch, calibrated against a plain copy); each is reported only
# while the sources it lists hash to its recorded value
TRAFFIC_RECORDS = {0: "profiles/gemm1_snippet_traffic.json",
                   1: "profiles/gemm1_decode_traffic.json",
                   2: "profiles/gemm1_prefill_traffic.json",
                   3: "profiles/gemm1_switch_traffic.json",
                   4: "profiles/gemm1_deepseek_traffic.json"}
MALL_FLUSH_MIB = 512           # > 2x the 256 MB Infinity Cache
DEFAULT_CONFIG = 2             # the prefill-shaped Mixtral layer: the largest workload
STAGES = ["route", "dispatch", "gemm1", "gemm2", "combine"]


def _hip():
    """The HIP runtime already loaded in this process (torch's copy)."""
    path = None
    for line in open("/proc/self/maps"):
        if "libamdhip64" in line:
            path = line.split()[-1]
            break
    h = ctypes.CDLL(path or "libamdhip64.so")
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    return h


class Events:
    def __init__(self, hip, n):
        self.hip = hip
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) == 0
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


def algorithmic_bytes(wl, kept_rows: int, used_experts: int, shared: bool, sent_rows=None):
    """Bytes each stage must move (read once, write once), per launch.
    kept_rows: rows of the executed experts; sent_rows: rows of the whole
    send buffer the dispatch packs (all ranks' segments)."""
    sent = kept_rows if sent_rows is None else sent_rows
    sa = 4 if wl.act_dtype == "f32" else 2
    sw = {"f32": 4, "bf16": 2, "fp8": 1}[wl.w_dtype]
    T, d, h, E, k = wl.T, wl.d, wl.h, wl.E, wl.k
    n1 = 2 if wl.act == "swiglu" else 1
    nx = kept_rows + (T if shared else 0)
    groups = used_experts + (1 if shared else 0)
    return {
        "route": T * d * sa + E * d * sa + 8 * T * k,
        "dispatch": 8 * T * k + 4 * sent + T * d * sa + sent * d * sa,
        "gemm1": n1 * h * d * sw * groups + nx * d * sa + nx * h * sa,
        "gemm2": d * h * sw * groups + nx * h * sa + nx * d * sa,
        "combine": kept_rows * d * sa + 2 * T * d * sa + (T * d * sa if shared else 0) + 8 * T * k,
    }


def gemm_flops(wl, kept_rows: int, shared: bool):
    nx = kept_rows + (wl.T if shared else 0)
    n1 = 2 if wl.act == "swiglu" else 1
    return {"gemm1": 2 * n1 * wl.d * wl.h * nx, "gemm2": 2 * wl.d * wl.h * nx}


def sources_sha256(files) -> str:
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def traffic_from_profiles(cfg: int, w_layout: str):
    """HBM bytes per launch of the workload's first expert GEMM from
    committed rocprofv3 counter runs, valid only while the kernel sources
    and the weight layout are the ones the counters were taken on."""
    name = TRAFFIC_RECORDS.get(cfg)
    path = os.path.join(ROOT, name) if name else None
    if not path or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256") != sources_sha256(rec.get("sources", [])) or \
            rec.get("w_layout") != w_layout:
        return None
    return rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def token_sample(wl, n: int):
    """The workload restricted to its first n tokens (same weights, router
    and offsets): the bounded sample the CPU oracle is timed on."""
    if n >= wl.T:
        return wl
    sub = types.SimpleNamespace(**vars(wl))
    sub.T = n
    sub.x = wl.x[:n]
    return sub


def cpu_baseline(wl, budget_s: float = 12.0, max_reps: int = 8, max_tokens: int = 2048):
    """The fp64 oracle on the host cores: whole-layer forwards of the
    workload's first ``max_tokens`` tokens (all of them for smaller
    workloads), repeated until about budget_s seconds of CPU work (at most
    max_reps); the rate is tokens over the total time.  Every forward decodes
    the expert weights to fp64 again, as the oracle does."""
    import threadpoolctl

    from oracle import oracle as O
    threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
                   if p.get("user_api") == "blas"), default=1)
    sub = token_sample(wl, max_tokens)
    reps, dt = 0, 0.0
    while reps < max_reps and (reps == 0 or dt < budget_s):
        t0 = time.perf_counter()
        O.layer(sub)
        dt += time.perf_counter() - t0
        reps += 1
    what = (f"all {wl.T} tokens" if sub.T == wl.T else
            f"the first {sub.T} of the {wl.T} tokens (same weights and routing rule)")
    return {"value": reps * sub.T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{reps} x the whole layer on {what} of the same workload, fp64, "
                      f"{dt:.1f} s in total (input generation excluded)"}


def extras(M, wl, layer, hip, args):
    """Measured outside the timed region: the auxiliary-loss kernel on
    logits of the workload's shape, and (workloads with a selection bias) a
    route -> dispatch -> bias-update loop on the workload's own router."""
    import numpy as np
    import torch
    ev = Events(hip, 2)
    logits = torch.randn((wl.T, wl.E), device="cuda:0")
    M.moe_aux_loss(logits, layer.counts, wl.k, M.SCORE[wl.score], 0.01)
    torch.cuda.synchronize()
    reps = 20
    st = torch.cuda.current_stream().cuda_stream
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventRecord(ev.ev[0], st)
    for _ in range(reps):
        M.moe_aux_loss(logits, layer.counts, wl.k, M.SCORE[wl.score], 0.01)
    hip.hipEventRecord(ev.ev[1], st)
    torch.cuda.synchronize()
    out = {"aux_loss_us": ev.ms(0, 1) * 1e3 / reps}
    ev.close()
    if wl.b_select is None or args.balance_steps <= 0:
        out["balance"] = None
        return out
    mean = wl.T * wl.k / wl.E
    loads = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.balance_steps):
        layer.route()
        layer.dispatch()
        loads.append(layer.counts.max())
        layer.update_bias(args.balance_gamma)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    loads = [int(x.item()) / mean for x in loads]
    out["balance"] = {"steps": args.balance_steps, "gamma": args.balance_gamma,
                      "max_over_mean_load": [round(loads[0], 3), round(min(loads), 3), round(loads[-1], 3)],
                      "ms_per_step": dt * 1e3 / args.balance_steps,
                      "step": "route + dispatch + bias update (wall clock, host loop)"}
    return out


def copy_probe(mib: int, steps: int):
    """A plain copy of known size (and a read-only reduction) on the device:
    the reference for scaling the rocprofv3 byte counters and the measured
    ceiling of HBM bandwidth on this machine."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    out = {}
    for name, fn, nbytes in (("copy", lambda: dst.copy_(src), 2 * n * 4),
                             ("read", lambda: src.sum(), n * 4)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        out[name] = {"bytes_per_launch": nbytes, "ms": ms, "GBps": nbytes / ms / 1e6}
    print(json.dumps({"copy_probe_mib": mib, **out}), flush=True)


def dense_reference(wl, steps: int):
    """The vendor library's rate on one dense GEMM with the flops of the
    workload's first expert GEMM at even routing: rows = the executed
    experts' share of the T*k assignments (plus T for a shared expert),
    N = n*h, K = d, bf16, one torch.matmul on the nn.Linear layout.  A
    reference point for the grouped kernels, not part of the layer."""
    import torch
    n1 = 2 if wl.act == "swiglu" else 1
    M = wl.T * wl.k * (wl.e_end - wl.e_begin) // wl.E + (wl.T if wl.shared else 0)
    N, K = n1 * wl.h, wl.d
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b.t()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        c = a @ b.t()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del c
    print(json.dumps({"dense_reference": f"torch.matmul bf16 [{M},{K}] x [{K},{N}]", "ms": ms,
                      "tflops": 2.0 * M * N * K / ms / 1e9}), flush=True)


def timed_steps(layer, K: int, W: int, hip):
    """W untimed forwards, then K timed back to back between synchronises;
    only the two events around the first expert GEMM are recorded (each
    recorded event delays the next kernel by a few microseconds): they give
    the dominant kernel's duration per step.  Returns (wall s, GEMM 1 ms)."""
    import numpy as np
    import torch
    for _ in range(W):
        layer.forward()
    torch.cuda.synchronize()
    ev = Events(hip, 2 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        layer.forward(events=[None, None, ev.ev[2 * s], ev.ev[2 * s + 1], None, None])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gemm1_ms = float(np.mean([ev.ms(2 * s, 2 * s + 1) for s in range(K)]))
    ev.close()
    return wall, gemm1_ms


def dominant_roofline(wl, cfg: int, gemm1_ms: float, nbytes, flops, w_layout: str):
    """The first expert GEMM against its roofline: HBM for the decode
    workload (it streams w1 and w3), the matrix cores otherwise."""
    g1_s = gemm1_ms / 1e3
    if cfg == 1:
        achieved = nbytes["gemm1"] / g1_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS}
        roof["kernel"] = "stream_gemm_kernel (expert GEMM 1: w1/w3 + SwiGLU, weight streaming)"
    else:
        # the MFMA instructions the kernel issues are bf16 (fp8 weights are
        # widened to bf16 in registers) or fp32: that dtype's peak
        peak = FP32_PEAK_TFLOPS if wl.act_dtype == "f32" else BF16_PEAK_TFLOPS
        achieved = flops["gemm1"] / g1_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
        roof["kernel"] = ("grouped_gemm_kernel (fp32 MFMA" if wl.act_dtype == "f32"
                          else "dma_gemm_kernel (bf16 MFMA") + ", expert GEMM 1 + activation)"
        if wl.w_dtype == "fp8":
            roof["frac_of_fp8_peak"] = achieved / FP8_PEAK_TFLOPS
    roof["traffic"] = traffic_from_profiles(cfg, w_layout)
    roof["algorithmic_bytes"] = nbytes["gemm1"]
    roof["algorithmic_flops"] = flops["gemm1"]
    return roof


def other_workload(M, cfg: int, hip, w_layout_arg, K: int = 20, W: int = 3):
    """Tokens/s and the first expert GEMM's roofline of another workload,
    timed as the main one on fewer steps (no stage breakdown, no extras)."""
    import numpy as np
    import torch
    from synth import make_workload
    print(f"[bench] other workload {cfg}", file=sys.stderr, flush=True)
    wl = make_workload(cfg)
    w_layout = w_layout_arg or ("rowmajor" if wl.act_dtype == "f32" else "tiled")
    layer = M.MoELayer(wl, device="cuda:0", keep_logits=False,
                       w_layout=M.MOE_W_TILED16 if w_layout == "tiled" else M.MOE_W_ROWMAJOR)
    wall, gemm1_ms = timed_steps(layer, K, W, hip)
    res = layer.results()
    off = res["off"]
    kept_rows = int(off[wl.e_end] - off[wl.e_begin])
    used = int(np.count_nonzero(res["kept"][wl.e_begin:wl.e_end]))
    shared = wl.shared is not None
    nbytes = algorithmic_bytes(wl, kept_rows, used, shared, sent_rows=int(off[wl.E]))
    flops = gemm_flops(wl, kept_rows, shared)
    roof = dominant_roofline(wl, cfg, gemm1_ms, nbytes, flops, w_layout)
    del layer
    torch.cuda.empty_cache()
    return {"workload": f"{wl.name}: T={wl.T}, d={wl.d}, E={wl.E}, top-{wl.k}, {wl.act} "
                        f"h={wl.h}{' + shared' if shared else ''}, capacity "
                        f"{'none' if wl.cf is None else wl.cf}",
            "value": wl.T * K / wall, "unit": "tokens/s", "steps": K, "warmup": W,
            "ms_per_step": wall * 1e3 / K, "gemm1_ms_timed": gemm1_ms,
            "dtype": wl.act_dtype if wl.w_dtype != "fp8" else "bf16 (fp8 e4m3 weights)",
            "expert_weight_layout": w_layout, "roofline": roof}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=None,
                    help=f"workload index 0-4 (default {DEFAULT_CONFIG}: the prefill-shaped "
                         "Mixtral layer, plus a short pass over the other four)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="without --config: skip the pass over the other four workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--w-layout", choices=["rowmajor", "tiled"], default=None,
                    help="expert weight layout (default: tiled, re-laid out once at load time, "
                         "wherever the kernels take it, i.e. bf16 activations; row-major for "
                         "the fp32 workload)")
    ap.add_argument("--balance-steps", type=int, default=30,
                    help="after the timed region: route -> dispatch -> bias update steps on "
                         "workloads with a selection bias (reports max/mean expert load)")
    ap.add_argument("--balance-gamma", type=float, default=0.01)
    ap.add_argument("--dense-reference", action="store_true",
                    help="instead of the layer: time torch.matmul (the vendor BLAS) on the dense "
                         "bf16 GEMM with the first expert GEMM's flops")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="instead of the layer: time a plain device copy of MIB MiB (HBM "
                         "calibration for the traffic counters) and a full read (sum)")
    args = ap.parse_args()
    others = args.config is None and not args.no_other_workloads
    if args.config is None:
        args.config = DEFAULT_CONFIG
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the MoE layer; runs on more than one GPU "
              "are not part of this build (no collectives). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import expert_token_routing_gemm_amd as M
    from synth import make_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    if args.dense_reference:
        from synth.gen import CONFIGS
        dense_reference(types.SimpleNamespace(**CONFIGS[args.config]), args.steps)
        return
    print(f"[bench] generating workload {args.config}", file=sys.stderr, flush=True)
    wl = make_workload(args.config)
    w_layout = args.w_layout or ("rowmajor" if wl.act_dtype == "f32" else "tiled")
    layer = M.MoELayer(wl, device="cuda:0", keep_logits=False,
                       w_layout=M.MOE_W_TILED16 if w_layout == "tiled" else M.MOE_W_ROWMAJOR)
    hip = _hip()
    K, W = args.steps, args.warmup
    print(f"[bench] warmup {W}, timed {K}", file=sys.stderr, flush=True)
    wall, gemm1_ms = timed_steps(layer, K, W, hip)
    n = M.MOE_LAYER_EVENTS
    ms_per_step = wall * 1e3 / K
    value = wl.T * K / wall

    # Stage breakdown, after the timed region: an event at every stage
    # boundary, and before each such step a 512 MiB read that evicts the
    # layer's buffers from the 256 MB Infinity Cache (outside the events), so
    # every stage starts cache-cold as in a model where other layers run in
    # between.  The eviction reads (a sum) rather than writes: a write would
    # leave the caches full of dirty lines whose write-back the first stage
    # would pay for.
    KB = min(K, 20)
    flush = torch.ones((MALL_FLUSH_MIB << 18,), dtype=torch.int32, device="cuda:0")
    flush.sum()
    ev = Events(hip, n * KB)
    for s in range(KB):
        flush.sum()
        layer.forward(events=ev.ev[s * n:(s + 1) * n])
    torch.cuda.synchronize()
    del flush
    per = {st: [] for st in STAGES}
    step_cold = []
    for s in range(KB):
        b = s * n
        per["route"].append(ev.ms(b + 0, b + 1))
        per["dispatch"].append(ev.ms(b + 1, b + 2))
        per["gemm1"].append(ev.ms(b + 2, b + 3))
        per["gemm2"].append(ev.ms(b + 3, b + 4))
        per["combine"].append(ev.ms(b + 4, b + 5))
        step_cold.append(ev.ms(b + 0, b + 5))
    step_cold_ms = float(np.mean(step_cold))
    ev.close()
    stage_ms = {k: float(np.mean(v)) for k, v in per.items()}

    res = layer.results()
    off = res["off"]
    kept_rows = int(off[wl.e_end] - off[wl.e_begin])
    used = int(np.count_nonzero(res["kept"][wl.e_begin:wl.e_end]))
    shared = wl.shared is not None
    nbytes = algorithmic_bytes(wl, kept_rows, used, shared, sent_rows=int(off[wl.E]))
    flops = gemm_flops(wl, kept_rows, shared)
    roof = dominant_roofline(wl, args.config, gemm1_ms, nbytes, flops, w_layout)
    stage_frac = {st: (nbytes[st] / (stage_ms[st] / 1e3) / 1e9) / HBM_PEAK_GBS for st in STAGES}

    out = {
        "metric": "MoE-layer tokens/s (route->dispatch->expert GEMM->combine)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.act_dtype if wl.w_dtype != "fp8" else "bf16 (fp8 e4m3 weights)",
        "data": "synthetic (seeded; random-init weights of the stated shapes)",
        "config": {"workload": f"{wl.name}: T={wl.T}, d={wl.d}, E={wl.E}, top-{wl.k}, "
                               f"{wl.act} h={wl.h}, executed experts {wl.e_begin}-{wl.e_end - 1}"
                               f"{' + shared' if shared else ''}, capacity "
                               f"{'none' if wl.cf is None else wl.cf}",
                   "tokens": wl.T, "expert_weight_layout": w_layout,
                   "parallelism": "one GPU's share (no collectives)"},
        "gemm1_ms_timed": gemm1_ms,
        "stages_ms": stage_ms,
        "stages_note": (f"stage times from {KB} further steps with an event at every stage "
                        f"boundary, each after a {MALL_FLUSH_MIB} MiB read that flushes the "
                        f"Infinity Cache ({step_cold_ms:.4f} ms per such step)"),
        "ms_per_step_cache_cold": step_cold_ms,
        "stages_hbm_frac": stage_frac,
        "gemm_tflops": {k: flops[k] / (stage_ms[k] / 1e3) / 1e12 for k in flops},
        "kept_rows": kept_rows,
        "wall_s": wall,
        "roofline": roof,
    }
    out["extras"] = extras(M, wl, layer, hip, args)
    if others:
        del layer
        torch.cuda.empty_cache()
        out["other_workloads"] = {
            str(c): other_workload(M, c, hip, args.w_layout) for c in range(5) if c != args.config}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
