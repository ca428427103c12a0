"""Benchmark of the Llama 4 MoE feed-forward block on one MI355X.

One step = one moe_forward over one batch of synthetic tokens: router GEMM,
top-1 + sigmoid gate, histogram / scan / permutation, grouped gate/up GEMM
with the SwiGLU epilogue (routed + shared), shared down GEMM, routed down
GEMM with un-permute + combine.  Inputs are generated on the GPU by the
seeded generator before timing and stay resident in HBM.

Prints ONE JSON line (rank 0, N = 1):
  value       tokens/s of the whole block (timed moe_forward calls)
  roofline    the dominant stage (largest average duration, timed with HIP
              events recorded by the library on its stream over a second
              timed region of moe_forward_timed calls, which run the stages in
              order on one stream) against the MFMA or HBM roofline, using
              algorithmic FLOPs / bytes of that stage
  clock_mhz   mean core clock during ~0.5 s of further moe_forward calls
              (sysfs pp_dpm_sclk), and the MFMA fractions against the peak at
              that clock (the quoted peaks assume 2.4 GHz)
  cpu_baseline  the fp64 CPU oracle timed on a bounded token sample

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# dense MFMA peak by weight dtype, FLOP/s (int8 weights are converted to
# bf16 and multiplied on the bf16 MFMA)
PEAK = {"bf16": 2516.6e12, "e4m3": 5033.2e12, "f32": 157.3e12, "i8": 2516.6e12, "i4": 2516.6e12}
HBM_PEAK = 8.0e12                                                 # bytes/s
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def esize(dt: str) -> int:
    return {"f32": 4, "bf16": 2, "e4m3": 1, "i8": 1, "i4": 0.5}[dt]


def stage_work(cfg, counts):
    """Algorithmic (FLOPs, bytes) per launch of each stage."""
    T, d, E, f, fs = cfg.T, cfg.d, cfg.E, cfg.f, cfg.fs
    Tr = T * cfg.top_k                          # routed rows: k picks per token
    xb, wb = esize(cfg.x_dtype), esize(cfg.w_dtype)
    hb = 4 if cfg.w_dtype == "f32" else 2
    ob = esize(cfg.out_dtype)
    touched = sum(1 for c in counts if c > 0)
    sc = 4 if cfg.w_dtype in ("e4m3", "i8", "i4") else 0     # fp32 column scales per weight column
    xin = 1 if cfg.w_dtype == "e4m3" else xb   # gate/up reads the e4m3 copy of x
    # RMSNorm in front of the block: x read, the normalised rows written (and
    # their e4m3 codes + scales for e4m3 weights), the gain read
    norm = 0
    if cfg.norm_eps is not None:
        norm = 2 * T * d * xb + d * xb + ((T * d + 4 * T) if cfg.w_dtype == "e4m3" else 0)
    return {
        "route": (2 * T * d * E, T * d * xb + d * E * xb + (4 * E if cfg.has_bias else 0) + T * 8 + norm),
        "gate_up": (4 * d * (Tr * f + T * fs),
                    touched * (d * 2 * f * wb + 2 * f * sc) + d * 2 * fs * wb + 2 * fs * sc
                    + T * d * xin + (Tr * f + T * fs) * hb),
        "down_shared": (2 * T * fs * d, fs * d * wb + d * sc + T * fs * hb + T * d * 4),
        "down_routed": (2 * Tr * f * d, touched * (f * d * wb + d * sc) + Tr * f * hb + T * d * 4 + T * d * ob
                        + (2 * Tr * d * 4 if cfg.top_k > 1 else 0)),
    }


def block_work(cfg, counts):
    """Whole-block algorithmic FLOPs and bytes (touched weights + x + out)."""
    T, d, E, f, fs = cfg.T, cfg.d, cfg.E, cfg.f, cfg.fs
    wb = esize(cfg.w_dtype)
    sc = 4 if cfg.w_dtype in ("e4m3", "i8", "i4") else 0
    touched = sum(1 for c in counts if c > 0)
    flops = 2 * T * (d * E + 3 * d * f * cfg.top_k + 3 * d * fs)
    byts = (touched * (3 * d * f * wb + (2 * f + d) * sc) + 3 * d * fs * wb + (2 * fs + d) * sc
            + d * E * esize(cfg.x_dtype) + T * d * esize(cfg.x_dtype) + T * d * esize(cfg.out_dtype))
    return flops, byts


def cpu_baseline(cfg, g, sample):
    """Time the fp64 oracle on the first `sample` tokens (weights copied per expert)."""
    import numpy as np
    import torch
    from oracle import block

    xs = g["x"][:sample].cpu()
    nw = None if g.get("norm_weight") is None else g["norm_weight"].cpu()

    def ex(e):
        s = g["s_gate_up"]
        sd = g["s_down"]
        return (g["w_gate_up"][e].cpu(), None if s is None else s[e].cpu(),
                g["w_down"][e].cpu(), None if sd is None else sd[e].cpu())

    shared = tuple(None if g[k] is None else g[k].cpu() for k in ("ws_gate_up", "ss_gate_up", "ws_down", "ss_down"))
    router = (g["w_router"].cpu(), None if g["router_bias"] is None else g["router_bias"].cpu())
    w = block.Weights(lambda: router, ex, lambda: shared)
    t0 = time.perf_counter()
    if nw is not None:
        xs = block.rmsnorm(xs, nw, float(np.float32(cfg.norm_eps)), cfg.x_dtype)
    if cfg.E == 0:
        out = block.dense(xs, w, cfg.fs, cfg.w_dtype)
        what = "dense gated MLP"
    else:
        out, r = block.forward(xs, w, cfg.f, cfg.fs, cfg.w_dtype, top_k=cfg.top_k)
        what = (f"routing + every touched expert + shared), {int(np.count_nonzero(r.counts))} experts touched")
    dt = time.perf_counter() - t0
    norm = "RMSNorm + " if nw is not None else ""
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    blas = None
    try:
        cfgd = np.show_config(mode="dicts")
        blas = cfgd.get("Build Dependencies", {}).get("blas", {}).get("name")
    except Exception:   # numpy without the dict form
        pass
    return {"value": sample / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "cpu_model": cpu_model, "blas": blas, "torch_threads": torch.get_num_threads(),
            "sample": f"first {sample} of {cfg.T} tokens, full fp64 block ({norm}{what}, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="scout_prefill_bf16")
    ap.add_argument("--cpu-sample", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--weight-sets", type=int, default=None,
                    help="independent copies of the weights the timed calls rotate over (default: 2 for "
                         "decode-sized calls, so every call streams its weights from HBM, else 1)")
    ap.add_argument("--latency-samples", type=int, default=None,
                    help="calls timed one by one with events for the median / p90 (default 50 prefill, "
                         "200 decode; 0 skips them, e.g. for profiler runs that count calls)")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the core-clock sampling bursts (for profiler runs that count calls)")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the library bf16 GEMM (torch.matmul, hipBLASLt) on the workload's dense shared-expert "
                         "shapes, for comparison with the block's own GEMM kernels, and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (reference for rocprofv3 "
                         "FETCH_SIZE / WRITE_SIZE scaling) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}))
        return
    if args.library_gemm:
        import synth
        print(json.dumps(library_gemm(synth.get_config(args.config))))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the block is measured at one "
                                   "GPU's share with no collectives; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import synth
    from sparse_moe_transformer_llama4_amd import moe

    dev = torch.device("cuda:0")
    cfg = synth.get_config(args.config)
    print(f"[bench] generating {cfg.name} on {dev}", file=sys.stderr, flush=True)
    g = synth.make_inputs(cfg, dev)
    # decode-sized calls rotate over independent weight copies (each far
    # larger than the 256 MB last-level cache), so no call finds the previous
    # call's weights in a cache
    nsets = args.weight_sets or (2 if cfg.T <= 64 else 1)
    gsets = [g] + [{k: (v if (v is None or k == "x") else v.clone()) for k, v in g.items()} for _ in range(nsets - 1)]
    torch.cuda.synchronize()
    plan = moe.Plan.for_shape(cfg)
    ws = torch.empty(max(moe.moe_workspace_size(plan, cfg.T), 256), dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.d), dtype=moe._TORCH_DT[moe._DT[cfg.out_dtype]], device=dev)
    routing = moe.new_routing(plan, cfg.T, dev) if cfg.E > 0 else None   # a dense layer routes nothing
    events = [moe.StageEvents() for _ in range(args.steps)]
    warm_ev = moe.StageEvents()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        moe.moe_forward(plan, g["x"], g, out=out, routing=routing, workspace=ws)
        moe.moe_forward_timed(plan, g["x"], g, warm_ev, out, ws, routing)
    torch.cuda.synchronize()
    counts = routing["counts"].cpu().tolist() if routing is not None else []

    # timed region 1: the library call itself (tokens/s)
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        gk = gsets[k % nsets]
        moe.moe_forward(plan, gk["x"], gk, out=out, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed / args.steps * 1e3

    # timed region 2: the same call with HIP events at the stage boundaries
    # (stages in order on one stream; decode-sized calls otherwise overlap the
    # shared expert with the routing and the routed gate/up on a side stream)
    print(f"[bench] timing {args.steps} stage-timed steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(args.steps):
        gk = gsets[k % nsets]
        moe.moe_forward_timed(plan, gk["x"], gk, events[k], out, ws, routing)
    torch.cuda.synchronize()
    ms_timed = (time.perf_counter() - t1) / args.steps * 1e3

    # per-call times (events on the caller's stream around each call): median, p90
    nlat = args.latency_samples if args.latency_samples is not None else (200 if cfg.T <= 64 else 50)
    ev_pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nlat)]
    for k, (e0, e1) in enumerate(ev_pairs):
        gk = gsets[k % nsets]
        e0.record()
        moe.moe_forward(plan, gk["x"], gk, out=out, routing=routing, workspace=ws)
        e1.record()
    torch.cuda.synchronize()
    lat = sorted(e0.elapsed_time(e1) for e0, e1 in ev_pairs)
    ms_median = lat[len(lat) // 2] if lat else None
    ms_p90 = lat[min(len(lat) - 1, int(0.9 * len(lat)))] if lat else None

    # core clock under this load (outside the timed regions): the MFMA peak
    # is quoted at 2.4 GHz, and the chip runs slower under heavy MFMA use
    import torch as _t

    def _burst():
        for _ in range(8):
            moe.moe_forward(plan, g["x"], g, out=out, routing=routing, workspace=ws)
        _t.cuda.synchronize()
    clock_mhz = None if args.no_clock else sample_clock_mhz(_burst)

    per_stage = [ev.durations_ms() for ev in events]
    avg = [sum(s[i] for s in per_stage) / len(per_stage) for i in range(moe.MOE_NUM_STAGES)]
    stage_ms = dict(zip(moe.STAGES, avg))
    work = stage_work(cfg, counts)
    dom = max(stage_ms, key=stage_ms.get)
    fl, by = work[dom]
    peak_f = PEAK[cfg.w_dtype]
    ridge = peak_f / HBM_PEAK
    t_dom = stage_ms[dom] * 1e-3
    if fl / by >= ridge:
        roof = {"bound": "mfma", "achieved": fl / t_dom / 1e12, "peak": peak_f / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": by / t_dom / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # second column: against the MFMA peak at the clock sustained under this load
    roof["clock_mhz"] = clock_mhz
    roof["frac_at_clock"] = (roof["frac"] * 2400.0 / clock_mhz
                             if clock_mhz and roof["bound"] == "mfma" else None)
    roof["kernel"] = dom
    roof["ms"] = stage_ms[dom]
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        tr = json.load(open(PROFILE_TRAFFIC)).get(cfg.name, {}).get(dom)
        if tr and tr.get("source_hash") == _kernel_source_hash():
            traffic = tr["bytes"]
    roof["traffic"] = traffic

    F, B = block_work(cfg, counts)
    t = ms * 1e-3
    result = {
        "metric": "MoE-layer tokens/s + % MFMA peak (prefill), % HBM BW (decode)",
        "value": cfg.T / t,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_per_step_stage_timed": ms_timed,
        "ms_median": ms_median,
        "ms_p90": ms_p90,
        "latency_samples": nlat,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.w_dtype,
        "data": "synthetic (seeded counter-based generator, random-init weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "f": cfg.f, "f_shared": cfg.fs,
                   "x_dtype": cfg.x_dtype, "w_dtype": cfg.w_dtype, "out_dtype": cfg.out_dtype,
                   "routing": cfg.bias, "experts_touched": sum(1 for c in counts if c > 0),
                   "rmsnorm_eps": cfg.norm_eps, "top_k": cfg.top_k, "weight_sets": nsets},
        "block_tflops": F / t / 1e12,
        "block_gbps": B / t / 1e9,
        "mfma_frac": F / t / peak_f,
        "clock_mhz": clock_mhz,
        "mfma_frac_at_clock": F / t / peak_f * 2400.0 / clock_mhz if clock_mhz else None,
        "hbm_frac": B / t / HBM_PEAK,
        "stage_ms": stage_ms,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or min(cfg.T, 4096 if cfg.E <= 16 else 512)
        print(f"[bench] cpu oracle on {sample} tokens", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(cfg, g, sample)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def sample_clock_mhz(run, seconds=0.5):
    """Mean GPU core clock (MHz) while run() keeps the GPU busy, from the active
    level the driver marks in sysfs pp_dpm_sclk (the busiest card, sampled
    every ~2 ms).  None when that file is not readable."""
    import glob
    import threading
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not paths:
        return None

    def read_mhz():
        best = None
        for path in paths:
            try:
                with open(path) as fh:
                    for line in fh:
                        if line.rstrip().endswith("*"):
                            v = float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
                            best = v if best is None else max(best, v)
            except (OSError, ValueError, IndexError):
                continue
        return best

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            v = read_mhz()
            if v is not None:
                samples.append(v)
            time.sleep(0.002)

    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        run()
    stop.set()
    th.join()
    if not samples:
        return None
    samples = samples[len(samples) // 5:]          # skip the ramp-up
    return sum(samples) / len(samples) if samples else None


def library_gemm(cfg, iters: int = 30) -> dict:
    """The library's bf16 GEMM (torch.matmul on contiguous operands) on the
    shared expert's two GEMM shapes, [T, d] x [d, 2 fs] and [T, fs] x [fs, d]:
    a reference point for the MFMA fraction, not part of the block."""
    import torch
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(0)
    out = []
    for m, k, n in ((cfg.T, cfg.d, 2 * cfg.fs), (cfg.T, cfg.fs, cfg.d)):
        a = (torch.randn(m, k, device=dev, generator=gen) * 0.05).to(torch.bfloat16).contiguous()
        b = (torch.randn(k, n, device=dev, generator=gen) * 0.05).to(torch.bfloat16).contiguous()
        for _ in range(5):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(iters):
            torch.matmul(a, b)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / iters
        tf = 2.0 * m * k * n / (ms * 1e-3) / 1e12
        out.append({"m": m, "k": k, "n": n, "us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                    "frac": round(tf * 1e12 / PEAK["bf16"], 4)})
        del a, b
    return {"library_gemm": out, "config": cfg.name, "library": "torch.matmul (hipBLASLt), bf16"}


def _kernel_source_hash() -> str:
    """Hash of the library's code (comments and whitespace left out): the
    recorded traffic is valid while this matches the hash stored with it."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_transformer_llama4_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            src = open(os.path.join(csrc, f)).read()
            src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
            src = re.sub(r"//[^\n]*", " ", src)
            h.update(f.encode() + b"\0" + " ".join(src.split()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
