"""Benchmark of the Llama 4 MoE feed-forward block on one MI355X.

One step = one moe_forward over one batch of synthetic tokens: router GEMM,
top-1 + sigmoid gate, histogram / scan / permutation, grouped gate/up GEMM
with the SwiGLU epilogue (routed + shared), shared down GEMM, routed down
GEMM with un-permute + combine.  Inputs are generated on the GPU by the
seeded generator before timing and stay resident in HBM.

Prints ONE JSON line (rank 0, N = 1) for the headline workload (default:
the Maverick-shaped fp8 prefill layer, T = 16384, the largest of the
workloads), with the other single-GPU workloads under "per_config":
  value       tokens/s of the whole block (timed moe_forward calls)
  kernels     every launch of the call, timed with HIP events the library
              records around each launch on the stream it goes to
              (moe_forward_traced: the same schedule and streams as
              moe_forward), with its algorithmic FLOPs / bytes and the
              fraction of its roofline
  roofline    the launch with the largest average duration (the dominant
              kernel) against the MFMA or HBM roofline, with the HBM bytes
              the rocprofv3 counters measured for it (profiles/traffic.json)
  clock_mhz   mean core clock during ~0.5 s of further moe_forward calls
              (sysfs pp_dpm_sclk); MFMA fractions at that clock beside the
              nominal ones (the quoted peaks assume 2.4 GHz)
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                       [--per-config NAMES | --no-per-config]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + % MFMA peak (prefill), % HBM BW (decode)"
HEADLINE = "maverick_prefill_fp8"
PER_CONFIG = ("scout_prefill_bf16", "scout_decode_bf16", "maverick_prefill_bf16")

# dense MFMA peak by weight dtype, FLOP/s (int8 / int4 weights are converted
# to bf16 and multiplied on the bf16 MFMA)
PEAK = {"bf16": 2516.6e12, "e4m3": 5033.2e12, "f32": 157.3e12, "i8": 2516.6e12, "i4": 2516.6e12}
HBM_PEAK = 8.0e12                                                 # bytes/s
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")


def esize(dt: str) -> float:
    return {"f32": 4, "bf16": 2, "e4m3": 1, "i8": 1, "i4": 0.5}[dt]


# ---------------------------------------------------------------- algorithmic work

def split_rows(n: int, bm: int, part: int) -> int:
    """Rows of a group of n rows that a launch covers: part 0 all of them;
    part 1 the main tiles (a last 1..32 rows past the group's full bm-row
    tiles are left to the tail tiles, so a group of at most 32 rows is all
    tail); part 2 those tail rows alone; part 3 all of them if the group's
    size class is bm (1..32 rows: 32, 33..128: 128, more: 256), else none."""
    if part == 3:
        cls = 0 if n <= 0 else 32 if n <= 32 else 128 if n <= 128 else 256
        return n if cls == bm else 0
    if part == 0 or not bm:
        return n
    r = n % bm
    tail = r if 1 <= r <= 32 else 0
    return n - tail if part == 1 else tail


def launch_work(cfg, counts, rec):
    """Algorithmic (FLOPs, bytes) of one launch of the call.  Bytes: the
    weights (+ column scales) of the experts the launch touches, read once,
    plus its activation rows read and its output rows written once."""
    name, _side, bm, groups, part = rec[:5]
    T, d, E, f, fs = cfg.T, cfg.d, cfg.E, cfg.f, cfg.fs
    k = cfg.top_k
    xb, wb, ob = esize(cfg.x_dtype), esize(cfg.w_dtype), esize(cfg.out_dtype)
    sc = 4 if cfg.w_dtype in ("e4m3", "i8", "i4") else 0
    fp8 = cfg.w_dtype == "e4m3"
    xin = 1 if fp8 else xb                    # the gate/up reads x's e4m3 codes
    hout = {"f32": 4, "e4m3": 3}.get(cfg.w_dtype, 2)   # h as the gate/up writes it (bf16; e4m3: 24 bits)
    hin = 1 if fp8 else hout                  # h as the down GEMMs read it (e4m3: its codes)
    rows = [split_rows(int(n), bm, part) for n in counts]
    R = sum(rows)
    touched = sum(1 for r in rows if r > 0)
    routed = groups in (0, 2)
    shared = groups in (1, 2)
    F = B = 0
    if name == "gateup":
        if routed:
            F += 4 * d * f * R
            B += touched * (d * 2 * f * wb + 2 * f * sc) + R * d * xin + R * f * hout + R * 4
        if shared:
            F += 4 * d * fs * T
            B += d * 2 * fs * wb + 2 * fs * sc + T * d * xin + T * fs * hout
    elif name == "down_shared":
        F = 2 * T * fs * d
        B = fs * d * wb + d * sc + T * fs * hin + T * d * 4
    elif name in ("down_routed", "down_routed_r"):
        F = 2 * R * f * d
        B = touched * (f * d * wb + d * sc) + R * f * hin
        if name == "down_routed_r" or k > 1:
            B += R * d * 4                    # fp32 rows into the workspace
        else:
            B += T * d * 4 + T * d * ob       # adds the shared output, writes out
        if shared:
            F += 2 * T * fs * d
            B += fs * d * wb + T * fs * hin + T * d * 4
    elif name in ("router", "router_gemm", "route_small"):
        F = 2 * T * d * E
        B = T * d * xb + d * E * xb
    elif name == "router_finish":
        B = T * E * 4 + T * k * 8
    elif name in ("scan", "perm", "fill"):
        B = T * k * 8
    elif name == "rmsnorm":
        B = 2 * T * d * xb + d * xb + ((T * d + 4 * T) if fp8 else 0)
    elif name == "quant_x":
        B = T * d * xb + T * d + 4 * T
    elif name == "quant_h":
        r_, n_ = (R, f) if groups == 0 else (T, fs)
        B = r_ * n_ * 3 + r_ * n_ + r_ * 8      # 24-bit h in, e4m3 codes and the row scale out
    elif name == "combine":
        B = 2 * T * d * 4 + T * d * ob
    elif name == "combine_topk":
        B = T * k * d * 4 + T * d * 4 + T * d * ob
    elif name == "swiglu_parts":
        B = T * 2 * fs * 4 + T * fs * 2
    return F, B


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


def launch_key(rec) -> str:
    """Stable name of a launch: kernel[routed|shared|both, all|main|tail, tile rows]."""
    name, side, bm, groups, part = rec[:5]
    g = {0: "routed", 1: "shared", 2: "routed+shared"}.get(groups)
    p = {0: "", 1: ",main", 2: ",tail", 3: ",class"}[part]
    inner = f"{g}{p},bm{bm}" if g else ""
    return f"{name}[{inner}]" if inner else name


def roofline_of(cfg, F, B, ms):
    t = ms * 1e-3
    peak_f = PEAK[cfg.w_dtype]
    if F > 0 and F / B >= peak_f / HBM_PEAK:
        return {"bound": "mfma", "achieved": F / t / 1e12, "peak": peak_f / 1e12, "unit": "TFLOP/s",
                "frac": F / t / peak_f}
    return {"bound": "hbm", "achieved": B / t / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": B / t / HBM_PEAK}


# ---------------------------------------------------------------- CPU oracle baseline

def cpu_baseline(cfg, g, routing_counts):
    """Time the fp64 oracle (as it stands) on the host cores.

    Small workloads run whole.  The Maverick-shaped ones (128 experts) run on
    a stratified sample: the oracle routes all T tokens, then evaluates the
    experts of 16 of the 128 groups (every 8th group in order of size, so hot
    and cold groups are both in it) on their tokens, with the shared expert
    on the same tokens.  The weights are copied to host memory before the
    clock starts.  The figure is scaled per token: the whole workload would
    take t_route + t_experts * T / n_sample."""
    import numpy as np
    import torch
    from oracle import block

    x = g["x"].cpu()
    nw = None if g.get("norm_weight") is None else g["norm_weight"].cpu()
    if cfg.E == 0:
        return cpu_baseline_dense(cfg, g, x)
    router = (g["w_router"].cpu(), None if g["router_bias"] is None else g["router_bias"].cpu())
    counts = np.asarray(routing_counts)
    if cfg.E > 16:
        order = np.argsort(-counts, kind="stable")
        experts = [int(e) for e in order[::8] if counts[e] > 0]
    else:
        experts = [int(e) for e in np.nonzero(counts)[0]]

    def host(e):
        s, sd = g.get("s_gate_up"), g.get("s_down")
        return (g["w_gate_up"][e].cpu(), None if s is None else s[e].cpu(),
                g["w_down"][e].cpu(), None if sd is None else sd[e].cpu())
    cache = {e: host(e) for e in experts}
    shared = tuple(None if g[k] is None else g[k].cpu() for k in ("ws_gate_up", "ss_gate_up", "ws_down", "ss_down"))
    w = block.Weights(lambda: router, lambda e: cache[e], lambda: shared)

    t0 = time.perf_counter()
    xs = block.rmsnorm(x, nw, float(np.float32(cfg.norm_eps)), cfg.x_dtype) if nw is not None else x
    if cfg.top_k > 1:
        r = block.route_topk(xs, *router, cfg.top_k)
        idx = r.idx
    else:
        r = block.route(xs, *router)
        idx = r.idx[:, None]
    t_route = time.perf_counter() - t0
    # the tokens all of whose picks fall in the sampled groups (all tokens
    # when every non-empty group is sampled)
    toks = np.nonzero(np.isin(idx, experts).all(axis=1))[0]
    t1 = time.perf_counter()
    sub = idx[toks]
    gate = block.sigmoid(np.take_along_axis(r.logits[toks], sub, axis=1))
    block.combine_topk(xs[toks], sub, gate, w, cfg.f, cfg.fs, cfg.w_dtype)
    t_exp = time.perf_counter() - t1
    n = len(toks)
    whole = n == cfg.T
    t_est = t_route + t_exp * (cfg.T / max(n, 1))
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    blas = None
    try:
        blas = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {}).get("name")
    except Exception:   # numpy without the dict form
        pass
    if whole:
        sample = (f"all {cfg.T} tokens, full fp64 block ({'RMSNorm + ' if nw is not None else ''}routing + "
                  f"{len(experts)} touched experts + shared), {t_route + t_exp:.1f} s")
    else:
        sample = (f"per-token-scaled stratified sample: oracle routing of all {cfg.T} tokens ({t_route:.1f} s), "
                  f"then the {n} tokens of {len(experts)} of the {cfg.E} expert groups (every 8th by size, "
                  f"{int(counts[experts].min())}..{int(counts[experts].max())} tokens each) through their "
                  f"experts and the shared expert ({t_exp:.1f} s); tokens/s = T / (t_route + t_experts * T / "
                  f"{n})")
    return {"value": cfg.T / t_est, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": sample, "cpu_model": cpu_model, "blas": blas, "torch_threads": torch.get_num_threads()}


def cpu_baseline_dense(cfg, g, x, sample=512):
    """A dense layer: the oracle's gated MLP on the first `sample` tokens."""
    import numpy as np
    import torch
    from oracle import block
    shared = tuple(None if g[k] is None else g[k].cpu() for k in ("ws_gate_up", "ss_gate_up", "ws_down", "ss_down"))
    w = block.Weights(lambda: None, lambda e: None, lambda: shared)
    n = min(cfg.T, sample)
    t0 = time.perf_counter()
    block.dense(x[:n], w, cfg.fs, cfg.w_dtype)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens through the fp64 dense gated MLP, {dt:.1f} s",
            "torch_threads": torch.get_num_threads(), "blas": None, "cpu_model": None}


# ---------------------------------------------------------------- one workload

def run_config(cfg, steps, warmup, nsets=None, latency_samples=None, clock=True, detail=True):
    import torch
    import synth
    from sparse_moe_transformer_llama4_amd import moe

    dev = torch.device("cuda:0")
    print(f"[bench] {cfg.name}: generating inputs on {dev}", file=sys.stderr, flush=True)
    g = synth.make_inputs(cfg, dev)
    # decode-sized calls rotate over independent weight copies (each far
    # larger than the 256 MB last-level cache), so no call finds the previous
    # call's weights in a cache
    nsets = nsets or (2 if cfg.T <= 64 else 1)
    gsets = [g] + [{k: (v if (v is None or k == "x") else v.clone()) for k, v in g.items()} for _ in range(nsets - 1)]
    torch.cuda.synchronize()
    plan = moe.Plan.for_shape(cfg)
    ws = torch.empty(max(moe.moe_workspace_size(plan, cfg.T), 256), dtype=torch.uint8, device=dev)
    out = torch.empty((cfg.T, cfg.d), dtype=moe._TORCH_DT[moe._DT[cfg.out_dtype]], device=dev)
    routing = moe.new_routing(plan, cfg.T, dev) if cfg.E > 0 else None   # a dense layer routes nothing
    lev = [moe.LaunchEvents() for _ in range(steps)]
    warm_ev = moe.LaunchEvents()

    print(f"[bench] {cfg.name}: warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        moe.moe_forward(plan, g["x"], g, out=out, routing=routing, workspace=ws)
        moe.moe_forward_traced(plan, g["x"], g, warm_ev, out, ws, routing)
    torch.cuda.synchronize()
    counts = routing["counts"].cpu().tolist() if routing is not None else []

    # timed region 1: the library call itself (tokens/s)
    print(f"[bench] {cfg.name}: timing {steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        gk = gsets[k % nsets]
        moe.moe_forward(plan, gk["x"], gk, out=out, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3

    # timed region 2: the same calls with an event pair around every launch
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for k in range(steps):
        gk = gsets[k % nsets]
        moe.moe_forward_traced(plan, gk["x"], gk, lev[k], out, ws, routing)
    torch.cuda.synchronize()
    ms_traced = (time.perf_counter() - t1) / steps * 1e3

    # per-call times (events on the caller's stream around each call): median, p90
    nlat = latency_samples if latency_samples is not None else (200 if cfg.T <= 64 else 50)
    ev_pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nlat)]
    for k, (e0, e1) in enumerate(ev_pairs):
        gk = gsets[k % nsets]
        e0.record()
        moe.moe_forward(plan, gk["x"], gk, out=out, routing=routing, workspace=ws)
        e1.record()
    torch.cuda.synchronize()
    lat = sorted(e0.elapsed_time(e1) for e0, e1 in ev_pairs)

    def _burst():
        for _ in range(8):
            moe.moe_forward(plan, g["x"], g, out=out, routing=routing, workspace=ws)
        torch.cuda.synchronize()
    clock_mhz = sample_clock_mhz(_burst) if clock else None

    # per-launch durations, averaged over the traced steps (the schedule is
    # the same every call)
    per = [ev.launches() for ev in lev]
    kernels = []
    for i, rec in enumerate(per[0]):
        avg = sum(p[i][5] for p in per) / len(per)
        F, B = launch_work(cfg, counts, rec)
        roof = roofline_of(cfg, F, B, avg)
        kernels.append({"launch": i, "kernel": launch_key(rec), "stream": "side" if rec[1] else "main",
                        "ms": avg, "gflop": F / 1e9, "gbytes": B / 1e9, "tflops": F / (avg * 1e-3) / 1e12,
                        "gbps": B / (avg * 1e-3) / 1e9, "bound": roof["bound"], "frac": roof["frac"]})
    dom = max(kernels, key=lambda kk: kk["ms"])
    F, B = launch_work(cfg, counts, per[0][dom["launch"]])
    roof = roofline_of(cfg, F, B, dom["ms"])
    roof["kernel"] = dom["kernel"]
    roof["ms"] = dom["ms"]
    roof["clock_mhz"] = clock_mhz
    roof["frac_at_clock"] = roof["frac"] * 2400.0 / clock_mhz if clock_mhz and roof["bound"] == "mfma" else None
    roof["traffic"] = stored_traffic(cfg.name, dom["kernel"])

    Fb, Bb = block_work(cfg, counts)
    t = ms * 1e-3
    peak_f = PEAK[cfg.w_dtype]
    res = {
        "value": cfg.T / t, "unit": "tokens/s", "ms_per_step": ms, "ms_per_step_traced": ms_traced,
        "ms_median": lat[len(lat) // 2] if lat else None,
        "ms_p90": lat[min(len(lat) - 1, int(0.9 * len(lat)))] if lat else None,
        "latency_samples": nlat,
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "f": cfg.f, "f_shared": cfg.fs,
                   "x_dtype": cfg.x_dtype, "w_dtype": cfg.w_dtype, "out_dtype": cfg.out_dtype,
                   "routing": cfg.bias, "experts_touched": sum(1 for c in counts if c > 0),
                   "rmsnorm_eps": cfg.norm_eps, "top_k": cfg.top_k, "weight_sets": nsets},
        "block_tflops": Fb / t / 1e12, "block_gbps": Bb / t / 1e9,
        "mfma_frac": Fb / t / peak_f, "hbm_frac": Bb / t / HBM_PEAK,
        "clock_mhz": clock_mhz,
        "mfma_frac_at_clock": Fb / t / peak_f * 2400.0 / clock_mhz if clock_mhz else None,
        "roofline": roof,
        "kernels": kernels if detail else [{k_: v for k_, v in kk.items() if k_ in ("kernel", "stream", "ms", "bound",
                                                                                    "frac")} for kk in kernels],
    }
    return res, g, counts


def stored_traffic(workload, kernel):
    """HBM bytes per launch measured by the rocprofv3 counters for this
    workload's kernel, while the library source is unchanged since."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    tr = json.load(open(PROFILE_TRAFFIC)).get(workload, {}).get(kernel)
    if tr and "symbol" in tr and tr.get("source_hash") == _kernel_source_hash(tr["symbol"]):
        return tr["bytes"]
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--per-config", default=None,
                    help="comma-separated workloads reported under per_config (default: the other single-GPU "
                         "workloads when --config is the headline one, none otherwise)")
    ap.add_argument("--no-per-config", action="store_true")
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
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR OUT [PATTERN]",
                    help="condense a rocprofv3 --pmc CSV directory into one line per dispatch of the kernels whose "
                         "name matches PATTERN (default: the library's) and exit")
    ap.add_argument("--record-traffic", nargs=7,
                    metavar=("KERNEL_KEY", "SYMBOL", "FETCH_SUMMARY", "WRITE_SUMMARY", "COPY_FETCH_SUMMARY",
                             "COPY_WRITE_SUMMARY", "COPY_MIB"),
                    help="store the HBM bytes per launch of --config's launch KERNEL_KEY (kernel symbol SYMBOL) "
                         "from --pmc-summary files of FETCH_SIZE and WRITE_SIZE runs, scaled by a --calibrate-copy "
                         "run's, in profiles/traffic.json, and exit")
    ap.add_argument("--trace-summary", nargs=4, metavar=("DIR", "OUT", "WARMUP", "STEPS"),
                    help="write a markdown summary of a rocprofv3 --kernel-trace --stats CSV directory of a bench.py "
                         "run made with --latency-samples 0 --no-clock and these --warmup / --steps (the library's "
                         "kernels: the --stats rows, then one call of timed region 1 launch by launch) and exit")
    args = ap.parse_args()
    if args.trace_summary:
        d, out, w, k = args.trace_summary
        print(f"{trace_summary(d, out, int(w), int(k))} library dispatches")
        return
    if args.pmc_summary:
        print(f"{pmc_summary(*args.pmc_summary)} dispatches")
        return
    if args.record_traffic:
        key, sym, fs, ws_, cfs, cws, mib = args.record_traffic
        print(json.dumps(record_traffic(args.config, key, sym, fs, ws_, cfs, cws, int(mib) << 20)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the block is measured at one "
                                   "GPU's share with no collectives (how it would shard is design only); "
                                   "--gpus must be 1"}))
        sys.exit(2)
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        # no fill: the copies are the only kernels, so the counters' copy
        # dispatches are exactly these
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 3}))
        return
    import synth
    if args.library_gemm:
        print(json.dumps(library_gemm(synth.get_config(args.config))))
        return

    import gc
    import torch
    cfg = synth.get_config(args.config)
    res, g, counts = run_config(cfg, args.steps, args.warmup, args.weight_sets, args.latency_samples,
                                clock=not args.no_clock)
    if not args.no_cpu_baseline:
        print(f"[bench] {cfg.name}: cpu oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, g, counts)
    else:
        res["cpu_baseline"] = None
    del g
    gc.collect()
    torch.cuda.empty_cache()

    if args.no_per_config:
        names = []
    elif args.per_config is not None:
        names = [n for n in args.per_config.split(",") if n]
    else:
        names = list(PER_CONFIG) if args.config == HEADLINE else []
    per_config = {cfg.name: {k: res[k] for k in ("value", "ms_per_step", "ms_median", "mfma_frac", "hbm_frac")}
                  | {"roofline": {k: res["roofline"][k] for k in ("kernel", "bound", "frac", "ms")},
                     "cpu_baseline": res["cpu_baseline"] and res["cpu_baseline"]["value"]}}
    for name in names:
        c = synth.get_config(name)
        r, g, cnt = run_config(c, max(5, args.steps // 2), args.warmup, latency_samples=20 if c.T > 64 else 100,
                               clock=False, detail=False)
        entry = {k: r[k] for k in ("value", "ms_per_step", "ms_median", "mfma_frac", "hbm_frac")}
        entry["dtype"] = c.w_dtype
        entry["roofline"] = {k: r["roofline"][k] for k in ("kernel", "bound", "frac", "ms", "traffic")}
        entry["kernels"] = r["kernels"]
        if not args.no_cpu_baseline:
            print(f"[bench] {c.name}: cpu oracle", file=sys.stderr, flush=True)
            cb = cpu_baseline(c, g, cnt)
            entry["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        per_config[name] = entry
        del g
        gc.collect()
        torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.w_dtype,
        "data": "synthetic (seeded counter-based generator, random-init weights)",
    }
    result.update({k: v for k, v in res.items() if k not in ("value", "unit", "ms_per_step")})
    result["per_config"] = per_config
    print(json.dumps(result), flush=True)


def pmc_summary(d: str, out: str, pattern: str = "moe::") -> int:
    """Condense a rocprofv3 --pmc CSV output directory into one line per
    dispatch of a kernel whose name matches `pattern` (a regular expression;
    by default the library's kernels, not the input generator's):
    'id|kernel|grid|counter=value,...' (per-dispatch values, summed over the
    counter's instances)."""
    import csv
    import glob
    import re
    rx = re.compile(pattern)
    rows = {}
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if not rx.search(r.get("Kernel_Name", "")):
                    continue
                key = (int(r.get("Dispatch_Id", 0) or 0), r.get("Kernel_Name", ""), r.get("Grid_Size", ""))
                ent = rows.setdefault(key, {})
                ent[r["Counter_Name"]] = ent.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    with open(out, "w") as fh:
        for (did, name, grid), ent in sorted(rows.items()):
            fh.write(f"{did}|{name}|{grid}|" + ",".join(f"{k}={v:.6g}" for k, v in sorted(ent.items())) + "\n")
    return len(rows)


KERNEL_ROLES = {
    "norm_route_kernel": "RMSNorm and/or e4m3 codes of x, and the router logits, per 16 rows",
    "wr_pack_kernel": "router weight into the fused kernel's layout",
    "rmsnorm_kernel": "RMSNorm of x (and its e4m3 codes)",
    "quant_x_kernel": "e4m3 codes and row scales of x",
    "quant_h_kernel": "e4m3 codes and row scales of h",
    "router_partial_kernel": "router logits, K-split partial sums",
    "router_finish_kernel": "top-k, gate, expert histograms",
    "route_small_kernel": "router for a few tokens: logits, top-k, counts, tables",
    "scan_kernel": "expert offsets and tile tables",
    "perm_kernel": "stable permutation of the routed rows",
    "combine_kernel": "out = routed rows + shared rows",
    "combine_topk_kernel": "out = gate-weighted routed rows + shared rows (top-k > 1)",
    "swiglu_parts_kernel": "SwiGLU of summed K-split gate/up partials",
    "fill_u32_kernel": "zero the per-row max |h|",
    "gemm_fp8_kernel": "e4m3 scaled-MFMA GEMM <MODE, tile rows>, 256 columns",
    "gemm_fp8_tall_kernel": "e4m3 scaled-MFMA GEMM <MODE>, 256 x 256 tiles",
    "gemm_bf16_kernel": "bf16 MFMA GEMM <MODE, tile rows, wave rows, wave columns>",
    "gemm_kernel": "bf16 MFMA GEMM (router logits / generic)",
    "gemm_decode_kernel": "weight-streaming GEMM for <= 32-row groups <MODE, 16-row fragments>",
    "gemm_decode_gateup_kernel": "weight-streaming gate/up + SwiGLU for <= 32-row groups",
    "gemm_q8_kernel": "int8 / int4 weight-streaming GEMM <MODE, 16-row fragments, code bits>",
}
MODE_NAMES = {"0": "gate/up + SwiGLU", "1": "shared down", "2": "routed down"}


def _short_kernel(name: str) -> str:
    """'void moe::(anonymous namespace)::f<1, 2>(Args)' -> 'f<1, 2>'."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):   # the argument list is the first top-level '('
        if ch in "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0 and not n[i:].startswith("(anonymous namespace)"):
            cut = i
            break
    n = n[:cut]
    return n.replace("(anonymous namespace)::", "").replace("moe::", "")


def _kernel_role(short: str) -> str:
    base = short.split("<")[0]
    role = KERNEL_ROLES.get(base, "")
    if short.startswith("gemm_bf16_kernel<1, 64,"):
        return "router logits (N = E) or a shared down of <= 64 rows: " + role
    if base.startswith("gemm_") and "<" in short:
        mode = short.split("<")[1].split(",")[0].split(">")[0].strip()
        if mode in MODE_NAMES and base != "gemm_kernel":
            role = f"{MODE_NAMES[mode]}: {role}"
    return role


def trace_summary(d: str, out: str, warmup: int, steps: int) -> int:
    """Markdown summary of a rocprofv3 --kernel-trace --stats CSV directory
    of one bench.py run (--latency-samples 0 --no-clock, so the library is
    called 2*warmup + 2*steps times: warm-up pairs of moe_forward and
    moe_forward_traced, then `steps` of each).  Lists the --stats rows of the
    library's kernels, then the launches of the last moe_forward call of
    timed region 1 with their queue, start and end."""
    import csv
    import glob
    stats = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "moe::" in r["Name"]:
                stats.append(r)
    trace = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if "moe::" in r["Kernel_Name"]:
                trace.append(r)
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    calls = 2 * warmup + 2 * steps
    if not trace or len(trace) % calls:
        raise SystemExit(f"{len(trace)} library dispatches do not split into {calls} calls")
    per = len(trace) // calls
    lines = ["| kernel | role | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        k = _short_kernel(r["Name"])
        lines.append(f"| `{k}` | {_kernel_role(k)} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    call = trace[(2 * warmup + steps - 1) * per:(2 * warmup + steps) * per]
    t0 = min(int(r["Start_Timestamp"]) for r in call)
    t1 = max(int(r["End_Timestamp"]) for r in call)
    qkey = "Stream_Id" if "Stream_Id" in call[0] else "Queue_Id"
    main_q = call[0][qkey]
    lines += ["", f"Launches of one `moe_forward` call (the last of timed region 1): {(t1 - t0) / 1e3:.1f} us "
                  f"from the first start to the last end; 'main' is the queue of the call's first launch.", "",
              "| kernel | queue | start us | end us | us |", "|---|---|---|---|---|"]
    for r in call:
        a, b = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        k = _short_kernel(r["Kernel_Name"])
        q = "main" if r[qkey] == main_q else "side"
        lines.append(f"| `{k}` | {q} | {(a - t0) / 1e3:.1f} | {(b - t0) / 1e3:.1f} | {(b - a) / 1e3:.1f} |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return len(trace)


def _read_pmc_summary(path: str):
    out = []
    for line in open(path):
        did, name, grid, vals = line.rstrip("\n").split("|", 3)
        out.append((int(did), name, grid, {k: float(v) for k, v in (kv.split("=") for kv in vals.split(",") if kv)}))
    return out


def record_traffic(workload: str, kernel: str, symbol: str, fetch_sum: str, write_sum: str, copy_fetch_sum: str,
                   copy_write_sum: str, copy_bytes: int) -> dict:
    """HBM bytes per launch of one kernel from two counter runs (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for a device-to-device copy of copy_bytes (its dispatches are the
    ones whose name mentions 'copy' or 'elementwise'); stored in
    profiles/traffic.json under the workload and the launch's key, with the
    library source hash it is valid for."""
    # SYMBOL#i/m: of the dispatches whose name contains SYMBOL, in dispatch
    # order, those at positions i, i + m, i + 2m ... (the launch's place among
    # m launches of that kernel in one call)
    sel_i, sel_m = 0, 1
    if "#" in symbol:
        symbol, sel = symbol.split("#")
        sel_i, sel_m = (int(v) for v in sel.split("/"))

    def per_dispatch(path, counter, match, pick=True):
        v = [c[counter] for _, name, _, c in _read_pmc_summary(path) if match(name) and counter in c]
        if pick:
            if len(v) % sel_m:
                raise SystemExit(f"{len(v)} dispatches of {symbol} in {path} are not calls of {sel_m}")
            v = v[sel_i::sel_m]
        if not v:
            raise SystemExit(f"no dispatch of {symbol if match is not copy_match else 'the copy'} with {counter} in {path}")
        return sum(v) / len(v), len(v)
    copy_match = lambda n: "copy" in n.lower() or "elementwise" in n.lower()
    kmatch = lambda n: symbol in n
    cf, _ = per_dispatch(copy_fetch_sum, "FETCH_SIZE", copy_match, False)
    cw, _ = per_dispatch(copy_write_sum, "WRITE_SIZE", copy_match, False)
    kf, nf = per_dispatch(fetch_sum, "FETCH_SIZE", kmatch)
    kw, nw = per_dispatch(write_sum, "WRITE_SIZE", kmatch)
    sf, sw = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    ent = {"bytes": (kf * sf + kw * sw) * 1024.0, "fetch_bytes": kf * sf * 1024.0, "write_bytes": kw * sw * 1024.0,
           "symbol": symbol, "source_hash": _kernel_source_hash(symbol),
           "note": f"{symbol} (dispatch {sel_i} of every {sel_m}): FETCH_SIZE x {sf:.3f} ({nf} dispatches) + "
                   f"WRITE_SIZE x {sw:.3f} ({nw}), factors from a "
                   f"{copy_bytes >> 20} MiB device-to-device copy"}
    data = json.load(open(PROFILE_TRAFFIC)) if os.path.exists(PROFILE_TRAFFIC) else {}
    data.setdefault(workload, {})[kernel] = ent
    with open(PROFILE_TRAFFIC, "w") as fh:
        json.dump(data, fh, indent=1)
    return ent


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


def _kernel_source_hash(symbol: str) -> str:
    """Hash of the code of the kernel `symbol` names (its function name, the
    part before any template arguments): every header of the library and each
    unit that mentions that name, comments and whitespace left out.  The
    recorded traffic is valid while this matches the hash stored with it."""
    import hashlib
    import re
    base = symbol.split("<")[0].strip()
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_transformer_llama4_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            src = open(os.path.join(csrc, f)).read()
            if f.endswith(".hip") and not re.search(r"\b" + re.escape(base) + r"\b", src):
                continue
            src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
            src = re.sub(r"//[^\n]*", " ", src)
            h.update(f.encode() + b"\0" + " ".join(src.split()).encode())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
