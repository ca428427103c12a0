"""HIP path vs the oracle, element by element, through the C ABI (needs a GPU)."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from oracle import block
from parity import assert_output, block_input, check_forward, check_routing, run_gpu, to_device

pytestmark = pytest.mark.gpu

SHAPES = ["tiny_fp32", "small_fp32", "small_bf16", "small_bf16_bias", "small_bf16_out16",
          "decode_like_bf16", "small_fp8", "small_bf16_split", "small_bf16_tall", "wide_bf16_tall"]


def _plan(cfg, **kw):
    from sparse_moe_transformer_llama4_amd import moe
    return moe.Plan.for_shape(cfg, **kw)


@pytest.mark.parametrize("name", SHAPES)
def test_forward_matches_oracle(gpu, name):
    cfg = synth.get_config(name)
    print(f"[parity] {name} T={cfg.T} d={cfg.d} E={cfg.E} f={cfg.f} fs={cfg.fs} {cfg.w_dtype}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    err, _ = check_forward(cfg, inp, out, routing)
    print(f"[parity] {name} max|err|/RMS = {err:.3e}", flush=True)


@pytest.mark.parametrize("name,over", [("small_bf16", dict(d=2560)), ("small_bf16_tall", dict(d=2304)),
                                       ("small_fp8", dict(d=2560)), ("small_bf16_tall", dict(d=2560, top_k=2)),
                                       ("small_bf16_tall", dict(d=3072)), ("small_fp8", dict(d=3072, T=1000)),
                                       ("small_bf16", dict(d=3072, top_k=3)), ("small_fp8", dict(d=1152)),
                                       ("small_fp8", dict(d=1152, T=1000))])
def test_down_ntiles_not_multiple_of_8(gpu, name, over):
    # down GEMMs with 9, 10 or 12 column tiles: whole column tiles per XCD
    # (9, 10), or (12) 4 column ranges x 2 row halves, one per XCD; and e4m3
    # with d = 1152, 4.5 column tiles of 256 (the last one half empty)
    cfg = dataclasses.replace(synth.get_config(name), name=f"{name}_d{over['d']}", **over)
    print(f"[parity] {cfg.name} T={cfg.T} d={cfg.d} {cfg.w_dtype} k={cfg.top_k}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    check_forward(cfg, inp, out, routing)


FP8_160_CASES = [dict(T=1000), dict(T=800, out_dtype="bf16"), dict(T=500, top_k=2), dict(T=1000, norm_eps=1e-5),
                 dict(T=1000, bias="cold", n_cold=0, hot=3)]


@pytest.mark.parametrize("over", FP8_160_CASES)
def test_fp8_gateup_160_row_tiles(gpu, over):
    # e4m3 with 100..125 routed rows per expert: the gate/up GEMM takes
    # 160-row tiles (one per group, or several for a hot expert); the down
    # GEMMs keep 128-row tiles
    over = dict(over)
    hot = over.pop("hot", None)
    cfg = dataclasses.replace(synth.get_config("small_fp8"), name="fp8_160", **over)
    print(f"[parity] fp8 160-row gate/up {over} hot={hot}", flush=True)
    inp = synth.make_inputs(cfg)
    if hot is not None:
        inp["router_bias"] = torch.full((cfg.E,), -60.0)
        inp["router_bias"][hot] = 60.0
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    if hot is not None:
        assert int(routing["counts"][hot]) == cfg.T
    err, _ = check_forward(cfg, inp, out, routing)
    print(f"[parity] fp8 160-row max|err|/RMS = {err:.3e}", flush=True)


@pytest.mark.parametrize("name", ["small_bf16", "small_fp32", "small_fp8"])
def test_deterministic(gpu, name):
    cfg = synth.get_config(name)
    inp = to_device(synth.make_inputs(cfg), gpu)
    p = _plan(cfg)
    o1, r1 = run_gpu(p, inp["x"], inp)
    o2, r2 = run_gpu(p, inp["x"], inp, poison_ws=False)
    assert torch.equal(o1, o2)
    for k in r1:
        assert torch.equal(r1[k], r2[k])


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 63, 64, 65, 129])
def test_ragged_token_counts(gpu, T):
    cfg = dataclasses.replace(synth.get_config("small_bf16"), T=T, name=f"ragged{T}")
    print(f"[parity] ragged T={T}", flush=True)
    inp = synth.make_inputs(cfg)
    out, routing = run_gpu(_plan(cfg), inp["x"].to(gpu), to_device(inp, gpu))
    check_forward(cfg, inp, out, routing)


def test_zero_tokens(gpu):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = synth.get_config("small_bf16")
    inp = to_device(synth.make_inputs(cfg), gpu)
    p = _plan(cfg)
    x0 = inp["x"][:0]
    routing = moe.new_routing(p, 0, gpu)
    routing["counts"].fill_(5)
    routing["offsets"].fill_(5)
    out = moe.moe_forward(p, x0, inp, routing=routing)
    torch.cuda.synchronize()
    assert out.shape == (0, cfg.d)
    assert (routing["counts"] == 0).all() and (routing["offsets"] == 0).all()


@pytest.mark.parametrize("dt", ["bf16", "f32", "e4m3"])
def test_all_tokens_to_one_expert(gpu, dt):
    base = {"bf16": "small_bf16", "f32": "small_fp32", "e4m3": "small_fp8"}[dt]
    cfg = dataclasses.replace(synth.get_config(base), bias="cold", n_cold=0)
    inp = synth.make_inputs(cfg)
    hot = cfg.E - 2
    inp["router_bias"] = torch.full((cfg.E,), -50.0)
    inp["router_bias"][hot] = 50.0
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    check_forward(cfg, inp, out, routing)
    assert int(routing["counts"][hot]) == cfg.T


@pytest.mark.parametrize("dt", ["bf16", "f32", "e4m3"])
def test_idle_experts_nan_poisoned(gpu, dt):
    base = {"bf16": "small_bf16", "f32": "small_fp32", "e4m3": "small_fp8"}[dt]
    cfg = dataclasses.replace(synth.get_config(base), bias="cold", n_cold=0)
    inp = synth.make_inputs(cfg)
    bias = torch.full((cfg.E,), -40.0)
    bias[1] = bias[3] = 0.0
    inp["router_bias"] = bias
    g = to_device(inp, gpu)
    p = _plan(cfg)
    out1, r1 = run_gpu(p, g["x"], g)
    used = set(torch.unique(r1["expert_idx"][:cfg.T]).tolist())
    assert used <= {1, 3}
    for e in range(cfg.E):
        if e not in used:
            if dt == "e4m3":
                g["w_gate_up"][e].fill_(0x7F); g["w_down"][e].fill_(0x7F)
            else:
                g["w_gate_up"][e].fill_(float("nan")); g["w_down"][e].fill_(float("nan"))
    out2, _ = run_gpu(p, g["x"], g)
    assert torch.equal(out1, out2)
    check_forward(cfg, inp, out2, r1)


def test_zero_router_gate_half_expert0(gpu):
    cfg = synth.get_config("small_bf16")
    inp = synth.make_inputs(cfg)
    inp["w_router"].zero_()
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    assert (routing["expert_idx"][:cfg.T] == 0).all()
    assert (routing["gate"][:cfg.T] == 0.5).all()
    check_forward(cfg, inp, out, routing)


def test_single_expert(gpu):
    cfg = dataclasses.replace(synth.get_config("small_bf16"), E=1, name="e1")
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    check_forward(cfg, inp, out, routing)


@pytest.mark.parametrize("case", ["w_down_swapped", "int4_unpacked", "scale_shape", "scale_missing",
                                  "bias_missing", "out_shape", "routing_short"])
def test_binding_rejects_wrong_shapes_before_the_call(gpu, case):
    # the C ABI takes bare pointers; the binding checks every tensor's shape
    # and dtype against the plan and raises before the library is called
    from sparse_moe_transformer_llama4_amd import moe
    name = {"int4_unpacked": "decode_like_bf16", "scale_shape": "small_fp8", "scale_missing": "small_fp8",
            "bias_missing": "small_bf16_bias"}.get(case, "small_bf16")
    cfg = synth.get_config(name)
    if case == "int4_unpacked":
        cfg = dataclasses.replace(cfg, w_dtype="i4")
    g = to_device(synth.make_inputs(cfg), gpu)
    p = _plan(cfg)
    out = None
    routing = None
    if case == "w_down_swapped":
        g["w_down"] = g["w_down"].transpose(1, 2).contiguous()      # [E, d, f] instead of [E, f, d]
    elif case == "int4_unpacked":
        g["w_gate_up"] = torch.zeros((cfg.E, cfg.d, 2 * cfg.f), dtype=torch.uint8, device=gpu)
    elif case == "scale_shape":
        g["s_down"] = g["s_down"][:, :-1].contiguous()
    elif case == "scale_missing":
        g["ss_down"] = None
    elif case == "bias_missing":
        g["router_bias"] = None
    elif case == "out_shape":
        out = torch.empty((cfg.T, cfg.d + 8), dtype=torch.float32, device=gpu)
    elif case == "routing_short":
        routing = moe.new_routing(p, cfg.T - 1, gpu)
    with pytest.raises(ValueError):
        moe.moe_forward(p, g["x"], g, out=out, routing=routing)


def test_route_only_entry_point(gpu):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = synth.get_config("small_bf16_bias")
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    r = moe.moe_route(_plan(cfg), g["x"], g)
    torch.cuda.synchronize()
    w = block.Weights.from_dict(inp)
    ro = block.route(inp["x"], *w.router())
    from parity import check_routing
    check_routing(cfg, ro, r)


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 31, 33, 64])
def test_decode_path_ragged(gpu, T):
    # decode-sized token counts on widths the weight-streaming kernels take
    cfg = dataclasses.replace(synth.get_config("decode_like_bf16"), T=T, name=f"decode{T}")
    print(f"[parity] decode T={T}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    check_forward(cfg, inp, out, routing)


def test_decode_path_one_hot_and_idle_nan(gpu):
    # all 40 tokens to one expert (several 16-row tiles of one group) and every
    # other expert's weights NaN
    cfg = dataclasses.replace(synth.get_config("decode_like_bf16"), T=40, bias="cold", n_cold=0, name="dec_hot")
    inp = synth.make_inputs(cfg)
    inp["router_bias"] = torch.full((cfg.E,), -60.0)
    inp["router_bias"][5] = 60.0
    g = to_device(inp, gpu)
    for e in range(cfg.E):
        if e != 5:
            g["w_gate_up"][e].fill_(float("nan")); g["w_down"][e].fill_(float("nan"))
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    assert int(routing["counts"][5]) == cfg.T
    check_forward(cfg, inp, out, routing)


@pytest.mark.parametrize("name,T,over", [("decode_like_bf16", 33, {}), ("small_bf16_split", None, {}),
                                         ("small_bf16_tall", None, {}), ("wide_bf16_tall", None, {}),
                                         ("small_fp8", None, {}), ("small_fp8", 1000, {}),
                                         ("small_fp8", None, dict(E=40)), ("small_fp8", 1000, dict(E=64))])
def test_side_stream_matches_serial_schedule(gpu, name, T, over):
    # Decode-sized bf16 calls run the shared expert's GEMMs, and prefill calls
    # the shared expert (and, bf16, the routed groups' tails) on a side
    # stream; e4m3 prefill with more than 32 experts (x quantised by its own
    # kernel, E = 40: router kernels, E = 64: router GEMM) forks before the
    # routing, its shared launches reading no tile tables.  Same kernels and arguments as the serial schedule
    # (moe_forward_timed): results must be identical bit for bit, also for
    # back-to-back calls with different inputs on a non-default stream,
    # sharing one workspace, with no host synchronisation in between (each
    # call's fork must wait for the previous call's reads of the workspace).
    from sparse_moe_transformer_llama4_amd import moe
    cfg = synth.get_config(name)
    if T is not None:
        cfg = dataclasses.replace(cfg, T=T, name=f"{name}_T{T}")
    if over:
        cfg = dataclasses.replace(cfg, name=f"{cfg.name}_E{over['E']}", **over)
    print(f"[parity] side stream {cfg.name}", flush=True)
    p = _plan(cfg)
    w = to_device(synth.make_inputs(cfg), gpu)
    xs = [w["x"], torch.roll(w["x"], 5, 0).contiguous(), (w["x"] * 0.5).contiguous(),
          torch.flip(w["x"], (0,)).contiguous()]
    ws = torch.empty(moe.moe_workspace_size(p, cfg.T), dtype=torch.uint8, device=gpu)
    odt = torch.float32 if cfg.out_dtype == "f32" else torch.bfloat16
    ev = moe.StageEvents()
    ref = []
    for x in xs:
        o = torch.empty((cfg.T, cfg.d), dtype=odt, device=gpu)
        moe.moe_forward_timed(p, x, w, ev, out=o, workspace=ws)
        torch.cuda.synchronize()
        ref.append(o.clone())
    outs = [torch.full((cfg.T, cfg.d), float("nan"), dtype=odt, device=gpu) for _ in xs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for rep in range(2):
            for x, o in zip(xs, outs):
                moe.moe_forward(p, x, w, out=o, workspace=ws, stream=s)
    s.synchronize()
    for i, (r, o) in enumerate(zip(ref, outs)):
        assert torch.equal(r, o), f"call {i}: side-stream schedule differs from the serial one"
    # and the serial result is the oracle's
    inp = synth.make_inputs(cfg)
    out, routing = run_gpu(p, w["x"], w)
    assert torch.equal(out, ref[0])
    check_forward(cfg, inp, out, routing)


def _assign_groups(inp, sizes, lift=4.0):
    """Route token t to a chosen expert: logits = x[:, :E] through an identity
    router block, with x[t, e] = lift for the chosen e and 0 for the others
    (margin = lift, gate = sigmoid(lift)).  Group sizes are exactly `sizes`."""
    E = len(sizes)
    T = inp["x"].shape[0]
    assert sum(sizes) == T
    assign = torch.repeat_interleave(torch.arange(E), torch.tensor(sizes))
    assign = assign[torch.randperm(T, generator=torch.Generator().manual_seed(5))]
    x = inp["x"].clone()
    x[:, :E] = 0
    x[torch.arange(T), assign] = lift
    inp["x"] = x.to(inp["x"].dtype)
    wr = torch.zeros_like(inp["w_router"])
    wr[torch.arange(E), torch.arange(E)] = 1
    inp["w_router"] = wr
    return assign


def test_side_stream_down_tails_wait_for_main_gateup(gpu):
    # 256-row gate/up tiles with 128-row down tiles (2200 tokens over 8
    # experts at d = 512): groups of 400, 150 and 386 rows end (n % 256 in
    # 129..160) in a down tail whose h rows a main gate/up tile writes.  The
    # side stream's tail down must wait for the main gate/up launch: compare
    # the two-stream schedule bit for bit with the serial one on a poisoned
    # workspace, several calls in a row, and the result with the oracle
    from sparse_moe_transformer_llama4_amd import moe
    cfg = synth.get_config("small_bf16_tall")
    sizes = [400, 150, 386, 280, 260, 300, 224, 200]
    inp = synth.make_inputs(cfg)
    assign = _assign_groups(inp, sizes)
    g = to_device(inp, gpu)
    p = _plan(cfg)
    ws = torch.empty(moe.moe_workspace_size(p, cfg.T), dtype=torch.uint8, device=gpu)
    ev = moe.StageEvents()
    ref = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device=gpu)
    ws.fill_(0xFF)
    moe.moe_forward_timed(p, g["x"], g, ev, out=ref, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        ws.fill_(0xFF)
        out = torch.full_like(ref, float("nan"))
        routing = moe.new_routing(p, cfg.T, gpu)
        moe.moe_forward(p, g["x"], g, out=out, routing=routing, workspace=ws)
        torch.cuda.synchronize()
        assert routing["counts"].cpu().tolist() == sizes
        assert torch.equal(out, ref), f"call {rep}: two-stream schedule differs from the serial one"
    assert (routing["expert_idx"].cpu().long() == assign).all()
    check_forward(cfg, inp, out, routing)


@pytest.mark.parametrize("k", [1, 2])
def test_class_tiles_every_size_class(gpu, k):
    # groups averaging under 192 rows take one tile height each by size
    # (1..32 rows: weight-streaming tiles, 33..128: one 128-row tile, more:
    # 256-row tiles): groups of 20, 40, 100, 128, 129, 200, 300 and 583 rows
    # (1500 tokens over 8 experts at d = 512); with k = 2 the picks spread
    # over the same classes.  Two-stream vs serial schedule bit for bit on a
    # poisoned workspace, and the oracle
    from sparse_moe_transformer_llama4_amd import moe
    # (k = 2: 750 tokens whose picks give groups of 260, 30, 60, 100, 150,
    # 220, 280 and 400 slots, 187.5 on average)
    sizes = [20, 40, 100, 128, 129, 200, 300, 583] if k == 1 else [10, 20, 40, 60, 90, 130, 150, 250]
    cfg = dataclasses.replace(synth.get_config("small_bf16_tall"), T=sum(sizes), top_k=k, name=f"classes_k{k}")
    inp = synth.make_inputs(cfg)
    assign = _assign_groups(inp, sizes)
    if k == 2:   # second pick: the next expert (its logit lifted to half the first's)
        x = inp["x"]
        x[torch.arange(cfg.T), (assign + 1) % cfg.E] = 2.0
        inp["x"] = x
    g = to_device(inp, gpu)
    p = _plan(cfg)
    ws = torch.empty(moe.moe_workspace_size(p, cfg.T), dtype=torch.uint8, device=gpu)
    ws.fill_(0xFF)
    ref = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device=gpu)
    moe.moe_forward_timed(p, g["x"], g, moe.StageEvents(), out=ref, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        ws.fill_(0xFF)
        out = torch.full_like(ref, float("nan"))
        routing = moe.new_routing(p, cfg.T, gpu)
        moe.moe_forward(p, g["x"], g, out=out, routing=routing, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"call {rep}: two-stream schedule differs from the serial one"
    if k == 1:
        assert routing["counts"].cpu().tolist() == sizes
    check_forward(cfg, inp, out, routing)


GRAPH_CASES = [("small_fp32", {}), ("small_fp8", {}), ("decode_like_bf16", {}), ("small_bf16_tall", {}),
               ("decode_like_bf16", dict(w_dtype="i8", T=33)), ("decode_like_bf16", dict(w_dtype="i4", T=33)),
               ("decode_like_bf16", dict(top_k=2, T=33)), ("small_bf16_tall", dict(top_k=2)),
               ("small_bf16_tall", dict(norm_eps=1e-5)), ("small_fp8", dict(norm_eps=1e-5, top_k=2)),
               ("small_dense_bf16", dict(T=40)), ("small_dense_bf16", dict(T=300)),
               ("small_fp8", dict(T=1000)), ("small_fp8", dict(E=40))]


@pytest.mark.parametrize("name,over", GRAPH_CASES)
def test_graph_capture_replays_match_eager(gpu, name, over):
    # moe_forward captured into a HIP graph (its side stream forks from and
    # joins the capturing stream) replays to the eager result, with eager
    # work on the GPU between the replays: every schedule, including int8 /
    # int4 weights, k picks per token, the RMSNorm in front and dense layers
    from sparse_moe_transformer_llama4_amd import moe
    cfg = dataclasses.replace(synth.get_config(name), **over)
    print(f"[parity] graph capture {name} {over}", flush=True)
    g = to_device(synth.make_inputs(cfg), gpu)
    p = _plan(cfg)
    ws = torch.empty(max(moe.moe_workspace_size(p, cfg.T), 256), dtype=torch.uint8, device=gpu)
    odt = torch.float32 if cfg.out_dtype == "f32" else torch.bfloat16
    out_e = torch.empty((cfg.T, cfg.d), dtype=odt, device=gpu)
    moe.moe_forward(p, g["x"], g, out=out_e, workspace=ws)       # eager (also creates the side stream)
    torch.cuda.synchronize()
    ref = out_e.clone()
    out_g = torch.full_like(out_e, float("nan"))
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            moe.moe_forward(p, g["x"], g, out=out_g, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        out_g.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {rep} differs from the eager call"


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,T", [("small_dense_bf16", 1), ("small_dense_bf16", 33), ("small_dense_bf16", 64),
                                     ("small_dense_bf16", 65), ("small_dense_bf16", 300), ("wide_dense_bf16", 5),
                                     ("wide_dense_bf16", 40)])
def test_dense_layer_matches_oracle(gpu, shape, T, out_dtype):
    # a dense layer (n_experts == 0): the shared gated MLP alone.  T <= 64
    # takes the weight-streaming tiles (both GEMMs split over K, partials
    # summed in order; the wide shape's down GEMM in unequal parts), larger T
    # the prefill tiles
    from parity import TOL
    from sparse_moe_transformer_llama4_amd import moe
    cfg = dataclasses.replace(synth.get_config(shape), T=T, out_dtype=out_dtype,
                              name=f"{shape}{T}_{out_dtype}")
    print(f"[parity] dense {shape} T={T} out={out_dtype}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    p = _plan(cfg)
    ws = torch.full((max(moe.moe_workspace_size(p, T), 256),), 0xFF, dtype=torch.uint8, device=gpu)
    out = moe.moe_forward(p, g["x"], g, workspace=ws)
    torch.cuda.synchronize()
    ref = block.dense(inp["x"], block.Weights.from_dict(inp), cfg.fs, cfg.w_dtype)
    err = assert_output(cfg, out, ref, TOL["bf16"])
    print(f"[parity] dense T={T} max|err|/RMS = {err:.3e}", flush=True)
    with pytest.raises(Exception):
        moe.moe_forward(p, g["x"], g, workspace=ws, routing=moe.new_routing(p, T, gpu))


# ------------------------------------------------------------ RMSNorm in front of the block

# bf16 blocks with a router and d a multiple of 128 up to 5120 take the norm
# fused with the router GEMM (E = 8, 16, 20, 32 experts; decode and prefill
# sizes); fp32 rows, dense layers and wider rows the stand-alone norm kernel,
# whose rows longer than it keeps in registers (8192 bf16 / 4096 fp32
# values) take its multi-pass path
_LONG = dict(E=2, f=128, fs=128)
NORM_CASES = [("small_bf16", None, 1e-5, {}), ("small_bf16", 65, 0.5, {}), ("small_fp32", None, 1e-5, {}),
              ("small_fp8", None, 1e-5, {}), ("small_bf16_out16", None, 1e-5, {}),
              ("decode_like_bf16", 33, 1e-5, {}), ("decode_like_bf16", 1, 1e-5, {}),
              ("small_bf16_tall", None, 1e-5, {}), ("small_dense_bf16", 33, 1e-5, {}),
              ("small_dense_bf16", 300, 1e-5, {}),
              ("small_bf16", 300, 1e-5, dict(E=20)), ("small_bf16_split", None, 1e-5, {}),
              ("small_bf16", 40, 1e-5, dict(d=8704, **_LONG)), ("small_fp32", 20, 1e-5, dict(d=4160, **_LONG)),
              ("small_fp8", 40, 1e-5, dict(d=8320, **_LONG))]


@pytest.mark.parametrize("name,T,eps,over", NORM_CASES)
def test_rmsnorm_block_matches_oracle(gpu, name, T, eps, over):
    # out = block(RMSNorm(x)) on every schedule (fp32, bf16 decode / prefill
    # with the side stream, e4m3 with the fused quantisation, dense layers);
    # x itself is left unchanged
    from parity import TOL
    from sparse_moe_transformer_llama4_amd import moe
    cfg = dataclasses.replace(synth.get_config(name), norm_eps=eps, name=f"{name}_norm", **over)
    if T is not None:
        cfg = dataclasses.replace(cfg, T=T)
    print(f"[parity] rmsnorm {cfg.name} T={cfg.T} d={cfg.d} eps={eps}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    p = _plan(cfg)
    if cfg.E == 0:
        ws = torch.full((max(moe.moe_workspace_size(p, cfg.T), 256),), 0xFF, dtype=torch.uint8, device=gpu)
        out = moe.moe_forward(p, g["x"], g, workspace=ws)
        torch.cuda.synchronize()
        ref = block.dense(block_input(cfg, inp), block.Weights.from_dict(inp), cfg.fs, cfg.w_dtype)
        err = assert_output(cfg, out, ref)
    else:
        out, routing = run_gpu(p, g["x"], g)
        err, _ = check_forward(cfg, inp, out, routing)
    print(f"[parity] rmsnorm {cfg.name} max|err|/RMS = {err:.3e}", flush=True)
    assert torch.equal(g["x"].cpu(), inp["x"])


def test_rmsnorm_route_only_and_timed_variant(gpu):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = dataclasses.replace(synth.get_config("small_bf16_tall"), norm_eps=1e-5, name="tall_norm")
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    p = _plan(cfg)
    r = moe.moe_route(p, g["x"], g)
    torch.cuda.synchronize()
    w = block.Weights.from_dict(inp)
    check_routing(cfg, block.route(block_input(cfg, inp), *w.router()), r)
    # the stage-timed variant (serial schedule, the norm inside the routing
    # stage) gives the same bits as moe_forward
    ws = torch.empty(moe.moe_workspace_size(p, cfg.T), dtype=torch.uint8, device=gpu)
    out = moe.moe_forward(p, g["x"], g, workspace=ws)
    ev = moe.StageEvents()
    out_t = torch.empty_like(out)
    moe.moe_forward_timed(p, g["x"], g, ev, out=out_t, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_t)
    ms = ev.durations_ms()
    assert all(v >= 0 for v in ms) and ms[0] > 0


# ------------------------------------------------------------ weight-only int8 (decode)

def _int8(name="decode_like_bf16", **kw):
    return dataclasses.replace(synth.get_config(name), w_dtype="i8", name=f"{name}_i8", **kw)


@pytest.mark.parametrize("T", [1, 2, 15, 16, 17, 31, 32, 33, 64])
def test_int8_decode_matches_oracle(gpu, T):
    cfg = _int8(T=T)
    print(f"[parity] int8 decode T={T}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    err, _ = check_forward(cfg, inp, out, routing)
    print(f"[parity] int8 decode T={T} max|err|/RMS = {err:.3e}", flush=True)


@pytest.mark.parametrize("over", [dict(out_dtype="bf16"), dict(d=640, f=384, fs=896, T=40),
                                  dict(norm_eps=1e-5, T=24)])
def test_int8_decode_shapes_and_options(gpu, over):
    # bf16 output; widths that leave partial 256-column tiles (d = 640) and
    # 128-column gate/up tiles (f = 384, fs = 896); the RMSNorm in front
    cfg = _int8(**over)
    print(f"[parity] int8 {over}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    check_forward(cfg, inp, out, routing)


def test_int8_one_hot_and_idle_scales_nan(gpu):
    # 40 tokens to one expert (three 16-row down tiles of one group); every
    # other expert's codes random and scales NaN: nothing of theirs is read
    cfg = _int8(T=40, bias="cold", n_cold=0)
    inp = synth.make_inputs(cfg)
    inp["router_bias"] = torch.full((cfg.E,), -60.0)
    inp["router_bias"][3] = 60.0
    g = to_device(inp, gpu)
    for e in range(cfg.E):
        if e != 3:
            g["s_gate_up"][e].fill_(float("nan")); g["s_down"][e].fill_(float("nan"))
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    assert int(routing["counts"][3]) == cfg.T
    check_forward(cfg, inp, out, routing)


def test_int8_side_stream_matches_serial_schedule(gpu):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = _int8(T=33)
    p = _plan(cfg)
    w = to_device(synth.make_inputs(cfg), gpu)
    ws = torch.empty(moe.moe_workspace_size(p, cfg.T), dtype=torch.uint8, device=gpu)
    out = moe.moe_forward(p, w["x"], w, workspace=ws)
    ev = moe.StageEvents()
    out_t = torch.empty_like(out)
    moe.moe_forward_timed(p, w["x"], w, ev, out=out_t, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_t)


# ------------------------------------------------------------ k experts per token

TOPK_CASES = [("decode_like_bf16", 33, 2), ("decode_like_bf16", 1, 4), ("decode_like_bf16", 64, 2),
              ("small_bf16", None, 2), ("small_bf16", None, 8), ("small_bf16_tall", None, 2),
              ("small_fp32", None, 3), ("small_fp8", None, 2), ("small_bf16_out16", None, 2),
              ("small_bf16_split", None, 3)]


@pytest.mark.parametrize("name,T,k", TOPK_CASES)
def test_topk_matches_oracle(gpu, name, T, k):
    # every schedule (decode with the side stream, bf16 prefill with tails and
    # the merged down launch, fp32, fp8) with k picks per token
    cfg = dataclasses.replace(synth.get_config(name), top_k=k, name=f"{name}_k{k}")
    if T is not None:
        cfg = dataclasses.replace(cfg, T=T)
    print(f"[parity] top-{k} {cfg.name} T={cfg.T}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    err, _ = check_forward(cfg, inp, out, routing)
    print(f"[parity] top-{k} {cfg.name} max|err|/RMS = {err:.3e}", flush=True)


@pytest.mark.parametrize("over", [dict(w_dtype="i8", T=33), dict(norm_eps=1e-5, T=40)])
def test_topk_int8_and_rmsnorm(gpu, over):
    cfg = dataclasses.replace(synth.get_config("decode_like_bf16"), top_k=2, name="dec_k2", **over)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    check_forward(cfg, inp, out, routing)


@pytest.mark.parametrize("name,T", [("decode_like_bf16", 33), ("small_bf16_tall", None)])
def test_topk_side_stream_matches_serial_schedule(gpu, name, T):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = dataclasses.replace(synth.get_config(name), top_k=2)
    if T is not None:
        cfg = dataclasses.replace(cfg, T=T)
    p = _plan(cfg)
    w = to_device(synth.make_inputs(cfg), gpu)
    ws = torch.empty(moe.moe_workspace_size(p, cfg.T), dtype=torch.uint8, device=gpu)
    out = moe.moe_forward(p, w["x"], w, workspace=ws)
    ev = moe.StageEvents()
    out_t = torch.empty_like(out)
    moe.moe_forward_timed(p, w["x"], w, ev, out=out_t, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_t)


def test_topk_route_only(gpu):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = dataclasses.replace(synth.get_config("small_bf16_bias"), top_k=3)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    r = moe.moe_route(_plan(cfg), g["x"], g)
    torch.cuda.synchronize()
    w = block.Weights.from_dict(inp)
    check_routing(cfg, block.route_topk(inp["x"], *w.router(), 3), r)


# ------------------------------------------------------------ weight-only int4 (decode)

def _int4(name="decode_like_bf16", **kw):
    return dataclasses.replace(synth.get_config(name), w_dtype="i4", name=f"{name}_i4", **kw)


@pytest.mark.parametrize("T", [1, 2, 16, 17, 33, 64])
def test_int4_decode_matches_oracle(gpu, T):
    cfg = _int4(T=T)
    print(f"[parity] int4 decode T={T}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    err, _ = check_forward(cfg, inp, out, routing)
    print(f"[parity] int4 decode T={T} max|err|/RMS = {err:.3e}", flush=True)


@pytest.mark.parametrize("over", [dict(out_dtype="bf16"), dict(d=768, f=512, fs=1280, T=40),
                                  dict(norm_eps=1e-5, T=24), dict(top_k=2, T=33)])
def test_int4_decode_shapes_and_options(gpu, over):
    # bf16 output; widths with a partial 256-column tile (d = 768) and
    # 128-column gate/up tiles (fs = 1280); the RMSNorm; two experts per token
    cfg = _int4(**over)
    print(f"[parity] int4 {over}", flush=True)
    inp = synth.make_inputs(cfg)
    g = to_device(inp, gpu)
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    check_forward(cfg, inp, out, routing)


def test_int4_one_hot_and_idle_scales_nan(gpu):
    cfg = _int4(T=40, bias="cold", n_cold=0)
    inp = synth.make_inputs(cfg)
    inp["router_bias"] = torch.full((cfg.E,), -60.0)
    inp["router_bias"][7] = 60.0
    g = to_device(inp, gpu)
    for e in range(cfg.E):
        if e != 7:
            g["s_gate_up"][e].fill_(float("nan")); g["s_down"][e].fill_(float("nan"))
    out, routing = run_gpu(_plan(cfg), g["x"], g)
    assert int(routing["counts"][7]) == cfg.T
    check_forward(cfg, inp, out, routing)


def test_int4_side_stream_matches_serial_schedule(gpu):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = _int4(T=33)
    p = _plan(cfg)
    w = to_device(synth.make_inputs(cfg), gpu)
    ws = torch.empty(moe.moe_workspace_size(p, cfg.T), dtype=torch.uint8, device=gpu)
    out = moe.moe_forward(p, w["x"], w, workspace=ws)
    ev = moe.StageEvents()
    out_t = torch.empty_like(out)
    moe.moe_forward_timed(p, w["x"], w, ev, out=out_t, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out_t)
