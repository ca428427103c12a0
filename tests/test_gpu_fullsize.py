"""The workloads at full size, in the launch configuration bench.py times.

Routing is compared with the oracle on every token (bit-exact rules); the
output is compared on the first and the last token of every expert's group
(every expert, including groups that run on the tail tiles alone), plus the
middle token of the hottest group, which the oracle computes one by one.
Inputs are generated on the GPU for the HIP path; the oracle reads x and the
router from the same counter-based generator on the CPU and the expert
weights copied from the GPU expert by expert (the generator gives equal
values on both devices, test_generator_gpu_equals_cpu)."""
import gc

import numpy as np
import pytest
import torch

import synth
from oracle import block
from parity import TOL, assert_output, block_input, check_routing

pytestmark = pytest.mark.gpu


def test_generator_gpu_equals_cpu(gpu):
    for name in ("small_bf16", "small_fp8", "small_fp32", "small_bf16_bias"):
        cfg = synth.get_config(name)
        a = synth.make_inputs(cfg, "cpu")
        b = synth.make_inputs(cfg, gpu)
        for k, v in a.items():
            if v is None:
                assert b[k] is None
            else:
                assert torch.equal(v, b[k].cpu()), (name, k)
    cfg = synth.CONFIGS["maverick_prefill_fp8"]
    assert torch.equal(synth.gen_x(cfg, "cpu", rows=slice(5000, 5004)),
                       synth.gen_x(cfg, gpu, rows=slice(5000, 5004)).cpu())
    w_c = synth.gen_expert(cfg, 77, "cpu")
    w_g = synth.gen_expert(cfg, 77, gpu)
    for u, v in zip(w_c, w_g):
        assert torch.equal(u, v.cpu())
    cfg = synth.CONFIGS["maverick_prefill_bf16"]
    for u, v in zip(synth.gen_expert(cfg, 5, "cpu"), synth.gen_expert(cfg, 5, gpu)):
        assert (u is None and v is None) or torch.equal(u, v.cpu())


def group_samples(idx2: np.ndarray, E: int):
    """Tokens whose outputs are compared at full size: the first and the last
    token of every non-empty expert's group (so every expert, every group of
    at most 32 tokens that runs on the tail tiles only, and the last rows of
    groups that end in a tail tile), the middle token of the hottest group,
    and token 0.  idx2: [T, k] picks."""
    toks = {0}
    counts = np.bincount(idx2.reshape(-1), minlength=E)
    for e in np.nonzero(counts)[0]:
        grp = np.nonzero((idx2 == e).any(axis=1))[0]
        toks.update((int(grp[0]), int(grp[-1])))
        if e == int(np.argmax(counts)):
            toks.add(int(grp[len(grp) // 2]))
    return np.array(sorted(toks)), counts


def device_weights(g: dict):
    """The weights the GPU call read, copied to the host one expert at a time
    (the seeded generator gives the same values on both devices:
    test_generator_gpu_equals_cpu)."""
    def ex(e):
        s, sd = g.get("s_gate_up"), g.get("s_down")
        return (g["w_gate_up"][e].cpu(), None if s is None else s[e].cpu(),
                g["w_down"][e].cpu(), None if sd is None else sd[e].cpu())
    shared = tuple(None if g.get(k) is None else g[k].cpu()
                   for k in ("ws_gate_up", "ss_gate_up", "ws_down", "ss_down"))
    return block.Weights(lambda: None, ex, lambda: shared)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_fp32", "scout_decode_bf16", "scout_prefill_bf16",
                                  "maverick_prefill_bf16", "maverick_prefill_fp8",
                                  "scout_prefill_bf16_rmsnorm", "maverick_prefill_fp8_rmsnorm",
                                  "scout_decode_int8", "scout_decode_int4"])
def test_fullsize_sampled(gpu, name):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = synth.get_config(name)
    print(f"[full] {name}: generating on GPU", flush=True)
    g = synth.make_inputs(cfg, gpu)
    plan = moe.Plan.for_shape(cfg)
    routing = moe.new_routing(plan, cfg.T, gpu)
    ws = torch.full((moe.moe_workspace_size(plan, cfg.T),), 0xFF, dtype=torch.uint8, device=gpu)
    out = moe.moe_forward(plan, g["x"], g, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    out_cpu = out.cpu()
    routing = {k: v.cpu() for k, v in routing.items()}
    del ws, out
    torch.cuda.empty_cache()

    print(f"[full] {name}: oracle routing on all {cfg.T} tokens", flush=True)
    # the block's input: x, or its RMSNorm (computed row by row, so the
    # sampled rows below are rows of the same array)
    x = block_input(cfg, {"x": synth.gen_x(cfg, "cpu"), "norm_weight": synth.gen_norm_weight(cfg, "cpu")})
    r = block.route(x, synth.gen_router(cfg, "cpu"), synth.gen_bias(cfg))
    idx = check_routing(cfg, r, routing)
    toks, counts = group_samples(idx[:, None], cfg.E)
    print(f"[full] {name}: oracle output on {len(toks)} tokens: first and last of all "
          f"{int(np.count_nonzero(counts))} experts' groups (sizes {int(counts[counts > 0].min())}.."
          f"{int(counts.max())})", flush=True)
    gate = block.sigmoid(r.logits[toks, idx[toks]])
    ref = block.combine(x[toks], idx[toks], gate, device_weights(g), cfg.f, cfg.fs, cfg.w_dtype)
    err = assert_output(cfg, out_cpu[toks], ref)
    print(f"[full] {name}: sampled max|err|/RMS = {err:.3e} (bound {TOL[cfg.w_dtype]})", flush=True)
    assert torch.isfinite(out_cpu.float()).all()
    del g
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["maverick_dense_decode_bf16", "maverick_dense_prefill_bf16"])
def test_fullsize_dense_sampled(gpu, name):
    # Maverick's dense layers (gated MLP of width 16384, no experts) at full
    # size; the oracle computes sampled tokens one by one
    from sparse_moe_transformer_llama4_amd import moe
    cfg = synth.get_config(name)
    print(f"[full] {name}: generating on GPU", flush=True)
    g = synth.make_inputs(cfg, gpu)
    plan = moe.Plan.for_shape(cfg)
    ws = torch.full((moe.moe_workspace_size(plan, cfg.T),), 0xFF, dtype=torch.uint8, device=gpu)
    out = moe.moe_forward(plan, g["x"], g, workspace=ws)
    torch.cuda.synchronize()
    out_cpu = out.cpu()
    del g, ws, out
    gc.collect()
    torch.cuda.empty_cache()
    toks = np.array(sorted({0, 1, cfg.T // 2, cfg.T - 1}))
    print(f"[full] {name}: oracle output on tokens {toks.tolist()}", flush=True)
    x = synth.gen_x(cfg, "cpu")
    shared = synth.gen_shared(cfg, "cpu")
    w = block.Weights(lambda: None, lambda e: None, lambda: shared)
    ref = block.dense(x[toks], w, cfg.fs, cfg.w_dtype)
    err = assert_output(cfg, out_cpu[toks], ref)
    print(f"[full] {name}: sampled max|err|/RMS = {err:.3e}", flush=True)
    assert torch.isfinite(out_cpu.float()).all()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["scout_decode_bf16_top2", "scout_prefill_bf16_top2"])
def test_fullsize_topk_sampled(gpu, name):
    # two experts per token at the Scout shape: routing on every token, the
    # output on the first and last token of every expert's group, the oracle
    # evaluated on the GPU's picks
    from sparse_moe_transformer_llama4_amd import moe
    cfg = synth.get_config(name)
    print(f"[full] {name}: generating on GPU", flush=True)
    g = synth.make_inputs(cfg, gpu)
    plan = moe.Plan.for_shape(cfg)
    routing = moe.new_routing(plan, cfg.T, gpu)
    ws = torch.full((moe.moe_workspace_size(plan, cfg.T),), 0xFF, dtype=torch.uint8, device=gpu)
    out = moe.moe_forward(plan, g["x"], g, routing=routing, workspace=ws)
    torch.cuda.synchronize()
    out_cpu = out.cpu()
    routing = {k: v.cpu() for k, v in routing.items()}
    del ws, out
    torch.cuda.empty_cache()

    x = synth.gen_x(cfg, "cpu")
    r = block.route_topk(x, synth.gen_router(cfg, "cpu"), synth.gen_bias(cfg), cfg.top_k)
    idx = check_routing(cfg, r, routing)
    toks, counts = group_samples(idx, cfg.E)
    print(f"[full] {name}: oracle output on {len(toks)} tokens (every expert's first and last)", flush=True)
    gate = block.sigmoid(np.take_along_axis(r.logits[toks], idx[toks], axis=1))
    ref = block.combine_topk(x[toks], idx[toks], gate, device_weights(g), cfg.f, cfg.fs, cfg.w_dtype)
    err = assert_output(cfg, out_cpu[toks], ref)
    print(f"[full] {name}: sampled max|err|/RMS = {err:.3e}", flush=True)
    assert torch.isfinite(out_cpu.float()).all()
    del g
    gc.collect()
    torch.cuda.empty_cache()
