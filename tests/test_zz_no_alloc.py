"""moe_forward_noalloc (the entry point for callers that cannot allocate)
against moe_forward on the same inputs, through the C ABI (needs a GPU)."""
import ctypes
import dataclasses

import pytest
import torch

import synth
from parity import to_device

pytestmark = pytest.mark.gpu


def _call_noalloc(moe, plan, x, g, out, routing):
    lib = moe.load_library()
    r = moe._routing(routing)
    return lib.moe_forward_noalloc(plan.handle, moe._ptr(x), x.shape[0], ctypes.byref(moe._weights(g)),
                                   moe._ptr(out), ctypes.byref(r) if r is not None else None,
                                   moe._stream(None))


@pytest.mark.parametrize("name,over,T2", [
    ("scout_decode_bf16", {}, 7),                         # the Scout-shaped decode layer, then 7 tokens
    ("decode_like_bf16", dict(T=64, top_k=2), 33),        # k = 2 picks, 64 then 33 tokens
    ("small_bf16", dict(T=300), 129),                     # prefill tiling (256-row tiles), then 129 tokens
    ("small_fp8", dict(T=300, norm_eps=1e-5), 257),       # e4m3 weights with the RMSNorm
])
def test_noalloc_matches_moe_forward_twice(gpu, name, over, T2):
    from sparse_moe_transformer_llama4_amd import moe
    cfg = dataclasses.replace(synth.get_config(name), **over)
    print(f"[noalloc] {name} {over} T={cfg.T} then {T2}", flush=True)
    g = to_device(synth.make_inputs(cfg), gpu)
    plan = moe.Plan.for_shape(cfg)
    assert moe.moe_workspace_size(plan, cfg.T) <= moe.MOE_SCRATCH_BYTES
    odt = torch.float32 if cfg.out_dtype == "f32" else torch.bfloat16
    for T in (cfg.T, T2):          # two calls in a row, the second smaller
        x = g["x"][:T].contiguous()
        ref = moe.moe_forward(plan, x, g)
        r_ref = moe.new_routing(plan, T, gpu)
        moe.moe_forward(plan, x, g, routing=r_ref)
        out = torch.full((T, cfg.d), float("nan"), dtype=odt, device=gpu)
        routing = moe.new_routing(plan, T, gpu)
        for v in routing.values():
            v.fill_(-7 if v.dtype == torch.int32 else float("nan"))
        assert _call_noalloc(moe, plan, x, g, out, routing) == 0
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"T={T}: output differs from moe_forward"
        for k in routing:
            assert torch.equal(routing[k], r_ref[k]), f"T={T}: routing[{k}] differs"
        # without a routing record (kept in the scratch array)
        out2 = torch.full_like(out, float("nan"))
        assert _call_noalloc(moe, plan, x, g, out2, None) == 0
        torch.cuda.synchronize()
        assert torch.equal(out2, ref)


def test_noalloc_rejects_calls_beyond_its_scratch(gpu):
    # the Scout-shaped prefill layer (4096 tokens) needs far more than the
    # scratch array holds: rejected before anything is enqueued
    from sparse_moe_transformer_llama4_amd import moe
    cfg = synth.get_config("scout_prefill_bf16")
    plan = moe.Plan.for_shape(cfg)
    assert moe.moe_workspace_size(plan, cfg.T) > moe.MOE_SCRATCH_BYTES
    lib = moe.load_library()
    P = 1 << 20
    w = moe._Weights(*([P] * 11))
    assert lib.moe_forward_noalloc(plan.handle, P, cfg.T, ctypes.byref(w), P, None, None) == -4
