"""The shared input generator: determinism, hash, distribution, recipes."""
import json
import os

import numpy as np
import pytest
import torch

import synth
from oracle import block

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "input_search.json")))


def test_mix32_tensor_matches_int():
    vals = [0, 1, 2, 0xFFFFFFFF, 0x80000000, 12345678, 0xDEADBEEF]
    rng = np.random.default_rng(0)
    vals += rng.integers(0, 2**32, 1000).tolist()
    t = synth._mix32(torch.tensor(vals, dtype=torch.int64))
    assert t.tolist() == [synth.mix32_int(v) for v in vals]
    # lowbias32 published test value: hash of 0 is 0, of 1 is nonzero and bijective on a sample
    assert synth.mix32_int(0) == 0
    s = synth._mix32(torch.arange(1 << 16, dtype=torch.int64))
    assert len(torch.unique(s)) == 1 << 16


def test_stream_slices_are_consistent():
    k = synth.stream_key(3, "x")
    a = synth.normal_fp32(k, 0, 5000, 1.0, chunk=777)
    b = synth.normal_fp32(k, 1234, 1000, 1.0)
    assert torch.equal(a[1234:2234], b)
    cfg = synth.CONFIGS["tiny_fp32"]
    x = synth.gen_x(cfg)
    assert torch.equal(synth.gen_x(cfg, rows=slice(10, 20)), x[10:20])


def test_normal_statistics():
    v = synth.normal_fp32(synth.stream_key(9, "x"), 0, 1 << 21, 0.02).double()
    assert abs(v.mean().item()) < 1e-4
    assert abs(v.std().item() / 0.02 - 1) < 5e-3
    z = v / 0.02
    # tails: P(|z|>3) ~ 0.0027
    assert abs((z.abs() > 3).double().mean().item() - 0.0027) < 4e-4
    assert z.abs().max().item() < 4.5


def test_fp8_weights_quantised_per_column():
    cfg = synth.get_config("small_fp8")
    wgu, s, wd, sd = synth.gen_expert(cfg, 1)
    assert wgu.dtype == torch.uint8 and s.shape == (2 * cfg.f,) and sd.shape == (cfg.d,)
    vals = wgu.view(torch.float8_e4m3fn).float()
    # every column reaches the largest code magnitude (scale = amax / 448)
    assert torch.all(vals.abs().amax(0) == 448.0)
    w32 = synth.normal_fp32(synth.stream_key(cfg.seed, "w_gate_up", 1), 0, cfg.d * 2 * cfg.f,
                            cfg.w_std).view(cfg.d, 2 * cfg.f)
    deq = vals * s[None, :]
    assert torch.max(torch.abs(deq - w32) / w32.abs().amax(0)[None, :]) < 2 ** -4


def test_decode_recipe_leaves_exactly_12_experts():
    cfg = synth.CONFIGS["scout_decode_bf16"]
    assert cfg.seed == GOLD["scout_decode_bf16"]["seed"]
    b = synth.gen_bias(cfg)
    assert int((b == -30).sum()) == 4 and int((b == 0).sum()) == 12
    r = block.route(synth.gen_x(cfg), synth.gen_router(cfg), b)
    assert int((r.counts > 0).sum()) == 12
    assert r.counts.tolist() == GOLD["scout_decode_bf16"]["counts"]
    assert (r.counts[b.numpy() == -30] == 0).all()


@pytest.mark.slow
def test_maverick_recipe_hot_expert_about_10x_mean():
    cfg = synth.CONFIGS["maverick_prefill_bf16"]
    assert cfg.zipf_alpha == GOLD["maverick_prefill_bf16"]["zipf_alpha"]
    r = block.route(synth.gen_x(cfg), synth.gen_router(cfg), synth.gen_bias(cfg))
    ratio = r.counts.max() / (cfg.T / cfg.E)
    assert 9.5 <= ratio <= 10.5
    assert (r.counts > 0).all()


def test_zipf_bias_shape():
    cfg = synth.CONFIGS["maverick_prefill_bf16"]
    b = synth.gen_bias(cfg).double()
    order = synth._seeded_order(cfg)
    # bias decreases along the seeded rank order
    assert all(b[order[i]] > b[order[i + 1]] for i in range(cfg.E - 1))
    p = torch.exp(b / cfg.zipf_alpha) / cfg.E
    assert abs(p.sum().item() - 1) < 1e-5


def test_configs_are_the_five_workloads():
    c = synth.CONFIGS
    assert [(v.T, v.d, v.E, v.f, v.fs) for v in c.values()] == [
        (64, 256, 4, 512, 512), (4096, 5120, 16, 8192, 8192), (32, 5120, 16, 8192, 8192),
        (8192, 5120, 128, 8192, 8192), (16384, 5120, 128, 8192, 8192)]
    assert c["maverick_prefill_fp8"].w_dtype == "e4m3" and c["maverick_prefill_fp8"].out_dtype == "bf16"


def test_int8_weights_round_trip_within_half_a_step():
    cfg = synth.MoEShape("q8", T=4, d=256, E=2, f=128, fs=128, w_dtype="i8", seed=9)
    inp = synth.make_inputs(cfg)
    assert inp["w_gate_up"].dtype == torch.int8 and inp["s_gate_up"].shape == (2, 256)
    w32 = synth.normal_fp32(synth.stream_key(cfg.seed, "w_gate_up", 1), 0, 256 * 256, cfg.w_std).view(256, 256)
    q, s = inp["w_gate_up"][1].double(), inp["s_gate_up"][1].double()
    assert (q.abs() <= 127).all() and (q.abs().amax(dim=0) == 127).all()     # each column reaches +-127
    assert ((q * s - w32.double()).abs() <= s / 2 * (1 + 1e-6)).all()


def test_int4_weights_pack_two_codes_per_byte_within_half_a_step():
    cfg = synth.MoEShape("q4", T=4, d=256, E=2, f=128, fs=128, w_dtype="i4", seed=9)
    inp = synth.make_inputs(cfg)
    assert inp["w_gate_up"].dtype == torch.uint8 and tuple(inp["w_gate_up"].shape) == (2, 128, 256)
    assert tuple(inp["w_down"].shape) == (2, 64, 256) and tuple(inp["ws_gate_up"].shape) == (128, 256)
    w32 = synth.normal_fp32(synth.stream_key(cfg.seed, "w_gate_up", 1), 0, 256 * 256, cfg.w_std).view(256, 256)
    b = inp["w_gate_up"][1].to(torch.int32)
    lo = (b & 15) - 16 * ((b & 15) >= 8).to(torch.int32)
    hi = (b >> 4) - 16 * ((b >> 4) >= 8).to(torch.int32)
    q = torch.stack([lo, hi], dim=1).reshape(256, 256).double()
    s = inp["s_gate_up"][1].double()
    assert (q.abs() <= 7).all() and (q.abs().amax(dim=0) == 7).all()
    assert ((q * s - w32.double()).abs() <= s / 2 * (1 + 1e-6)).all()
