"""oracle.block pinned against brute force, special cases and invariants."""
import math

import numpy as np
import pytest
import torch

from oracle import block, brute
from oracle.numerics import e4m3_decode
import synth


def _tiny(T, d, E, f, fs, mode, seed, bias=None):
    cfg = synth.MoEShape("t", T=T, d=d, E=E, f=f, fs=fs,
                         x_dtype="f32" if mode == "f32" else "bf16",
                         w_dtype={"f32": "f32", "bf16": "bf16", "e4m3": "e4m3", "i8": "i8", "i4": "i4"}[mode],
                         out_dtype="f32", seed=seed, w_std=0.3)
    inp = synth.make_inputs(cfg)
    if bias is not None:
        inp["router_bias"] = torch.tensor(bias, dtype=torch.float32)
    return cfg, inp


def _lists(inp, E, mode=None):
    w = block.Weights.from_dict(inp)
    ex = [w.expert(e) for e in range(E)]
    sh = w.shared()
    L = lambda a: a.tolist()

    def deq(a, s):
        # int8 / int4 codes dequantised here with torch (not through oracle.block)
        if s is not None and a.dtype == torch.int8:
            return (a.double() * s.double()[None, :]).numpy()
        if s is not None and mode == "i4":
            b = a.to(torch.int32)
            lo = (b & 15) - 16 * ((b & 15) >= 8).to(torch.int32)
            hi = (b >> 4) - 16 * ((b >> 4) >= 8).to(torch.int32)
            q = torch.stack([lo, hi], dim=1).reshape(2 * b.shape[0], b.shape[1])
            return (q.double() * s.double()[None, :]).numpy()
        return block.weight_f64(a, s)
    return dict(
        x=L(block.to_f64(inp["x"])), wr=L(block.to_f64(inp["w_router"])),
        bias=None if inp["router_bias"] is None else L(block.to_f64(inp["router_bias"])),
        w_gate_up=[L(deq(a, s)) for a, s, _, _ in ex],
        w_down=[L(deq(c, sd)) for _, _, c, sd in ex],
        ws_gate_up=L(deq(sh[0], sh[1])), ws_down=L(deq(sh[2], sh[3])))


CASES = [(0, 8, 4, 8, 8, "f32"), (1, 8, 1, 4, 4, "f32"), (7, 16, 3, 8, 4, "f32"),
         (16, 8, 5, 4, 8, "f32"), (9, 16, 4, 8, 8, "bf16"), (12, 16, 2, 8, 16, "bf16"),
         (8, 16, 4, 8, 8, "e4m3"), (11, 8, 3, 4, 8, "e4m3"), (10, 16, 4, 8, 8, "i8"), (6, 8, 2, 4, 16, "i8"),
         (9, 16, 3, 8, 8, "i4"), (5, 8, 4, 4, 16, "i4")]


@pytest.mark.parametrize("T,d,E,f,fs,mode", CASES)
def test_oracle_matches_brute_force(T, d, E, f, fs, mode):
    cfg, inp = _tiny(T, d, E, f, fs, mode, seed=T * 31 + E)
    w = block.Weights.from_dict(inp)
    out, r = block.forward(inp["x"], w, f, fs, mode)
    lists = _lists(inp, E, mode)
    bo, bidx, bgate = brute.forward(lists["x"], lists["wr"], lists["bias"], lists["w_gate_up"],
                                    lists["w_down"], lists["ws_gate_up"], lists["ws_down"], f, fs, mode)
    assert out.shape == (T, d)
    if T == 0:
        return
    np.testing.assert_array_equal(r.idx, bidx)
    np.testing.assert_allclose(r.gate, bgate, rtol=1e-14)
    bo = np.array(bo)
    scale = np.sqrt(np.mean(bo * bo))
    assert np.max(np.abs(out - bo)) <= 1e-12 * scale


@pytest.mark.parametrize("T,d,fs,mode", [(0, 8, 8, "bf16"), (5, 16, 8, "bf16"), (7, 8, 16, "f32"),
                                         (3, 16, 4, "e4m3")])
def test_dense_matches_brute_force(T, d, fs, mode):
    # a dense layer: the shared gated MLP alone, token by token in plain Python
    cfg = synth.MoEShape("dense", T=T, d=d, E=0, f=0, fs=fs, x_dtype="f32" if mode == "f32" else "bf16",
                         w_dtype=mode, out_dtype="f32", seed=T * 7 + fs, w_std=0.3)
    inp = synth.make_inputs(cfg)
    assert inp["w_router"] is None and inp["w_gate_up"] is None
    w = block.Weights.from_dict(inp)
    out = block.dense(inp["x"], w, fs, mode)
    assert out.shape == (T, d)
    if T == 0:
        return
    sh = w.shared()
    wsgu = block.weight_f64(sh[0], sh[1]).tolist()
    wsd = block.weight_f64(sh[2], sh[3]).tolist()
    xin = block.expert_input(inp["x"], mode)[0].tolist() if mode == "e4m3" else block.to_f64(inp["x"]).tolist()
    bo = np.array([brute._swiglu_mlp(xin[t], wsgu, wsd, fs, mode) for t in range(T)])
    scale = np.sqrt(np.mean(bo * bo))
    assert np.max(np.abs(out - bo)) <= 1e-12 * scale
    # and it is the block with no routed token
    ref = block.combine(inp["x"], np.zeros(0, dtype=np.int64), np.zeros(0), w, 0, fs, mode)
    np.testing.assert_array_equal(out, ref)


def test_brute_force_with_bias_and_ties():
    # bias makes expert 2 win for every token; equal logits must pick the lowest index
    cfg, inp = _tiny(5, 8, 4, 4, 4, "f32", seed=3, bias=[0.0, 0.0, 50.0, 50.0])
    w = block.Weights.from_dict(inp)
    inp["w_router"].zero_()
    out, r = block.forward(inp["x"], w, 4, 4, "f32")
    assert (r.idx == 2).all()
    lists = _lists(inp, 4)
    bo, bidx, _ = brute.forward(lists["x"], lists["wr"], lists["bias"], lists["w_gate_up"],
                                lists["w_down"], lists["ws_gate_up"], lists["ws_down"], 4, 4)
    assert bidx == [2] * 5
    np.testing.assert_allclose(out, np.array(bo), rtol=0, atol=1e-14)


def _small(mode="f32", seed=5, T=40, d=32, E=4, f=16, fs=24):
    cfg = synth.MoEShape("s", T=T, d=d, E=E, f=f, fs=fs, x_dtype="f32" if mode == "f32" else "bf16",
                         w_dtype=mode, out_dtype="f32", seed=seed, w_std=0.2)
    return cfg, synth.make_inputs(cfg)


def test_s1_zero_router_goes_to_expert0_with_half_gate():
    cfg, inp = _small()
    inp["w_router"].zero_()
    w = block.Weights.from_dict(inp)
    out, r = block.forward(inp["x"], w, cfg.f, cfg.fs, "f32")
    assert (r.idx == 0).all() and (r.gate == 0.5).all()
    x = block.to_f64(inp["x"])
    wgu = block.to_f64(inp["w_gate_up"][0]); wd = block.to_f64(inp["w_down"][0])
    swgu = block.to_f64(inp["ws_gate_up"]); swd = block.to_f64(inp["ws_down"])
    silu = torch.nn.functional.silu
    def mlp(u, a, b, n):
        t = torch.from_numpy(u @ a)
        return (silu(t[:, :n]) * t[:, n:]).numpy() @ b
    ref = mlp(x, swgu, swd, cfg.fs) + mlp(x / 2, wgu, wd, cfg.f)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_s2_one_hot_bias_routes_everything_to_one_expert():
    cfg, inp = _small()
    inp["router_bias"] = torch.tensor([0, 0, 0, 1000.0])
    out, r = block.forward(inp["x"], block.Weights.from_dict(inp), cfg.f, cfg.fs, "f32")
    assert (r.idx == 3).all()
    np.testing.assert_array_equal(r.counts, [0, 0, 0, cfg.T])
    np.testing.assert_array_equal(r.offsets, [0, 0, 0, 0, cfg.T])
    np.testing.assert_array_equal(r.perm, np.arange(cfg.T))
    np.testing.assert_allclose(r.gate, 1.0)


def test_s3_zero_shared_or_zero_down_isolates_paths():
    cfg, inp = _small()
    w = block.Weights.from_dict(inp)
    full, r = block.forward(inp["x"], w, cfg.f, cfg.fs, "f32")
    a = dict(inp); a["ws_down"] = torch.zeros_like(inp["ws_down"])
    routed_only, _ = block.forward(inp["x"], block.Weights.from_dict(a), cfg.f, cfg.fs, "f32")
    b = dict(inp); b["w_down"] = torch.zeros_like(inp["w_down"])
    shared_only, _ = block.forward(inp["x"], block.Weights.from_dict(b), cfg.f, cfg.fs, "f32")
    np.testing.assert_allclose(routed_only + shared_only, full, rtol=1e-13, atol=1e-14)
    # the shared path never sees the gate: doubling the router weights changes only routed_only
    x = block.to_f64(inp["x"]); t = torch.from_numpy(x @ block.to_f64(inp["ws_gate_up"]))
    ref_shared = (torch.nn.functional.silu(t[:, :cfg.fs]) * t[:, cfg.fs:]).numpy() @ block.to_f64(inp["ws_down"])
    np.testing.assert_allclose(shared_only, ref_shared, rtol=1e-12, atol=1e-14)


def test_s4_gate_is_on_the_input_not_the_output():
    cfg, inp = _small(seed=9)
    inp["w_gate_up"] *= 4.0   # SiLU in its nonlinear range
    w = block.Weights.from_dict(inp)
    out, r = block.forward(inp["x"], w, cfg.f, cfg.fs, "f32")
    b = dict(inp); b["w_down"] = torch.zeros_like(inp["w_down"])
    shared_only, _ = block.forward(inp["x"], block.Weights.from_dict(b), cfg.f, cfg.fs, "f32")
    routed = out - shared_only
    x = block.to_f64(inp["x"])
    for t in range(cfg.T):
        e = r.idx[t]
        wgu = block.to_f64(inp["w_gate_up"][e]); wd = block.to_f64(inp["w_down"][e])
        def expert(u):
            a = torch.from_numpy(u @ wgu)
            return (torch.nn.functional.silu(a[:cfg.f]) * a[cfg.f:]).numpy() @ wd
        g = r.gate[t]
        on_input = expert(g * x[t])
        on_output = g * expert(x[t])
        np.testing.assert_allclose(routed[t], on_input, rtol=1e-11, atol=1e-13)
        # the output-gated reading is clearly different (the test discriminates)
        assert np.max(np.abs(on_output - on_input)) > 1e-3 * np.max(np.abs(on_input))


def test_s5_swiglu_form_identity_weights():
    d = f = 16
    alpha = 1.75  # exact in fp32
    cfg = synth.MoEShape("i", T=20, d=d, E=1, f=f, fs=f, x_dtype="f32", w_dtype="f32", seed=4)
    inp = synth.make_inputs(cfg)
    I = torch.eye(d)
    inp["w_router"].zero_()  # gate 0.5
    inp["w_gate_up"][0] = torch.cat([alpha * I, I], dim=1)
    inp["w_down"][0] = I
    inp["ws_gate_up"].zero_(); inp["ws_down"].zero_()
    out, r = block.forward(inp["x"], block.Weights.from_dict(inp), f, f, "f32")
    u = inp["x"].to(torch.float64) * 0.5
    ref = torch.nn.functional.silu(alpha * u) * u
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-14, atol=1e-15)
    assert np.isinf(r.margin).all()


@pytest.mark.parametrize("mode", ["f32", "bf16", "e4m3"])
def test_s6_untouched_experts_contribute_nothing(mode):
    cfg, inp = _small(mode=mode, E=6, T=30, seed=21)
    inp["router_bias"] = torch.tensor([0, 40.0, 0, 40.0, 0, 0])
    w = block.Weights.from_dict(inp)
    out, r = block.forward(inp["x"], w, cfg.f, cfg.fs, mode)
    assert set(np.unique(r.idx)) <= {1, 3}
    p = dict(inp)
    p["w_gate_up"] = inp["w_gate_up"].clone(); p["w_down"] = inp["w_down"].clone()
    for e in (0, 2, 4, 5):
        if mode == "e4m3":
            p["w_gate_up"][e] = 0x7F; p["w_down"][e] = 0x7F   # NaN codes
        else:
            p["w_gate_up"][e] = float("nan"); p["w_down"][e] = float("nan")
    out2, _ = block.forward(inp["x"], block.Weights.from_dict(p), cfg.f, cfg.fs, mode)
    np.testing.assert_array_equal(out, out2)


def test_routing_invariants_on_random_logits():
    rng = np.random.default_rng(7)
    for T, E in [(0, 3), (1, 1), (100, 7), (513, 16), (200, 128)]:
        lg = rng.standard_normal((T, E)).round(1)   # rounding creates exact ties
        idx, margin = block.top1(lg)
        counts, offsets, perm, inv = block.routing_record(idx, E)
        assert counts.sum() == T and offsets[-1] == T and (np.diff(offsets) == counts).all()
        assert sorted(perm.tolist()) == list(range(T))
        assert (inv[perm] == np.arange(T)).all()
        for e in range(E):
            grp = perm[offsets[e]:offsets[e + 1]]
            assert (idx[grp] == e).all() and (np.diff(grp) > 0).all()
        for t in range(T):  # brute-force lowest-index argmax
            best = 0
            for e in range(1, E):
                if lg[t, e] > lg[t, best]:
                    best = e
            assert idx[t] == best
            assert margin[t] >= 0


def test_rounding_point_r1_is_emulated():
    # bf16 mode differs from f32 mode exactly by the rounding of h
    cfg, inp = _small(mode="bf16", seed=33)
    w = block.Weights.from_dict(inp)
    o32, _ = block.forward(inp["x"], w, cfg.f, cfg.fs, "f32")
    o16, _ = block.forward(inp["x"], w, cfg.f, cfg.fs, "bf16")
    rel = block.rel_err(o16, o32)
    assert 1e-5 < rel < 2e-2


def test_e4m3_activation_quantisation_per_token():
    rng = np.random.default_rng(1)
    v = (rng.standard_normal((6, 50)) * rng.uniform(0.01, 100, (6, 1))).astype(np.float32)
    v[2] = 0
    q, s = block.quant_rows_e4m3(v)
    assert s[2] == 1.0 and (q[2] == 0).all()
    for t in range(6):
        amax = np.abs(v[t]).max()
        if amax:
            assert s[t] == np.float32(amax) / np.float32(448)
            codes = torch.from_numpy(np.clip(v[t] / s[t], -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
            np.testing.assert_array_equal(q[t], codes.to(torch.float64).numpy() * np.float64(s[t]))


# ------------------------------------------------------------ RMSNorm (step 0)

def test_rmsnorm_worked_example():
    # x = (3, 4): mean square 12.5, root 5 / sqrt(2); xn = (3, 4) * sqrt(2) / 5
    xn = block.rmsnorm(np.array([[3.0, 4.0]]), np.array([1.0, 1.0]), 0.0, "f32")
    np.testing.assert_allclose(xn[0], [0.848528137423857, 1.131370849898476], rtol=2 ** -24)
    # a gain scales each feature; eps sits under the root with the mean square
    xn = block.rmsnorm(np.array([[3.0, 4.0]]), np.array([2.0, -0.5]), 3.5, "f32")
    np.testing.assert_allclose(xn[0], [2 * 3 / 4.0, -0.5 * 4 / 4.0], rtol=2 ** -24)


def test_rmsnorm_constant_rows_and_gain_per_feature():
    # constant row c: xn[j] = c / sqrt(c^2 + eps) * w[j], w indexed by feature
    w = np.array([1.0, 2.0, 3.0, 4.0])
    x = np.array([[0.01] * 4, [-2.0] * 4, [5.0] * 4])
    xn = block.rmsnorm(x, w, 1e-4, "f32")
    for t, c in enumerate((0.01, -2.0, 5.0)):
        np.testing.assert_allclose(xn[t], c / np.sqrt(c * c + 1e-4) * w, rtol=2 ** -23)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 40)) * np.array([0.01, 0.3, 1, 4, 50, 1e3])[:, None]
    xn = block.rmsnorm(x, np.ones(40), 0.0, "f32")
    np.testing.assert_allclose(np.mean(xn * xn, axis=1), 1.0, rtol=1e-6)   # each row, not each column
    # powers of two commute with every step: bit-identical output
    for k in (-20, -3, 5, 30):
        np.testing.assert_array_equal(block.rmsnorm(x * 2.0 ** k, np.ones(40), 0.0, "f32"), xn)
    # with eps > 0 the mean square of the output is ms / (ms + eps) < 1
    ms = np.mean(x * x, axis=1)
    xe = block.rmsnorm(x, np.ones(40), 0.5, "f32")
    np.testing.assert_allclose(np.mean(xe * xe, axis=1), ms / (ms + 0.5), rtol=1e-6)
    # a zero row stays zero when eps > 0
    assert (block.rmsnorm(np.zeros((1, 8)), np.ones(8), 1e-5, "bf16") == 0).all()


def test_rmsnorm_brute_force_and_bf16_rounding():
    # pure-Python loops (math.fsum, math.sqrt) and the struct-based bf16
    # rounding of oracle.brute against block.rmsnorm
    import math
    from oracle import brute
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((5, 64)) * 3).to(torch.bfloat16)
    w = torch.from_numpy(1 + 0.1 * rng.standard_normal(64)).to(torch.bfloat16)
    eps = float(np.float32(1e-5))
    got = block.rmsnorm(x, w, eps, "bf16")
    xs, ws = x.double().tolist(), w.double().tolist()
    for t in range(5):
        r = 1.0 / math.sqrt(math.fsum(v * v for v in xs[t]) / 64 + eps)
        exact = [xs[t][j] * r * ws[j] for j in range(64)]
        # exact values are irrational: no float32-level tie, so brute's
        # float32-then-bf16 route equals a single rounding here
        assert got[t].tolist() == [brute._bf16(v) for v in exact]


def test_int8_weights_dequantise_to_code_times_column_scale():
    codes = torch.tensor([[-127, 0, 5], [127, -1, 64]], dtype=torch.int8)
    scale = torch.tensor([0.5, 2.0, 0.125], dtype=torch.float32)
    got = block.dequant_cols(codes, scale)
    np.testing.assert_array_equal(got, [[-63.5, 0.0, 0.625], [63.5, -2.0, 8.0]])
    # e4m3 codes (uint8) of the same bits decode differently: the dtype decides
    e4 = block.dequant_cols(codes.view(torch.uint8), torch.ones(3))
    assert not np.array_equal(e4, codes.double().numpy())
    with pytest.raises(TypeError):
        block.dequant_cols(codes.to(torch.int16), scale)


# ------------------------------------------------------------ k experts per token

@pytest.mark.parametrize("T,d,E,f,fs,mode,k", [(9, 16, 4, 8, 8, "bf16", 2), (7, 8, 5, 4, 8, "f32", 3),
                                                (6, 16, 4, 8, 8, "e4m3", 2), (5, 16, 3, 8, 8, "i8", 3),
                                                (6, 16, 4, 8, 8, "i4", 2),
                                                (8, 8, 4, 4, 4, "f32", 4)])
def test_topk_matches_brute_force(T, d, E, f, fs, mode, k):
    cfg, inp = _tiny(T, d, E, f, fs, mode, seed=T * 17 + E + k)
    w = block.Weights.from_dict(inp)
    out, r = block.forward(inp["x"], w, f, fs, mode, top_k=k)
    lists = _lists(inp, E, mode)
    bo, bidx, bgate = brute.forward(lists["x"], lists["wr"], lists["bias"], lists["w_gate_up"],
                                    lists["w_down"], lists["ws_gate_up"], lists["ws_down"], f, fs, mode, top_k=k)
    np.testing.assert_array_equal(r.idx, np.array(bidx))
    np.testing.assert_allclose(r.gate, np.array(bgate), rtol=1e-14)
    bo = np.array(bo)
    assert np.max(np.abs(out - bo)) <= 1e-12 * np.sqrt(np.mean(bo * bo))
    # the record groups the T k slots by expert, ascending within a group
    assert r.counts.sum() == T * k and (np.diff(r.offsets) == r.counts).all()
    flat = r.idx.reshape(-1)
    for e in range(E):
        grp = r.perm[r.offsets[e]:r.offsets[e + 1]]
        assert (flat[grp] == e).all() and (np.diff(grp) > 0).all()


def test_topk_order_ties_and_margin():
    lg = np.array([[1.0, 3.0, 3.0, 2.0], [0.5, 0.5, 0.5, 0.5], [4.0, 1.0, 2.0, 3.0]])
    idx, margin = block.topk(lg, 2)
    np.testing.assert_array_equal(idx, [[1, 2], [0, 1], [0, 3]])   # equal logits: lower index first
    np.testing.assert_array_equal(margin, [0.0, 0.0, 1.0])
    idx3, m3 = block.topk(lg, 3)
    np.testing.assert_array_equal(idx3, [[1, 2, 3], [0, 1, 2], [0, 3, 2]])
    idx4, m4 = block.topk(lg, 4)   # k == E: gaps among all four
    np.testing.assert_array_equal(idx4[2], [0, 3, 2, 1])
    assert m4[2] == 1.0
    # k = 1 is top1
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 7))
    i1, m1 = block.topk(lg, 1)
    t1, tm = block.top1(lg)
    np.testing.assert_array_equal(i1[:, 0], t1)
    np.testing.assert_array_equal(m1, tm)


def test_topk_with_every_expert_is_order_free():
    # k = E: every expert fires on every token with its own gate, so relabelling
    # the experts (router columns and weights together) leaves the output as is
    cfg, inp = _tiny(6, 16, 4, 8, 8, "f32", seed=5)
    w = block.Weights.from_dict(inp)
    out, r = block.forward(inp["x"], w, 8, 8, "f32", top_k=4)
    assert (r.counts == 6).all()
    p = [2, 0, 3, 1]
    inp2 = dict(inp)
    inp2["w_router"] = inp["w_router"][:, p]
    inp2["w_gate_up"] = inp["w_gate_up"][p]
    inp2["w_down"] = inp["w_down"][p]
    out2, _ = block.forward(inp2["x"], block.Weights.from_dict(inp2), 8, 8, "f32", top_k=4)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-12 * np.abs(out).max())
    # and it equals the shared expert plus every expert on its gated input
    lg = block.router_logits(inp["x"], inp["w_router"])
    g = block.sigmoid(lg)
    ref = block.combine_topk(inp["x"], np.tile(np.arange(4), (6, 1)), g, w, 8, 8, "f32")
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * np.abs(out).max())


def test_int4_codes_unpack_two_per_byte_along_k():
    # byte (i, n): low nibble = code(2i, n), high nibble = code(2i+1, n), two's complement
    packed = np.array([[0x7F, 0x89], [0x10, 0xF0]], dtype=np.uint8)
    np.testing.assert_array_equal(block.unpack_int4(packed), [[-1, -7], [7, -8], [0, 0], [1, -1]])
    got = block.dequant_cols(torch.from_numpy(packed), torch.tensor([0.5, 2.0]), "i4")
    np.testing.assert_array_equal(got, [[-0.5, -14.0], [3.5, -16.0], [0.0, 0.0], [0.5, -2.0]])
