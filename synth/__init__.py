"""Seeded synthetic inputs for the Llama 4 MoE feed-forward block.

This module is the one piece shared by the CPU oracle and the GPU path: it
draws the block's *inputs* (token activations, router weights and bias,
expert and shared-expert weights, fp8 weight codes with their scales) and
nothing else.  It holds none of the block's arithmetic: no router, no
selection, no gate, no SwiGLU, no activation quantisation.

Generator (counter-based, identical on CPU and GPU):
  * key     = lowbias32 chain over (seed, stream id, expert index), computed
              with Python integers on the host;
  * counter = flat row-major element index inside one tensor slice (< 2**32);
  * u       = lowbias32(lowbias32(counter XOR key) + 0x9E3779B9) -- the
              32-bit integer hash "lowbias32" published by C. Wellons
              (hash-prospector); every step is exact 32-bit integer math
              carried in int64 torch tensors, so CPU and GPU agree bit for bit;
  * value   = Q[u >> 16] * std, where Q[i] is the standard-normal quantile at
              (i + 0.5) / 65536 (65536-level discretised N(0,1), tails cut at
              about 4.3 sigma), the product taken in fp32, then rounded to
              the storage dtype with torch's round-to-nearest-even casts.

fp8 weights (OCP e4m3fn) are drawn in fp32 the same way and quantised per
output column of the [K, N] layout: scale = amax over K / 448 (fp32), code =
torch's float8_e4m3fn cast of clamp(w / scale, -448, 448).  int8 weights
likewise: scale = amax over K / 127, code = round-half-even(w / scale); int4
with 7 in place of 127, two codes per byte along K (low nibble = even row).

Workloads with the RMSNorm in front of the block (norm_eps set) also draw its
gain, w[j] = 1 + 0.1 * Q (fp32, then rounded to x's dtype), and give every
token row its own scale, x[t, :] *= 0.25 + |Q_t| (fp32, from a stream of its
own), so that rows differ in RMS as the residual stream's rows do.
"""
from __future__ import annotations

import dataclasses
import math
import statistics
from typing import Optional

import torch

__all__ = [
    "MoEShape", "CONFIGS", "TEST_SHAPES", "get_config", "mix32_int",
    "normal_fp32", "gen_x", "gen_router", "gen_bias", "gen_expert",
    "gen_shared", "gen_norm_weight", "make_inputs", "DTYPES",
]

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.float8_e4m3fn, "i8": torch.int8,
          "i4": torch.uint8}

# ---------------------------------------------------------------- configs


@dataclasses.dataclass(frozen=True)
class MoEShape:
    """Shape, dtypes and input recipe of one MoE-block workload."""
    name: str
    T: int                 # tokens (batch * seq)
    d: int                 # model width (embed_dim / hidden_size)
    E: int                 # routed experts
    f: int                 # routed SwiGLU width
    fs: int                # shared SwiGLU width
    x_dtype: str = "bf16"  # activations and router weight dtype
    w_dtype: str = "bf16"  # expert / shared weight dtype ("e4m3" = fp8, "i8" = int8, + fp32 scales)
    out_dtype: str = "f32"
    bias: str = "none"     # "none" | "cold" (4 experts at -30) | "zipf"
    n_cold: int = 4
    zipf_s: float = 1.1
    zipf_alpha: float = 0.0
    seed: int = 0
    x_std: float = 1.0
    w_std: float = 0.02
    norm_eps: Optional[float] = None   # RMSNorm in front of the block (None = none)
    top_k: int = 1         # experts per token

    @property
    def has_bias(self) -> bool:
        return self.bias != "none"


# The five named workloads.  The decode seed and the Zipf strength were
# searched by tests/golden/search_inputs.py (which calls only the oracle) so
# that exactly 12 of 16 experts receive tokens, resp. the hottest expert
# receives about 10x the mean load; tests/test_synth.py re-checks both.
CONFIGS = {
    "tiny_fp32": MoEShape("tiny_fp32", T=64, d=256, E=4, f=512, fs=512,
                          x_dtype="f32", w_dtype="f32", out_dtype="f32", seed=0),
    "scout_prefill_bf16": MoEShape("scout_prefill_bf16", T=4096, d=5120, E=16, f=8192, fs=8192,
                                   seed=1),
    "scout_decode_bf16": MoEShape("scout_decode_bf16", T=32, d=5120, E=16, f=8192, fs=8192,
                                  bias="cold", seed=2),
    "maverick_prefill_bf16": MoEShape("maverick_prefill_bf16", T=8192, d=5120, E=128, f=8192,
                                      fs=8192, bias="zipf", zipf_alpha=0.40, seed=3),
    "maverick_prefill_fp8": MoEShape("maverick_prefill_fp8", T=16384, d=5120, E=128, f=8192,
                                     fs=8192, w_dtype="e4m3", out_dtype="bf16", seed=4),
}

# Workloads beyond the five: Maverick's dense layers (every other layer: a
# gated MLP of width d_ff = 16384, no experts), prefill and decode.
EXTRA_CONFIGS = {
    "maverick_dense_prefill_bf16": MoEShape("maverick_dense_prefill_bf16", T=8192, d=5120, E=0, f=0,
                                            fs=16384, seed=5),
    "maverick_dense_decode_bf16": MoEShape("maverick_dense_decode_bf16", T=32, d=5120, E=0, f=0,
                                           fs=16384, seed=6),
    # the MoE layer with the RMSNorm that precedes it (eps 1e-5)
    "scout_prefill_bf16_rmsnorm": MoEShape("scout_prefill_bf16_rmsnorm", T=4096, d=5120, E=16, f=8192,
                                           fs=8192, seed=7, norm_eps=1e-5),
    "scout_decode_int4": MoEShape("scout_decode_int4", T=32, d=5120, E=16, f=8192, fs=8192, w_dtype="i4",
                                  bias="cold", seed=2),
    # weight-only int8 decode on the Scout-shaped layer (the bf16 decode
    # workload's seed and routing)
    "scout_decode_int8": MoEShape("scout_decode_int8", T=32, d=5120, E=16, f=8192, fs=8192, w_dtype="i8",
                                  bias="cold", seed=2),
    # two experts per token on the Scout-shaped layer (prefill and decode)
    "scout_prefill_bf16_top2": MoEShape("scout_prefill_bf16_top2", T=4096, d=5120, E=16, f=8192, fs=8192,
                                        seed=9, top_k=2),
    "scout_decode_bf16_top2": MoEShape("scout_decode_bf16_top2", T=32, d=5120, E=16, f=8192, fs=8192,
                                       seed=10, top_k=2),
    "maverick_prefill_fp8_rmsnorm": MoEShape("maverick_prefill_fp8_rmsnorm", T=16384, d=5120, E=128,
                                             f=8192, fs=8192, w_dtype="e4m3", out_dtype="bf16", seed=8,
                                             norm_eps=1e-5),
}

# Smaller shapes for element-by-element parity: several tiles in every
# dimension plus ragged tails, small enough for the fp64 oracle in seconds.
TEST_SHAPES = {
    "small_fp32": MoEShape("small_fp32", T=300, d=320, E=5, f=192, fs=256,
                           x_dtype="f32", w_dtype="f32", out_dtype="f32", seed=11),
    "small_bf16": MoEShape("small_bf16", T=777, d=512, E=8, f=384, fs=320, seed=12),
    "small_bf16_bias": MoEShape("small_bf16_bias", T=1000, d=640, E=16, f=256, fs=512,
                                bias="zipf", zipf_alpha=0.6, seed=13),
    "small_bf16_out16": MoEShape("small_bf16_out16", T=257, d=256, E=4, f=128, fs=192,
                                 out_dtype="bf16", seed=14),
    "small_fp8": MoEShape("small_fp8", T=650, d=1024, E=8, f=8192, fs=8064,
                          w_dtype="e4m3", out_dtype="bf16", seed=15),
    "decode_like_bf16": MoEShape("decode_like_bf16", T=32, d=1024, E=16, f=512, fs=512,
                                 bias="cold", seed=16),
    # skewed routing over 32 experts: 25 groups of 1..32 tokens (6 of them
    # 17..32) next to 7 larger ones; f == fs (one down launch for the routed
    # main tiles and the shared expert)
    "small_bf16_split": MoEShape("small_bf16_split", T=1200, d=512, E=32, f=384, fs=384,
                                 bias="zipf", zipf_alpha=0.3, seed=17),
    # ~275 tokens per expert (256-row routed tiles): four groups end in a
    # 3..27-row tail past a full 256-row tile, two in a 38- / 50-row one;
    # f == fs
    "small_bf16_tall": MoEShape("small_bf16_tall", T=2200, d=512, E=8, f=384, fs=384, seed=22),
    # a dense layer (no routed experts): the shared gated MLP alone
    "small_dense_bf16": MoEShape("small_dense_bf16", T=300, d=512, E=0, f=0, fs=384, seed=24),
    # a wider dense layer at decode sizes: d / 128 = 16 column tiles, so both
    # GEMMs split K (the down GEMM into 8 parts over 10 units of 128 rows)
    "wide_dense_bf16": MoEShape("wide_dense_bf16", T=40, d=2048, E=0, f=0, fs=1280, seed=25),
    # Scout-like tiling at a narrow f: d = 5120 and ~512 tokens per expert give
    # 256-row routed and down tiles, so the routed main tiles and the shared
    # expert share one down launch (f == fs)
    "wide_bf16_tall": MoEShape("wide_bf16_tall", T=4096, d=5120, E=8, f=256, fs=256, seed=23),
}


def get_config(name: str) -> MoEShape:
    if name in CONFIGS:
        return CONFIGS[name]
    if name in EXTRA_CONFIGS:
        return EXTRA_CONFIGS[name]
    return TEST_SHAPES[name]


# ---------------------------------------------------------------- generator

_M32 = 0xFFFFFFFF
_GOLDEN = 0x9E3779B9
_C1 = 0x7FEB352D
_C2 = 0x846CA68B

STREAMS = {"x": 1, "w_router": 2, "bias": 3, "w_gate_up": 4, "w_down": 5,
           "ws_gate_up": 6, "ws_down": 7, "norm_weight": 8, "x_row_scale": 9}


def mix32_int(x: int) -> int:
    """lowbias32 on a Python int (host-side keys and tests)."""
    x &= _M32
    x ^= x >> 16
    x = (x * _C1) & _M32
    x ^= x >> 15
    x = (x * _C2) & _M32
    x ^= x >> 16
    return x


def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    # (x * c) mod 2**32 for int64 x in [0, 2**32) without int64 overflow:
    # split x into 16-bit halves; every partial product stays below 2**49.
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & _M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, _C1)
    x = x ^ (x >> 15)
    x = _mul32(x, _C2)
    x = x ^ (x >> 16)
    return x


def stream_key(seed: int, stream: str, expert: int = 0) -> int:
    k = mix32_int(seed * 2654435761 + 12345)
    k = mix32_int(k ^ STREAMS[stream])
    return mix32_int(k ^ (expert * 0x85EBCA6B + 0x27D4EB2F))


_QTAB: dict = {}


def _quantile_table(device) -> torch.Tensor:
    dev = torch.device(device)
    key = str(dev)
    if key not in _QTAB:
        if "cpu" not in _QTAB:
            nd = statistics.NormalDist(0.0, 1.0)
            vals = [nd.inv_cdf((i + 0.5) / 65536.0) for i in range(65536)]
            _QTAB["cpu"] = torch.tensor(vals, dtype=torch.float64).to(torch.float32)
        _QTAB[key] = _QTAB["cpu"].to(dev)
    return _QTAB[key]


def normal_fp32(key: int, start: int, count: int, std: float, device="cpu",
                chunk: int = 1 << 24) -> torch.Tensor:
    """Elements [start, start+count) of the stream `key` as fp32 N(0, std)."""
    if start < 0 or start + count > (1 << 32):
        raise ValueError("stream counter out of range")
    dev = torch.device(device)
    tab = _quantile_table(dev)
    out = torch.empty(count, dtype=torch.float32, device=dev)
    stdv = torch.tensor(std, dtype=torch.float32, device=dev)
    for c0 in range(0, count, chunk):
        n = min(chunk, count - c0)
        i = torch.arange(start + c0, start + c0 + n, dtype=torch.int64, device=dev)
        u = _mix32(i ^ key)
        u = _mix32((u + _GOLDEN) & _M32)
        out[c0:c0 + n] = tab[u >> 16] * stdv
    return out


def _round_to(w32: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return w32
    if dtype == "bf16":
        return w32.to(torch.bfloat16)
    raise ValueError(dtype)


def _quant_cols_e4m3(w32: torch.Tensor):
    """[K, N] fp32 -> (e4m3 codes as uint8 [K, N], fp32 scale [N])."""
    amax = w32.abs().amax(dim=0)
    scale = amax / torch.tensor(448.0, dtype=torch.float32, device=w32.device)
    scale = torch.where(amax > 0, scale, torch.ones_like(scale))
    q = (w32 / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale


def gen_x(cfg: MoEShape, device="cpu", rows: Optional[slice] = None) -> torch.Tensor:
    """Token activations x [T, d] in cfg.x_dtype (rows: optional row slice)."""
    r0, r1 = (0, cfg.T) if rows is None else (rows.start or 0, rows.stop)
    key = stream_key(cfg.seed, "x")
    v = normal_fp32(key, r0 * cfg.d, (r1 - r0) * cfg.d, cfg.x_std, device).view(r1 - r0, cfg.d)
    if cfg.norm_eps is not None:   # per-row scales 0.25 + |Q_t|
        q = normal_fp32(stream_key(cfg.seed, "x_row_scale"), r0, r1 - r0, 1.0, device)
        v = v * (q.abs() + torch.tensor(0.25, dtype=torch.float32, device=v.device))[:, None]
    return _round_to(v, cfg.x_dtype)


def gen_norm_weight(cfg: MoEShape, device="cpu") -> Optional[torch.Tensor]:
    """RMSNorm gain [d] in cfg.x_dtype, 1 + 0.1 * Q (None without a norm)."""
    if cfg.norm_eps is None:
        return None
    v = normal_fp32(stream_key(cfg.seed, "norm_weight"), 0, cfg.d, 0.1, device)
    return _round_to(v + torch.tensor(1.0, dtype=torch.float32, device=v.device), cfg.x_dtype)


def gen_router(cfg: MoEShape, device="cpu") -> torch.Tensor:
    """Router weight [d, E] in cfg.x_dtype."""
    v = normal_fp32(stream_key(cfg.seed, "w_router"), 0, cfg.d * cfg.E, cfg.w_std, device)
    return _round_to(v, cfg.x_dtype).view(cfg.d, cfg.E)


def _seeded_order(cfg: MoEShape):
    keys = [mix32_int(stream_key(cfg.seed, "bias") ^ mix32_int(e + 1)) for e in range(cfg.E)]
    return sorted(range(cfg.E), key=lambda e: (keys[e], e))


def gen_bias(cfg: MoEShape) -> Optional[torch.Tensor]:
    """Per-expert router bias fp32 [E] (None when the workload has none).

    "cold": the first n_cold experts of a seeded order get -30, the rest 0.
    "zipf": rank r_e (1-based, seeded order) gives p_e ~ r_e**-s and
            b_e = alpha * ln(E * p_e), p normalised to sum 1.
    """
    if cfg.bias == "none":
        return None
    order = _seeded_order(cfg)
    b = [0.0] * cfg.E
    if cfg.bias == "cold":
        for e in order[:cfg.n_cold]:
            b[e] = -30.0
    elif cfg.bias == "zipf":
        w = [0.0] * cfg.E
        for rank, e in enumerate(order, start=1):
            w[e] = rank ** (-cfg.zipf_s)
        z = sum(w)
        b = [cfg.zipf_alpha * math.log(cfg.E * wi / z) for wi in w]
    else:
        raise ValueError(cfg.bias)
    return torch.tensor(b, dtype=torch.float64).to(torch.float32)


def _quant_cols_int8(w32: torch.Tensor):
    """[K, N] fp32 -> (int8 codes [K, N] in -127..127, fp32 scale [N]):
    scale = amax over K / 127, code = round-half-even(w / scale)."""
    amax = w32.abs().amax(dim=0)
    scale = amax / torch.tensor(127.0, dtype=torch.float32, device=w32.device)
    scale = torch.where(amax > 0, scale, torch.ones_like(scale))
    q = torch.round(w32 / scale).clamp_(-127.0, 127.0).to(torch.int8)
    return q, scale


def _quant_cols_int4(w32: torch.Tensor):
    """[K, N] fp32 -> (int4 codes packed along K as uint8 [K/2, N], fp32 scale [N]):
    scale = amax over K / 7, code = round-half-even(w / scale) in -7..7, byte
    (i, n) = code(2i, n) & 15 | (code(2i+1, n) & 15) << 4."""
    amax = w32.abs().amax(dim=0)
    scale = amax / torch.tensor(7.0, dtype=torch.float32, device=w32.device)
    scale = torch.where(amax > 0, scale, torch.ones_like(scale))
    q = torch.round(w32 / scale).clamp_(-7.0, 7.0).to(torch.int32)
    packed = (q[0::2] & 15) | ((q[1::2] & 15) << 4)
    return packed.to(torch.uint8), scale


def _gen_matrix(cfg: MoEShape, stream: str, expert: int, K: int, N: int, device):
    v = normal_fp32(stream_key(cfg.seed, stream, expert), 0, K * N, cfg.w_std, device).view(K, N)
    if cfg.w_dtype == "e4m3":
        return _quant_cols_e4m3(v)
    if cfg.w_dtype == "i8":
        return _quant_cols_int8(v)
    if cfg.w_dtype == "i4":
        return _quant_cols_int4(v)
    return _round_to(v, cfg.w_dtype), None


def gen_expert(cfg: MoEShape, e: int, device="cpu"):
    """Routed expert e: (w_gate_up [d,2f], s_gate_up [2f] | None, w_down [f,d], s_down [d] | None).

    Columns [0, f) of w_gate_up feed the SiLU branch, [f, 2f) the linear branch.
    e4m3 weights come back as uint8 codes.
    """
    wgu, sgu = _gen_matrix(cfg, "w_gate_up", e, cfg.d, 2 * cfg.f, device)
    wd, sd = _gen_matrix(cfg, "w_down", e, cfg.f, cfg.d, device)
    return wgu, sgu, wd, sd


def gen_shared(cfg: MoEShape, device="cpu"):
    """Shared expert: (ws_gate_up [d,2fs], ss_gate_up, ws_down [fs,d], ss_down)."""
    wgu, sgu = _gen_matrix(cfg, "ws_gate_up", 0, cfg.d, 2 * cfg.fs, device)
    wd, sd = _gen_matrix(cfg, "ws_down", 0, cfg.fs, cfg.d, device)
    return wgu, sgu, wd, sd


def make_inputs(cfg: MoEShape, device="cpu") -> dict:
    """Every input of the block, materialised on `device`.

    Expert stacks are filled one expert at a time so the temporaries stay
    at one expert's size.
    """
    dev = torch.device(device)
    wdt = torch.uint8 if cfg.w_dtype == "e4m3" else DTYPES[cfg.w_dtype]
    scaled = cfg.w_dtype in ("e4m3", "i8", "i4")
    kd = 2 if cfg.w_dtype == "i4" else 1       # int4: two K rows per byte row
    E, d, f, fs = cfg.E, cfg.d, cfg.f, cfg.fs
    if E == 0:   # a dense layer: the shared gated MLP alone
        wsgu, ssgu, wsd, ssd = gen_shared(cfg, dev)
        return {"x": gen_x(cfg, dev), "w_router": None, "router_bias": None, "w_gate_up": None, "w_down": None,
                "s_gate_up": None, "s_down": None,
                "ws_gate_up": wsgu, "ss_gate_up": ssgu, "ws_down": wsd, "ss_down": ssd,
                "norm_weight": gen_norm_weight(cfg, dev)}
    out = {
        "x": gen_x(cfg, dev),
        "w_router": gen_router(cfg, dev),
        "router_bias": None if not cfg.has_bias else gen_bias(cfg).to(dev),
        "w_gate_up": torch.empty((E, d // kd, 2 * f), dtype=wdt, device=dev),
        "w_down": torch.empty((E, f // kd, d), dtype=wdt, device=dev),
        "s_gate_up": None, "s_down": None, "ss_gate_up": None, "ss_down": None,
        "norm_weight": gen_norm_weight(cfg, dev),
    }
    if scaled:
        out["s_gate_up"] = torch.empty((E, 2 * f), dtype=torch.float32, device=dev)
        out["s_down"] = torch.empty((E, d), dtype=torch.float32, device=dev)
    for e in range(E):
        wgu, sgu, wd, sd = gen_expert(cfg, e, dev)
        out["w_gate_up"][e].copy_(wgu)
        out["w_down"][e].copy_(wd)
        if sgu is not None:
            out["s_gate_up"][e].copy_(sgu)
            out["s_down"][e].copy_(sd)
        del wgu, wd, sgu, sd
    wsgu, ssgu, wsd, ssd = gen_shared(cfg, dev)
    out.update(ws_gate_up=wsgu, ss_gate_up=ssgu, ws_down=wsd, ss_down=ssd)
    return out
