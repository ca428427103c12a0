"""The MoE feed-forward block in float64 -- plain, slow and direct.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Steps, in the order the pages give them:

1. Router: one logit per expert, l[t, e] = sum_j x[t, j] * Wr[j, e] + b[e]
   (superteams.ai "Llama 4", section "Mixture of Experts: Why Total and
   Active Parameters Diverge", the routing sketch: "one logit per expert").
   The bias b is optional (zero when absent); the pages name none, the
   skewed workloads need one.
2. Top-1: the expert with the largest logit, ties to the lowest index
   (same sketch: argmax; KerasFormers "Llama 4", section "What is unusual
   about the block": Scout routes 1 of 16, Maverick 1 of 128;
   llm-architectures-explained "Llama 4 Maverick", table "Every
   architecture field", ffns.moe.active = 1).
3. Gate: g = sigmoid(l[t, e*]) of the selected logit, applied to the
   token's input of the routed expert only (KerasFormers "Llama 4", "What is
   unusual about the block": the chosen expert receives the token multiplied
   by the sigmoid of its logit).
   No softmax, no renormalisation.  Because the expert's first layer is
   linear, g * (x W) = (g x) W; the oracle uses the former.
4. Routed expert e*: SwiGLU MLP, h = SiLU(u Wg) * (u Wu), y = h Wd, with
   Wg / Wu the column halves [0, f) / [f, 2f) of W_gate_up[e*] and
   SiLU(z) = z / (1 + exp(-z)) (llm-architectures-explained "Llama 4
   Maverick", "Every architecture field": experts are gated MLPs of width
   intermediate_size = 8192).
5. Shared expert: the same SwiGLU form of width fs on every token, no gate
   (same table: ffns.moe.shared = 1, d_shared = 8192; torchtune
   llama4_decoder, Parameters: use_shared_expert).
6. Combine: out = shared(x) + routed (superteams.ai routing sketch; the
   other experts contribute nothing).

With k experts per token (torchtune llama4_decoder, Parameters:
experts_per_token, whose docstring names 2 as its default; Llama 4 itself
uses 1) steps 2-4 run for each of the token's k largest logits (lower
expert index first among equal logits), each pick with the sigmoid of its
own logit as the gate on its input, and step 6 adds the k routed outputs to
the shared one.  No softmax or renormalisation over the picks: the plain
generalisation of the top-1 gate.

Optional step 0, the RMSNorm in front of the block (llm-architectures-explained
"Llama 4 Maverick", table "Every architecture field": RMSNorm before the MLP;
KerasFormers "Llama 4", Llama4Model arguments: norm_eps 1e-5): each row is
divided by the root of its mean square plus eps and multiplied by the gain,
xn = x / sqrt(mean(x^2) + eps) * w, exactly in float64 and rounded once
(RNE) to the dtype of x; steps 1-6 then take xn in place of x.  The pages
name the norm and its eps, not its formula: this is the standard RMSNorm
(root-mean-square layer normalisation with a learned per-feature gain).

Rounding points of the reduced-precision variants (the pages fix none; they
follow the data types of the workloads):
  R1 (bf16 weights): the SwiGLU output h is rounded to bf16 (RNE, from its
     float32 value) before the down projection.
  R0 (e4m3 weights): per token, s_x = fp32(max_j |x[t, j]|) / 448 in float32
     (1 for an all-zero row), q = e4m3(fp32(x) / s_x); the shared expert sees
     q * s_x and the routed expert q * (g * s_x).
  R1 (e4m3 weights): h is quantised per token exactly like R0, from its
     float32 value: s_h = fp32(max_j |h[t, j]|) / 448, code = e4m3(fp32(h) / s_h).
     (A bf16 intermediate is deliberately absent: a scale taken from a
     bf16-rounded row lets a one-ulp difference in the row's largest element
     re-round every code of that row.)
  R1 (int8 and int4 weights, dequantised to code * column scale): as for
     bf16 -- the activations stay bf16 and h is rounded to bf16.
  The output itself is returned unrounded in float64.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import numpy as np
import torch

from .numerics import bf16_round, e4m3_round, e4m3_decode, round_f64_to

NEAR_TIE = 1e-3   # top-2 logit margin below which either choice is accepted


# ------------------------------------------------------------ input decoding

def to_f64(t) -> np.ndarray:
    """fp32 / bf16 torch tensor (or numpy array) -> exact float64 numpy array."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def unpack_int4(packed) -> np.ndarray:
    """[K/2, N] bytes, byte (i, n) = code(2i, n) in the low nibble and
    code(2i+1, n) in the high one (two's complement) -> int codes [K, N]."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo, hi = b & 15, b >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((2 * b.shape[0], b.shape[1]), dtype=np.int64)
    out[0::2], out[1::2] = lo, hi
    return out


def dequant_cols(codes, scale, fmt=None) -> np.ndarray:
    """Weight codes [K, N] with one fp32 scale per column N -> float64 values:
    e4m3 codes (uint8) decode to their e4m3 values, int8 codes are integers,
    int4 codes (fmt "i4") come packed two per byte along K; value = code
    value * scale[n]."""
    c = codes.numpy() if isinstance(codes, torch.Tensor) else np.asarray(codes)
    s = to_f64(scale)
    if fmt == "i4":
        return unpack_int4(c).astype(np.float64) * s[None, :]
    if c.dtype == np.int8:
        return c.astype(np.float64) * s[None, :]
    if c.dtype != np.uint8:
        raise TypeError(f"weight codes of dtype {c.dtype}")
    return e4m3_decode(c) * s[None, :]


def weight_f64(w, scale=None, fmt=None) -> np.ndarray:
    if scale is None:
        return to_f64(w)
    return dequant_cols(w, scale, fmt)


# ------------------------------------------------------------ routing

@dataclasses.dataclass
class Routing:
    logits: np.ndarray   # [T, E] float64
    idx: np.ndarray      # [T] int64, chosen expert
    gate: np.ndarray     # [T] float64, sigmoid of the chosen logit
    margin: np.ndarray   # [T] float64, chosen logit minus best other (inf if E == 1)
    counts: np.ndarray   # [E] int64
    offsets: np.ndarray  # [E + 1] int64
    perm: np.ndarray     # [T] int64, tokens grouped by expert, ascending within a group
    inv: np.ndarray      # [T] int64, inverse of perm


def rmsnorm(x, w, eps: float, dtype: str) -> np.ndarray:
    """Step 0: xn[t, j] = x[t, j] / sqrt(mean_j x[t, j]^2 + eps) * w[j] in
    float64, rounded once to `dtype` ("bf16" / "f32"); float64 values out."""
    x64 = to_f64(x)
    w64 = to_f64(w)
    ms = np.mean(x64 * x64, axis=1) if x64.shape[1] else np.zeros(x64.shape[0])
    y = x64 / np.sqrt(ms + float(eps))[:, None] * w64[None, :]
    return round_f64_to(y, dtype)


def router_logits(x, wr, bias=None) -> np.ndarray:
    lg = to_f64(x) @ to_f64(wr)
    if bias is not None:
        lg = lg + to_f64(bias)[None, :]
    return lg


def top1(logits: np.ndarray):
    """Lowest index among the maxima of each row, and the top-2 margin."""
    T, E = logits.shape
    mx = logits.max(axis=1) if E else np.zeros(T)
    idx = np.argmax(logits == mx[:, None], axis=1).astype(np.int64)
    if E == 1:
        margin = np.full(T, np.inf)
    else:
        others = logits.copy()
        others[np.arange(T), idx] = -np.inf
        margin = mx - others.max(axis=1)
    return idx, margin


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def routing_record(idx: np.ndarray, E: int):
    counts = np.bincount(idx, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    perm = np.argsort(idx, kind="stable").astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm), dtype=np.int64)
    return counts, offsets, perm, inv


def topk(logits: np.ndarray, k: int):
    """The k largest logits of each row, best first, the lower expert index
    first among equal logits; margin = the smallest gap between consecutive
    values among the k + 1 largest (the k largest when E == k; inf for
    k == E == 1).  k = 1 gives top1()."""
    T, E = logits.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -logits), axis=-1)
    idx = order[:, :k].astype(np.int64)
    top = np.take_along_axis(logits, order[:, :min(k + 1, E)], axis=1)
    gaps = top[:, :-1] - top[:, 1:]
    margin = gaps.min(axis=1) if gaps.shape[1] else np.full(T, np.inf)
    return idx, margin


def route_topk(x, wr, bias, k: int) -> Routing:
    """Routing with k experts per token (the block generalised: each of the
    token's k picks is an expert of the top-1 kind, with its own sigmoid gate
    on its input; the routed outputs add up).  idx and gate are [T, k]; the
    record groups the T * k slots (slot t * k + j = token t's j-th pick) by
    expert, ascending slot order within a group."""
    lg = router_logits(x, wr, bias)
    idx, margin = topk(lg, k)
    gate = sigmoid(np.take_along_axis(lg, idx, axis=1))
    counts, offsets, perm, inv = routing_record(idx.reshape(-1), lg.shape[1])
    return Routing(lg, idx, gate, margin, counts, offsets, perm, inv)


def route(x, wr, bias=None) -> Routing:
    lg = router_logits(x, wr, bias)
    idx, margin = top1(lg)
    gate = sigmoid(lg[np.arange(lg.shape[0]), idx])
    counts, offsets, perm, inv = routing_record(idx, lg.shape[1])
    return Routing(lg, idx, gate, margin, counts, offsets, perm, inv)


# ------------------------------------------------------------ experts

def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu(a: np.ndarray, width: int) -> np.ndarray:
    return silu(a[:, :width]) * a[:, width:]


def quant_rows_e4m3(v32: np.ndarray):
    """Per-row e4m3 quantisation of float32-valued rows -> (values q*s as float64, s)."""
    v32 = np.asarray(v32, dtype=np.float32)
    amax = np.abs(v32).max(axis=1) if v32.shape[1] else np.zeros(v32.shape[0], np.float32)
    s = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    s = np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)
    q = e4m3_round((v32 / s[:, None]).astype(np.float32))
    return q * s.astype(np.float64)[:, None], s


def round_h(h: np.ndarray, mode: str) -> np.ndarray:
    """Rounding point R1 applied to SwiGLU outputs (rows = tokens)."""
    if mode == "f32":
        return h
    if mode in ("bf16", "i8", "i4"):   # int8 / int4 weights: bf16 activations, h rounded like bf16
        return bf16_round(h.astype(np.float32))
    if mode == "e4m3":
        return quant_rows_e4m3(h.astype(np.float32))[0]
    raise ValueError(mode)


def swiglu_mlp(u: np.ndarray, wgu: np.ndarray, wd: np.ndarray, width: int, mode: str,
               row_scale: Optional[np.ndarray] = None) -> np.ndarray:
    a = u @ wgu
    if row_scale is not None:
        a = a * row_scale[:, None]
    h = round_h(swiglu(a, width), mode)
    return h @ wd


# ------------------------------------------------------------ the block

class Weights:
    """Access to the block's weights as torch CPU tensors.

    router() -> (w_router [d,E], bias [E] | None)
    expert(e) -> (w_gate_up [d,2f], s_gate_up | None, w_down [f,d], s_down | None)
    shared() -> (ws_gate_up [d,2fs], ss_gate_up | None, ws_down [fs,d], ss_down | None)
    """

    def __init__(self, router: Callable, expert: Callable, shared: Callable):
        self.router, self.expert, self.shared = router, expert, shared

    @staticmethod
    def from_dict(inp: dict) -> "Weights":
        def ex(e):
            s = inp.get("s_gate_up")
            sd = inp.get("s_down")
            return (inp["w_gate_up"][e], None if s is None else s[e],
                    inp["w_down"][e], None if sd is None else sd[e])
        return Weights(lambda: (inp["w_router"], inp.get("router_bias")), ex,
                       lambda: (inp["ws_gate_up"], inp.get("ss_gate_up"),
                                inp["ws_down"], inp.get("ss_down")))


def expert_input(x, mode: str):
    """The expert path's view of x: (float64 values, per-token scale or None)."""
    x64 = to_f64(x)
    if mode != "e4m3":
        return x64, None
    xq, s = quant_rows_e4m3(x64.astype(np.float32))
    return xq, s


def combine(x, idx: np.ndarray, gate: np.ndarray, w: Weights, f: int, fs: int,
            mode: str) -> np.ndarray:
    """out[t] = shared(x[t]) + expert_{idx[t]}(gate[t] * x[t]) for given choices."""
    xin, _ = expert_input(x, mode)
    T = xin.shape[0]
    wsgu, ssgu, wsd, ssd = w.shared()
    out = swiglu_mlp(xin, weight_f64(wsgu, ssgu, mode), weight_f64(wsd, ssd, mode), fs, mode)
    for e in np.unique(idx):
        rows = np.nonzero(idx == e)[0]
        wgu, sgu, wd, sd = w.expert(int(e))
        out[rows] += swiglu_mlp(xin[rows], weight_f64(wgu, sgu, mode), weight_f64(wd, sd, mode), f, mode,
                                row_scale=gate[rows])
    assert out.shape[0] == T
    return out


def combine_topk(x, idx: np.ndarray, gate: np.ndarray, w: Weights, f: int, fs: int,
                 mode: str) -> np.ndarray:
    """out[t] = shared(x[t]) + sum_j expert_{idx[t,j]}(gate[t,j] * x[t]), idx and
    gate [T, k] (a token's picks are distinct experts)."""
    xin, _ = expert_input(x, mode)
    wsgu, ssgu, wsd, ssd = w.shared()
    out = swiglu_mlp(xin, weight_f64(wsgu, ssgu, mode), weight_f64(wsd, ssd, mode), fs, mode)
    for e in np.unique(idx):
        rows, cols = np.nonzero(idx == e)
        wgu, sgu, wd, sd = w.expert(int(e))
        out[rows] += swiglu_mlp(xin[rows], weight_f64(wgu, sgu, mode), weight_f64(wd, sd, mode), f, mode,
                                row_scale=gate[rows, cols])
    return out


def dense(x, w: Weights, fs: int, mode: str) -> np.ndarray:
    """A dense layer (llm-architectures-explained "Llama 4 Maverick", table
    "Every architecture field": the non-MoE layers' FFN is a gated MLP of
    width d_ff, 16384): out = SwiGLU(x) with the shared weights and width fs,
    no router and no gate.  The same computation as combine() with no routed
    token."""
    xin, _ = expert_input(x, mode)
    wsgu, ssgu, wsd, ssd = w.shared()
    return swiglu_mlp(xin, weight_f64(wsgu, ssgu, mode), weight_f64(wsd, ssd, mode), fs, mode)


def forward(x, w: Weights, f: int, fs: int, mode: str, top_k: int = 1):
    """Whole block: returns (out float64 [T, d], Routing)."""
    wr, b = w.router()
    if top_k > 1:
        r = route_topk(x, wr, b, top_k)
        return combine_topk(x, r.idx, r.gate, w, f, fs, mode), r
    r = route(x, wr, b)
    out = combine(x, r.idx, r.gate, w, f, fs, mode)
    return out, r


def rel_err(got, ref) -> float:
    """max |got - ref| / RMS(ref)."""
    g = to_f64(got)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0:
        return float(np.max(np.abs(g - ref)))
    return float(np.max(np.abs(g - ref)) / rms)
