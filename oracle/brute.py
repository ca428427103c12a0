"""Brute force for tiny inputs: pure-Python loops, every expert evaluated.

TEST INFRASTRUCTURE ONLY (see the package docstring).

For each token this computes *all* E routed experts on the gated input and
only afterwards keeps the one the router chose, so a wrong selection, a
wrong gate placement or a leak from an unselected expert shows up as a
mismatch against oracle.block.  It shares no helper with oracle.block:
logits, argmax, sigmoid, SiLU, matrix products and the rounding points are
written again here, with plain Python floats (binary64).

Rounding points use different routes from oracle.numerics:
  bf16  -- integer round-to-nearest-even on the IEEE float32 bit pattern
           (struct pack / unpack);
  e4m3  -- torch's float8_e4m3fn cast (a library routine) of the clamped
           float32 quotient.
"""
from __future__ import annotations

import math
import struct

import torch


def _f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16(v: float) -> float:
    bits = struct.unpack("<I", struct.pack("<f", _f32(v)))[0]
    lsb = (bits >> 16) & 1
    bits = (bits + 0x7FFF + lsb) & 0xFFFF0000
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def _f32_div(a: float, b: float) -> float:
    return float(torch.tensor(a, dtype=torch.float32) / torch.tensor(b, dtype=torch.float32))


def _e4m3(v32: float) -> float:
    c = max(-448.0, min(448.0, v32))
    return float(torch.tensor(c, dtype=torch.float32).to(torch.float8_e4m3fn).to(torch.float64))


def _quant_row(row):
    amax = _f32(max(abs(v) for v in row)) if row else 0.0
    s = _f32_div(amax, 448.0) if amax > 0 else 1.0
    return [_e4m3(_f32_div(_f32(v), s)) * s for v in row], s


def _matvec(u, W):  # u [K], W [K][N] -> [N]
    K, N = len(W), len(W[0])
    return [sum(u[k] * W[k][n] for k in range(K)) for n in range(N)]


def _swiglu_mlp(u, wgu, wd, width, mode, scale=1.0):
    a = [scale * v for v in _matvec(u, wgu)]
    h = []
    for j in range(width):
        z = a[j]
        h.append(z / (1.0 + math.exp(-z)) * a[width + j])
    if mode in ("bf16", "i8", "i4"):
        h = [_bf16(v) for v in h]
    if mode == "e4m3":
        h, _ = _quant_row([_f32(v) for v in h])
    return _matvec(h, wd)


def forward(x, wr, bias, w_gate_up, w_down, ws_gate_up, ws_down, f, fs, mode="f32", top_k=1):
    """All arguments are nested Python lists of floats (weights already dequantised).

    Returns (out [T][d], idx [T], gate [T]); with top_k > 1 idx and gate hold
    one list of the token's picks (best first) per token.
    """
    T = len(x)
    E = len(wr[0]) if wr else 0
    d = len(x[0]) if T else 0
    outs, idxs, gates = [], [], []
    for t in range(T):
        row = list(x[t])
        logits = []
        for e in range(E):
            acc = 0.0
            for j in range(d):
                acc += row[j] * wr[j][e]
            logits.append(acc + (bias[e] if bias is not None else 0.0))
        if top_k > 1:
            # every expert densely, then keep the top_k by (larger logit, lower index)
            picks = sorted(range(E), key=lambda e: (-logits[e], e))[:top_k]
            gs = [1.0 / (1.0 + math.exp(-logits[e])) for e in picks]
            xin = _quant_row(row)[0] if mode == "e4m3" else row
            dense = [_swiglu_mlp(xin, w_gate_up[e], w_down[e], f, mode,
                                 scale=1.0 / (1.0 + math.exp(-logits[e]))) for e in range(E)]
            shared = _swiglu_mlp(xin, ws_gate_up, ws_down, fs, mode)
            o = list(shared)
            for e in picks:
                o = [o[n] + dense[e][n] for n in range(d)]
            outs.append(o)
            idxs.append(picks)
            gates.append(gs)
            continue
        best = 0
        for e in range(1, E):
            if logits[e] > logits[best]:
                best = e
        g = 1.0 / (1.0 + math.exp(-logits[best]))
        if mode == "e4m3":
            xin, _ = _quant_row(row)
        else:
            xin = row
        # every expert, densely, on the gated input
        dense = [_swiglu_mlp(xin, w_gate_up[e], w_down[e], f, mode, scale=g) for e in range(E)]
        shared = _swiglu_mlp(xin, ws_gate_up, ws_down, fs, mode)
        outs.append([shared[n] + dense[best][n] for n in range(d)])
        idxs.append(best)
        gates.append(g)
    return outs, idxs, gates
