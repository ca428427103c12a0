"""Parameter, FLOP and KV-cache arithmetic of Llama 4 text stacks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Closed forms from the architecture fields on the pages:
  * llm-architectures-explained "Llama 4 Maverick", table "Every
    architecture field": d_model 5120, vocab 202048, untied embeddings,
    40 query / 8 key-value heads of width 128, dense FFN d_ff 16384 (gated),
    MoE with 128 experts, 1 active, expert width 8192, one shared expert of
    width 8192, layout = dense and MoE layers alternating (MoE layers are
    range(step - 1, L, step) with step 2), 48 layers (36 chunked + 12 full
    attention in the "Architecture, drawn from the data" line); its table
    "Modelled costs" prints the totals these reproduce.
  * KerasFormers "Llama 4", API table of Llama4Model: the Scout defaults
    (16 experts, interleave step 1, mlp_dim 8192, 48 layers, 40/8 heads of
    128, vocab 202048, untied embeddings).
  * superteams.ai "Llama 4", "Mixture of Experts" section: Scout ~109B
    stored / ~17B active; Maverick ~400B / ~17B.

Counting rules (the pages' "Modelled costs" are reproduced only with these):
  gated MLP of width w:       3 * d * w        (gate, up, down)
  MoE block:                  E * 3*d*f + 3*d*fs + d*E   (experts, shared, router)
  active MoE block:           3*d*f + 3*d*fs + d*E       (top-1)
  attention per layer:        2*d*H*hd + 2*d*KV*hd       (q, o, k, v)
  RMSNorm weights:            2*d per layer + d final
  embeddings + untied head:   2*V*d
  decode FLOPs / token:       2*(active params w/o embeddings + head) + 4*L*H*hd*ctx
  prefill FLOPs (n tokens):   n*2*active_no_emb + sum_{p=1..n} 4*L*H*hd*p + 2*V*d
                              (LM head only on the last token)
  KV bytes / token (bf16):    layers whose cache grows with context (the full
                              attention layers) * 2 * KV * hd * 2
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class StackConfig:
    d: int = 5120
    vocab: int = 202048
    layers: int = 48
    heads: int = 40
    kv_heads: int = 8
    head_dim: int = 128
    experts: int = 16
    f: int = 8192          # routed expert width
    fs: int = 8192         # shared expert width
    dense_ff: int = 16384  # width of the non-MoE layers' MLP
    moe_step: int = 1      # interleave_moe_layer_step
    rope_interval: int = 4  # every 4th layer is a full-attention (NoPE) layer
    chunk: int = 8192


SCOUT = StackConfig(experts=16, moe_step=1)
MAVERICK = StackConfig(experts=128, moe_step=2)


def gated_mlp_params(d: int, w: int) -> int:
    return 3 * d * w


def moe_block_params(d: int, E: int, f: int, fs: int) -> int:
    return E * gated_mlp_params(d, f) + gated_mlp_params(d, fs) + d * E


def moe_block_active(d: int, E: int, f: int, fs: int) -> int:
    return gated_mlp_params(d, f) + gated_mlp_params(d, fs) + d * E


def moe_block_flops_per_token(d: int, E: int, f: int, fs: int) -> int:
    """Multiply-adds counted as 2 FLOPs: router + one routed expert + shared expert."""
    return 2 * moe_block_active(d, E, f, fs)


def moe_layers(c: StackConfig):
    return list(range(c.moe_step - 1, c.layers, c.moe_step))


def attn_params(c: StackConfig) -> int:
    return 2 * c.d * c.heads * c.head_dim + 2 * c.d * c.kv_heads * c.head_dim


def params(c: StackConfig) -> dict:
    n_moe = len(moe_layers(c))
    n_dense = c.layers - n_moe
    attn = c.layers * attn_params(c)
    norms = 2 * c.d * c.layers + c.d
    emb = 2 * c.vocab * c.d
    moe_total = n_moe * moe_block_params(c.d, c.experts, c.f, c.fs)
    moe_active = n_moe * moe_block_active(c.d, c.experts, c.f, c.fs)
    dense = n_dense * gated_mlp_params(c.d, c.dense_ff)
    total_no_emb = attn + norms + moe_total + dense
    active_no_emb = attn + norms + moe_active + dense
    return {
        "total": total_no_emb + emb,
        "active": active_no_emb + emb,
        "total_no_emb": total_no_emb,
        "active_no_emb": active_no_emb,
        "embeddings": emb,
    }


def decode_flops(c: StackConfig, ctx: int) -> int:
    p = params(c)
    return 2 * (p["active_no_emb"] + c.vocab * c.d) + 4 * c.layers * c.heads * c.head_dim * ctx


def prefill_flops(c: StackConfig, n: int) -> int:
    p = params(c)
    attn = 4 * c.layers * c.heads * c.head_dim * (n * (n + 1) // 2)
    return n * 2 * p["active_no_emb"] + attn + 2 * c.vocab * c.d


def full_attention_layers(c: StackConfig) -> int:
    return sum(1 for i in range(c.layers) if (i + 1) % c.rope_interval == 0)


def kv_bytes_per_token(c: StackConfig) -> int:
    return full_attention_layers(c) * 2 * c.kv_heads * c.head_dim * 2


def kv_bytes_at(c: StackConfig, ctx: int) -> int:
    chunked = c.layers - full_attention_layers(c)
    per_layer_tok = 2 * c.kv_heads * c.head_dim * 2
    return kv_bytes_per_token(c) * ctx + chunked * min(ctx, c.chunk) * per_layer_tok
