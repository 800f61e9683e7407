"""Bytes and FLOPs per decoded token, in closed form (TEST INFRASTRUCTURE and bench reporting).

The HBM-roofline accounting is the pages' own: interactivity bound = aggregate HBM
bandwidth / active bytes per token (TileRT article, "Ultra-High Interactivity on
NVIDIA GPUs? TileRT on InferenceX": the 64 TB/s / 21 GB worked example in the
introduction and the 38.4 TB/s / 42 GB example in "But What Exactly is TileRT?"),
and weight bytes = parameters x bits per weight / 8 (Vera Rubin article, section
"Lookup Table Weight Decompression in Rubin SM107 Tensor Core", MXFP4 4.25 and LUT
3.125 bits per weight). SwiGLU costs 2*d*m + 2*d*m + 2*m*d = 6*d*m FLOPs per token
(Kimi K3 article, LatentMoE section).

Algorithmic bytes of one decode layer-token (this project's definition): every stored
byte of the weights it reads (linear weights, FP8 block scales, norm gains, router
bias; only the selected and shared experts), the KV rows attention reads (all p+1 rows
for dense attention; the selected rows plus every index key for sparse attention),
the appended cache row, and the bf16 input and output vectors.
"""
from __future__ import annotations

import math

from synth.configs import LayerShape


def tokens_per_s_user(bandwidth_bytes_per_s: float, bytes_per_token: float) -> float:
    return bandwidth_bytes_per_s / bytes_per_token


def weight_bytes(n_params: float, bits_per_weight: float) -> float:
    return n_params * bits_per_weight / 8.0


def swiglu_flops(d: int, m: int) -> int:
    return 2 * d * m + 2 * d * m + 2 * m * d


def _mat_bytes(out_dim: int, in_dim: int, fmt: str) -> int:
    if fmt == "lut3":   # 3-bit indices + one 8-byte codebook per 8 x 64 block = 3.125 bits per weight
        return out_dim * in_dim * 3 // 8 + (out_dim // 8) * (in_dim // 64) * 8
    if fmt == "fp8":
        return out_dim * in_dim + 4 * math.ceil(out_dim / 128) * math.ceil(in_dim / 128)
    return 2 * out_dim * in_dim


def layer_weight_bytes(s: LayerShape) -> dict:
    """Storage bytes by group for one layer-token (selected + shared experts only)."""
    f = s.wfmt
    H = s.hidden
    g = {}
    if s.attn == "gqa":
        g["attn"] = (_mat_bytes(s.n_heads * s.head_dim, H, f) + 2 * _mat_bytes(s.n_kv_heads * s.head_dim, H, f)
                     + _mat_bytes(H, s.o_dim, f))
    elif s.attn == "kda":
        qd = s.q_dim
        g["attn"] = (4 * _mat_bytes(qd, H, f) + _mat_bytes(s.n_heads, H, f) + _mat_bytes(s.kda_rank, H, f)
                     + _mat_bytes(qd, s.kda_rank, f) + _mat_bytes(H, s.o_dim, f))
        g["conv"] = 4 * 3 * qd * s.conv_width
    else:
        g["attn"] = (_mat_bytes(s.q_lora, H, f) + _mat_bytes(s.n_heads * (s.nope_dim + s.rope_dim), s.q_lora, f)
                     + _mat_bytes(s.kv_lora + s.rope_dim, H, f) + _mat_bytes(s.n_heads * s.nope_dim, s.kv_lora, f)
                     + _mat_bytes(s.n_heads * s.v_dim, s.kv_lora, f) + _mat_bytes(H, s.o_dim, f))
        if s.index_topk:
            g["indexer"] = (_mat_bytes(s.index_heads * s.index_dim, s.q_lora, f) + _mat_bytes(s.index_heads, H, "bf16")
                            + _mat_bytes(s.index_dim, H, f))
    n_active = 1 if s.ffn == "dense" else s.top_k + s.n_shared
    fe = s.expert_fmt or f
    g["experts"] = n_active * (2 * _mat_bytes(s.inter, H, fe) + _mat_bytes(H, s.inter, fe))
    if s.ffn == "moe":
        g["router"] = 2 * s.n_experts * H + (4 * s.n_experts if s.router == "sigmoid_bias" else 0)
    g["norms"] = 4 * (2 * H + ((s.q_lora + s.kv_lora) if s.attn == "mla" else 0)
                      + (s.head_dim if s.attn == "kda" else 0))
    return g


def kda_state_bytes_per_head(d: int) -> int:
    """fp32 recurrent state of one KDA head, read once and written once per token: 8 d^2 bytes
    (the page's decode memory-traffic estimate)."""
    return 2 * 4 * d * d


def kda_state_flops_per_head(d: int) -> int:
    """Decode FLOPs of one KDA head's state step, counted as the page does (about 7 d^2): the
    decay D S (d^2 multiplies), S'^T k (2 d^2), the update S' + k u^T (2 d^2), S^T q (2 d^2)."""
    return d * d + 2 * d * d + 2 * d * d + 2 * d * d


def layer_kv_bytes(s: LayerShape, pos: int) -> dict:
    if s.attn == "kda":
        ring = 4 * (s.conv_width - 1) * 3 * s.q_dim
        st = s.n_heads * kda_state_bytes_per_head(s.head_dim) // 2
        return {"kv_read": st + ring, "kv_write": st + 4 * 3 * s.q_dim}
    T = pos + 1
    if s.attn == "gqa":
        row = 2 * s.n_kv_heads * s.head_dim * 2          # K and V, bf16
        return {"kv_read": T * row, "kv_write": row}
    row = 2 * s.latent_dim
    if s.index_topk:
        n_sel = min(s.index_topk, T)
        return {"kv_read": n_sel * row + T * (s.index_dim + 4), "kv_write": row + s.index_dim + 4}
    return {"kv_read": T * row, "kv_write": row}


def layer_bytes(s: LayerShape, pos: int) -> int:
    """Algorithmic bytes of one decode layer-token at position ``pos``."""
    return (sum(layer_weight_bytes(s).values()) + sum(layer_kv_bytes(s, pos).values())
            + 2 * 2 * s.hidden)


def head_bytes(hidden: int, vocab: int, fmt: str = "fp8") -> int:
    return _mat_bytes(vocab, hidden, fmt) + 4 * hidden + 2 * hidden   # head, final gain, embedding row


def expected_union_experts(n_experts: int, top_k: int, n_query: int) -> float:
    """Expected number of distinct routed experts over n_query positions that each pick top_k
    of n_experts, under uniform independent routing: E * (1 - (1 - k/E)^n)."""
    return n_experts * (1.0 - (1.0 - top_k / n_experts) ** n_query)


def verify_layer_bytes(s: LayerShape, pos: int, n_query: int) -> float:
    """Algorithmic bytes of one layer in an n_query-position verify (positions pos..pos+n-1):
    attention weights and the cache rows once, the expected union of the positions' routed
    experts plus the shared ones, the n appended rows and the n input/output vectors."""
    g = layer_weight_bytes(s)
    f = s.expert_fmt or s.wfmt
    one_expert = 2 * _mat_bytes(s.inter, s.hidden, f) + _mat_bytes(s.hidden, s.inter, f)
    experts = (expected_union_experts(s.n_experts, s.top_k, n_query) + s.n_shared) * one_expert
    other = sum(v for k, v in g.items() if k != "experts")
    last = pos + n_query - 1
    kv = layer_kv_bytes(s, last)["kv_read"] + n_query * layer_kv_bytes(s, last)["kv_write"]
    return other + experts + kv + n_query * 2 * 2 * s.hidden
