"""Test helpers: small shapes and a dictionary-backed weight source."""
from __future__ import annotations

import numpy as np

from synth import gen
from synth.configs import LayerShape, scaled, C1, C2, C3, C4


def tiny_gqa(**kw) -> LayerShape:
    base = dict(name="tiny_gqa", hidden=64, attn="gqa", n_heads=4, n_kv_heads=2, head_dim=16,
                wfmt="bf16", ffn="moe", inter=32, n_experts=6, top_k=2, n_shared=1,
                router="softmax", cache_len=7, max_seq=16)
    base.update(kw)
    return LayerShape(**base)


def tiny_mla(**kw) -> LayerShape:
    base = dict(name="tiny_mla", hidden=128, attn="mla", n_heads=4, q_lora=64, kv_lora=64, rope_dim=16,
                nope_dim=32, v_dim=32, wfmt="fp8", ffn="moe", inter=64, n_experts=8, top_k=2, n_shared=1,
                router="sigmoid_bias", router_std=0.02, cache_len=9, max_seq=32)
    base.update(kw)
    return LayerShape(**base)


class DictWeights:
    """Weight source with explicit fp32 matrices (stored as bf16) and optional overrides."""

    def __init__(self, shape, base=None, overrides=None, norms=None, bias=None, conv=None):
        self.s = shape
        self.base = base if base is not None else gen.LayerWeights(shape, 0, 0)
        self.ov = overrides or {}
        self.norms = norms or {}
        self.bias = bias
        self.conv = conv

    def matrix(self, name, expert=0):
        key = (name, expert)
        if key in self.ov:
            v = np.asarray(self.ov[key], dtype=np.float32)
            return {"fmt": "bf16", "bits": gen.f32_to_bf16_bits(v).reshape(v.shape)}
        if (name, None) in self.ov:
            v = np.asarray(self.ov[(name, None)], dtype=np.float32)
            return {"fmt": "bf16", "bits": gen.f32_to_bf16_bits(v).reshape(v.shape)}
        return self.base.matrix(name, expert)

    def norm(self, name):
        if name in self.norms:
            return np.asarray(self.norms[name], np.float32)
        return self.base.norm(name)

    def router_bias(self):
        if self.bias is not None:
            return np.asarray(self.bias, np.float32)
        return self.base.router_bias()

    def conv_weights(self):
        if self.conv is not None:
            return np.asarray(self.conv, np.float32)
        return self.base.conv_weights()


def tiny_kda(**kw) -> LayerShape:
    base = dict(name="tiny_kda", hidden=128, attn="kda", n_heads=4, head_dim=16, kda_rank=16, conv_width=4,
                wfmt="fp8", ffn="moe", inter=64, n_experts=8, top_k=2, n_shared=1, router="sigmoid_bias",
                router_std=0.02, cache_len=9, max_seq=32)
    base.update(kw)
    return LayerShape(**base)
