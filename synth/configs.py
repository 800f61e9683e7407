"""Workload shapes for the batch-1 decode layers.

These are plain shape and distribution records. They hold no arithmetic of the
decode method; both the CPU oracle and the HIP library read them.

The five workloads are the decode layers that the TileRT article ("Ultra-High
Interactivity on NVIDIA GPUs? TileRT on InferenceX", sections "But What Exactly is
TileRT?" and "PD Disaggregated Engine") and the vLLM Kimi K3 backend article
("Kernels collapse the decode loop", "Four changes drive the gains") talk about:
RMSNorm, projections, attention over a growing KV cache (dense, GQA, absorbed MLA
or indexer-selected sparse MLA), output projection, router top-k and SwiGLU experts.
The pages give no layer sizes; the sizes below are this project's chosen test and
benchmark workloads.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict


@dataclass(frozen=True)
class LayerShape:
    name: str
    hidden: int
    attn: str                 # "gqa" (MHA is the n_kv_heads == n_heads case), "mla" or "kda"
    n_heads: int
    # GQA / MHA
    n_kv_heads: int = 0
    head_dim: int = 0
    # MLA
    q_lora: int = 0
    kv_lora: int = 0
    rope_dim: int = 0
    nope_dim: int = 0
    v_dim: int = 0
    # KDA linear attention (attn == "kda"): n_heads heads of head_dim key/value channels,
    # a low-rank decay projection and a causal depthwise convolution over q, k, v
    kda_rank: int = 0
    conv_width: int = 0
    # sparse indexer (MLA only); index_topk == 0 means dense attention
    index_heads: int = 0
    index_dim: int = 0
    index_topk: int = 0
    # weights
    wfmt: str = "bf16"        # "bf16" or "fp8" (e4m3fn, fp32 scale per 128x128 block)
    expert_fmt: str = ""      # "" (as wfmt) or "lut3": expert matrices as 3-bit indices into an
                              # 8-entry E4M3 codebook per 8x64 block (3.125 bits per weight)
    # FFN
    ffn: str = "dense"        # "dense" or "moe"
    inter: int = 0            # dense FFN width, or per-expert width
    n_experts: int = 0
    top_k: int = 0
    n_shared: int = 0
    router: str = "softmax"   # "softmax" (top-k, softmax renormalised) or "sigmoid_bias"
    # cache
    cache_len: int = 0        # prefilled positions 0 .. cache_len-1
    max_seq: int = 0          # cache capacity (rows)
    # constants
    eps: float = 1e-6
    rope_base: float = 10000.0
    # synthetic value distributions
    w_std: float = 0.02
    router_std: float = 0.1
    bias_std: float = 0.1
    norm_std: float = 0.02    # gamma = 1 + norm_std * N(0,1)
    x_std: float = 1.0
    cache_std: float = 1.0
    state_std: float = 0.1    # prefilled KDA state entries
    conv_std: float = 0.5     # KDA convolution taps

    # ---- derived sizes -------------------------------------------------
    @property
    def q_dim(self) -> int:
        if self.attn in ("gqa", "kda"):
            return self.n_heads * self.head_dim
        return self.n_heads * (self.nope_dim + self.rope_dim)

    @property
    def o_dim(self) -> int:
        """Width of the concatenated attention output fed to W_O."""
        if self.attn in ("gqa", "kda"):
            return self.n_heads * self.head_dim
        return self.n_heads * self.v_dim

    @property
    def latent_dim(self) -> int:
        return self.kv_lora + self.rope_dim

    @property
    def n_expert_slots(self) -> int:
        """Routed experts plus shared experts (shared experts are stored last)."""
        return self.n_experts + self.n_shared

    @property
    def wbytes(self) -> int:
        return 1 if self.wfmt == "fp8" else 2


@dataclass(frozen=True)
class ModelShape:
    """A stack of identical-shape decode layers with an LM head (multi-layer workload)."""
    layer: LayerShape
    n_layers: int
    vocab: int
    n_tokens: int = 1
    n_verify: int = 6
    head_fmt: str = "fp8"
    emb_std: float = 1.0


# ---------------------------------------------------------------------------
# The workloads.
# ---------------------------------------------------------------------------
C1 = LayerShape(
    name="c1_tiny_dense_mha",
    hidden=256, attn="gqa", n_heads=4, n_kv_heads=4, head_dim=64,
    wfmt="bf16", ffn="dense", inter=1024,
    cache_len=128, max_seq=256,
)

C2 = LayerShape(
    name="c2_gqa_moe64_bf16",
    hidden=4096, attn="gqa", n_heads=32, n_kv_heads=8, head_dim=128,
    wfmt="bf16", ffn="moe", inter=1536, n_experts=64, top_k=8, n_shared=1,
    router="softmax",
    cache_len=8192, max_seq=8192 + 64,
)

C3 = LayerShape(
    name="c3_mla_moe256_fp8",
    hidden=6144, attn="mla", n_heads=64,
    q_lora=1536, kv_lora=512, rope_dim=64, nope_dim=128, v_dim=128,
    wfmt="fp8", ffn="moe", inter=2048, n_experts=256, top_k=8, n_shared=1,
    router="sigmoid_bias", router_std=0.02,
    cache_len=8192, max_seq=8192 + 64,
)

C4 = LayerShape(
    name="c4_sparse_mla_moe64_bf16",
    hidden=4096, attn="mla", n_heads=32,
    q_lora=1536, kv_lora=512, rope_dim=64, nope_dim=128, v_dim=128,
    index_heads=8, index_dim=64, index_topk=2048,
    wfmt="bf16", ffn="moe", inter=1536, n_experts=64, top_k=8, n_shared=1,
    router="softmax",
    cache_len=32768, max_seq=32768 + 64,
)

C5_LAYER = replace(C3, name="c5_layer_mla_moe256_fp8", max_seq=8192 + 256 + 8)

# KDA linear-attention decode layer (the Kimi K3 article's KDA, "FlashKDA Algorithm"): the
# FP8 MLA layer's hidden size and MoE, with 32 KDA heads of 128 key/value channels, a
# rank-128 decay projection and a width-4 causal convolution; the per-head fp32 state
# replaces the KV cache, so the position only indexes the convolution ring.
C6 = LayerShape(
    name="c6_kda_moe256_fp8",
    hidden=6144, attn="kda", n_heads=32, head_dim=128, kda_rank=128, conv_width=4,
    wfmt="fp8", ffn="moe", inter=2048, n_experts=256, top_k=8, n_shared=1,
    router="sigmoid_bias", router_std=0.02,
    cache_len=8192, max_seq=8192 + 64,
)
C5 = ModelShape(layer=C5_LAYER, n_layers=24, vocab=32768, n_tokens=256, n_verify=6)

# The FP8 MLA layer with lookup-table expert weights: every routed and shared expert matrix
# stores a 3-bit index per weight into the 8-entry E4M3 codebook of its 8x64 block (the
# Vera Rubin article's "Lookup Table Weight Decompression", 3.125 bits per weight), decoded
# in registers by the GEMV; attention stays FP8.
C7 = replace(C3, name="c7_mla_moe256_lut3_experts", expert_fmt="lut3")

LAYERS: Dict[str, LayerShape] = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5_LAYER, "c6": C6, "c7": C7}


def scaled(shape: LayerShape, **kw) -> LayerShape:
    """A copy with some fields changed (used for small test variants)."""
    return replace(shape, **kw)
