"""CPU oracle of a stack of decode layers with an LM head (TEST INFRASTRUCTURE).

* One launch decoding many tokens through many layers is the persistent "Engine
  Kernel" of the TileRT article ("Ultra-High Interactivity on NVIDIA GPUs? TileRT on
  InferenceX", section "But What Exactly is TileRT?"); this oracle only fixes what that
  launch must produce, token by token and layer by layer.
* The multi-token verify step follows the speculative decoding with a draft of six
  tokens in the vLLM Kimi K3 backend article (summary bullets and the table in
  "Throughput holds across the tested range", DSpark AL=6). Its plain definition:
  the n query positions p..p+n-1 are n sequential single-token decode steps fed the
  last accepted token followed by the n-1 draft tokens (causal attention among the new
  rows is exactly what sequential steps give); greedy acceptance keeps draft d_j while
  d_j equals the argmax at position j-1.

Readings: greedy argmax with ties to the lower token id; the next input is the
embedding row of the chosen token; layer outputs are bf16.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np

from . import numerics as nx
from .layer import append_to_cache, decode_layer, weight_f64


def head_logits(layer_shape, head_m, final_gamma, out_bits) -> np.ndarray:
    """logits = W_head RMSNorm(out; gamma_final), fp64."""
    h = nx.bf16_to_f64(out_bits)
    hn = nx.rmsnorm(h, final_gamma, layer_shape.eps)
    return weight_f64(head_m) @ hn


def argmax_lowest(v: np.ndarray) -> int:
    """Index of the maximum, lowest index on ties (np.argmax returns the first maximum)."""
    return int(np.argmax(np.asarray(v, dtype=np.float64)))


def decode_tokens(layer_shape, layer_srcs: Sequence, caches: List[dict], embed_fn, head_m, final_gamma,
                  token0: int, start_pos: int, n_tokens: int, records=None):
    """Greedy autoregressive decode: returns (tokens produced, list of per-token logits).

    ``embed_fn(token) -> bf16 bits [hidden]``; ``caches`` are mutated (rows appended).
    """
    toks, logits_all = [], []
    tok = token0
    for t in range(n_tokens):
        x = embed_fn(tok)
        for li, W in enumerate(layer_srcs):
            rec = decode_layer(layer_shape, W, caches[li], x, start_pos + t)
            append_to_cache(layer_shape, caches[li], rec, start_pos + t)
            if records is not None:
                records.append((t, li, rec))
            x = rec["out_bits"]
        lg = head_logits(layer_shape, head_m, final_gamma, x)
        tok = argmax_lowest(lg)
        toks.append(tok)
        logits_all.append(lg)
    return toks, logits_all


def verify_step(layer_shape, layer_srcs, caches, embed_fn, head_m, final_gamma,
                token0: int, drafts: Sequence[int], pos: int):
    """Score n = 1 + len(drafts) positions and apply greedy acceptance.

    Returns dict(tokens=[argmax at each position], logits=[...], accepted=m) where m is
    the number of leading drafts accepted; the caller's cache is valid up to pos+m+1.
    """
    inputs = [int(token0)] + [int(d) for d in drafts]
    toks, logits = [], []
    for j, tin in enumerate(inputs):
        x = embed_fn(tin)
        for li, W in enumerate(layer_srcs):
            rec = decode_layer(layer_shape, W, caches[li], x, pos + j)
            append_to_cache(layer_shape, caches[li], rec, pos + j)
            x = rec["out_bits"]
        lg = head_logits(layer_shape, head_m, final_gamma, x)
        logits.append(lg)
        toks.append(argmax_lowest(lg))
    m = 0
    for j in range(1, len(inputs)):
        if inputs[j] == toks[j - 1]:
            m += 1
        else:
            break
    return {"tokens": toks, "logits": logits, "accepted": m}
