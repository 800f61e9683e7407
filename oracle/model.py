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

Temperature sampling (the vLLM Kimi K3 backend article leaves the sampling policy to the
caller and names temperature sampling among its serving settings, "A narrow deployment
lane"): the Gumbel-max form of sampling from softmax(logits / T): token = argmax_i
(logit_i / T - log(-log u_i)), u_i uniform in (0, 1), ties to the lower id; T = 0 is greedy.
The uniforms come from a counter-based generator keyed by (seed, position of the step,
token id), so a token depends only on its position's logits and the seed. Consequence used
by the tests: speculative decoding that accepts a draft exactly when it equals the
position's sample (for a deterministic drafter this is the speculative-sampling acceptance
rule: accepted with probability p(draft), and on rejection the sample follows p without the
draft, renormalised) reproduces plain sampled decoding token for token.

Generator (SplitMix64, Steele, Lea and Flood, OOPSLA 2014; the mixer of Vigna's
splitmix64.c), all arithmetic mod 2**64 with G = 0x9E3779B97F4A7C15:
  k = mix(seed * G + pos);  r_i = mix(k + (i + 1) * G);  u_i = (2 * (r_i >> 12) + 1) * 2**-53
(u_i is exact in fp64 and never 0 or 1).
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


_G = 0x9E3779B97F4A7C15
_M64 = (1 << 64) - 1


def splitmix_mix(z):
    """The SplitMix64 output mixer on uint64 arrays (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        return z ^ (z >> np.uint64(31))


def sample_uniforms(seed: int, pos: int, n: int) -> np.ndarray:
    """u_i in (0, 1), i = 0..n-1, of the step at position ``pos`` (see the module docstring)."""
    k = splitmix_mix(np.uint64(((seed * _G) + pos) & _M64))
    i = np.arange(n, dtype=np.uint64)
    with np.errstate(over="ignore"):
        r = splitmix_mix(k + (i + np.uint64(1)) * np.uint64(_G))
    return ((r >> np.uint64(12)).astype(np.float64) * 2.0 + 1.0) * 2.0 ** -53


def sample_token(logits: np.ndarray, temperature: float, seed: int, pos: int) -> int:
    """Gumbel-max sample of softmax(logits / T) at position ``pos``; T = 0 is greedy argmax."""
    lg = np.asarray(logits, dtype=np.float64)
    if temperature == 0:
        return argmax_lowest(lg)
    u = sample_uniforms(seed, pos, lg.shape[0])
    return argmax_lowest(lg / float(temperature) - np.log(-np.log(u)))


def decode_tokens(layer_shape, layer_srcs: Sequence, caches: List[dict], embed_fn, head_m, final_gamma,
                  token0: int, start_pos: int, n_tokens: int, records=None, temperature: float = 0.0,
                  seed: int = 0):
    """Autoregressive decode (greedy, or sampled at temperature T): returns (tokens produced,
    list of per-token logits).

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
        tok = sample_token(lg, temperature, seed, start_pos + t)
        toks.append(tok)
        logits_all.append(lg)
    return toks, logits_all


def verify_step(layer_shape, layer_srcs, caches, embed_fn, head_m, final_gamma,
                token0: int, drafts: Sequence[int], pos: int, temperature: float = 0.0, seed: int = 0):
    """Score n = 1 + len(drafts) positions and apply the acceptance rule: a draft is kept
    while it equals the token chosen at the position before it (greedy argmax, or the
    position's sample at temperature T).

    Returns dict(tokens=[token chosen at each position], logits=[...], accepted=m) where m is
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
        toks.append(sample_token(lg, temperature, seed, pos + j))
    m = 0
    for j in range(1, len(inputs)):
        if inputs[j] == toks[j - 1]:
            m += 1
        else:
            break
    return {"tokens": toks, "logits": logits, "accepted": m}
