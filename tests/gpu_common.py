"""Shared pieces of the GPU parity tests: device inputs (synth.device), oracle references
(oracle/, fed only by the host generator), and the comparison metric."""
from __future__ import annotations

import sys

import numpy as np

from oracle import layer as OL
from oracle import numerics as nx
from synth import gen

TOL = 2e-2   # max relative error ||g - o||_inf / ||o||_inf for hidden states and logits


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def bf16_tensor_to_f64(t) -> np.ndarray:
    return nx.bf16_to_f64(t.detach().cpu().numpy().view(np.uint16))


def host_cache(s, seed=0, layer=0, fill_len=None):
    """Host copy of a prefilled cache, padded to max_seq rows (positions >= fill_len are zero)."""
    n = s.cache_len if fill_len is None else fill_len
    out = {}
    if s.attn == "gqa":
        pos = np.arange(n)
        for kind, key in (("k_cache", "k"), ("v_cache", "v")):
            z = np.zeros((s.n_kv_heads, s.max_seq, s.head_dim), np.uint16)
            for g in range(s.n_kv_heads):
                z[g, :n] = gen.kv_rows(s, kind, g, pos, seed, layer)
            out[key] = z
    else:
        z = np.zeros((s.max_seq, s.latent_dim), np.uint16)
        z[:n] = gen.latent_rows(s, np.arange(n), seed, layer)
        out["latent"] = z
        if s.index_topk:
            codes = np.zeros((s.max_seq, s.index_dim), np.uint8)
            scales = np.zeros(s.max_seq, np.float32)
            c, sc = gen.index_key_rows(s, np.arange(n), seed, layer)
            codes[:n], scales[:n] = c, sc
            out["index_codes"], out["index_scales"] = codes, scales
    return out


def oracle_step(s, seed, layer, cache, x_bits, pos, weights=None):
    W = weights if weights is not None else gen.LayerWeights(s, seed, layer)
    rec = OL.decode_layer(s, W, cache, x_bits, pos)
    OL.append_to_cache(s, cache, rec, pos)
    return rec
