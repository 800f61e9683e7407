"""Device fills of the seeded inputs (ctypes binding of synth/libsynth_gen.so).

Writes the same bytes as the host generator in ``synth/gen.py`` straight into torch
device tensors, so large weight sets never cross PCIe. Holds no arithmetic of the
decode method.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import gen
from .configs import LayerShape, ModelShape

_LIB = None
_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth_gen.so")


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is not built; run python -m persistent_latency_bound_amd.build")
        L = ctypes.CDLL(_PATH)
        u64, i32, f32, vp, i64 = ctypes.c_uint64, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64
        L.synth_fill_bf16_3d.argtypes = [vp, i32, i32, i32, i32, u64, u64, f32, vp]
        L.synth_fill_f32.argtypes = [vp, i64, u64, u64, f32, f32, i32, vp]
        L.synth_fill_fp8_block.argtypes = [vp, vp, i32, i32, u64, u64, f32, vp]
        L.synth_fill_fp8_rows.argtypes = [vp, vp, i32, i32, u64, u64, f32, vp]
        L.synth_fill_lut3.argtypes = [vp, vp, i32, i32, u64, u64, f32, vp]
        for f in (L.synth_fill_bf16_3d, L.synth_fill_f32, L.synth_fill_fp8_block, L.synth_fill_fp8_rows,
                  L.synth_fill_lut3):
            f.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _chk(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with hip error {rc}")


def fill_bf16_matrix(t: torch.Tensor, seed: int, tid: int, std: float):
    rows, cols = t.shape[-2], t.shape[-1]
    _chk(lib().synth_fill_bf16_3d(ctypes.c_void_p(t.data_ptr()), 1, rows, rows, cols, seed, tid, std, _stream()),
         "fill_bf16_matrix")


def fill_bf16_cache(t: torch.Tensor, n_heads: int, n_pos: int, stride_pos: int, row: int, seed: int, tid: int, std: float):
    _chk(lib().synth_fill_bf16_3d(ctypes.c_void_p(t.data_ptr()), n_heads, n_pos, stride_pos, row, seed, tid, std,
                                  _stream()), "fill_bf16_cache")


def fill_f32(t: torch.Tensor, seed: int, tid: int, std: float, mean=None):
    _chk(lib().synth_fill_f32(ctypes.c_void_p(t.data_ptr()), t.numel(), seed, tid, std, 0.0 if mean is None else mean,
                              0 if mean is None else 1, _stream()), "fill_f32")


def fill_fp8_matrix(codes: torch.Tensor, scales: torch.Tensor, seed: int, tid: int, std: float):
    rows, cols = codes.shape[-2], codes.shape[-1]
    _chk(lib().synth_fill_fp8_block(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), rows, cols,
                                    seed, tid, std, _stream()), "fill_fp8_matrix")


def fill_lut3_matrix(idx: torch.Tensor, cb: torch.Tensor, seed: int, tid: int, std: float):
    rows, cols = idx.shape[-2], idx.shape[-1] * 8 // 3
    _chk(lib().synth_fill_lut3(ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(cb.data_ptr()), rows, cols, seed, tid,
                               std, _stream()), "fill_lut3_matrix")


def fill_fp8_rows(codes: torch.Tensor, scales: torch.Tensor, n_rows: int, seed: int, tid: int, std: float):
    d = codes.shape[-1]
    _chk(lib().synth_fill_fp8_rows(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()), n_rows, d,
                                   seed, tid, std, _stream()), "fill_fp8_rows")


# ---------------------------------------------------------------------------
def _mat(s: LayerShape, name: str, n_slots: int, dev, seed: int, layer: int):
    out_dim, in_dim = gen.layer_matrices(s)[name]
    std = s.router_std if name == "router" else s.w_std
    expert = name in gen.EXPERT_MATS
    shape = (n_slots, out_dim, in_dim) if expert else (out_dim, in_dim)
    if gen.weight_format(s, name) == "lut3":
        idx = torch.empty(shape[:-1] + (in_dim * 3 // 8,), dtype=torch.uint8, device=dev)
        cb = torch.empty(((n_slots,) if expert else ()) + (out_dim // 8, in_dim // 64, 8), dtype=torch.uint8, device=dev)
        for e in range(n_slots if expert else 1):
            fill_lut3_matrix(idx[e] if expert else idx, cb[e] if expert else cb, seed,
                             gen.tensor_id(name, layer, e if expert else 0), std)
        return {"fmt": "lut3", "data": idx, "scales": cb}
    if gen.weight_format(s, name) == "fp8":
        codes = torch.empty(shape, dtype=torch.uint8, device=dev)
        nb = (-(-out_dim // 128), -(-in_dim // 128))
        scales = torch.empty(((n_slots,) if expert else ()) + nb, dtype=torch.float32, device=dev)
        if expert:
            for e in range(n_slots):
                fill_fp8_matrix(codes[e], scales[e], seed, gen.tensor_id(name, layer, e), std)
        else:
            fill_fp8_matrix(codes, scales, seed, gen.tensor_id(name, layer, 0), std)
        return {"fmt": "fp8", "data": codes, "scales": scales}
    t = torch.empty(shape, dtype=torch.int16, device=dev)
    if expert:
        for e in range(n_slots):
            fill_bf16_matrix(t[e], seed, gen.tensor_id(name, layer, e), std)
    else:
        fill_bf16_matrix(t, seed, gen.tensor_id(name, layer, 0), std)
    return {"fmt": "bf16", "data": t, "scales": None}


def layer_weights(s: LayerShape, seed: int = 0, layer: int = 0, device="cuda") -> dict:
    """All weights of one layer in device memory (expert slots: routed then shared)."""
    n_slots = s.n_expert_slots if s.ffn == "moe" else 1
    W = {}
    for name in gen.layer_matrices(s):
        W[name] = _mat(s, name, n_slots, device, seed, layer)
    for name, n in gen.layer_norms(s).items():
        t = torch.empty(n, dtype=torch.float32, device=device)
        fill_f32(t, seed, gen.tensor_id(name, layer), s.norm_std, mean=1.0)
        W[name] = t
    if s.ffn == "moe" and s.router == "sigmoid_bias":
        t = torch.empty(s.n_experts, dtype=torch.float32, device=device)
        fill_f32(t, seed, gen.tensor_id("router_bias", layer), s.bias_std)
        W["router_bias"] = t
    if s.attn == "kda":
        t = torch.empty((3 * s.q_dim, s.conv_width), dtype=torch.float32, device=device)
        fill_f32(t, seed, gen.tensor_id("conv_w", layer), s.conv_std)
        W["conv_taps"] = t
    return W


def _u16(shape, device):
    return torch.zeros(shape, dtype=torch.int16, device=device)


def kv_cache(s: LayerShape, seed: int = 0, layer: int = 0, device="cuda", fill_len=None) -> dict:
    """A prefilled cache: positions 0..fill_len-1 (default cache_len) hold seeded values, the rest zero."""
    n = s.cache_len if fill_len is None else fill_len
    C = {}
    if s.attn == "kda":
        st = torch.empty((s.n_heads, s.head_dim, s.head_dim), dtype=torch.float32, device=device)
        fill_f32(st, seed, gen.tensor_id("kda_state", layer), s.state_std)
        ring = torch.empty((s.conv_width - 1, 3 * s.q_dim), dtype=torch.float32, device=device)
        fill_f32(ring, seed, gen.tensor_id("conv_state", layer), s.cache_std)
        C["kda_state"], C["conv_ring"] = st, ring
        return C
    if s.attn == "gqa":
        for kind, key in (("k_cache", "k"), ("v_cache", "v")):
            t = _u16((s.n_kv_heads, s.max_seq, s.head_dim), device)
            fill_bf16_cache(t, s.n_kv_heads, n, s.max_seq, s.head_dim, seed, gen.tensor_id(kind, layer), s.cache_std)
            C[key] = t
    else:
        t = _u16((s.max_seq, s.latent_dim), device)
        fill_bf16_cache(t, 1, n, s.max_seq, s.latent_dim, seed, gen.tensor_id("latent", layer), s.cache_std)
        C["latent"] = t
        if s.index_topk:
            codes = torch.zeros((s.max_seq, s.index_dim), dtype=torch.uint8, device=device)
            scales = torch.zeros(s.max_seq, dtype=torch.float32, device=device)
            fill_fp8_rows(codes, scales, n, seed, gen.tensor_id("index_k", layer), s.cache_std)
            C["index_codes"], C["index_scales"] = codes, scales
    return C


def input_hidden(s: LayerShape, seed: int = 0, step: int = 0, layer: int = 0, device="cuda") -> torch.Tensor:
    t = _u16((s.hidden,), device)
    _chk(lib().synth_fill_bf16_3d(ctypes.c_void_p(t.data_ptr()), 1, 1, 1, s.hidden, seed,
                                  gen.tensor_id("x", layer, step), s.x_std, _stream()), "input_hidden")
    return t


def embedding(m: ModelShape, seed: int = 0, device="cuda") -> torch.Tensor:
    t = _u16((m.vocab, m.layer.hidden), device)
    fill_bf16_matrix(t, seed, gen.tensor_id("embed"), m.emb_std)
    return t


def head(m: ModelShape, seed: int = 0, device="cuda") -> dict:
    H, V = m.layer.hidden, m.vocab
    if m.head_fmt == "fp8":
        codes = torch.empty((V, H), dtype=torch.uint8, device=device)
        scales = torch.empty((-(-V // 128), -(-H // 128)), dtype=torch.float32, device=device)
        fill_fp8_matrix(codes, scales, seed, gen.tensor_id("head"), m.layer.w_std)
        return {"fmt": "fp8", "data": codes, "scales": scales}
    t = _u16((V, H), device)
    fill_bf16_matrix(t, seed, gen.tensor_id("head"), m.layer.w_std)
    return {"fmt": "bf16", "data": t, "scales": None}


def final_norm(m: ModelShape, seed: int = 0, device="cuda") -> torch.Tensor:
    t = torch.empty(m.layer.hidden, dtype=torch.float32, device=device)
    fill_f32(t, seed, gen.tensor_id("final_norm"), m.layer.norm_std, mean=1.0)
    return t
