"""Seeded synthetic inputs: the host (NumPy) half of one counter-based generator.

This module makes weights, caches and input vectors. It is shared by the CPU
oracle's tests and by the HIP path's tests and benchmark, and it holds none of the
decode method's arithmetic: no norms, projections, attention, routing or selection.
The device half (``synth/csrc/synth_gen.hip``) implements the same definition and
the tests check that both write identical bytes.

Definition (every step is integer or a single correctly rounded fp32 operation, so
host and device agree bit for bit):

* SplitMix64 mixer ``mix(z)`` (Steele, Lea and Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014; the constants of Vigna's
  ``splitmix64.c``): ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31``.
* Stream key of tensor ``tid`` under ``seed``:
  ``key = mix(seed * G + mix(tid * G + G))`` with ``G = 0x9E3779B97F4A7C15``, mod 2**64.
* Raw 64-bit draw ``i``: ``r_i = mix(key + (i + 1) * G)``.
* Approximate standard normal (Irwin-Hall of four 16-bit lanes):
  ``n_i = fp32(l0 + l1 + l2 + l3 - 131070) * INV_SIGMA`` where ``l_j`` are the four
  16-bit lanes of ``r_i`` and ``INV_SIGMA = 0x1.bb67aep-16`` = fp32(1/sqrt(4*(2**32-1)/12)).
  The integer is exact in fp32; the product is one fp32 multiply.
* Scaled value: ``v = n * std`` (one fp32 multiply), or ``v = (n * std) + mean``
  (two fp32 operations, no fused multiply-add) for norm gains.
* bf16 storage: round-to-nearest-even of the fp32 value.
* FP8 storage (OCP E4M3FN) with an fp32 scale per 128x128 block of an ``[out, in]``
  matrix (edge blocks cover what is left): ``scale = amax / 448`` (fp32 division;
  1.0 when the block is all zero), ``q = v / scale`` (fp32 division), clamped to
  [-448, 448], then rounded to the nearest E4M3FN value, ties to the even code; the
  sign bit is the sign of ``q`` (a negative value that rounds to zero gives 0x80).
* Index-key rows use the same FP8 rule with one scale per row.
* Lookup-table (LUT3) matrices [out, in] (out a multiple of 8, in of 128): draw i = n*in + k
  gives weight (n, k) the index r_i & 7; draw i = out*in + b gives block b = (n/8)*(in/64) +
  k/64 its spread s_b = 0.75 + (r_i >> 40) * 2**-24 * 0.5 (fp32 operations), and the block's
  codebook entry e is the E4M3FN code of fp32(fp32(std * Z_e) * s_b), Z_e the fixed fp32
  normal quantiles below. Storage: codebook bytes [out/8][in/64][8]; indices as three bit
  planes per group of 128 weights of a row: 48 bytes, plane p = bytes [16p, 16p + 16) as four
  little-endian u32, bit j of word d = bit p of the index of weight 32d + j of the group.
"""
from __future__ import annotations

import os

import numpy as np

from .configs import LayerShape, ModelShape

U64 = np.uint64
G = U64(0x9E3779B97F4A7C15)
M1 = U64(0xBF58476D1CE4E5B9)
M2 = U64(0x94D049BB133111EB)
INV_SIGMA = np.float32(float.fromhex("0x1.bb67aep-16"))
FP8_MAX = np.float32(448.0)

# tensor kinds (part of the tensor id)
KIND = {
    "x": 1, "attn_norm": 2, "wq": 3, "wk": 4, "wv": 5, "wo": 6,
    "w_dq": 7, "q_norm": 8, "w_uq": 9, "w_dkv": 10, "kv_norm": 11, "w_uk": 12, "w_uv": 13,
    "w_qi": 14, "w_w": 15, "w_ki": 16,
    "ffn_norm": 17, "w_gate": 18, "w_up": 19, "w_down": 20, "router": 21, "router_bias": 22,
    "k_cache": 23, "v_cache": 24, "latent": 25, "index_k": 26,
    "embed": 27, "final_norm": 28, "head": 29, "token": 30,
    "w_g": 31, "w_beta": 32, "w_adown": 33, "w_aup": 34, "conv_w": 35, "o_norm": 36, "kda_state": 37,
    "conv_state": 38,
}
POS_STRIDE = 1 << 20  # cache element index = ((head << 20) | pos) * row + col


def tensor_id(kind: str, layer: int = 0, sub: int = 0) -> int:
    return (int(layer) << 40) | (KIND[kind] << 24) | int(sub)


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> U64(30))) * M1
    z = (z ^ (z >> U64(27))) * M2
    return z ^ (z >> U64(31))


def stream_key(seed: int, tid: int) -> np.uint64:
    with np.errstate(over="ignore"):
        t = np.array([tid], dtype=U64)
        s = np.array([seed], dtype=U64)
        return _mix(s * G + _mix(t * G + G))[0]


def raw_u64(seed: int, tid: int, index: np.ndarray) -> np.ndarray:
    key = np.array([stream_key(seed, tid)], dtype=U64)
    i = np.asarray(index, dtype=U64)
    with np.errstate(over="ignore"):
        return _mix(key + (i + U64(1)) * G)


def normal_f32(seed: int, tid: int, index: np.ndarray) -> np.ndarray:
    r = raw_u64(seed, tid, index)
    m = U64(0xFFFF)
    s = (r & m) + ((r >> U64(16)) & m) + ((r >> U64(32)) & m) + (r >> U64(48))
    s = s.astype(np.int64) - 131070
    return s.astype(np.float32) * INV_SIGMA


def _scaled_normal_1(seed, tid, index, std, mean):
    v = normal_f32(seed, tid, index) * np.float32(std)
    if mean is not None:
        v = v + np.float32(mean)
    return v


_POOL = None


def scaled_normal(seed, tid, index, std, mean=None) -> np.ndarray:
    """std * N(0,1) (+ mean) at the given element indices (large requests run in threads)."""
    index = np.asarray(index, dtype=U64)
    n = index.size
    if n < (1 << 21):
        return _scaled_normal_1(seed, tid, index, std, mean)
    global _POOL
    if _POOL is None:
        from concurrent.futures import ThreadPoolExecutor
        _POOL = ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1))
    flat = index.reshape(-1)
    parts = np.array_split(np.arange(n), 16)
    outs = list(_POOL.map(lambda ix: _scaled_normal_1(seed, tid, flat[ix], std, mean), parts))
    return np.concatenate(outs).reshape(index.shape)


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + U64(0x7FFF) + ((b >> U64(16)) & U64(1))) >> U64(16)
    return b.astype(np.uint16)


# --- E4M3FN storage rule (input generation only) ---------------------------
def _e4m3_positive_table() -> np.ndarray:
    vals = np.zeros(127, dtype=np.float64)
    for c in range(127):
        e, m = c >> 3, c & 7
        vals[c] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_E4M3_POS = _e4m3_positive_table()


def f32_to_e4m3_codes(q: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code of fp32 values already clamped to [-448, 448], ties to the even code.

    Normal range (|q| >= 2^-6): round the fp32 pattern to 3 mantissa bits (ties to even)
    and re-bias the exponent from 127 to 7. Subnormal range: the code is |q| * 2^9
    rounded half to even. Sign bit = sign of q.
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    bits = q.view(np.uint32)
    mag = bits & np.uint32(0x7FFFFFFF)
    rounded = (mag + np.uint32(0x7FFFF) + ((mag >> np.uint32(20)) & np.uint32(1))) >> np.uint32(20)
    normal = rounded.astype(np.int64) - (120 << 3)
    sub = np.rint(np.abs(q) * np.float32(512.0)).astype(np.int64)
    code = np.where(mag >= np.uint32(0x3C800000), normal, sub)       # 0x3C800000 = 2^-6
    code = np.minimum(code, 126)
    sign = (bits >> np.uint32(31)).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def _f32_to_e4m3_codes_table(q: np.ndarray) -> np.ndarray:
    """Same rule by nearest-value search in the table of E4M3FN values (used to cross-check)."""
    q = np.asarray(q, dtype=np.float32).astype(np.float64)
    a = np.abs(q)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(a >= _E4M3_POS[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    sign = np.signbit(q).astype(np.uint8) << 7
    return code | sign


def fp8_block_quantize(v: np.ndarray, block: int = 128):
    """fp32 [out, in] -> (uint8 codes [out, in], fp32 scales [ceil(out/128), ceil(in/128)])."""
    out_dim, in_dim = v.shape
    nb_o, nb_i = -(-out_dim // block), -(-in_dim // block)
    if (out_dim, in_dim) == (nb_o * block, nb_i * block):
        pad = np.asarray(v, dtype=np.float32)
    else:
        pad = np.zeros((nb_o * block, nb_i * block), dtype=np.float32)
        pad[:out_dim, :in_dim] = v
    blocks = pad.reshape(nb_o, block, nb_i, block)
    amax = np.abs(blocks).max(axis=(1, 3)).astype(np.float32)
    scales = np.where(amax > 0, amax / FP8_MAX, np.float32(1.0)).astype(np.float32)
    q = np.minimum(np.maximum(blocks / scales[:, None, :, None], -FP8_MAX), FP8_MAX)
    codes = f32_to_e4m3_codes(q).reshape(nb_o * block, nb_i * block)[:out_dim, :in_dim]
    return np.ascontiguousarray(codes), scales


# fp32 normal quantiles at (e + 0.5) / 8, the eight codebook positions before the block spread
LUT_Z = np.array([-1.5341205, -0.88714653, -0.48877642, -0.15731068, 0.15731068, 0.48877642, 0.88714653,
                  1.5341205], dtype=np.float32)


def lut3_matrix(seed: int, tid: int, out_dim: int, in_dim: int, std: float):
    """(indices uint8 [out, 3*in/8] in bit planes, codebook uint8 [out/8, in/64, 8]) of a LUT3 matrix."""
    assert out_dim % 8 == 0 and in_dim % 128 == 0
    n_w = out_dim * in_dim
    idx = (raw_u64(seed, tid, np.arange(n_w, dtype=np.uint64)) & U64(7)).astype(np.uint8).reshape(out_dim, in_dim)
    nb = (out_dim // 8) * (in_dim // 64)
    rb = raw_u64(seed, tid, np.arange(n_w, n_w + nb, dtype=np.uint64))
    u = (rb >> U64(40)).astype(np.float32) * np.float32(2.0 ** -24)
    spread = np.float32(0.75) + u * np.float32(0.5)
    vals = (np.float32(std) * LUT_Z)[None, :] * spread[:, None]          # [nb, 8] fp32
    cb = f32_to_e4m3_codes(vals.astype(np.float32)).reshape(out_dim // 8, in_dim // 64, 8)
    g = idx.reshape(out_dim, in_dim // 128, 4, 32)                        # [row, group, word, bit]
    planes = np.zeros((out_dim, in_dim // 128, 3, 4), dtype=np.uint32)
    for p in range(3):
        bits = ((g >> p) & 1).astype(np.uint32)
        planes[:, :, p, :] = np.sum(bits << np.arange(32, dtype=np.uint32), axis=3, dtype=np.uint32)
    packed = planes.view(np.uint8).reshape(out_dim, 3 * in_dim // 8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(cb)


def fp8_row_quantize(v: np.ndarray):
    """fp32 [rows, d] -> (codes [rows, d], scales [rows]) with one scale per row."""
    amax = np.abs(v).max(axis=1).astype(np.float32)
    scales = np.where(amax > 0, amax / FP8_MAX, np.float32(1.0)).astype(np.float32)
    q = np.clip(v.astype(np.float32) / scales[:, None], -FP8_MAX, FP8_MAX)
    return f32_to_e4m3_codes(q), scales


# ---------------------------------------------------------------------------
# Tensor catalogue of one layer
# ---------------------------------------------------------------------------
def layer_matrices(s: LayerShape):
    """name -> (out, in, std kind) of every linear weight; expert weights are per expert."""
    m = {}
    H = s.hidden
    if s.attn == "gqa":
        m["wq"] = (s.n_heads * s.head_dim, H)
        m["wk"] = (s.n_kv_heads * s.head_dim, H)
        m["wv"] = (s.n_kv_heads * s.head_dim, H)
    elif s.attn == "kda":
        qd = s.n_heads * s.head_dim
        m["wq"] = (qd, H)
        m["wk"] = (qd, H)
        m["wv"] = (qd, H)
        m["w_g"] = (qd, H)                # output gate
        m["w_beta"] = (s.n_heads, H)      # delta-rule strength per head
        m["w_adown"] = (s.kda_rank, H)    # low-rank decay projection
        m["w_aup"] = (qd, s.kda_rank)
    else:
        m["w_dq"] = (s.q_lora, H)
        m["w_uq"] = (s.n_heads * (s.nope_dim + s.rope_dim), s.q_lora)
        m["w_dkv"] = (s.kv_lora + s.rope_dim, H)
        m["w_uk"] = (s.n_heads * s.nope_dim, s.kv_lora)
        m["w_uv"] = (s.n_heads * s.v_dim, s.kv_lora)
        if s.index_topk:
            m["w_qi"] = (s.index_heads * s.index_dim, s.q_lora)
            m["w_w"] = (s.index_heads, H)
            m["w_ki"] = (s.index_dim, H)
    m["wo"] = (H, s.o_dim)
    m["w_gate"] = (s.inter, H)
    m["w_up"] = (s.inter, H)
    m["w_down"] = (H, s.inter)
    if s.ffn == "moe":
        m["router"] = (s.n_experts, H)
    return m


def layer_norms(s: LayerShape):
    n = {"attn_norm": s.hidden, "ffn_norm": s.hidden}
    if s.attn == "mla":
        n["q_norm"] = s.q_lora
        n["kv_norm"] = s.kv_lora
    if s.attn == "kda":
        n["o_norm"] = s.head_dim
    return n


EXPERT_MATS = ("w_gate", "w_up", "w_down")
# Linear weights that stay bf16 in an FP8 layer: the router and the indexer's small
# head-weight projection feed exact selections.
BF16_ALWAYS = ("router", "w_w")


def weight_format(s: LayerShape, name: str) -> str:
    if name in BF16_ALWAYS:
        return "bf16"
    if name in EXPERT_MATS and s.expert_fmt:
        return s.expert_fmt
    return s.wfmt


class LayerWeights:
    """Lazily generated storage arrays of one layer.

    ``matrix(name, expert)`` returns ``{"fmt": "bf16", "bits": uint16[out, in]}`` or
    ``{"fmt": "fp8", "codes": uint8[out, in], "scales": float32[nbo, nbi]}``.
    ``norm(name)`` returns float32 gains, ``router_bias()`` float32 [n_experts].
    Expert ``n_experts + j`` is shared expert ``j``.
    """

    def __init__(self, shape: LayerShape, seed: int = 0, layer: int = 0, cache_size: int = 64):
        self.s, self.seed, self.layer = shape, seed, layer
        self._cache = {}
        self._cache_size = cache_size
        self.mats = layer_matrices(shape)

    def _std(self, name):
        return self.s.router_std if name == "router" else self.s.w_std

    def matrix(self, name: str, expert: int = 0):
        key = (name, expert)
        if key in self._cache:
            return self._cache[key]
        out_dim, in_dim = self.mats[name]
        sub = expert if name in EXPERT_MATS else 0
        tid = tensor_id(name, self.layer, sub)
        if weight_format(self.s, name) == "lut3":
            idx, cb = lut3_matrix(self.seed, tid, out_dim, in_dim, self._std(name))
            res = {"fmt": "lut3", "idx": idx, "codebook": cb}
            if len(self._cache) >= self._cache_size:
                self._cache.pop(next(iter(self._cache)))
            self._cache[key] = res
            return res
        v = scaled_normal(self.seed, tid, np.arange(out_dim * in_dim, dtype=np.uint64),
                          self._std(name)).reshape(out_dim, in_dim)
        if weight_format(self.s, name) == "fp8":
            codes, scales = fp8_block_quantize(v)
            res = {"fmt": "fp8", "codes": codes, "scales": scales}
        else:
            res = {"fmt": "bf16", "bits": f32_to_bf16_bits(v).reshape(out_dim, in_dim)}
        if len(self._cache) >= self._cache_size:
            self._cache.pop(next(iter(self._cache)))
        self._cache[key] = res
        return res

    def norm(self, name: str) -> np.ndarray:
        n = layer_norms(self.s)[name]
        return scaled_normal(self.seed, tensor_id(name, self.layer), np.arange(n, dtype=np.uint64),
                             self.s.norm_std, mean=1.0)

    def router_bias(self) -> np.ndarray:
        return scaled_normal(self.seed, tensor_id("router_bias", self.layer),
                             np.arange(self.s.n_experts, dtype=np.uint64), self.s.bias_std)

    def conv_weights(self) -> np.ndarray:
        """fp32 [3 * q_dim][conv_width] taps of the KDA causal convolution (q, k, v channels)."""
        n = 3 * self.s.q_dim * self.s.conv_width
        return scaled_normal(self.seed, tensor_id("conv_w", self.layer), np.arange(n, dtype=np.uint64),
                             self.s.conv_std).reshape(3 * self.s.q_dim, self.s.conv_width)


def input_hidden(shape: LayerShape, seed: int = 0, step: int = 0, layer: int = 0) -> np.ndarray:
    """bf16 bits [hidden] of a decode input vector."""
    v = scaled_normal(seed, tensor_id("x", layer, step), np.arange(shape.hidden, dtype=np.uint64),
                      shape.x_std)
    return f32_to_bf16_bits(v)


def _cache_index(head, pos, row, col):
    return ((np.uint64(head) << np.uint64(20)) | np.asarray(pos, dtype=np.uint64)[:, None]) \
        * np.uint64(row) + np.asarray(col, dtype=np.uint64)[None, :]


def kv_rows(shape: LayerShape, kind: str, head: int, positions, seed=0, layer=0) -> np.ndarray:
    """bf16 bits [len(positions), head_dim] of prefilled K or V rows of one kv head."""
    d = shape.head_dim
    idx = _cache_index(head, positions, d, np.arange(d))
    v = scaled_normal(seed, tensor_id(kind, layer), idx.ravel(), shape.cache_std)
    return f32_to_bf16_bits(v).reshape(len(positions), d)


def latent_rows(shape: LayerShape, positions, seed=0, layer=0) -> np.ndarray:
    """bf16 bits [len(positions), kv_lora + rope_dim] of prefilled MLA latent rows."""
    d = shape.latent_dim
    idx = _cache_index(0, positions, d, np.arange(d))
    v = scaled_normal(seed, tensor_id("latent", layer), idx.ravel(), shape.cache_std)
    return f32_to_bf16_bits(v).reshape(len(positions), d)


def index_key_rows(shape: LayerShape, positions, seed=0, layer=0):
    """(codes uint8 [n, index_dim], scales fp32 [n]) of prefilled indexer keys."""
    d = shape.index_dim
    idx = _cache_index(0, positions, d, np.arange(d))
    v = scaled_normal(seed, tensor_id("index_k", layer), idx.ravel(), shape.cache_std)
    return fp8_row_quantize(v.reshape(len(positions), d))


def full_cache(shape: LayerShape, seed=0, layer=0):
    """Host copies of a whole prefilled cache (for small shapes and for the oracle)."""
    pos = np.arange(shape.cache_len)
    out = {}
    if shape.attn == "gqa":
        out["k"] = np.stack([kv_rows(shape, "k_cache", g, pos, seed, layer) for g in range(shape.n_kv_heads)])
        out["v"] = np.stack([kv_rows(shape, "v_cache", g, pos, seed, layer) for g in range(shape.n_kv_heads)])
    else:
        out["latent"] = latent_rows(shape, pos, seed, layer)
        if shape.index_topk:
            out["index_codes"], out["index_scales"] = index_key_rows(shape, pos, seed, layer)
    return out


# --- model-level tensors (multi-layer workload) -----------------------------
def embedding_rows(model: ModelShape, tokens, seed=0) -> np.ndarray:
    H = model.layer.hidden
    tokens = np.asarray(tokens, dtype=np.uint64)
    idx = tokens[:, None] * np.uint64(H) + np.arange(H, dtype=np.uint64)[None, :]
    v = scaled_normal(seed, tensor_id("embed"), idx.ravel(), model.emb_std)
    return f32_to_bf16_bits(v).reshape(len(tokens), H)


def final_norm(model: ModelShape, seed=0) -> np.ndarray:
    H = model.layer.hidden
    return scaled_normal(seed, tensor_id("final_norm"), np.arange(H, dtype=np.uint64),
                         model.layer.norm_std, mean=1.0)


def head_matrix(model: ModelShape, seed=0, rows=None):
    """LM head [vocab, hidden]: FP8 codes + block scales (rows: optional row-block range)."""
    H, V = model.layer.hidden, model.vocab
    r0, r1 = (0, V) if rows is None else rows
    assert r0 % 128 == 0
    idx = (np.arange(r0, r1, dtype=np.uint64)[:, None] * np.uint64(H)
           + np.arange(H, dtype=np.uint64)[None, :])
    v = scaled_normal(seed, tensor_id("head"), idx.ravel(), model.layer.w_std).reshape(r1 - r0, H)
    if model.head_fmt == "fp8":
        codes, scales = fp8_block_quantize(v)
        return {"fmt": "fp8", "codes": codes, "scales": scales}
    return {"fmt": "bf16", "bits": f32_to_bf16_bits(v)}


def first_token(model: ModelShape, seed=0, step=0) -> int:
    r = raw_u64(seed, tensor_id("token", 0, step), np.arange(1, dtype=np.uint64))
    return int(r[0] % np.uint64(model.vocab))


def draft_tokens(model: ModelShape, n: int, seed=0, step=0) -> np.ndarray:
    r = raw_u64(seed, tensor_id("token", 1, step), np.arange(n, dtype=np.uint64))
    return (r % np.uint64(model.vocab)).astype(np.int64)


def padded_cache(shape: LayerShape, seed=0, layer=0, fill_len=None) -> dict:
    """Host copy of a prefilled cache with max_seq rows: positions 0..fill_len-1 (default
    cache_len) hold the seeded rows, the rest zero (the layout the device fill writes)."""
    n = shape.cache_len if fill_len is None else fill_len
    out = {}
    if shape.attn == "kda":
        return {"kda_state": kda_state(shape, seed, layer), "conv_ring": conv_state(shape, seed, layer)}
    if shape.attn == "gqa":
        pos = np.arange(n)
        for kind, key in (("k_cache", "k"), ("v_cache", "v")):
            z = np.zeros((shape.n_kv_heads, shape.max_seq, shape.head_dim), np.uint16)
            for g in range(shape.n_kv_heads):
                z[g, :n] = kv_rows(shape, kind, g, pos, seed, layer)
            out[key] = z
    else:
        z = np.zeros((shape.max_seq, shape.latent_dim), np.uint16)
        z[:n] = latent_rows(shape, np.arange(n), seed, layer)
        out["latent"] = z
        if shape.index_topk:
            codes = np.zeros((shape.max_seq, shape.index_dim), np.uint8)
            scales = np.zeros(shape.max_seq, np.float32)
            c, sc = index_key_rows(shape, np.arange(n), seed, layer)
            codes[:n], scales[:n] = c, sc
            out["index_codes"], out["index_scales"] = codes, scales
    return out


def kda_state(shape: LayerShape, seed=0, layer=0) -> np.ndarray:
    """fp32 [n_heads][head_dim][head_dim] prefilled KDA state (row: key channel, column: value)."""
    D = shape.head_dim
    n = shape.n_heads * D * D
    return scaled_normal(seed, tensor_id("kda_state", layer), np.arange(n, dtype=np.uint64),
                         shape.state_std).reshape(shape.n_heads, D, D)


def conv_state(shape: LayerShape, seed=0, layer=0) -> np.ndarray:
    """fp32 [conv_width - 1][3 * q_dim] ring of the last projection outputs (slot = position mod
    (conv_width - 1)), prefilled."""
    w = shape.conv_width - 1
    n = w * 3 * shape.q_dim
    return scaled_normal(seed, tensor_id("conv_state", layer), np.arange(n, dtype=np.uint64),
                         shape.cache_std).reshape(w, 3 * shape.q_dim)
