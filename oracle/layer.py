"""Plain fp64 CPU oracle of one batch-1 decode layer.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's CPU
baseline use it; the HIP library shares no code with it and never calls it.

What is computed, and where the pages describe it:

* The layer order RMSNorm -> projections (GEMM/GEMV) -> (sparse) attention ->
  output projection + residual follows the description of an attention layer's
  workers in the TileRT article ("Ultra-High Interactivity on NVIDIA GPUs? TileRT on
  InferenceX", section "But What Exactly is TileRT?"), and the decode step reading a
  growing KV cache follows its section "PD Disaggregated Engine with vLLM and TileRT".
* Absorbed MLA is named in the Kimi K3 article's section on Kimi Linear ("absorption
  trick"); this oracle computes MLA *non-absorbed* (per-head keys and values
  materialised), so the absorbed GPU form is checked against the plain definition.
* Top-k with a "biased router score" cutoff follows the Quantile Balancing section
  of the Kimi K3 article; the bias steers selection only and the gates use the
  unbiased sigmoid scores.
* SwiGLU experts with three matrix products per expert follow the LatentMoE
  derivation in the Kimi K3 article ("Up projection / Gate projection / Down
  projection"); the shared expert next to the routed ones follows the vLLM Kimi K3
  backend article, section "Four changes drive the gains" (sharded MoE routing).
* The indexer that scores every cached token and keeps the top 2048 follows the
  "Sparse Indexer worker" of the TileRT article (section "But What Exactly is
  TileRT?") and the DeepSeek sparse attention mentioned in the Kimi K3 article.
* KDA linear attention follows the Kimi K3 article, section "FlashKDA Algorithm" (the
  decode recurrence u_t = beta_t (v_t - (D_t S_{t-1})^T k_t), S_t = D_t S_{t-1} + k_t u_t^T,
  o_t^T = q_t^T S_t with D_t the diagonal decay, and the cumulative decay written with
  exp2), and the paragraph after it in "Kimi Linear" (linear projections and a short
  convolution for q, k and v, L2-normalised q and k, a low-rank decay projection, a down
  projection for beta, a per-head output norm and an output gate that is a linear layer,
  then the output projection that mixes the heads).

The pages fix none of the formulas below; each reading taken where they are silent
is listed in the module-level table ``READINGS``.

Storage rounding that is part of the method (and therefore done here too): the
appended cache row is stored as bf16 (the indexer key as FP8 + scale), and the
layer output is a bf16 vector. Everything else is fp64.

Indexer decision path: the selection is an integer result decided by floating point,
so the values that feed it are taken at the precision the kernel stores them in:
``a`` and ``c_q`` as fp32, ``q_I`` as bf16, head weights ``w`` and the new key as fp32,
key codes as FP8; the score is then evaluated in fp64 in one fixed order with plain
multiplies and adds.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from . import numerics as nx

READINGS = {
    "cache_len": "a cache of N tokens holds positions 0..N-1; the decode token is written at p=N and attends over N+1 rows",
    "rope": "interleaved pairs (2i, 2i+1), theta_i = base^(-2i/d_rot), base 10000; GQA rotates whole heads, MLA only the 64 rope dims",
    "eps_gamma": "eps = 1e-6 everywhere; gains gamma = 1 + 0.02 N(0,1)",
    "gqa_groups": "q head h uses kv head floor(h * n_kv / n_q) (contiguous groups)",
    "mla_dims": "qk_nope 128, rope 64, v 128, scale 1/sqrt(192); RMSNorm on c_q and c_kv",
    "sparse_shapes": "sparse workload: hidden 4096, 32 heads, MLA 512+64 latent, q_lora 1536, bf16 weights, 64-expert MoE top-8 softmax, inter 1536, 1 shared",
    "indexer": "q_I = bf16(W_qI c_q) [8x64], w = W_w a [8], k_I = W_kI a [64] -> FP8 with scale amax/448; "
               "score_t = sum_h w_h * max(0, s_t * sum_i q_I[h,i] dec(code_t[i])), fp64, i then h ascending, no FMA; "
               "the current token is a candidate; top-2048 by (score desc, index asc)",
    "router": "softmax router: logits r = W_r b, top-8 by (r desc, idx asc), gates = softmax(r[sel]); "
              "sigmoid router: s = sigmoid(r), top-8 by (s + bias desc, idx asc), gates = s[sel]/sum(s[sel])",
    "shared_expert": "shared expert has the routed width and gate weight 1; no routed scaling factor",
    "fp8": "OCP E4M3FN, fp32 scale per 128x128 block of [out, in] (edge blocks their own), weight-only",
    "ties": "every top-k breaks ties to the lower index",
    "output": "the layer output is stored as bf16; multi-layer stacks pass bf16 hidden states",
    "kda": "32 heads of 128 key/value channels at hidden 6144; q, k, v = causal depthwise convolution (width 4, no "
           "activation; taps fp32, the last tap on the current position; the previous projection outputs are kept as "
           "fp32 in a ring indexed by position mod 3) of W_q a, W_k a, W_v a; q and k L2-normalised per head "
           "(eps 1e-6) and q scaled by head_dim^-1/2; beta = sigmoid(W_beta a) per head; log2 decay "
           "g = -softplus(W_aup W_adown a) per key channel (rank 128), D_t = diag(2^g); fp32 state [head][key][value] "
           "stored after every step; o per head RMSNorm-ed (gain [head_dim], eps 1e-6) and multiplied by "
           "sigmoid(W_g a); y = W_o concat(o)",
}


class Counted:
    """Wraps a weight source and counts the storage bytes of every distinct tensor read."""

    def __init__(self, src):
        self.src = src
        self.bytes = 0
        self._seen = set()

    def _count(self, key, n):
        if key not in self._seen:
            self._seen.add(key)
            self.bytes += n

    def matrix(self, name, expert=0):
        m = self.src.matrix(name, expert)
        if m["fmt"] == "lut3":
            self._count((name, expert), m["idx"].size + m["codebook"].size)
        elif m["fmt"] == "fp8":
            self._count((name, expert), m["codes"].size + 4 * m["scales"].size)
        else:
            self._count((name, expert), 2 * m["bits"].size)
        return m

    def norm(self, name):
        g = self.src.norm(name)
        self._count(("norm", name), 4 * g.size)
        return g

    def router_bias(self):
        b = self.src.router_bias()
        self._count(("router_bias",), 4 * b.size)
        return b

    def conv_weights(self):
        w = self.src.conv_weights()
        self._count(("conv_w",), 4 * w.size)
        return w


def weight_f64(m: Dict) -> np.ndarray:
    if m["fmt"] == "lut3":
        return nx.dequant_lut3(m["idx"], m["codebook"])
    if m["fmt"] == "fp8":
        return nx.dequant_fp8_block(m["codes"], m["scales"])
    return nx.bf16_to_f64(m["bits"])


def _linear(W, name, v, expert=0):
    return weight_f64(W.matrix(name, expert)) @ v


# ---------------------------------------------------------------------------
# attention families
# ---------------------------------------------------------------------------
def gqa_attention(s, W, cache, a, pos, rec):
    """MHA/GQA: q,k,v projections, RoPE, cache append, softmax attention, concat heads."""
    hd, nh, nkv = s.head_dim, s.n_heads, s.n_kv_heads
    q = _linear(W, "wq", a).reshape(nh, hd)
    k = _linear(W, "wk", a).reshape(nkv, hd)
    v = _linear(W, "wv", a).reshape(nkv, hd)
    q = nx.rope(q, pos, s.rope_base)
    k = nx.rope(k, pos, s.rope_base)
    k_st = nx.round_to_bf16(k)
    v_st = nx.round_to_bf16(v)
    rec["q"], rec["k_new"], rec["v_new"] = q, k_st, v_st
    K = np.concatenate([nx.bf16_to_f64(cache["k"][:, :pos, :]), k_st[:, None, :]], axis=1)
    V = np.concatenate([nx.bf16_to_f64(cache["v"][:, :pos, :]), v_st[:, None, :]], axis=1)
    rec["kv_bytes_read"] = 2 * K.size * 2
    rec["kv_bytes_written"] = 2 * (k_st.size + v_st.size)
    o = np.empty((nh, hd))
    for h in range(nh):
        g = (h * nkv) // nh
        sc = K[g] @ q[h] / math.sqrt(hd)
        p = nx.softmax(sc)
        o[h] = p @ V[g]
    rec["o"] = o
    return _linear(W, "wo", o.reshape(-1))


def indexer_select(s, W, cache, a, pos, rec):
    """Score every cached token (and the new one) and keep the top index_topk positions.

    The inputs of the score are formed from fp32 ``a`` and fp32 ``c_q`` (recomputed from
    fp32 ``a``), at the precision the kernel holds them in; see the module docstring.
    """
    a32 = nx.round_to_f32(a)
    cq32 = nx.round_to_f32(nx.rmsnorm(_linear(W, "w_dq", a32), W.norm("q_norm"), s.eps))
    q_i = nx.round_to_bf16(_linear(W, "w_qi", cq32)).reshape(s.index_heads, s.index_dim)
    w = nx.round_to_f32(_linear(W, "w_w", a32))
    k_i = nx.round_to_f32(_linear(W, "w_ki", a32))
    # FP8 quantisation of the new key: fp32 scale amax/448, fp32 quotient, RNE, saturate
    k32 = k_i.astype(np.float32)
    amax = np.float32(np.max(np.abs(k32)))
    sig = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    quo = np.clip(k32 / sig, np.float32(-448.0), np.float32(448.0))
    code_new = nx.e4m3_encode_f32(quo)
    rec["q_i"], rec["w_idx"], rec["k_i"] = q_i, w, k_i
    rec["index_code_new"], rec["index_scale_new"] = code_new, sig
    codes = np.concatenate([cache["index_codes"][:pos], code_new[None, :]], axis=0)
    scales = np.concatenate([np.asarray(cache["index_scales"][:pos], np.float32), [sig]]).astype(np.float64)
    dec = nx.E4M3[codes]                         # [T, 64], exact
    T = codes.shape[0]
    score = np.zeros(T)
    for h in range(s.index_heads):
        d = np.zeros(T)
        for i in range(s.index_dim):
            d = d + q_i[h, i] * dec[:, i]        # separate multiply and add, i ascending
        r = scales * d
        r = np.maximum(r, 0.0)
        score = score + w[h] * r
    rec["index_score"] = score
    rec["index_bytes_read"] = T * (s.index_dim + 4)
    k = min(s.index_topk, T)
    sel = np.sort(nx.topk_desc(score, k))
    rec["index_sel"] = sel
    return sel


def kda_state_step(S, q, k, v, beta, alpha):
    """One decode step of a KDA head in the order of the recurrence: S' = diag(alpha) S,
    u = beta (v - S'^T k), S_new = S' + k u^T, o = S_new^T q. S is [key][value]."""
    Sd = alpha[:, None] * S
    u = beta * (v - Sd.T @ k)
    S_new = Sd + np.outer(k, u)
    return S_new, S_new.T @ q


def softplus(z):
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def kda_attention(s, W, cache, a, pos, rec):
    """KDA linear attention for one token: convolution ring and per-head state advance in place."""
    nh, D = s.n_heads, s.head_dim
    qd = nh * D
    cw = s.conv_width
    x = np.concatenate([_linear(W, "wq", a), _linear(W, "wk", a), _linear(W, "wv", a)])   # [3 qd]
    x32 = nx.round_to_f32(x)                                   # the stored projection outputs
    taps = np.asarray(W.conv_weights(), np.float64)           # [3 qd][cw]
    ring = np.asarray(cache["conv_ring"], np.float64)        # [cw-1][3 qd]
    y = taps[:, cw - 1] * x32
    for j in range(1, cw):                                     # tap cw-1-j sees position pos-j
        y = y + taps[:, cw - 1 - j] * ring[(pos - j) % (cw - 1)]
    q = y[:qd].reshape(nh, D)
    k = y[qd:2 * qd].reshape(nh, D)
    v = y[2 * qd:].reshape(nh, D)
    q = q / np.sqrt(np.sum(q * q, axis=1, keepdims=True) + s.eps) / math.sqrt(D)
    k = k / np.sqrt(np.sum(k * k, axis=1, keepdims=True) + s.eps)
    beta = nx.sigmoid(_linear(W, "w_beta", a))                # [nh]
    g = -softplus(_linear(W, "w_aup", _linear(W, "w_adown", a))).reshape(nh, D)
    alpha = np.exp2(g)
    gate = nx.sigmoid(_linear(W, "w_g", a)).reshape(nh, D)
    gam = np.asarray(W.norm("o_norm"), np.float64)
    S = np.asarray(cache["kda_state"], np.float64)
    o = np.empty((nh, D))
    S_new = np.empty_like(S)
    for h in range(nh):
        S_new[h], o[h] = kda_state_step(S[h], q[h], k[h], v[h], beta[h], alpha[h])
    rec["kda_q"], rec["kda_k"], rec["kda_v"], rec["kda_beta"], rec["kda_alpha"] = q, k, v, beta, alpha
    rec["kda_x32"] = x32
    rec["kda_state_new"] = nx.round_to_f32(S_new)
    rec["o_raw"] = o
    on = np.stack([nx.rmsnorm(o[h], gam, s.eps) for h in range(nh)]) * gate
    rec["o"] = on
    rec["kv_bytes_read"] = 4 * S.size + 4 * ring.size
    rec["kv_bytes_written"] = 4 * S.size + 4 * 3 * qd
    return _linear(W, "wo", on.reshape(-1))


def mla_attention(s, W, cache, a, pos, rec):
    """MLA, computed without absorption: per-head keys/values are materialised from c_kv."""
    nh, nope, rd, vd, L = s.n_heads, s.nope_dim, s.rope_dim, s.v_dim, s.kv_lora
    c_q = nx.rmsnorm(_linear(W, "w_dq", a), W.norm("q_norm"), s.eps)
    qf = _linear(W, "w_uq", c_q).reshape(nh, nope + rd)
    q_nope = qf[:, :nope]
    q_rope = nx.rope(qf[:, nope:], pos, s.rope_base)
    kv = _linear(W, "w_dkv", a)
    c_kv = nx.rmsnorm(kv[:L], W.norm("kv_norm"), s.eps)
    k_rope = nx.rope(kv[L:], pos, s.rope_base)
    row = nx.round_to_bf16(np.concatenate([c_kv, k_rope]))
    rec["c_q"], rec["q_nope"], rec["q_rope"], rec["latent_new"] = c_q, q_nope, q_rope, row
    C = np.concatenate([nx.bf16_to_f64(cache["latent"][:pos]), row[None, :]], axis=0)   # [T, L+rd]
    T = C.shape[0]
    rows = np.arange(T)
    if s.index_topk:
        rows = indexer_select(s, W, cache, a, pos, rec)
    Cs = C[rows]
    rec["kv_bytes_read"] = Cs.size * 2
    rec["kv_bytes_written"] = row.size * 2 + (s.index_dim + 4 if s.index_topk else 0)
    W_uk = weight_f64(W.matrix("w_uk")).reshape(nh, nope, L)
    W_uv = weight_f64(W.matrix("w_uv")).reshape(nh, vd, L)
    ckv, kr = Cs[:, :L], Cs[:, L:]
    scale = 1.0 / math.sqrt(nope + rd)
    o = np.empty((nh, vd))
    for h in range(nh):
        k_nope = ckv @ W_uk[h].T                 # [T, nope]   key of head h
        v_h = ckv @ W_uv[h].T                    # [T, vd]     value of head h
        sc = (k_nope @ q_nope[h] + kr @ q_rope[h]) * scale
        p = nx.softmax(sc)
        o[h] = p @ v_h
    rec["o"] = o
    return _linear(W, "wo", o.reshape(-1))


# ---------------------------------------------------------------------------
# FFN
# ---------------------------------------------------------------------------
def expert(W, e, b, rec=None, slot=0):
    """SwiGLU expert e on b; with ``rec``, its activation m = silu(g) * u is recorded under
    rec["m"][slot] (slot = rank of a routed expert in the selection, then the shared ones)."""
    g = _linear(W, "w_gate", b, e)
    u = _linear(W, "w_up", b, e)
    m = nx.silu(g) * u
    if rec is not None:
        rec.setdefault("m", {})[slot] = m
    return _linear(W, "w_down", m, e)


def route(s, W, b, rec):
    r = nx.bf16_to_f64(W.matrix("router")["bits"]) @ b
    rec["router_logits"] = r
    if s.router == "softmax":
        sel = nx.topk_desc(r, s.top_k)
        gates = nx.softmax(r[sel])
    else:
        sc = nx.sigmoid(r)
        bias = np.asarray(W.router_bias(), np.float64)
        sel = nx.topk_desc(sc + bias, s.top_k)
        gates = sc[sel] / np.sum(sc[sel])
    rec["router_sel"], rec["gates"] = sel, gates
    return sel, gates


def ffn(s, W, b, rec):
    if s.ffn == "dense":
        return expert(W, 0, b, rec, 0)
    sel, gates = route(s, W, b, rec)
    f = np.zeros(s.hidden)
    for slot, (e, g) in enumerate(zip(sel, gates)):
        f = f + g * expert(W, int(e), b, rec, slot)
    for j in range(s.n_shared):
        f = f + expert(W, s.n_experts + j, b, rec, s.top_k + j)
    return f


# ---------------------------------------------------------------------------
def decode_layer(s, W, cache, x_bits: np.ndarray, pos: int, record: Optional[dict] = None) -> dict:
    """Decode one token at position ``pos`` through one layer.

    ``W``: weight source (``matrix(name, expert)``, ``norm(name)``, ``router_bias()``).
    ``cache``: host arrays holding at least positions 0..pos-1 (bf16 bits; FP8 codes +
    fp32 scales for index keys). ``x_bits``: bf16 [hidden]. Returns a dict with ``out``
    (fp64 values of the bf16 output), ``out_bits`` and the intermediates.
    """
    rec = {} if record is None else record
    CW = Counted(W)
    h = nx.bf16_to_f64(x_bits)
    a = nx.rmsnorm(h, CW.norm("attn_norm"), s.eps)
    rec["a"] = a
    if s.attn == "gqa":
        y = gqa_attention(s, CW, cache, a, pos, rec)
    elif s.attn == "kda":
        y = kda_attention(s, CW, cache, a, pos, rec)
    else:
        y = mla_attention(s, CW, cache, a, pos, rec)
    h2 = h + y
    b = nx.rmsnorm(h2, CW.norm("ffn_norm"), s.eps)
    rec["y"], rec["h2"], rec["b"] = y, h2, b
    f = ffn(s, CW, b, rec)
    out = h2 + f
    rec["f"] = f
    rec["out_f64"] = out
    rec["out"] = nx.round_to_bf16(out)
    rec["out_bits"] = nx.bf16_bits_of(rec["out"])
    rec["weight_bytes"] = CW.bytes
    return rec


def append_to_cache(s, cache, rec, pos):
    """Write the rows the step appended into a host cache (mutates ``cache``)."""
    if s.attn == "gqa":
        cache["k"][:, pos, :] = nx.bf16_bits_of(rec["k_new"])
        cache["v"][:, pos, :] = nx.bf16_bits_of(rec["v_new"])
    elif s.attn == "kda":
        cache["kda_state"][...] = rec["kda_state_new"]
        cache["conv_ring"][pos % (s.conv_width - 1)] = rec["kda_x32"]
    else:
        cache["latent"][pos] = nx.bf16_bits_of(rec["latent_new"])
        if s.index_topk:
            cache["index_codes"][pos] = rec["index_code_new"]
            cache["index_scales"][pos] = rec["index_scale_new"]
