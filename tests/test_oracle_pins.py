"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a library routine (torch casts, torch RMSNorm,
scipy softmax), a closed form, brute force on tiny inputs, an algebraic identity that
uses a different formula (absorbed vs non-absorbed MLA, duplicated-kv GQA vs MHA), or a
number the pages print (tests/golden/page_worked_examples.json).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import accounting, numerics as nx
from oracle import layer as OL
from oracle import model as OM
from synth import configs, gen

from helpers import DictWeights, tiny_gqa, tiny_kda, tiny_mla

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_worked_examples.json")


# --------------------------------------------------------------------------- formats
def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    o = nx.E4M3[codes]
    both_nan = np.isnan(t) & np.isnan(o)
    assert np.all(both_nan | (t == o))
    assert set(np.nonzero(np.isnan(o))[0]) == {0x7F, 0xFF}
    assert o[0x7E] == 448.0 and o[0x01] == 2.0 ** -9 and o[0x08] == 2.0 ** -6 and o[0x38] == 1.0


def _e4m3_sweep():
    rng = np.random.default_rng(3)
    vals = nx.E4M3[:127]
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)
    q = np.concatenate([
        np.clip(rng.standard_normal(200000).astype(np.float32) * s, -448, 448) for s in (1e-3, 0.03, 1, 30, 300)
    ] + [vals.astype(np.float32), mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e4)),
         np.float32([0.0, 448.0, -448.0, 2 ** -10, 3 * 2 ** -11])])
    return np.clip(q, -448, 448).astype(np.float32)


def test_e4m3_encode_matches_torch_cast():
    q = _e4m3_sweep()
    t = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    o = nx.e4m3_encode_f32(q)
    # torch keeps the sign on zero as well
    assert np.array_equal(o, t)


def test_bf16_decode_and_round_match_torch():
    rng = np.random.default_rng(0)
    x32 = (rng.standard_normal(100000) * 3).astype(np.float32)
    t_bits = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nx.bf16_bits_of(nx.round_to_bf16(x32.astype(np.float64))), t_bits)
    assert np.array_equal(nx.bf16_to_f64(t_bits),
                          torch.from_numpy(t_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy())


def test_bf16_round_from_f64_brute_force():
    """Direct fp64 -> bf16 rounding: the nearest of the two bf16 neighbours, ties to even."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal(2000) * 10
    # add exact midpoints between bf16 neighbours (where rounding twice would go wrong)
    base = nx.round_to_bf16(x[:200])
    x = np.concatenate([x, base + np.ldexp(1.0, np.frexp(base)[1] - 9)])
    r = nx.round_to_bf16(x)
    for xi, ri in zip(x, r):
        b = np.float32(xi).view(np.uint32) >> 16
        cands = [(np.uint32(c) << 16).view(np.float32).astype(np.float64) for c in (b - 1, b, b + 1, b + 2)]
        d = [abs(c - xi) for c in cands]
        best = min(d)
        ok = [c for c, di in zip(cands, d) if di == best]
        if len(ok) == 1:
            assert ri == ok[0]
        else:
            evens = [c for c in ok if (np.float32(c).view(np.uint32) >> 16) % 2 == 0]
            assert ri == evens[0]


def test_fp8_block_dequant_round_trip_and_block_index():
    s = tiny_mla()
    W = gen.LayerWeights(s, 0, 0)
    for name in ("w_dkv", "w_uq", "wo"):
        m = W.matrix(name)
        out_dim, in_dim = W.mats[name]
        v = gen.scaled_normal(0, gen.tensor_id(name, 0, 0), np.arange(out_dim * in_dim, dtype=np.uint64),
                              s.w_std).reshape(out_dim, in_dim).astype(np.float64)
        deq = OL.weight_f64(m)
        # error <= half the E4M3 spacing at that magnitude times the block scale (RNE)
        sc = m["scales"][np.arange(out_dim)[:, None] // 128, np.arange(in_dim)[None, :] // 128]
        q = np.abs(v) / sc
        spacing = np.ldexp(1.0, np.maximum(np.frexp(q)[1] - 1, -6) - 3)
        assert np.all(np.abs(deq - v) <= 0.5 * spacing * sc * (1 + 1e-6))
    # block index arithmetic, edge blocks included: codes all 1.0, distinct scales
    out_dim, in_dim = 300, 260
    scales = (np.arange(3 * 3, dtype=np.float32) + 1).reshape(3, 3)
    codes = np.full((out_dim, in_dim), 0x38, dtype=np.uint8)
    d = nx.dequant_fp8_block(codes, scales)
    for n in (0, 127, 128, 255, 256, 299):
        for k in (0, 127, 128, 255, 256, 259):
            assert d[n, k] == scales[n // 128, k // 128]


# --------------------------------------------------------------------------- elementwise math
def test_rmsnorm_closed_form_and_torch():
    for c in (0.5, 3.0):
        h = np.full(64, c)
        g = np.linspace(0.5, 1.5, 64)
        assert np.allclose(nx.rmsnorm(h, g, 1e-6), g * c / math.sqrt(c * c + 1e-6), rtol=1e-15, atol=0)
    rng = np.random.default_rng(2)
    h = rng.standard_normal(4096)
    g = 1 + 0.02 * rng.standard_normal(4096)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h)[None], (4096,), torch.from_numpy(g), eps=1e-6)[0].numpy()
    assert np.allclose(nx.rmsnorm(h, g, 1e-6), ref, rtol=1e-13, atol=1e-15)
    y = nx.rmsnorm(h, np.ones(4096), 0.0)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-14


def test_rope_identity_norm_relative_and_direction():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 64))
    k = rng.standard_normal((3, 64))
    assert np.array_equal(nx.rope(q, 0, 10000.0), q)
    for p in (1, 7, 8191):
        assert np.allclose(np.linalg.norm(nx.rope(q, p, 1e4), axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    # <R_p q, R_s k> depends only on p - s
    d = [np.sum(nx.rope(q, p, 1e4) * nx.rope(k, p - 5, 1e4), axis=-1) for p in (5, 50, 3000)]
    assert np.allclose(d[0], d[1], rtol=1e-10) and np.allclose(d[0], d[2], rtol=1e-10)
    # direction and frequency by hand: pair i rotates by pos * base^(-2i/d), counter-clockwise
    x = np.zeros(4)
    x[0], x[2] = 1.0, 1.0
    r = nx.rope(x, 3, 10000.0)
    assert np.allclose(r, [math.cos(3), math.sin(3), math.cos(0.03), math.sin(0.03)], rtol=0, atol=1e-15)


def test_softmax_sums_and_scipy():
    from scipy.special import softmax as sp_softmax
    rng = np.random.default_rng(5)
    s = rng.standard_normal((10, 300)) * 20
    p = nx.softmax(s)
    assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-15)
    assert np.allclose(p, sp_softmax(s, axis=-1), rtol=1e-12, atol=0)


def test_silu_sigmoid_closed_forms():
    z = np.array([-30.0, -1.0, 0.0, 1.0, 30.0])
    assert np.allclose(nx.sigmoid(z), [1 / (1 + math.exp(30)), 1 / (1 + math.e), 0.5, 1 / (1 + 1 / math.e), 1 / (1 + math.exp(-30))], rtol=1e-15)
    assert np.allclose(nx.silu(z), z * nx.sigmoid(z), rtol=1e-15)
    assert nx.silu(np.array([0.0]))[0] == 0.0


# --------------------------------------------------------------------------- selection
def test_topk_equals_full_stable_sort_brute_force():
    rng = np.random.default_rng(6)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, n + 1))
        sc = rng.integers(-3, 4, size=n).astype(np.float64)     # many exact ties
        got = list(nx.topk_desc(sc, k))
        ref = sorted(range(n), key=lambda i: (-sc[i], i))[:k]
        assert got == ref
    assert list(nx.topk_desc(np.zeros(10), 4)) == [0, 1, 2, 3]


def test_softmax_renorm_gates_equal_renormalised_full_softmax():
    s = tiny_gqa()
    W = gen.LayerWeights(s, 0, 0)
    rng = np.random.default_rng(7)
    b = rng.standard_normal(s.hidden)
    rec = {}
    sel, gates = OL.route(s, W, b, rec)
    full = nx.softmax(rec["router_logits"])
    assert np.allclose(gates, full[sel] / full[sel].sum(), rtol=1e-13)
    assert abs(gates.sum() - 1) < 1e-15


def test_sigmoid_gates_and_zero_bias_reduces_to_logit_topk():
    s = tiny_mla()
    rng = np.random.default_rng(8)
    b = rng.standard_normal(s.hidden)
    rec = {}
    sel, gates = OL.route(s, gen.LayerWeights(s, 0, 0), b, rec)
    assert abs(gates.sum() - 1) < 1e-15
    sc = 1 / (1 + np.exp(-rec["router_logits"]))
    assert np.allclose(gates, sc[sel] / sc[sel].sum(), rtol=1e-14)
    W0 = DictWeights(s, bias=np.zeros(s.n_experts))
    rec0 = {}
    sel0, _ = OL.route(s, W0, b, rec0)
    assert list(sel0) == sorted(range(s.n_experts), key=lambda i: (-rec0["router_logits"][i], i))[: s.top_k]


def test_biased_router_selection_and_gates_by_hand():
    """Biased-score routing with a nonzero bias, worked by hand. Logits r (via b = e_0 and a
    router whose first column holds r) and biases over four live experts (the other four
    have r = -6, bias -1 and never compete):

        expert        0       1       2       3
        r           6.0     0.0     0.5    -0.5
        bias       -0.6     0.0     0.3     0.2
        sigmoid(r) .9975   .5000   .6225   .3775
        sig + bias .3975   .5000   .9225   .5775   -> top-2 = [2, 3]
        r + bias    5.4     0.0     0.8    -0.3    -> top-2 = {0, 2}  (a misreading)
        sigmoid(r) alone                           -> top-2 = {0, 2}  (bias ignored)

    The gates are the unbiased sigmoid scores renormalised over the selection:
    sigmoid(0.5) / (sigmoid(0.5) + sigmoid(-0.5)) = sigmoid(0.5), since sigmoid(x) +
    sigmoid(-x) = 1; so gates = [sigmoid(0.5), sigmoid(-0.5)] = [0.62245933, 0.37754067].
    The selection also equals a brute-force full sort of sigmoid(r) + bias."""
    s = tiny_mla(n_experts=8, top_k=2)
    r = np.array([6.0, 0.0, 0.5, -0.5, -6.0, -6.0, -6.0, -6.0])
    bias = np.array([-0.6, 0.0, 0.3, 0.2, -1.0, -1.0, -1.0, -1.0], np.float32)
    wr = np.zeros((s.n_experts, s.hidden), np.float32)
    wr[:, 0] = r                                   # bf16-exact values
    W = DictWeights(s, overrides={("router", None): wr}, bias=bias)
    b = np.zeros(s.hidden)
    b[0] = 1.0
    rec = {}
    sel, gates = OL.route(s, W, b, rec)
    assert np.array_equal(rec["router_logits"], r)
    assert list(sel) == [2, 3]
    assert np.allclose(gates, [0.6224593312018546, 0.3775406687981454], rtol=0, atol=1e-15)
    # the misreadings pick another set
    assert set(np.argsort(-(r + bias))[:2]) == {0, 2}
    assert set(np.argsort(-(1 / (1 + np.exp(-r))))[:2]) == {0, 2}
    # brute force: a full sort of every expert's biased score, ties to the lower index
    key = 1 / (1 + np.exp(-r)) + bias.astype(np.float64)
    order = sorted(range(s.n_experts), key=lambda i: (-key[i], i))
    assert list(sel) == order[:2]


# --------------------------------------------------------------------------- attention
def _tiny_case(s, seed=0):
    W = gen.LayerWeights(s, seed, 0)
    cache = gen.padded_cache(s, seed)
    x = gen.input_hidden(s, seed)
    return W, cache, x


def _pad_cache(s, cache):
    out = {}
    for k, v in cache.items():
        shape = list(v.shape)
        ax = 1 if k in ("k", "v") else 0
        shape[ax] = s.max_seq
        z = np.zeros(shape, dtype=v.dtype)
        if ax == 1:
            z[:, : v.shape[1]] = v
        else:
            z[: v.shape[0]] = v
        out[k] = z
    return out


def test_attention_length_one_and_two_by_hand():
    s = tiny_gqa()
    W, cache, x = _tiny_case(s)
    rec = OL.decode_layer(s, W, cache, x, 0)          # only the new row: o = v_new
    for h in range(s.n_heads):
        g = h * s.n_kv_heads // s.n_heads
        assert np.array_equal(rec["o"][h], rec["v_new"][g])
    rec = OL.decode_layer(s, W, cache, x, 1)          # one cached row + the new row
    for h in range(s.n_heads):
        g = h * s.n_kv_heads // s.n_heads
        k0 = nx.bf16_to_f64(cache["k"][g, 0])
        v0 = nx.bf16_to_f64(cache["v"][g, 0])
        s0 = float(rec["q"][h] @ k0) / math.sqrt(s.head_dim)
        s1 = float(rec["q"][h] @ rec["k_new"][g]) / math.sqrt(s.head_dim)
        w0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        assert np.allclose(rec["o"][h], w0 * v0 + (1 - w0) * rec["v_new"][g], rtol=1e-12, atol=1e-14)


def test_gqa_grouping_equals_mha_with_duplicated_kv_heads():
    s_g = tiny_gqa()                                   # 4 q heads, 2 kv heads
    s_m = tiny_gqa(n_kv_heads=4)                       # MHA
    base = gen.LayerWeights(s_g, 0, 0)
    wk = OL.weight_f64(base.matrix("wk")).reshape(2, s_g.head_dim, s_g.hidden)
    wv = OL.weight_f64(base.matrix("wv")).reshape(2, s_g.head_dim, s_g.hidden)
    dup = [0, 0, 1, 1]                                 # contiguous groups
    Wm = DictWeights(s_m, base=base, overrides={("wk", 0): wk[dup].reshape(-1, s_g.hidden),
                                                ("wv", 0): wv[dup].reshape(-1, s_g.hidden)})
    cache = _pad_cache(s_g, gen.full_cache(s_g))
    cache_m = {"k": cache["k"][dup], "v": cache["v"][dup]}
    x = gen.input_hidden(s_g)
    rg = OL.decode_layer(s_g, base, cache, x, s_g.cache_len)
    rm = OL.decode_layer(s_m, Wm, cache_m, x, s_m.cache_len)
    assert np.array_equal(rg["o"], rm["o"])
    assert np.array_equal(rg["out_bits"], rm["out_bits"])


def test_mla_absorbed_equals_non_absorbed():
    s = tiny_mla()
    W, cache, x = _tiny_case(s)
    pos = s.cache_len
    rec = OL.decode_layer(s, W, cache, x, pos)
    L = s.kv_lora
    C = np.concatenate([nx.bf16_to_f64(cache["latent"][:pos]), rec["latent_new"][None]], 0)
    W_uk = OL.weight_f64(W.matrix("w_uk")).reshape(s.n_heads, s.nope_dim, L)
    W_uv = OL.weight_f64(W.matrix("w_uv")).reshape(s.n_heads, s.v_dim, L)
    for h in range(s.n_heads):
        q_lat = W_uk[h].T @ rec["q_nope"][h]                       # absorbed query in latent space
        sc = (C[:, :L] @ q_lat + C[:, L:] @ rec["q_rope"][h]) / math.sqrt(s.nope_dim + s.rope_dim)
        p = np.exp(sc - sc.max())
        p /= p.sum()
        o_lat = p @ C[:, :L]
        assert np.allclose(W_uv[h] @ o_lat, rec["o"][h], rtol=1e-11, atol=1e-13)


def test_sparse_with_short_cache_equals_dense_mla():
    sd = tiny_mla(wfmt="bf16", router="softmax", cache_len=20, max_seq=40)
    ss = tiny_mla(wfmt="bf16", router="softmax", cache_len=20, max_seq=40,
                  index_heads=2, index_dim=16, index_topk=64)
    W = gen.LayerWeights(ss, 0, 0)
    cache = _pad_cache(ss, gen.full_cache(ss))
    x = gen.input_hidden(ss)
    rs = OL.decode_layer(ss, W, cache, x, 20)
    rd = OL.decode_layer(sd, W, cache, x, 20)
    assert list(rs["index_sel"]) == list(range(21))
    assert np.array_equal(rs["out_bits"], rd["out_bits"])


def test_indexer_score_exact_bound_and_invariants():
    ss = tiny_mla(wfmt="bf16", router="softmax", cache_len=300, max_seq=320,
                  index_heads=4, index_dim=16, index_topk=37)
    W = gen.LayerWeights(ss, 0, 0)
    cache = _pad_cache(ss, gen.full_cache(ss))
    x = gen.input_hidden(ss)
    rec = OL.decode_layer(ss, W, cache, x, 300)
    codes = np.concatenate([cache["index_codes"][:300], rec["index_code_new"][None]])
    scales = np.concatenate([cache["index_scales"][:300], [rec["index_scale_new"]]]).astype(np.float64)
    dec = nx.E4M3[codes]
    # exact evaluation with fsum: the fixed-order fp64 score is within its rounding bound
    for t in range(0, 301, 17):
        terms = []
        tot_abs = 0.0
        for h in range(ss.index_heads):
            dot = math.fsum(float(rec["q_i"][h, i]) * float(dec[t, i]) for i in range(ss.index_dim))
            r = max(0.0, float(scales[t]) * dot)
            terms.append(float(rec["w_idx"][h]) * r)
            tot_abs += abs(float(rec["w_idx"][h])) * abs(float(scales[t])) * sum(
                abs(float(rec["q_i"][h, i]) * float(dec[t, i])) for i in range(ss.index_dim))
        exact = math.fsum(terms)
        assert abs(rec["index_score"][t] - exact) <= 80 * 2.0 ** -53 * tot_abs + 1e-300
    # selection = brute-force top-k by (score desc, index asc), sorted ascending
    sc = rec["index_score"]
    ref = sorted(sorted(range(301), key=lambda t: (-sc[t], t))[:37])
    assert list(rec["index_sel"]) == ref
    # the new key is a candidate and its code is the FP8 quantisation of k_I
    assert len(sc) == 301
    k32 = rec["k_i"].astype(np.float32)
    sig = np.float32(np.max(np.abs(k32)) / np.float32(448))
    t_codes = torch.from_numpy(np.clip(k32 / sig, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(rec["index_code_new"], t_codes)


def test_indexer_all_zero_query_selects_lowest_indices():
    ss = tiny_mla(wfmt="bf16", router="softmax", cache_len=100, max_seq=128,
                  index_heads=2, index_dim=16, index_topk=10)
    base = gen.LayerWeights(ss, 0, 0)
    W = DictWeights(ss, base=base, overrides={("w_qi", 0): np.zeros((32, ss.q_lora))})
    cache = _pad_cache(ss, gen.full_cache(ss))
    rec = OL.decode_layer(ss, W, cache, gen.input_hidden(ss), 100)
    assert np.all(rec["index_score"] == 0)
    assert list(rec["index_sel"]) == list(range(10))


# --------------------------------------------------------------------------- whole-layer special cases
def test_layer_with_zero_output_and_expert_weights_is_identity():
    s = tiny_gqa()
    base = gen.LayerWeights(s, 0, 0)
    ov = {("wo", 0): np.zeros((s.hidden, s.o_dim))}
    for e in range(s.n_expert_slots):
        ov[("w_down", e)] = np.zeros((s.hidden, s.inter))
    W = DictWeights(s, base=base, overrides=ov)
    cache = _pad_cache(s, gen.full_cache(s))
    x = gen.input_hidden(s)
    rec = OL.decode_layer(s, W, cache, x, s.cache_len)
    assert np.array_equal(rec["out_bits"], x)


def test_zero_query_gives_uniform_attention():
    s = tiny_gqa()
    base = gen.LayerWeights(s, 0, 0)
    W = DictWeights(s, base=base, overrides={("wq", 0): np.zeros((s.q_dim, s.hidden))})
    cache = _pad_cache(s, gen.full_cache(s))
    rec = OL.decode_layer(s, W, cache, gen.input_hidden(s), s.cache_len)
    for h in range(s.n_heads):
        g = h * s.n_kv_heads // s.n_heads
        V = np.concatenate([nx.bf16_to_f64(cache["v"][g, : s.cache_len]), rec["v_new"][g][None]])
        assert np.allclose(rec["o"][h], V.mean(0), rtol=1e-13, atol=1e-15)


def test_moe_zero_routed_experts_leaves_shared_only_and_linearity_of_gates():
    s = tiny_gqa()
    base = gen.LayerWeights(s, 0, 0)
    ov = {("w_down", e): np.zeros((s.hidden, s.inter)) for e in range(s.n_experts)}
    W = DictWeights(s, base=base, overrides=ov)
    b = np.random.default_rng(9).standard_normal(s.hidden)
    rec = {}
    f = OL.ffn(s, W, b, rec)
    shared = OL.expert(W, s.n_experts, b)
    assert np.array_equal(f, shared)
    # with real weights: f - shared = sum_i gate_i E_i(b)
    rec = {}
    f = OL.ffn(s, base, b, rec)
    manual = sum(g * OL.expert(base, int(e), b) for e, g in zip(rec["router_sel"], rec["gates"]))
    assert np.allclose(f - OL.expert(base, s.n_experts, b), manual, rtol=1e-12, atol=1e-14)


def test_expert_is_swiglu_of_three_products():
    s = tiny_gqa()
    rng = np.random.default_rng(10)
    Wg, Wu, Wd = (rng.standard_normal(sh) * 0.1 for sh in ((s.inter, s.hidden), (s.inter, s.hidden), (s.hidden, s.inter)))
    W = DictWeights(s, overrides={("w_gate", 0): Wg, ("w_up", 0): Wu, ("w_down", 0): Wd})
    b = rng.standard_normal(s.hidden)
    g = nx.bf16_to_f64(gen.f32_to_bf16_bits(Wg.astype(np.float32))).reshape(Wg.shape) @ b
    u = nx.bf16_to_f64(gen.f32_to_bf16_bits(Wu.astype(np.float32))).reshape(Wu.shape) @ b
    d = nx.bf16_to_f64(gen.f32_to_bf16_bits(Wd.astype(np.float32))).reshape(Wd.shape)
    ref = d @ ((g / (1 + np.exp(-g))) * u)
    assert np.allclose(OL.expert(W, 0, b), ref, rtol=1e-13)


# --------------------------------------------------------------------------- accounting and page examples
def test_page_worked_examples():
    g = json.load(open(GOLDEN))
    e = g["hbm_roofline_b200"]
    v = accounting.tokens_per_s_user(e["bandwidth_bytes_per_s"], e["bytes_per_token"])
    assert math.floor(v) == e["printed_tokens_per_s_user"]
    e = g["hbm_roofline_h200"]
    v = accounting.tokens_per_s_user(e["bandwidth_bytes_per_s"], e["bytes_per_token"])
    assert 900 < v < e["printed_tokens_per_s_user"] and round(v, 1) == 914.3
    e4, e3 = g["weight_bytes_mxfp4"], g["weight_bytes_lut"]
    a = accounting.weight_bytes(e4["n_params"], e4["bits_per_weight"]) / 1e9
    b = accounting.weight_bytes(e3["n_params"], e3["bits_per_weight"]) / 1e9
    assert a == e4["printed_gb"]
    assert round(b) == e3["printed_gb"]
    assert round(a - round(b), 1) == e3["printed_difference_gb"]
    for d, m in g["swiglu_flops"]["cases"]:
        assert accounting.swiglu_flops(d, m) == 6 * d * m
    lc = g["launch_collapse"]
    assert lc["standard_launches"] - lc["specialized_launches"] == 10


@pytest.mark.parametrize("shape_fn", [tiny_gqa, tiny_mla, tiny_kda,
                                      lambda: tiny_mla(wfmt="bf16", router="softmax", index_heads=2,
                                                       index_dim=16, index_topk=4)])
def test_oracle_byte_count_equals_closed_form(shape_fn):
    s = shape_fn()
    W, cache, x = _tiny_case(s)
    rec = OL.decode_layer(s, W, cache, x, s.cache_len)
    closed_w = sum(accounting.layer_weight_bytes(s).values())
    assert rec["weight_bytes"] == closed_w
    kv = accounting.layer_kv_bytes(s, s.cache_len)
    got_read = rec["kv_bytes_read"] + rec.get("index_bytes_read", 0)
    assert got_read == kv["kv_read"]
    assert rec["kv_bytes_written"] == kv["kv_write"]


def test_closed_form_bytes_of_the_workloads():
    """Active parameters x bytes per weight (+ scales, norms, KV) for the named workloads."""
    c2 = configs.C2
    w = accounting.layer_weight_bytes(c2)
    H = 4096
    assert w["attn"] == 2 * (4096 * H + 2 * 1024 * H + H * 4096)
    assert w["experts"] == 9 * 2 * 3 * 1536 * H
    assert accounting.layer_kv_bytes(c2, 8192)["kv_read"] == 8193 * 8 * 128 * 2 * 2
    c3 = configs.C3
    w3 = accounting.layer_weight_bytes(c3)
    assert w3["experts"] == 9 * (3 * 2048 * 6144 + 4 * 3 * 16 * 48)


# --------------------------------------------------------------------------- model level
def test_argmax_lowest_index_on_ties():
    assert OM.argmax_lowest(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert OM.argmax_lowest(np.zeros(5)) == 0


def test_verify_with_greedy_drafts_accepts_all_and_matches_decode():
    s = tiny_mla(wfmt="bf16", router="softmax", cache_len=5, max_seq=32)
    model = configs.ModelShape(layer=s, n_layers=2, vocab=64, head_fmt="bf16")
    srcs = [gen.LayerWeights(s, 0, l) for l in range(2)]
    head = gen.head_matrix(model)
    fg = gen.final_norm(model)
    emb = lambda t: gen.embedding_rows(model, [t])[0]
    caches = [_pad_cache(s, gen.full_cache(s, 0, l)) for l in range(2)]
    toks, _ = OM.decode_tokens(s, srcs, [{k: v.copy() for k, v in c.items()} for c in caches], emb, head, fg,
                               token0=3, start_pos=5, n_tokens=4)
    res = OM.verify_step(s, srcs, [{k: v.copy() for k, v in c.items()} for c in caches], emb, head, fg,
                         token0=3, drafts=toks[:3], pos=5)
    assert res["accepted"] == 3 and res["tokens"] == toks
    bad = list(toks[:3])
    bad[1] = (bad[1] + 1) % 64
    res = OM.verify_step(s, srcs, [{k: v.copy() for k, v in c.items()} for c in caches], emb, head, fg,
                         token0=3, drafts=bad, pos=5)
    assert res["accepted"] == 1 and res["tokens"][:2] == toks[:2]


# --------------------------------------------------------------------------- generator
def test_generator_moments_and_determinism():
    v = gen.normal_f32(0, gen.tensor_id("wq"), np.arange(400000, dtype=np.uint64))
    assert abs(v.mean()) < 0.01 and abs(v.var() - 1) < 0.01
    assert np.array_equal(v[:1000], gen.normal_f32(0, gen.tensor_id("wq"), np.arange(1000, dtype=np.uint64)))
    assert not np.array_equal(v[:1000], gen.normal_f32(1, gen.tensor_id("wq"), np.arange(1000, dtype=np.uint64)))
    q = _e4m3_sweep()
    assert np.array_equal(gen.f32_to_e4m3_codes(q), gen._f32_to_e4m3_codes_table(q))


def test_layer_residuals_closed_form():
    """W_q = 0 (uniform attention), W_O = I, no FFN output: out = bf16(x + concat_h mean(V_g(h)))."""
    s = tiny_gqa()
    assert s.o_dim == s.hidden
    base = gen.LayerWeights(s, 0, 0)
    ov = {("wq", 0): np.zeros((s.q_dim, s.hidden)), ("wo", 0): np.eye(s.hidden)}
    for e in range(s.n_expert_slots):
        ov[("w_down", e)] = np.zeros((s.hidden, s.inter))
    W = DictWeights(s, base=base, overrides=ov)
    cache = _pad_cache(s, gen.full_cache(s))
    x = gen.input_hidden(s)
    rec = OL.decode_layer(s, W, cache, x, s.cache_len)
    means = []
    for h in range(s.n_heads):
        g = h * s.n_kv_heads // s.n_heads
        V = np.concatenate([nx.bf16_to_f64(cache["v"][g, : s.cache_len]), rec["v_new"][g][None]])
        means.append(V.mean(0))
    ref = nx.bf16_to_f64(x) + np.concatenate(means)
    assert np.allclose(rec["out_f64"], ref, rtol=1e-13, atol=1e-13)
    # with the attention output switched off, the FFN residual is x + ffn(RMSNorm(x))
    W2 = DictWeights(s, base=base, overrides={("wo", 0): np.zeros((s.hidden, s.o_dim))})
    rec2 = OL.decode_layer(s, W2, cache, x, s.cache_len)
    h = nx.bf16_to_f64(x)
    f = OL.ffn(s, base, nx.rmsnorm(h, base.norm("ffn_norm"), s.eps), {})
    assert np.allclose(rec2["out_f64"], h + f, rtol=1e-13, atol=1e-13)


def test_expected_union_of_routed_experts_by_enumeration():
    """E * (1 - (1 - k/E)^n) equals the mean number of distinct experts over every
    combination of n independent top-k choices (uniform routing), enumerated exactly."""
    import itertools
    from oracle import accounting
    for E, k, n in [(4, 2, 2), (5, 2, 3), (6, 3, 2)]:
        subsets = list(itertools.combinations(range(E), k))
        tot = 0
        for combo in itertools.product(subsets, repeat=n):
            tot += len(set().union(*combo))
        mean = tot / len(subsets) ** n
        assert abs(mean - accounting.expected_union_experts(E, k, n)) < 1e-12, (E, k, n)


# --------------------------------------------------------------------------- sampling
def test_splitmix_reference_outputs_and_second_implementation():
    """The sampler's mixer against the published SplitMix64 outputs from state 0 (Vigna's
    splitmix64.c: the state advances by G, the output is the mix of the state) and against the
    input generator's independent implementation of the same mixer."""
    G = 0x9E3779B97F4A7C15
    ref = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    for k, want in enumerate(ref, start=1):
        assert int(OM.splitmix_mix(np.uint64((k * G) & ((1 << 64) - 1)))) == want
    z = np.random.default_rng(3).integers(0, 2**63, 1000, dtype=np.int64).astype(np.uint64) * np.uint64(2)
    assert np.array_equal(OM.splitmix_mix(z), gen._mix(z))


def test_sampling_uniforms_range_and_moments():
    u = np.concatenate([OM.sample_uniforms(7, p, 4096) for p in range(8)])
    assert np.all(u > 0) and np.all(u < 1)
    assert abs(u.mean() - 0.5) < 4 * math.sqrt(1 / 12 / u.size)
    assert abs(u.var() - 1 / 12) < 0.01
    # distinct positions and seeds give different streams
    assert not np.array_equal(OM.sample_uniforms(7, 0, 64), OM.sample_uniforms(7, 1, 64))
    assert not np.array_equal(OM.sample_uniforms(7, 0, 64), OM.sample_uniforms(8, 0, 64))


def test_gumbel_max_sampling_follows_softmax():
    """Over many positions the sampled tokens follow softmax(logits / T) (chi-square), T = 0
    is the argmax, a constant added to every logit changes nothing, and a logit gap far above
    the Gumbel spread always wins."""
    from scipy.stats import chisquare
    lg = np.array([1.0, 0.0, -1.0, 2.0, 0.5])
    T = 0.7
    p = np.exp(lg / T) / np.exp(lg / T).sum()
    n = 20000
    toks = np.array([OM.sample_token(lg, T, 11, pos) for pos in range(n)])
    counts = np.bincount(toks, minlength=lg.size)
    assert chisquare(counts, p * n).pvalue > 1e-4
    assert OM.sample_token(lg, 0.0, 11, 5) == 3
    for pos in range(50):
        assert OM.sample_token(lg + 123.25, T, 11, pos) == OM.sample_token(lg, T, 11, pos)
    big = np.zeros(1000)
    big[417] = 200.0
    assert all(OM.sample_token(big, 1.0, 5, pos) == 417 for pos in range(50))


# --------------------------------------------------------------------------- KDA
def _kda_chunk_form(S, Q, K, V, beta, G):
    """The chunked matrix form printed in the Kimi K3 article ("FlashKDA Algorithm"), written
    out independently of the per-token recurrence: a = exp2(cumsum(g)), K_decay = Diag(a) K,
    Q_decay = Diag(a) Q, K_inv = Diag(a)^-1 K, K_restore = a[-1] K_inv, L = StrictTril(Diag(beta)
    K_decay K_inv^T), U = (I + L)^-1 Diag(beta) (V - K_decay S), O = Q_decay S + tril(Q_decay
    K_inv^T) U, S_out = Diag(a[-1]) S + K_restore^T U."""
    C = Q.shape[0]
    a = np.exp2(np.cumsum(G, axis=0))
    K_decay, Q_decay, K_inv = a * K, a * Q, K / a
    K_restore = a[-1] * K_inv
    L = np.tril(beta[:, None] * (K_decay @ K_inv.T), -1)
    U = np.linalg.solve(np.eye(C) + L, beta[:, None] * (V - K_decay @ S))
    O = Q_decay @ S + np.tril(Q_decay @ K_inv.T) @ U
    return O, a[-1][:, None] * S + K_restore.T @ U


def test_kda_recurrence_equals_the_pages_chunked_form():
    """Eight tokens through the oracle's per-token state step equal two chunks of four through
    the chunked form (outputs of every token and the final state, to rounding)."""
    rng = np.random.default_rng(21)
    Dk, Dv, T, C = 8, 6, 8, 4
    S0 = rng.standard_normal((Dk, Dv))
    Q, K, V = rng.standard_normal((T, Dk)), rng.standard_normal((T, Dk)), rng.standard_normal((T, Dv))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    G = -np.log1p(np.exp(rng.standard_normal((T, Dk))))        # log2 decays <= 0
    S, outs = S0.copy(), []
    for t in range(T):
        S, o = OL.kda_state_step(S, Q[t], K[t], V[t], beta[t], np.exp2(G[t]))
        outs.append(o)
    Sc, oc = S0.copy(), []
    for c0 in range(0, T, C):
        O, Sc = _kda_chunk_form(Sc, Q[c0:c0 + C], K[c0:c0 + C], V[c0:c0 + C], beta[c0:c0 + C], G[c0:c0 + C])
        oc.append(O)
    assert np.allclose(np.stack(outs), np.concatenate(oc), rtol=0, atol=1e-12)
    assert np.allclose(S, Sc, rtol=0, atol=1e-12)


def test_kda_delta_rule_stores_the_value_at_its_key():
    """With no decay and beta = 1, the delta rule overwrites what the state returns for a unit
    key: after the step S^T k = v exactly (to rounding), whatever S held before."""
    rng = np.random.default_rng(5)
    S = rng.standard_normal((16, 12))
    k = rng.standard_normal(16)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(12)
    S1, o = OL.kda_state_step(S, k, k, v, 1.0, np.ones(16))
    assert np.allclose(S1.T @ k, v, atol=1e-13)
    assert np.allclose(o, v, atol=1e-13)          # querying with the key itself
    # beta = 0 only decays: S1 = diag(alpha) S
    al = rng.uniform(0.2, 1.0, 16)
    S2, _ = OL.kda_state_step(S, k, k, v, 0.0, al)
    assert np.array_equal(S2, al[:, None] * S)


def test_kda_state_cost_matches_the_pages_decode_figures():
    """Per head and token: about 7 D^2 FLOPs and 8 D^2 bytes (fp32 state read and written)."""
    for d in (64, 128, 256):
        assert accounting.kda_state_flops_per_head(d) == 7 * d * d
        assert accounting.kda_state_bytes_per_head(d) == 8 * d * d


def test_kda_convolution_taps_by_hand():
    """The causal depthwise convolution: taps [0, 0, 0, 1] pass the current projection through,
    taps [1, 0, 0, 0] return the ring entry of position pos - 3, and the ring slot of pos is
    overwritten by the current projection (fp32)."""
    s = tiny_kda()
    nq = 3 * s.q_dim
    base = gen.LayerWeights(s, 0, 0)
    cache = gen.padded_cache(s)
    x = gen.input_hidden(s)
    pos = 10
    a = nx.rmsnorm(nx.bf16_to_f64(x), base.norm("attn_norm"), s.eps)
    for taps, want in (([0, 0, 0, 1], None), ([1, 0, 0, 0], cache["conv_ring"][(pos - 3) % 3].astype(np.float64))):
        W = DictWeights(s, base=base, conv=np.tile(np.asarray(taps, np.float32), (nq, 1)))
        c = {k: v.copy() for k, v in cache.items()}
        rec = {}
        OL.kda_attention(s, W, c, a, pos, rec)
        proj = rec["kda_x32"]
        got = np.concatenate([rec["kda_v"].reshape(-1)])          # v is not normalised: the conv output itself
        ref = (proj if want is None else want)[2 * s.q_dim:]
        assert np.array_equal(got, ref)
    # the ring slot of pos now holds the fp32 projection after append
    c = {k: v.copy() for k, v in cache.items()}
    rec = OL.decode_layer(s, base, c, x, pos)
    OL.append_to_cache(s, c, rec, pos)
    assert np.array_equal(c["conv_ring"][pos % 3], rec["kda_x32"].astype(np.float32))
    assert np.array_equal(c["conv_ring"][(pos + 1) % 3], cache["conv_ring"][(pos + 1) % 3])


# --------------------------------------------------------------------------- LUT3 weights
def test_lut3_footprint_is_the_pages_3125_bits_per_weight():
    """3 bits of index per weight plus one 8-byte codebook per 8 x 64 block: 3.125 bits per
    weight, the stored footprint the page computes (2.8e12 x 3.125 / 8 = 1,093.75 GB)."""
    for out_dim, in_dim in ((8, 128), (2048, 6144), (6144, 2048)):
        b = accounting._mat_bytes(out_dim, in_dim, "lut3")
        assert b * 8 == 3.125 * out_dim * in_dim
    assert accounting.weight_bytes(2.8e12, 3.125) == 1093.75e9


def test_lut3_decode_by_hand_from_bytes():
    """The oracle's decode against a byte-level reading of the planes written out here
    (bit j % 8 of byte 16 p + 4 d + j // 8 of the group), and every weight is one of the
    8 E4M3 values of its block's codebook."""
    out_dim, in_dim = 16, 256
    idx, cb = gen.lut3_matrix(0, 77, out_dim, in_dim, 0.02)
    W = nx.dequant_lut3(idx, cb)
    for n in range(out_dim):
        for k in range(in_dim):
            g, w = divmod(k, 128)
            d, j = divmod(w, 32)
            i = 0
            for p in range(3):
                byte = idx[n, 48 * g + 16 * p + 4 * d + j // 8]
                i |= ((int(byte) >> (j % 8)) & 1) << p
            assert W[n, k] == nx.E4M3[cb[n // 8, k // 64, i]]
    # the drawn indices are the low 3 bits of the generator's draws
    raw = gen.raw_u64(0, 77, np.arange(out_dim * in_dim, dtype=np.uint64)) & np.uint64(7)
    for n, k in ((0, 0), (3, 200), (15, 255)):
        assert W[n, k] == nx.E4M3[cb[n // 8, k // 64, int(raw[n * in_dim + k])]]


def test_layer_with_lut3_experts_equals_explicit_dequantised_weights():
    """A layer whose experts are LUT3 equals the same layer given those experts as explicit
    (bf16-exact E4M3) matrices: the lookup is the only difference in the definition."""
    s = tiny_mla(wfmt="fp8", expert_fmt="lut3", hidden=128, inter=128)
    base = gen.LayerWeights(s, 0, 0)
    cache = gen.padded_cache(s)
    x = gen.input_hidden(s)
    ov = {}
    for e in range(s.n_experts + s.n_shared):
        for name in ("w_gate", "w_up", "w_down"):
            ov[(name, e)] = nx.dequant_lut3(base.matrix(name, e)["idx"], base.matrix(name, e)["codebook"])
    ref = OL.decode_layer(s, DictWeights(s, base=base, overrides=ov), {k: v.copy() for k, v in cache.items()}, x,
                          s.cache_len)
    got = OL.decode_layer(s, base, {k: v.copy() for k, v in cache.items()}, x, s.cache_len)
    assert np.array_equal(got["out_f64"], ref["out_f64"])
