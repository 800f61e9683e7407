"""GPU parity of the FP8 MLA MoE decode layer against the CPU oracle.

Workload: hidden 6144, 64 heads, q_lora 1536, kv_lora 512 + rope 64 (nope 128, v 128),
FP8 E4M3 weights with fp32 128x128 block scales, 256 routed experts top-8 with the
biased-score (sigmoid + bias) router, one shared expert, expert width 2048, latent cache.
The GPU runs attention in absorbed form on the matrix cores (q and P rounded to bf16); the
oracle computes it non-absorbed in fp64, so the two meet only through the mathematics.

Bars: hidden state within TOL (max-norm relative); router top-k identical; the appended
latent row within one bf16 rounding step of the oracle's.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_common import TOL, bf16_tensor_to_f64, check_branches, host_cache, oracle_step, rel_err, say  # noqa: E402
from oracle import numerics as nx  # noqa: E402
from synth import configs, gen  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decoder(s, seeds_layers):
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    Ws = [sdev.layer_weights(s, seed, layer) for seed, layer in seeds_layers]
    Cs = [sdev.kv_cache(s, seed, layer) for seed, layer in seeds_layers]
    return pld.Decoder(s, Ws, Cs), Ws, Cs


def _run_step(dec, s, layer, x, pos):
    out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    dec.step(layer, x, pos, out)
    torch.cuda.synchronize()
    st = dec.status()
    assert st.code == 0, f"device status {st.code} wait {st.stage} layer {st.layer} wg {st.wg}"
    return out


def _check_layer(dec, s, rec, out, pos, cache_dev, tag, x_bits):
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    say(f"{tag}: out rel err {err:.3e}")
    assert err < TOL, f"{tag}: out rel err {err}"
    assert rel_err(dec.debug("a").cpu().numpy(), rec["a"]) < 1e-5, tag
    qn = dec.debug("q").cpu().numpy().reshape(s.n_heads, s.nope_dim)
    e_qn = rel_err(qn, rec["q_nope"])
    # q_rope travels as bf16 (the attention's matrix cores take it in bf16): the GPU's bf16
    # value is within one bf16 step of the oracle's value, plus the fp32 error of the value
    # before its rounding (1e-4 of the vector's largest entry)
    qr = nx.bf16_to_f64(dec.debug("qrope").cpu().numpy().view(np.uint16)[:s.n_heads * s.rope_dim])
    qr = qr.reshape(s.n_heads, s.rope_dim)
    ref_qr = rec["q_rope"]
    tol_qr = np.abs(ref_qr) * 2.0 ** -8 + 1e-4 * np.abs(ref_qr).max()
    assert np.all(np.abs(qr - ref_qr) <= tol_qr), f"{tag}: q_rope beyond one bf16 step"
    e_qr = rel_err(qr, ref_qr)
    o = dec.debug("o").cpu().numpy().reshape(s.n_heads, s.v_dim)
    e_o = rel_err(o, rec["o"])
    h2 = dec.debug("h2").cpu().numpy()
    e_h2 = rel_err(h2, rec["h2"])
    say(f"{tag}: q_nope {e_qn:.2e} q_rope {e_qr:.2e} o {e_o:.2e} h2 {e_h2:.2e}")
    assert e_qn < 1e-4 and e_qr < 2.0 ** -8, tag
    assert e_o < 1e-2, f"{tag}: attention output rel err {e_o}"
    assert e_h2 < 1e-2, tag
    assert rel_err(dec.debug("b").cpu().numpy(), rec["b"]) < 1e-2, tag
    # the appended latent row: the oracle's bf16 row up to one rounding step
    got = nx.bf16_to_f64(cache_dev["latent"][pos].cpu().numpy().view(np.uint16))
    ref = rec["latent_new"]
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30), f"{tag}: latent row"
    sel = dec.debug("sel").cpu().numpy()
    assert list(sel) == list(rec["router_sel"]), f"{tag}: router selection {sel} vs {rec['router_sel']}"
    gates = dec.debug("gates").cpu().numpy()
    assert np.allclose(gates, rec["gates"], rtol=1e-3, atol=1e-5), tag
    check_branches(dec, s, rec, x_bits, tag)


@pytest.mark.parametrize("cache_len,positions", [(300, [300, 301]), (37, [0, 37])])
def test_mla_fp8_layer_parity_small_cache(cache_len, positions):
    _need_gpu()
    s = configs.scaled(configs.C3, cache_len=cache_len, max_seq=cache_len + 64)
    say(f"case: MLA FP8 layer, cache {cache_len}, positions {positions}")
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    hc = host_cache(s)
    W = gen.LayerWeights(s, 0, 0)
    from synth import device as sdev
    for i, pos in enumerate(positions):
        x = sdev.input_hidden(s, 0, i)
        out = _run_step(dec, s, 0, x, pos)
        xb = gen.input_hidden(s, 0, i)
        rec = oracle_step(s, 0, 0, hc, xb, pos, weights=W)
        _check_layer(dec, s, rec, out, pos, Cs[0], f"mla cache {cache_len} pos {pos}", xb)


def test_mla_fp8_layer_parity_full_cache_chain():
    """The 8192-token cache, chained launches at positions 8192 and 8193. From 8193 on the
    history rows no longer split into whole 32-row sub-blocks of 64 chunks: one chunk holds
    129 rows (a fifth, one-row sub-block), and row 8192 was written by the previous launch."""
    _need_gpu()
    s = configs.C3
    say("case: MLA FP8 layer, 8192-token cache, chained positions 8192, 8193")
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    from synth import device as sdev
    hc = host_cache(s)
    W = gen.LayerWeights(s, 0, 0)
    for i, pos in enumerate((8192, 8193)):
        x = sdev.input_hidden(s, 0, i)
        out = _run_step(dec, s, 0, x, pos)
        xb = gen.input_hidden(s, 0, i)
        rec = oracle_step(s, 0, 0, hc, xb, pos, weights=W)
        _check_layer(dec, s, rec, out, pos, Cs[0], f"mla pos {pos}", xb)


def test_mla_fp8_layer_parity_ragged_chunks():
    """An 8200-token cache at position 8200: 8200 history rows over 64 chunks, eight of
    them 129 rows long."""
    _need_gpu()
    s = configs.scaled(configs.C3, cache_len=8200, max_seq=8264)
    say("case: MLA FP8 layer, 8200-token cache, pos 8200")
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    out = _run_step(dec, s, 0, x, s.cache_len)
    xb = gen.input_hidden(s, 0, 0)
    rec = oracle_step(s, 0, 0, host_cache(s), xb, s.cache_len)
    _check_layer(dec, s, rec, out, s.cache_len, Cs[0], "mla pos 8200", xb)


def test_mla_fp8_two_layer_stack_one_launch():
    _need_gpu()
    s = configs.scaled(configs.C3, cache_len=200, max_seq=264)
    say("case: MLA FP8 2-layer stack, one persistent launch")
    dec, Ws, Cs = _decoder(s, [(0, 0), (0, 1)])
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    dec.persistent(start_pos=200, in_hidden=x, out_hidden=out)
    torch.cuda.synchronize()
    assert dec.status().code == 0
    xb = gen.input_hidden(s, 0, 0)
    for layer in range(2):
        rec = oracle_step(s, 0, layer, host_cache(s, 0, layer), xb, 200)
        xb = rec["out_bits"]
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    say(f"2-layer MLA stack rel err {err:.3e}")
    assert err < TOL
