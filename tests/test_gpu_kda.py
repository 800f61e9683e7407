"""GPU parity of the KDA linear-attention MoE decode layer against the CPU oracle.

Workload: hidden 6144, 32 KDA heads of 128 key/value channels, decay rank 128, width-4
causal convolution, FP8 E4M3 weights with fp32 128x128 block scales, 256 routed experts
top-8 (biased-score router) + one shared expert of width 2048. The per-head fp32 state and
the convolution ring are the layer's cache; every step rewrites both in place.

Bars: hidden state within TOL; y, f and m within the branch bars; the head outputs before
their norm and gate (o) within 1e-3 of their max-norm; the new state and the ring slot of
the position within 1e-4 (fp32 arithmetic on both sides of the comparison, the oracle in
fp64); router top-k identical.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_common import TOL, bf16_tensor_to_f64, check_branches, oracle_step, rel_err, say  # noqa: E402
from synth import configs, gen  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _decoder(s, layers):
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    Ws = [sdev.layer_weights(s, 0, l) for l in layers]
    Cs = [sdev.kv_cache(s, 0, l) for l in layers]
    return pld.Decoder(s, Ws, Cs), Ws, Cs


def _check(dec, s, rec, out, pos, C, tag, xb):
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    o = dec.debug("o").cpu().numpy().reshape(s.n_heads, s.head_dim)
    e_o = rel_err(o, rec["o_raw"])
    st = C["kda_state"].cpu().numpy()
    e_s = rel_err(st, rec["kda_state_new"])
    ring = C["conv_ring"][pos % (s.conv_width - 1)].cpu().numpy()
    e_r = rel_err(ring, rec["kda_x32"])
    say(f"{tag}: out {err:.2e}, o {e_o:.2e}, state {e_s:.2e}, ring {e_r:.2e}")
    assert err < TOL, tag
    assert e_o < 1e-3, f"{tag}: head outputs"
    assert e_s < 1e-4, f"{tag}: state"
    assert e_r < 1e-4, f"{tag}: convolution ring"
    assert rel_err(dec.debug("a").cpu().numpy(), rec["a"]) < 1e-5, tag
    sel = dec.debug("sel").cpu().numpy()
    assert list(sel) == list(rec["router_sel"]), f"{tag}: router selection {sel} vs {rec['router_sel']}"
    check_branches(dec, s, rec, xb, tag)


def test_kda_layer_parity_chained_steps():
    """Three chained one-layer launches at positions 100-102: the state and the ring written
    by each step are what the next one reads."""
    _need_gpu()
    s = configs.scaled(configs.C6, cache_len=100, max_seq=164)
    say("case: KDA layer, chained positions 100, 101, 102")
    dec, Ws, Cs = _decoder(s, [0])
    from synth import device as sdev
    W = gen.LayerWeights(s, 0, 0)
    hc = gen.padded_cache(s)
    for i, pos in enumerate((100, 101, 102)):
        x = sdev.input_hidden(s, 0, i)
        out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
        dec.step(0, x, pos, out)
        torch.cuda.synchronize()
        assert dec.status().code == 0
        xb = gen.input_hidden(s, 0, i)
        rec = oracle_step(s, 0, 0, hc, xb, pos, weights=W)
        _check(dec, s, rec, out, pos, Cs[0], f"kda pos {pos}", xb)


def test_kda_two_layer_stack_one_launch():
    _need_gpu()
    s = configs.scaled(configs.C6, cache_len=7, max_seq=64)
    say("case: KDA 2-layer stack, one persistent launch at position 7")
    dec, Ws, Cs = _decoder(s, [0, 1])
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    dec.persistent(start_pos=7, in_hidden=x, out_hidden=out)
    torch.cuda.synchronize()
    assert dec.status().code == 0
    xb = gen.input_hidden(s, 0, 0)
    for layer in range(2):
        hc = gen.padded_cache(s, 0, layer)
        rec = oracle_step(s, 0, layer, hc, xb, 7)
        e_s = rel_err(Cs[layer]["kda_state"].cpu().numpy(), rec["kda_state_new"])
        say(f"layer {layer}: state {e_s:.2e}")
        assert e_s < 1e-4
        xb = rec["out_bits"]
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    say(f"2-layer KDA stack rel err {err:.3e}")
    assert err < TOL
