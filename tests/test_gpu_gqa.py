"""GPU parity of the GQA/MHA decode layers against the CPU oracle.

Workloads: the tiny dense MHA layer (hidden 256, 4 heads x 64, FFN 1024, 128-token cache)
and the GQA MoE layer (hidden 4096, 32 q / 8 kv heads x 128, 64 experts top-8 softmax,
inter 1536, 1 shared expert, 8192-token cache). Every input comes from the seeded
generator; the oracle never sees a value produced by the HIP path.

Bars: hidden states within TOL (max-norm relative); router top-k indices identical
(the logits are accumulated in fp64 on both sides); appended cache rows equal the
oracle's bf16 rows to within one bf16 rounding step.
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
    assert st.code == 0, f"device status {st.code} stage {st.stage} layer {st.layer} wg {st.wg}"
    return out


def test_device_generator_matches_host():
    _need_gpu()
    from synth import device as sdev
    say("case: generator host==device")
    for s in (configs.C1, configs.C3):
        Wd = sdev.layer_weights(s, 0, 0) if s is configs.C1 else None
        Wh = gen.LayerWeights(s, 0, 0)
        if s is configs.C1:
            for name in ("wq", "wo", "w_down"):
                d = Wd[name]["data"]
                d = d[0] if d.dim() == 3 else d
                assert np.array_equal(d.cpu().numpy().view(np.uint16), Wh.matrix(name)["bits"]), name
            assert np.array_equal(Wd["attn_norm"].cpu().numpy(), Wh.norm("attn_norm"))
        else:
            # FP8 block-quantised matrices, including an edge block (576 rows)
            for name, shape in (("w_dkv", (576, 6144)), ("w_uk", (8192, 512))):
                codes = torch.empty(shape, dtype=torch.uint8, device="cuda")
                scales = torch.empty((-(-shape[0] // 128), -(-shape[1] // 128)), dtype=torch.float32, device="cuda")
                sdev.fill_fp8_matrix(codes, scales, 0, gen.tensor_id(name, 0, 0), s.w_std)
                h = Wh.matrix(name)
                assert np.array_equal(scales.cpu().numpy(), h["scales"]), name
                assert np.array_equal(codes.cpu().numpy(), h["codes"]), name
    s = configs.scaled(configs.C4, cache_len=300, max_seq=320)
    C = sdev.kv_cache(s, 0, 0)
    H = host_cache(s, 0, 0)
    assert np.array_equal(C["latent"].cpu().numpy().view(np.uint16), H["latent"])
    assert np.array_equal(C["index_codes"].cpu().numpy(), H["index_codes"])
    assert np.array_equal(C["index_scales"].cpu().numpy(), H["index_scales"])
    x = sdev.input_hidden(configs.C2, 0, 3)
    assert np.array_equal(x.cpu().numpy().view(np.uint16), gen.input_hidden(configs.C2, 0, 3))


def _check_layer(dec, s, rec, out, pos, cache_dev, tag, x_bits):
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    say(f"{tag}: out rel err {err:.3e}")
    assert err < TOL, f"{tag}: out rel err {err}"
    a = dec.debug("a").cpu().numpy()
    assert rel_err(a, rec["a"]) < 1e-5, tag
    h2 = dec.debug("h2").cpu().numpy()
    assert rel_err(h2, rec["h2"]) < 1e-3, tag
    b = dec.debug("b").cpu().numpy()
    assert rel_err(b, rec["b"]) < 1e-3, tag
    q = dec.debug("q").cpu().numpy().reshape(s.n_heads, s.head_dim)
    assert rel_err(q, rec["q"]) < 1e-4, tag
    o = dec.debug("o").cpu().numpy().reshape(s.n_heads, s.head_dim)
    assert rel_err(o, rec["o"]) < 5e-3, tag
    # the appended cache rows: equal to the oracle's bf16 rows up to one rounding step
    for key, ref in (("k", rec["k_new"]), ("v", rec["v_new"])):
        got = nx.bf16_to_f64(cache_dev[key][:, pos, :].cpu().numpy().view(np.uint16))
        assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30), f"{tag}: cache row {key}"
    if s.ffn == "moe":
        sel = dec.debug("sel").cpu().numpy()
        assert list(sel) == list(rec["router_sel"]), f"{tag}: router selection {sel} vs {rec['router_sel']}"
        gates = dec.debug("gates").cpu().numpy()
        assert np.allclose(gates, rec["gates"], rtol=1e-3, atol=1e-5), tag
    check_branches(dec, s, rec, x_bits, tag)


@pytest.mark.parametrize("positions", [[128], [128, 129, 130], [0], [5, 6], [255]])
def test_tiny_dense_layer_parity(positions):
    _need_gpu()
    s = configs.C1
    say(f"case: tiny dense layer, positions {positions}")
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    hc = host_cache(s)
    from synth import device as sdev
    for i, pos in enumerate(positions):
        x = sdev.input_hidden(s, 0, i)
        out = _run_step(dec, s, 0, x, pos)
        xb = gen.input_hidden(s, 0, i)
        rec = oracle_step(s, 0, 0, hc, xb, pos)
        _check_layer(dec, s, rec, out, pos, Cs[0], f"tiny pos {pos}", xb)


def test_gqa_moe_layer_parity_full_cache():
    _need_gpu()
    s = configs.C2
    say("case: GQA MoE layer, 8192-token cache, pos 8192")
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    out = _run_step(dec, s, 0, x, s.cache_len)
    xb = gen.input_hidden(s, 0, 0)
    rec = oracle_step(s, 0, 0, host_cache(s), xb, s.cache_len)
    _check_layer(dec, s, rec, out, s.cache_len, Cs[0], "gqa-moe pos 8192", xb)


@pytest.mark.parametrize("cache_len,positions", [(300, [300, 301]), (37, [0, 37])])
def test_gqa_moe_layer_parity_ragged_cache(cache_len, positions):
    _need_gpu()
    s = configs.scaled(configs.C2, cache_len=cache_len, max_seq=cache_len + 64)
    say(f"case: GQA MoE layer, cache {cache_len}, positions {positions}")
    dec, Ws, Cs = _decoder(s, [(1, 0)])
    hc = host_cache(s, 1, 0)
    from synth import device as sdev
    W = gen.LayerWeights(s, 1, 0)
    for i, pos in enumerate(positions):
        x = sdev.input_hidden(s, 1, i)
        out = _run_step(dec, s, 0, x, pos)
        xb = gen.input_hidden(s, 1, i)
        rec = oracle_step(s, 1, 0, hc, xb, pos, weights=W)
        _check_layer(dec, s, rec, out, pos, Cs[0], f"gqa-moe cache {cache_len} pos {pos}", xb)


def test_gqa_moe_two_layer_stack_one_launch():
    _need_gpu()
    s = configs.scaled(configs.C2, cache_len=512, max_seq=576)
    say("case: GQA MoE 2-layer stack, one persistent launch")
    dec, Ws, Cs = _decoder(s, [(0, 0), (0, 1)])
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    dec.persistent(start_pos=512, in_hidden=x, out_hidden=out)
    torch.cuda.synchronize()
    assert dec.status().code == 0
    xb = gen.input_hidden(s, 0, 0)
    for layer in range(2):
        rec = oracle_step(s, 0, layer, host_cache(s, 0, layer), xb, 512)
        xb = rec["out_bits"]
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    say(f"2-layer stack rel err {err:.3e}")
    assert err < TOL
