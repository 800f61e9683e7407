"""GPU parity of the FP8 MLA MoE layer with LUT3 expert weights against the CPU oracle.

Workload: the FP8 MLA layer (hidden 6144, 64 heads, latent 512 + rope 64, 256 experts top-8
of width 2048, one shared expert) whose routed and shared expert matrices store a 3-bit index
per weight into the 8-entry E4M3 codebook of its 8x64 block (3.125 bits per weight), decoded
in registers by the GEMV. Attention weights stay FP8.

Bars: hidden state within TOL; y, f and every expert slot's m within the branch bars (the
expert activations m exercise the LUT gate/up GEMV directly, f the LUT down GEMV); router
top-k identical. The device fill of LUT3 matrices equals the host generator byte for byte.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_common import TOL, bf16_tensor_to_f64, check_branches, host_cache, oracle_step, rel_err, say  # noqa: E402
from synth import configs, gen  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_device_lut3_generator_matches_host():
    _need_gpu()
    from synth import device as sdev
    say("case: LUT3 generator host == device")
    for rows, cols, tid in ((2048, 6144, 1234), (6144, 2048, 99)):
        idx = torch.empty((rows, cols * 3 // 8), dtype=torch.uint8, device="cuda")
        cb = torch.empty((rows // 8, cols // 64, 8), dtype=torch.uint8, device="cuda")
        sdev.fill_lut3_matrix(idx, cb, 0, tid, 0.02)
        hi, hc = gen.lut3_matrix(0, tid, rows, cols, 0.02)
        assert np.array_equal(idx.cpu().numpy(), hi), (rows, cols)
        assert np.array_equal(cb.cpu().numpy(), hc), (rows, cols)


def _check(dec, s, rec, out, tag, xb):
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    say(f"{tag}: out rel err {err:.3e}")
    assert err < TOL, tag
    sel = dec.debug("sel").cpu().numpy()
    assert list(sel) == list(rec["router_sel"]), f"{tag}: router selection {sel} vs {rec['router_sel']}"
    assert np.allclose(dec.debug("gates").cpu().numpy(), rec["gates"], rtol=1e-3, atol=1e-5), tag
    check_branches(dec, s, rec, xb, tag)


@pytest.mark.parametrize("cache_len,positions", [(300, [300, 301]), (8192, [8192])])
def test_lut3_layer_parity(cache_len, positions):
    _need_gpu()
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    s = configs.scaled(configs.C7, cache_len=cache_len, max_seq=cache_len + 64)
    say(f"case: MLA layer with LUT3 experts, cache {cache_len}, positions {positions}")
    Ws = [sdev.layer_weights(s, 0, 0)]
    Cs = [sdev.kv_cache(s, 0, 0)]
    dec = pld.Decoder(s, Ws, Cs)
    hc = host_cache(s)
    W = gen.LayerWeights(s, 0, 0)
    for i, pos in enumerate(positions):
        x = sdev.input_hidden(s, 0, i)
        out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
        dec.step(0, x, pos, out)
        torch.cuda.synchronize()
        assert dec.status().code == 0
        xb = gen.input_hidden(s, 0, i)
        rec = oracle_step(s, 0, 0, hc, xb, pos, weights=W)
        _check(dec, s, rec, out, f"lut3 pos {pos}", xb)
