"""The no-allocation entry point (decode_layer_init_static) against decode_layer_init.

decode_layer_init_static sets a handle up on the library's own static device array
instead of a caller-allocated workspace. Two calls in a row on one GPU, the second with a
smaller workspace (a 2-layer FP8 MLA stack, then the tiny dense layer): each must give
bit-identical outputs to a handle made by decode_layer_init on the same weights and
inputs (same kernel, same workspace layout, another base address). A configuration whose
workspace exceeds the array is refused with PLD_E_CAPACITY.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_common import TOL, bf16_tensor_to_f64, host_cache, oracle_step, rel_err, say  # noqa: E402
from synth import configs, gen  # noqa: E402

pytestmark = pytest.mark.gpu


def _run(s, n_layers, static, Ws, pos):
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    Cs = [sdev.kv_cache(s, 0, l) for l in range(n_layers)]     # fresh caches for each handle
    dec = pld.Decoder(s, Ws, Cs, static=static)
    x = sdev.input_hidden(s, 0, 0)
    out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    dec.persistent(start_pos=pos, in_hidden=x, out_hidden=out)
    torch.cuda.synchronize()
    assert dec.status().code == 0
    return dec, out.cpu().numpy()


def test_static_init_matches_workspace_init():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    cases = [("FP8 MLA 2-layer stack, cache 300", configs.scaled(configs.C3, cache_len=300, max_seq=364), 2, 300),
             ("tiny dense layer, cache 128", configs.C1, 1, 128)]
    sizes = []
    for tag, s, n, pos in cases:
        say(f"case: no-allocation init, {tag}")
        Ws = [sdev.layer_weights(s, 0, l) for l in range(n)]
        sizes.append(pld.lib().pld_workspace_bytes(ctypes.byref(pld.config_from_shape(s)), n))
        dref, ref = _run(s, n, False, Ws, pos)
        dst, got = _run(s, n, True, Ws, pos)
        assert np.array_equal(got, ref), f"{tag}: static handle output differs"
        if n == 1:
            rec = oracle_step(s, 0, 0, host_cache(s), gen.input_hidden(s, 0, 0), pos)
            err = rel_err(bf16_tensor_to_f64(torch.from_numpy(got)), rec["out"])
            assert err < TOL, err
        say(f"  identical to decode_layer_init ({sizes[-1]} workspace bytes)")
        del dst, dref
    assert sizes[1] < sizes[0]
    # a workspace beyond the 32 MiB array is refused before anything is touched (the FP8 MLA
    # layer with room for 150000 rows: its RoPE table alone is 38 MB)
    big_shape = configs.scaled(configs.C3, max_seq=150000)
    big = pld.config_from_shape(big_shape)
    assert pld.lib().pld_workspace_bytes(ctypes.byref(big), 1) > (32 << 20)
    h = ctypes.c_void_p()
    rc = pld.lib().decode_layer_init_static(ctypes.byref(big), 1, (pld.PldLayerWeights * 1)(),
                                            (pld.PldKvCache * 1)(), None, ctypes.byref(h))
    assert rc == pld.PLD_E_CAPACITY and not h.value
