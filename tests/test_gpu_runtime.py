"""GPU tests of the persistent runtime's failure and ordering paths (all forced from the
host; every kernel still exits normally).

* Watchdog: with the test hook that makes workgroup 0 leave at the start of a launch (a
  producer that never publishes), the other workgroups' bounded waits expire; the status
  names the first expired wait, later launches are refused with PLD_E_STATE, and after
  decode_reset the same step matches the oracle.
* Ordering stress: with seeded per-workgroup delays at the start of four stages, the
  outputs and intermediates are bit-identical to an undelayed run (every sum has a fixed
  order, so timing must not matter).
* Stale handoffs: every LL word left by the previous launch gets a NaN payload under its old
  epoch; the next launch must not consume any of them (bit-identical output).
These follow the ordering and evidence concerns of the vLLM Kimi K3 backend article
("Agent-written kernels face evidence gates").
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


def _decoder(s, layers):
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    Ws = [sdev.layer_weights(s, 0, l) for l in layers]
    Cs = [sdev.kv_cache(s, 0, l) for l in layers]
    return pld.Decoder(s, Ws, Cs), Ws, Cs


def _launch(dec, s, x, pos):
    out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    dec.persistent(start_pos=pos, in_hidden=x, out_hidden=out)
    torch.cuda.synchronize()
    return out


# (wait ids of the status word: 0 x, 1 q/k/v, 2 new k/v row, 3 partials, 4 o, 5 h2, 6 router logits, 7 m, ...)
def test_watchdog_expiry_state_and_reset():
    _need_gpu()
    import persistent_latency_bound_amd as pld
    s = configs.scaled(configs.C2, cache_len=300, max_seq=364)
    say("case: watchdog, GQA MoE layer (cache 300): workgroup 0 withheld, 2 ms budget")
    dec, Ws, Cs = _decoder(s, [0])
    nwg, _ = dec.launch_shape()
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    dec.set_watchdog_us(2000)
    dec.set_test_hooks(pld.PLD_HOOK_DROP_WG0)
    out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    dec.step(0, x, 300, out)                  # asynchronous: the launch itself is accepted
    st = dec.status()
    say(f"status: code {st.code} wait {st.stage} layer {st.layer} token {st.token} wg {st.wg}")
    assert st.code == pld.PLD_E_DEVICE_TIMEOUT
    assert 0 <= st.stage <= 15 and st.layer == 0 and st.token == 0 and 1 <= st.wg < nwg
    with pytest.raises(pld.PldError) as e:
        dec.step(0, x, 300, out)
    assert e.value.code == pld.PLD_E_STATE
    dec.reset()
    dec.set_watchdog_us(2_000_000)
    out = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    dec.step(0, x, 300, out)
    torch.cuda.synchronize()
    assert dec.status().code == 0
    xb = gen.input_hidden(s, 0, 0)
    rec = oracle_step(s, 0, 0, host_cache(s), xb, 300)
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    say(f"after reset: out rel err {err:.2e}")
    assert err < TOL
    check_branches(dec, s, rec, xb, "after reset")


SNAP = {"gqa": ("q", "o", "h2", "m", "b", "f", "sel", "gates"),
        "mla": ("q", "qlat", "olat", "o", "h2", "m", "b", "f", "sel", "gates")}


def _snapshot(dec, s):
    names = SNAP[s.attn] + (("isel",) if s.index_topk else ())
    return {n: dec.debug(n).cpu().numpy().copy() for n in names}


CASES = [
    ("gqa", lambda: configs.scaled(configs.C2, cache_len=512, max_seq=576), 512),
    ("mla_fp8", lambda: configs.scaled(configs.C3, cache_len=300, max_seq=364), 300),
    ("sparse", lambda: configs.scaled(configs.C4, cache_len=500, max_seq=564, index_topk=128), 500),
]


@pytest.mark.parametrize("name,shape_fn,pos", CASES, ids=[c[0] for c in CASES])
def test_seeded_delays_do_not_change_results(name, shape_fn, pos):
    _need_gpu()
    import persistent_latency_bound_amd as pld
    s = shape_fn()
    say(f"case: seeded delays, {name} 2-layer stack at pos {pos}")
    dec, Ws, Cs = _decoder(s, [0, 1])
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    ref = _launch(dec, s, x, pos).cpu().numpy()
    assert dec.status().code == 0
    snap = _snapshot(dec, s)
    for seed in (1, 2, 3):
        dec.set_test_hooks(pld.PLD_HOOK_DELAY, seed)
        got = _launch(dec, s, x, pos).cpu().numpy()
        assert dec.status().code == 0
        assert np.array_equal(got, ref), f"{name}: output changed under delays (seed {seed})"
        for n, v in _snapshot(dec, s).items():
            assert np.array_equal(v, snap[n]), f"{name}: {n} changed under delays (seed {seed})"
        say(f"  seed {seed}: identical")
    dec.set_test_hooks(0)


POISON = {"gqa": ("x", "q", "kv", "part", "o", "h2", "logits", "m"),
          "mla": ("x", "q", "qrope", "cq", "ckv", "qlat", "part", "olat", "o", "h2", "logits", "m")}


@pytest.mark.parametrize("name,shape_fn,pos", CASES, ids=[c[0] for c in CASES])
def test_stale_handoff_words_are_never_consumed(name, shape_fn, pos):
    _need_gpu()
    s = shape_fn()
    say(f"case: NaN-poisoned stale handoff words, {name} 2-layer stack at pos {pos}")
    dec, Ws, Cs = _decoder(s, [0, 1])
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    ref = _launch(dec, s, x, pos).cpu().numpy()
    assert dec.status().code == 0
    names = POISON[s.attn] + (("qi", "ixr", "ilist", "isel") if s.index_topk else ())
    for n in names:
        w = dec.debug_raw(n).view(torch.int32).view(-1, 2)   # (payload, epoch) words
        w[:, 0] = 0x7FC07FC0                                  # a NaN as fp32 and as both bf16 halves
    torch.cuda.synchronize()
    got = _launch(dec, s, x, pos).cpu().numpy()
    assert dec.status().code == 0
    assert np.array_equal(got, ref), f"{name}: a stale (NaN) handoff word reached the output"
    say(f"  {len(names)} LL buffers poisoned: output identical")
