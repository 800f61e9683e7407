"""Shared pieces of the GPU parity tests: device inputs (synth.device), oracle references
(oracle/, fed only by the host generator), and the comparison metric."""
from __future__ import annotations

import sys

import numpy as np

from oracle import layer as OL
from oracle import numerics as nx
from synth import gen

TOL = 2e-2   # max relative error ||g - o||_inf / ||o||_inf for hidden states and logits


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def bf16_tensor_to_f64(t) -> np.ndarray:
    return nx.bf16_to_f64(t.detach().cpu().numpy().view(np.uint16))


def host_cache(s, seed=0, layer=0, fill_len=None):
    """Host copy of a prefilled cache, padded to max_seq rows (positions >= fill_len are zero)."""
    return gen.padded_cache(s, seed, layer, fill_len)


def oracle_step(s, seed, layer, cache, x_bits, pos, weights=None):
    W = weights if weights is not None else gen.LayerWeights(s, seed, layer)
    rec = OL.decode_layer(s, W, cache, x_bits, pos)
    OL.append_to_cache(s, cache, rec, pos)
    return rec


# Direct bars on the two residual branches and the expert activations, each relative to its
# own max-norm (the hidden state is dominated by the residual, so a bar on it alone would
# admit a large error in y or f). y = h2 - x is recovered from the fp32 h2 words (the
# subtraction is exact to an fp32 step of h2, far below these bars); f is the kernel's fp32
# FFN output before the residual add; m[slot] = silu(gate) * up of each expert slot.
BAR_Y = 5e-3
BAR_F = 5e-3
BAR_M = 5e-3


def check_branches(dec, s, rec, x_bits, tag, bar_y=BAR_Y, bar_f=BAR_F, bar_m=BAR_M):
    x = nx.bf16_to_f64(np.asarray(x_bits).view(np.uint16))
    h2 = dec.debug("h2").cpu().numpy().astype(np.float64)
    e_y = rel_err(h2 - x, rec["y"])
    f = dec.debug("f").cpu().numpy().astype(np.float64)
    e_f = rel_err(f, rec["f"])
    slots = s.top_k + s.n_shared if s.ffn == "moe" else 1
    m = dec.debug("m").cpu().numpy().astype(np.float64).reshape(slots, s.inter)
    e_m = [rel_err(m[j], rec["m"][j]) for j in range(slots)]
    say(f"{tag}: y {e_y:.2e} (|y| {np.abs(rec['y']).max():.3f}), f {e_f:.2e} (|f| {np.abs(rec['f']).max():.3f}), "
        f"m max {max(e_m):.2e}")
    assert e_y < bar_y, f"{tag}: W_O output y rel err {e_y}"
    assert e_f < bar_f, f"{tag}: FFN output f rel err {e_f}"
    assert max(e_m) < bar_m, f"{tag}: expert activations m rel err {e_m}"
