"""Host-side checks of the C-ABI boundary (no GPU needed).

* libpld.so loads and exports every function that include/pld.h declares;
* the Python binding's ctypes structs have the same sizes and field offsets as the C
  structs (a gcc-compiled probe of the header prints them);
* status strings and the binding's config marshalling.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import persistent_latency_bound_amd as pld
from synth import configs

HDR = pld.HEADER_PATH


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_declares_the_binding_exports():
    assert sorted(pld.EXPORTS) == declared_functions()


def test_library_loads_and_exports_every_declared_symbol():
    L = pld.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", pld.LIB_PATH], capture_output=True, text=True).stdout
    syms = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for name in declared_functions():
        assert name in syms, f"{name} not exported"


def _c_layout():
    src = r'''
#include <stdio.h>
#include <stddef.h>
#include "pld.h"
#define P(T, f) printf("%s.%s %zu\n", #T, #f, offsetof(T, f));
int main(void) {
  printf("pld_config %zu\n", sizeof(pld_config));
  printf("pld_matrix %zu\n", sizeof(pld_matrix));
  printf("pld_layer_weights %zu\n", sizeof(pld_layer_weights));
  printf("pld_kv_cache %zu\n", sizeof(pld_kv_cache));
  printf("pld_head_weights %zu\n", sizeof(pld_head_weights));
  printf("pld_device_status %zu\n", sizeof(pld_device_status));
  printf("pld_persistent_args %zu\n", sizeof(pld_persistent_args));
  P(pld_config, eps) P(pld_config, rope_base) P(pld_config, vocab) P(pld_config, max_seq)
  P(pld_layer_weights, wo) P(pld_layer_weights, router) P(pld_layer_weights, w_down)
  P(pld_layer_weights, w_aup) P(pld_layer_weights, o_norm) P(pld_config, kda_rank)
  P(pld_config, expert_wfmt) P(pld_config, max_query)
  P(pld_persistent_args, in_hidden) P(pld_persistent_args, out_accepted)
  P(pld_persistent_args, temperature) P(pld_persistent_args, sample_seed)
  printf("pld_spec_args %zu\n", sizeof(pld_spec_args));
  P(pld_spec_args, temperature) P(pld_spec_args, out_tokens) P(pld_spec_args, out_stats)
  printf("pld_batch_args %zu\n", sizeof(pld_batch_args));
  P(pld_batch_args, in_token) P(pld_batch_args, out_logits) P(pld_batch_args, temperature)
  P(pld_batch_args, sample_seed) P(pld_config, max_batch)
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "probe.c")
        exe = os.path.join(d, "probe")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HDR), "-o", exe, c], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    return dict((k, int(v)) for k, v in (line.split() for line in out.splitlines()))


def test_ctypes_struct_layout_matches_c():
    lay = _c_layout()
    assert lay["pld_config"] == ctypes.sizeof(pld.PldConfig)
    assert lay["pld_matrix"] == ctypes.sizeof(pld.PldMatrix)
    assert lay["pld_layer_weights"] == ctypes.sizeof(pld.PldLayerWeights)
    assert lay["pld_kv_cache"] == ctypes.sizeof(pld.PldKvCache)
    assert lay["pld_head_weights"] == ctypes.sizeof(pld.PldHeadWeights)
    assert lay["pld_device_status"] == ctypes.sizeof(pld.PldDeviceStatus)
    assert lay["pld_persistent_args"] == ctypes.sizeof(pld.PldPersistentArgs)
    assert lay["pld_spec_args"] == ctypes.sizeof(pld.PldSpecArgs)
    assert lay["pld_batch_args"] == ctypes.sizeof(pld.PldBatchArgs)
    for key, off in lay.items():
        if "." in key:
            T, f = key.split(".")
            cls = {"pld_config": pld.PldConfig, "pld_layer_weights": pld.PldLayerWeights,
                   "pld_persistent_args": pld.PldPersistentArgs, "pld_spec_args": pld.PldSpecArgs,
                   "pld_batch_args": pld.PldBatchArgs}[T]
            assert getattr(cls, f).offset == off, key


def test_status_strings():
    L = pld.lib()
    assert L.pld_status_string(0) == b"ok"
    assert b"unsupported" in L.pld_status_string(pld.PLD_E_UNSUPPORTED)
    assert L.pld_status_string(12345) == b"unknown status"


def test_null_arguments_are_rejected_before_any_device_work():
    L = pld.lib()
    h = ctypes.c_void_p()
    assert L.decode_layer_init(None, 1, None, None, None, None, 0, ctypes.byref(h)) == pld.PLD_E_INVALID
    assert L.decode_step(None, 0, None, 0, None, None) == pld.PLD_E_INVALID
    assert L.decode_layers_persistent(None, None, None) == pld.PLD_E_INVALID
    assert L.decode_verify_batched(None, None, None) == pld.PLD_E_INVALID
    assert L.decode_batch(None, None, None) == pld.PLD_E_INVALID
    assert L.decode_reset(None) == pld.PLD_E_INVALID
    L.decode_layer_destroy(None)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_config_marshalling(name):
    s = configs.LAYERS[name]
    c = pld.config_from_shape(s)
    assert c.hidden == s.hidden and c.max_seq == s.max_seq and c.eps == s.eps and c.inter == s.inter
    assert c.attn_kind == (pld.PLD_ATTN_GQA if s.attn == "gqa" else pld.PLD_ATTN_MLA)
    assert c.wfmt == (pld.PLD_WFMT_FP8_BLOCK128 if s.wfmt == "fp8" else pld.PLD_WFMT_BF16)
