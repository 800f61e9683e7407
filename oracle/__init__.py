"""CPU oracle of the batch-1 decode layer: plain, slow, fp64 NumPy.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import, call or run anything in this package. It
shares no code with the HIP library (``persistent_latency_bound_amd``), neither
imports the other, and the library never falls back to it. The only code both sides
use is the seeded input generator in ``synth/``, which holds none of the method's
arithmetic.

Modules:
  numerics    storage formats (bf16, OCP E4M3FN), RMSNorm, RoPE, softmax, SwiGLU, top-k
  layer       one decode layer: GQA/MHA, MLA (non-absorbed), sparse indexer, MoE router, experts
  model       a layer stack with LM head, greedy decode loop, multi-token verify
  accounting  closed-form bytes and FLOPs per token

Pins: see tests/test_oracle_pins.py. The end-to-end layer and stack functions are
compositions of pinned pieces plus whole-layer special cases (zero weights, uniform
attention, single-row caches); no page prints a numeric example of a whole layer.
"""
