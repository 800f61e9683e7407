"""Benchmark of the persistent batch-1 decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Workload (default, mla_stack24_fp8_greedy256): 24 stacked MLA + FP8 MoE decode layers
(hidden 6144, 64 heads, latent 512 + rope 64, q_lora 1536, 256 experts top-8 of width 2048
with the biased-score router, one shared expert, FP8 E4M3 weights with fp32 128x128 block
scales, each layer with its own seeded weights) and an FP8 LM head over 32768 tokens. One
step is ONE launch of decode_layers_persistent that decodes 256 consecutive greedy tokens
from an 8192-token prefilled cache (positions 8192..8447) through every layer and the
head. The 24 layers hold 235 GB of FP8 weights, far more than the 256 MB Infinity Cache,
so every byte comes from HBM.

Other workloads (--workload), one token through R = --layers independent seeded copies of
one layer per launch (R copies keep the weights cold; each step has its own seeded input,
so the routed experts change from step to step, and the step rewrites the same cache row):
  gqa_moe_bf16_decode_layer           hidden 4096, GQA 32 q / 8 kv heads x 128, 8192-token
                                      cache, 64 experts top-8 (softmax) of width 1536 + 1
                                      shared, bf16 weights
  mla_moe256_fp8_decode_layer         one layer of the default stack's shape, 8192-token cache
  sparse_mla_moe64_bf16_decode_layer  hidden 4096, 32 MLA heads, indexer 8x64 with FP8 keys
                                      choosing 2048 of 32769 cached tokens, 64 experts of
                                      width 1536, bf16 weights, at position 32768
  mla_stack24_fp8_verify6             the default stack, one 6-position verify per launch

Prints ONE JSON line: value = microseconds per layer (lower is better), plus the HBM
roofline of the kernel (algorithmic bytes per launch / measured launch time), the HBM bytes
the counters saw (when profiles/ holds counter runs of the current kernel sources), and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X published HBM3E bandwidth
WORKLOADS = {   # name -> (synth.configs attribute, traffic file stem, dtype of the arithmetic)
    "gqa_moe_bf16_decode_layer": ("C2", "traffic_gqa_moe_bf16", "bf16"),
    "mla_moe256_fp8_decode_layer": ("C3", "traffic_mla_moe256_fp8", "fp8-e4m3 weights, fp32 accumulate"),
    # sparse MLA: indexer (fp64 scores over every cached token) + top-2048 attention, bf16 weights
    "sparse_mla_moe64_bf16_decode_layer": ("C4", "traffic_sparse_mla_moe64_bf16",
                                           "bf16 weights, fp32 accumulate; indexer scores fp64"),
    # 24 stacked FP8 MLA layers + FP8 LM head, greedy loop over 256 tokens in one launch
    "mla_stack24_fp8_greedy256": ("C5", "traffic_mla_stack24_fp8", "fp8-e4m3 weights, fp32 accumulate, fp64 head"),
    # the FP8 MLA layer with LUT3 experts (3-bit indices into 8-entry E4M3 codebooks, 3.125 bits/weight)
    "mla_moe256_lut3_decode_layer": ("C7", "traffic_mla_moe256_lut3",
                                     "lut3 expert weights (E4M3 codebooks) + fp8 attention, fp32 accumulate"),
    # KDA linear attention (32 heads x 128, fp32 state) + the FP8 256-expert MoE
    "kda_moe256_fp8_decode_layer": ("C6", "traffic_kda_moe256_fp8", "fp8-e4m3 weights, fp32 accumulate and state"),
    # the same stack, one 6-position speculative verify per launch (seeded drafts)
    "mla_stack24_fp8_verify6": ("C5", "traffic_mla_stack24_fp8_verify6",
                                "fp8-e4m3 weights, fp32 accumulate, fp64 head"),
    "mla_stack24_fp8_batch8": ("C5", "traffic_mla_stack24_fp8_batch8",
                               "fp8-e4m3 weights widened to bf16, bf16 activations, fp32 accumulate "
                               "(matrix cores); fp64 router and head"),
    "mla_stack24_fp8_verify6_batched": ("C5", "traffic_mla_stack24_fp8_verify6_batched",
                                        "fp8-e4m3 weights widened to bf16, bf16 activations, fp32 accumulate "
                                        "(matrix cores); fp64 router and head"),
}
DEFAULT_WORKLOAD = "mla_stack24_fp8_greedy256"
KERNEL_SOURCES = [os.path.join(ROOT, "persistent_latency_bound_amd", "csrc", f)
                  for f in ("pld_kernel.hip", "pld_device.hpp", "pld_mla.hpp", "pld_kda.hpp", "pld_math.hpp", "pld_batch.hpp")]


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_per_launch(workload: str, layers: int, tokens: int = 1):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", WORKLOADS[workload][1] + ".json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("kernel_sha") != kernel_sha() or t.get("layers_per_launch") != layers:
        return None
    if t.get("tokens_per_launch", 1) != tokens:
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(shape, pos: int, budget_s: float = 20.0, max_n: int = 8) -> dict:
    """The CPU oracle (unchanged) on a bounded sample: whole layer-tokens of the same workload."""
    from oracle import layer as OL
    from synth import gen

    W = gen.LayerWeights(shape, 0, 0, cache_size=256)
    cache = gen.padded_cache(shape)
    x = gen.input_hidden(shape, 0, 0)
    OL.decode_layer(shape, W, cache, x, pos)          # generates and caches the weights it touches
    n, t0 = 0, time.perf_counter()
    while True:
        OL.decode_layer(shape, W, cache, x, pos)
        n += 1
        if time.perf_counter() - t0 > budget_s / 2 or n >= max_n:
            break
    dt = (time.perf_counter() - t0) / n
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": round(dt * 1e6, 1), "unit": "us/layer", "cores": cores, "kind": "oracle",
            "sample": f"{n} layer-token(s) of layer 0 ({shape.name}) at position {pos} after one warm-up call that "
                      f"generates the weights; fp64 NumPy, BLAS and generator threads = {cores}"}


def stream_copy_gbps() -> float:
    """Measured HBM rate of a plain 4 GiB device-to-device copy (bytes read + bytes written per
    second), reported beside the 8 TB/s published peak."""
    import torch
    src = torch.ones(1 << 32, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record()
    for _ in range(n):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * src.numel() * n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


TR_SLOTS = 56   # stamps per (step, workgroup) written by the device trace
TR_WAIT = 50    # not a stamp: ticks a workgroup spent inside its dependency waits during the step
TICK_US = 1e-2  # wall_clock64 runs at 100 MHz on MI355X (hipDeviceAttributeWallClockRate = 100000 kHz)
SLOT_NAMES = {32: "head_ready", 33: "head_gemv", 34: "token", 0: "start", 1: "x_ready", 2: "qkv_done", 3: "att_ready", 4: "att_done", 5: "o_ready", 6: "wo_done",
              7: "h2_ready", 8: "router_ready", 9: "ffn_done", 10: "m_ready", 11: "down_done", 12: "att_q",
              13: "att_softmax", 14: "att_partial", 15: "att_merged", 16: "topk", 18: "m_stored", 19: "down_gemv",
              20: "down_epi", 21: "qkv_gemv", 22: "shared_gemv", 23: "att_pv", 24: "x_normed", 25: "merge_start",
              26: "merge_fetched", 27: "router_logit", 28: "att_drained", 30: "att_scores", 17: "blk0_staged", 31: "blk0_done",
              35: "idx_done", 36: "sel_keys", 37: "sel_passes", 38: "sel_done", 39: "sel_pass0", 40: "sel_pass1",
              41: "sel_pass2", 42: "sel_pass3", 43: "sel_pass4", 44: "sel_pass5", 45: "sel_rank_loaded",
              46: "sel_lists_arrived", 47: "sel_fetch_start",
              48: "cq_ready", 49: "q_gemv"}


def write_trace_summary(dec, x, out, R, path, pos):
    """One extra (untimed) launch with the device trace on. For every stamped slot: median
    time since the step's first stamp (over workgroups and layers), in stamp order, and the
    gaps between consecutive medians."""
    import numpy as np
    import torch
    nwg, _ = dec.launch_shape()
    buf = torch.zeros(R * nwg * TR_SLOTS, dtype=torch.int64, device="cuda")
    dec.set_trace(buf)
    dec.persistent(start_pos=pos, in_hidden=x, out_hidden=out)
    torch.cuda.synchronize()
    dec.set_trace(None)
    t = buf.cpu().numpy().reshape(R, nwg, TR_SLOTS).astype(np.float64)
    tick_us = 1e-2   # wall_clock64 runs at 100 MHz on MI355X (hipDeviceAttributeWallClockRate = 100000 kHz)
    start = t[:, :, 0].min(axis=1, keepdims=True)
    rows = []
    for slot in range(TR_SLOTS):
        if slot == TR_WAIT:
            continue
        v = t[:, :, slot]
        msk = v > 0
        if not msk.any():
            continue
        rel = (v - start)[msk] * tick_us
        rows.append((float(np.median(rel)), slot, float(np.max(rel)), int(msk.sum())))
    rows.sort()
    stamps, prev = [], 0.0
    for med, slot, mx, cnt in rows:
        stamps.append({"slot": SLOT_NAMES.get(slot, str(slot)), "median_us": round(med, 2), "max_us": round(mx, 2),
                       "gap_us": round(med - prev, 2), "stamps": cnt})
        prev = med
    layer_us = [(t[l, :, 11].max() - t[l, :, 0].min()) * tick_us for l in range(R)]
    wait = np.median(t[:, :, TR_WAIT], axis=1) * tick_us
    summary = {"layers": R, "nwg": nwg, "stamps_from_layer_start": stamps,
               "wait_us_per_layer_median_wg": [round(float(v), 2) for v in wait],
               "layer_critical_path_us": [round(float(v), 2) for v in layer_us]}
    with open(path, "w") as f:
        json.dump(summary, f, indent=1)
    np.save(os.path.splitext(path)[0] + "_raw.npy", t)   # [layer][workgroup][slot] wall-clock ticks


def idle_per_token(dec, one_launch, n_layers, tokens_traced=2):
    """One extra (untimed) launch with the device trace on for its first tokens. Per step (one
    layer of one token), every workgroup's summed dependency-wait time; the median over
    workgroups, summed over the layers of a token, averaged over the traced tokens. Also the
    per-token critical path from the first stamp to the token's last stamp."""
    import numpy as np
    import torch
    nwg, _ = dec.launch_shape()
    nst = tokens_traced * n_layers
    buf = torch.zeros(nst * nwg * TR_SLOTS, dtype=torch.int64, device="cuda")
    dec.set_trace(buf)
    one_launch()
    torch.cuda.synchronize()
    dec.set_trace(None)
    t = buf.cpu().numpy().reshape(nst, nwg, TR_SLOTS).astype(np.float64)
    wait = np.median(t[:, :, TR_WAIT], axis=1) * TICK_US            # [steps]
    per_tok = wait.reshape(tokens_traced, n_layers).sum(axis=1)
    return float(per_tok.mean()), t


def run_stack(args):
    """The multi-layer workload: one launch = n_tokens greedy tokens through every layer and the head."""
    import torch
    import persistent_latency_bound_amd as pld
    from oracle import accounting
    from synth import configs, device as sdev, gen
    m = configs.C5
    L = m.layer
    pos0, n_tok = L.cache_len, args.tokens
    # (not in counter runs: rocprofv3 --pmc has crashed on the 4 GiB fill and copies)
    copy_rate = None if args.calib_copy else stream_copy_gbps()
    Ws = [sdev.layer_weights(L, 0, l) for l in range(m.n_layers)]
    Cs = [sdev.kv_cache(L, 0, l) for l in range(m.n_layers)]
    head = {"embed": sdev.embedding(m), "final_norm": sdev.final_norm(m), "head": sdev.head(m)}
    dec = pld.Decoder(L, Ws, Cs, head=head, vocab=m.vocab)
    out = torch.zeros(L.hidden, dtype=torch.int16, device="cuda")
    toks = torch.zeros(n_tok, dtype=torch.int32, device="cuda")
    tok0 = gen.first_token(m)
    torch.cuda.synchronize()

    def one():
        dec.persistent(start_pos=pos0, in_token=tok0, n_tokens=n_tok, out_hidden=out, out_tokens=toks)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    st = dec.status()
    if st.code != 0:
        raise SystemExit(f"device status {st.code} wait {st.stage}")
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        one()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    st = dec.status()
    if st.code != 0:
        raise SystemExit(f"device status {st.code} wait {st.stage}")
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    lt = m.n_layers * n_tok
    us_lt = ms * 1e3 / lt
    layer_b = sum(accounting.layer_bytes(L, pos0 + t) for t in range(n_tok)) * m.n_layers
    head_b = accounting.head_bytes(L.hidden, m.vocab) * n_tok
    achieved = (layer_b + head_b) / (ms * 1e-3) / 1e9
    traffic = traffic_per_launch(args.workload, m.n_layers, n_tok)
    # one layer per launch through decode_step (launch cost included), after the timed region
    single_us = None
    if not args.no_single_launch:
        x = sdev.input_hidden(L, 0, 0)
        xo = torch.zeros(L.hidden, dtype=torch.int16, device="cuda")
        for _ in range(3):
            dec.step(0, x, pos0, xo)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n1 = 20
        e0.record(stream)
        for i in range(n1):
            dec.step(i % m.n_layers, x, pos0, xo)
        e1.record(stream)
        torch.cuda.synchronize()
        single_us = e0.elapsed_time(e1) * 1e3 / n1
    idle_us = None
    if not args.no_idle:
        idle_us, t = idle_per_token(dec, one, m.n_layers)
        if args.trace:
            import numpy as np
            np.save(os.path.splitext(args.trace)[0] + "_raw.npy", t)   # [step][workgroup][slot] ticks
    line = {
        "metric": "batch-1 decode us/layer (achieved HBM TB/s vs peak, implied tokens/s/user)",
        "value": round(us_lt, 3), "unit": "us/layer", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 3), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": WORKLOADS[args.workload][2], "data": "synthetic",
        "config": {"workload": args.workload, "layers": m.n_layers, "tokens_per_launch": n_tok, "start_pos": pos0,
                   "vocab": m.vocab, "hidden": L.hidden, "batch": 1},
        "tokens_per_s_user": round(n_tok / (ms * 1e-3), 1),
        "us_per_token": round(ms * 1e3 / n_tok, 2),
        "p90_ms_per_launch": round(per[min(len(per) - 1, int(0.9 * len(per)))], 3),
        "achieved_TBps": round(achieved / 1e3, 3), "frac_of_peak": round(achieved / PEAK_HBM_GBPS, 4),
        "measured_copy_GBps": None if copy_rate is None else round(copy_rate, 1),
        "frac_of_measured_copy_rate": None if copy_rate is None else round(achieved / copy_rate, 4),
        "algorithmic_bytes_per_launch": int(layer_b + head_b),
        "launches_per_token": round(1.0 / n_tok, 6),
        "idle_us_per_token": None if idle_us is None else round(idle_us, 1),
        "single_launch_us_per_layer": None if single_us is None else round(single_us, 2),
        "wall_s_timed_region": round(wall, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 1)},
        "hbm_bytes_per_launch_counters": traffic,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(L, pos0, budget_s=30.0, max_n=2)
    print(json.dumps(line), flush=True)


def run_verify(args):
    """One launch = one 6-position verify through every layer and the head (seeded drafts).
    Reported per verify step, per layer, and as tokens/s at an acceptance length of six."""
    import torch
    import persistent_latency_bound_amd as pld
    from oracle import accounting
    from synth import configs, device as sdev, gen
    m = configs.C5
    L = m.layer
    nq = m.n_verify
    pos0 = L.cache_len
    Ws = [sdev.layer_weights(L, 0, l) for l in range(m.n_layers)]
    Cs = [sdev.kv_cache(L, 0, l) for l in range(m.n_layers)]
    head = {"embed": sdev.embedding(m), "final_norm": sdev.final_norm(m), "head": sdev.head(m)}
    batched = args.workload.endswith("_batched")
    dec = pld.Decoder(L, Ws, Cs, head=head, vocab=m.vocab, max_query=nq if batched else 0)
    out = torch.zeros(L.hidden, dtype=torch.int16, device="cuda")
    toks = torch.zeros(nq, dtype=torch.int32, device="cuda")
    acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    drafts = torch.tensor([int(d) for d in gen.draft_tokens(m, nq - 1)], dtype=torch.int32, device="cuda")
    tok0 = gen.first_token(m)
    torch.cuda.synchronize()

    def one():
        if batched:
            dec.verify_batched(pos0, tok0, drafts, out, out_tokens=toks, out_accepted=acc)
        else:
            dec.persistent(start_pos=pos0, in_token=tok0, n_query=nq, draft_tokens=drafts, out_hidden=out,
                           out_tokens=toks, out_accepted=acc)

    for _ in range(args.warmup):
        one()
    torch.cuda.synchronize()
    if dec.status().code != 0:
        raise SystemExit("device status after warm-up")
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        one()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    if dec.status().code != 0:
        raise SystemExit("device status after the timed launches")
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    layer_b = accounting.verify_layer_bytes(L, pos0, nq) * m.n_layers
    head_b = accounting.head_bytes(L.hidden, m.vocab)   # the head matrix once per verify step
    achieved = (layer_b + head_b) / (ms * 1e-3) / 1e9
    line = {
        "metric": "batch-1 decode us/layer (achieved HBM TB/s vs peak, implied tokens/s/user)",
        "value": round(ms * 1e3 / m.n_layers, 3), "unit": "us/layer (6-position verify step)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": WORKLOADS[args.workload][2], "data": "synthetic",
        "config": {"workload": args.workload, "layers": m.n_layers, "positions_per_verify": nq, "start_pos": pos0,
                   "vocab": m.vocab, "hidden": L.hidden, "batch": 1,
                   "expected_union_routed_experts": round(
                       accounting.expected_union_experts(L.n_experts, L.top_k, nq), 2)},
        "ms_per_verify_step": round(ms, 3),
        "tokens_per_s_user_at_AL6": round(nq / (ms * 1e-3), 1),
        "accepted_drafts_last_step": int(acc.item()),
        "p90_ms_per_launch": round(per[min(len(per) - 1, int(0.9 * len(per)))], 3),
        "achieved_TBps": round(achieved / 1e3, 3), "frac_of_peak": round(achieved / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_launch": int(layer_b + head_b), "wall_s_timed_region": round(wall, 3),
        "implementation": ("positions batched through every layer: dense projections, shared experts and the union "
                           "of the routed experts as skinny GEMMs on the matrix cores (weights read once per verify); "
                           "the LM head runs once per position") if batched else
                          "positions run as sequential steps inside the launch (weights read once per position)",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None},
    }
    print(json.dumps(line), flush=True)


def run_batch(args):
    """Batched decoding: B sequences of the 24-layer stack, each with its own 8192-row history,
    decode args.tokens tokens together per launch. One line for B = 8 with the curve over
    B = 1 (the single-sequence stack launch), 2, 4, 8 beside it."""
    import torch
    import persistent_latency_bound_amd as pld
    from oracle import accounting
    from synth import configs, device as sdev, gen
    m = configs.C5
    L = m.layer
    pos0 = L.cache_len
    n_tok = args.tokens
    Ws = [sdev.layer_weights(L, 0, l) for l in range(m.n_layers)]
    head = {"embed": sdev.embedding(m), "final_norm": sdev.final_norm(m), "head": sdev.head(m)}
    curve = {}
    for nb in (1, 2, 4, 8):
        if nb == 1:
            Cs = [sdev.kv_cache(L, 0, l) for l in range(m.n_layers)]
            dec = pld.Decoder(L, Ws, Cs, head=head, vocab=m.vocab)
        else:
            Cs = [{"latent": torch.cat([sdev.kv_cache(L, b, l)["latent"] for b in range(nb)], dim=0).contiguous()}
                  for l in range(m.n_layers)]
            dec = pld.Decoder(L, Ws, Cs, head=head, vocab=m.vocab, max_batch=nb)
        out = torch.zeros(L.hidden, dtype=torch.int16, device="cuda")
        tk = torch.zeros((n_tok, nb), dtype=torch.int32, device="cuda")
        toks0 = [(gen.first_token(m) + 977 * b) % m.vocab for b in range(nb)]

        def one():
            if nb == 1:
                dec.persistent(start_pos=pos0, in_token=toks0[0], n_tokens=n_tok, out_hidden=out, out_tokens=tk)
            else:
                dec.batch([pos0] * nb, toks0, n_tok, tk, out)

        for _ in range(args.warmup):
            one()
        torch.cuda.synchronize()
        if dec.status().code != 0:
            raise SystemExit(f"device status after warm-up (batch {nb})")
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            one()
        e1.record(stream)
        torch.cuda.synchronize()
        if dec.status().code != 0:
            raise SystemExit(f"device status after the timed launches (batch {nb})")
        ms = e0.elapsed_time(e1) / args.steps
        us_step = ms * 1e3 / n_tok
        union = accounting.expected_union_experts(L.n_experts, L.top_k, nb)
        curve[nb] = {"us_per_step": round(us_step, 1), "us_per_layer_step": round(us_step / m.n_layers, 2),
                     "tokens_per_s_user": round(1e6 / us_step, 1), "tokens_per_s_total": round(nb * 1e6 / us_step, 1),
                     "expected_union_routed_experts": round(union, 2)}
        del dec, Cs
        torch.cuda.empty_cache()
    c8 = curve[8]
    # algorithmic bytes of one 8-sequence step per layer: shared weights once, the expected union
    # of the routed experts, each sequence's own history and appended row
    layer_b = accounting.verify_layer_bytes(L, pos0, 8) + 7 * accounting.layer_kv_bytes(L, pos0)["kv_read"]
    step_b = layer_b * m.n_layers + accounting.head_bytes(L.hidden, m.vocab)
    achieved = step_b / (c8["us_per_step"] * 1e-6) / 1e9
    line = {
        "metric": "batch-1 decode us/layer (achieved HBM TB/s vs peak, implied tokens/s/user)",
        "value": c8["us_per_layer_step"], "unit": "us/layer (one step of 8 sequences)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(c8["us_per_step"] * n_tok / 1e3, 3),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": WORKLOADS[args.workload][2],
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": m.n_layers, "sequences": 8, "tokens_per_launch": n_tok,
                   "start_pos": pos0, "vocab": m.vocab, "hidden": L.hidden},
        "tokens_per_s_total": c8["tokens_per_s_total"], "tokens_per_s_user": c8["tokens_per_s_user"],
        "curve_by_batch": curve,
        "achieved_TBps": round(achieved / 1e3, 3), "frac_of_peak": round(achieved / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_step": int(step_b),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed launches (default 20 for the stack, 100 for a layer)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed launches first (default 3 / 10)")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--single-launch", action="store_true",
                    help="also time decode_step (one layer per launch, launch cost included)")
    ap.add_argument("--trace", default=None, help="write a per-stage device-trace summary (JSON) to this path")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None,
                    help="tokens per launch (multi-layer workloads; default 256 for the stack, 32 for the batch)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--no-single-launch", action="store_true",
                    help="stack: skip the decode_step (one layer per launch) timing")
    ap.add_argument("--no-idle", action="store_true", help="stack: skip the traced launch that measures wait time")
    args = ap.parse_args()
    stack = args.workload.startswith("mla_stack24")
    if args.steps is None:
        args.steps = (20 if args.workload == "mla_stack24_fp8_greedy256" else 3 if args.workload.endswith("batch8")
                      else 10 if stack else 100)
    if args.warmup is None:
        args.warmup = 3 if stack else 10
    if args.tokens is None:
        args.tokens = 32 if args.workload.endswith("batch8") else 256
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU path is not built.",
              file=sys.stderr)
        sys.exit(2)

    if args.calib_copy:
        import torch
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload == "mla_stack24_fp8_greedy256":
        return run_stack(args)
    if args.workload.startswith("mla_stack24_fp8_verify6"):
        return run_verify(args)
    if args.workload == "mla_stack24_fp8_batch8":
        return run_batch(args)

    import torch
    import persistent_latency_bound_amd as pld
    from oracle import accounting
    from synth import configs, device as sdev

    shape = getattr(configs, WORKLOADS[args.workload][0])
    pos = shape.cache_len
    R = args.layers
    Ws = [sdev.layer_weights(shape, 0, l) for l in range(R)]
    Cs = [sdev.kv_cache(shape, 0, l) for l in range(R)]
    n_in = args.steps + args.warmup
    xs = [sdev.input_hidden(shape, 0, i) for i in range(n_in)]
    out = torch.zeros(shape.hidden, dtype=torch.int16, device="cuda")
    dec = pld.Decoder(shape, Ws, Cs)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        dec.persistent(start_pos=pos, in_hidden=xs[i], out_hidden=out)
    torch.cuda.synchronize()
    st = dec.status()
    if st.code != 0:
        raise SystemExit(f"device status {st.code} at stage {st.stage}")

    # timed region: K launches back to back on the launch stream, one event between launches
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        dec.persistent(start_pos=pos, in_hidden=xs[args.warmup + i], out_hidden=out)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    st = dec.status()
    if st.code != 0:
        raise SystemExit(f"device status {st.code} at stage {st.stage}")
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    ms_per_step = ev[0].elapsed_time(ev[-1]) / args.steps
    us_per_layer = ms_per_step * 1e3 / R
    p50 = per[len(per) // 2] * 1e3 / R
    p90 = per[min(len(per) - 1, int(0.9 * len(per)))] * 1e3 / R

    single_us = None
    if args.single_launch:
        # decode_step: one layer per launch, launch cost included (same kernel symbol, so this
        # is kept out of the default run that the kernel-trace profile averages over)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(5):
            dec.step(0, xs[0], pos, out)
        torch.cuda.synchronize()
        e0.record(stream)
        n1 = 50
        for i in range(n1):
            dec.step(i % R, xs[0], pos, out)
        e1.record(stream)
        torch.cuda.synchronize()
        single_us = e0.elapsed_time(e1) * 1e3 / n1

    if args.trace:
        write_trace_summary(dec, xs[0], out, R, args.trace, pos)

    bytes_layer = accounting.layer_bytes(shape, pos)
    bytes_launch = bytes_layer * R
    achieved = bytes_launch / (ms_per_step * 1e-3) / 1e9
    traffic = traffic_per_launch(args.workload, R)
    line = {
        "metric": "batch-1 decode us/layer (achieved HBM TB/s vs peak, implied tokens/s/user)",
        "value": round(us_per_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": WORKLOADS[args.workload][2],
        "data": "synthetic",
        "config": {"workload": args.workload, "hidden": shape.hidden,
                   "attention": (f"GQA {shape.n_heads}q/{shape.n_kv_heads}kv x {shape.head_dim}" if shape.attn == "gqa" else
                                 f"KDA {shape.n_heads} heads x {shape.head_dim}, decay rank {shape.kda_rank}, "
                                 f"conv {shape.conv_width}, fp32 state" if shape.attn == "kda" else
                                 f"MLA {shape.n_heads} heads, latent {shape.kv_lora}+{shape.rope_dim}, q_lora {shape.q_lora}"
                                 + (f", indexer {shape.index_heads}x{shape.index_dim} top-{shape.index_topk}"
                                    if shape.index_topk else "")),
                   "weights": shape.wfmt + (f", experts {shape.expert_fmt}" if shape.expert_fmt else ""),
                   "kv_cache_tokens": pos,
                   "experts": f"{shape.n_experts} top-{shape.top_k} + {shape.n_shared} shared ({shape.router})",
                   "expert_inter": shape.inter, "layers_per_launch": R, "tokens_per_step": 1, "batch": 1},
        "achieved_TBps": round(achieved / 1e3, 3),
        "frac_of_peak": round(achieved / PEAK_HBM_GBPS, 4),
        "implied_tokens_per_s_user_24_layers": round(1e6 / (us_per_layer * 24), 1),
        "p50_us_per_layer": round(p50, 3),
        "p90_us_per_layer": round(p90, 3),
        "single_launch_us_per_layer": None if single_us is None else round(single_us, 3),
        "launches_per_layer": round(1.0 / R, 4),
        "launches_per_token_24_layers": round(24.0 / R, 2),
        "algorithmic_bytes_per_layer": bytes_layer,
        "wall_s_timed_region": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic / (ms_per_step * 1e-3) / 1e9, 1)},
        "hbm_bytes_per_launch_counters": traffic,
        "algorithmic_bytes_per_launch": bytes_launch,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(shape, pos)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
