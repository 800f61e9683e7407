"""GPU parity of the sparse MLA MoE decode layer (indexer top-k attention) against the CPU oracle.

Workload: hidden 4096, 32 heads, q_lora 1536, kv_lora 512 + rope 64 (nope 128, v 128),
bf16 weights, indexer of 8 heads x 64 dims with FP8 keys (E4M3 codes + fp32 scale per
token), top-2048 selection, 64 routed experts top-8 (softmax router) + one shared expert,
expert width 1536.

Bars:
* the indexer decision path is bit-exact: q_I (bf16), w and k_I (fp32), the appended FP8
  key row and its scale, every token's fp64 score, and the selected rows;
* the hidden state within TOL (max-norm relative); router top-k identical.

Cases: a real selection among 301 tokens (top-64), T <= top-k (every token), the full
32768-token cache with top-2048, a tie-heavy cache (250 identical all-zero keys, cut by
token index), and a cluster of 200 nearly equal keys (equal high halves, different low
halves) straddling the cut.
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


def _scores_from_keys(dec, T):
    hi = dec.debug("ikh").cpu().numpy().view(np.uint32)[:T].astype(np.uint64)
    lo = dec.debug("ikl").cpu().numpy().view(np.uint32)[:T].astype(np.uint64)
    key = (hi << np.uint64(32)) | lo
    top = np.uint64(1) << np.uint64(63)
    bits = np.where(key & top, key & ~top, ~key)
    return bits.view(np.float64)


def _bf16_bits(x):
    return nx.bf16_bits_of(np.asarray(x, np.float64))


def _check_indexer(dec, s, rec, pos, cache_dev, tag):
    T = pos + 1
    # indexer inputs: q_I (bf16), w and k_I (fp32) -- bit-exact
    qi = dec.debug("qi").cpu().numpy().view(np.uint16)[: s.index_heads * s.index_dim]
    assert np.array_equal(qi, _bf16_bits(rec["q_i"]).reshape(-1)), \
        f"{tag}: q_I differs in {np.count_nonzero(qi != _bf16_bits(rec['q_i']).reshape(-1))} entries"
    ixr = dec.debug("ixr").cpu().numpy().astype(np.float64)
    assert np.array_equal(ixr[: s.index_heads], rec["w_idx"]), f"{tag}: indexer head weights"
    assert np.array_equal(ixr[s.index_heads: s.index_heads + s.index_dim], rec["k_i"]), f"{tag}: indexer key"
    # the appended FP8 key row and scale
    codes = cache_dev["index_codes"][pos].cpu().numpy()
    assert np.array_equal(codes, rec["index_code_new"]), f"{tag}: appended key codes"
    assert cache_dev["index_scales"][pos].item() == float(rec["index_scale_new"]), f"{tag}: appended key scale"
    # every score, then the selection
    k = min(s.index_topk, T)
    sel = dec.debug("isel").cpu().numpy()[:k]
    sc = _scores_from_keys(dec, T)
    bad = np.flatnonzero(sc != rec["index_score"])
    assert bad.size == 0, f"{tag}: {bad.size} scores differ, first at token {bad[0]}"
    assert np.array_equal(sel, rec["index_sel"]), \
        f"{tag}: selection differs in {np.count_nonzero(sel != rec['index_sel'])} of {k} entries"
    say(f"{tag}: indexer exact (q_I, w, k_I, key row, {T} scores, {k} selected)")


def _check_layer(dec, s, rec, out, pos, cache_dev, tag, x_bits):
    _check_indexer(dec, s, rec, pos, cache_dev, tag)
    err = rel_err(bf16_tensor_to_f64(out), rec["out"])
    o = dec.debug("o").cpu().numpy().reshape(s.n_heads, s.v_dim)
    e_o = rel_err(o, rec["o"])
    say(f"{tag}: out rel err {err:.3e}, attention output {e_o:.2e}")
    assert e_o < 1e-2, f"{tag}: attention output rel err {e_o}"
    assert err < TOL, f"{tag}: out rel err {err}"
    got = nx.bf16_to_f64(cache_dev["latent"][pos].cpu().numpy().view(np.uint16))
    ref = rec["latent_new"]
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-30), f"{tag}: latent row"
    sel = dec.debug("sel").cpu().numpy()
    assert list(sel) == list(rec["router_sel"]), f"{tag}: router selection {sel} vs {rec['router_sel']}"
    check_branches(dec, s, rec, x_bits, tag)


@pytest.mark.parametrize("cache_len,topk,positions", [(300, 64, [300, 301]), (37, 2048, [0, 37])])
def test_sparse_mla_layer_small_cache(cache_len, topk, positions):
    _need_gpu()
    s = configs.scaled(configs.C4, cache_len=cache_len, max_seq=cache_len + 64, index_topk=topk)
    say(f"case: sparse MLA layer, cache {cache_len}, top-{topk}, positions {positions}")
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    hc = host_cache(s)
    W = gen.LayerWeights(s, 0, 0)
    from synth import device as sdev
    for i, pos in enumerate(positions):
        x = sdev.input_hidden(s, 0, i)
        out = _run_step(dec, s, 0, x, pos)
        xb = gen.input_hidden(s, 0, i)
        rec = oracle_step(s, 0, 0, hc, xb, pos, weights=W)
        _check_layer(dec, s, rec, out, pos, Cs[0], f"sparse cache {cache_len} top-{topk} pos {pos}", xb)


def test_sparse_mla_layer_full_cache():
    _need_gpu()
    s = configs.C4
    say("case: sparse MLA layer, 32768-token cache, top-2048, pos 32768")
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    out = _run_step(dec, s, 0, x, s.cache_len)
    xb = gen.input_hidden(s, 0, 0)
    rec = oracle_step(s, 0, 0, host_cache(s), xb, s.cache_len)
    _check_layer(dec, s, rec, out, s.cache_len, Cs[0], "sparse pos 32768", xb)


def test_sparse_selection_ties_cut_by_index():
    """250 all-zero keys score exactly 0 and tie; fewer than 64 tokens score above 0, so the
    cut falls inside the tie and is decided by token index."""
    _need_gpu()
    s = configs.scaled(configs.C4, cache_len=300, max_seq=364, index_topk=64)
    say("case: sparse selection, 250 tied zero keys, top-64 of 301")
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    hc = host_cache(s)
    hc["index_codes"][:250] = 0
    Cs[0]["index_codes"][:250] = 0
    torch.cuda.synchronize()
    from synth import device as sdev
    out = _run_step(dec, s, 0, sdev.input_hidden(s, 0, 0), 300)
    rec = oracle_step(s, 0, 0, hc, gen.input_hidden(s, 0, 0), 300)
    npos = int(np.count_nonzero(rec["index_score"] > 0))
    say(f"  {npos} tokens score above 0; the rest of the 64 come from the tie")
    assert npos < 64 and np.count_nonzero(rec["index_score"] == 0) >= 250
    _check_layer(dec, s, rec, out, 300, Cs[0], "ties", gen.input_hidden(s, 0, 0))


def test_sparse_selection_near_equal_cluster():
    """200 tokens share the key codes of the best-scoring token with scales one fp32 step
    apart: their scores agree in the high 32 key bits in runs and differ below, and the
    top-64 cut falls inside the cluster."""
    _need_gpu()
    s = configs.scaled(configs.C4, cache_len=300, max_seq=364, index_topk=64)
    say("case: sparse selection, 200 nearly equal keys around the cut, top-64 of 301")
    probe = oracle_step(s, 0, 0, host_cache(s), gen.input_hidden(s, 0, 0), 300)
    best = int(np.argmax(probe["index_score"][:300]))
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    hc = host_cache(s)
    s0 = np.float32(hc["index_scales"][best])
    sc = np.empty(200, np.float32)
    sc[0] = s0
    for i in range(1, 200):
        sc[i] = np.nextafter(sc[i - 1], np.float32(np.inf))
    hc["index_codes"][:200] = hc["index_codes"][best]
    hc["index_scales"][:200] = sc
    Cs[0]["index_codes"][:200] = torch.from_numpy(np.repeat(hc["index_codes"][best][None], 200, 0)).cuda()
    Cs[0]["index_scales"][:200] = torch.from_numpy(sc).cuda()
    torch.cuda.synchronize()
    from synth import device as sdev
    out = _run_step(dec, s, 0, sdev.input_hidden(s, 0, 0), 300)
    rec = oracle_step(s, 0, 0, hc, gen.input_hidden(s, 0, 0), 300)
    cl = rec["index_score"][:200]
    hi = (cl.view(np.uint64) >> np.uint64(32))
    say(f"  cluster: {np.unique(cl).size} distinct scores, {np.unique(hi).size} distinct high halves; "
        f"{np.count_nonzero(rec['index_sel'] < 200)} of 64 chosen from it")
    _check_layer(dec, s, rec, out, 300, Cs[0], "cluster", gen.input_hidden(s, 0, 0))


def test_sparse_two_layer_stack_one_launch():
    """Two sparse layers in one persistent launch. The launch equals two chained one-layer
    launches bit for bit (output and layer 1's selection). Layer 1's selection is an integer
    that floating point decides, so it is checked exactly against the oracle run on the GPU's
    own layer-1 input (the layer-0 output of the chained launch); each layer's output is
    within TOL of the oracle on the same input."""
    _need_gpu()
    s = configs.scaled(configs.C4, cache_len=500, max_seq=564, index_topk=128)
    say("case: sparse MLA 2-layer stack, one persistent launch, top-128 of 501")
    from synth import device as sdev
    x = sdev.input_hidden(s, 0, 0)
    decA, _, _ = _decoder(s, [(0, 0), (0, 1)])
    outA = torch.zeros(s.hidden, dtype=torch.int16, device="cuda")
    decA.persistent(start_pos=500, in_hidden=x, out_hidden=outA)
    torch.cuda.synchronize()
    assert decA.status().code == 0
    selA = decA.debug("isel").cpu().numpy()[:128].copy()
    # chained one-layer launches on fresh caches
    decB, _, _ = _decoder(s, [(0, 0), (0, 1)])
    x0 = _run_step(decB, s, 0, x, 500)
    outB = _run_step(decB, s, 1, x0, 500)
    selB = decB.debug("isel").cpu().numpy()[:128].copy()
    assert np.array_equal(outA.cpu().numpy(), outB.cpu().numpy()), "one launch vs chained launches: output"
    assert np.array_equal(selA, selB), "one launch vs chained launches: layer 1 selection"
    # the oracle, layer by layer, on the GPU's inputs
    rec0 = oracle_step(s, 0, 0, host_cache(s, 0, 0), gen.input_hidden(s, 0, 0), 500)
    e0 = rel_err(bf16_tensor_to_f64(x0), rec0["out"])
    x0_bits = x0.cpu().numpy().view(np.uint16)
    rec1 = oracle_step(s, 0, 1, host_cache(s, 0, 1), x0_bits, 500)
    e1 = rel_err(bf16_tensor_to_f64(outB), rec1["out"])
    say(f"2-layer sparse stack: layer 0 rel err {e0:.3e}, layer 1 rel err {e1:.3e} (on the GPU's layer-1 input)")
    assert e0 < TOL and e1 < TOL
    assert np.array_equal(selB, rec1["index_sel"]), "layer 1 selection on the GPU's own input"


def _full_cache_case(tag, edit):
    """The full 32768-token cache with the host and device index keys edited the same way."""
    s = configs.C4
    dec, Ws, Cs = _decoder(s, [(0, 0)])
    hc = host_cache(s)
    edit(hc)
    Cs[0]["index_codes"].copy_(torch.from_numpy(hc["index_codes"]).cuda())
    Cs[0]["index_scales"].copy_(torch.from_numpy(hc["index_scales"]).cuda())
    torch.cuda.synchronize()
    from synth import device as sdev
    out = _run_step(dec, s, 0, sdev.input_hidden(s, 0, 0), s.cache_len)
    rec = oracle_step(s, 0, 0, hc, gen.input_hidden(s, 0, 0), s.cache_len)
    _check_layer(dec, s, rec, out, s.cache_len, Cs[0], tag, gen.input_hidden(s, 0, 0))
    return rec


def test_sparse_selection_weak_bound_all_tokens():
    """Tokens t with t % 256 < 128 get scales 2^-20 smaller: half of the scoring workgroups
    hold only tiny keys, the published bound admits more than 8192 keys, and the selection
    runs over every token (distinct keys)."""
    _need_gpu()
    say("case: sparse selection, weak bound (half the scales x 2^-20), top-2048 of 32769")

    def edit(hc):
        t = np.arange(configs.C4.cache_len)
        hc["index_scales"][: configs.C4.cache_len] = np.where(
            t % 256 < 128, hc["index_scales"][: configs.C4.cache_len] * np.float32(2.0 ** -20),
            hc["index_scales"][: configs.C4.cache_len]).astype(np.float32)

    rec = _full_cache_case("weak bound", edit)
    sc = rec["index_score"]
    say(f"  {np.count_nonzero(sc > 0)} positive scores, {np.unique(sc).size} distinct")


def test_sparse_selection_massive_tie_all_tokens():
    """Only every 16th token keeps its key codes; the other ~30700 score exactly 0, so the
    top-2048 cut falls inside a tie far larger than any candidate list and is decided by
    token index over every token."""
    _need_gpu()
    say("case: sparse selection, ~30700 tied zero keys, top-2048 of 32769")

    def edit(hc):
        n = configs.C4.cache_len
        keep = np.arange(n) % 16 == 0
        hc["index_codes"][:n][~keep] = 0

    rec = _full_cache_case("massive tie", edit)
    sc = rec["index_score"]
    say(f"  {np.count_nonzero(sc > 0)} tokens score above 0, {np.count_nonzero(sc == 0)} score 0")
    assert np.count_nonzero(sc > 0) < 2048 <= np.count_nonzero(sc >= 0)
