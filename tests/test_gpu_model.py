"""GPU parity of the multi-layer greedy decode loop with the LM head.

A stack of FP8 MLA MoE layers (the c5 layer shape) with an FP8 LM head over a vocabulary of
32768 runs in ONE persistent launch per call: per token, every layer, then RMSNorm + head
GEMV (fp64 accumulation) + argmax (lowest token id on ties) + the embedding row of the
chosen token as the next token's input.

Checks:
* head stage, exact: the oracle's fp64 head on the GPU's own final hidden state picks the
  same token, and the logits agree to fp64 rounding (the decision is taken in fp64 on
  both sides);
* the loop: one launch of n tokens gives bit-identical tokens, logits and hidden state to
  n chained one-token launches;
* end to end with teacher forcing: the oracle, fed the same input tokens, gives logits
  within TOL; where its argmax differs, the two logits it compares are within TOL.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_common import TOL, host_cache, rel_err, say  # noqa: E402
from oracle import layer as OL  # noqa: E402
from oracle import model as OM  # noqa: E402
from synth import configs, gen  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _model(n_layers, cache_len, n_tokens):
    L = configs.scaled(configs.C5_LAYER, cache_len=cache_len, max_seq=cache_len + 64)
    return configs.ModelShape(layer=L, n_layers=n_layers, vocab=32768, n_tokens=n_tokens)


def _decoder(m):
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    Ws = [sdev.layer_weights(m.layer, 0, l) for l in range(m.n_layers)]
    Cs = [sdev.kv_cache(m.layer, 0, l) for l in range(m.n_layers)]
    head = {"embed": sdev.embedding(m), "final_norm": sdev.final_norm(m), "head": sdev.head(m)}
    return pld.Decoder(m.layer, Ws, Cs, head=head, vocab=m.vocab)


def _launch(dec, m, pos, tok, n):
    H, V = m.layer.hidden, m.vocab
    out = torch.zeros(H, dtype=torch.int16, device="cuda")
    lg = torch.zeros((n, V), dtype=torch.float32, device="cuda")
    tk = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    dec.persistent(start_pos=pos, in_token=tok, n_tokens=n, out_hidden=out, out_logits=lg, out_tokens=tk)
    torch.cuda.synchronize()
    st = dec.status()
    assert st.code == 0, f"device status {st.code} wait {st.stage} layer {st.layer} token {st.token} wg {st.wg}"
    return out.cpu().numpy().view(np.uint16), lg.cpu().numpy(), [int(v) for v in tk.cpu().numpy()]


def test_greedy_loop_with_head():
    _need_gpu()
    m = _model(n_layers=2, cache_len=100, n_tokens=3)
    pos, n = 100, 3
    tok0 = gen.first_token(m)
    say(f"case: 2-layer FP8 MLA stack + head (vocab {m.vocab}), pos {pos}, {n} tokens from token {tok0}")
    # chained one-token launches: every token's final hidden state is visible
    decA = _decoder(m)
    toks, logits, xs = [], [], []
    tin = tok0
    for t in range(n):
        x, lg, tk = _launch(decA, m, pos + t, tin, 1)
        toks.append(tk[0])
        logits.append(lg[0])
        xs.append(x)
        tin = tk[0]
    say(f"tokens (chained launches): {toks}")
    # one launch of n tokens on fresh caches: identical bits
    decB = _decoder(m)
    xB, lgB, tkB = _launch(decB, m, pos, tok0, n)
    assert tkB == toks, f"one launch {tkB} vs chained {toks}"
    assert np.array_equal(lgB, np.stack(logits)), "logits differ between one launch and chained launches"
    assert np.array_equal(xB, xs[-1]), "final hidden state differs"
    # head stage: oracle fp64 head on the GPU's own hidden state decides the same token
    head_m = gen.head_matrix(m)
    fg = gen.final_norm(m)
    for t in range(n):
        lo = OM.head_logits(m.layer, head_m, fg, xs[t])
        e = rel_err(logits[t], lo)
        say(f"token {t}: head logits rel err {e:.2e} (GPU fp64 -> fp32 output)")
        assert e < 1e-6, t
        assert OM.argmax_lowest(lo) == toks[t], f"token {t}: oracle argmax {OM.argmax_lowest(lo)} vs GPU {toks[t]}"
    # end to end, teacher forced with the GPU's tokens
    Wl = [gen.LayerWeights(m.layer, 0, l) for l in range(m.n_layers)]
    caches = [host_cache(m.layer, 0, l) for l in range(m.n_layers)]
    tin = tok0
    for t in range(n):
        x = gen.embedding_rows(m, [tin])[0]
        for l in range(m.n_layers):
            rec = OL.decode_layer(m.layer, Wl[l], caches[l], x, pos + t)
            OL.append_to_cache(m.layer, caches[l], rec, pos + t)
            x = rec["out_bits"]
        lo = OM.head_logits(m.layer, head_m, fg, x)
        e = rel_err(logits[t], lo)
        to = OM.argmax_lowest(lo)
        say(f"token {t}: end-to-end logits rel err {e:.2e}; oracle token {to}, GPU token {toks[t]}")
        assert e < TOL, t
        if to != toks[t]:
            assert abs(lo[to] - lo[toks[t]]) <= TOL * np.max(np.abs(lo)), f"token {t}: decisive difference"
        tin = toks[t]


def _verify(dec, m, pos, tok, drafts):
    V = m.vocab
    n = len(drafts) + 1
    out = torch.zeros(m.layer.hidden, dtype=torch.int16, device="cuda")
    lg = torch.zeros((n, V), dtype=torch.float32, device="cuda")
    tk = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    acc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    dr = torch.tensor(list(drafts), dtype=torch.int32, device="cuda")
    dec.persistent(start_pos=pos, in_token=tok, n_query=n, draft_tokens=dr, out_hidden=out, out_logits=lg,
                   out_tokens=tk, out_accepted=acc)
    torch.cuda.synchronize()
    st = dec.status()
    assert st.code == 0, f"device status {st.code} wait {st.stage} layer {st.layer} token {st.token} wg {st.wg}"
    return lg.cpu().numpy(), [int(v) for v in tk.cpu().numpy()], int(acc.item())


def test_verify_six_positions():
    """Six-position verify in one launch: position j > 0 is fed draft j-1, every position's
    logits and argmax come out, and greedy acceptance counts the leading drafts equal to
    the argmax before them. Drafts that follow the greedy continuation give the greedy
    run's logits bit for bit; a wrong draft stops the acceptance; the oracle's verify
    step agrees within TOL (same tokens unless two logits are within TOL)."""
    _need_gpu()
    m = _model(n_layers=2, cache_len=100, n_tokens=6)
    pos, n = 100, 6
    tok0 = gen.first_token(m)
    say(f"case: 2-layer FP8 MLA stack + head, verify {n} positions at pos {pos} from token {tok0}")
    decG = _decoder(m)
    _, lgG, tkG = _launch(decG, m, pos, tok0, n)   # greedy reference: 6 tokens, one launch
    say(f"greedy tokens: {tkG}")
    # all drafts follow the greedy continuation: everything accepted, logits identical
    decA = _decoder(m)
    lgA, tkA, accA = _verify(decA, m, pos, tok0, tkG[:5])
    say(f"verify (greedy drafts): tokens {tkA}, accepted {accA}")
    assert accA == 5 and tkA == tkG
    assert np.array_equal(lgA, lgG), "verify logits differ from the greedy launch"
    # a wrong draft at position 4: three accepted, positions 0..3 as in the greedy run
    wrong = (tkG[3] + 1) % m.vocab
    drafts = [tkG[0], tkG[1], tkG[2], wrong, tkG[4]]
    decB = _decoder(m)
    lgB, tkB, accB = _verify(decB, m, pos, tok0, drafts)
    say(f"verify (wrong draft 4): tokens {tkB}, accepted {accB}")
    assert accB == 3, accB
    assert np.array_equal(lgB[:4], lgG[:4]) and tkB[:4] == tkG[:4]
    # the oracle's verify step on the same drafts
    Wl = [gen.LayerWeights(m.layer, 0, l) for l in range(m.n_layers)]
    caches = [host_cache(m.layer, 0, l) for l in range(m.n_layers)]
    ref = OM.verify_step(m.layer, Wl, caches, lambda t: gen.embedding_rows(m, [t])[0], gen.head_matrix(m),
                         gen.final_norm(m), tok0, drafts, pos)
    say(f"oracle verify: tokens {ref['tokens']}, accepted {ref['accepted']}")
    assert ref["accepted"] == accB
    for j in range(n):
        e = rel_err(lgB[j], ref["logits"][j])
        say(f"position {j}: logits rel err {e:.2e}")
        assert e < TOL, j
        if ref["tokens"][j] != tkB[j]:
            lo = ref["logits"][j]
            assert abs(lo[ref["tokens"][j]] - lo[tkB[j]]) <= TOL * np.max(np.abs(lo)), f"position {j}: decisive"


def test_stack_at_full_cache_greedy_then_verify():
    """The stack at the 24-layer workload's own positions: 2 layers of the FP8 MLA shape over
    an 8192-token cache. One launch decodes 4 greedy tokens at positions 8192-8195, so the
    last chunks mix static history rows with rows written inside the launch, and from 8193
    on one chunk holds a fifth sub-block. Then one 6-position verify from 8192 on the same
    caches with drafts [g0, g1, g2, wrong, g3]. The oracle is teacher-forced with the GPU's
    tokens; its verify positions 0-3 are exactly the greedy run's steps (same inputs at the
    same positions), so only positions 4 and 5 are computed on."""
    _need_gpu()
    m = _model(n_layers=2, cache_len=8192, n_tokens=4)
    pos, n = 8192, 4
    tok0 = gen.first_token(m)
    say(f"case: 2-layer FP8 MLA stack + head, 8192-token cache, {n} tokens in one launch from token {tok0}")
    dec = _decoder(m)
    _, lg, toks = _launch(dec, m, pos, tok0, n)
    say(f"GPU greedy tokens: {toks}")
    head_m = gen.head_matrix(m)
    fg = gen.final_norm(m)
    Wl = [gen.LayerWeights(m.layer, 0, l) for l in range(m.n_layers)]
    caches = [host_cache(m.layer, 0, l) for l in range(m.n_layers)]
    ref_logits, ref_toks = [], []

    def oracle_position(tin, p):
        x = gen.embedding_rows(m, [tin])[0]
        for l in range(m.n_layers):
            rec = OL.decode_layer(m.layer, Wl[l], caches[l], x, p)
            OL.append_to_cache(m.layer, caches[l], rec, p)
            x = rec["out_bits"]
        lo = OM.head_logits(m.layer, head_m, fg, x)
        ref_logits.append(lo)
        ref_toks.append(OM.argmax_lowest(lo))
        return lo

    def compare(got, lo, gtok, tag):
        e = rel_err(got, lo)
        to = OM.argmax_lowest(lo)
        say(f"{tag}: logits rel err {e:.2e}; oracle token {to}, GPU token {gtok}")
        assert e < TOL, tag
        if to != gtok:
            assert abs(lo[to] - lo[gtok]) <= TOL * np.max(np.abs(lo)), f"{tag}: decisive difference"

    tin = tok0
    for t in range(n):
        lo = oracle_position(tin, pos + t)
        compare(lg[t], lo, toks[t], f"greedy token {t} (pos {pos + t})")
        tin = toks[t]
    # verify from 8192 on the same caches (its rows 8192.. are rewritten in order)
    wrong = (toks[3] + 1) % m.vocab
    drafts = [toks[0], toks[1], toks[2], wrong, toks[3]]
    lgV, tkV, accV = _verify(dec, m, pos, tok0, drafts)
    say(f"GPU verify: tokens {tkV}, accepted {accV}")
    oracle_position(wrong, pos + 4)
    oracle_position(toks[3], pos + 5)
    inputs = [tok0] + drafts
    acc_ref = 0
    for j in range(1, 6):
        if inputs[j] != ref_toks[j - 1]:
            break
        acc_ref += 1
    for j in range(6):
        compare(lgV[j], ref_logits[j], tkV[j], f"verify position {j} (pos {pos + j})")
    # the verify's first four positions repeat the greedy launch's steps
    assert np.array_equal(lgV[:4], lg[:4]) and tkV[:4] == toks[:4], "verify positions 0-3 vs the greedy launch"
    say(f"oracle accepted {acc_ref}")
    assert accV == acc_ref == 3


def _launch_sampled(dec, m, pos, tok, n, temperature, seed):
    H, V = m.layer.hidden, m.vocab
    out = torch.zeros(H, dtype=torch.int16, device="cuda")
    lg = torch.zeros((n, V), dtype=torch.float32, device="cuda")
    tk = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    dec.persistent(start_pos=pos, in_token=tok, n_tokens=n, out_hidden=out, out_logits=lg, out_tokens=tk,
                   temperature=temperature, sample_seed=seed)
    torch.cuda.synchronize()
    st = dec.status()
    assert st.code == 0, f"device status {st.code} wait {st.stage} layer {st.layer} token {st.token} wg {st.wg}"
    return out.cpu().numpy().view(np.uint16), lg.cpu().numpy(), [int(v) for v in tk.cpu().numpy()]


def test_sampled_decode_matches_oracle_sampler():
    """Temperature sampling on the device (Gumbel-max over fp64 logits with the counter-based
    noise). Stage-wise exact: on the GPU's own final hidden state of every token (chained
    one-token launches), the oracle's fp64 head and sampler pick the GPU's token. One launch
    of n tokens equals the chained launches bit for bit. End to end (teacher forced): logits
    within TOL."""
    _need_gpu()
    m = _model(n_layers=2, cache_len=100, n_tokens=4)
    pos, n, T, seed = 100, 4, 0.8, 5
    tok0 = gen.first_token(m)
    say(f"case: sampled decode T={T} seed {seed}, 2-layer stack + head, pos {pos}, {n} tokens")
    decA = _decoder(m)
    toks, logits, xs = [], [], []
    tin = tok0
    for t in range(n):
        x, lg, tk = _launch_sampled(decA, m, pos + t, tin, 1, T, seed)
        toks.append(tk[0])
        logits.append(lg[0])
        xs.append(x)
        tin = tk[0]
    decB = _decoder(m)
    xB, lgB, tkB = _launch_sampled(decB, m, pos, tok0, n, T, seed)
    say(f"sampled tokens {toks}; one launch {tkB}")
    assert tkB == toks and np.array_equal(lgB, np.stack(logits)) and np.array_equal(xB, xs[-1])
    head_m = gen.head_matrix(m)
    fg = gen.final_norm(m)
    greedy_differs = 0
    for t in range(n):
        lo = OM.head_logits(m.layer, head_m, fg, xs[t])
        assert OM.sample_token(lo, T, seed, pos + t) == toks[t], f"token {t}: oracle sampler disagrees"
        greedy_differs += OM.argmax_lowest(lo) != toks[t]
    say(f"stage-wise: the oracle's sampler picks every GPU token ({greedy_differs} of {n} differ from the argmax)")
    Wl = [gen.LayerWeights(m.layer, 0, l) for l in range(m.n_layers)]
    caches = [host_cache(m.layer, 0, l) for l in range(m.n_layers)]
    tin = tok0
    for t in range(n):
        x = gen.embedding_rows(m, [tin])[0]
        for l in range(m.n_layers):
            rec = OL.decode_layer(m.layer, Wl[l], caches[l], x, pos + t)
            OL.append_to_cache(m.layer, caches[l], rec, pos + t)
            x = rec["out_bits"]
        lo = OM.head_logits(m.layer, head_m, fg, x)
        e = rel_err(logits[t], lo)
        say(f"token {t}: end-to-end logits rel err {e:.2e}")
        assert e < TOL
        tin = toks[t]


@pytest.mark.parametrize("T", [0.0, 0.8])
def test_speculative_loop_reproduces_plain_decoding(T):
    """decode_speculative gives exactly the tokens of plain decoding of the target with the
    same temperature and seed: once with a 1-layer drafter (the target's first layer with its
    own cache: few drafts kept) and once with a drafter identical to the target (every draft
    kept, so the loop takes its catch-up step)."""
    _need_gpu()
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    m = _model(n_layers=2, cache_len=100, n_tokens=12)
    L = m.layer
    pos, n, seed = 100, 12, 9
    tok0 = gen.first_token(m)
    Ws = [sdev.layer_weights(L, 0, l) for l in range(2)]
    head = {"embed": sdev.embedding(m), "final_norm": sdev.final_norm(m), "head": sdev.head(m)}

    def handle(layers):
        return pld.Decoder(L, [Ws[l] for l in layers], [sdev.kv_cache(L, 0, l) for l in layers], head=head,
                           vocab=m.vocab)

    plain = handle([0, 1])
    out = torch.zeros(L.hidden, dtype=torch.int16, device="cuda")
    tk = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    plain.persistent(start_pos=pos, in_token=tok0, n_tokens=n, out_hidden=out, out_tokens=tk, temperature=T,
                     sample_seed=seed)
    torch.cuda.synchronize()
    ref = [int(v) for v in tk.cpu().numpy()]
    say(f"case: speculative loop T={T}, plain tokens {ref}")
    for tag, dlayers in (("1-layer drafter", [0]), ("drafter = target", [0, 1])):
        target, draft = handle([0, 1]), handle(dlayers)
        got = torch.full((n,), -1, dtype=torch.int32, device="cuda")
        verifies, kept = target.speculative(draft, pos, tok0, n, 5, got, temperature=T, sample_seed=seed)
        torch.cuda.synchronize()
        assert target.status().code == 0 and draft.status().code == 0
        gl = [int(v) for v in got.cpu().numpy()]
        say(f"  {tag}: {verifies} verify launches, {kept} drafts kept; tokens {gl}")
        assert gl == ref, f"{tag}: speculative tokens differ from plain decoding"
        if dlayers == [0, 1]:
            # 12 tokens, 5 drafts per round, all kept: two rounds of 6 tokens
            assert (verifies, kept) == (2, 10)
