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
