"""GPU parity of the batched multi-token verify (decode_verify_batched) against the CPU oracle.

The batched verify runs the n_query positions of one verify through every layer together:
the dense projections, the shared expert and the union of the routed experts run as skinny
GEMMs on the matrix cores with bf16 activation operands, attention reads the shared history
once per pair of positions, and each position sees the new rows up to its own.

Reference: the oracle's decode step per position in order (positions pos, pos + 1, ...,
each appending its cache rows before the next), fed the same input tokens, then its fp64
head; acceptance = the leading drafts equal to the token chosen at the position before.

Bars (relative to each vector's own max-norm):
* TOL (2e-2) on logits;
* BAR_VB (1e-2) on the attention branch y = h2 - x and the FFN output f of every position
  (one-layer stack, where the layer input is the exact embedding row on both sides). Each
  GEMM rounds its normalised input to bf16 once (relative error up to 2^-9, rms about
  1.1e-3 per element); a dot product of random-signed terms carries about that relative
  error, and a branch passes through at most six such roundings (the attention chain c_q,
  q, q_lat and P, o_lat, o; the FFN chain b, m), so its error stays near 3e-3; 1e-2 leaves
  a factor of about three.
* the expert choice of every position identical to the oracle's (the router stays fp64 from
  the fp32 activation), and the chosen tokens identical unless the two logits are within TOL.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_common import TOL, host_cache, rel_err, say  # noqa: E402
from oracle import layer as OL  # noqa: E402
from oracle import model as OM  # noqa: E402
from oracle import numerics as nx  # noqa: E402
from synth import configs, gen  # noqa: E402

pytestmark = pytest.mark.gpu

BAR_VB = 1e-2


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _model(n_layers, cache_len):
    L = configs.scaled(configs.C5_LAYER, cache_len=cache_len, max_seq=cache_len + 64)
    return configs.ModelShape(layer=L, n_layers=n_layers, vocab=32768, n_tokens=8)


def _decoder(m, max_query=8):
    import persistent_latency_bound_amd as pld
    from synth import device as sdev
    Ws = [sdev.layer_weights(m.layer, 0, l) for l in range(m.n_layers)]
    Cs = [sdev.kv_cache(m.layer, 0, l) for l in range(m.n_layers)]
    head = {"embed": sdev.embedding(m), "final_norm": sdev.final_norm(m), "head": sdev.head(m)}
    return pld.Decoder(m.layer, Ws, Cs, head=head, vocab=m.vocab, max_query=max_query)


def _status_ok(dec, tag):
    st = dec.status()
    assert st.code == 0, f"{tag}: device status {st.code} wait {st.stage} layer {st.layer} token {st.token} wg {st.wg}"


def _batched(dec, m, pos, tok, drafts, temperature=0.0, seed=0):
    n = len(drafts) + 1
    out = torch.zeros(m.layer.hidden, dtype=torch.int16, device="cuda")
    lg = torch.zeros((n, m.vocab), dtype=torch.float32, device="cuda")
    tk = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    acc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    dr = torch.tensor(list(drafts), dtype=torch.int32, device="cuda")
    dec.verify_batched(pos, tok, dr, out, out_logits=lg, out_tokens=tk, out_accepted=acc, temperature=temperature,
                       sample_seed=seed)
    torch.cuda.synchronize()
    _status_ok(dec, "batched verify")
    return lg.cpu().numpy(), [int(v) for v in tk.cpu().numpy()], int(acc.item()), out.cpu().numpy().view(np.uint16)


def _sequential(dec, m, pos, tok, drafts, temperature=0.0, seed=0):
    n = len(drafts) + 1
    out = torch.zeros(m.layer.hidden, dtype=torch.int16, device="cuda")
    lg = torch.zeros((n, m.vocab), dtype=torch.float32, device="cuda")
    tk = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    acc = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    dr = torch.tensor(list(drafts), dtype=torch.int32, device="cuda")
    dec.persistent(start_pos=pos, in_token=tok, n_query=n, draft_tokens=dr, out_hidden=out, out_logits=lg,
                   out_tokens=tk, out_accepted=acc, temperature=temperature, sample_seed=seed)
    torch.cuda.synchronize()
    _status_ok(dec, "sequential verify")
    return lg.cpu().numpy(), [int(v) for v in tk.cpu().numpy()], int(acc.item())


class _Oracle:
    """Teacher-forced oracle over the positions of one verify (caches advance in order)."""

    def __init__(self, m):
        self.m = m
        self.W = [gen.LayerWeights(m.layer, 0, l) for l in range(m.n_layers)]
        self.caches = [host_cache(m.layer, 0, l) for l in range(m.n_layers)]
        self.head = gen.head_matrix(m)
        self.fg = gen.final_norm(m)

    def position(self, tin, p, temperature=0.0, seed=0):
        x = gen.embedding_rows(self.m, [tin])[0]
        recs = []
        for l in range(self.m.n_layers):
            rec = OL.decode_layer(self.m.layer, self.W[l], self.caches[l], x, p)
            OL.append_to_cache(self.m.layer, self.caches[l], rec, p)
            rec["x_in"] = x
            recs.append(rec)
            x = rec["out_bits"]
        lo = OM.head_logits(self.m.layer, self.head, self.fg, x)
        return lo, OM.sample_token(lo, temperature, seed, p), recs


def _accepted(inputs, toks):
    a = 0
    for j in range(1, len(inputs)):
        if inputs[j] != toks[j - 1]:
            break
        a += 1
    return a


def _compare_logits(got, lo, gtok, otok, tag):
    e = rel_err(got, lo)
    say(f"{tag}: logits rel err {e:.2e}; oracle token {otok}, GPU token {gtok}")
    assert e < TOL, tag
    if otok != gtok:
        assert abs(lo[otok] - lo[gtok]) <= TOL * np.max(np.abs(lo)), f"{tag}: decisive difference"


def test_batched_verify_one_layer_branches_vs_oracle():
    """One layer, a 300-row history (64 chunks of 4-5 rows), 8 positions (the maximum): per
    position y, f, the expert choice, logits and tokens against the oracle; drafts follow the
    oracle's own greedy tokens for the first four positions, then one wrong draft."""
    _need_gpu()
    m = _model(n_layers=1, cache_len=300)
    pos, n = 300, 8
    tok0 = gen.first_token(m)
    say(f"case: 1-layer FP8 MLA stack + head, batched verify of {n} positions at pos {pos} from token {tok0}")
    orc = _Oracle(m)
    # drafts: the oracle's greedy continuation for 4 positions, one wrong token, then greedy again
    inputs, ref = [tok0], []
    for j in range(n):
        lo, tk, recs = orc.position(inputs[-1], pos + j)
        ref.append((lo, tk, recs))
        if j < n - 1:
            inputs.append(tk if j != 4 else (tk + 7) % m.vocab)
    drafts = inputs[1:]
    dec = _decoder(m)
    lg, toks, acc, _ = _batched(dec, m, pos, tok0, drafts)
    say(f"GPU tokens {toks}, accepted {acc}; oracle tokens {[r[1] for r in ref]}")
    H = m.layer.hidden
    vh2 = dec.debug("vh2").cpu().numpy().astype(np.float64).reshape(8, H)
    vf = dec.debug("vf").cpu().numpy().astype(np.float64).reshape(8, H)
    vsel = dec.debug("vsel").cpu().numpy()
    errs = []
    for j in range(n):
        rec = ref[j][2][0]
        x = nx.bf16_to_f64(np.asarray(rec["x_in"]).view(np.uint16))
        e_y = rel_err(vh2[j] - x, rec["y"])
        e_f = rel_err(vf[j], rec["f"])
        e_l = rel_err(lg[j], ref[j][0])
        sel = [int(v) for v in vsel[j * 8: j * 8 + m.layer.top_k]]
        say(f"position {j}: y {e_y:.2e}, f {e_f:.2e}, logits {e_l:.2e}, experts {sel} (oracle {list(rec['router_sel'])})")
        errs.append((e_y, e_f, sel == list(rec["router_sel"])))
    for j, (e_y, e_f, same) in enumerate(errs):
        assert e_y < BAR_VB, f"position {j}: y rel err {e_y}"
        assert e_f < BAR_VB, f"position {j}: f rel err {e_f}"
        assert same, f"position {j}: expert choice differs"
        _compare_logits(lg[j], ref[j][0], toks[j], ref[j][1], f"position {j}")
    assert acc == _accepted(inputs, [r[1] for r in ref]) == 4


def test_batched_verify_full_cache_two_layers_vs_oracle():
    """Two layers over the 8192-token history of the stack workload, 6 positions from 8192
    (drafts: the oracle's greedy tokens except a wrong fourth): logits, tokens and the
    accepted count against the oracle."""
    _need_gpu()
    m = _model(n_layers=2, cache_len=8192)
    pos, n = 8192, 6
    tok0 = gen.first_token(m)
    say(f"case: 2-layer FP8 MLA stack + head, 8192-token cache, batched verify of {n} positions")
    orc = _Oracle(m)
    inputs, ref = [tok0], []
    for j in range(n):
        lo, tk, _ = orc.position(inputs[-1], pos + j)
        ref.append((lo, tk))
        if j < n - 1:
            inputs.append(tk if j != 3 else (tk + 1) % m.vocab)
    dec = _decoder(m)
    lg, toks, acc, _ = _batched(dec, m, pos, tok0, inputs[1:])
    say(f"GPU tokens {toks}, accepted {acc}; oracle tokens {[r[1] for r in ref]}")
    for j in range(n):
        _compare_logits(lg[j], ref[j][0], toks[j], ref[j][1], f"position {j} (pos {pos + j})")
    assert acc == _accepted(inputs, [r[1] for r in ref]) == 3


def _router_gap(rec, s, W):
    """Smallest gap, at the top-k boundary, between the selection keys of the oracle's router."""
    r = np.asarray(rec["router_logits"], np.float64)
    key = 1.0 / (1.0 + np.exp(-r)) + np.asarray(W.router_bias(), np.float64)
    o = np.sort(key)[::-1]
    return float(o[s.top_k - 1] - o[s.top_k])


@pytest.mark.parametrize("nq,temperature", [(2, 0.0), (3, 0.0), (5, 0.8), (8, 0.0)])
def test_batched_matches_sequential_verify(nq, temperature):
    """The batched and the sequential verify on the same stack and drafts (two layers, a
    ragged 517-row history; drafts = the tokens plain decoding chooses, so all are accepted):
    the same tokens and accepted count, and logits within TOL of each other. Where two
    positions' logits differ by more, the oracle must explain it: the batched logits are
    within TOL of the oracle's, and the oracle's router has a near-tie (the k-th and
    (k+1)-th selection keys within 1e-3) at that position, so the two device paths, whose
    activations differ at the 1e-3 level, may each take a different one of two equally
    good experts. (At position 518, greedy, the oracle's keys of layer 1 are 3.8e-5 apart
    and the sequential path takes the other expert.)"""
    _need_gpu()
    m = _model(n_layers=2, cache_len=517)
    pos = 517
    tok0 = gen.first_token(m)
    say(f"case: batched vs sequential verify, {nq} positions at pos {pos}, T {temperature}")
    decS = _decoder(m, max_query=0)
    tk = torch.full((nq - 1,), -1, dtype=torch.int32, device="cuda")
    out = torch.zeros(m.layer.hidden, dtype=torch.int16, device="cuda")
    decS.persistent(start_pos=pos, in_token=tok0, n_tokens=nq - 1, out_hidden=out, out_tokens=tk,
                    temperature=temperature, sample_seed=11)
    torch.cuda.synchronize()
    _status_ok(decS, "plain decoding")
    drafts = [int(v) for v in tk.cpu().numpy()]
    decS2 = _decoder(m, max_query=0)
    lgS, tkS, accS = _sequential(decS2, m, pos, tok0, drafts, temperature, 11)
    decB = _decoder(m)
    lgB, tkB, accB, _ = _batched(decB, m, pos, tok0, drafts, temperature, 11)
    say(f"sequential tokens {tkS} accepted {accS}; batched tokens {tkB} accepted {accB}")
    errs = [rel_err(lgB[j], lgS[j]) for j in range(nq)]
    say("batched vs sequential logits rel err per position: " + ", ".join(f"{e:.2e}" for e in errs))
    assert accB == accS == nq - 1
    assert tkB == tkS
    if max(errs) >= TOL:
        orc = _Oracle(m)
        inputs = [tok0] + drafts
        for j in range(nq):
            lo, _, recs = orc.position(inputs[j], pos + j, temperature, 11)
            if errs[j] < TOL:
                continue
            e_b, e_s = rel_err(lgB[j], lo), rel_err(lgS[j], lo)
            gaps = [_router_gap(r, m.layer, orc.W[l]) for l, r in enumerate(recs)]
            say(f"position {j}: vs oracle batched {e_b:.2e}, sequential {e_s:.2e}; router key gaps {gaps}")
            assert e_b < TOL, f"position {j}: batched vs oracle {e_b}"
            assert min(gaps) < 1e-3, f"position {j}: the paths differ without a router near-tie"


def test_batched_verify_argument_errors():
    _need_gpu()
    import persistent_latency_bound_amd as pld
    m = _model(n_layers=1, cache_len=64)
    say("case: batched verify argument errors")
    dec0 = _decoder(m, max_query=0)
    out = torch.zeros(m.layer.hidden, dtype=torch.int16, device="cuda")
    with pytest.raises(pld.PldError) as e:
        dec0.verify_batched(64, 1, torch.zeros(3, dtype=torch.int32, device="cuda"), out)
    assert e.value.code == pld.PLD_E_UNSUPPORTED
    dec = _decoder(m, max_query=4)
    with pytest.raises(pld.PldError) as e:
        dec.verify_batched(64, 1, torch.zeros(4, dtype=torch.int32, device="cuda"), out)   # 5 > max_query
    assert e.value.code == pld.PLD_E_INVALID
    with pytest.raises(pld.PldError) as e:
        dec.verify_batched(125, 1, torch.zeros(3, dtype=torch.int32, device="cuda"), out)   # past max_seq
    assert e.value.code == pld.PLD_E_CAPACITY
