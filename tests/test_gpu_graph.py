"""A verify step replayed from a captured HIP graph (what `bench.py --graph` times) gives
the eager step's results bit for bit: logits and row statistics, accepted counts and
committed tokens, the K/V pages and the committed length.  The kernels reduce in a
fixed order, so equality is exact.  Every replay is checked, with eager work of the
program and a synchronisation between replays, and the eager step is checked against
the oracle first."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_verify_amd as sdv  # noqa: E402
from oracle import decoder as odec  # noqa: E402
from synth import MINI_BF16, MINI_F32, make_random_kv, make_weights, uniform_tokens  # noqa: E402
from tests.gpu_helpers import compare_logits, mode_of  # noqa: E402


def _snapshot(ver, acc, kv):
    torch.cuda.synchronize()
    return {"logits": ver.logits.clone(), "argmax": ver.argmax.clone(), "margin": ver.margin.clone(),
            "lse": ver.lse.clone(), "n": acc["n"].clone(), "next": acc["next"].clone(),
            "keep": acc["keep"].clone(), "seq_len": kv.seq_len.clone(), "k": kv.k_pages.clone(),
            "v": kv.v_pages.clone(), "err": ver.err.clone(), "acc_err": acc["err"].clone()}


@pytest.mark.parametrize("drafts", ["uniform", "greedy"])
@pytest.mark.parametrize("shape,lens,L_a,gamma", [
    (MINI_BF16, (37, 70), 5, 6),
    (MINI_F32, (50, 3, 17), 4, 9),
])
def test_graph_replays_equal_the_eager_step(shape, lens, L_a, gamma, drafts):
    """drafts "greedy": the model's own continuation of the audio, so every draft is
    accepted (n = gamma) and the commit keeps the whole chunk."""
    print(f"case {shape.name} lens={lens} L_a={L_a} gamma={gamma} drafts={drafts}", flush=True)
    B, T = len(lens), L_a + gamma
    w = make_weights(shape, seed=211, gain_noise=0.1)
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=212)
    toks = np.stack([uniform_tokens(T, shape.vocab, 213 + b, "chunk") for b in range(B)]).astype(np.int32)
    rows = list(range(L_a - 1, T))
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(shape, B, max(lens) + T + 16)
    kv.load(kvh)
    ver = sdv.Verifier(model, kv, T, L_a, rows, max_ctx=max(lens), want_logits=True)
    ver.set_tokens(toks)
    keep_c = torch.tensor(list(lens), dtype=torch.int32, device="cuda")
    acc = None

    def step():
        nonlocal acc
        sdv.kv_rollback(model, kv, keep_c)
        res = ver.forward()
        acc = sdv.accept_greedy(B, T, L_a, ver.tokens, None, ver.logit_rows, res.argmax, base_len=kv.seq_len,
                                out=acc)
        sdv.kv_rollback(model, kv, acc["keep"], acc["move_src"], acc["move_dst"], acc["err"])

    if drafts == "greedy":
        # each eager pass fixes one more draft: row L_a - 1 + j predicts draft j + 1
        for _ in range(gamma):
            step()
            torch.cuda.synchronize()
            toks[:, L_a:] = ver.argmax.cpu().numpy()[:, :gamma]
            ver.set_tokens(toks)
    step()
    eager = _snapshot(ver, acc, kv)
    if drafts == "greedy":
        assert eager["n"].tolist() == [gamma] * B
    assert int(eager["err"].abs().sum()) == 0 and int(eager["acc_err"].abs().sum()) == 0
    o = odec.verify_forward(w, odec.Cache(kvh.k, kvh.v), toks, None, rows, mode_of(shape))
    g = {"logits": eager["logits"].cpu().numpy().astype(np.float64), "argmax": eager["argmax"].cpu().numpy(),
         "margin": eager["margin"].cpu().numpy(), "lse": eager["lse"].cpu().numpy()}
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  eager vs oracle: logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)

    # capture on a side stream after a warm-up there, as the bench does
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for r in range(3):
        # eager work of the program between replays (a whole eager step, which starts by
        # rolling the cache back to its context), then the outputs clobbered, so a
        # replay that skipped a write would show
        step()
        torch.cuda.synchronize()
        for t in (ver.logits, ver.margin, ver.lse):
            t.fill_(float("nan"))
        for t in (ver.argmax, acc["n"], acc["next"], acc["keep"]):
            t.fill_(-7)
        graph.replay()
        got = _snapshot(ver, acc, kv)
        for key, ref in eager.items():
            assert torch.equal(got[key], ref), f"replay {r}: {key} differs from the eager step"
        print(f"  replay {r}: equal to the eager step (n = {got['n'].tolist()})", flush=True)
