"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

  * toy fp32 decoder (2 layers, d=256, V=4096): context of 512 uniform tokens prefilled
    through the model on each side independently, drafts = greedy decoding under 12
    silence tokens; exact (fp64) oracle, tolerance 1e-5;
  * 1.7B-shape bf16 decoder (24 layers, d=2048, V=49152), synthetic context C=4096, 25
    audio + 16 drafts: random chunk, and audio = silence with drafts = greedy decoding
    under silence (full acceptance);
  * 8B-shape bf16 decoder (36 layers, d=4096, 32/8 heads x 128, V=151936), C=8192,
    25 audio + 32 drafts + an 8-token runner-up branch under the tree mask, and a
    top-4 sibling tree; in both a non-first branch carries the oracle's next token, so
    the walk takes it and the commit compacts its rows.
The oracle runs the same pass in fp64 (bf16 rounding mode for bf16 models); logits,
argmax (flags below 1e-3 top-2 margin), layer-0 keys/values and greedy acceptance are
compared (tests/gpu_helpers.py).
"""
import numpy as np
import pytest
import torch

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_verify_amd as sdv  # noqa: E402
from oracle import EXACT, BF16_KV  # noqa: E402
from oracle import decoder as odec  # noqa: E402
from oracle.numerics import memoize_f64  # noqa: E402
from synth import (make_weights, make_random_kv, uniform_tokens, toy_workload, w1p7b_workload,  # noqa: E402
                   w8b_tree_workload)
from tests.gpu_helpers import compare_logits, greedy_expectation  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _accept(ver, kv, T, L_a, parent_t):
    acc = sdv.accept_greedy(1, T, L_a, ver.tokens, parent_t, ver.logit_rows, ver.argmax, base_len=kv.seq_len)
    torch.cuda.synchronize()
    return int(acc["n"][0]), int(acc["next"][0])


def compare_kv_layer0(sh, kv, o, C, T):
    k, v = kv.gather(0, 0, C, C + T)
    for gt, ot in ((k.cpu().numpy(), o["k_new"][0][0]), (v.cpu().numpy(), o["v_new"][0][0])):
        bad = np.abs(gt - ot) > np.abs(ot) * 2.0 ** -7 + 1e-6
        assert bad.mean() < 1e-3 and not np.any(np.abs(gt - ot) > np.abs(ot) * 2.0 ** -6 + 1e-5)


@pytest.mark.timeout(600)
def test_full_toy_f32_prefilled():
    wl = toy_workload()
    sh = wl.shape
    C, L_a, gamma = wl.ctx[0], wl.L_a, wl.gamma
    T = wl.T
    w = make_weights(sh, seed=wl.seed)
    ctx = uniform_tokens(C, sh.vocab, wl.seed + 2000, "ctx")
    # GPU prefill
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(sh, 1, C + T + 64)
    sdv.prefill(model, kv, ctx[None, :])
    torch.cuda.synchronize()
    assert int(kv.seq_len[0]) == C
    # oracle prefill (exact)
    cache = odec.Cache.empty(1, sh.n_layers, sh.n_kv_heads, sh.head_dim)
    odec.prefill(w, cache, ctx[None, :], EXACT, chunk=128)
    for l in range(sh.n_layers):
        k, v = kv.gather(0, l, 0, C)
        np.testing.assert_allclose(k.cpu().numpy(), cache.k[0][l], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(v.cpu().numpy(), cache.v[0][l], rtol=1e-5, atol=1e-5)
    sil = np.zeros(L_a, dtype=np.int32)
    drafts, _ = odec.greedy_decode(w, cache.copy(), sil, gamma + 1, EXACT)
    rows = wl.logit_rows()
    for scen in ("random", "silence"):
        audio = sil if scen == "silence" else uniform_tokens(L_a, sh.vocab, wl.seed + 4000, "audio")
        toks = np.concatenate([audio, drafts[:gamma]]).astype(np.int32)
        ver = sdv.Verifier(model, kv, T, L_a, rows, max_ctx=C, want_logits=True, want_hidden=True)
        ver.set_tokens(toks[None, :])
        res = ver.forward()
        torch.cuda.synchronize()
        g = dict(logits=res.logits.cpu().numpy().astype(np.float64), argmax=res.argmax.cpu().numpy(),
                 margin=res.margin.cpu().numpy(), lse=res.lse.cpu().numpy())
        o = odec.verify_forward(w, cache, toks[None, :], None, rows, EXACT)
        err, flagged, n = compare_logits(sh, g, o)
        _say(f"toy {scen}: rel err {err:.2e}, flagged {flagged}/{n}")
        on, onext, _, fl = greedy_expectation(toks, None, L_a, rows, o["logits"][0])
        gn, gnext = _accept(ver, kv, T, L_a, None)
        if not fl:
            assert (gn, gnext) == (on, onext)
        if scen == "silence":
            assert on == gamma and onext == drafts[gamma]


@pytest.mark.timeout(900)
def test_full_1p7b_random_and_silence():
    wl = w1p7b_workload()
    sh = wl.shape
    C, L_a, gamma, T = wl.ctx[0], wl.L_a, wl.gamma, wl.T
    _say("generating 1.7B-shape weights")
    w = make_weights(sh, seed=wl.seed)
    kvh = make_random_kv(sh, [C], capacity=C + T, seed=wl.seed + 1000)
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(sh, 1, C + T + 64)
    kv.load(kvh)
    rows = wl.logit_rows()
    cache = odec.Cache(kvh.k, kvh.v)
    with memoize_f64():
        sil = np.zeros(L_a, dtype=np.int32)
        _say("oracle greedy drafting under silence")
        drafts, _ = odec.greedy_decode(w, cache.copy(), sil, gamma + 1, BF16_KV)
        for scen in ("random", "silence"):
            if scen == "random":
                toks = np.concatenate([uniform_tokens(L_a, sh.vocab, 77, "a"), uniform_tokens(gamma, sh.vocab, 78, "d")])
            else:
                toks = np.concatenate([sil, drafts[:gamma]])
            toks = toks.astype(np.int32)
            ver = sdv.Verifier(model, kv, T, L_a, rows, max_ctx=C, want_logits=True)
            ver.set_tokens(toks[None, :])
            res = ver.forward()
            torch.cuda.synchronize()
            g = dict(logits=res.logits.cpu().numpy().astype(np.float64), argmax=res.argmax.cpu().numpy(),
                     margin=res.margin.cpu().numpy(), lse=res.lse.cpu().numpy())
            _say(f"oracle verify pass ({scen})")
            o = odec.verify_forward(w, cache, toks[None, :], None, rows, BF16_KV)
            err, flagged, n = compare_logits(sh, g, o)
            _say(f"1.7b {scen}: rel err {err:.2e}, flagged {flagged}/{n}")
            compare_kv_layer0(sh, kv, o, C, T)
            on, onext, _, fl = greedy_expectation(toks, None, L_a, rows, o["logits"][0])
            gn, gnext = _accept(ver, kv, T, L_a, None)
            if not fl:
                assert (gn, gnext) == (on, onext)
            if scen == "silence" and not fl:
                assert on == gamma


def _commit_and_check_moves(sh, ver, kv, acc, C, L_a, T):
    """Commit with the plan of accept_greedy: accepted row path[i] must land in slot
    C + L_a + i of every layer (bit-identical K/V)."""
    n = int(acc["n"][0])
    path = acc["path"][0, :n].cpu().tolist()
    before = [kv.gather(0, l, C, C + T) for l in range(sh.n_layers)]
    sdv.kv_rollback(ver.model, kv, acc["keep"], acc["move_src"], acc["move_dst"], acc["err"])
    torch.cuda.synchronize()
    assert int(kv.seq_len[0]) == C + L_a + n and int(acc["err"][0]) == 0
    for l in range(sh.n_layers):
        k, v = kv.gather(0, l, C + L_a, C + L_a + n)
        assert torch.equal(k, before[l][0][path]) and torch.equal(v, before[l][1][path])
    return n, path


@pytest.mark.timeout(1200)
def test_full_8b_tree():
    """The 8B tree workload (25 audio + 32 drafts + an 8-token branch forking at the last
    audio row), and a top-k tree of 4 siblings (8 + 3 x 4 tokens) on the same model.  In
    both, one non-first branch starts with the oracle's argmax at the last audio row (from
    an oracle pass over the audio alone) and the main draft does not, so the walk takes
    that branch and the commit moves its rows at 36 layers, 8 kv heads, dh 128."""
    wl = w8b_tree_workload()
    sh = wl.shape
    C, L_a, gamma, nb, T = wl.ctx[0], wl.L_a, wl.gamma, wl.n_branch, wl.T
    _say("generating 8B-shape weights")
    w = make_weights(sh, seed=wl.seed)
    kvh = make_random_kv(sh, [C], capacity=C + T, seed=wl.seed + 1000)
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(sh, 1, C + T + 64)
    kv.load(kvh)
    cache = odec.Cache(kvh.k, kvh.v)
    audio = uniform_tokens(L_a, sh.vocab, 80, "a")
    keep_c = torch.tensor([C], dtype=torch.int32, device="cuda")
    with memoize_f64():
        _say("oracle pass over the audio alone")
        a1 = int(np.argmax(odec.verify_forward(w, cache, audio[None, :], None, [L_a - 1], BF16_KV)["logits"][0, 0]))
        cases = []
        main = uniform_tokens(gamma, sh.vocab, 81, "m")
        branch = uniform_tokens(nb, sh.vocab, 82, "b")
        branch[0] = a1
        if main[0] == a1:
            main[0] = (a1 + 1) % sh.vocab
        cases.append(("C3 tree", wl.parent(), [main, branch]))
        sib = [uniform_tokens(n, sh.vocab, 90 + k, "s") for k, n in enumerate([8, 4, 4, 4])]
        firsts = [(a1 + 1 + 17 * k) % sh.vocab for k in range(4)]
        firsts[2] = a1
        for k in range(4):
            sib[k][0] = firsts[k]
        cases.append(("top-4 tree", sdv.tree_parent(L_a, [8, 4, 4, 4]), sib))
        for name, parent, branches in cases:
            toks = np.concatenate([audio] + [np.asarray(b, np.int32) for b in branches]).astype(np.int32)
            Tc = len(toks)
            rows = list(range(L_a - 1, Tc))
            sdv.kv_rollback(model, kv, keep_c)
            ver = sdv.Verifier(model, kv, Tc, L_a, rows, parent=parent, max_ctx=C, want_logits=True)
            ver.set_tokens(toks[None, :])
            res = ver.forward()
            torch.cuda.synchronize()
            g = dict(logits=res.logits.cpu().numpy().astype(np.float64), argmax=res.argmax.cpu().numpy(),
                     margin=res.margin.cpu().numpy(), lse=res.lse.cpu().numpy())
            _say(f"oracle verify pass ({name}, T={Tc})")
            o = odec.verify_forward(w, cache, toks[None, :], parent, rows, BF16_KV)
            err, flagged, n_rows = compare_logits(sh, g, o, max_flag_frac=0.02)
            _say(f"8b {name}: rel err {err:.2e}, flagged {flagged}/{n_rows}")
            compare_kv_layer0(sh, kv, o, C, Tc)
            on, onext, opath, fl = greedy_expectation(toks, parent, L_a, rows, o["logits"][0])
            acc = sdv.accept_greedy(1, Tc, L_a, ver.tokens, ver.parent, ver.logit_rows, ver.argmax,
                                    base_len=kv.seq_len)
            torch.cuda.synchronize()
            if not fl:
                assert (int(acc["n"][0]), int(acc["next"][0])) == (on, onext)
                assert on >= 1 and toks[opath[0]] == a1 and opath[0] != L_a     # a non-first branch won
            n, path = _commit_and_check_moves(sh, ver, kv, acc, C, L_a, Tc)
            _say(f"8b {name}: accepted {n} rows {path}")
