"""GPU parity of the multi-codebook stream bookkeeping (page 2, "An Efficient
vLLM-Based Inference Pipeline for Unified Audio Understanding and Generation": delay
pattern and de-interleave, primary / auxiliary streams, phase machine with the
dynamic vocabulary mask and the drain) through the C ABI.

A batch of sessions runs many verify passes over synthetic logits and codebook codes
steered so that every phase and transition occurs (text runs, switches to audio,
bridge tokens, audio segments of different lengths ended by the end-of-audio code,
drains, partial acceptance everywhere).  Per pass the library's phase mask, modality,
greedy walk and commit are compared with the oracle's (oracle.streams and
oracle.accept), and after each pass the phase state and the whole code matrix must be
identical.  The drafts come from the oracle's masked choices.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_verify_amd as sdv  # noqa: E402
from oracle import accept as oacc  # noqa: E402
from oracle import streams as ost  # noqa: E402

S, VC, TEXT_END, BASE = 3, 16, 40, 44
V = BASE + S * VC
CFG = ost.StreamCfg(S=S, Vc=VC, base=BASE, text_end=TEXT_END, eoa_code=15, pad_code=14, bridge=[41, 42],
                    max_frames=40)


def _pass_inputs(rng, states, R):
    """Logits [B, R, V], codebook codes [B, R, S] and the depth at which each session's
    drafts stop matching, steered by each session's phase."""
    B = len(states)
    logits = rng.standard_normal((B, R, V)).astype(np.float32)
    codes = rng.integers(0, 14, size=(B, R, S)).astype(np.int32)
    for b, s in enumerate(states):
        for r in range(R):
            if s.phase == ost.TEXT:
                logits[b, r, int(rng.integers(0, TEXT_END))] += 6.0
            elif s.phase == ost.AUDIO:
                logits[b, r, BASE + codes[b, r, 0]] += 6.0
        if s.phase == ost.TEXT and rng.random() < 0.5:
            logits[b, int(rng.integers(0, R)), BASE + int(rng.integers(0, VC))] += 9.0      # switch to audio
        if s.phase == ost.AUDIO and rng.random() < 0.35:
            r = int(rng.integers(0, R))
            codes[b, r, 0] = CFG.eoa_code
            logits[b, r, BASE + CFG.eoa_code] += 9.0
    return logits, codes


def test_phase_machine_and_delay_matrix_over_many_passes():
    rng = np.random.default_rng(11)
    B, L_a, gamma = 5, 2, 6
    T = L_a + gamma
    R = gamma + 1
    rows = list(range(L_a - 1, T))
    streams = sdv.Streams(B, S, VC, BASE, TEXT_END, CFG.eoa_code, CFG.pad_code, CFG.bridge, CFG.max_frames)
    states = [ost.StreamState().init(CFG) for _ in range(B)]
    depth = torch.arange(R, dtype=torch.int32, device="cuda")
    rows_t = torch.tensor(rows, dtype=torch.int32, device="cuda")
    seen = set()
    completed = 0
    for p in range(60):
        logits, codes = _pass_inputs(rng, states, R)
        tokens = np.zeros((B, T), dtype=np.int32)
        o_am = np.zeros((B, R), dtype=np.int64)
        o_mod = np.zeros((B, R), dtype=np.int64)
        for b, s in enumerate(states):
            for r in range(R):
                o_am[b, r], o_mod[b, r] = ost.masked_choice(logits[b, r].astype(np.float64), s, r, CFG)
            stop = int(rng.integers(0, R + 1))          # drafts follow the masked choices up to here
            tokens[b, :L_a] = rng.integers(0, V, size=L_a)
            for i in range(gamma):
                want = int(o_am[b, i])
                tokens[b, L_a + i] = want if (i < stop and want >= 0) else (max(want, 0) + 1) % V
        tok_t = torch.from_numpy(tokens).cuda()
        am, mod = streams.mask(torch.from_numpy(logits).cuda(), depth)
        acc = sdv.accept_greedy(B, T, L_a, tok_t, None, rows_t, am)
        cb = torch.from_numpy(codes).cuda()
        streams.commit(T, L_a, tok_t, rows_t, acc, cb, mod)
        torch.cuda.synchronize()
        assert np.array_equal(am.cpu().numpy(), o_am), p
        assert np.array_equal(mod.cpu().numpy(), o_mod), p
        g_n, g_next = acc["n"].cpu().numpy(), acc["next"].cpu().numpy()
        for b, s in enumerate(states):
            start = s.phase
            n, nxt, path = oacc.accept_greedy(list(tokens[b]), None, L_a, rows, list(o_am[b]))
            assert (int(g_n[b]), int(g_next[b])) == (n, nxt), (p, b)
            committed = [int(tokens[b, j]) for j in path] + ([nxt] if nxt >= 0 else [])
            pred = [L_a - 1] + path
            cs = [list(codes[b, rows.index(pred[i])]) for i in range(len(committed))]
            stop_row = pred[n]
            switched = nxt < 0 and start == ost.TEXT and o_mod[b, rows.index(stop_row)] == ost.MOD_AUDIO
            ost.commit(s, CFG, committed, cs, switched)
            seen.add((start, s.phase))
            if start in (ost.AUDIO, ost.DRAIN) and s.phase == ost.TEXT:
                completed += 1
        g = [x.cpu().numpy() for x in (streams.phase, streams.phase_pos, streams.step, streams.frames, streams.matrix)]
        for b, s in enumerate(states):
            assert (g[0][b], g[1][b], g[2][b], g[3][b]) == (s.phase, s.pos, s.t, s.frames), (p, b)
            assert np.array_equal(g[4][b], s.matrix), (p, b)
    # every phase began some pass, and audio segments were completed
    assert {a for a, _ in seen} == {ost.TEXT, ost.TRANSITION, ost.AUDIO, ost.DRAIN}, seen
    assert completed > 0
