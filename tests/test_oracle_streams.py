"""Pins of the oracle's multi-codebook stream bookkeeping (CPU only).

Page 2 ("An Efficient vLLM-Based Inference Pipeline for Unified Audio Understanding
and Generation"): stream s is delayed by s steps and the S x T matrix is
de-interleaved at the end; the phase machine goes text -> transition (bridge tokens)
-> audio -> drain (S - 1 padding tokens flush the delay buffer) -> text; the
modality is the vocabulary partition of the unmasked argmax.  Pinned by the
delay-pattern round trip (interleaving a known matrix step by step, in passes cut
at random, gives the matrix back), by the lengths of the transition and drain
phases, and by brute-force checks of the mask.
"""
import numpy as np
import pytest

from oracle import streams as st

CFG = st.StreamCfg(S=4, Vc=16, base=44, text_end=40, eoa_code=15, pad_code=14, bridge=[41, 42, 43], max_frames=64)


def _interleaved_steps(M, cfg, rng):
    """The committed steps of one audio segment under the delay pattern: step t carries
    frame t of stream 0 (t < F), the end-of-audio code at t = F, pad codes after; stream
    s carries frame t - s when it exists (anything else otherwise)."""
    S, F = M.shape
    steps = []
    for t in range(F + S):
        codes = [int(M[s, t - s]) if 0 <= t - s < F else int(rng.integers(0, 14)) for s in range(S)]
        if t < F:
            tok = cfg.base + codes[0]
        elif t == F:
            tok = cfg.base + cfg.eoa_code
            codes[0] = cfg.eoa_code
        else:
            tok = cfg.base + cfg.pad_code
            codes[0] = cfg.pad_code
        steps.append((tok, codes))
    return steps


@pytest.mark.parametrize("F", [1, 5, 23])
def test_delay_pattern_round_trip_in_random_passes(F):
    rng = np.random.default_rng(F)
    M = rng.integers(0, 14, size=(CFG.S, F))
    s = st.StreamState().init(CFG)
    s.phase = st.AUDIO
    steps = _interleaved_steps(M, CFG, rng)[:F + CFG.S]     # audio steps, the end, S - 1 drain steps
    i = 0
    while i < len(steps):
        k = int(rng.integers(1, 6))
        chunk = steps[i:i + k]
        st.commit(s, CFG, [t for t, _ in chunk], [c for _, c in chunk], False)
        i += k
    assert s.frames == F
    assert np.array_equal(s.matrix[:, :F], M)
    assert np.all(s.matrix[:, F:] == -1)
    assert s.phase == st.TEXT and s.pos == 0


def test_transition_takes_the_bridge_then_audio():
    s = st.StreamState().init(CFG)
    st.commit(s, CFG, [3, 7], None, True)            # text tokens, then the switch
    assert s.phase == st.TRANSITION and s.pos == 0
    st.commit(s, CFG, CFG.bridge[:2], None, False)
    assert s.phase == st.TRANSITION and s.pos == 2
    st.commit(s, CFG, CFG.bridge[2:], None, False)
    assert s.phase == st.AUDIO and s.t == 0 and s.frames == -1


def test_drain_is_s_minus_one_steps():
    s = st.StreamState().init(CFG)
    s.phase = st.AUDIO
    codes = [[1, 2, 3, 4]] * 10
    st.commit(s, CFG, [CFG.base + 1, CFG.base + 1, CFG.base + CFG.eoa_code], codes, False)
    assert s.phase == st.DRAIN and s.frames == 2
    for j in range(CFG.S - 2):
        st.commit(s, CFG, [CFG.base + CFG.pad_code], codes, False)
        assert s.phase == st.DRAIN
    st.commit(s, CFG, [CFG.base + CFG.pad_code], codes, False)
    assert s.phase == st.TEXT


def test_mask_by_phase_against_brute_force():
    rng = np.random.default_rng(5)
    V = CFG.base + CFG.S * CFG.Vc
    for trial in range(300):
        row = rng.standard_normal(V)
        if trial % 3 == 0:
            row[CFG.base + int(rng.integers(0, CFG.Vc))] += 5.0
        s = st.StreamState().init(CFG)
        s.phase = int(rng.integers(0, 4))
        s.pos = int(rng.integers(0, 3))
        k = int(rng.integers(0, 4))
        tok, mod = st.masked_choice(row, s, k, CFG)
        top = max(range(V), key=lambda i: (row[i], -i))
        want_mod = st.MOD_TEXT if top < CFG.text_end else (
            st.MOD_AUDIO if CFG.base <= top < CFG.base + CFG.Vc else st.MOD_OTHER)
        assert mod == want_mod
        if s.phase == st.TEXT:
            want = -1 if mod == st.MOD_AUDIO else max(range(CFG.text_end), key=lambda i: (row[i], -i))
        elif s.phase == st.TRANSITION:
            want = CFG.bridge[s.pos + k] if s.pos + k < len(CFG.bridge) else -1
        elif s.phase == st.AUDIO:
            want = max(range(CFG.base, CFG.base + CFG.Vc), key=lambda i: (row[i], -i))
        else:
            want = CFG.base + CFG.pad_code if s.pos + k < CFG.S - 1 else -1
        assert tok == want
