"""Oracle multi-codebook stream bookkeeping (test infrastructure only).

"An Efficient vLLM-Based Inference Pipeline for Unified Audio Understanding and
Generation" (page 2):
  * delay-pattern interleave: with S codebook streams, stream s is shifted by s steps,
    so the code of frame f of stream s is produced at audio step f + s; at the end the
    S x T code matrix is de-interleaved ("why a single-stream loop cannot hold
    multi-layer audio generation");
  * primary / auxiliary decomposition: one stream (codebook 0) is the token the engine
    sees, the other S - 1 are taken inside the logits stage and buffered per request;
  * phase state machine with a dynamic vocabulary mask: the text phase allows only
    text tokens, a transition phase injects fixed bridge tokens, the audio phase
    activates all S streams, and after it ends a drain sub-phase emits S - 1 padding
    tokens to flush the delay buffer so the matrix is complete; the current modality is
    read from which vocabulary partition the argmax of the UNMASKED distribution falls
    in.

Readings where the page is silent (the plainest ones; the verify pass sees one phase):
  * partitions: ids [0, text_end) are text, ids [base, base + Vc) are codebook 0's codes
    (the primary stream); anything else is neither;
  * a pass keeps the phase it starts in; the token at prediction depth k of the pass is
    masked by that phase: text -> text ids; transition -> only bridge[pos + k]; audio ->
    codebook-0 ids; drain -> only the pad code while pos + k < S - 1;
  * a row stops acceptance (no token, -1) when it leaves the phase: in the text phase
    when its unmasked argmax is a codebook-0 id (the model switches to audio), in the
    transition phase past the last bridge token, in the drain phase past its S - 1 steps;
  * the audio phase ends with the end-of-audio code of codebook 0 at audio step F: the
    segment has F frames (steps 0..F-1 carry frame t of stream 0), and the codes with
    frame index t - s < F are kept through the end-of-audio step and the S - 1 drain
    steps that follow it.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

TEXT, TRANSITION, AUDIO, DRAIN = 0, 1, 2, 3
MOD_TEXT, MOD_AUDIO, MOD_OTHER = 0, 1, 2


@dataclass
class StreamCfg:
    S: int
    Vc: int
    base: int            # backbone id of code 0 of codebook 0
    text_end: int        # ids below are text
    eoa_code: int        # codebook-0 code that ends the audio phase
    pad_code: int        # codebook-0 code emitted while draining
    bridge: List[int]    # backbone ids injected in the transition phase
    max_frames: int


@dataclass
class StreamState:
    phase: int = TEXT
    pos: int = 0          # tokens taken in the current phase (transition / drain)
    t: int = 0            # audio steps of the current segment
    frames: int = -1      # frames of the segment once its end-of-audio code arrived
    matrix: Optional[np.ndarray] = None   # [S, max_frames] codes, -1 where none yet

    def init(self, cfg: StreamCfg) -> "StreamState":
        self.matrix = np.full((cfg.S, cfg.max_frames), -1, dtype=np.int64)
        return self


def modality(row: np.ndarray, cfg: StreamCfg) -> int:
    """Partition of the unmasked argmax (lowest index on ties)."""
    i = int(np.argmax(row))
    if i < cfg.text_end:
        return MOD_TEXT
    if cfg.base <= i < cfg.base + cfg.Vc:
        return MOD_AUDIO
    return MOD_OTHER


def masked_choice(row: np.ndarray, st: StreamState, k: int, cfg: StreamCfg):
    """(token or -1, modality) of the prediction at depth k of a pass that started in
    state st; row: logits over the whole vocabulary."""
    mod = modality(row, cfg)
    if st.phase == TEXT:
        if mod == MOD_AUDIO:
            return -1, mod
        return int(np.argmax(row[:cfg.text_end])), mod
    if st.phase == TRANSITION:
        j = st.pos + k
        return (cfg.bridge[j] if j < len(cfg.bridge) else -1), mod
    if st.phase == AUDIO:
        return cfg.base + int(np.argmax(row[cfg.base:cfg.base + cfg.Vc])), mod
    return (cfg.base + cfg.pad_code if st.pos + k < cfg.S - 1 else -1), mod


def _put(st: StreamState, cfg: StreamCfg, codes: Sequence[int]) -> None:
    """Audio step st.t: stream s carries frame st.t - s."""
    for s in range(cfg.S):
        f = st.t - s
        if 0 <= f < cfg.max_frames and (st.frames < 0 or f < st.frames):
            st.matrix[s, f] = int(codes[s])
    st.t += 1


def commit(st: StreamState, cfg: StreamCfg, tokens: Sequence[int], codes: Optional[Sequence[Sequence[int]]],
           stopped_by_switch: bool) -> None:
    """Apply the committed tokens of one pass in order (codes[i]: the S codebook codes of
    step i, needed in the audio and drain phases), then the phase switch when the pass
    stopped at a text row whose unmasked argmax was a codebook-0 id."""
    for i, x in enumerate(tokens):
        if st.phase == TEXT:
            pass
        elif st.phase == TRANSITION:
            st.pos += 1
            if st.pos == len(cfg.bridge):
                st.phase, st.pos, st.t, st.frames = AUDIO, 0, 0, -1
        elif st.phase == AUDIO:
            if int(x) - cfg.base == cfg.eoa_code:
                st.frames = st.t
                _put(st, cfg, codes[i])
                st.phase, st.pos = DRAIN, 0
            else:
                _put(st, cfg, codes[i])
        else:
            _put(st, cfg, codes[i])
            st.pos += 1
            if st.pos == cfg.S - 1:
                st.phase, st.pos = TEXT, 0
    if stopped_by_switch and st.phase == TEXT:
        st.phase, st.pos = (TRANSITION, 0) if cfg.bridge else (AUDIO, 0)
        if st.phase == AUDIO:
            st.t, st.frames = 0, -1
