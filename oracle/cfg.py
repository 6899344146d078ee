"""Codebook heads and classifier-free guidance (test infrastructure only).

Follows "An Efficient vLLM-Based Inference Pipeline for Unified Audio Understanding
and Generation" (page 2):
  * architecture (Figure 1): the vocabulary is split into a text part and S audio
    sub-vocabularies; for an audio step every stream adds its own learned stream
    embedding to the backbone hidden state h_t and a matrix shared by all streams
    turns that sum into the stream's logits;
  * paired scheduling for guidance: a conditional request and its unconditional
    companion share one backbone forward; their logits are combined per codebook
    with a weight w > 1 and the resulting token is appended to both histories.
The combination is u + w (c - u) (c conditional, u unconditional logits), applied
to every codebook.

Readings where the page is silent (listed with the others in the design notes):
  * h_t is the backbone output after the final RMSNorm (what the text LM head reads);
  * codebook 0 carries the token the serving engine sees: acceptance of a verify pass
    is decided on merged codebook 0, whose code c is backbone id `base + c`;
  * both rows of a pair are fed the same tokens, keep separate caches of equal
    length, and commit the same number of tokens.

Everything is fp64.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import accept as oacc
from . import decoder as odec
from .numerics import bits_to_f64


def codebook_logits(w, hidden: np.ndarray) -> np.ndarray:
    """Logits of every codebook for hidden rows `hidden` [N, d] (residual stream
    before the final norm): out[n, s, :] = W_cb (RMSNorm(h_n) + e_s).  [N, S, Vc]"""
    sh = w.shape
    hn = odec.rmsnorm(np.asarray(hidden, np.float64), bits_to_f64(w.final_norm), sh.eps)
    wcb = bits_to_f64(w.codebook)                       # [Vc, d]
    e = np.asarray(w.stream_emb, np.float64)            # [S, d]
    out = np.empty((hn.shape[0], sh.n_codebooks, sh.codebook_size))
    for s in range(sh.n_codebooks):
        out[:, s, :] = (hn + e[s]) @ wcb.T
    return out


def cfg_merge(c: np.ndarray, u: np.ndarray, weight: float) -> np.ndarray:
    """Guided logits u + w (c - u)."""
    return u + weight * (c - u)


def check_partners(partner: Sequence[int]) -> None:
    """partner[b] is the other row of b's pair (or -1); pairs must be mutual."""
    B = len(partner)
    for b, p in enumerate(partner):
        if p >= 0 and not (p < B and p != b and partner[p] == b):
            raise ValueError(f"row {b}: partner {p} is not mutual")


def verify_codebook(w, cache, tokens: np.ndarray, parent: Optional[Sequence[int]], logit_rows: Sequence[int],
                    partner: Sequence[int], weight: float, base: int, mode: str) -> dict:
    """A verify pass whose next-token distributions come from the codebook heads.

    Returns
      logits  [B, R, S, Vc]  guided logits for rows of a pair (identical for both rows:
                             the lower-indexed row of a pair is the conditional one),
                             the row's own codebook logits otherwise
      argmax  [B, R, S]      per-codebook argmax (lowest index on ties)
      token   [B, R]         backbone id of codebook 0's argmax (base + code)
      margin  [B, R]         top-1 minus top-2 of codebook 0
      res                    the decoder verify result (hidden rows, K/V written)
    """
    check_partners(partner)
    res = odec.verify_forward(w, cache, tokens, parent, logit_rows, mode)
    hidden = res["hidden"]                                # [B, T, d]
    B = hidden.shape[0]
    own = np.stack([codebook_logits(w, hidden[b][list(logit_rows)]) for b in range(B)])  # [B, R, S, Vc]
    out = own.copy()
    for b in range(B):
        p = partner[b]
        if p >= 0:
            c, u = (b, p) if b < p else (p, b)
            out[b] = cfg_merge(own[c], own[u], weight)
    R, S = out.shape[1], out.shape[2]
    am = np.empty((B, R, S), dtype=np.int64)
    margin = np.empty((B, R))
    for b in range(B):
        for r in range(R):
            for s in range(S):
                am[b, r, s] = oacc.argmax_lowest(out[b, r, s])
            margin[b, r] = oacc.top2_margin(out[b, r, 0])
    return {"logits": out, "argmax": am, "token": base + am[:, :, 0], "margin": margin, "res": res}
