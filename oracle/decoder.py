"""Oracle decoder forward for the single-forward verify step (test infrastructure only).

Follows "Decode Before You Hear: Speculative Listening" (page 1), section
"Method steps", step 4: with the cache holding x_{<t}, one forward over the
audio chunk a_t and the draft y~ yields, for every draft position i, the target
distribution p_i = p(. | x_{<t}, a_t, y~_{<i}); p_1 comes from the last audio
row and p_{i+1} from the row of draft token i.  The "KV cache and
prefill/decode" prerequisite on the same page states why this costs about one
decode step.

The decoder is a pre-norm transformer: RMSNorm, grouped-query attention with
rotary positions (rotate-half pairing), SwiGLU FFN, untied LM head.  A chunk
may be a tree (runner-up branch, step 2 of the method): row j sees every cached
slot plus the chunk rows that are j itself or its ancestors, and sits at
position C + depth(j).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np

from . import BF16, BF16_KV, EXACT
from .numerics import bits_to_f64, round_bf16, round_f32


def _identity(x):
    return x


class _Rounding:
    """Where values are rounded: bf16 activations, the fp32 residual stream, and the
    bf16 keys/values written to the cache."""

    def __init__(self, mode: str):
        if mode not in (EXACT, BF16, BF16_KV):
            raise ValueError(mode)
        self.act = round_bf16 if mode == BF16 else _identity
        self.res = round_f32 if mode == BF16 else _identity
        self.kv = round_bf16 if mode in (BF16, BF16_KV) else _identity


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half form: element i pairs with i + dh/2 and both
    rotate by the angle pos * theta^(-2i/dh).  x: [T, n_heads, dh]."""
    dh = x.shape[-1]
    half = dh // 2
    inv = theta ** (-(2.0 * np.arange(half)) / dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def tree_depths(T: int, parent: Optional[Sequence[int]]) -> np.ndarray:
    """depth(0) = 0; depth(j) = depth(parent(j)) + 1.  parent=None means a chain."""
    if parent is None:
        return np.arange(T)
    depth = np.zeros(T, dtype=np.int64)
    for j in range(T):
        p = parent[j]
        if j == 0:
            if p != -1:
                raise ValueError("row 0 must be the root")
            continue
        if not (0 <= p < j):
            raise ValueError(f"parent of row {j} must be an earlier row")
        depth[j] = depth[p] + 1
    return depth


def visible_chunk_rows(T: int, parent: Optional[Sequence[int]]) -> np.ndarray:
    """vis[i, j] is True when chunk row j is row i or one of its ancestors."""
    vis = np.zeros((T, T), dtype=bool)
    for i in range(T):
        j = i
        while j >= 0:
            vis[i, j] = True
            j = (j - 1) if parent is None else parent[j]
    return vis


def attend(q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, k: np.ndarray, v: np.ndarray,
           vis: np.ndarray) -> np.ndarray:
    """softmax(q k^T / sqrt(dh)) v for every chunk row and query head.

    q [T, H, dh]; cached keys/values Kc, Vc [C, Hkv, dh]; chunk keys/values k, v
    [T, Hkv, dh]; vis [T, T] chunk visibility.  Query head h reads kv head h // G with
    G = H / Hkv (consecutive query heads share a kv head).  Returns [T, H * dh]."""
    T, H, dh = q.shape
    Hkv = Kc.shape[1]
    G = H // Hkv
    C = Kc.shape[0]
    scale = 1.0 / math.sqrt(dh)
    qg = q.reshape(T, Hkv, G, dh).transpose(1, 0, 2, 3).reshape(Hkv, T * G, dh)
    s_cache = np.matmul(qg, Kc.transpose(1, 2, 0)) * scale           # [Hkv, T*G, C]
    s_chunk = np.matmul(qg, k.transpose(1, 2, 0)) * scale            # [Hkv, T*G, T]
    s_chunk = s_chunk.reshape(Hkv, T, G, T)
    s_chunk = np.where(vis[None, :, None, :], s_chunk, -np.inf).reshape(Hkv, T * G, T)
    s = np.concatenate([s_cache, s_chunk], axis=-1)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    o = (np.matmul(p[..., :C], Vc.transpose(1, 0, 2))
         + np.matmul(p[..., C:], v.transpose(1, 0, 2)))              # [Hkv, T*G, dh]
    return o.reshape(Hkv, T, G, dh).transpose(1, 0, 2, 3).reshape(T, H * dh)


class Cache:
    """Per-sequence, per-layer cached keys and values in fp64: k[b][l] is [len_b, Hkv, dh]."""

    def __init__(self, k: List[List[np.ndarray]], v: List[List[np.ndarray]]):
        self.k = [[bits_to_f64(a) for a in kb] for kb in k]
        self.v = [[bits_to_f64(a) for a in vb] for vb in v]

    @classmethod
    def empty(cls, B: int, n_layers: int, n_kv: int, dh: int) -> "Cache":
        z = np.zeros((0, n_kv, dh))
        return cls([[z] * n_layers for _ in range(B)], [[z] * n_layers for _ in range(B)])

    def length(self, b: int) -> int:
        return self.k[b][0].shape[0]

    def append(self, b: int, k_rows: List[np.ndarray], v_rows: List[np.ndarray]) -> None:
        for l in range(len(self.k[b])):
            self.k[b][l] = np.concatenate([self.k[b][l], k_rows[l]], axis=0)
            self.v[b][l] = np.concatenate([self.v[b][l], v_rows[l]], axis=0)

    def truncate(self, b: int, n: int) -> None:
        for l in range(len(self.k[b])):
            self.k[b][l] = self.k[b][l][:n]
            self.v[b][l] = self.v[b][l][:n]

    def copy(self) -> "Cache":
        c = Cache.__new__(Cache)
        c.k = [[a.copy() for a in kb] for kb in self.k]
        c.v = [[a.copy() for a in vb] for vb in self.v]
        return c


def verify_forward(w, cache: Cache, tokens: np.ndarray, parent: Optional[Sequence[int]],
                   logit_rows: Sequence[int], mode: str = EXACT, want_attn: bool = False) -> dict:
    """One forward over the chunk rows `tokens` [B, T] on top of `cache`.

    Returns a dict with
      logits  fp64 [B, R, V]   LM-head logits of the rows `logit_rows`
      k_new   k_new[b][l] fp64 [T, Hkv, dh]: keys written for the chunk rows (after RoPE)
      v_new   likewise for values
      hidden  fp64 [B, T, d]   residual stream after the last layer (before the final norm)
      attn    (want_attn) attn[b][l] fp64 [T, H*dh]: attention output of each layer
    The cache itself is not modified.
    """
    sh = w.shape
    rnd = _Rounding(mode)
    tokens = np.asarray(tokens)
    B, T = tokens.shape
    H, Hkv, dh = sh.n_heads, sh.n_kv_heads, sh.head_dim
    G = H // Hkv
    depth = tree_depths(T, parent)
    vis = visible_chunk_rows(T, parent)

    embed = w.embed
    x = np.stack([bits_to_f64(embed[tokens[b]]) for b in range(B)])  # [B, T, d]
    k_new = [[None] * sh.n_layers for _ in range(B)]
    v_new = [[None] * sh.n_layers for _ in range(B)]
    attn = [[None] * sh.n_layers for _ in range(B)]

    for l, lw in enumerate(w.layers):
        wq, wk, wv, wo = (bits_to_f64(lw.wq), bits_to_f64(lw.wk), bits_to_f64(lw.wv), bits_to_f64(lw.wo))
        wg, wu, wd = bits_to_f64(lw.wg), bits_to_f64(lw.wu), bits_to_f64(lw.wd)
        g1, g2 = bits_to_f64(lw.attn_norm), bits_to_f64(lw.ffn_norm)
        for b in range(B):
            C = cache.length(b)
            pos = C + depth
            a = rnd.act(rmsnorm(x[b], g1, sh.eps))
            q = (a @ wq.T).reshape(T, H, dh)
            k = (a @ wk.T).reshape(T, Hkv, dh)
            v = (a @ wv.T).reshape(T, Hkv, dh)
            q = rnd.act(rope(q, pos, sh.rope_theta))
            k = rnd.kv(rope(k, pos, sh.rope_theta))
            v = rnd.kv(v)
            k_new[b][l], v_new[b][l] = k, v

            o = attend(q, cache.k[b][l], cache.v[b][l], k, v, vis)
            o = rnd.act(o)
            if want_attn:
                attn[b][l] = o
            x[b] = rnd.res(x[b] + o @ wo.T)

            hn = rnd.act(rmsnorm(x[b], g2, sh.eps))
            u = rnd.act(silu(hn @ wg.T) * (hn @ wu.T))
            x[b] = rnd.res(x[b] + u @ wd.T)
        del wq, wk, wv, wo, wg, wu, wd

    rows = list(logit_rows)
    gf = bits_to_f64(w.final_norm)
    wlm = bits_to_f64(w.lm_head)
    logits = np.stack([rnd.act(rmsnorm(x[b, rows], gf, sh.eps)) @ wlm.T for b in range(B)])
    out = dict(logits=logits, k_new=k_new, v_new=v_new, hidden=x)
    if want_attn:
        out["attn"] = attn
    return out


def commit_rows(cache: Cache, b: int, res: dict, rows: Sequence[int]) -> None:
    """Append the K/V of the listed chunk rows (in order) to sequence b of the cache."""
    rows = list(rows)
    L = len(cache.k[b])
    cache.append(b, [res["k_new"][b][l][rows] for l in range(L)],
                 [res["v_new"][b][l][rows] for l in range(L)])


def prefill(w, cache: Cache, tokens: np.ndarray, mode: str = EXACT, chunk: int = 128) -> None:
    """Feed tokens [B, n] through the model in chunks and append their K/V to the cache."""
    tokens = np.asarray(tokens)
    n = tokens.shape[1]
    for s in range(0, n, chunk):
        t = tokens[:, s:s + chunk]
        res = verify_forward(w, cache, t, None, [t.shape[1] - 1], mode)
        for b in range(tokens.shape[0]):
            commit_rows(cache, b, res, range(t.shape[1]))


def greedy_decode(w, cache: Cache, prefix: np.ndarray, n_steps: int, mode: str = EXACT,
                  exclude_first: Optional[int] = None):
    """Greedy AR decoding of one sequence (B = 1): feed `prefix` (1-D tokens), then
    repeatedly take y = argmax p(. | ...) (lowest index on ties) and feed it back.

    Returns (tokens, logits_list): the n_steps decoded tokens and the fp64 logits each
    was chosen from.  With exclude_first = y, the first choice is argmax over V minus {y}
    (the runner-up of step 2 of the method).  The cache is advanced by the prefix and
    all decoded tokens but the last (which has not been fed yet)."""
    out, lg = [], []
    feed = np.asarray(prefix, dtype=np.int64)[None, :]
    for step in range(n_steps):
        res = verify_forward(w, cache, feed, None, [feed.shape[1] - 1], mode)
        commit_rows(cache, 0, res, range(feed.shape[1]))
        logits = res["logits"][0, 0]
        if step == 0 and exclude_first is not None:
            l2 = logits.copy()
            l2[exclude_first] = -np.inf
            y = int(np.argmax(l2))
        else:
            y = int(np.argmax(logits))
        out.append(y)
        lg.append(logits)
        feed = np.array([[y]], dtype=np.int64)
    return out, lg
