"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the bench.

Holds random-number generation and storage encoding only (bf16 bit patterns,
page permutations), none of the verify method's arithmetic.

Recipes:
  * matrices and embeddings: N(0, 0.02) drawn in fp32 and stored as fp32 or,
    for bf16 shapes, rounded to nearest-even bf16 bit patterns (uint16);
  * norm gains: 1 (optionally 1 + N(0, gain_noise) for tests);
  * codebook stream embeddings: N(0, 1);
  * synthetic KV-cache contents: uniform on (-sqrt 3, sqrt 3) (unit variance);
  * audio tokens: uniform on [1, V); token 0 stands for silence;
  * speculative-sampling inputs: Gaussian logits calibrated to a top-1 mass,
    draft logits = target logits + sigma * N(0, 1), uniforms from Philox4x32-10.

Large tensors are drawn in 16M-element chunks, each from its own PCG64 stream
keyed by (seed, tensor id, chunk), so generation is parallel and the values do
not depend on the thread count.
"""
from __future__ import annotations

import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from .configs import ModelShape, SampleWorkload

CHUNK = 1 << 24


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _tensor_key(name: str) -> int:
    return zlib.crc32(name.encode()) & 0x7FFFFFFF


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _fill(shape, seed: int, name: str, kind: str, scale: float, dtype: str) -> np.ndarray:
    """Draw a tensor chunk-parallel.  kind: 'normal' (N(0,scale)) or 'uniform' (U(-scale, scale))."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    key = _tensor_key(name)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, c])))
        if kind == "normal":
            v = g.standard_normal(hi - lo, dtype=np.float32)
            v *= np.float32(scale)
        else:
            v = g.random(hi - lo, dtype=np.float32)
            v = (v * np.float32(2.0) - np.float32(1.0)) * np.float32(scale)
        out[lo:hi] = to_bf16_bits(v) if dtype == "bf16" else v

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


@dataclass
class LayerWeights:
    attn_norm: np.ndarray   # [d] fp32
    wq: np.ndarray          # [H*dh, d]
    wk: np.ndarray          # [Hkv*dh, d]
    wv: np.ndarray          # [Hkv*dh, d]
    wo: np.ndarray          # [d, H*dh]
    ffn_norm: np.ndarray    # [d] fp32
    wg: np.ndarray          # [F, d]
    wu: np.ndarray          # [F, d]
    wd: np.ndarray          # [d, F]


@dataclass
class ModelWeights:
    shape: ModelShape
    embed: np.ndarray        # [V, d]
    layers: List[LayerWeights]
    final_norm: np.ndarray   # [d] fp32
    lm_head: np.ndarray      # [V, d] (untied)
    codebook: Optional[np.ndarray] = None     # [codebook_size, d]
    stream_emb: Optional[np.ndarray] = None   # [n_codebooks, d] fp32

    @property
    def storage(self) -> str:
        return self.shape.dtype


def make_weights(shape: ModelShape, seed: int, scales: Optional[Dict[str, float]] = None,
                 gain_noise: float = 0.0, std: float = 0.02) -> ModelWeights:
    """Seeded N(0, std) weights for `shape`.  `scales` multiplies named matrices
    (e.g. {'wq': 8, 'wk': 8, 'wo': 20}) before storage rounding."""
    scales = scales or {}
    dt = shape.dtype
    d, F, V = shape.d, shape.ffn, shape.vocab
    qd, kd = shape.q_dim, shape.kv_dim

    def mat(name, rows, cols, lname=None):
        key = lname or name
        return _fill((rows, cols), seed, key, "normal", std * scales.get(name, 1.0), dt)

    def gain(name):
        if gain_noise == 0.0:
            return np.ones(d, dtype=np.float32)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _tensor_key(name)])))
        return (1.0 + gain_noise * g.standard_normal(d)).astype(np.float32)

    layers = []
    for l in range(shape.n_layers):
        p = f"L{l}."
        layers.append(LayerWeights(
            attn_norm=gain(p + "attn_norm"),
            wq=mat("wq", qd, d, p + "wq"), wk=mat("wk", kd, d, p + "wk"),
            wv=mat("wv", kd, d, p + "wv"), wo=mat("wo", d, qd, p + "wo"),
            ffn_norm=gain(p + "ffn_norm"),
            wg=mat("wg", F, d, p + "wg"), wu=mat("wu", F, d, p + "wu"),
            wd=mat("wd", d, F, p + "wd")))
    w = ModelWeights(shape=shape, embed=mat("embed", V, d), layers=layers,
                     final_norm=gain("final_norm"), lm_head=mat("lm_head", V, d))
    if shape.n_codebooks:
        w.codebook = mat("codebook", shape.codebook_size, d)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _tensor_key("stream_emb")])))
        w.stream_emb = g.standard_normal((shape.n_codebooks, d)).astype(np.float32)
    return w


@dataclass
class KVCache:
    """Logical (unpaged) cache contents: k[b][l], v[b][l] of shape [len_b, Hkv, dh],
    fp32 or bf16 bits.  `capacity` is the slot count reserved per sequence."""
    k: List[List[np.ndarray]]
    v: List[List[np.ndarray]]
    lens: List[int]
    capacity: int


def make_random_kv(shape: ModelShape, lens, capacity: int, seed: int) -> KVCache:
    ks, vs = [], []
    s3 = math.sqrt(3.0)
    for b, n in enumerate(lens):
        kb, vb = [], []
        for l in range(shape.n_layers):
            kb.append(_fill((n, shape.n_kv_heads, shape.head_dim), seed, f"kv.k.{b}.{l}", "uniform", s3, shape.dtype))
            vb.append(_fill((n, shape.n_kv_heads, shape.head_dim), seed, f"kv.v.{b}.{l}", "uniform", s3, shape.dtype))
        ks.append(kb)
        vs.append(vb)
    return KVCache(ks, vs, list(lens), capacity)


# -- hashed synthetic KV: caches of tens of GB generated where they are used --------
#
# Every value is a function of its coordinates only.  The element's linear index
# (token * n_heads + head) * dh + dim inside its (stream, layer, k/v) block, plus a
# per-block key, goes through a 32-bit integer hash (two rounds of xorshift-16 and
# multiply by 0x45d9f3b); the top 24 bits u give (2u + 1 - 2^24) / 2^24 * sqrt(3) in
# fp32, uniform on (-sqrt 3, sqrt 3), rounded to bf16 (nearest even).  The integer
# steps stay below 2^63, so NumPy (hashed_kv_np) and torch on the GPU
# (hashed_kv_torch) produce identical bit patterns: the GPU fills the cache, the host
# regenerates any slice the oracle needs.

_HASH_MUL = 0x45D9F3B
_M32_INT = 0xFFFFFFFF
_S3_F32 = float(np.float32(math.sqrt(3.0)))


def _mix32(x: int) -> int:
    x = ((x >> 16) ^ x) * _HASH_MUL & _M32_INT
    x = ((x >> 16) ^ x) * _HASH_MUL & _M32_INT
    return (x >> 16) ^ x


def hashed_kv_key(seed: int, stream: int, layer: int, kind: int) -> int:
    """Key of one (stream, layer, kind) block; kind 0 = keys, 1 = values."""
    k = _mix32((seed * 0x9E3779B1 + 0x632BE5AB) & _M32_INT)
    for v in (stream, layer, kind):
        k = _mix32((k ^ (v * 0x85EBCA6B + 0xC2B2AE35)) & _M32_INT)
    return k


def hashed_kv_np(seed: int, stream: int, layer: int, kind: int, n_tok: int, n_heads: int, dh: int,
                 tok0: int = 0) -> np.ndarray:
    """bf16 bit patterns [n_tok, n_heads, dh] of tokens tok0 .. tok0 + n_tok - 1."""
    key = np.int64(hashed_kv_key(seed, stream, layer, kind))
    m = np.int64(_M32_INT)
    mul = np.int64(_HASH_MUL)
    x = np.arange(tok0 * n_heads * dh, (tok0 + n_tok) * n_heads * dh, dtype=np.int64)
    x = (x + key) & m
    x = (((x >> 16) ^ x) * mul) & m
    x = (((x >> 16) ^ x) * mul) & m
    x = (x >> 16) ^ x
    a = (2 * (x >> 8) + 1 - (1 << 24)).astype(np.float32) * np.float32(2.0 ** -24) * np.float32(_S3_F32)
    return to_bf16_bits(a).reshape(n_tok, n_heads, dh)


def hashed_kv_torch(seed: int, stream: int, layer: int, kind: int, n_tok: int, n_heads: int, dh: int,
                    device, tok0: int = 0):
    """The same values as hashed_kv_np, generated by torch on `device` (bfloat16)."""
    import torch
    key = hashed_kv_key(seed, stream, layer, kind)
    x = torch.arange(tok0 * n_heads * dh, (tok0 + n_tok) * n_heads * dh, dtype=torch.int64, device=device)
    x = (x + key) & _M32_INT
    x = (((x >> 16) ^ x) * _HASH_MUL) & _M32_INT
    x = (((x >> 16) ^ x) * _HASH_MUL) & _M32_INT
    x = (x >> 16) ^ x
    a = (2 * (x >> 8) + 1 - (1 << 24)).to(torch.float32) * (2.0 ** -24) * _S3_F32
    return a.to(torch.bfloat16).reshape(n_tok, n_heads, dh)


class _HashedSide:
    def __init__(self, owner, kind):
        self.owner, self.kind = owner, kind

    def __getitem__(self, b):
        o = self.owner
        return [o.block(b, l, self.kind) for l in range(o.shape.n_layers)] if o.eager else _HashedRow(o, b, self.kind)

    def __len__(self):
        return len(self.owner.lens)


class _HashedRow:
    def __init__(self, owner, b, kind):
        self.owner, self.b, self.kind = owner, b, kind

    def __getitem__(self, l):
        return self.owner.block(self.b, l, self.kind)

    def __len__(self):
        return self.owner.shape.n_layers


class HashedKV:
    """Logical cache contents like KVCache (k[b][l], v[b][l] of shape [len_b, Hkv, dh]),
    generated on access from the hashed recipe: bf16 bit patterns on the host
    (device=None) or bfloat16 tensors on a torch device.  Stream of row b = streams[b]."""

    def __init__(self, shape: ModelShape, lens, capacity: int, seed: int, streams=None, device=None,
                 eager: bool = False):
        self.shape, self.lens, self.capacity, self.seed = shape, list(lens), capacity, seed
        self.streams = list(range(len(self.lens))) if streams is None else list(streams)
        self.device, self.eager = device, eager
        self.k, self.v = _HashedSide(self, 0), _HashedSide(self, 1)

    def block(self, b: int, l: int, kind: int):
        sh = self.shape
        n = self.lens[b]
        if self.device is None:
            return hashed_kv_np(self.seed, self.streams[b], l, kind, n, sh.n_kv_heads, sh.head_dim)
        return hashed_kv_torch(self.seed, self.streams[b], l, kind, n, sh.n_kv_heads, sh.head_dim, self.device)


def page_table(lens, capacity_extra: int, page: int, seed: int):
    """Per-row block tables over one shared pool of physical blocks, placed by a seeded
    permutation: row b owns ceil((lens[b] + capacity_extra) / page) blocks; unused
    table entries are -1.  Returns (table int32 [B, max_blocks], n_blocks)."""
    need = [(n + capacity_extra + page - 1) // page for n in lens]
    n_blocks = int(sum(need))
    perm = page_permutation(n_blocks, seed)
    table = np.full((len(lens), max(need)), -1, dtype=np.int32)
    at = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[at:at + nb]
        at += nb
    return table, n_blocks


def page_permutation(n_blocks: int, seed: int) -> np.ndarray:
    """Seeded permutation of physical KV blocks (fragmented placement)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _tensor_key("pages")])))
    return g.permutation(n_blocks).astype(np.int32)


def uniform_tokens(n: int, vocab: int, seed: int, tag: str = "audio") -> np.ndarray:
    """Tokens uniform on [1, vocab) (0 is reserved for the silence token)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _tensor_key(tag)])))
    return g.integers(1, vocab, size=n, dtype=np.int64).astype(np.int32)


# -- Philox4x32-10 (Salmon, Moraes, Dror, Shaw: "Parallel random numbers: as easy
#    as 1, 2, 3", SC'11): a 10-round counter-based generator, here vectorised
#    over many counters at once. -----------------------------------------------

_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = np.uint32(0x9E3779B9)
_PHILOX_W1 = np.uint32(0xBB67AE85)
_M32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """ctr: uint32 [..., 4]; key: uint32 [2] or [..., 2].  Returns uint32 [..., 4]."""
    c = [np.asarray(ctr[..., i], dtype=np.uint32).copy() for i in range(4)]
    key = np.asarray(key, dtype=np.uint32)
    k0 = np.broadcast_to(key[..., 0], c[0].shape).astype(np.uint32)
    k1 = np.broadcast_to(key[..., 1], c[0].shape).astype(np.uint32)
    for r in range(10):
        p0 = c[0].astype(np.uint64) * _PHILOX_M0
        p1 = c[2].astype(np.uint64) * _PHILOX_M1
        hi0, lo0 = (p0 >> np.uint64(32)).astype(np.uint32), (p0 & _M32).astype(np.uint32)
        hi1, lo1 = (p1 >> np.uint64(32)).astype(np.uint32), (p1 & _M32).astype(np.uint32)
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        if r < 9:
            k0 = ((k0.astype(np.uint64) + np.uint64(_PHILOX_W0)) & _M32).astype(np.uint32)
            k1 = ((k1.astype(np.uint64) + np.uint64(_PHILOX_W1)) & _M32).astype(np.uint32)
    return np.stack(c, axis=-1)


def philox_uniforms(seed: int, seq: np.ndarray, pos: np.ndarray, stream: int):
    """Two uniforms per (seq, pos) counter under key (seed): U0 = r0 * 2^-32 (acceptance
    test), U1 = 53-bit (r1 * 2^21 + r2 >> 11) * 2^-53 (sampling).  `stream` selects the
    fourth counter word so that independent draws never share a counter."""
    seq = np.asarray(seq, dtype=np.uint32)
    pos = np.asarray(pos, dtype=np.uint32)
    seq, pos = np.broadcast_arrays(seq, pos)
    ctr = np.stack([seq, pos, np.zeros_like(seq), np.full_like(seq, stream)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint32)
    r = philox4x32_10(ctr, key)
    u0 = r[..., 0].astype(np.float64) * 2.0 ** -32
    u1 = ((r[..., 1].astype(np.uint64) << np.uint64(21)) + (r[..., 2].astype(np.uint64) >> np.uint64(11))
          ).astype(np.float64) * 2.0 ** -53
    return u0, u1


# -- speculative-sampling inputs ------------------------------------------------

def _top1_of_temperature(zc: np.ndarray, tau: float) -> float:
    """zc: logits minus their maximum (fp32)."""
    e = np.exp(zc * np.float32(1.0 / tau))
    return float(1.0 / e.sum(dtype=np.float64))


def calibrate_temperature(z: np.ndarray, top1: float, iters: int = 30) -> float:
    """Bisection on log(tau) so that softmax(z / tau) has the given top-1 mass (to ~1e-6)."""
    zc = (z - z.max()).astype(np.float32)
    lo, hi = math.log(1e-4), math.log(1e3)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if _top1_of_temperature(zc, math.exp(mid)) > top1:
            lo = mid
        else:
            hi = mid
    return math.exp(0.5 * (lo + hi))


@dataclass
class SampleInputs:
    target_logits: np.ndarray   # fp32 [B, k+1, V]
    draft_logits: np.ndarray    # fp32 [B, k, V]
    drafts: np.ndarray          # int32 [B, k], x_i ~ q_i
    u_accept: np.ndarray        # fp64 [B, k]
    u_sample: np.ndarray        # fp64 [B, k+1]
    temperature: float = 1.0
    seed: int = 0               # Philox key of u_accept / u_sample (sequence b uses counter word b)


def make_sample_inputs(w: SampleWorkload, batch: Optional[int] = None, vocab: Optional[int] = None,
                       k: Optional[int] = None) -> SampleInputs:
    """Rows b < B/2 are peaked (top-1 mass w.peaked_top1), the rest flat (w.flat_top1).
    Draft logits add sigma * N(0,1) noise to the target logits; each draft token is
    drawn from softmax(draft logits) by the Gumbel-max construction."""
    B = batch or w.batch
    V = vocab or w.vocab
    k = k or w.k
    tl = np.empty((B, k + 1, V), dtype=np.float32)
    dl = np.empty((B, k, V), dtype=np.float32)
    drafts = np.empty((B, k), dtype=np.int32)

    def one(b):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, _tensor_key("spec"), b])))
        top1 = w.peaked_top1 if b < B // 2 else w.flat_top1
        for i in range(k + 1):
            z = g.standard_normal(V)
            tau = calibrate_temperature(z, top1)
            zp = (z / tau).astype(np.float32)
            tl[b, i] = zp
            if i < k:
                zq = (zp.astype(np.float64) + w.noise_sigma * g.standard_normal(V)).astype(np.float32)
                dl[b, i] = zq
                drafts[b, i] = int(np.argmax(zq.astype(np.float64) + g.gumbel(size=V)))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(B)))
    u0, _ = philox_uniforms(w.seed, np.arange(B)[:, None], np.arange(k)[None, :], stream=0)
    _, u1 = philox_uniforms(w.seed, np.arange(B)[:, None], np.arange(k + 1)[None, :], stream=1)
    return SampleInputs(tl, dl, drafts, u0, u1, seed=w.seed)
