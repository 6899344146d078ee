"""Model shapes and verify workloads used by tests, the bench and the CPU baseline.

Every workload is synthetic and seeded.  The shapes follow the decoder families
named for the verify step of "Decode Before You Hear: Speculative Listening"
(page 1, section "Method steps", step 4): a decoder with a KV cache of length C
ingests an audio chunk of L_a tokens plus a greedy draft of gamma tokens (and,
optionally, a runner-up branch that forks at the first draft position, step 2)
in one forward pass.

This module holds sizes and recipes only; it contains none of the method's
arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    dtype: str  # "f32" or "bf16": storage type of weights and KV cache
    eps: float = 1e-6
    rope_theta: float = 10000.0
    # codebook heads (multi-codebook audio output); 0 means none
    n_codebooks: int = 0
    codebook_size: int = 0

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def layer_params(self) -> int:
        d, f = self.d, self.ffn
        return (self.q_dim * d + 2 * self.kv_dim * d + d * self.q_dim
                + 3 * d * f + 2 * d)


@dataclass(frozen=True)
class VerifyWorkload:
    """One verify pass: B sequences, each with a cache of ctx[b] tokens.

    Rows 0..L_a-1 of the chunk are audio tokens, the following gamma rows the
    main draft; n_branch more rows form a runner-up branch whose first row
    is a sibling of the first draft row (both children of the last audio row).
    """
    shape: ModelShape
    batch: int
    ctx: Tuple[int, ...]          # cached length per sequence
    L_a: int
    gamma: int
    n_branch: int = 0
    seed: int = 0
    silence_id: int = 0
    page: int = 16                # tokens per KV page
    kv_init: str = "random"       # "random": synthetic unit-variance KV; "prefill": run tokens through the model;
                                  # "hashed": the coordinate-hashed unit-variance KV (generated on the device)
    cfg_pairs: bool = False       # rows 2i (conditional) and 2i+1 (unconditional) form CFG pairs
    cfg_w: float = 2.0

    @property
    def T(self) -> int:
        return self.L_a + self.gamma + self.n_branch

    @property
    def R(self) -> int:
        # rows whose distributions acceptance needs: last audio row and every draft row
        return self.T - self.L_a + 1

    def logit_rows(self):
        return list(range(self.L_a - 1, self.T))

    def parent(self) -> Optional[list]:
        """Tree parents (row -> parent row, -1 for row 0) or None for a plain chain."""
        if self.n_branch == 0:
            return None
        par = [j - 1 for j in range(self.T)]
        par[0] = -1
        b0 = self.L_a + self.gamma
        par[b0] = self.L_a - 1
        return par


# -- the decoder shapes -------------------------------------------------------

TOY_F32 = ModelShape("toy-f32", n_layers=2, d=256, n_heads=4, n_kv_heads=4, head_dim=64,
                     ffn=1024, vocab=4096, dtype="f32")
SHAPE_1P7B = ModelShape("1.7b-bf16", n_layers=24, d=2048, n_heads=32, n_kv_heads=32,
                        head_dim=64, ffn=8192, vocab=49152, dtype="bf16")
SHAPE_8B = ModelShape("8b-bf16", n_layers=36, d=4096, n_heads=32, n_kv_heads=8,
                      head_dim=128, ffn=12288, vocab=151936, dtype="bf16")
SHAPE_8B_CB = replace(SHAPE_8B, name="8b-bf16-codebook", n_codebooks=8, codebook_size=1024)

# small shapes for parity tests: several tiles plus ragged tails everywhere
MINI_BF16 = ModelShape("mini-bf16", n_layers=2, d=320, n_heads=6, n_kv_heads=2, head_dim=64,
                       ffn=704, vocab=3001, dtype="bf16")
MINI_BF16_D128 = ModelShape("mini-bf16-dh128", n_layers=2, d=512, n_heads=4, n_kv_heads=2,
                            head_dim=128, ffn=640, vocab=2053, dtype="bf16")
MINI_F32 = ModelShape("mini-f32", n_layers=2, d=192, n_heads=3, n_kv_heads=1, head_dim=64,
                      ffn=448, vocab=1537, dtype="f32")
# the 1.7B model width on a small vocabulary (parity at d = 2048 in seconds)
MINI_BF16_D2048 = ModelShape("mini-bf16-d2048", n_layers=3, d=2048, n_heads=16, n_kv_heads=4, head_dim=128,
                             ffn=4096, vocab=1009, dtype="bf16")
MINI_F32_D2048 = ModelShape("mini-f32-d2048", n_layers=3, d=2048, n_heads=16, n_kv_heads=4, head_dim=128,
                            ffn=4096, vocab=1009, dtype="f32")

# the 8B FFN width on a narrow model: 2 x 12288 gate/up rows = 1536 packed tiles
MINI_BF16_FFN12K = ModelShape("mini-bf16-ffn12288", n_layers=2, d=256, n_heads=4, n_kv_heads=2, head_dim=64,
                              ffn=12288, vocab=2003, dtype="bf16")
MINI_F32_FFN12K = ModelShape("mini-f32-ffn12288", n_layers=2, d=256, n_heads=4, n_kv_heads=2, head_dim=64,
                             ffn=12288, vocab=2003, dtype="f32")

# a vocabulary of 70,001 (4376 packed LM-head tiles): with more than 80 logit rows the LM
# head takes the tiled kernel at 8 tile columns per wave
MINI_BF16_V70K = ModelShape("mini-bf16-v70001", n_layers=1, d=256, n_heads=4, n_kv_heads=2, head_dim=64,
                            ffn=512, vocab=70001, dtype="bf16")
MINI_F32_V70K = ModelShape("mini-f32-v70001", n_layers=1, d=256, n_heads=4, n_kv_heads=2, head_dim=64,
                           ffn=512, vocab=70001, dtype="f32")

SHAPES = {s.name: s for s in (TOY_F32, SHAPE_1P7B, SHAPE_8B, SHAPE_8B_CB,
                              MINI_BF16, MINI_BF16_D128, MINI_F32, MINI_BF16_D2048, MINI_F32_D2048,
                              MINI_BF16_FFN12K, MINI_F32_FFN12K, MINI_BF16_V70K, MINI_F32_V70K)}


# -- the verify workloads --------------------------------------------------------

def toy_workload(seed: int = 1) -> VerifyWorkload:
    """Toy fp32 decoder: cache prefilled from 512 uniform tokens; 12 audio + 8 drafts."""
    return VerifyWorkload(TOY_F32, batch=1, ctx=(512,), L_a=12, gamma=8, seed=seed,
                          kv_init="prefill")


def w1p7b_workload(seed: int = 2) -> VerifyWorkload:
    """1.7B-shape bf16 decoder, context 4096; 25 audio tokens (1 s at 25 Hz) + 16 drafts."""
    return VerifyWorkload(SHAPE_1P7B, batch=1, ctx=(4096,), L_a=25, gamma=16, seed=seed)


def w8b_tree_workload(seed: int = 3) -> VerifyWorkload:
    """8B-shape bf16 decoder, context 8192; 25 audio + 32 drafts + an 8-token runner-up branch."""
    return VerifyWorkload(SHAPE_8B, batch=1, ctx=(8192,), L_a=25, gamma=32, n_branch=8, seed=seed)


def c5_contexts(seed: int = 5, sessions: int = 32, lo: int = 2048, hi: int = 16384):
    """Cached lengths of the batched multi-codebook workload: one seeded integer in
    [lo, hi] per session, shared by the session's conditional and unconditional rows."""
    import numpy as np
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xC5])))
    per = g.integers(lo, hi + 1, size=sessions)
    return tuple(int(c) for c in np.repeat(per, 2))


def c5_workload(seed: int = 5) -> VerifyWorkload:
    """8B-shape backbone with 8 codebook heads of 1024: 32 sessions x (conditional,
    unconditional) rows, contexts in [2048, 16384], 25 audio + 16 draft codes per
    session, guidance weight 2; acceptance on codebook 0."""
    return VerifyWorkload(SHAPE_8B_CB, batch=64, ctx=c5_contexts(seed), L_a=25, gamma=16, seed=seed,
                          kv_init="hashed", cfg_pairs=True, cfg_w=2.0)


WORKLOADS = {
    "toy-f32": toy_workload,
    "1.7b-bf16": w1p7b_workload,
    "8b-bf16-tree": w8b_tree_workload,
    "c5-codebook": c5_workload,
}


@dataclass(frozen=True)
class SampleWorkload:
    """Speculative-sampling acceptance alone: B sequences x k draft positions over V."""
    batch: int = 64
    k: int = 7
    vocab: int = 151936
    seed: int = 4
    peaked_top1: float = 0.9
    flat_top1: float = 0.2
    noise_sigma: float = 0.5


SAMPLE_FULL = SampleWorkload()
