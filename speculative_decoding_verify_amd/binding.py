"""Thin ctypes binding of libsdv (argument marshalling only).

Every step of the verify path runs in the HIP kernels of libsdv.so; PyTorch
provides device memory and the stream.  The library is loaded from this package
directory; if it is missing, loading raises instead of falling back to anything.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsdv.so")

SDV_F32, SDV_BF16 = 0, 1
PAGE = 16
MAX_T = 128

ERR_BITS = {0x1: "bad token", 0x2: "bad parent/logit row", 0x4: "cache overflow",
            0x8: "bad rollback move", 0x10: "duplicate sibling token"}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


PACK_PLAIN, PACK_QKV, PACK_GATE_UP = 0, 1, 2
HEAD_LM, HEAD_CODEBOOK = 0, 1


class SdvLayer(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("attn_norm", "wqkv", "wo", "ffn_norm", "wgu", "wd")]


class SdvModel(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("d", _i32), ("n_heads", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("ffn", _i32), ("vocab", _i32), ("dtype", _i32),
                ("eps", ctypes.c_float), ("rope_theta", ctypes.c_float),
                ("embed", _vp), ("final_norm", _vp), ("lm_head", _vp),
                ("layers", ctypes.POINTER(SdvLayer)),
                ("n_codebooks", _i32), ("codebook_size", _i32), ("codebook_base", _i32),
                ("codebook", _vp), ("stream_emb", _vp)]


class SdvKV(ctypes.Structure):
    _fields_ = [("k_pages", _vp), ("v_pages", _vp), ("block_table", _vp), ("seq_len", _vp),
                ("n_blocks", _i32), ("max_blocks", _i32), ("batch", _i32)]


class SdvVerifyIn(ctypes.Structure):
    _fields_ = [("batch", _i32), ("T", _i32), ("L_a", _i32), ("R", _i32), ("max_ctx", _i32),
                ("tokens", _vp), ("parent", _vp), ("logit_rows", _vp),
                ("head", _i32), ("cfg_partner", _vp), ("cfg_w", ctypes.c_float)]


class SdvVerifyOut(ctypes.Structure):
    _fields_ = [("logits", _vp), ("argmax", _vp), ("margin", _vp), ("lse", _vp),
                ("hidden", _vp), ("err", _vp), ("prof_events", ctypes.POINTER(_vp)),
                ("n_prof_events", _i32), ("cb_argmax", _vp),
                ("attn_prof_events", ctypes.POINTER(_vp)), ("n_attn_prof_events", _i32)]


class SdvDraftIn(ctypes.Structure):
    _fields_ = [("batch", _i32), ("L_a", _i32), ("n_branches", _i32), ("max_ctx", _i32),
                ("chunk", _vp), ("branch_len", ctypes.POINTER(_i32))]


class SdvPool(ctypes.Structure):
    _fields_ = [("tokens", _vp), ("seg_end", _vp), ("keys", _vp), ("vals", _vp), ("count", _vp),
                ("capacity", _i32), ("n_slots", _i32), ("max_n", _i32)]


class SdvStreamCfg(ctypes.Structure):
    _fields_ = [("n_codebooks", _i32), ("codebook_size", _i32), ("codebook_base", _i32), ("text_end", _i32),
                ("eoa_code", _i32), ("pad_code", _i32), ("n_bridge", _i32), ("max_frames", _i32), ("bridge", _vp)]


class SdvStreamState(ctypes.Structure):
    _fields_ = [("phase", _vp), ("phase_pos", _vp), ("step", _vp), ("frames", _vp), ("matrix", _vp)]


class SdvError(RuntimeError):
    pass


_LIB = None
ABI_VERSION = 9   # SDV_ABI_VERSION of include/sdv.h that these signatures follow


def lib():
    """Load libsdv.so (once).  Raises if it is not built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise SdvError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.sdv_abi_version.restype = _i32
        if L.sdv_abi_version() != ABI_VERSION:
            raise SdvError(f"{LIB_PATH} has ABI version {L.sdv_abi_version()}, this binding needs "
                           f"{ABI_VERSION}; rebuild with __graft_entry__.build()")
        L.sdv_last_error.restype = ctypes.c_char_p
        L.sdv_verify_workspace_size.restype = ctypes.c_size_t
        L.sdv_verify_workspace_size.argtypes = [ctypes.POINTER(SdvModel), _i32, _i32, _i32, _i32]
        L.sdv_verify_forward.restype = ctypes.c_int
        L.sdv_verify_forward.argtypes = [ctypes.POINTER(SdvModel), ctypes.POINTER(SdvKV),
                                         ctypes.POINTER(SdvVerifyIn), ctypes.POINTER(SdvVerifyOut),
                                         _vp, ctypes.c_size_t, _vp]
        L.sdv_verify_forward_noalloc.restype = ctypes.c_int
        L.sdv_verify_forward_noalloc.argtypes = [ctypes.POINTER(SdvModel), ctypes.POINTER(SdvKV),
                                                 ctypes.POINTER(SdvVerifyIn), ctypes.POINTER(SdvVerifyOut), _vp]
        L.sdv_draft_workspace_size.restype = ctypes.c_size_t
        L.sdv_draft_workspace_size.argtypes = [ctypes.POINTER(SdvModel), _i32, _i32, _i32, ctypes.POINTER(_i32), _i32]
        L.sdv_draft_tree.restype = ctypes.c_int
        L.sdv_draft_tree.argtypes = [ctypes.POINTER(SdvModel), ctypes.POINTER(SdvKV), ctypes.POINTER(SdvDraftIn),
                                     _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.sdv_pool_clear.restype = ctypes.c_int
        L.sdv_pool_clear.argtypes = [ctypes.POINTER(SdvPool), _vp]
        L.sdv_pool_insert.restype = ctypes.c_int
        L.sdv_pool_insert.argtypes = [ctypes.POINTER(SdvPool), _vp, _i32, _vp, _vp]
        L.sdv_pool_lookup.restype = ctypes.c_int
        L.sdv_pool_lookup.argtypes = [ctypes.POINTER(SdvPool), _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]
        L.sdv_phase_mask.restype = ctypes.c_int
        L.sdv_phase_mask.argtypes = [ctypes.POINTER(SdvStreamCfg), _i32, _i32, _vp, ctypes.c_int64, _i32, _i32, _vp,
                                     ctypes.POINTER(SdvStreamState), _vp, _vp, _vp]
        L.sdv_stream_commit.restype = ctypes.c_int
        L.sdv_stream_commit.argtypes = [ctypes.POINTER(SdvStreamCfg), _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, ctypes.POINTER(SdvStreamState), _vp]
        L.sdv_accept_greedy.restype = ctypes.c_int
        L.sdv_accept_greedy.argtypes = [_i32, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
        L.sdv_kv_rollback.restype = ctypes.c_int
        L.sdv_kv_rollback.argtypes = [ctypes.POINTER(SdvModel), ctypes.POINTER(SdvKV), _vp, _vp, _vp,
                                      _i32, _vp, _vp]
        L.sdv_sample_workspace_size.restype = ctypes.c_size_t
        L.sdv_sample_workspace_size.argtypes = [_i32, _i32, _i32]
        L.sdv_packed_bytes.restype = ctypes.c_size_t
        L.sdv_packed_bytes.argtypes = [_i32, _i32, _i32]
        L.sdv_pack_weights.restype = ctypes.c_int
        L.sdv_pack_weights.argtypes = [_i32, _i32, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _i32, _vp,
                                       ctypes.c_size_t, _vp]
        L.sdv_accept_sample.restype = ctypes.c_int
        L.sdv_accept_sample.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, ctypes.c_float, ctypes.c_uint64, _vp,
                                        _vp, _vp, _vp, _vp, ctypes.c_size_t, ctypes.POINTER(_vp), _vp]
        L.sdv_philox_uniforms.restype = ctypes.c_int
        L.sdv_philox_uniforms.argtypes = [ctypes.c_uint64, _vp, _i32, _i32, _vp, _vp, _vp]
        _LIB = L
    return _LIB


def _check(status: int, what: str) -> None:
    if status != 0:
        raise SdvError(f"{what} failed ({status}): {lib().sdv_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev_tensor(a, device) -> torch.Tensor:
    """numpy fp32 -> float32 tensor; numpy uint16 (bf16 bit patterns) -> bfloat16 tensor;
    a torch tensor is moved to `device` as it is."""
    if isinstance(a, torch.Tensor):
        return a.to(device)
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def pack_weights(kind: int, sources: Sequence[np.ndarray], head_dim: int = 0, device="cuda") -> torch.Tensor:
    """Upload row-major matrices (numpy: fp32, or uint16 bf16 bit patterns) and pack
    them on the device with sdv_pack_weights; returns the packed byte tensor."""
    dev = torch.device(device)
    srcs = [_dev_tensor(a, dev) for a in sources]
    K = int(sources[0].shape[1])
    dtype = SDV_BF16 if sources[0].dtype == np.uint16 else SDV_F32
    rows = [int(a.shape[0]) for a in sources] + [0] * (3 - len(sources))
    ptrs = [ctypes.c_void_p(t.data_ptr()) for t in srcs] + [None] * (3 - len(srcs))
    nbytes = lib().sdv_packed_bytes(dtype, sum(rows), K)
    if nbytes == 0:
        raise SdvError("sdv_packed_bytes rejected the shape")
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(lib().sdv_pack_weights(kind, dtype, K, head_dim, ptrs[0], rows[0], ptrs[1], rows[1], ptrs[2], rows[2],
                                  ctypes.c_void_p(dst.data_ptr()), nbytes, _stream()), "sdv_pack_weights")
    torch.cuda.current_stream().synchronize()  # the sources are freed on return
    return dst


class DeviceModel:
    """Decoder weights resident on the device (projections packed) plus the sdv_model descriptor."""

    def __init__(self, w, device="cuda"):
        sh = w.shape
        self.shape = sh
        self.device = torch.device(device)
        t = lambda a: _dev_tensor(a, self.device)
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.device)
        pk = lambda kind, srcs, hd=0: pack_weights(kind, srcs, hd, self.device)
        self.embed = t(w.embed)
        self.final_norm = f(w.final_norm)
        self.lm_head = pk(PACK_PLAIN, [w.lm_head])
        self.layers = []
        for lw in w.layers:
            self.layers.append(dict(attn_norm=f(lw.attn_norm),
                                    wqkv=pk(PACK_QKV, [lw.wq, lw.wk, lw.wv], sh.head_dim),
                                    wo=pk(PACK_PLAIN, [lw.wo]), ffn_norm=f(lw.ffn_norm),
                                    wgu=pk(PACK_GATE_UP, [lw.wg, lw.wu]), wd=pk(PACK_PLAIN, [lw.wd])))
        has_cb = getattr(w, "codebook", None) is not None and sh.n_codebooks > 0
        self.codebook = pk(PACK_PLAIN, [w.codebook]) if has_cb else None
        self.stream_emb = f(w.stream_emb) if has_cb else None
        # codebook 0's codes are the backbone ids after the text part of the vocabulary
        self.codebook_base = sh.vocab - sh.n_codebooks * sh.codebook_size if has_cb else 0
        self._build_desc()

    def _build_desc(self):
        sh = self.shape
        arr = (SdvLayer * sh.n_layers)()
        for i, L in enumerate(self.layers):
            for k, v in L.items():
                setattr(arr[i], k, v.data_ptr())
        self._layer_arr = arr
        self.desc = SdvModel(sh.n_layers, sh.d, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.ffn, sh.vocab,
                             SDV_BF16 if sh.dtype == "bf16" else SDV_F32, sh.eps, sh.rope_theta,
                             self.embed.data_ptr(), self.final_norm.data_ptr(), self.lm_head.data_ptr(),
                             ctypes.cast(arr, ctypes.POINTER(SdvLayer)),
                             sh.n_codebooks if self.codebook is not None else 0,
                             sh.codebook_size if self.codebook is not None else 0, self.codebook_base,
                             _ptr(self.codebook), _ptr(self.stream_emb))

    @property
    def weight_bytes(self) -> int:
        n = self.lm_head.numel() * self.lm_head.element_size()
        for L in self.layers:
            for k, v in L.items():
                n += v.numel() * v.element_size()
        return n


class PagedKV:
    """Paged cache: k_pages [L][n_blocks][Hkv][16][dh], v_pages [L][n_blocks][Hkv][dh][16],
    block_table [B, max_blocks], seq_len [B]."""

    def __init__(self, shape, batch: int, capacity: int, device="cuda", perm: Optional[np.ndarray] = None,
                 n_blocks: Optional[int] = None, table: Optional[np.ndarray] = None):
        """table: optional int32 [batch, max_blocks] block table (-1 = unused entry) over
        n_blocks physical blocks, for rows of different capacities."""
        self.shape = shape
        self.device = torch.device(device)
        self.batch = batch
        self.max_blocks = (capacity + PAGE - 1) // PAGE if table is None else int(table.shape[1])
        self.n_blocks = n_blocks or batch * self.max_blocks
        dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
        L, Hkv, dh = shape.n_layers, shape.n_kv_heads, shape.head_dim
        self.k_pages = torch.zeros((L, self.n_blocks, Hkv, PAGE, dh), dtype=dt, device=self.device)
        self.v_pages = torch.zeros((L, self.n_blocks, Hkv, dh, PAGE), dtype=dt, device=self.device)
        if table is not None:
            self.block_table = torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(self.device)
        else:
            ids = np.arange(batch * self.max_blocks, dtype=np.int32) if perm is None else np.asarray(perm, np.int32)
            self.block_table = torch.from_numpy(ids[:batch * self.max_blocks].reshape(batch, self.max_blocks).copy()).to(self.device)
        self.seq_len = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.desc = SdvKV(self.k_pages.data_ptr(), self.v_pages.data_ptr(), self.block_table.data_ptr(),
                          self.seq_len.data_ptr(), self.n_blocks, self.max_blocks, batch)

    def load(self, kv) -> None:
        """Write logical cache contents (synth KVCache: k[b][l] [len, Hkv, dh]) into the pages."""
        sh = self.shape
        lens = list(kv.lens)
        bt = self.block_table.cpu().numpy()
        for b, n in enumerate(lens):
            nb = (n + PAGE - 1) // PAGE
            if nb == 0:
                continue
            pages = torch.from_numpy(bt[b, :nb].astype(np.int64)).to(self.device)
            for l in range(sh.n_layers):
                for src, dst, vt in ((kv.k[b][l], self.k_pages, False), (kv.v[b][l], self.v_pages, True)):
                    x = _dev_tensor(src, self.device)
                    pad = torch.zeros((nb * PAGE, sh.n_kv_heads, sh.head_dim), dtype=x.dtype, device=self.device)
                    pad[:n] = x
                    pg = pad.view(nb, PAGE, sh.n_kv_heads, sh.head_dim)
                    pg = pg.permute(0, 2, 3, 1) if vt else pg.permute(0, 2, 1, 3)
                    dst[l, pages] = pg.contiguous()
        self.seq_len.copy_(torch.tensor(lens, dtype=torch.int32))

    def gather(self, b: int, l: int, lo: int, hi: int):
        """Logical slots [lo, hi) of sequence b, layer l as (k, v) fp32 [n, Hkv, dh] tensors."""
        slots = torch.arange(lo, hi, device=self.device)
        bt = self.block_table[b].long()
        pg = bt[slots // PAGE]
        off = slots % PAGE
        k = self.k_pages[l, pg, :, off, :]           # [n, Hkv, dh]
        v = self.v_pages[l, pg, :, :, off]           # [n, Hkv, dh]
        return k.float(), v.float()


@dataclass
class VerifyResult:
    argmax: torch.Tensor
    margin: torch.Tensor
    lse: torch.Tensor
    err: torch.Tensor
    logits: Optional[torch.Tensor] = None
    hidden: Optional[torch.Tensor] = None
    cb_argmax: Optional[torch.Tensor] = None


class Verifier:
    """Holds the device-side inputs and outputs of verify passes of one shape, so that
    repeated passes (and graph capture) reuse the same buffers."""

    def __init__(self, model: DeviceModel, kv: PagedKV, T: int, L_a: int, logit_rows: Sequence[int],
                 parent: Optional[Sequence[int]] = None, max_ctx: Optional[int] = None,
                 want_logits: bool = True, want_hidden: bool = False, head: int = HEAD_LM,
                 cfg_partner: Optional[Sequence[int]] = None, cfg_w: float = 1.0):
        self.model, self.kv = model, kv
        dev = model.device
        B = kv.batch
        self.B, self.T, self.L_a = B, T, L_a
        self.R = len(logit_rows)
        self.max_ctx = int(max_ctx if max_ctx is not None else kv.max_blocks * PAGE - T)
        self.tokens = torch.zeros((B, T), dtype=torch.int32, device=dev)
        self.logit_rows = torch.tensor(list(logit_rows), dtype=torch.int32, device=dev)
        self.parent = None if parent is None else torch.tensor(list(parent), dtype=torch.int32, device=dev)
        V = model.shape.vocab
        sh = model.shape
        self.head = head
        lshape = (B, self.R, V) if head == HEAD_LM else (B, self.R, sh.n_codebooks, sh.codebook_size)
        self.logits = torch.empty(lshape, dtype=torch.float32, device=dev) if want_logits else None
        self.cb_argmax = (torch.empty((B, self.R, sh.n_codebooks), dtype=torch.int32, device=dev)
                          if head == HEAD_CODEBOOK else None)
        self.cfg_partner = (None if cfg_partner is None
                            else torch.tensor(list(cfg_partner), dtype=torch.int32, device=dev))
        self.hidden = torch.empty((B, T, model.shape.d), dtype=torch.float32, device=dev) if want_hidden else None
        self.argmax = torch.empty((B, self.R), dtype=torch.int32, device=dev)
        self.margin = torch.empty((B, self.R), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, self.R), dtype=torch.float32, device=dev)
        self.err = torch.zeros(B, dtype=torch.int32, device=dev)
        nbytes = lib().sdv_verify_workspace_size(ctypes.byref(model.desc), B, T, self.R, self.max_ctx)
        if nbytes == 0:
            raise SdvError("unsupported verify shape: " + lib().sdv_last_error().decode())
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.inp = SdvVerifyIn(B, T, L_a, self.R, self.max_ctx, self.tokens.data_ptr(),
                               None if self.parent is None else self.parent.data_ptr(),
                               self.logit_rows.data_ptr(), head, _ptr(self.cfg_partner), float(cfg_w))
        self.out = SdvVerifyOut(_ptr(self.logits), self.argmax.data_ptr(), self.margin.data_ptr(),
                                self.lse.data_ptr(), _ptr(self.hidden), self.err.data_ptr(), None, 0,
                                _ptr(self.cb_argmax), None, 0)

    def set_profile_events(self, events, attn_events=None) -> None:
        """events: list of torch.cuda.Event (enable_timing=True), recorded by the library
        in pairs around its GEMM launches; attn_events likewise around each layer's
        attention; None disables."""
        self._prof = []
        for evs, fp, fn in ((events, "prof_events", "n_prof_events"),
                            (attn_events, "attn_prof_events", "n_attn_prof_events")):
            if not evs:
                setattr(self.out, fp, None)
                setattr(self.out, fn, 0)
                continue
            for e in evs:          # torch creates the underlying event on first record
                e.record()
            arr = (_vp * len(evs))(*[e.cuda_event for e in evs])
            self._prof.append((evs, arr))
            setattr(self.out, fp, ctypes.cast(arr, ctypes.POINTER(_vp)))
            setattr(self.out, fn, len(evs))

    def set_tokens(self, tokens) -> None:
        t = torch.as_tensor(np.asarray(tokens, dtype=np.int32).reshape(self.B, self.T))
        self.tokens.copy_(t)

    def forward(self, stream=None, noalloc: bool = False) -> VerifyResult:
        """noalloc: call sdv_verify_forward_noalloc (the library's static scratch) instead
        of passing this Verifier's workspace."""
        if noalloc:
            _check(lib().sdv_verify_forward_noalloc(ctypes.byref(self.model.desc), ctypes.byref(self.kv.desc),
                                                    ctypes.byref(self.inp), ctypes.byref(self.out), _stream(stream)),
                   "sdv_verify_forward_noalloc")
        else:
            _check(lib().sdv_verify_forward(ctypes.byref(self.model.desc), ctypes.byref(self.kv.desc),
                                            ctypes.byref(self.inp), ctypes.byref(self.out),
                                            ctypes.c_void_p(self.workspace.data_ptr()), self.workspace.numel(),
                                            _stream(stream)), "sdv_verify_forward")
        return VerifyResult(self.argmax, self.margin, self.lse, self.err, self.logits, self.hidden, self.cb_argmax)


class Drafter:
    """Idle-window drafting (sdv_draft_tree) with reusable buffers: branch k of the tree
    starts from the (k+1)-th ranked first token under the hypothesised chunk and is
    continued greedily to branch_len[k] tokens."""

    def __init__(self, model: DeviceModel, kv: PagedKV, L_a: int, branch_len: Sequence[int],
                 max_ctx: Optional[int] = None):
        self.model, self.kv = model, kv
        dev = model.device
        B = kv.batch
        self.B, self.L_a, self.K = B, L_a, len(branch_len)
        self.branch_len = list(int(x) for x in branch_len)
        self.max_len = max(self.branch_len)
        self._len = (_i32 * self.K)(*self.branch_len)
        self.max_ctx = int(max_ctx if max_ctx is not None else kv.max_blocks * PAGE - L_a - 1)
        self.chunk = torch.zeros((B, L_a), dtype=torch.int32, device=dev)
        self.drafts = torch.empty((B, self.K, self.max_len), dtype=torch.int32, device=dev)
        self.err = torch.zeros(B, dtype=torch.int32, device=dev)
        nbytes = lib().sdv_draft_workspace_size(ctypes.byref(model.desc), B, L_a, self.K, self._len, self.max_ctx)
        if nbytes == 0:
            raise SdvError("unsupported drafting shape: " + lib().sdv_last_error().decode())
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.inp = SdvDraftIn(B, L_a, self.K, self.max_ctx, self.chunk.data_ptr(), self._len)

    def set_chunk(self, tokens) -> None:
        self.chunk.copy_(torch.as_tensor(np.asarray(tokens, dtype=np.int32).reshape(self.B, self.L_a)))

    def run(self, stream=None) -> dict:
        _check(lib().sdv_draft_tree(ctypes.byref(self.model.desc), ctypes.byref(self.kv.desc), ctypes.byref(self.inp),
                                    _ptr(self.drafts), _ptr(self.err), _ptr(self.workspace), self.workspace.numel(),
                                    _stream(stream)), "sdv_draft_tree")
        return {"drafts": self.drafts, "err": self.err}


class HypothesisPool:
    """Device-resident hypothesis pool (sdv_pool_*): drafts stored in insertion order and
    indexed by their n-grams, n = 1..max_n."""

    def __init__(self, capacity: int, n_slots: int, max_n: int = 8, device="cuda"):
        dev = torch.device(device)
        self.tokens = torch.empty(capacity, dtype=torch.int32, device=dev)
        self.seg_end = torch.empty(capacity, dtype=torch.int32, device=dev)
        self.keys = torch.empty(n_slots, dtype=torch.int64, device=dev)
        self.vals = torch.empty(n_slots, dtype=torch.int32, device=dev)
        self.count = torch.empty(1, dtype=torch.int32, device=dev)
        self.err = torch.zeros(1, dtype=torch.int32, device=dev)
        self.max_n = max_n
        self.desc = SdvPool(self.tokens.data_ptr(), self.seg_end.data_ptr(), self.keys.data_ptr(),
                            self.vals.data_ptr(), self.count.data_ptr(), capacity, n_slots, max_n)
        self.clear()

    def clear(self, stream=None) -> None:
        _check(lib().sdv_pool_clear(ctypes.byref(self.desc), _stream(stream)), "sdv_pool_clear")

    def insert(self, draft: torch.Tensor, stream=None) -> None:
        """draft: int32 device tensor [len]."""
        _check(lib().sdv_pool_insert(ctypes.byref(self.desc), _ptr(draft), int(draft.numel()), _ptr(self.err),
                                     _stream(stream)), "sdv_pool_insert")

    def lookup(self, suffix: torch.Tensor, suffix_len: torch.Tensor, max_out: int, stream=None):
        """suffix int32 [B, cap], suffix_len int32 [B] (device).  Returns (cont [B, max_out],
        cont_len [B], match_n [B]) device tensors."""
        B, cap = suffix.shape
        dev = suffix.device
        cont = torch.empty((B, max_out), dtype=torch.int32, device=dev)
        clen = torch.empty(B, dtype=torch.int32, device=dev)
        mn = torch.empty(B, dtype=torch.int32, device=dev)
        _check(lib().sdv_pool_lookup(ctypes.byref(self.desc), B, _ptr(suffix), _ptr(suffix_len), cap, max_out,
                                     _ptr(cont), _ptr(clen), _ptr(mn), _stream(stream)), "sdv_pool_lookup")
        return cont, clen, mn


PHASE_TEXT, PHASE_TRANSITION, PHASE_AUDIO, PHASE_DRAIN = 0, 1, 2, 3
MOD_TEXT, MOD_AUDIO, MOD_OTHER = 0, 1, 2


class Streams:
    """Per-session multi-codebook stream state (phase machine and delay-pattern code
    matrix) with the phase mask and the commit of sdv_stream_commit."""

    def __init__(self, B: int, n_codebooks: int, codebook_size: int, codebook_base: int, text_end: int,
                 eoa_code: int, pad_code: int, bridge: Sequence[int], max_frames: int, device="cuda"):
        dev = torch.device(device)
        self.B, self.S, self.max_frames = B, n_codebooks, max_frames
        self.bridge = torch.tensor(list(bridge) or [0], dtype=torch.int32, device=dev)
        self.cfg = SdvStreamCfg(n_codebooks, codebook_size, codebook_base, text_end, eoa_code, pad_code,
                                len(bridge), max_frames, self.bridge.data_ptr())
        self.phase = torch.zeros(B, dtype=torch.int32, device=dev)
        self.phase_pos = torch.zeros(B, dtype=torch.int32, device=dev)
        self.step = torch.zeros(B, dtype=torch.int32, device=dev)
        self.frames = torch.full((B,), -1, dtype=torch.int32, device=dev)
        self.matrix = torch.full((B, n_codebooks, max_frames), -1, dtype=torch.int32, device=dev)
        self.state = SdvStreamState(self.phase.data_ptr(), self.phase_pos.data_ptr(), self.step.data_ptr(),
                                    self.frames.data_ptr(), self.matrix.data_ptr())

    def mask(self, logits: torch.Tensor, depth: torch.Tensor, id_offset: int = 0, stream=None):
        """logits fp32 [B, R, n_ids] (contiguous rows); returns (argmax [B, R], modality [B, R])."""
        B, R, n = logits.shape
        am = torch.empty((B, R), dtype=torch.int32, device=logits.device)
        mod = torch.empty((B, R), dtype=torch.int32, device=logits.device)
        _check(lib().sdv_phase_mask(ctypes.byref(self.cfg), B, R, _ptr(logits), n, id_offset, n, _ptr(depth),
                                    ctypes.byref(self.state), _ptr(am), _ptr(mod), _stream(stream)), "sdv_phase_mask")
        return am, mod

    def commit(self, T: int, L_a: int, tokens: torch.Tensor, logit_rows: torch.Tensor, acc: dict,
               cb_argmax: Optional[torch.Tensor], modality: Optional[torch.Tensor], stream=None) -> None:
        _check(lib().sdv_stream_commit(ctypes.byref(self.cfg), self.B, T, L_a, logit_rows.numel(), _ptr(tokens),
                                       _ptr(logit_rows), _ptr(acc["n"]), _ptr(acc["next"]), _ptr(acc["path"]),
                                       _ptr(cb_argmax), _ptr(modality), ctypes.byref(self.state), _stream(stream)),
               "sdv_stream_commit")


def tree_parent(L_a: int, branch_lens: Sequence[int]) -> List[int]:
    """Parents of a verify chunk [audio (L_a rows); branch 0; branch 1; ...]: the audio
    rows form a chain, every branch is a chain whose first row hangs under the last
    audio row."""
    par = [j - 1 for j in range(L_a)]
    at = L_a
    for n in branch_lens:
        for i in range(n):
            par.append(L_a - 1 if i == 0 else at + i - 1)
        at += n
    return par


def accept_greedy(B: int, T: int, L_a: int, tokens: torch.Tensor, parent: Optional[torch.Tensor],
                  logit_rows: torch.Tensor, argmax: torch.Tensor, base_len: Optional[torch.Tensor] = None,
                  out: Optional[dict] = None, stream=None) -> dict:
    dev = tokens.device
    R = logit_rows.numel()
    if out is None:
        out = dict(n=torch.empty(B, dtype=torch.int32, device=dev), next=torch.empty(B, dtype=torch.int32, device=dev),
                   path=torch.empty((B, T), dtype=torch.int32, device=dev),
                   err=torch.zeros(B, dtype=torch.int32, device=dev))
        if base_len is not None:
            out.update(keep=torch.empty(B, dtype=torch.int32, device=dev),
                       move_src=torch.empty((B, T), dtype=torch.int32, device=dev),
                       move_dst=torch.empty((B, T), dtype=torch.int32, device=dev))
    _check(lib().sdv_accept_greedy(B, T, L_a, _ptr(tokens), _ptr(parent), R, _ptr(logit_rows), _ptr(argmax),
                                   _ptr(base_len), _ptr(out["n"]), _ptr(out["next"]), _ptr(out["path"]),
                                   _ptr(out.get("keep")), _ptr(out.get("move_src")), _ptr(out.get("move_dst")),
                                   _ptr(out["err"]), _stream(stream)), "sdv_accept_greedy")
    return out


def kv_rollback(model: DeviceModel, kv: PagedKV, keep_len: torch.Tensor, move_src: Optional[torch.Tensor] = None,
                move_dst: Optional[torch.Tensor] = None, err: Optional[torch.Tensor] = None, stream=None) -> None:
    max_move = 0 if move_src is None else move_src.shape[-1]
    _check(lib().sdv_kv_rollback(ctypes.byref(model.desc), ctypes.byref(kv.desc), _ptr(keep_len), _ptr(move_src),
                                 _ptr(move_dst), max_move, _ptr(err), _stream(stream)), "sdv_kv_rollback")


def prefill(model: DeviceModel, kv: PagedKV, tokens, chunk: int = MAX_T, stream=None) -> None:
    """Append `tokens` [B, n] to the cache through verify passes of at most `chunk` rows,
    committing each chunk (chunked prefill; every sequence starts at the same length)."""
    tokens = np.asarray(tokens, dtype=np.int32)
    B, n = tokens.shape
    start = int(kv.seq_len.max().item())
    done = 0
    while done < n:
        t = min(chunk, n - done)
        ver = Verifier(model, kv, t, t, [t - 1], max_ctx=start + done, want_logits=False)
        ver.set_tokens(tokens[:, done:done + t])
        ver.forward(stream)
        done += t
        keep = torch.full((B,), start + done, dtype=torch.int32, device=model.device)
        kv_rollback(model, kv, keep, stream=stream)


SAMPLE_NEAR_ACCEPT, SAMPLE_NEAR_DRAW, SAMPLE_BAD_DRAFT = 0x1, 0x2, 0x100


class Sampler:
    """Speculative-sampling acceptance with reusable workspace and outputs."""

    def __init__(self, B: int, k: int, V: int, device="cuda"):
        self.B, self.k, self.V = B, k, V
        nbytes = lib().sdv_sample_workspace_size(B, k, V)
        if nbytes == 0:
            raise SdvError(f"unsupported sampling shape B={B} k={k} V={V}")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.n = torch.empty(B, dtype=torch.int32, device=device)
        self.tok = torch.empty(B, dtype=torch.int32, device=device)
        self.flags = torch.empty(B, dtype=torch.int32, device=device)   # uint32 bits

    def __call__(self, tgt: torch.Tensor, drf: torch.Tensor, drafts: torch.Tensor, seed: int,
                 seq_ids: Optional[torch.Tensor] = None, temperature: float = 1.0, stream=None,
                 prof_events=None):
        """Returns (n, tok, flags) device tensors.  prof_events: None or two
        torch.cuda.Event (enable_timing=True) that the library records around its
        row-statistics launch."""
        ev = None
        if prof_events is not None:
            if len(prof_events) != 2:
                raise ValueError("prof_events takes exactly two events")
            for e in prof_events:     # torch creates the underlying event on first record
                e.record()
            ev = (_vp * 2)(*[e.cuda_event for e in prof_events])
        _check(lib().sdv_accept_sample(self.B, self.k, self.V, _ptr(tgt), _ptr(drf), _ptr(drafts),
                                       float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(seq_ids),
                                       _ptr(self.n), _ptr(self.tok), _ptr(self.flags),
                                       _ptr(self.workspace), self.workspace.numel(),
                                       None if ev is None else ctypes.cast(ev, ctypes.POINTER(_vp)),
                                       _stream(stream)),
               "sdv_accept_sample")
        return self.n, self.tok, self.flags


def philox_uniforms(seed: int, B: int, n_pos: int, seq_ids: Optional[torch.Tensor] = None, device="cuda",
                    stream=None):
    """(u0, u1) fp64 [B, n_pos] device tensors from sdv_philox_uniforms."""
    u0 = torch.empty((B, n_pos), dtype=torch.float64, device=device)
    u1 = torch.empty((B, n_pos), dtype=torch.float64, device=device)
    _check(lib().sdv_philox_uniforms(int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(seq_ids), B, n_pos, _ptr(u0), _ptr(u1),
                                     _stream(stream)), "sdv_philox_uniforms")
    return u0, u1
