"""sdv_verify_forward_noalloc (the verify forward on the library's static scratch)
against sdv_verify_forward with a caller workspace, through the C ABI: identical
logits, statistics, hidden rows and written K/V pages, on two calls in a row where
the second pass is smaller than the first."""
import ctypes

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_verify_amd as sdv  # noqa: E402
from speculative_decoding_verify_amd import binding  # noqa: E402
from synth import MINI_BF16, MINI_F32, make_weights, make_random_kv, uniform_tokens  # noqa: E402


def _outputs(ver, res):
    out = [res.logits, res.argmax, res.margin, res.lse, res.hidden, res.err]
    return [t.clone() for t in out]


def _pass(model, shape, lens, L_a, gamma, seed):
    T = L_a + gamma
    kv_host = make_random_kv(shape, lens, capacity=max(lens) + T, seed=seed)
    kv = sdv.PagedKV(shape, len(lens), max(lens) + T + 16)
    kv.load(kv_host)
    ver = sdv.Verifier(model, kv, T, L_a, list(range(L_a - 1, T)), max_ctx=max(lens), want_hidden=True)
    toks = np.stack([uniform_tokens(T, shape.vocab, seed + b, "nx") for b in range(len(lens))])
    ver.set_tokens(toks)
    return ver, kv


def _compare(ver, kv):
    """Workspace entry first, then the no-alloc entry with fresh outputs; the pages the
    first call wrote are restored before the second so both start from the same cache."""
    k0, v0 = kv.k_pages.clone(), kv.v_pages.clone()
    ref = _outputs(ver, ver.forward())
    k1, v1 = kv.k_pages.clone(), kv.v_pages.clone()
    kv.k_pages.copy_(k0)
    kv.v_pages.copy_(v0)
    for t in (ver.logits, ver.margin, ver.lse, ver.hidden):
        t.fill_(float("nan"))
    ver.argmax.fill_(-7)
    ver.err.zero_()
    got = _outputs(ver, ver.forward(noalloc=True))
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float32 else a,
                           b.view(torch.uint8) if b.dtype == torch.float32 else b)
    assert torch.equal(kv.k_pages.view(torch.uint8), k1.view(torch.uint8))
    assert torch.equal(kv.v_pages.view(torch.uint8), v1.view(torch.uint8))
    assert int(ver.err.abs().sum()) == 0


@pytest.mark.parametrize("shape", [MINI_BF16, MINI_F32], ids=lambda s: s.name)
def test_noalloc_matches_workspace_entry_on_two_calls(shape):
    model = sdv.DeviceModel(make_weights(shape, seed=401))
    ver, kv = _pass(model, shape, [700, 133, 419], L_a=9, gamma=21, seed=402)     # 3 x 30 rows
    _compare(ver, kv)
    ver2, kv2 = _pass(model, shape, [57], L_a=3, gamma=4, seed=403)               # 1 x 7 rows
    _compare(ver2, kv2)


def test_noalloc_rejects_a_pass_beyond_its_scratch():
    """The batched codebook pass needs far more than the static scratch: the call returns
    SDV_ERR_WORKSPACE before anything is enqueued (checked on a descriptor whose device
    pointers are never touched)."""
    from synth import SHAPE_8B_CB
    sh = SHAPE_8B_CB
    lay = (binding.SdvLayer * sh.n_layers)()
    for i in range(sh.n_layers):
        for f in ("attn_norm", "wqkv", "wo", "ffn_norm", "wgu", "wd"):
            setattr(lay[i], f, 256)
    m = binding.SdvModel(sh.n_layers, sh.d, sh.n_heads, sh.n_kv_heads, sh.head_dim, sh.ffn, sh.vocab, 1, sh.eps,
                         sh.rope_theta, 256, 256, 256, ctypes.cast(lay, ctypes.POINTER(binding.SdvLayer)),
                         8, 1024, sh.vocab - 8192, 256, 256)
    kvd = binding.SdvKV(256, 256, 256, 256, 64 * 1100, 1100, 64)
    inp = binding.SdvVerifyIn(64, 41, 25, 17, 16384, 256, None, 256, 1, None, 2.0)
    out = binding.SdvVerifyOut(None, 256, 256, 256, None, 256, None, 0, 256)
    L = sdv.lib()
    need = L.sdv_verify_workspace_size(ctypes.byref(m), 64, 41, 17, 16384)
    assert need > (64 << 20)
    st = L.sdv_verify_forward_noalloc(ctypes.byref(m), ctypes.byref(kvd), ctypes.byref(inp), ctypes.byref(out), None)
    assert st == -4 and b"static scratch" in L.sdv_last_error()
