"""GPU parity of the verify forward, greedy acceptance and rollback (through the C ABI).

Each case runs the HIP path and the CPU oracle on the same seeded inputs and
compares element by element (tolerances in tests/gpu_helpers.py).  Shapes span
several MFMA tiles with ragged tails (vocab 3001 / 2053 / 1537, d = 320 / 192,
T not a multiple of 16, GQA groups of 1, 2 and 3).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_verify_amd as sdv  # noqa: E402
from oracle import decoder as odec  # noqa: E402
from synth import (MINI_BF16, MINI_BF16_D128, MINI_BF16_D2048, MINI_F32, MINI_F32_D2048,  # noqa: E402
                   MINI_BF16_FFN12K, MINI_F32_FFN12K, MINI_BF16_V70K, MINI_F32_V70K, make_weights,
                   make_random_kv, uniform_tokens)
from synth.configs import ModelShape  # noqa: E402
from tests.gpu_helpers import (run_pair, compare_logits, compare_kv, greedy_expectation,  # noqa: E402
                               mode_of, logit_tol as logit_tol_of)


def _tokens(B, T, V, seed):
    return np.stack([uniform_tokens(T, V, seed + b, "chunk") for b in range(B)])


@pytest.mark.parametrize("shape,lens,L_a,gamma", [
    (MINI_BF16, (37, 70), 5, 6),
    (MINI_BF16, (0,), 1, 3),        # empty cache
    (MINI_BF16, (129,), 9, 0),      # audio only (R = 1)
    (MINI_F32, (50, 3, 17), 4, 9),
    (MINI_BF16_D128, (40,), 7, 12),
])
def test_verify_parity(shape, lens, L_a, gamma):
    print(f"case {shape.name} lens={lens} L_a={L_a} gamma={gamma}", flush=True)
    w = make_weights(shape, seed=101, gain_noise=0.1)
    T = L_a + gamma
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=102)
    toks = _tokens(len(lens), T, shape.vocab, 103)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=104)
    assert np.all(g["err"] == 0)
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    compare_kv(shape, kv, o, list(lens), T)
    tol = 2e-2 if shape.dtype == "bf16" else 1e-5
    hd = np.max(np.abs(g["hidden"] - o["hidden"])) / np.max(np.abs(o["hidden"]))
    assert hd <= tol, hd


@pytest.mark.parametrize("shape,lens,L_a,gamma", [
    (MINI_BF16, (37, 70, 5, 0, 101), 6, 16),            # 110 rows, 85 logit rows: one ragged 128-row block
    (MINI_F32, (9, 40, 3, 66, 12, 20, 1, 51, 30), 4, 16),  # 180 rows: two row blocks
    (MINI_BF16_D128, (40, 17, 90, 3, 61, 8), 5, 15),    # 120 rows, 66 logit rows
])
def test_verify_parity_many_rows(shape, lens, L_a, gamma):
    """A batch with more than 80 chunk rows takes the tiled many-row GEMM for every
    projection (and, above 80 logit rows, for the LM head)."""
    print(f"case {shape.name} lens={lens} L_a={L_a} gamma={gamma}", flush=True)
    w = make_weights(shape, seed=111, gain_noise=0.1)
    T = L_a + gamma
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=112)
    toks = _tokens(len(lens), T, shape.vocab, 113)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=114)
    assert np.all(g["err"] == 0)
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    compare_kv(shape, kv, o, list(lens), T)
    tol = 2e-2 if shape.dtype == "bf16" else 1e-5
    hd = np.max(np.abs(g["hidden"] - o["hidden"])) / np.max(np.abs(o["hidden"]))
    assert hd <= tol, hd


@pytest.mark.parametrize("shape", [MINI_BF16, MINI_F32], ids=lambda s: s.name)
@pytest.mark.parametrize("B,L_a,gamma", [
    (1, 4, 12),    # 16 chunk rows: one whole row tile, 13 logit rows
    (1, 5, 12),    # 17 rows: a one-row tail tile; 13 logit rows
    (2, 4, 12),    # 32 rows, 26 logit rows (two tiles, a ten-row tail)
    (5, 4, 12),    # 80 rows, the most the few-row GEMM takes; 65 logit rows (one-row tail)
    (3, 4, 23),    # 81 rows: the first batch on the tiled GEMM; 72 logit rows
    (4, 4, 23),    # 108 rows, 96 logit rows: the LM head on the tiled GEMM too
])
def test_row_tile_boundaries(shape, B, L_a, gamma):
    """Activation operands are stored in whole 16-row tiles whose padding rows are
    never written: chunk-row and logit-row counts at and around the tile, few-row and
    many-row boundaries all match the oracle."""
    T = L_a + gamma
    lens = [23 + 17 * b for b in range(B)]
    print(f"case {shape.name} B={B} T={T} rows={B * T} logit rows={B * (gamma + 1)}", flush=True)
    w = make_weights(shape, seed=121, gain_noise=0.1)
    kvh = make_random_kv(shape, lens, capacity=max(lens) + T, seed=122)
    toks = _tokens(B, T, shape.vocab, 123)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=124)
    assert np.all(g["err"] == 0)
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    compare_kv(shape, kv, o, lens, T)
    tol = 2e-2 if shape.dtype == "bf16" else 1e-5
    hd = np.max(np.abs(g["hidden"] - o["hidden"])) / np.max(np.abs(o["hidden"]))
    assert hd <= tol, hd


@pytest.mark.parametrize("shape", [MINI_BF16_D2048, MINI_F32_D2048], ids=lambda s: s.name)
@pytest.mark.parametrize("lens,L_a,gamma", [
    ((37, 70), 5, 16),           # 42 rows
    ((12,), 1, 0),               # a single row
    ((9, 51, 30, 66), 5, 25),    # 120 rows: the tiled GEMM, K split in 4 for o and down
    ((40, 58), 5, 28),           # 66 rows: the column-split GEMM, K split on every projection
])
def test_parity_d2048(shape, lens, L_a, gamma):
    """The 1.7B model width (d = 2048, 256 threads x 8 columns in the norms, K = 2048
    and 4096 in the projections) on a small vocabulary: logits, hidden rows and the
    written K/V match the oracle."""
    print(f"case {shape.name} lens={lens} L_a={L_a} gamma={gamma}", flush=True)
    w = make_weights(shape, seed=131, gain_noise=0.1)
    T = L_a + gamma
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=132)
    toks = _tokens(len(lens), T, shape.vocab, 133)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=134)
    assert np.all(g["err"] == 0), g["err"]
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    compare_kv(shape, kv, o, list(lens), T)
    tol = 2e-2 if shape.dtype == "bf16" else 1e-5
    hd = np.max(np.abs(g["hidden"] - o["hidden"])) / np.max(np.abs(o["hidden"]))
    assert hd <= tol, hd


@pytest.mark.parametrize("shape", [MINI_BF16_FFN12K, MINI_F32_FFN12K], ids=lambda s: s.name)
@pytest.mark.parametrize("lens,L_a,gamma", [
    ((50,), 25, 40),       # 65 rows (5 row tiles, a one-row tail), 41 logit rows
    ((20, 33), 5, 25),     # 60 rows (4 row tiles), 52 logit rows
])
def test_wide_ffn_six_tile_gate_up(shape, lens, L_a, gamma):
    """1536 gate/up tiles at 4-5 row tiles: the gate/up launch takes six tiles per
    workgroup (256 workgroups); 33-48 logit rows put the LM head on six tiles too."""
    print(f"case {shape.name} lens={lens} L_a={L_a} gamma={gamma}", flush=True)
    w = make_weights(shape, seed=141, gain_noise=0.1)
    T = L_a + gamma
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=142)
    toks = _tokens(len(lens), T, shape.vocab, 143)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=144)
    assert np.all(g["err"] == 0), g["err"]
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    compare_kv(shape, kv, o, list(lens), T)
    tol = 2e-2 if shape.dtype == "bf16" else 1e-5
    hd = np.max(np.abs(g["hidden"] - o["hidden"])) / np.max(np.abs(o["hidden"]))
    assert hd <= tol, hd


@pytest.mark.parametrize("shape", [MINI_BF16_V70K, MINI_F32_V70K], ids=lambda s: s.name)
def test_large_vocab_tiled_lm_head(shape):
    """90 logit rows over a vocabulary of 70,001: the LM head runs on the tiled kernel at
    8 tile columns per wave, whose epilogue (logits and row statistics) works on 64-row
    halves of the 128-row block."""
    lens, L_a, gamma = (21, 40, 7), 4, 29
    print(f"case {shape.name} lens={lens} L_a={L_a} gamma={gamma}", flush=True)
    w = make_weights(shape, seed=151, gain_noise=0.1)
    T = L_a + gamma
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=152)
    toks = _tokens(len(lens), T, shape.vocab, 153)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=154)
    assert np.all(g["err"] == 0), g["err"]
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    assert n == len(lens) * (gamma + 1)
    compare_kv(shape, kv, o, list(lens), T)


def test_many_sequences_fine_query_groups():
    """128 sequences x 2 kv heads fill the GPU with (sequence, head) pairs alone, so the
    chunk attention splits each head's 5 query tiles into groups of at most 4 and takes
    no key splits; logits and K/V match the oracle."""
    shape = MINI_BF16_D128
    B, L_a, gamma = 128, 8, 32
    T = L_a + gamma
    rng = np.random.default_rng(141)
    lens = [int(x) for x in rng.integers(3, 60, size=B)]
    print(f"case {shape.name} B={B} T={T} heads={B * shape.n_kv_heads}", flush=True)
    w = make_weights(shape, seed=142, gain_noise=0.1)
    kvh = make_random_kv(shape, lens, capacity=max(lens) + T, seed=143)
    toks = _tokens(B, T, shape.vocab, 144)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=145)
    assert np.all(g["err"] == 0)
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    compare_kv(shape, kv, o, lens, T)


def test_attention_dominant_hidden():
    """Scaled q/k/o weights make attention dominate the residual stream, so a wrong
    attention kernel cannot hide under the FFN's contribution."""
    shape = MINI_BF16_D128
    w = make_weights(shape, seed=201, scales={"wq": 8.0, "wk": 8.0, "wo": 20.0, "wd": 0.05})
    lens = (75, 33)
    L_a, gamma = 6, 10
    T = L_a + gamma
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=202)
    toks = _tokens(2, T, shape.vocab, 203)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=204)
    hd = np.max(np.abs(g["hidden"] - o["hidden"]), axis=-1) / np.max(np.abs(o["hidden"]), axis=-1)
    assert hd.max() <= 2e-2, hd.max()
    compare_logits(shape, g, o)


def test_tree_branch_and_greedy_commit():
    """A runner-up branch forking at the first draft position, verified under a tree mask;
    the branch carries the true continuation, so acceptance follows it and the commit
    compacts its rows."""
    shape = MINI_BF16
    w = make_weights(shape, seed=301)
    C, L_a, gamma, nb = 45, 5, 6, 4
    T = L_a + gamma + nb
    kvh = make_random_kv(shape, [C], capacity=C + T, seed=302)
    audio = uniform_tokens(L_a, shape.vocab, 303, "a")
    ar, _ = odec.greedy_decode(w, odec.Cache(kvh.k, kvh.v), audio, nb + 1, mode_of(shape))
    main = [(ar[0] + 7) % shape.vocab] + list(uniform_tokens(gamma - 1, shape.vocab, 304, "m"))
    toks = np.concatenate([audio, main, ar[:nb]])[None, :]
    parent = [j - 1 for j in range(T)]
    parent[L_a + gamma] = L_a - 1
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, parent=parent, perm_seed=305)
    compare_logits(shape, g, o)
    compare_kv(shape, kv, o, [C], T)
    rows = list(range(L_a - 1, T))
    n, nxt, path, flagged = greedy_expectation(toks[0], parent, L_a, rows, o["logits"][0])
    acc = sdv.accept_greedy(1, T, L_a, ver.tokens, ver.parent, ver.logit_rows, ver.argmax, base_len=kv.seq_len)
    torch.cuda.synchronize()
    if not flagged:
        assert int(acc["n"][0]) == n and int(acc["next"][0]) == nxt
        assert acc["path"][0, :n].cpu().tolist() == path
    assert n == nb and path == list(range(L_a + gamma, T))
    # commit: rows of the branch move to slots C + L_a + i
    k_before = [kv.gather(0, l, C + L_a + gamma, C + T)[0].clone() for l in range(shape.n_layers)]
    sdv.kv_rollback(ver.model, kv, acc["keep"], acc["move_src"], acc["move_dst"], acc["err"])
    torch.cuda.synchronize()
    assert int(kv.seq_len[0]) == C + L_a + n
    assert int(acc["err"][0]) == 0
    for l in range(shape.n_layers):
        k_after = kv.gather(0, l, C + L_a, C + L_a + n)[0]
        assert torch.equal(k_after, k_before[l][:n])


@pytest.mark.parametrize("shape", [MINI_BF16, MINI_F32], ids=lambda s: s.name)
def test_maximum_chunk_wide_tree(shape):
    """The largest chunk (T = 128 rows) as a wide tree: 6 audio rows, a main draft of 62
    and five branches of 12 hanging off different main rows, two batch rows with
    different cached lengths (one empty).  Every chunk row is a logit row."""
    w = make_weights(shape, seed=351)
    L_a, gamma, nbr, blen = 6, 62, 5, 12
    T = L_a + gamma + nbr * blen
    assert T == sdv.binding.MAX_T
    parent = [j - 1 for j in range(T)]
    for k in range(nbr):
        first = L_a + gamma + k * blen
        parent[first] = L_a - 1 + 11 * k      # forks at the last audio row, main rows 11, 22, ...
    lens = [77, 0]
    kvh = make_random_kv(shape, lens, capacity=max(lens) + T, seed=352)
    toks = _tokens(2, T, shape.vocab, 353)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, parent=parent, logit_rows=range(T), perm_seed=354)
    assert np.all(g["err"] == 0)
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  T=128 tree: logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    compare_kv(shape, kv, o, lens, T)
    acc = sdv.accept_greedy(2, T, L_a, ver.tokens, ver.parent, ver.logit_rows, ver.argmax)
    torch.cuda.synchronize()
    rows = list(range(T))
    for b in range(2):
        ne, nxt, path, fl = greedy_expectation(toks[b], parent, L_a, rows, o["logits"][b])
        if not fl:
            assert int(acc["n"][b]) == ne and int(acc["next"][b]) == nxt


@pytest.mark.parametrize("scenario", ["silence", "corrupt3", "random"])
def test_greedy_scenarios(scenario):
    """Drafts = greedy decoding under silence.  Audio == silence: full acceptance plus the
    bonus; draft 3 corrupted: n = 2; random audio: whatever the oracle says."""
    shape = MINI_BF16
    w = make_weights(shape, seed=401)
    C, L_a, gamma = 30, 4, 7
    T = L_a + gamma
    kvh = make_random_kv(shape, [C], capacity=C + T, seed=402)
    sil = np.zeros(L_a, dtype=np.int32)
    drafts, _ = odec.greedy_decode(w, odec.Cache(kvh.k, kvh.v), sil, gamma + 1, mode_of(shape))
    d = list(drafts[:gamma])
    audio = sil if scenario != "random" else uniform_tokens(L_a, shape.vocab, 403, "a")
    if scenario == "corrupt3":
        d[2] = (d[2] + 1) % shape.vocab
    toks = np.concatenate([audio, d])[None, :]
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=404)
    compare_logits(shape, g, o)
    rows = list(range(L_a - 1, T))
    n, nxt, path, flagged = greedy_expectation(toks[0], None, L_a, rows, o["logits"][0])
    if scenario == "silence":
        assert n == gamma and nxt == drafts[gamma]
    if scenario == "corrupt3":
        assert n == 2
    acc = sdv.accept_greedy(1, T, L_a, ver.tokens, None, ver.logit_rows, ver.argmax, base_len=kv.seq_len)
    torch.cuda.synchronize()
    if not flagged:
        assert int(acc["n"][0]) == n and int(acc["next"][0]) == nxt
    assert int(acc["n"][0]) + 1 >= 1


def test_poisoned_dead_slots_do_not_leak():
    """NaN in every slot beyond the committed length (including the tail of the last
    page) must not reach any output."""
    shape = MINI_BF16
    w = make_weights(shape, seed=501)
    C, L_a, gamma = 21, 3, 5
    T = L_a + gamma
    kvh = make_random_kv(shape, [C], capacity=C + T, seed=502)
    toks = _tokens(1, T, shape.vocab, 503)
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(shape, 1, C + T + 40)
    kv.k_pages.fill_(float("nan"))
    kv.v_pages.fill_(float("nan"))
    kv.load(kvh)
    # load() writes whole pages (zero padded); poison the padded tail again
    for l in range(shape.n_layers):
        pg = int(kv.block_table[0, C // 16])
        kv.k_pages[l, pg, :, C % 16:, :] = float("nan")
        kv.v_pages[l, pg, :, :, C % 16:] = float("nan")
    ver = sdv.Verifier(model, kv, T, L_a, list(range(L_a - 1, T)), max_ctx=C + 16)
    ver.set_tokens(toks)
    res = ver.forward()
    torch.cuda.synchronize()
    assert torch.isfinite(res.logits).all()
    o = odec.verify_forward(w, odec.Cache(kvh.k, kvh.v), toks, None, list(range(L_a - 1, T)), mode_of(shape))
    compare_logits(shape, dict(logits=res.logits.cpu().numpy().astype(np.float64), argmax=res.argmax.cpu().numpy(),
                               margin=res.margin.cpu().numpy(), lse=res.lse.cpu().numpy()), o)


def test_paged_placement_is_bit_identical():
    """Identity and shuffled block tables give bit-identical results."""
    shape = MINI_BF16
    w = make_weights(shape, seed=601)
    lens = (50, 77)
    T = 9
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=602)
    toks = _tokens(2, T, shape.vocab, 603)
    model = sdv.DeviceModel(w)
    outs = []
    for perm_seed in (None, 11, 12):
        g, _, _, _ = run_pair(w, kvh, toks, 3, perm_seed=perm_seed, model=model)
        outs.append(g)
    for g in outs[1:]:
        assert np.array_equal(g["logits"], outs[0]["logits"])
        assert np.array_equal(g["hidden"], outs[0]["hidden"])


@pytest.mark.parametrize("shape", [MINI_BF16_D128, MINI_BF16], ids=["dh128", "dh64"])
def test_tight_block_table_tail_tile(shape):
    """LDS-DMA attention (more query tiles than the register path takes) where the
    longest sequence ends in the first page of its last 32-key tile and the block table
    has no entry for that tile's second page: the staging copies the missing page from
    the zero page, so every wave issues the same loads for every tile and the
    load-counter waits stay exact.  The logits match the oracle, and a table with room
    to spare gives the same results bit for bit."""
    w = make_weights(shape, seed=631)
    lens, T, L_a = (40, 75), 30, 6          # 75 + 30 = 105 = 3 * 32 + 9 keys: page 7 of 7 is missing
    print(f"case {shape.name} lens={lens} T={T}", flush=True)
    kvh = make_random_kv(shape, list(lens), capacity=max(lens) + T, seed=632)
    toks = _tokens(2, T, shape.vocab, 633)
    model = sdv.DeviceModel(w)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, model=model, extra_capacity=0)
    assert 2 * ((max(lens) + T - 1) // 32) + 1 == kv.max_blocks   # the last tile's second page has no entry
    compare_logits(shape, g, o)
    g2, _, _, _ = run_pair(w, kvh, toks, L_a, model=model, extra_capacity=48)
    assert np.array_equal(g["logits"], g2["logits"])
    assert np.array_equal(g["hidden"], g2["hidden"])


def test_device_errors_are_reported():
    shape = MINI_BF16
    w = make_weights(shape, seed=701)
    C, T = 10, 6
    kvh = make_random_kv(shape, [C, C], capacity=C + T, seed=702)
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(shape, 2, C + T + 16)
    kv.load(kvh)
    ver = sdv.Verifier(model, kv, T, 2, list(range(1, T)), max_ctx=C)
    toks = _tokens(2, T, shape.vocab, 703)
    toks[1, 3] = shape.vocab + 5           # invalid token in sequence 1 only
    ver.set_tokens(toks)
    ver.forward()
    torch.cuda.synchronize()
    err = ver.err.cpu().numpy()
    assert err[0] == 0 and (err[1] & 0x1)
    # host-checkable errors return a status before anything runs
    with pytest.raises(sdv.SdvError):
        sdv.Verifier(model, kv, 200, 2, list(range(1, 200)), max_ctx=C)
    # rollback beyond the capacity is refused on the device, the sequence is untouched
    keep = torch.tensor([C + 1, 10 ** 6], dtype=torch.int32, device="cuda")
    e = torch.zeros(2, dtype=torch.int32, device="cuda")
    sdv.kv_rollback(model, kv, keep, err=e)
    torch.cuda.synchronize()
    assert e.cpu().tolist() == [0, 0x8]
    assert kv.seq_len.cpu().tolist() == [C + 1, C]


def test_rollback_idempotent_and_ordered_moves():
    shape = MINI_F32
    w = make_weights(shape, seed=801)
    C = 40
    kvh = make_random_kv(shape, [C], capacity=C, seed=802)
    model = sdv.DeviceModel(w)
    kv = sdv.PagedKV(shape, 1, C + 16)
    kv.load(kvh)
    ref = [kv.gather(0, l, 0, C) for l in range(shape.n_layers)]
    # ordered moves: slot 5 -> 3, then slot 3's new content stays, slot 10 -> 5
    src = torch.tensor([[5, 10, -1]], dtype=torch.int32, device="cuda")
    dst = torch.tensor([[3, 5, -1]], dtype=torch.int32, device="cuda")
    keep = torch.tensor([20], dtype=torch.int32, device="cuda")
    for _ in range(2):
        sdv.kv_rollback(model, kv, keep, src if _ == 0 else None, dst if _ == 0 else None)
    torch.cuda.synchronize()
    assert int(kv.seq_len[0]) == 20
    for l in range(shape.n_layers):
        k, v = kv.gather(0, l, 0, C)
        assert torch.equal(k[3], ref[l][0][5]) and torch.equal(k[5], ref[l][0][10])
        assert torch.equal(v[3], ref[l][1][5]) and torch.equal(k[4], ref[l][0][4])


# d = 256 with 32 MHA heads of 64 (6144 q/k/v rows) and FFN 12288: with 11 sequences x 120
# rows (1320 rows, 11 row blocks) the tiled GEMM takes 8 MFMA column tiles per wave for the
# q/k/v projection (rotary + paged append epilogue) and gate/up (SwiGLU epilogue), whose
# epilogues run on 64-row halves of the 128-row block
WIDE_MHA_BF16 = ModelShape("mini-bf16-wide-mha", n_layers=1, d=256, n_heads=32, n_kv_heads=32, head_dim=64,
                           ffn=12288, vocab=1000, dtype="bf16")
WIDE_MHA_F32 = ModelShape("mini-f32-wide-mha", n_layers=1, d=256, n_heads=32, n_kv_heads=32, head_dim=64,
                          ffn=12288, vocab=1000, dtype="f32")


@pytest.mark.parametrize("shape", [WIDE_MHA_BF16, WIDE_MHA_F32], ids=lambda s: s.name)
def test_tiled_gemm_eight_column_epilogues(shape):
    w = make_weights(shape, seed=701)
    B, L_a, gamma = 11, 100, 20
    T = L_a + gamma
    lens = [int(x) for x in np.random.default_rng(702).integers(5, 61, size=B)]
    kvh = make_random_kv(shape, lens, capacity=max(lens) + T, seed=703)
    toks = _tokens(B, T, shape.vocab, 704)
    g, o, ver, kv = run_pair(w, kvh, toks, L_a, perm_seed=705)
    assert np.all(g["err"] == 0)
    err, flagged, n = compare_logits(shape, g, o)
    print(f"  1320 rows, tiled 8-column epilogues: logits rel err {err:.2e}; flagged {flagged}/{n}", flush=True)
    compare_kv(shape, kv, o, lens, T)
    hd = np.max(np.abs(g["hidden"] - o["hidden"]), axis=2) / np.max(np.abs(o["hidden"]), axis=2)
    assert hd.max() <= logit_tol_of(shape), hd.max()
