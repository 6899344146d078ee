"""GPU parity of speculative-sampling acceptance against the oracle (through the C ABI).

The library draws its Philox4x32-10 uniforms itself from (seed, sequence, position);
the oracle takes the same numbers as inputs from the input generator's Philox.
Accepted lengths and drawn tokens must match bit-exactly, except sequences whose
oracle decision lies within 1e-6 of a threshold (flagged: acceptance ratio vs
uniform, or the inverse-CDF target vs a partial sum), which are counted and
excluded.  Flagged sequences are bounded: at most 1/8 of a batch (the full-size
batch flags 4 of 64: its flat rows spread p over 151,936 entries of about 7e-6
each, so a draw target often lies within 1e-6 of a partial sum), and the library's
own flags agree with the oracle's on all but at most 1/32 of the sequences.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import speculative_decoding_verify_amd as sdv  # noqa: E402
from oracle import spec_sampling as ss  # noqa: E402
from synth import SAMPLE_FULL, SampleWorkload, make_sample_inputs  # noqa: E402


def _run(si, temperature=1.0, seq_ids=None):
    B, k1, V = si.target_logits.shape
    k = k1 - 1
    dev = "cuda"
    tgt = torch.from_numpy(si.target_logits).to(dev)
    drf = torch.from_numpy(si.draft_logits).to(dev)
    drafts = torch.from_numpy(si.drafts).to(dev)
    sid = None if seq_ids is None else torch.from_numpy(np.asarray(seq_ids, dtype=np.int32)).to(dev)
    smp = sdv.Sampler(B, k, V)
    n, tok, fl = smp(tgt, drf, drafts, si.seed, sid, temperature)
    torch.cuda.synchronize()
    return n.cpu().numpy(), tok.cpu().numpy(), fl.cpu().numpy().astype(np.uint32)


def _check(si, temperature=1.0):
    n, tok, gfl = _run(si, temperature)
    on, otok, fl = ss.accept_sample(si.target_logits.astype(np.float64), si.draft_logits.astype(np.float64),
                                    si.drafts, si.u_accept, si.u_sample, temperature)
    ok = ~fl
    assert np.array_equal(n[ok], on[ok]), np.nonzero(n != on)
    assert np.array_equal(tok[ok], otok[ok]), np.nonzero(tok != otok)
    assert np.all((n >= 0) & (n <= si.drafts.shape[1]))
    B = len(n)
    gflagged = (gfl & (sdv.SAMPLE_NEAR_ACCEPT | sdv.SAMPLE_NEAR_DRAW)) != 0
    assert not np.any(gfl & sdv.SAMPLE_BAD_DRAFT)
    assert fl.sum() <= max(1, B // 8) and gflagged.sum() <= max(1, B // 8), (fl.sum(), gflagged.sum())
    # the two sides flag from their own arithmetic; they may differ only where a value
    # sits within rounding of the 1e-6 band itself
    assert np.sum(fl != gflagged) <= max(1, B // 32), (np.nonzero(fl)[0], np.nonzero(gflagged)[0])
    print(f"flagged: oracle {int(fl.sum())}, library {int(gflagged.sum())} of {B}", flush=True)
    return int(fl.sum())


@pytest.mark.parametrize("B,k,V", [(8, 3, 5000), (5, 1, 777), (16, 7, 4099)])
def test_sampling_parity_small(B, k, V):
    w = SampleWorkload(batch=B, k=k, vocab=V, seed=900 + V)
    si = make_sample_inputs(w)
    _check(si)


def test_sampling_parity_temperature():
    w = SampleWorkload(batch=8, k=4, vocab=3001, seed=950)
    si = make_sample_inputs(w)
    _check(si, temperature=0.7)


def test_sampling_identical_distributions_accept_all():
    """p == q: every draft is accepted (ratio 1 > u) and the bonus comes from p."""
    w = SampleWorkload(batch=6, k=5, vocab=2000, seed=960)
    si = make_sample_inputs(w)
    si.draft_logits[:] = si.target_logits[:, :5]
    n, tok, _ = _run(si)
    assert np.all(n == 5)
    _check(si)


def test_sampling_parity_full_size():
    """Batch 64 x 7 draft positions over V = 151936: half peaked, half flat rows."""
    si = make_sample_inputs(SAMPLE_FULL)
    _check(si)


def test_sampling_masked_logits():
    """Logits of -inf have probability 0.  Some rows are masked over their first 12000
    entries, longer than any thread's first group of loads, so threads start on -inf;
    some drafts sit on entries masked in q only (accepted iff p can produce them) or in
    both (always rejected)."""
    w = SampleWorkload(batch=12, k=4, vocab=20011, seed=970)
    si = make_sample_inputs(w)
    rng = np.random.default_rng(971)
    ninf = np.float32(-np.inf)
    for arr in (si.target_logits, si.draft_logits):
        mask = rng.random(arr.shape) < 0.3
        arr[mask] = ninf
        arr[:, 1, :12000] = ninf
    # keep at least the rows' largest entries finite so every row has support
    si.target_logits[:, :, 12000] = 3.0
    si.draft_logits[:, :, 12001] = 3.0
    for b in range(0, 12, 3):
        x = int(si.drafts[b, 0])
        si.draft_logits[b, 0, x] = ninf          # q(x) = 0
        if b % 2 == 0:
            si.target_logits[b, 0, x] = ninf     # and p(x) = 0
    with np.errstate(invalid="ignore"):
        _check(si)
    n, tok, _ = _run(si)
    on, otok, _ = ss.accept_sample(si.target_logits.astype(np.float64), si.draft_logits.astype(np.float64),
                                   si.drafts, si.u_accept, si.u_sample)
    rows = np.arange(12)
    tgt_at = si.target_logits[rows, n, tok]
    assert np.all(np.isfinite(tgt_at))   # an emitted token is never masked in p


def test_sampling_more_chunks_than_threads():
    """V = 1,100,003: 269 chunks of 4096 entries, more than the 256 threads of the
    draw's workgroup (several chunks per thread), and a ragged last chunk."""
    w = SampleWorkload(batch=3, k=2, vocab=1_100_003, seed=980)
    _check(make_sample_inputs(w))


def test_sampling_more_drafts_than_a_wave():
    """k = 70 draft positions: the decision ballots positions in groups of 64.  The
    first 66 draft rows equal the target rows (p = q: always accepted), so the first
    rejection, if any, falls in the second group."""
    w = SampleWorkload(batch=4, k=70, vocab=3001, seed=990)
    si = make_sample_inputs(w)
    si.draft_logits[:, :66] = si.target_logits[:, :66]
    n, _, _ = _run(si)
    assert np.all(n >= 66)
    _check(si)


def test_device_uniforms_equal_the_input_generator():
    """sdv_philox_uniforms (the numbers sdv_accept_sample draws) equal the input
    generator's Philox bit for bit, with and without explicit sequence ids."""
    from synth.gen import philox_uniforms
    B, n_pos, seed = 37, 9, 0x1234_5678_9ABC_DEF0
    for ids in (None, np.array([(7919 * b + 3) % 100003 for b in range(B)], dtype=np.int32)):
        sid = None if ids is None else torch.from_numpy(ids).cuda()
        u0, u1 = sdv.philox_uniforms(seed, B, n_pos, sid)
        seq = np.arange(B) if ids is None else ids
        r0, _ = philox_uniforms(seed, seq[:, None], np.arange(n_pos)[None, :], stream=0)
        _, r1 = philox_uniforms(seed, seq[:, None], np.arange(n_pos)[None, :], stream=1)
        assert np.array_equal(u0.cpu().numpy().view(np.uint64), r0.view(np.uint64))
        assert np.array_equal(u1.cpu().numpy().view(np.uint64), r1.view(np.uint64))


def test_sequence_ids_select_the_counters():
    """With seq_ids, sequence b draws from counter word seq_ids[b]: the oracle fed the
    uniforms of those counters gives the same decisions."""
    from synth.gen import philox_uniforms
    w = SampleWorkload(batch=10, k=4, vocab=3001, seed=1001)
    si = make_sample_inputs(w)
    ids = np.array([90 + 7 * b for b in range(10)], dtype=np.int32)
    n, tok, _ = _run(si, seq_ids=ids)
    ua, _ = philox_uniforms(si.seed, ids[:, None], np.arange(4)[None, :], stream=0)
    _, us = philox_uniforms(si.seed, ids[:, None], np.arange(5)[None, :], stream=1)
    on, otok, fl = ss.accept_sample(si.target_logits.astype(np.float64), si.draft_logits.astype(np.float64),
                                    si.drafts, ua, us)
    ok = ~fl
    assert np.array_equal(n[ok], on[ok]) and np.array_equal(tok[ok], otok[ok])


def test_bad_draft_ids_are_reported():
    """A draft id outside [0, V) marks its sequence (flag bit, n and token -1); the
    other sequences are unaffected."""
    w = SampleWorkload(batch=6, k=3, vocab=2003, seed=1002)
    si = make_sample_inputs(w)
    good = si.drafts.copy()
    si.drafts[1, 2] = 2003
    si.drafts[4, 0] = -5
    n, tok, fl = _run(si)
    assert n[1] == -1 and tok[1] == -1 and n[4] == -1 and tok[4] == -1
    assert fl[1] & sdv.SAMPLE_BAD_DRAFT and fl[4] & sdv.SAMPLE_BAD_DRAFT
    si.drafts[:] = good
    on, otok, ofl = ss.accept_sample(si.target_logits.astype(np.float64), si.draft_logits.astype(np.float64),
                                     si.drafts, si.u_accept, si.u_sample)
    for b in (0, 2, 3, 5):
        assert not fl[b] & sdv.SAMPLE_BAD_DRAFT
        if not ofl[b]:
            assert n[b] == on[b] and tok[b] == otok[b]


def test_near_threshold_decisions_are_flagged():
    """A uniform placed on the acceptance ratio: both sides flag that sequence.  With q
    uniform (q(x) = 1/V) and p = softmax of zeros except log c at x, p(x)/q(x) =
    c V / (c + V - 1); c is chosen so that this equals the sequence's own U0 at position
    0, up to the fp32 rounding of log c (a few 1e-7)."""
    from synth.gen import philox_uniforms
    B, k, V = 4, 2, 1024
    w = SampleWorkload(batch=B, k=k, vocab=V, seed=1003)
    si = make_sample_inputs(w)
    u0, _ = philox_uniforms(si.seed, np.arange(B), np.zeros(B, dtype=np.int64), stream=0)
    b = 2
    x = int(si.drafts[b, 0])
    si.draft_logits[b, 0] = 0.0
    c = u0[b] * (V - 1) / (V - u0[b])
    si.target_logits[b, 0] = 0.0
    si.target_logits[b, 0, x] = np.float32(np.log(c))
    p = ss.softmax(si.target_logits[b, 0].astype(np.float64))
    assert abs(u0[b] - p[x] * V) < 1e-6
    n, tok, fl = _run(si)
    _, _, ofl = ss.accept_sample(si.target_logits.astype(np.float64), si.draft_logits.astype(np.float64),
                                 si.drafts, si.u_accept, si.u_sample)
    assert ofl[b] and fl[b] & sdv.SAMPLE_NEAR_ACCEPT
