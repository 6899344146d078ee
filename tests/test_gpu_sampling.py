"""GPU parity of speculative-sampling acceptance against the oracle (through the C ABI).

Accepted lengths and drawn tokens must match bit-exactly, except sequences whose
oracle decision lies within 1e-6 of a threshold (flagged: acceptance ratio vs
uniform, or the inverse-CDF target vs a partial sum), which are counted and
excluded.
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


def _run(si, temperature=1.0):
    B, k1, V = si.target_logits.shape
    k = k1 - 1
    dev = "cuda"
    tgt = torch.from_numpy(si.target_logits).to(dev)
    drf = torch.from_numpy(si.draft_logits).to(dev)
    drafts = torch.from_numpy(si.drafts).to(dev)
    ua = torch.from_numpy(si.u_accept).to(dev)
    us = torch.from_numpy(si.u_sample).to(dev)
    smp = sdv.Sampler(B, k, V)
    n, tok = smp(tgt, drf, drafts, ua, us, temperature)
    torch.cuda.synchronize()
    return n.cpu().numpy(), tok.cpu().numpy()


def _check(si, temperature=1.0):
    n, tok = _run(si, temperature)
    on, otok, fl = ss.accept_sample(si.target_logits.astype(np.float64), si.draft_logits.astype(np.float64),
                                    si.drafts, si.u_accept, si.u_sample, temperature)
    ok = ~fl
    assert np.array_equal(n[ok], on[ok]), np.nonzero(n != on)
    assert np.array_equal(tok[ok], otok[ok]), np.nonzero(tok != otok)
    assert np.all((n >= 0) & (n <= si.drafts.shape[1]))
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
    n, tok = _run(si)
    assert np.all(n == 5)
    _check(si)


def test_sampling_parity_full_size():
    """Batch 64 x 7 draft positions over V = 151936: half peaked, half flat rows."""
    si = make_sample_inputs(SAMPLE_FULL)
    flagged = _check(si)
    print(f"flagged {flagged} / {SAMPLE_FULL.batch}", flush=True)


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
    n, tok = _run(si)
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
    n, _ = _run(si)
    assert np.all(n >= 66)
    _check(si)
