"""GPU parity of sv_verify_coupled against the oracle (oracle.coupled).

The target's choices and the emitted tokens must be bit-exact, except in
rows the oracle flags as near ties (two best scores within 1e-9).
"""
import numpy as np
import pytest
import torch

import oracle
from verify_pass_sv_amd import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _sv():
    import verify_pass_sv_amd as sv
    return sv


def _run(tgt, tok, seed, offset=0):
    sv = _sv()
    t, k_ = to_dev(tgt, tok)
    out = sv.sv_verify_coupled(t, k_, seed, offset, choices=True)
    torch.cuda.synchronize()
    res = oracle.verify_coupled(tgt.numpy(), tok.numpy(), seed, offset)
    return out, res


def _compare(out, res):
    n_acc = out["n_acc"].cpu().numpy()
    status = out["status"].cpu().numpy()
    toks = out["tokens"].cpu().numpy()
    ch = out["choices"].cpu().numpy()
    flagged = 0
    for b, r in enumerate(res):
        assert status[b] == r.status, (b, status[b], r.status)
        if r.status != 0:
            assert n_acc[b] == -1 and np.all(toks[b] == -1) and np.all(ch[b] == -1)
            continue
        flags = r.extra["flags"]
        if any(flags):
            flagged += 1
            first = flags.index(True)
            assert ch[b, :first].tolist() == r.extra["choices"][:first]
            continue
        assert ch[b].tolist() == r.extra["choices"], b
        assert n_acc[b] == r.n_acc
        assert toks[b, :r.n_out].tolist() == r.tokens
        assert np.all(toks[b, r.n_out:] == -1)
    return flagged


@pytest.mark.parametrize("sigma", [0.1, 1.0, 3.0])
def test_matches_oracle(sigma):
    B, k, V = 64, 4, 1000
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=12, sigma=sigma)
    tok = torch.from_numpy(oracle.coupled_drafts(dft.numpy(), 5, offset=2))
    out, res = _run(tgt, tok, seed=5, offset=2)
    assert _compare(out, res) <= 1
    assert any(r.n_acc < k for r in res)


def test_many_trials_in_one_call():
    # 3000 trials: the choose launch's z dimension and one decide wave per
    # trial well past one row of workgroups; vocabulary 33 (one ragged span)
    B, k, V = 3000, 2, 33
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=43, sigma=1.0)
    tok = torch.from_numpy(oracle.coupled_drafts(dft.numpy(), 5, offset=1))
    out, res = _run(tgt, tok, seed=5, offset=1)
    assert _compare(out, res) <= B // 50


def test_equal_distributions_accept_every_draft():
    B, k, V = 32, 6, 3000
    tgt, _, _ = synth.accept_inputs(B, k, V, seed=4, sigma=1.0)
    tok = torch.from_numpy(oracle.coupled_drafts(tgt[:, :k].numpy(), 77))
    sv = _sv()
    t, k_ = to_dev(tgt, tok)
    out = sv.sv_verify_coupled(t, k_, 77)
    torch.cuda.synchronize()
    assert (out["n_acc"] == k).all() and (out["status"] == 0).all()


def test_full_vocab_k32():
    B, k, V = 2, 32, 152000
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=19, sigma=0.1)
    tok = torch.from_numpy(oracle.coupled_drafts(dft.numpy(), 3))
    out, res = _run(tgt, tok, seed=3)
    assert _compare(out, res) == 0


@pytest.mark.parametrize("V", [5000, 4099])
def test_screened_noise_edge_rows(V):
    # the choose launch screens entries in binary32 before the binary64
    # noise: large scores (the margin's relative part), widely spread
    # logits, rows of -inf with a few equal finite entries, all-equal rows
    # (the noise alone decides), and a ragged last span
    B, k = 8, 3
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=29, sigma=1.0)
    tgt[0] += 1.0e6
    tgt[1] = -tgt[1].abs() * 1.0e4
    tgt[2, :, :] = float("-inf")
    tgt[2, :, ::97] = 0.5
    tgt[3] = 2.0
    tok = torch.from_numpy(oracle.coupled_drafts(dft.numpy(), 9))
    out, res = _run(tgt, tok, seed=9)
    assert _compare(out, res) <= 1


def test_invalid_inputs_report_status():
    B, k, V = 5, 3, 50
    tgt, _, tok = synth.accept_inputs(B, k, V, seed=5, sigma=1.0)
    tok[1, 2] = V
    tok[2, 0] = -1
    tgt[3, 1, 7] = float("nan")
    tgt[4, 3, :] = float("-inf")
    out, res = _run(tgt, tok, seed=1)
    _compare(out, res)
    assert out["status"].cpu().tolist() == [0, 1, 1, 2, 2]


def test_argument_errors():
    sv = _sv()
    tgt, _, tok = to_dev(*synth.accept_inputs(2, 4, 100, seed=1, sigma=1.0))
    with pytest.raises(sv.SvError):
        sv.sv_verify_coupled(tgt, tok, 0, offset=1 << 24)
