"""GPU parity of sv_verify_sampled against the oracle (oracle.sampling).

Token decisions must be bit-exact except where the oracle flags a near tie: an
accept decision with |u q' - p'| < 1e-6 (p', q' > 0), a residual threshold
within 1e-6 S of a bin edge, or a top-p boundary within 1e-9 of top_p in any
row of the trial (the library sums masses in binary64).  Kept probabilities of
the drafts within 2e-3 relative.
"""
import numpy as np
import pytest
import torch

import oracle
from verify_pass_sv_amd import synth
from conftest import load_worked_example
from gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu


def _sv():
    import verify_pass_sv_amd as sv
    return sv


def _f32(settings):
    """The settings as the binary32 values the library receives."""
    T, top_k, top_p = settings
    return float(np.float32(T)), int(top_k), float(np.float32(top_p))


def _run(tgt, dft, tok, seed, settings, offset=0):
    sv = _sv()
    t, d, k_ = to_dev(tgt, dft, tok)
    out = sv.sv_verify_sampled(t, d, k_, seed, offset, *settings, diagnostics=True)
    torch.cuda.synchronize()
    res = oracle.verify_accept_sampled(tgt.numpy(), dft.numpy(), tok.numpy(), seed, offset,
                                       *_f32(settings))
    return out, res


def _compare(out, res):
    n_acc = out["n_acc"].cpu().numpy()
    status = out["status"].cpu().numpy()
    toks = out["tokens"].cpu().numpy()
    p = out["p_at"].cpu().numpy()
    q = out["q_at"].cpu().numpy()
    flagged = 0
    for b, r in enumerate(res):
        assert status[b] == r.status, (b, status[b], r.status)
        if r.status != 0:
            assert n_acc[b] == -1 and np.all(toks[b] == -1)
            assert np.all(np.isnan(p[b])) and np.all(np.isnan(q[b]))
            continue
        if r.extra.get("top_p_flags"):
            flagged += 1
            continue
        np.testing.assert_allclose(p[b], r.p_at, rtol=2e-3, atol=1e-9)
        np.testing.assert_allclose(q[b], r.q_at, rtol=2e-3, atol=1e-9)
        if r.accept_flags is not None and r.accept_flags.any():
            flagged += 1
            first = int(np.argmax(r.accept_flags))
            assert toks[b, :first].tolist() == r.tokens[:first]
            continue
        assert n_acc[b] == r.n_acc, (b, n_acc[b], r.n_acc)
        assert toks[b, :r.n_acc].tolist() == r.tokens[:r.n_acc]
        assert np.all(toks[b, r.n_out:] == -1)
        if r.residual_flag:
            flagged += 1
            continue
        assert toks[b, r.n_acc] == r.tokens[r.n_acc], (b, toks[b], r.tokens)
    return flagged


SETTINGS = [
    (0.0, 0, 1.0),          # greedy
    (1.0, 0, 1.0),          # plain
    (0.7, 0, 1.0),          # temperature
    (1.0, 50, 1.0),         # top-k
    (1.0, 0, 0.9),          # top-p
    (0.8, 100, 0.95),       # all three
    (1.3, 1, 1.0),          # a single kept token: greedy verification
]


@pytest.mark.parametrize("settings", SETTINGS, ids=lambda s: f"T{s[0]}_k{s[1]}_p{s[2]}")
@pytest.mark.parametrize("sigma", [0.3, 2.0])
def test_matches_oracle_tiny(settings, sigma):
    B, k, V = 64, 4, 1000
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=31, sigma=sigma)
    tok = torch.from_numpy(oracle.sample_drafts(dft.numpy(), 7, *settings))
    out, res = _run(tgt, dft, tok, seed=11, settings=settings, offset=3)
    assert _compare(out, res) <= 2
    assert any(r.n_acc < k for r in res) and any(r.n_acc > 0 for r in res)


@pytest.mark.parametrize("settings", [(1.0, 3, 1.0), (1.0, 0, 0.5), (0.5, 8, 0.8),
                                      (0.0, 0, 1.0)],
                         ids=lambda s: f"T{s[0]}_k{s[1]}_p{s[2]}")
def test_tied_logits_at_the_boundary(settings):
    # logits on a coarse lattice: many equal values at the top-k / top-p
    # boundaries, so the smaller-index-first tie cut decides the kept set
    B, k, V = 48, 3, 97
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=5, sigma=1.0)
    tgt = torch.round(tgt * 2) / 2
    dft = torch.round(dft * 2) / 2
    tok = torch.from_numpy(oracle.sample_drafts(dft.numpy(), 9, *settings))
    out, res = _run(tgt, dft, tok, seed=4, settings=settings)
    assert _compare(out, res) <= 2


def test_drafts_outside_the_draft_kept_set():
    # arbitrary drafts: q' = 0 for most of them, accepted iff p' > 0
    B, k, V = 64, 4, 300
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=6, sigma=0.2)
    g = torch.Generator().manual_seed(3)
    tok = torch.randint(0, V, (B, k), generator=g, dtype=torch.int32)
    out, res = _run(tgt, dft, tok, seed=2, settings=(1.0, 20, 1.0))
    assert _compare(out, res) <= 2
    assert any(r.q_at is not None and (r.q_at == 0).any() for r in res)


@pytest.mark.parametrize("settings", [(0.0, 0, 1.0), (0.7, 0, 0.9), (1.0, 1000, 1.0)],
                         ids=lambda s: f"T{s[0]}_k{s[1]}_p{s[2]}")
def test_full_vocab_k32(settings):
    B, k, V = 3, 32, 152000
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=17, sigma=0.1)
    tok = torch.from_numpy(oracle.sample_drafts(dft.numpy(), 21, *settings))
    out, res = _run(tgt, dft, tok, seed=13, settings=settings)
    assert _compare(out, res) <= 1


@pytest.mark.parametrize("settings", [(0.9, 5, 0.8), (0.0, 0, 1.0), (1.0, 0, 1.0)],
                         ids=["T0.9_k5_p0.8", "greedy", "plain"])
def test_many_trials_in_one_call(settings):
    # 3000 trials: grids well past one row of workgroups per launch (the rows
    # launch's y dimension, the greedy chain's z dimension); vocabulary 33 (a
    # ragged residual block and span)
    B, k, V = 3000, 2, 33
    tgt, dft, tok = synth.accept_inputs(B, k, V, seed=41, sigma=1.0)
    out, res = _run(tgt, dft, tok, seed=9, settings=settings)
    flagged = _compare(out, res)
    assert flagged <= B // 50


def test_greedy_on_the_page_example():
    ex = load_worked_example("worked_example_page1.txt")
    t = torch.from_numpy(ex["target"]).float()[None]
    d = torch.from_numpy(ex["draft"]).float()[None]
    tok = torch.from_numpy(ex["tokens"]).to(torch.int32)[None]
    out, res = _run(t, d, tok, seed=0, settings=(0.0, 0, 1.0))
    _compare(out, res)
    assert out["n_acc"].item() == ex["expect_n_acc"]
    assert out["tokens"][0, :3].tolist() == ex["expect_tokens"]


def test_invalid_inputs_report_status():
    B, k, V = 6, 3, 50
    tgt, dft, tok = synth.accept_inputs(B, k, V, seed=5, sigma=1.0)
    tok[1, 2] = V
    tok[2, 0] = -1
    tgt[3, 1, 7] = float("nan")
    dft[4, 0, :] = float("-inf")
    tgt[5, 3, 0] = float("inf")
    for settings in [(0.9, 10, 0.8), (0.0, 0, 1.0)]:
        out, res = _run(tgt, dft, tok, seed=1, settings=settings)
        _compare(out, res)
        st = out["status"].cpu().tolist()
        assert st[1] == 1 and st[2] == 1 and st[3] == 2 and st[5] == 2
        # greedy verification does not read the draft rows
        assert st[4] == (0 if settings[0] == 0.0 else 2)


@pytest.mark.parametrize("V", [20000, 20001])
@pytest.mark.parametrize("settings", [(1.0, 0, 1.0), (0.9, 10, 0.8), (1.3, 1, 1.0)],
                         ids=["plain", "k10_p0.8", "k1"])
def test_rows_split_over_slices(V, settings):
    # few rows of a long vocabulary: each row's full passes run over several
    # workgroups and merge in slice order; invalid rows, equal maxima in the
    # first and last slice, and a row length that is not a multiple of 4
    B, k = 6, 3
    tgt, dft, tok = synth.accept_inputs(B, k, V, seed=12, sigma=1.0)
    tgt[1, 1, V - 2] = float("nan")
    dft[2, 0, :] = float("-inf")
    tgt[3, 3, V // 2] = float("inf")
    for t in (tgt, dft):
        t[0, 0, 3] = 40.0
        t[0, 0, V - 1] = 40.0
    tok[0, 0] = V - 1
    out, res = _run(tgt, dft, tok, seed=3, settings=settings)
    flagged = _compare(out, res)
    st = out["status"].cpu().tolist()
    assert st == [0, 2, 2, 2, 0, 0]
    # trials 0, 4 and 5 are valid: at least two of them compared unflagged
    assert 3 - flagged >= 2

    # the same six trials inside a call of 40 (one workgroup per row, no
    # slices; a trial's uniforms depend on its index only): same statuses,
    # and the same tokens wherever the oracle flags nothing
    sv = _sv()
    Bb = 40
    tb, db, kb = synth.accept_inputs(Bb, k, V, seed=13, sigma=1.0)
    tb[:B], db[:B], kb[:B] = tgt, dft, tok
    t, d, kk = to_dev(tb, db, kb)
    big = sv.sv_verify_sampled(t, d, kk, 3, 0, *settings, diagnostics=True)
    torch.cuda.synchronize()
    assert big["status"][:B].cpu().tolist() == st
    for b, r in enumerate(res):
        if r.status != 0:
            continue
        np.testing.assert_allclose(big["p_at"][b].cpu().numpy(), out["p_at"][b].cpu().numpy(),
                                   rtol=1e-6, atol=1e-12)
        np.testing.assert_allclose(big["q_at"][b].cpu().numpy(), out["q_at"][b].cpu().numpy(),
                                   rtol=1e-6, atol=1e-12)
        if r.extra.get("top_p_flags") or (r.accept_flags is not None and r.accept_flags.any()) \
                or r.residual_flag:
            continue
        assert big["n_acc"][b].item() == out["n_acc"][b].item()
        assert torch.equal(big["tokens"][b], out["tokens"][b])


def test_default_settings_agree_with_the_plain_entry_point():
    sv = _sv()
    B, k, V = 32, 5, 2000
    tgt, dft, tok = to_dev(*synth.accept_inputs(B, k, V, seed=8, sigma=1.0))
    a = sv.sv_verify_accept(tgt, dft, tok, 77, 1)
    b = sv.sv_verify_sampled(tgt, dft, tok, 77, 1)
    torch.cuda.synchronize()
    same = (a["tokens"] == b["tokens"]).all(dim=1).sum().item()
    assert same >= B - 1          # both binary32 paths; a near tie may split them
    assert torch.equal(a["status"], b["status"])


def test_argument_errors():
    sv = _sv()
    tgt, dft, tok = to_dev(*synth.accept_inputs(2, 4, 100, seed=1, sigma=1.0))
    with pytest.raises(sv.SvError):
        sv.sv_verify_sampled(tgt, dft, tok, 0, temperature=-0.5)
    with pytest.raises(sv.SvError):
        sv.sv_verify_sampled(tgt, dft, tok, 0, top_p=0.0)
    with pytest.raises(sv.SvError):
        sv.sv_verify_sampled(tgt, dft, tok, 0, top_k=-2)


@pytest.mark.parametrize("n_tied,settings", [
    (1500, (1.0, 2600, 1.0)),       # boundary bin of 1500+ tokens: sorted in LDS
    (5000, (1.0, 2600, 1.0)),       # more than the LDS list: radix fallback
    (5000, (0.9, 0, 0.3)),          # top-p boundary inside a 5000-token tie
    (5000, (1.0, 4000, 0.5)),       # both, the top-p boundary in the top-k bin
], ids=["sorted_1500", "radix_topk_5000", "radix_topp_5000", "radix_both_5000"])
def test_large_tied_boundary_bins(n_tied, settings):
    # many tokens share one logit near the top of each row, so the boundary
    # bin holds n_tied tokens at least
    B, k, V = 4, 3, 20000
    tgt, dft, _ = synth.accept_inputs(B, k, V, seed=23, sigma=0.5)
    g = torch.Generator().manual_seed(7)
    for t in (tgt, dft):
        for b in range(B):
            for i in range(t.shape[1]):
                idx = torch.randperm(V, generator=g)[:n_tied]
                t[b, i, idx] = 3.0
    tok = torch.from_numpy(oracle.sample_drafts(dft.numpy(), 5, *settings))
    out, res = _run(tgt, dft, tok, seed=8, settings=settings)
    assert _compare(out, res) <= 1


@pytest.mark.parametrize("settings", [(1.0, 0, 1.0), (1.0, 50, 1.0), (0.7, 0, 0.9),
                                      (0.8, 100, 0.95)],
                         ids=["plain", "k50", "T0.7_p0.9", "T0.8_k100_p0.95"])
@pytest.mark.parametrize("B", [6, 40], ids=["sliced_rows", "one_workgroup_per_row"])
def test_rows_whose_first_entries_mislead_the_pass(B, settings):
    # The pass bins a row against a reference taken from its first 4096
    # entries (their maximum raised by min(4, 8 T)), and for top-k lists the
    # tokens above a bin predicted from their counts.  Rows where that
    # misleads: a later logit above the reference (the pass is taken again
    # against the row maximum), first entries shifted up (the list falls
    # short of top_k) or down (the list overflows), and a lone huge logit
    # far into one row.  The outputs must still match the oracle.
    k, V = 3, 20000
    tgt, dft, tok = synth.accept_inputs(B, k, V, seed=31, sigma=1.0)
    for t in (tgt, dft):
        for i in range(t.shape[1]):
            t[0, i, 10000] = t[0, i, :4096].max() + 4.5
        t[1, :, :4096] += 3.0
        t[2, :, :4096] -= 3.0
        t[3, 1, 15000] = 50.0
    out, res = _run(tgt, dft, tok, seed=4, settings=settings)
    flagged = _compare(out, res)
    assert (out["status"] == 0).all()
    # (at V = 20000 a draft's p is about 5e-5, so the 1e-6 band of the
    # accept test flags a few percent of the decisions)
    assert flagged <= max(2, B // 5)
