"""GPU parity of sv_verify_tree against the oracle (oracle.tree).

Greedy tree verification takes only exact decisions (binary32 compares and
integer checks), so every output is bit-exact: the emitted tokens, the path
length, the status and the accepted node indices.
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


def _run(tgt, tok, par):
    sv = _sv()
    t, k_, p_ = to_dev(tgt, tok, par)
    out = sv.sv_verify_tree(t, k_, p_, path=True)
    torch.cuda.synchronize()
    res = oracle.verify_tree(tgt.numpy(), tok.numpy(), par.numpy())
    return out, res


def _compare(out, res):
    n_acc = out["n_acc"].cpu().numpy()
    status = out["status"].cpu().numpy()
    toks = out["tokens"].cpu().numpy()
    path = out["path"].cpu().numpy()
    for b, r in enumerate(res):
        assert status[b] == r.status, (b, status[b], r.status)
        if r.status != 0:
            assert n_acc[b] == -1 and np.all(toks[b] == -1) and np.all(path[b] == -1)
            continue
        assert n_acc[b] == r.n_acc, (b, n_acc[b], r.n_acc)
        assert toks[b, :r.n_out].tolist() == r.tokens, b
        assert np.all(toks[b, r.n_out:] == -1)
        assert path[b, :r.n_acc].tolist() == r.extra["path"], b
        assert np.all(path[b, r.n_acc:] == -1)


@pytest.mark.parametrize("n,chain", [(16, 0.7), (16, 0.3), (32, 0.9), (5, 0.5)])
def test_matches_oracle(n, chain):
    B, V = 64, 1000
    tgt, tok, par = synth.tree_inputs(B, n, V, seed=n + 7, chain=chain)
    out, res = _run(tgt, tok, par)
    _compare(out, res)
    lens = [r.n_acc for r in res]
    assert min(lens) < max(lens)          # the cases span several path lengths


def test_full_vocab_max_nodes():
    B, n, V = 4, 32, 152000
    tgt, tok, par = synth.tree_inputs(B, n, V, seed=3, chain=0.8, agree=0.9)
    out, res = _run(tgt, tok, par)
    _compare(out, res)


@pytest.mark.parametrize("V", [1, 3, 4095, 4096, 4097, 12289])
def test_ragged_vocabulary(V):
    B, n = 16, 8
    tgt, tok, par = synth.tree_inputs(B, n, V, seed=V, chain=0.6)
    out, res = _run(tgt, tok, par)
    _compare(out, res)


def test_chain_tree_equals_greedy_verification_on_the_gpu():
    sv = _sv()
    B, k, V = 32, 8, 3000
    tgt, tok, par = synth.tree_inputs(B, k, V, seed=11, chain=1.0, agree=0.85)
    t, k_, p_ = to_dev(tgt, tok, par)
    tree = sv.sv_verify_tree(t, k_, p_)
    greedy = sv.sv_verify_sampled(t, torch.zeros_like(t[:, :k]), k_, 0, temperature=0.0)
    torch.cuda.synchronize()
    assert torch.equal(tree["n_acc"], greedy["n_acc"])
    assert torch.equal(tree["tokens"], greedy["tokens"])


def test_hand_built_trees():
    # the oracle's hand-worked cases: longest valid branch, equal lengths
    V = 6
    rows = np.zeros((8, V), dtype=np.float32)
    for r, c in enumerate([2, 4, 0, 1, 0, 3, 0, 0]):
        rows[r, c] = 5.0
    toks = [2, 3, 4, 5, 1, 4, 0]
    par = [-1, -1, 0, 0, 2, 1, 4]
    rows2 = np.zeros((8, V), dtype=np.float32)
    for r, c in enumerate([1, 2, 3, 0, 4, 0, 0, 0]):
        rows2[r, c] = 5.0
    toks2 = [1, 1, 3, 2, 4, 0, 0]
    par2 = [-1, -1, 1, 0, 3, 4, 5]        # node 3 -> 4 -> 5 -> 6 extends the branch of node 0
    tgt = torch.from_numpy(np.stack([rows, rows2]))
    tok = torch.tensor([toks, toks2], dtype=torch.int32)
    p = torch.tensor([par, par2], dtype=torch.int32)
    out, res = _run(tgt, tok, p)
    _compare(out, res)
    assert out["path"][0, :3].tolist() == [0, 2, 4]
    assert out["path"][1].tolist() == [0, 3, 4, 5, 6, -1, -1]


def test_ties_take_the_smallest_index():
    # rounded logits make many equal maxima per row
    B, n, V = 32, 12, 500
    g = torch.Generator().manual_seed(5)
    tgt = torch.randint(0, 4, (B, n + 1, V), generator=g).float()
    tok = torch.randint(0, 3, (B, n), generator=g, dtype=torch.int32)
    j = torch.arange(n)
    par = ((torch.rand((B, n), generator=g) * (j + 1)).floor() - 1).to(torch.int32)
    out, res = _run(tgt, tok, par)
    _compare(out, res)
    assert any(r.n_acc > 0 for r in res)


def test_statuses_and_their_order():
    B, n, V = 6, 4, 50
    tgt, tok, par = synth.tree_inputs(B, n, V, seed=9)
    tok[0, 2] = V                          # token out of range
    par[1, 3] = 3                          # parent not before the node
    par[2, 0] = -2                         # parent below -1
    tgt[3, 2, 7] = float("nan")            # NaN row
    tgt[4, 1, :] = float("-inf")           # no finite logit
    tok[5, 0] = -1                         # token out of range, with a bad parent too
    par[5, 1] = 5
    out, res = _run(tgt, tok, par)
    _compare(out, res)
    assert out["status"].tolist() == [1, 3, 3, 2, 2, 1]


def test_single_node_and_many_trials():
    B, n, V = 2048, 1, 777
    tgt, tok, par = synth.tree_inputs(B, n, V, seed=21)
    out, res = _run(tgt, tok, par)
    _compare(out, res)
