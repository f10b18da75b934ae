"""GPU parity of the fused LM-head verify against the oracle (oracle.lmhead).

* The softmax-statistics epilogue of the pass executor (sv_pass_gemm.stats)
  in all three formats: the group maxima and sums against the binary64
  statistics of the oracle's product, and against the kernel's own outputs
  (the maximum is the exact maximum of the written y).
* sv_verify_accept_stats on given statistics against oracle.accept.
* The fused verify -- a W4 vocabulary projection with the epilogue, then
  sv_verify_accept_stats -- against oracle.lmhead.lm_head_verify, from
  several tiles with ragged groups up to the full 152 000-entry vocabulary.
Accept decisions and tokens are bit-exact except at the oracle's flagged
near ties.
"""
import numpy as np
import pytest
import torch

import oracle
from verify_pass_sv_amd import synth
from gpu_util import DEV, to_dev, bf16_bits, assert_rows_close

pytestmark = pytest.mark.gpu


def _sv():
    import verify_pass_sv_amd as sv
    return sv


def _check_stats(st, y_ref, y_gpu, what):
    """st [m, G, 2] from the kernel; y_ref binary64 [m, N]; y_gpu the kernel's y."""
    M, S, bad = oracle.group_softmax_stats(y_ref)
    assert not bad.any()
    gm, gs = st[..., 0].astype(np.float64), st[..., 1].astype(np.float64)
    assert np.all(np.abs(gm - M) <= 1e-4 * (1 + np.abs(M))), what
    assert np.allclose(gs, S, rtol=2e-4, atol=0), what
    # consistency with the kernel's own outputs (a property of the kernel's
    # y, computed here, not by the oracle): each group's maximum is one of
    # its y values exactly, and its sum of exp(y - M) matches
    yg = y_gpu.astype(np.float64)
    m_, n_ = yg.shape
    for g in range(gm.shape[1]):
        blk = yg[:, 64 * g:min(n_, 64 * g + 64)]
        mg = blk.max(axis=1)
        assert np.array_equal(gm[:, g], mg), what
        sg = np.exp(blk - mg[:, None]).sum(axis=1)
        assert np.allclose(gs[:, g], sg, rtol=1e-5, atol=0), what


# (K, N): ragged 64-groups (N % 64 = 48, 32, 16), one group, several items
STATS_SHAPES = [(512, 1008), (256, 64), (1024, 4000), (640, 528)]


@pytest.mark.parametrize("fmt", ["w4", "w8", "w4_i8"])
@pytest.mark.parametrize("m", [1, 5, 16, 17, 32])
def test_stats_epilogue_matches_oracle(fmt, m):
    sv = _sv()
    gemms, refs = [], []
    for i, (K, N) in enumerate(STATS_SHAPES):
        seed = 1300 + 17 * i + m
        y = torch.full((m, N), float("nan"), dtype=torch.float32, device=DEV)
        st = torch.full((m, (N + 63) // 64, 2), float("nan"), dtype=torch.float32, device=DEV)
        if fmt == "w8":
            codes, scales = synth.w8_matrix(N, K, seed=seed)
            x = synth.activations(m, K, seed=seed + 1, scale=0.3)
            gemms.append((x.to(DEV), sv.sv_w8_pack(codes.to(DEV)), scales.to(DEV), N, y, st))
            refs.append(lambda x=x, c=codes, s=scales: oracle.qgemm_w8(bf16_bits(x), c.numpy(),
                                                                       s.numpy()))
        else:
            codes, scales, zeros = synth.w4_matrix(N, K, seed=seed)
            pc, ps = sv.sv_w4_pack(*to_dev(codes, scales, zeros))
            if fmt == "w4":
                x = synth.activations(m, K, seed=seed + 1, scale=0.15)
                gemms.append((x.to(DEV), pc, ps, N, y, st))
                refs.append(lambda x=x, c=codes, s=scales, z=zeros: oracle.qgemm_w4(
                    bf16_bits(x), c.numpy(), s.numpy(), z.numpy()))
            else:
                xq, xs = synth.int8_activations(m, K, seed=seed + 1)
                gemms.append((xq.to(DEV), xs.to(DEV), pc, ps, N, y, st))
                refs.append(lambda xq=xq, xs=xs, c=codes, s=scales, z=zeros: oracle.qgemm_w4_i8(
                    xq.numpy(), xs.numpy(), c.numpy(), s.numpy(), z.numpy()))
    p = sv.sv_pass_plan(fmt, gemms)
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    for (K, N), g, ref in zip(STATS_SHAPES, gemms, refs):
        y_ref = ref()
        y = g[-2].cpu().numpy()
        assert_rows_close(y, y_ref, what=f"{fmt} m={m} N={N}")
        _check_stats(g[-1].cpu().numpy(), y_ref, y, f"{fmt} m={m} K={K} N={N}")


def test_stats_only_where_asked():
    sv = _sv()
    m, K, N = 16, 512, 1024
    codes, scales, zeros = synth.w4_matrix(N, K, seed=5)
    pc, ps = sv.sv_w4_pack(*to_dev(codes, scales, zeros))
    x = synth.activations(m, K, seed=6, scale=0.15).to(DEV)
    y1 = torch.empty((m, N), device=DEV)
    y2 = torch.empty((m, N), device=DEV)
    st = torch.full((m, N // 64, 2), -7.0, device=DEV)
    guard = torch.full((m, N // 64, 2), -7.0, device=DEV)
    p = sv.sv_pass_plan("w4", [(x, pc, ps, N, y1, st), (x, pc, ps, N, y2)])
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert not torch.equal(st, guard) and torch.equal(guard, torch.full_like(guard, -7.0))


def _ties(res, tokens, n_acc, status, tol=None):
    """Compare GPU outputs with oracle results.  Trials with a flagged accept
    decision are skipped; a flagged residual draw must be valid: with
    tol = the oracle's residual width, the GPU's token is one whose bin lies
    within tol S of the threshold (otherwise it must equal the oracle's).
    Returns the number of trials skipped."""
    skipped = 0
    for b, r in enumerate(res):
        assert status[b] == r.status, (b, status[b], r.status)
        if r.status != 0:
            continue
        if r.accept_flags.any() or (r.residual_flag and tol is None):
            skipped += 1
            continue
        assert n_acc[b] == r.n_acc, (b, n_acc[b], r.n_acc)
        assert tokens[b, :r.n_acc].tolist() == r.tokens[:r.n_acc], b
        assert np.all(tokens[b, r.n_out:] == -1)
        v = int(tokens[b, r.n_acc])
        if not r.residual_flag:
            assert v == r.tokens[-1], (b, v, r.tokens[-1])
        else:
            csum, thr = r.extra["residual_csum"], r.extra["residual_thr"]
            S = csum[-1]
            lo = csum[v - 1] if v > 0 else 0.0
            assert lo - tol * S <= thr <= csum[v] + tol * S, (b, v, r.tokens[-1])
    return skipped


def test_accept_with_given_statistics_matches_oracle():
    sv = _sv()
    B, k, V = 48, 5, 3000
    tgt, dft, tok = synth.accept_inputs(B, k, V, seed=31, sigma=1.0)
    M, S, bad = oracle.group_softmax_stats(tgt.numpy())
    st = torch.from_numpy(np.stack([M, S], axis=-1).astype(np.float32))
    st[3, 2, 10, 1] = float("nan")        # an invalid group makes trial 3 invalid
    t, d, kk, s_ = to_dev(tgt, dft, tok, st)
    out = sv.sv_verify_accept_stats(t, s_, d, kk, seed=4, offset=2, diagnostics=True)
    ref = sv.sv_verify_accept(t, d, kk, seed=4, offset=2, diagnostics=True)
    torch.cuda.synchronize()
    res = oracle.verify_accept(tgt.numpy(), dft.numpy(), tok.numpy(), 4, 2, ties=(1e-5, 1e-5))
    res[3] = oracle.AcceptResult(status=2, n_acc=-1, tokens=[])
    flagged = _ties(res, out["tokens"].cpu().numpy(), out["n_acc"].cpu().numpy(),
                    out["status"].cpu().numpy())
    assert flagged <= 2
    assert out["n_acc"][3].item() == -1
    ok = [b for b in range(B) if b != 3]
    lse_a = out["lse"].cpu().numpy()[ok]
    lse_b = ref["lse"].cpu().numpy()[ok]
    assert np.allclose(lse_a, lse_b, rtol=1e-6, atol=1e-6)


def _head(V, K, seed):
    sv = _sv()
    codes, scales, zeros = synth.w4_matrix(V, K, seed=seed)
    pc, ps = sv.sv_w4_pack(*to_dev(codes, scales, zeros))
    return (codes.numpy(), scales.numpy(), zeros.numpy()), (pc, ps)


def _fused(B, k, V, K, seed, head=None):
    sv = _sv()
    m = B * (k + 1)
    host, (pc, ps) = head if head is not None else _head(V, K, seed)
    h = synth.activations(m, K, seed=seed + 1, scale=0.15)
    dft, tok = synth.lm_head_drafts(B, k, V, seed=seed + 2)
    y = torch.empty((m, V), dtype=torch.float32, device=DEV)
    st = torch.empty((m, (V + 63) // 64, 2), dtype=torch.float32, device=DEV)
    p = sv.sv_pass_plan("w4", [(h.to(DEV), pc, ps, V, y, st)])
    d, kk = to_dev(dft, tok)
    sv.sv_pass_run(p)
    out = sv.sv_verify_accept_stats(y.view(B, k + 1, V), st.view(B, k + 1, -1, 2), d, kk,
                                    seed=seed, offset=3)
    torch.cuda.synchronize()
    return h, dft, tok, host, y, st, out


@pytest.mark.parametrize("B,k,V,K", [(2, 7, 4000, 512), (3, 9, 1008, 256), (1, 31, 2048, 384),
                                     (16, 1, 640, 128)])
def test_fused_verify_matches_oracle(B, k, V, K):
    h, dft, tok, (c, s, z), y, st, out = _fused(B, k, V, K, seed=100 + V + k)
    logits, res = oracle.lm_head_verify(bf16_bits(h), c, s, z, dft.numpy(), tok.numpy(),
                                        seed=100 + V + k, offset=3)
    y = y.cpu().numpy()
    assert_rows_close(y, logits.reshape(-1, V), what="projection")
    _check_stats(st.cpu().numpy(), logits.reshape(-1, V), y, "fused stats")
    skipped = _ties(res, out["tokens"].cpu().numpy(), out["n_acc"].cpu().numpy(),
                    out["status"].cpu().numpy(), tol=oracle.NEAR_TIE_LMHEAD[1])
    assert skipped <= max(1, B // 4)
    assert any(r.n_acc > 0 for r in res) or B == 1     # the batch reaches past position 0


def test_fused_verify_full_vocabulary():
    # the 9B-class head: hidden 4096, vocabulary 152 000, 16 scored rows
    B, k, V, K = 1, 15, 152000, 4096
    h, dft, tok, (c, s, z), y, st, out = _fused(B, k, V, K, seed=7)
    logits, res = oracle.lm_head_verify(bf16_bits(h), c, s, z, dft.numpy(), tok.numpy(),
                                        seed=7, offset=3)
    y = y.cpu().numpy()
    assert_rows_close(y, logits.reshape(-1, V), what="152k projection")
    _check_stats(st.cpu().numpy(), logits.reshape(-1, V), y, "152k stats")
    skipped = _ties(res, out["tokens"].cpu().numpy(), out["n_acc"].cpu().numpy(),
                    out["status"].cpu().numpy(), tol=oracle.NEAR_TIE_LMHEAD[1])
    assert skipped == 0


def test_fused_equals_unfused_on_the_same_logits():
    sv = _sv()
    B, k, V, K = 2, 7, 4000, 512
    h, dft, tok, host, y, st, out = _fused(B, k, V, K, seed=55)
    d, kk = to_dev(dft, tok)
    ref = sv.sv_verify_accept(y.view(B, k + 1, V), d, kk, seed=55, offset=3)
    torch.cuda.synchronize()
    assert torch.equal(out["n_acc"], ref["n_acc"])
    assert torch.equal(out["tokens"], ref["tokens"])


def test_accept_stats_argument_errors():
    sv = _sv()
    B, k, V = 1, 2, 100
    t = torch.zeros((B, k + 1, V), device=DEV)
    d = torch.zeros((B, k, V), device=DEV)
    kk = torch.zeros((B, k), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        sv.sv_verify_accept_stats(t, torch.zeros((B, k + 1, 1, 2), device=DEV), d, kk, 0)
