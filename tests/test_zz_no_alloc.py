"""sv_verify_accept_noalloc: the accept step on the library's fixed
per-device workspace, for callers that cannot allocate device memory.

Checked against sv_verify_accept (caller's workspace) on the same inputs:
the two run the same kernels, so every output must be bitwise equal.  Two
calls in a row, the second with a smaller problem (the fixed array keeps the
first call's contents).
"""
import pytest

pytestmark = pytest.mark.gpu


def _outs(torch, B, k, dev):
    return {"tokens": torch.full((B, k + 1), -7, dtype=torch.int32, device=dev),
            "n_acc": torch.full((B,), -7, dtype=torch.int32, device=dev),
            "status": torch.full((B,), -7, dtype=torch.int32, device=dev),
            "p_at": torch.full((B, k), float("nan"), dtype=torch.float32, device=dev),
            "q_at": torch.full((B, k), float("nan"), dtype=torch.float32, device=dev),
            "lse": torch.full((B, 2 * k + 1), float("nan"), dtype=torch.float32, device=dev)}


@pytest.mark.parametrize("shapes", [((64, 32, 152000), (4, 8, 1000))])
def test_noalloc_matches_workspace_entry_point(shapes):
    import torch
    import verify_pass_sv_amd as sv
    from verify_pass_sv_amd import synth
    dev = torch.device("cuda:0")
    for call, (B, k, V) in enumerate(shapes):
        print(f"noalloc call {call}: B={B} k={k} V={V}", flush=True)
        assert sv.sv_verify_accept_workspace_bytes(B, k, V) <= \
            sv.sv_verify_accept_noalloc_max_bytes()
        tgt, dft, tok = synth.accept_inputs(B, k, V, seed=500 + call, sigma=1.0, device=dev)
        ref = sv.sv_verify_accept(tgt, dft, tok, seed=9 + call, offset=3,
                                  out=_outs(torch, B, k, dev))
        got = sv.sv_verify_accept_noalloc(tgt, dft, tok, seed=9 + call, offset=3,
                                          out=_outs(torch, B, k, dev))
        torch.cuda.synchronize()
        for name in ("tokens", "n_acc", "status"):
            assert torch.equal(got[name], ref[name]), name
        for name in ("p_at", "q_at", "lse"):
            assert torch.equal(got[name].view(torch.int32), ref[name].view(torch.int32)), name
        assert (got["status"] == 0).all()


def test_noalloc_rejects_sizes_beyond_the_array():
    import torch
    import verify_pass_sv_amd as sv
    dev = torch.device("cuda:0")
    B, k, V = 256, 32, 152000
    assert sv.sv_verify_accept_workspace_bytes(B, k, V) > sv.sv_verify_accept_noalloc_max_bytes()
    t = torch.zeros((B, k + 1, V), dtype=torch.float32, device=dev)
    d = torch.zeros((B, k, V), dtype=torch.float32, device=dev)
    tok = torch.zeros((B, k), dtype=torch.int32, device=dev)
    out = _outs(torch, B, k, dev)
    with pytest.raises(sv.SvError) as e:
        sv.sv_verify_accept_noalloc(t, d, tok, seed=0, out=out)
    assert e.value.status == 5                       # SV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out["n_acc"] == -7).all()                # nothing was enqueued
