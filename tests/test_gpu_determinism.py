"""Run-to-run determinism of the verification entry points and the passes.

Every reduction in the library has one fixed order (or, for histogram bins
filled by many threads at once, integer arithmetic that is exact in any
order), so repeating a call on the same inputs must reproduce every output
bit for bit: tokens, counts, statuses and the binary32 diagnostics.  Before
each repeat the workspace and the outputs are overwritten with random bytes
(their earlier contents must not matter).
"""
import pytest
import torch

from verify_pass_sv_amd import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu

REPEATS = 3


def _sv():
    import verify_pass_sv_amd as sv
    return sv


def _scramble(*ts):
    for t in ts:
        if t is not None:
            t.view(torch.uint8).random_(0, 256)


def _bits(out):
    return {n: (t.view(torch.int32) if t.dtype == torch.float32 else t).clone()
            for n, t in out.items()}


def _repeat(call, out, ws, repeats=REPEATS):
    """Runs call() `repeats` times, scrambling out and ws before each; returns
    the outputs' bit patterns of every run."""
    runs = []
    for _ in range(repeats):
        _scramble(ws, *out.values())
        call()
        torch.cuda.synchronize()
        runs.append(_bits(out))
    return runs


def _assert_same(runs, what):
    for r in runs[1:]:
        for n in runs[0]:
            assert torch.equal(r[n], runs[0][n]), f"{what}: output {n} differs between runs"


def _outs(B, k, extra=()):
    o = {"tokens": torch.empty((B, k + 1), dtype=torch.int32, device=DEV),
         "n_acc": torch.empty((B,), dtype=torch.int32, device=DEV),
         "status": torch.empty((B,), dtype=torch.int32, device=DEV)}
    for name, shape, dt in extra:
        o[name] = torch.empty(shape, dtype=dt, device=DEV)
    return o


@pytest.mark.parametrize("B,k,V", [(1, 32, 152000), (8, 32, 152000), (64, 4, 1000)])
def test_accept_repeats_bitwise(B, k, V):
    sv = _sv()
    print(f"accept B={B} k={k} V={V}", flush=True)
    t, d, tok = synth.accept_inputs(B, k, V, seed=201, sigma=1.0, device=DEV)
    out = _outs(B, k, [("p_at", (B, k), torch.float32), ("q_at", (B, k), torch.float32),
                       ("lse", (B, 2 * k + 1), torch.float32)])
    ws = torch.empty(sv.sv_verify_accept_workspace_bytes(B, k, V), dtype=torch.uint8, device=DEV)
    runs = _repeat(lambda: sv.sv_verify_accept(t, d, tok, 5, 1, out=out, workspace=ws), out, ws)
    _assert_same(runs, "sv_verify_accept")
    assert (runs[0]["status"] == 0).all()


def _tied_rows(t, n_tied, seed):
    g = torch.Generator().manual_seed(seed)
    B, R, V = t.shape
    for b in range(B):
        for i in range(R):
            idx = torch.randperm(V, generator=g)[:n_tied].to(t.device)
            t[b, i, idx] = 3.0


@pytest.mark.parametrize("settings", [(0.7, 0, 0.9), (0.8, 100, 0.95), (1.0, 50, 1.0),
                                      (1.0, 0, 1.0), (0.0, 0, 1.0)],
                         ids=["T0.7_p0.9", "T0.8_k100_p0.95", "k50", "plain", "greedy"])
@pytest.mark.parametrize("B,k,V", [(1, 32, 152000), (8, 32, 152000)],
                         ids=["sliced_rows", "one_workgroup_per_row"])
def test_sampled_repeats_bitwise(settings, B, k, V):
    sv = _sv()
    print(f"sampled B={B} k={k} V={V} settings={settings}", flush=True)
    t, d, tok = synth.accept_inputs(B, k, V, seed=202, sigma=1.0, device=DEV)
    out = _outs(B, k, [("p_at", (B, k), torch.float32), ("q_at", (B, k), torch.float32)])
    ws = torch.empty(max(16, sv.sv_verify_sampled_workspace_bytes(B, k, V)), dtype=torch.uint8,
                     device=DEV)
    # sliced rows hand the histogram and the candidates between workgroups
    # of one launch: more repeats there
    runs = _repeat(lambda: sv.sv_verify_sampled(t, d, tok, 6, 2, *settings, out=out,
                                                workspace=ws), out, ws,
                   repeats=4 * REPEATS if B == 1 else REPEATS)
    _assert_same(runs, f"sv_verify_sampled {settings}")
    assert (runs[0]["status"] == 0).all()


@pytest.mark.parametrize("settings", [(1.0, 2600, 1.0), (0.9, 0, 0.3), (1.0, 4000, 0.5)],
                         ids=["radix_topk", "radix_topp", "radix_both"])
@pytest.mark.parametrize("B", [2, 40], ids=["sliced_rows", "one_workgroup_per_row"])
def test_sampled_radix_fallback_repeats_bitwise(settings, B):
    # 5000 tokens share one logit near the top of each row: the boundary bin
    # exceeds the LDS list and the radix passes run (binary64 digit masses)
    sv = _sv()
    k, V = 3, 20000
    print(f"sampled radix B={B} settings={settings}", flush=True)
    t, d, tok = synth.accept_inputs(B, k, V, seed=203, sigma=0.5, device=DEV)
    _tied_rows(t, 5000, 1)
    _tied_rows(d, 5000, 2)
    out = _outs(B, k, [("p_at", (B, k), torch.float32), ("q_at", (B, k), torch.float32)])
    ws = torch.empty(max(16, sv.sv_verify_sampled_workspace_bytes(B, k, V)), dtype=torch.uint8,
                     device=DEV)
    runs = _repeat(lambda: sv.sv_verify_sampled(t, d, tok, 7, 0, *settings, out=out,
                                                workspace=ws), out, ws)
    _assert_same(runs, f"sv_verify_sampled radix {settings}")


@pytest.mark.parametrize("B,k,V", [(1, 32, 152000), (8, 32, 152000)])
def test_coupled_repeats_bitwise(B, k, V):
    sv = _sv()
    print(f"coupled B={B} k={k} V={V}", flush=True)
    t, _, tok = synth.accept_inputs(B, k, V, seed=204, sigma=1.0, device=DEV)
    out = _outs(B, k, [("choices", (B, k + 1), torch.int32)])
    ws = torch.empty(max(16, sv.sv_verify_coupled_workspace_bytes(B, k, V)), dtype=torch.uint8,
                     device=DEV)
    runs = _repeat(lambda: sv.sv_verify_coupled(t, tok, 8, 3, out=out, workspace=ws), out, ws)
    _assert_same(runs, "sv_verify_coupled")
    assert (runs[0]["status"] == 0).all()


@pytest.mark.parametrize("B,n,V", [(1, 32, 152000), (8, 16, 152000)])
def test_tree_repeats_bitwise(B, n, V):
    sv = _sv()
    print(f"tree B={B} n={n} V={V}", flush=True)
    t, tk, par = synth.tree_inputs(B, n, V, seed=205, device=DEV)
    out = _outs(B, n, [("path", (B, n), torch.int32)])
    ws = torch.empty(max(16, sv.sv_verify_tree_workspace_bytes(B, n, V)), dtype=torch.uint8,
                     device=DEV)
    runs = _repeat(lambda: sv.sv_verify_tree(t, tk, par, out=out, workspace=ws), out, ws)
    _assert_same(runs, "sv_verify_tree")
    assert (runs[0]["status"] == 0).all()


def _w4_links(sv, m, layers):
    H, F = 4096, 12288
    links, gemms = [], []
    h = synth.activations(m, H, seed=206, device=DEV)
    xf = synth.activations(m, F, seed=207, device=DEV)
    for layer in range(layers):
        for i, (N, K, cols) in enumerate(((3 * H, H, H), (H, H, H), (2 * F, H, F), (H, F, H))):
            c, s, z = synth.w4_matrix(N, K, seed=300 + 10 * layer + i, device=DEV)
            pc, ps = sv.sv_w4_pack(c, s, z)
            del c, s, z
            y = torch.empty((m, N), dtype=torch.float32, device=DEV)
            xo = torch.empty((m, cols), dtype=torch.bfloat16, device=DEV)
            links.append((h, pc, ps, N, y, xo, 0.05))
            gemms.append((h if K == H else xf, pc, ps, N,
                          torch.empty((m, N), dtype=torch.float32, device=DEV)))
            h = xo
    return links, gemms


@pytest.mark.parametrize("m", [1, 16, 32])
def test_passes_repeat_bitwise(m):
    # the chain (model order) and the unordered executor: every output
    # element is one fixed-order sum of the partial sums of 8 waves
    sv = _sv()
    print(f"passes m={m}", flush=True)
    links, gemms = _w4_links(sv, m, 2)
    chain = sv.sv_pass_chain_plan(links)
    flat = sv.sv_pass_plan("w4", gemms)
    outs = [l[4] for l in links] + [l[5] for l in links] + [g[4] for g in gemms]
    runs = []
    for _ in range(REPEATS):
        _scramble(*outs)
        sv.sv_pass_run(chain)
        sv.sv_pass_run(flat)
        torch.cuda.synchronize()
        runs.append([o.view(torch.int16 if o.dtype == torch.bfloat16 else torch.int32).clone()
                     for o in outs])
    assert sv.sv_pass_status(chain) == 0
    for r in runs[1:]:
        for i, (a, b) in enumerate(zip(runs[0], r)):
            assert torch.equal(a, b), f"output {i} differs between runs"


@pytest.mark.parametrize("m", [1, 16, 32])
def test_single_gemms_repeat_bitwise(m):
    # the single-GEMM entry points on their streaming kernels: row-major and
    # packed W4, int8 x W4 and W8, on a 4096-channel and a 24576-channel matrix
    sv = _sv()
    print(f"single GEMMs m={m}", flush=True)
    for N, K in ((4096, 12288), (24576, 4096)):
        c, s, z = synth.w4_matrix(N, K, seed=N + K, device=DEV)
        pc, ps = sv.sv_w4_pack(c, s, z)
        c8, s8 = synth.w8_matrix(N, K, seed=N + K + 1, device=DEV)
        x = synth.activations(m, K, seed=K, device=DEV)
        xq, xs = synth.int8_activations(m, K, seed=K + 1, device=DEV)
        calls = {
            "w4": lambda y: sv.sv_qgemm_w4(x, c, s, z, y=y),
            "w4_packed": lambda y: sv.sv_qgemm_w4_packed(x, pc, ps, N, y=y),
            "w4_i8": lambda y: sv.sv_qgemm_w4_i8(xq, xs, c, s, z, y=y),
            "w8": lambda y: sv.sv_qgemm_w8(x, c8, s8, y=y),
        }
        for name, call in calls.items():
            y = torch.empty((m, N), dtype=torch.float32, device=DEV)
            runs = _repeat(lambda: call(y), {"y": y}, None)
            _assert_same(runs, f"{name} {N}x{K} m={m}")
