"""GPU parity of the verify pass in model order (sv_pass_chain_plan +
sv_pass_run): a chain of W4 GEMMs, each handing bf16(alpha * y) to the next,
run in one launch with device-wide phase barriers.

Source: Karpathy's Trick for Faster Local LLMs, "How Uzu optimizes bytes and
tokens per pass" (the forward pass hands intermediate values from layer to
layer) and "Why batch-one decoding is memory-bound".

What is compared how (the oracle only ever sees seeded inputs):
* Links whose x is a seeded input (every link of the independent-link test,
  the first link of every chain): y against the binary64 oracle row-wise at
  2e-3, xo inside the oracle's hand-off of the binary64 y widened by its
  error bound.
* Every link: the hand-off rounds the kernel's binary32 y to bf16, so xo
  must equal the binary32 -> bf16 round-to-nearest-even of fl32(alpha y) of
  the link's own y, bit for bit (torch's conversion, the library routine the
  oracle's bf16_rne is pinned to); and y must be the product of the x the
  chain handed to the link (numpy, with the oracle's dequantized weights of
  the seeded codes) at 2e-3 -- a link that ran before its input was written
  reads the NaN the xo buffers are filled with and fails.
* The whole chain against the oracle's own trajectory (binary64 GEMMs, its
  hand-off of fl32(y)) from the same seeded first input: the trajectory is
  not unique (a bf16 re-rounding of a binary32 sum can fall on the other
  side of a rounding boundary than the binary64 sum's, and the difference
  spreads through later links), so y of link j must lie within
  2e-3 + j 2^-8 norm-wise per row of it (one bf16 half-unit, 2^-9, per
  hand-off, doubled).
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


def alpha_for(K):
    """Keeps chained activations near unit scale for the synthetic weights:
    E[w^2] = E[(c - z)^2] E[s^2] with c, z ~ U{0..15}, s ~ U(0.01, 0.05)."""
    ew2 = (2 * 255 / 12.0) * ((0.05 ** 3 - 0.01 ** 3) / (3 * 0.04))
    return float(np.float32(1.0 / np.sqrt(K * ew2)))


def _weights(N, K, seed):
    sv = _sv()
    codes, scales, zeros = synth.w4_matrix(N, K, seed=seed)
    pc, ps = sv.sv_w4_pack(*to_dev(codes, scales, zeros))
    return (codes.numpy(), scales.numpy(), zeros.numpy()), pc, ps


def _nan(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


def _rne_handoff(y32, alpha, cols):
    """bf16 bits of fl32(alpha * y[:, :cols]) by torch's binary32 -> bf16
    conversion (round to nearest even)."""
    y = torch.as_tensor(np.ascontiguousarray(np.asarray(y32, dtype=np.float32)[:, :cols]))
    return bf16_bits((y * torch.tensor(np.float32(alpha))).to(torch.bfloat16))


def _check_xo(xo_gpu, y64, y32, alpha, cols, what):
    """xo of a link with seeded input: the round-to-nearest-even hand-off of
    the kernel's binary32 y bit for bit, and inside the oracle's hand-off of
    the binary64 y widened by 2^-16 of the row's largest |y| (the binary32
    sums of the bias-128 codes stay within about 1e-6 of it)."""
    got = bf16_bits(xo_gpu)
    assert np.array_equal(got, _rne_handoff(y32, alpha, cols)), f"{what}: xo != hand-off"
    err = np.abs(y64).max(axis=1, keepdims=True) * 2.0 ** -16
    lo, hi = oracle.chain_glue_candidates(y64, err, alpha, cols)
    g, a, b = (oracle.bf16_bits_to_f64(v) for v in (got, lo, hi))
    assert np.all((a <= g) & (g <= b)), f"{what}: xo outside the rounding interval of y"


# (K, N, xo_cols): one 128-k block (7 of 8 waves idle), a partial window of 5
# blocks, two partial windows, four full windows; 40 to 240 tiles (the grid
# is 40 workgroups: 1 to 6 tiles each, two rounds at m > 16)
LINKS = [(640, 1920, 640), (128, 640, 640), (1920, 640, 0), (4096, 3840, 1920),
         (1152, 1280, 1280)]


@pytest.mark.parametrize("m", [1, 5, 16, 17, 32])
def test_chain_links_match_oracle(m):
    """Independent links (no barrier): every y and xo from seeded inputs."""
    sv = _sv()
    links, refs = [], []
    for i, (K, N, cols) in enumerate(LINKS):
        host, pc, ps = _weights(N, K, seed=700 + 13 * i + m)
        x = synth.activations(m, K, seed=800 + i + m)
        y = _nan((m, N), torch.float32)
        xo = _nan((m, cols), torch.bfloat16) if cols else None
        a = alpha_for(K)
        links.append((x.to(DEV), pc, ps, N, y, xo, a))
        refs.append((x, host, a, cols))
    p = sv.sv_pass_chain_plan(links)
    assert p.grid == 40 and p.info.chain == 1
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p) == 0
    for (K, N, cols), (x, pc, ps, _, y, xo, a), (xh, host, _a, _c) in zip(LINKS, links, refs):
        xb = bf16_bits(xh)
        y64 = oracle.qgemm_w4(xb, *host)
        got = y.cpu().numpy()
        assert np.isfinite(got).all()
        assert_rows_close(got, y64, what=f"chain link m={m} K={K} N={N}")
        if cols:
            _check_xo(xo.cpu(), y64, got, a, cols, f"m={m} K={K} N={N}")


# Rounds longer than the weight ring: ragged k-block counts (35 and 19
# blocks: the last step of some waves is empty), 1, 2 and 6 tiles per
# workgroup, and a 96-block link (12 steps per wave).  The grid is 40
# workgroups.
LONG_LINKS = [(256, 640, 640), (4480, 640, 640), (2432, 1280, 1280), (12288, 640, 640),
              (4096, 3840, 0), (640, 640, 0)]


@pytest.mark.parametrize("m", [1, 16, 17])
def test_chain_long_rounds_match_oracle(m):
    sv = _sv()
    links, refs = [], []
    for i, (K, N, cols) in enumerate(LONG_LINKS):
        host, pc, ps = _weights(N, K, seed=900 + 17 * i + m)
        x = synth.activations(m, K, seed=950 + i + m)
        y = _nan((m, N), torch.float32)
        xo = _nan((m, cols), torch.bfloat16) if cols else None
        a = alpha_for(K)
        links.append((x.to(DEV), pc, ps, N, y, xo, a))
        refs.append((x, host, a, cols))
    p = sv.sv_pass_chain_plan(links)
    assert p.grid == 40 and p.info.chain == 1
    for _ in range(2):                                  # the same plan twice
        sv.sv_pass_run(p)
        torch.cuda.synchronize()
        assert sv.sv_pass_status(p) == 0
        for (K, N, cols), (x, pc, ps, _, y, xo, a), (xh, host, _a, _c) in zip(LONG_LINKS, links, refs):
            y64 = oracle.qgemm_w4(bf16_bits(xh), *host)
            got = y.cpu().numpy()
            assert np.isfinite(got).all()
            assert_rows_close(got, y64, what=f"chain link m={m} K={K} N={N}")
            if cols:
                _check_xo(xo.cpu(), y64, got, a, cols, f"m={m} K={K} N={N}")
            y.fill_(float("nan"))


def _decoder_chain(layers, m, H, F, seed, h0=None):
    """qkv -> o -> gate|up -> down per layer; each link's x is the previous
    link's xo (q, gate and down part as the hand-off)."""
    h = h0 if h0 is not None else synth.activations(m, H, seed=seed).to(DEV)
    links, hosts = [], []
    for layer in range(layers):
        for i, (N, K, cols) in enumerate(((3 * H, H, H), (H, H, H), (2 * F, H, F), (H, F, H))):
            host, pc, ps = _weights(N, K, seed=seed + 1000 * layer + i)
            xo = _nan((m, cols), torch.bfloat16)
            links.append((h, pc, ps, N, _nan((m, N), torch.float32), xo, alpha_for(K)))
            hosts.append(host)
            h = xo
    return links, hosts


def _as_f64(x):
    return x.detach().cpu().to(torch.float64).numpy()


def _check_chain(links, hosts):
    """Each link against its own input (property) and the chain against the
    oracle's trajectory from the same first input (independent)."""
    xo_ref = None
    for j, ((x, pc, ps, N, y, xo, a), host) in enumerate(zip(links, hosts)):
        w64 = oracle.dequant_w4(*host)                     # seeded codes only
        got = y.cpu().numpy()
        assert np.isfinite(got).all(), f"link {j}: unwritten or NaN-fed outputs"
        assert_rows_close(got, _as_f64(x) @ w64.T, what=f"chain link {j} N={N} (own input)")
        cols = xo.shape[1]
        assert np.array_equal(bf16_bits(xo), _rne_handoff(got, a, cols)), \
            f"link {j}: xo is not the hand-off of y"
        # the oracle's trajectory
        xin = bf16_bits(x) if j == 0 else xo_ref
        y64 = oracle.qgemm_w4(xin, *host)
        assert_rows_close(got, y64, rtol=2e-3 + j * 2.0 ** -8,
                          what=f"chain link {j} N={N} (oracle trajectory)")
        xo_ref = oracle.chain_glue(y64.astype(np.float32), a, cols)


@pytest.mark.parametrize("m", [1, 16, 32])
def test_chain_two_layers_in_order(m):
    sv = _sv()
    H, F = 640, 1920
    links, hosts = _decoder_chain(2, m, H, F, seed=900 + m)
    p = sv.sv_pass_chain_plan(links)
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p) == 0
    _check_chain(links, hosts)
    # the first link's xo against the binary64 result of its seeded input
    x0 = links[0][0].cpu()
    y64 = oracle.qgemm_w4(bf16_bits(x0), *hosts[0])
    _check_xo(links[0][5].cpu(), y64, links[0][4].cpu().numpy(), links[0][6], H, "first link")
    # launches again: same bits (fixed-order sums; the barrier counters carry
    # over from launch to launch)
    first = [(l[4].clone(), l[5].clone()) for l in links]
    for l in links:
        l[5].fill_(float("nan"))
    for _ in range(2):
        sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p) == 0
    for (y0, xo0), l in zip(first, links):
        assert torch.equal(y0, l[4]) and torch.equal(xo0.view(torch.int16), l[5].view(torch.int16))


def test_chain_graph_replays():
    """Captured once, replayed three times with eager work in between; every
    replay reproduces the eager result bit for bit."""
    sv = _sv()
    links, hosts = _decoder_chain(2, 16, 640, 1920, seed=1700)
    p = sv.sv_pass_chain_plan(links)
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    want = [(l[4].clone(), l[5].view(torch.int16).clone()) for l in links]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sv.sv_pass_run(p, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for l in links:
            l[4].fill_(float("nan"))
            l[5].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = torch.randn(1024, device=DEV).sum().item()     # eager work between replays
        for (y0, xo0), l in zip(want, links):
            assert torch.equal(y0, l[4]), f"replay {rep}"
            assert torch.equal(xo0, l[5].view(torch.int16)), f"replay {rep}"
    assert sv.sv_pass_status(p) == 0


@pytest.mark.parametrize("m", [16, 1, 32])
def test_chain_9b_stack_sampled(m):
    """The 32-layer, 3.93 GB stack chained in model order at k = m, in the
    launch configuration of the benchmark (k = 16) and of its k sweep (k = 1;
    k = 32, where gate/up runs as two rounds): 16 sampled channels of every y
    against the product of the link's actual input with the oracle's
    dequantized weights (the first link against the oracle outright), every
    xo bit-exactly the hand-off of its y."""
    sv = _sv()
    H, F = 4096, 12288
    h = synth.activations(m, H, seed=11, device=DEV)
    links, hosts, samples = [], [], []
    rng = np.random.default_rng(2025)
    for layer in range(32):
        for i, (N, K, cols) in enumerate(((3 * H, H, H), (H, H, H), (2 * F, H, F), (H, F, H))):
            c, s, z = synth.w4_matrix(N, K, seed=1000 * layer + i, device=DEV)
            pc, ps = sv.sv_w4_pack(c, s, z)
            rows = np.sort(rng.choice(N, size=16, replace=False))
            ri = torch.as_tensor(rows, device=DEV)
            samples.append((rows, c[ri].cpu().numpy(), s[ri].cpu().numpy(), z[ri].cpu().numpy()))
            del c, s, z
            xo = _nan((m, cols), torch.bfloat16)
            links.append((h, pc, ps, N, _nan((m, N), torch.float32), xo, alpha_for(K)))
            h = xo
    p = sv.sv_pass_chain_plan(links)
    assert p.grid == torch.cuda.get_device_properties(0).multi_processor_count
    for _ in range(2):
        sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p) == 0
    for j, ((x, pc, ps, N, y, xo, a), (rows, c, s, z)) in enumerate(zip(links, samples)):
        got = y.cpu().numpy()
        assert np.isfinite(got).all(), f"link {j}"
        ref = _as_f64(x) @ oracle.dequant_w4(c, s, z).T
        assert_rows_close(got[:, rows], ref, what=f"9B chain link {j} N={N}")
        assert np.array_equal(bf16_bits(xo), _rne_handoff(got, a, xo.shape[1])), j
        if j == 0:
            y64 = oracle.qgemm_w4(bf16_bits(x), c, s, z)
            assert_rows_close(got[:, rows], y64, what="9B chain first link (oracle)")
    # the hand-offs stay at unit scale through 128 links
    last = oracle.bf16_bits_to_f64(bf16_bits(links[-1][5]))
    assert 0.2 < np.sqrt((last ** 2).mean()) < 5.0


def test_stale_plan_is_refused_and_reported():
    sv = _sv()
    m = 5
    links, _ = _decoder_chain(1, m, 640, 1920, seed=77)
    p1 = sv.sv_pass_chain_plan(links)
    # (1) the buffer planned again (other rows): the old descriptor is refused
    # before any launch
    links3, _ = _decoder_chain(1, 3, 640, 1920, seed=78)
    buf = p1.plan[(-p1.plan.data_ptr()) % 256:]
    p2 = sv.sv_pass_chain_plan(links3, plan=buf)
    with pytest.raises(sv.SvError):
        sv.sv_pass_run(p1)
    sv.sv_pass_run(p2)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p2) == 0
    # (2) a descriptor that no longer matches the plan in its buffer (here
    # its row count): the kernel computes nothing and reports it
    for l in links3:
        l[4].fill_(float("nan"))
    p2.info.m = 4
    sv.sv_pass_run(p2)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p2) == sv.PASS_STATUS_STALE
    assert all(torch.isnan(l[4]).all() for l in links3)
    # (3) the unordered executor refuses a re-planned buffer as well
    g = [(links[0][0], links[0][1], links[0][2], links[0][3], links[0][4])]
    q1 = sv.sv_pass_plan("w4", g)
    sv.sv_pass_plan("w4", g, plan=q1.plan)
    with pytest.raises(sv.SvError):
        sv.sv_pass_run(q1)


def test_barrier_timeout_is_reported_and_the_launch_ends():
    """Forced from the host: the plan's barrier targets are raised past what
    the launch can reach and its poll bound lowered to 64, so the first
    waiting link gives up; every workgroup ends, the status word says so, and
    a plan made again runs normally."""
    sv = _sv()
    links, hosts = _decoder_chain(1, 16, 640, 1920, seed=91)
    p = sv.sv_pass_chain_plan(links)
    base = (-p.plan.data_ptr()) % 256
    hdr = p.plan[base:base + 128]
    words = hdr.view(torch.int32)
    words[8] = 64                                   # spin_limit
    words[10:26] = 1 << 20                          # workgroups per barrier counter
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p) & sv.PASS_STATUS_TIMEOUT
    p = sv.sv_pass_chain_plan(links)
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p) == 0
    _check_chain(links, hosts)


def alpha_for_w8(K):
    """The same for the synthetic W8 weights: E[w^2] = E[c^2] E[s^2] with c
    uniform on -127..127 (E[c^2] = 127 * 128 / 3) and s ~ U(0.01, 0.05)."""
    ew2 = (127 * 128 / 3.0) * ((0.05 ** 3 - 0.01 ** 3) / (3 * 0.04))
    return float(np.float32(1.0 / np.sqrt(K * ew2)))


def _weights8(N, K, seed):
    codes, scales = synth.w8_matrix(N, K, seed=seed)
    sv = _sv()
    return (codes.numpy(), scales.numpy()), sv.sv_w8_pack(codes.to(DEV)), scales.to(DEV)


@pytest.mark.parametrize("m", [1, 16, 17, 32])
def test_w8_chain_links_match_oracle(m):
    """The W8 chain on independent links (one to six tiles per workgroup, two
    rounds at m > 16, ragged k-block counts): every y against the oracle's W8
    GEMM, every xo bit-exactly the hand-off of its y."""
    sv = _sv()
    links, refs = [], []
    for i, (K, N, cols) in enumerate(LINKS + LONG_LINKS[1:3]):
        host, pc, sc = _weights8(N, K, seed=1300 + 7 * i + m)
        x = synth.activations(m, K, seed=1400 + i + m)
        y = _nan((m, N), torch.float32)
        xo = _nan((m, cols), torch.bfloat16) if cols else None
        a = alpha_for_w8(K)
        links.append((x.to(DEV), pc, sc, N, y, xo, a))
        refs.append((x, host, a, cols))
    p = sv.sv_pass_chain_plan(links, fmt="w8")
    assert p.grid == 40 and p.info.chain == 1
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p) == 0
    for (x, pc, sc, N, y, xo, a), (xh, host, _a, cols) in zip(links, refs):
        y64 = oracle.qgemm_w8(bf16_bits(xh), *host)
        got = y.cpu().numpy()
        assert np.isfinite(got).all()
        assert_rows_close(got, y64, what=f"W8 chain link m={m} K={xh.shape[1]} N={N}")
        if cols:
            assert np.array_equal(bf16_bits(xo), _rne_handoff(got, a, cols)), (m, N)


def test_w8_chain_9b_stack_sampled():
    """The 32-layer W8 stack (6.98 GB) in model order at k = 16: 16 sampled
    channels of every y against the link's actual input times the oracle's
    dequantized weights, the first link against the oracle outright, every xo
    the hand-off of its y."""
    sv = _sv()
    H, F, m = 4096, 12288, 16
    h = synth.activations(m, H, seed=21, device=DEV)
    links, samples = [], []
    rng = np.random.default_rng(2026)
    for layer in range(32):
        for i, (N, K, cols) in enumerate(((3 * H, H, H), (H, H, H), (2 * F, H, F), (H, F, H))):
            c, s = synth.w8_matrix(N, K, seed=3000 + 10 * layer + i, device=DEV)
            pc = sv.sv_w8_pack(c)
            rows = np.sort(rng.choice(N, size=16, replace=False))
            ri = torch.as_tensor(rows, device=DEV)
            samples.append((rows, c[ri].cpu().numpy(), s[ri].cpu().numpy()))
            del c
            xo = _nan((m, cols), torch.bfloat16)
            links.append((h, pc, s, N, _nan((m, N), torch.float32), xo, alpha_for_w8(K)))
            h = xo
    p = sv.sv_pass_chain_plan(links, fmt="w8")
    sv.sv_pass_run(p)
    torch.cuda.synchronize()
    assert sv.sv_pass_status(p) == 0
    for j, ((x, pc, s, N, y, xo, a), (rows, c, sc)) in enumerate(zip(links, samples)):
        got = y.cpu().numpy()
        assert np.isfinite(got).all(), f"link {j}"
        ref = _as_f64(x) @ oracle.dequant_w8(c, sc).T
        assert_rows_close(got[:, rows], ref, what=f"W8 9B chain link {j} N={N}")
        assert np.array_equal(bf16_bits(xo), _rne_handoff(got, a, xo.shape[1])), j
        if j == 0:
            assert_rows_close(got[:, rows], oracle.qgemm_w8(bf16_bits(x), c, sc),
                              what="W8 9B chain first link (oracle)")
