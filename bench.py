#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

One step = one verify pass of a synthetic 9B-class decoder weight stack
(32 layers, hidden 4096, FFN 12288; q/k/v/o 4096x4096, gate/up 4096x12288,
down 12288x4096; W4 asymmetric, group 64) at k = 16 bf16 draft rows, run in
MODEL ORDER -- per layer fused qkv -> o -> fused gate|up -> down, each GEMM
reading the bf16 hand-off of the one before (sv_pass_chain_plan; one launch,
a device-wide barrier between dependent GEMMs) -- followed by the
accept/correct call for those k drafts over a 152000-entry vocabulary.  The
step is captured in a HIP graph and replayed; inputs are resident in HBM
before timing starts.

Printed: one JSON line.  `value` is drafted tokens per second (k / step
time).  Extra fields report the weight stream of the ordered pass, the
roofline of its kernel, the same 128 GEMMs without ordering (the unordered
executor: an upper bound, not a model pass), the accept latency, the k sweeps
(W4 ordered and unordered, W8 unordered), the per-GEMM-launch variant, the
int8 path, accept statistics over 4096 trials per noise level, the measured
HBM read peak, a warm-up curve, and the CPU oracle baseline.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 200] [--quick]
       python bench.py --profile-pass [--format w4|w4_unordered|w8|w4_i8] [--k K]
                        (copy kernel, read probe and 40 executor passes, for
                         rocprofv3 counters)
       python bench.py --profile-accept [--k K] [--trials B]
                        (copy kernel and accept calls at V = 152000, for
                         rocprofv3 counters)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("verify-pass weight GB/s and drafted tokens/s at k=16, 9B-shape W4; accept µs")
WARMUP_CURVE_STEPS = 20
PROFILE_PASSES = 40


def handoff_alpha_w8(K):
    """The same for the synthetic W8 weights (codes uniform on -127..127,
    scales uniform on [0.01, 0.05]): E[w^2] = E[c^2] E[s^2]."""
    import numpy as np
    ew2 = (127 * 128 / 3.0) * ((0.05 ** 3 - 0.01 ** 3) / (3 * 0.04))
    return float(np.float32(1.0 / np.sqrt(K * ew2)))


def handoff_alpha(K):
    """Scale of the bf16 hand-off between chained GEMMs that keeps the
    activations near unit size for the synthetic weights (codes and zero
    points uniform on 0..15, scales uniform on [0.01, 0.05]):
    1 / sqrt(K E[w^2]), E[w^2] = E[(c - z)^2] E[s^2]."""
    import numpy as np
    ew2 = (2 * 255 / 12.0) * ((0.05 ** 3 - 0.01 ** 3) / (3 * 0.04))
    return float(np.float32(1.0 / np.sqrt(K * ew2)))
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2500.0
LAYERS, HIDDEN, FFN, GROUP = 32, 4096, 12288, 64
VOCAB = 152000


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- workloads --
def make_w4_stack(torch, synth, sv, dev, layers=LAYERS):
    """Per layer: fused qkv [3H, H], o [H, H], fused gate|up [2F, H], down [H, F];
    each matrix kept row-major and in the packed streaming layout."""
    shapes = [("qkv", 3 * HIDDEN, HIDDEN), ("o", HIDDEN, HIDDEN),
              ("gateup", 2 * FFN, HIDDEN), ("down", HIDDEN, FFN)]
    stack = []
    for l in range(layers):
        layer = []
        for i, (name, N, K) in enumerate(shapes):
            c, s, z = synth.w4_matrix(N, K, seed=1000 * l + i, device=dev)
            pc, ps = sv.sv_w4_pack(c, s, z)
            layer.append((name, N, K, c, s, z, pc, ps))
        stack.append(layer)
    return stack


def make_w8_stack(torch, synth, dev, layers=LAYERS):
    shapes = [("qkv", 3 * HIDDEN, HIDDEN), ("o", HIDDEN, HIDDEN),
              ("gateup", 2 * FFN, HIDDEN), ("down", HIDDEN, FFN)]
    stack = []
    for l in range(layers):
        layer = []
        for i, (name, N, K) in enumerate(shapes):
            c, s = synth.w8_matrix(N, K, seed=5000 + 1000 * l + i, device=dev)
            layer.append((name, N, K, c, s))
        stack.append(layer)
    return stack


def w4_bytes(stack):
    return sum(N * K // 2 + 4 * N * (K // GROUP) for layer in stack
               for (_, N, K, *_r) in layer)


def w8_bytes(stack):
    return sum(N * K + 2 * N for layer in stack for (_, N, K, *_r) in layer)


# ------------------------------------------------------------------- timing --
def time_graph(torch, fn, steps, warmup):
    """Capture fn() in a HIP graph, replay warmup + steps times; ms per replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # first eager call outside capture (one-time attribute setup)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, g


def recorded_traffic(name, k, kernel="pass_kernel"):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the copy-kernel reading), or None
    when it was taken at another k or on other kernel sources."""
    from verify_pass_sv_amd import rocprof_summary
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if f"_k{k}" not in name or rec.get("sources_sha256") != rocprof_summary.sources_sha256(
            kernel):
        return None
    return rec.get("traffic_bytes")


def recorded_counters(name):
    """The committed rocprofv3 summary's counters for the pass kernel (dict),
    or None when it was taken on other kernel sources."""
    from verify_pass_sv_amd import rocprof_summary
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("sources_sha256") != rocprof_summary.sources_sha256("pass_kernel"):
        return None
    return rec


def int8_quant_error(torch, sv, synth, layer, k, dev):
    """Relative error (Frobenius, over the layer's 4 products at k rows) of the
    int8 path against the bf16 path, with and without the rotation.  The
    stored 4-bit weights play the weights in the basis the activations are
    quantized in (rotated offline when the activations are rotated), so:
      with:    int8 path (sv_hadamard_i8 + sv_qgemm_w4_i8) vs sv_qgemm_w4 on
               the rotated activations rounded to bf16;
      without: per-token int8 of the raw activations + sv_qgemm_w4_i8 vs
               sv_qgemm_w4 on the raw activations.
    Torch forms only the measurement's baselines here (the rotation in
    binary32, by the Sylvester matrix, and the unrotated quantization); both
    products run in the library."""
    B4 = 4096
    idx = torch.arange(B4, device=dev)
    pc = torch.zeros((B4, B4), dtype=torch.int64, device=dev)
    a = idx[:, None] & idx[None, :]
    for _ in range(12):                         # popcount(i & j) parity
        pc ^= a & 1
        a = a >> 1
    H = (1 - 2 * pc).to(torch.float32) / 64.0   # orthonormal Sylvester matrix
    num = {"with_rotation": 0.0, "without_rotation": 0.0}
    den = {"with_rotation": 0.0, "without_rotation": 0.0}
    for i, (name, N, K, c, s_, z, *_r) in enumerate(layer):
        x = synth.outlier_activations(k, K, seed=900 + i, device=dev)[0]
        signs = synth.hadamard_signs(K, seed=901 + i, device=dev)
        xq, xs = sv.sv_hadamard_i8(x, signs, B4)
        y_q = sv.sv_qgemm_w4_i8(xq, xs, c, s_, z)
        xr = ((x.float() * signs.float()).view(k, K // B4, B4) @ H).view(k, K)
        y_r = sv.sv_qgemm_w4(xr.to(torch.bfloat16), c, s_, z)
        xf = x.float()
        s0 = (xf.abs().amax(dim=1) / 127.0).clamp_min(1e-30)
        xq0 = torch.round(xf / s0[:, None]).clamp(-127, 127).to(torch.int8)
        y_q0 = sv.sv_qgemm_w4_i8(xq0, s0.contiguous(), c, s_, z)
        y_0 = sv.sv_qgemm_w4(x, c, s_, z)
        for key, (yq, yr) in (("with_rotation", (y_q, y_r)), ("without_rotation", (y_q0, y_0))):
            num[key] += float(((yq - yr).double() ** 2).sum())
            den[key] += float((yr.double() ** 2).sum())
    torch.cuda.synchronize()
    return {key: round((num[key] / den[key]) ** 0.5, 5) for key in num}


# --------------------------------------------------------------- cpu oracle --
def cpu_baseline(k=16, min_seconds=6.0, accept_trials=8, dev=None):
    """The binary64 oracle on the host, timed on bounded samples of each
    workload (only the oracle calls are timed; synthetic inputs are made
    before each clock starts):

    * the headline: whole layers of the W4 stack at k rows (7 matrices,
      dequantize + matmul, rows in chunks), as many as fill about
      min_seconds, extrapolated to 32 layers, plus one accept trial at
      V = 152000 -> drafted tokens/s of one step;
    * the one-layer problem in full (K = 512, N = 1024, k = 4, accept over
      V = 1000);
    * one W8 layer and one int8-path layer (rotation + quantization + int8
      GEMM) at k rows, extrapolated to 32 layers;
    * accept at scale (V = 152000, k = 32): accept_trials trials per sigma in
      {0.1, 1, 3}, reported per trial (inputs drawn on `dev` when given).
    """
    import numpy as np
    import torch
    import oracle
    from verify_pass_sv_amd import synth
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = 1
    shapes = [(N, K) for _, N, K in oracle.decoder_stack_shapes(HIDDEN, FFN)]
    as_bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    xs = {K: as_bits(synth.activations(k, K, seed=7)) for K in (HIDDEN, FFN)}

    def chunks(n, step=2048):
        return [(r0, min(n, r0 + step)) for r0 in range(0, n, step)]

    # W4 layers
    t_layers, n_layers = 0.0, 0
    while n_layers < LAYERS and (n_layers == 0 or t_layers < min_seconds):
        mats = []
        for i, (N, K) in enumerate(shapes):
            c, s, z = synth.w4_matrix(N, K, seed=900 + 100 * n_layers + i)
            mats.append((K, c.numpy(), s.numpy(), z.numpy()))
        t0 = time.perf_counter()
        for K, c, s, z in mats:
            for r0, r1 in chunks(c.shape[0]):
                oracle.qgemm_w4(xs[K], c[r0:r1], s[r0:r1], z[r0:r1])
        t_layers += time.perf_counter() - t0
        n_layers += 1
        del mats
    t_layer = t_layers / n_layers
    tgt, dft, tok = synth.accept_inputs(1, k, VOCAB, seed=3, sigma=1.0)
    t1 = time.perf_counter()
    oracle.verify_accept(tgt.numpy(), dft.numpy(), tok.numpy(), seed=0)
    t_acc = time.perf_counter() - t1
    t_step = LAYERS * t_layer + t_acc
    del tgt, dft, tok

    # the one-layer problem, in full
    c, s, z = synth.w4_matrix(1024, 512, seed=1)
    x = as_bits(synth.activations(4, 512, seed=2))
    tt, td, tk = synth.accept_inputs(1, 4, 1000, seed=3, sigma=1.0)
    t0 = time.perf_counter()
    oracle.qgemm_w4(x, c.numpy(), s.numpy(), z.numpy())
    oracle.verify_accept(tt.numpy(), td.numpy(), tk.numpy(), seed=0)
    t_tiny = time.perf_counter() - t0

    # one W8 layer, one int8-path layer
    t_w8 = 0.0
    for i, (N, K) in enumerate(shapes):
        c, s = synth.w8_matrix(N, K, seed=5000 + i)
        c, s = c.numpy(), s.numpy()
        t0 = time.perf_counter()
        for r0, r1 in chunks(N):
            oracle.qgemm_w8(xs[K], c[r0:r1], s[r0:r1])
        t_w8 += time.perf_counter() - t0
    signs = {K: np.where(np.random.default_rng(K).random(K) < 0.5, -1, 1).astype(np.int8)
             for K in (HIDDEN, FFN)}
    t_i8 = 0.0
    for i, (N, K) in enumerate(shapes):
        c, s, z = synth.w4_matrix(N, K, seed=900 + i)
        c, s, z = c.numpy(), s.numpy(), z.numpy()
        t0 = time.perf_counter()
        xq, xsc, _ = oracle.hadamard_i8(xs[K], signs[K], 4096)
        for r0, r1 in chunks(N):
            oracle.qgemm_w4_i8(xq, xsc, c[r0:r1], s[r0:r1], z[r0:r1])
        t_i8 += time.perf_counter() - t0

    # accept at scale: V = 152000, k = 32, per sigma
    per_sigma = {}
    for sigma in (0.1, 1.0, 3.0):
        tt, td, tk = synth.accept_inputs(accept_trials, 32, VOCAB, seed=71, sigma=sigma,
                                         device=dev if dev is not None else "cpu")
        tt, td, tk = tt.cpu().numpy(), td.cpu().numpy(), tk.cpu().numpy()
        t0 = time.perf_counter()
        r = oracle.verify_accept(tt, td, tk, seed=0)
        per_sigma[str(sigma)] = {
            "us_per_trial": round((time.perf_counter() - t0) / accept_trials * 1e6, 1),
            "mean_accepted": round(float(np.mean([t.n_acc for t in r])), 3)}
        del tt, td, tk

    ext = lambda t: round(LAYERS * t, 2)
    return {"value": k / t_step, "unit": "drafted tokens/s", "cores": blas_threads,
            "kind": "oracle",
            "sample": (f"{n_layers} of 32 layers (7 W4 matrices each, k={k}, binary64 "
                       f"dequantize+matmul) timed {t_layers:.1f} s, {t_layer:.2f} s per layer "
                       f"extrapolated x32, plus 1 accept trial (V={VOCAB}, k={k}) "
                       f"{t_acc:.2f} s; {t_step:.1f} s per step"),
            "os_cpu_count": os.cpu_count(), "blas_threads": blas_threads,
            "tiny_full_s": round(t_tiny, 4),
            "tiny_full": "W4 K=512 N=1024 k=4 GEMM + accept over V=1000, timed in full",
            "w8_layer_s": round(t_w8, 3), "w8_pass_s_extrapolated_x32": ext(t_w8),
            "int8_layer_s": round(t_i8, 3), "int8_pass_s_extrapolated_x32": ext(t_i8),
            "accept_v152000_k32": per_sigma,
            "accept_sample": (f"{accept_trials} trials per sigma (a bounded sample; "
                              f"the 4096-trial statistics run in the test suite)")}


# --------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The clock and power controller of the GPU settles over a few hundred
    # passes; the defaults time the settled state (about 0.4 s in total).
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--k", type=int, default=16)
    ap.add_argument("--quick", action="store_true", help="skip sweeps, stats and cpu baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--format", default="w4", choices=("w4", "w4_unordered", "w8", "w4_i8"),
                    help="weight path of --profile-pass (w4: the pass in model order; the "
                         "others: every GEMM on a fixed input, no ordering)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="copy kernel + read probe + 40 eager passes, then exit")
    ap.add_argument("--profile-accept", action="store_true",
                    help="copy kernel + eager sv_verify_accept calls (V=152000), then exit")
    ap.add_argument("--trials", type=int, default=1,
                    help="B of --profile-accept and --profile-verify")
    ap.add_argument("--profile-verify", choices=("sampled", "coupled", "tree"),
                    help="copy kernel + eager calls of one verification rule "
                         "(V=152000; sampled at --sampling; tree with --k nodes), "
                         "then exit")
    ap.add_argument("--sampling", default="0.7,0,0.9",
                    help="temperature,top_k,top_p of --profile-verify sampled")
    ap.add_argument("--profile-single", action="store_true",
                    help="single-GEMM entry points (row-major and packed W4, int8 x W4, "
                         "W8) on 8 layers of the 9B shapes at --k rows, 13 rounds each, "
                         "then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import verify_pass_sv_amd as sv
    from verify_pass_sv_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    k = args.k

    if args.profile_accept:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        dst.copy_(src)  # plain copy kernel of 256 MiB (counter scale reference)
        B = args.trials
        t, d, tk = synth.accept_inputs(B, k, VOCAB, seed=31 + B, sigma=1.0, device=dev)
        out = {"tokens": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
               "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
               "status": torch.empty((B,), dtype=torch.int32, device=dev)}
        ws = torch.empty(sv.sv_verify_accept_workspace_bytes(B, k, VOCAB), dtype=torch.uint8,
                         device=dev)
        calls = 20 if B == 1 else 4
        for i in range(calls):
            sv.sv_verify_accept(t, d, tk, seed=i, out=out, workspace=ws)
        torch.cuda.synchronize()
        log(f"profile-accept: {calls} calls at B={B}, k={k}, V={VOCAB}")
        return
    if args.profile_single:
        # 8 layers x (qkv, o, gate|up, down), so that the weights of one round
        # (0.9-1.7 GB) come from HBM, not from the 256 MB memory-side cache
        shapes = [(3 * HIDDEN, HIDDEN), (HIDDEN, HIDDEN), (2 * FFN, HIDDEN), (HIDDEN, FFN)]
        xs = {K: synth.activations(k, K, seed=6 + K, device=dev) for K in (HIDDEN, FFN)}
        xq = {K: synth.int8_activations(k, K, seed=7 + K, device=dev) for K in (HIDDEN, FFN)}
        ys = {N: torch.empty((k, N), dtype=torch.float32, device=dev) for N, _ in shapes}
        w4, w8 = [], []
        for layer in range(8):
            for N, K in shapes:
                c, s_, z = synth.w4_matrix(N, K, seed=100 * layer + N + K, device=dev)
                pc, ps = sv.sv_w4_pack(c, s_, z)
                w4.append((N, K, c, s_, z, pc, ps))
                w8.append((N, K) + tuple(synth.w8_matrix(N, K, seed=100 * layer + N + K,
                                                         device=dev)))
        calls = {
            "sv_qgemm_w4": lambda: [sv.sv_qgemm_w4(xs[K], c, s_, z, y=ys[N])
                                    for (N, K, c, s_, z, pc, ps) in w4],
            "sv_qgemm_w4_packed": lambda: [sv.sv_qgemm_w4_packed(xs[K], pc, ps, N, y=ys[N])
                                           for (N, K, c, s_, z, pc, ps) in w4],
            "sv_qgemm_w4_i8": lambda: [sv.sv_qgemm_w4_i8(xq[K][0], xq[K][1], c, s_, z, y=ys[N])
                                       for (N, K, c, s_, z, pc, ps) in w4],
            "sv_qgemm_w8": lambda: [sv.sv_qgemm_w8(xs[K], c, s_, y=ys[N])
                                    for (N, K, c, s_) in w8],
        }
        torch.cuda.synchronize()
        for name, fn in calls.items():
            for _ in range(13):
                fn()
            torch.cuda.synchronize()
            log(f"profile-single: {name}, 13 rounds of 32 GEMMs at k={k}")
        return
    if args.profile_verify:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        dst.copy_(src)  # plain copy kernel of 256 MiB (counter scale reference)
        B, rule = args.trials, args.profile_verify
        out = {"tokens": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
               "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
               "status": torch.empty((B,), dtype=torch.int32, device=dev)}
        if rule == "tree":
            t, tk, par = synth.tree_inputs(B, k, VOCAB, seed=61 + B + k, device=dev)
            ws = torch.empty(max(16, sv.sv_verify_tree_workspace_bytes(B, k, VOCAB)),
                             dtype=torch.uint8, device=dev)
            call = lambda i: sv.sv_verify_tree(t, tk, par, out=out, workspace=ws)
        else:
            t, d, tk = synth.accept_inputs(B, k, VOCAB, seed=41 + B, sigma=1.0, device=dev)
            if rule == "sampled":
                ws = torch.empty(max(16, sv.sv_verify_sampled_workspace_bytes(B, k, VOCAB)),
                                 dtype=torch.uint8, device=dev)
                temp, top_k, top_p = args.sampling.split(",")
                setting = (float(temp), int(top_k), float(top_p))
                call = lambda i: sv.sv_verify_sampled(t, d, tk, i, 0, *setting, out=out,
                                                      workspace=ws)
            else:
                ws = torch.empty(max(16, sv.sv_verify_coupled_workspace_bytes(B, k, VOCAB)),
                                 dtype=torch.uint8, device=dev)
                call = lambda i: sv.sv_verify_coupled(t, tk, i, 0, out=out, workspace=ws)
        calls = 20 if B == 1 else 4
        for i in range(calls):
            call(i)
        torch.cuda.synchronize()
        log(f"profile-verify: {calls} {rule} calls at B={B}, k={k}, V={VOCAB}")
        return
    log(f"device {torch.cuda.get_device_name(0)}; building W4 stack")
    w4 = make_w4_stack(torch, synth, sv, dev)
    x_h = synth.activations(32, HIDDEN, seed=11, device=dev)
    x_f = synth.activations(32, FFN, seed=12, device=dev)
    ys = {N: torch.empty((32, N), dtype=torch.float32, device=dev)
          for N in (3 * HIDDEN, HIDDEN, 2 * FFN)}
    # one output per GEMM of the pass (the executor runs them concurrently)
    y_own = [[torch.empty((32, N), dtype=torch.float32, device=dev)
              for (_, N, *_r) in layer] for layer in w4]

    def w4_gemms(kk):
        xh, xf = x_h[:kk].contiguous(), x_f[:kk].contiguous()
        return [(xh if K == HIDDEN else xf, pc, ps, N, y_own[li][gi][:kk])
                for li, layer in enumerate(w4)
                for gi, (name, N, K, c, s, z, pc, ps) in enumerate(layer)]

    def w4_pass(kk):
        return sv.sv_pass_plan("w4", w4_gemms(kk))

    # the same stack in model order: each GEMM reads the bf16 hand-off of the
    # one before it (the q part of qkv, the gate part of gate|up)
    h0 = synth.activations(32, HIDDEN, seed=11, device=dev)
    handed = {"qkv": HIDDEN, "o": HIDDEN, "gateup": FFN, "down": HIDDEN}
    chain_xo = [[torch.empty((32, handed[name]), dtype=torch.bfloat16, device=dev)
                 for (name, *_r) in layer] for layer in w4]

    def w4_chain(kk):
        h, links = h0[:kk], []
        for li, layer in enumerate(w4):
            for gi, (name, N, K, c, s, z, pc, ps) in enumerate(layer):
                xo = chain_xo[li][gi][:kk]
                links.append((h, pc, ps, N, y_own[li][gi][:kk], xo, handoff_alpha(K)))
                h = xo
        return sv.sv_pass_chain_plan(links)

    def w4_launches(kk, packed=True):
        xh, xf = x_h[:kk].contiguous(), x_f[:kk].contiguous()
        out = {N: y[:kk] for N, y in ys.items()}
        L = []
        for li, layer in enumerate(w4):
            for (name, N, K, c, s, z, pc, ps) in layer:
                xx = xh if K == HIDDEN else xf
                yy = out[N]
                if packed:
                    fn = (lambda xx=xx, pc=pc, ps=ps, N=N, yy=yy:
                          sv.sv_qgemm_w4_packed(xx, pc, ps, N, yy))
                else:
                    fn = (lambda xx=xx, c=c, s=s, z=z, yy=yy: sv.sv_qgemm_w4(xx, c, s, z, yy))
                L.append(((name, N, K), fn))
        return L

    pass_bytes = w4_bytes(w4)
    torch.cuda.synchronize()

    if args.profile_pass:
        src = torch.empty(1 << 28, dtype=torch.uint8, device=dev).random_(0, 255)
        dst = torch.empty_like(src)
        dst.copy_(src)  # plain copy kernel of 256 MiB (counter scale reference)
        sink = torch.empty(sv.sv_read_probe_sink_words(), dtype=torch.int32, device=dev)
        sv.sv_read_bandwidth_probe(src, sink)
        if args.format == "w4":
            p = w4_chain(k)
        elif args.format == "w4_unordered":
            p = w4_pass(k)
        elif args.format == "w4_i8":
            xi = {K: synth.int8_activations(k, K, seed=13 + K, device=dev) for K in (HIDDEN, FFN)}
            p = sv.sv_pass_plan("w4_i8", [(xi[K][0], xi[K][1], pc, ps, N, y_own[li][gi][:k])
                                          for li, layer in enumerate(w4)
                                          for gi, (nm, N, K, c, s_, z, pc, ps) in enumerate(layer)])
        else:
            xh, xf = x_h[:k].contiguous(), x_f[:k].contiguous()
            g8 = []
            for li, layer in enumerate(make_w8_stack(torch, synth, dev)):
                for gi, (nm, N, K, c, s_) in enumerate(layer):
                    g8.append((xh if K == HIDDEN else xf, sv.sv_w8_pack(c), s_, N,
                               y_own[li][gi][:k]))
                    del c
            p = sv.sv_pass_plan("w8", g8)
        # several passes, so the trace's average is dominated by warm launches
        for _ in range(PROFILE_PASSES):
            sv.sv_pass_run(p)
        torch.cuda.synchronize()
        assert sv.sv_pass_status(p) == 0
        log("profile pass done")
        return

    # ---- the step: the W4 pass in model order at k rows + accept over
    # V = 152000 (three launches: the chain, the accept statistics, decide) ----
    tgt, dft, tok = synth.accept_inputs(1, k, VOCAB, seed=21, sigma=1.0, device=dev)
    acc_out = {"tokens": torch.empty((1, k + 1), dtype=torch.int32, device=dev),
               "n_acc": torch.empty((1,), dtype=torch.int32, device=dev),
               "status": torch.empty((1,), dtype=torch.int32, device=dev)}
    acc_ws = torch.empty(sv.sv_verify_accept_workspace_bytes(1, k, VOCAB), dtype=torch.uint8,
                         device=dev)
    plan = w4_chain(k)

    def step():
        sv.sv_pass_run(plan)
        sv.sv_verify_accept(tgt, dft, tok, seed=0, out=acc_out, workspace=acc_ws)

    # warm-up curve: the first steps of the process, each timed on its own
    # (events around one eager step), before any other timing
    curve = []
    for _ in range(WARMUP_CURVE_STEPS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        curve.append(round(e0.elapsed_time(e1), 4))
    log(f"timing the step (graph replay); chain plan: {plan.items} rounds on {plan.grid} "
        f"workgroups")
    ms_step, _ = time_graph(torch, step, args.steps, args.warmup)
    assert sv.sv_pass_status(plan) == 0, "chain plan reported a barrier timeout"

    # ---- roofline of the chain kernel: one launch per pass.  Its average
    # launch duration is event-timed on the stream the kernel runs on, over
    # graph replays of REPS back-to-back launches (amortizing the replay's
    # own launch latency) ----
    REPS = 8
    ms_rep, _ = time_graph(torch, lambda: [sv.sv_pass_run(plan) for _ in range(REPS)],
                           max(2, args.steps // REPS), max(1, args.warmup // REPS))
    ms_pass = ms_rep / REPS
    weight_gbps = pass_bytes / (ms_pass * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(weight_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(weight_gbps / HBM_PEAK_GBPS, 4),
                "traffic": recorded_traffic("w4_chain_9b_k16", k, "chain_kernel"),
                "kernel": "chain_kernel<1> (the 128 GEMMs of the pass in model order, "
                          "one launch, device-wide barriers between dependent GEMMs)",
                "bytes_per_launch": pass_bytes, "launch_us": round(ms_pass * 1e3, 2)}
    # the same GEMMs without ordering (each reads a fixed input; the executor
    # runs them in any order): an upper bound of the weight stream, not a pass
    plan_u = w4_pass(k)
    ms_rep_u, _ = time_graph(torch, lambda: [sv.sv_pass_run(plan_u) for _ in range(REPS)],
                             max(2, args.steps // REPS), max(1, args.warmup // REPS))
    ms_u = ms_rep_u / REPS
    gbps_u = pass_bytes / (ms_u * 1e-3) / 1e9
    unordered = {"pass_ms": round(ms_u, 4), "GBps": round(gbps_u, 1),
                 "frac_of_8TBps": round(gbps_u / HBM_PEAK_GBPS, 4),
                 "kernel": "pass_kernel<W4>",
                 "traffic": recorded_traffic("w4_pass_9b_k16", k, "pass_kernel"),
                 "note": "128 GEMMs on fixed inputs in one launch, no ordering: "
                         "an upper bound of the weight stream, not a model pass"}

    # ---- accept latency at k = 32 (B = 1) and throughput at B = 64 ----
    def accept_bench(B, kk):
        t, d, tk = synth.accept_inputs(B, kk, VOCAB, seed=31 + B, sigma=1.0, device=dev)
        out = {"tokens": torch.empty((B, kk + 1), dtype=torch.int32, device=dev),
               "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
               "status": torch.empty((B,), dtype=torch.int32, device=dev)}
        ws = torch.empty(sv.sv_verify_accept_workspace_bytes(B, kk, VOCAB), dtype=torch.uint8,
                         device=dev)
        ms, _ = time_graph(torch, lambda: sv.sv_verify_accept(t, d, tk, seed=0, out=out,
                                                              workspace=ws), 50, 5)
        # host wall time of one eager call: launch through synchronize (median)
        walls = []
        for i in range(60):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            sv.sv_verify_accept(t, d, tk, seed=i, out=out, workspace=ws)
            torch.cuda.synchronize()
            walls.append(time.perf_counter() - t0)
        del t, d, tk
        return ms * 1e3, sorted(walls[10:])[len(walls[10:]) // 2] * 1e6

    log(f"step {ms_step:.3f} ms, pass {ms_pass:.3f} ms ({weight_gbps:.0f} GB/s); timing accept")
    accept_us_b1, accept_host_us_b1 = accept_bench(1, 32)
    accept_us_b64, _ = accept_bench(64, 32)
    accept_bytes = ((2 * 32 + 1) * VOCAB * 4 + 2 * VOCAB * 4)
    extra = {"weight_GBps": round(weight_gbps, 1),
             "weight_frac_of_8TBps": round(weight_gbps / HBM_PEAK_GBPS, 4),
             "pass_ms": round(ms_pass, 4), "pass_weight_bytes": pass_bytes,
             "pass_order": "model order (chain)",
             "unordered_upper_bound": unordered,
             "warmup_curve_ms": curve,
             "accept_us_k32_B1": round(accept_us_b1, 2),
             "accept_host_wall_us_k32_B1": round(accept_host_us_b1, 1),
             "accept_us_per_trial_k32_B64": round(accept_us_b64 / 64, 3),
             "accept_GBps_B64": round(64 * accept_bytes / (accept_us_b64 * 1e-6) / 1e9, 1)}

    if not args.quick:
        # measured read peak
        big = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
        sink = torch.empty(sv.sv_read_probe_sink_words(), dtype=torch.int32, device=dev)
        ms_rd, _ = time_graph(torch, lambda: sv.sv_read_bandwidth_probe(big, sink), 10, 2)
        extra["read_probe_GBps"] = round(big.numel() / (ms_rd * 1e-3) / 1e9, 1)
        extra["weight_frac_of_read_probe"] = round(weight_gbps / extra["read_probe_GBps"], 4)
        del big
        log(f"read probe {extra['read_probe_GBps']} GB/s; W4 k sweep")
        # the same pass as 128 separate launches (packed and row-major layouts)
        for key, packed in (("w4_per_gemm_launches", True), ("w4_row_major_launches", False)):
            Ls = w4_launches(k, packed=packed)
            ms_l, _ = time_graph(torch, lambda Ls=Ls: [fn() for _, fn in Ls], 20, 20)
            extra[key] = {"pass_ms": round(ms_l, 4),
                          "GBps": round(pass_bytes / (ms_l * 1e-3) / 1e9, 1)}
        # W4 k sweeps (model order and unordered): latency ratio t(32)/t(1)
        sweep, sweep_u = {}, {}
        for kk in (1, 4, 8, 16, 32):
            for table, mk in ((sweep, w4_chain), (sweep_u, w4_pass)):
                pk = mk(kk)
                ms, _ = time_graph(torch, lambda pk=pk: sv.sv_pass_run(pk), 40, 40)
                table[kk] = {"pass_ms": round(ms, 4),
                             "GBps": round(pass_bytes / (ms * 1e-3) / 1e9, 1),
                             "drafted_tok_s": round(kk / (ms * 1e-3), 1)}
                del pk
        extra["w4_k_sweep"] = sweep
        extra["w4_latency_ratio_k32_over_k1"] = round(sweep[32]["pass_ms"] / sweep[1]["pass_ms"], 3)
        extra["w4_k_sweep_unordered"] = sweep_u
        extra["w4_latency_ratio_k32_over_k1_unordered"] = round(
            sweep_u[32]["pass_ms"] / sweep_u[1]["pass_ms"], 3)
        # MFMA utilisation of the unordered W4 executor at k = 1, 16 and 32
        # (the kernel whose counters are recorded): the useful flops (2 k per
        # weight) over its measured pass time against the dense bf16 peak,
        # and from the recorded counters the fraction of cycles the MFMA pipe
        # was busy (SQ_VALU_MFMA_BUSY_CYCLES per SIMD over the active cycles
        # GRBM_GUI_ACTIVE per XCD) with the clock they imply.  At k = 1 the
        # pass streams at the read probe's rate, so the MFMA form costs the
        # small-k case nothing a vector form could win back.
        n_weights = sum(N * K for layer in w4 for (_, N, K, *_r) in layer)
        n_simd = 4 * torch.cuda.get_device_properties(0).multi_processor_count
        mfma = {"kernel": "pass_kernel<W4> (unordered)"}
        for kk in (1, 16, 32):
            tf = 2.0 * kk * n_weights / (sweep_u[kk]["pass_ms"] * 1e-3) / 1e12
            row = {"useful_TFLOPs": round(tf, 1),
                   "frac_of_bf16_dense_peak": round(tf / BF16_DENSE_PEAK_TFLOPS, 4),
                   "GBps": sweep_u[kk]["GBps"]}
            rec = recorded_counters(f"w4_pass_9b_k{kk}")
            if rec:
                c = rec["counters"]
                active = c["GRBM_GUI_ACTIVE"] / 8
                row["mfma_busy_frac"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] / n_simd / active, 4)
                row["clock_GHz"] = round(active / (rec["avg_duration_us"] * 1e3), 3)
                row["mfma_instructions"] = c["SQ_INSTS_MFMA"]
            mfma[f"k{kk}"] = row
        extra["w4_mfma"] = mfma
        log("int8 path")
        # int8 path: every activation row of the pass (4 inputs per layer, 41 or
        # 123 outlier channels x50) rotated by the block-4096 Hadamard and
        # quantized per token -- batched into one call per input width, and
        # timed again as one call per link as a model runs it -- then all 128
        # int8 x W4 GEMMs in one executor launch
        n_h, n_f = 3 * LAYERS, LAYERS               # qkv, o, gate|up inputs; down inputs
        signs_h = synth.hadamard_signs(HIDDEN, seed=3, device=dev)
        signs_f = synth.hadamard_signs(FFN, seed=4, device=dev)
        xo_h = torch.cat([synth.outlier_activations(k, HIDDEN, seed=500 + i, device=dev)[0]
                          for i in range(n_h)])
        xo_f = torch.cat([synth.outlier_activations(k, FFN, seed=700 + i, device=dev)[0]
                          for i in range(n_f)])
        xq_h = torch.empty((n_h * k, HIDDEN), dtype=torch.int8, device=dev)
        xq_f = torch.empty((n_f * k, FFN), dtype=torch.int8, device=dev)
        sc_h = torch.empty((n_h * k,), dtype=torch.float32, device=dev)
        sc_f = torch.empty((n_f * k,), dtype=torch.float32, device=dev)
        gi8, ih, jf = [], 0, 0
        for li, layer in enumerate(w4):
            for gi, (name, N, K, c, s, z, pc, ps) in enumerate(layer):
                if K == HIDDEN:
                    xq, xs = xq_h[ih * k:(ih + 1) * k], sc_h[ih * k:(ih + 1) * k]
                    ih += 1
                else:
                    xq, xs = xq_f[jf * k:(jf + 1) * k], sc_f[jf * k:(jf + 1) * k]
                    jf += 1
                gi8.append((xq, xs, pc, ps, N, y_own[li][gi][:k]))
        p8 = sv.sv_pass_plan("w4_i8", gi8)

        def rotate():
            sv.sv_hadamard_i8(xo_h, signs_h, 4096, xq_h, sc_h)
            sv.sv_hadamard_i8(xo_f, signs_f, 4096, xq_f, sc_f)

        def int8_pass():
            rotate()
            sv.sv_pass_run(p8)

        ms_i8, _ = time_graph(torch, int8_pass, 60, 60)
        ms_i8g, _ = time_graph(torch, lambda: sv.sv_pass_run(p8), 60, 60)
        ms_rot, _ = time_graph(torch, rotate, 20, 5)
        # In a model each rotation waits for the link before it, so it runs as
        # one call per GEMM input (k rows each), 128 calls in layer order.
        rot_calls, ih, jf = [], 0, 0
        for layer in w4:
            for (name, N, K, *_rest) in layer:
                if K == HIDDEN:
                    xin, sg, ih = xo_h[ih * k:(ih + 1) * k], signs_h, ih + 1
                else:
                    xin, sg, jf = xo_f[jf * k:(jf + 1) * k], signs_f, jf + 1
                outq = torch.empty((k, K), dtype=torch.int8, device=dev)
                outs = torch.empty((k,), dtype=torch.float32, device=dev)
                rot_calls.append(lambda xin=xin, sg=sg, outq=outq, outs=outs:
                                 sv.sv_hadamard_i8(xin, sg, 4096, outq, outs))
        ms_rot_link, _ = time_graph(torch, lambda: [fn() for fn in rot_calls], 20, 5)
        del rot_calls
        # the same int8 x W4 GEMMs as 128 single launches on the row-major codes
        L8 = [(lambda xq=xq, xs=xs, c=c, s=s, z=z, yy=yy:
               sv.sv_qgemm_w4_i8(xq, xs, c, s, z, y=yy))
              for (xq, xs, pc, ps, N, yy), (name, N2, K, c, s, z, pc2, ps2)
              in zip(gi8, [g for layer in w4 for g in layer])]
        ms_i8l, _ = time_graph(torch, lambda: [fn() for fn in L8], 20, 20)
        del L8
        extra["int8_path"] = {"pass_ms": round(ms_i8, 4),
                              "GBps": round(pass_bytes / (ms_i8 * 1e-3) / 1e9, 1),
                              "gemm_launch_ms": round(ms_i8g, 4),
                              "gemm_GBps": round(pass_bytes / (ms_i8g * 1e-3) / 1e9, 1),
                              "hadamard_ms_all_rows": round(ms_rot, 4),
                              "hadamard_rows": int((n_h + n_f) * k),
                              "hadamard_ms_per_link_calls": round(ms_rot_link, 4),
                              "hadamard_calls_per_link": len(w4) * len(w4[0]),
                              "row_major_launches_ms": round(ms_i8l, 4),
                              "row_major_launches_GBps": round(
                                  pass_bytes / (ms_i8l * 1e-3) / 1e9, 1)}
        extra["int8_path"]["quant_error"] = int8_quant_error(torch, sv, synth, w4[0], k, dev)
        del xo_h, xo_f
        log("W8 k sweep")
        # W8 k sweep on the executor (8-bit stack packed once)
        w8 = make_w8_stack(torch, synth, dev)
        b8 = w8_bytes(w8)
        # the pass's W8 GEMMs as 128 single launches on the row-major codes
        xh, xf = x_h[:k].contiguous(), x_f[:k].contiguous()
        L8 = [(lambda xx=(xh if K == HIDDEN else xf), c=c, s=s, yy=y_own[li][gi][:k]:
               sv.sv_qgemm_w8(xx, c, s, y=yy))
              for li, layer in enumerate(w8) for gi, (name, N, K, c, s) in enumerate(layer)]
        ms_l8, _ = time_graph(torch, lambda: [fn() for fn in L8], 20, 20)
        extra["w8_row_major_launches"] = {"pass_ms": round(ms_l8, 4),
                                          "GBps": round(b8 / (ms_l8 * 1e-3) / 1e9, 1)}
        del L8
        w8p = [[(N, K, sv.sv_w8_pack(c), s) for (name, N, K, c, s) in layer] for layer in w8]
        del w8
        sweep8 = {}
        for kk in (1, 4, 8, 16, 32):
            xh, xf = x_h[:kk].contiguous(), x_f[:kk].contiguous()
            g8 = [(xh if K == HIDDEN else xf, pc, s, N, y_own[li][gi][:kk])
                  for li, layer in enumerate(w8p) for gi, (N, K, pc, s) in enumerate(layer)]
            pk = sv.sv_pass_plan("w8", g8)
            ms, _ = time_graph(torch, lambda pk=pk: sv.sv_pass_run(pk), 40, 40)
            sweep8[kk] = {"pass_ms": round(ms, 4), "GBps": round(b8 / (ms * 1e-3) / 1e9, 1)}
        extra["w8_k_sweep"] = sweep8
        extra["w8_latency_ratio_k32_over_k1"] = round(sweep8[32]["pass_ms"] /
                                                      sweep8[1]["pass_ms"], 3)
        # the W8 stack in model order (the same hand-offs as the W4 chain)
        chain8 = {}
        for kk in (1, 16, 32):
            h, links = h0[:kk], []
            for li, layer in enumerate(w8p):
                for gi, (N, K, pc, s) in enumerate(layer):
                    xo = chain_xo[li][gi][:kk]
                    links.append((h, pc, s, N, y_own[li][gi][:kk], xo, handoff_alpha_w8(K)))
                    h = xo
            pk = sv.sv_pass_chain_plan(links, fmt="w8")
            ms, _ = time_graph(torch, lambda pk=pk: sv.sv_pass_run(pk), 40, 40)
            if sv.sv_pass_status(pk) != 0:
                raise RuntimeError(f"W8 chain status {sv.sv_pass_status(pk)}")
            chain8[kk] = {"pass_ms": round(ms, 4), "GBps": round(b8 / (ms * 1e-3) / 1e9, 1)}
        extra["w8_k_sweep_model_order"] = chain8
        del w8p
        log("accept statistics")
        # accept statistics: 4096 trials per noise level, k = 32
        stats = {}
        B = 64
        out = {"tokens": torch.empty((B, 33), dtype=torch.int32, device=dev),
               "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
               "status": torch.empty((B,), dtype=torch.int32, device=dev)}
        ws = torch.empty(sv.sv_verify_accept_workspace_bytes(B, 32, VOCAB), dtype=torch.uint8,
                         device=dev)
        for sigma in (0.1, 1.0, 3.0):
            tot = 0
            for rep in range(4096 // B):
                t, d, tk = synth.accept_inputs(B, 32, VOCAB, seed=100000 * int(sigma * 10) + rep,
                                               sigma=sigma, device=dev)
                sv.sv_verify_accept(t, d, tk, seed=0, offset=rep, out=out, workspace=ws)
                tot += int(out["n_acc"].sum().item())
            mean_acc = tot / 4096
            stats[str(sigma)] = {"mean_accepted": round(mean_acc, 3),
                                 "tokens_per_pass": round(mean_acc + 1, 3)}
        extra["accept_stats_k32"] = stats
        log("sampled verification")
        # verification under sampling settings (sv_verify_sampled), k = 32
        sampled = {}
        for name, cfg in (("greedy", (0.0, 0, 1.0)), ("T0.7_p0.9", (0.7, 0, 0.9)),
                          ("k50", (1.0, 50, 1.0)), ("T0.8_k100_p0.95", (0.8, 100, 0.95))):
            row = {}
            for B in (1, 64):
                t, d, tk = synth.accept_inputs(B, 32, VOCAB, seed=41 + B, sigma=1.0, device=dev)
                out = {"tokens": torch.empty((B, 33), dtype=torch.int32, device=dev),
                       "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
                       "status": torch.empty((B,), dtype=torch.int32, device=dev)}
                ws = torch.empty(max(16, sv.sv_verify_sampled_workspace_bytes(B, 32, VOCAB)),
                                 dtype=torch.uint8, device=dev)
                ms, _ = time_graph(torch, lambda: sv.sv_verify_sampled(
                    t, d, tk, 0, 0, *cfg, out=out, workspace=ws), 20, 3)
                row["us_B1" if B == 1 else "us_per_trial_B64"] = round(
                    ms * 1e3 / B, 3 if B > 1 else 2)
                del t, d, tk
            sampled[name] = row
        extra["sampled_verify_k32"] = sampled
        log("coupled verification")
        # Gumbel-max coupled verification (sv_verify_coupled), k = 32: timing,
        # and the mean accepted drafts when the drafter draws with the same
        # noise (its draws: the kernel's choices on the draft rows)
        coupled = {}
        for B in (1, 64):
            t, d, tk = synth.accept_inputs(B, 32, VOCAB, seed=51 + B, sigma=1.0, device=dev)
            out = {"tokens": torch.empty((B, 33), dtype=torch.int32, device=dev),
                   "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
                   "status": torch.empty((B,), dtype=torch.int32, device=dev)}
            ws = torch.empty(max(16, sv.sv_verify_coupled_workspace_bytes(B, 32, VOCAB)),
                             dtype=torch.uint8, device=dev)
            ms, _ = time_graph(torch, lambda: sv.sv_verify_coupled(t, tk, 0, 0, out=out,
                                                                   workspace=ws), 20, 3)
            coupled["us_B1" if B == 1 else "us_per_trial_B64"] = round(ms * 1e3 / B, 3)
            del t, d, tk
        stats = {}
        B = 64
        for sigma in (0.1, 1.0, 3.0):
            tot = 0
            for rep in range(8):
                t, d, _ = synth.accept_inputs(B, 32, VOCAB, seed=200000 * int(sigma * 10) + rep,
                                              sigma=sigma, device=dev)
                dpad = torch.cat([d, d[:, :1]], dim=1).contiguous()
                zeros = torch.zeros((B, 32), dtype=torch.int32, device=dev)
                drafts = sv.sv_verify_coupled(dpad, zeros, 0, rep, choices=True)["choices"]
                res = sv.sv_verify_coupled(t, drafts[:, :32].contiguous(), 0, rep)
                tot += int(res["n_acc"].sum().item())
            stats[str(sigma)] = {"mean_accepted": round(tot / (8 * B), 3),
                                 "tokens_per_pass": round(tot / (8 * B) + 1, 3)}
        coupled["accept_stats"] = stats
        extra["coupled_verify_k32"] = coupled
        log("tree verification")
        # greedy verification of a 16-node and a 32-node draft tree
        # (sv_verify_tree) over the full vocabulary
        tree = {}
        for n in (16, 32):
            row = {}
            for B in (1, 64):
                t, tk, par = synth.tree_inputs(B, n, VOCAB, seed=61 + B + n, device=dev)
                out = {"tokens": torch.empty((B, n + 1), dtype=torch.int32, device=dev),
                       "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
                       "status": torch.empty((B,), dtype=torch.int32, device=dev)}
                ws = torch.empty(max(16, sv.sv_verify_tree_workspace_bytes(B, n, VOCAB)),
                                 dtype=torch.uint8, device=dev)
                ms, _ = time_graph(torch, lambda: sv.sv_verify_tree(t, tk, par, out=out,
                                                                    workspace=ws), 20, 3)
                row["us_B1" if B == 1 else "us_per_trial_B64"] = round(ms * 1e3 / B, 3)
                if B == 64:
                    row["mean_path"] = round(float(out["n_acc"].float().mean().item()), 3)
                del t, tk, par
            tree["n%d" % n] = row
        extra["tree_verify"] = tree
        log("fused LM-head verify")
        # the vocabulary projection (W4, 4096 -> 152 000) as one more GEMM of
        # the pass, 16 scored rows (k = 15 drafts); fused: its epilogue writes
        # the softmax statistics and sv_verify_accept_stats merges them;
        # unfused: the plain GEMM and sv_verify_accept re-reading the logits
        kk, G = 15, (VOCAB + 63) // 64
        hc, hs, hz = synth.w4_matrix(VOCAB, HIDDEN, seed=90, device=dev)
        hpc, hps = sv.sv_w4_pack(hc, hs, hz)
        del hc, hs, hz
        hh = synth.activations(kk + 1, HIDDEN, seed=91, device=dev, scale=0.15)
        lg = torch.empty((kk + 1, VOCAB), dtype=torch.float32, device=dev)
        lst = torch.empty((kk + 1, G, 2), dtype=torch.float32, device=dev)
        ldft, ltok = synth.lm_head_drafts(1, kk, VOCAB, seed=92, device=dev)
        lout = {"tokens": torch.empty((1, kk + 1), dtype=torch.int32, device=dev),
                "n_acc": torch.empty((1,), dtype=torch.int32, device=dev),
                "status": torch.empty((1,), dtype=torch.int32, device=dev)}
        lws = torch.empty(sv.sv_verify_accept_workspace_bytes(1, kk, VOCAB), dtype=torch.uint8,
                          device=dev)
        stack = w4_gemms(kk + 1)
        p_fused = sv.sv_pass_plan("w4", stack + [(hh, hpc, hps, VOCAB, lg, lst)])
        p_plain = sv.sv_pass_plan("w4", stack + [(hh, hpc, hps, VOCAB, lg)])
        lg3, lst4 = lg.view(1, kk + 1, VOCAB), lst.view(1, kk + 1, G, 2)

        def acc_fused():
            sv.sv_verify_accept_stats(lg3, lst4, ldft, ltok, 0, out=lout, workspace=lws)

        def acc_plain():
            sv.sv_verify_accept(lg3, ldft, ltok, 0, out=lout, workspace=lws)

        n = max(20, args.steps // 4)
        fused = {"k": kk, "rows": kk + 1, "vocab": VOCAB, "hidden": HIDDEN,
                 "head_weight_bytes": VOCAB * HIDDEN // 2 + VOCAB * (HIDDEN // GROUP) * 4}
        for name, fn in (("step_fused_ms", lambda: (sv.sv_pass_run(p_fused), acc_fused())),
                         ("step_unfused_ms", lambda: (sv.sv_pass_run(p_plain), acc_plain())),
                         ("pass_with_head_stats_ms", lambda: sv.sv_pass_run(p_fused)),
                         ("pass_with_head_ms", lambda: sv.sv_pass_run(p_plain))):
            ms, _ = time_graph(torch, fn, n, n)
            fused[name] = round(ms, 4)
        for name, fn in (("accept_stats_us", acc_fused), ("accept_us", acc_plain)):
            ms, _ = time_graph(torch, fn, 50, 5)
            fused[name] = round(ms * 1e3, 2)
        extra["lm_head_verify_k15"] = fused
        del hpc, hps, lg, lst, p_fused, p_plain

    cpu = None
    if not (args.quick or args.no_cpu):
        log("timing the CPU oracle baseline")
        cpu = cpu_baseline(k, dev=dev)

    line = {
        "metric": METRIC, "value": round(k / (ms_step * 1e-3), 1), "unit": "drafted tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "9B-class decoder weight stack, W4 asymmetric group 64, "
                               "32 layers (hidden 4096, ffn 12288), k=16 bf16 draft rows, "
                               "then accept/correct over V=152000",
                   "k": k, "layers": LAYERS, "hidden": HIDDEN, "ffn": FFN, "group": GROUP,
                   "vocab": VOCAB, "launches_per_step": 3, "pass_order": "model order",
                   "graph": "hipGraph replay"},
        "roofline": roofline, "cpu_baseline": cpu, **extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
