"""ctypes binding of libspecverify with the same entry-point names.

Each wrapper takes torch tensors, checks dtype/shape/device, passes raw
device pointers plus the current HIP stream to the C ABI, and raises SvError
on a non-zero status.  No arithmetic of the method happens here.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libspecverify.so")

SV_MAX_ROWS = 32

EXPORTED_SYMBOLS = (
    "sv_status_str", "sv_version", "sv_qgemm_w4", "sv_qgemm_w8", "sv_hadamard_i8",
    "sv_qgemm_w4_i8", "sv_verify_accept_workspace_bytes", "sv_verify_accept",
    "sv_verify_accept_noalloc_max_bytes", "sv_verify_accept_noalloc",
    "sv_philox4x32_10", "sv_read_probe_sink_words", "sv_read_bandwidth_probe",
    "sv_w4_packed_codes_bytes", "sv_w4_packed_sz_bytes", "sv_w4_pack", "sv_qgemm_w4_packed",
    "sv_w8_pack", "sv_pass_plan_bytes", "sv_pass_plan", "sv_pass_run",
    "sv_verify_sampled_workspace_bytes", "sv_verify_sampled",
    "sv_verify_coupled_workspace_bytes", "sv_verify_coupled",
    "sv_verify_tree_workspace_bytes", "sv_verify_tree", "sv_verify_accept_stats",
    "sv_pass_status", "sv_pass_chain_bytes", "sv_pass_chain_image", "sv_pass_chain_plan",
)

_STATUS = {0: "SV_OK", 1: "SV_ERR_NULL", 2: "SV_ERR_INVALID_ARG", 3: "SV_ERR_ALIGN",
           4: "SV_ERR_UNSUPPORTED", 5: "SV_ERR_WORKSPACE", 6: "SV_ERR_HIP"}


class SvPassGemm(ctypes.Structure):
    """C struct sv_pass_gemm: one GEMM of a verify pass."""
    _fields_ = [("x", ctypes.c_void_p), ("xscale", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("y", ctypes.c_void_p), ("K", ctypes.c_int),
                ("N", ctypes.c_int), ("stats", ctypes.c_void_p)]


class SvPass(ctypes.Structure):
    """C struct sv_pass: host descriptor of a planned pass."""
    _fields_ = [("plan", ctypes.c_void_p), ("format", ctypes.c_int), ("m", ctypes.c_int),
                ("count", ctypes.c_int), ("grid", ctypes.c_int), ("items", ctypes.c_int),
                ("max_steps", ctypes.c_int), ("stats", ctypes.c_int), ("chain", ctypes.c_int),
                ("id", ctypes.c_uint32)]


class SvPassLink(ctypes.Structure):
    """C struct sv_pass_link: one GEMM of a chain (verify pass in model order)."""
    _fields_ = [("x", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("xo", ctypes.c_void_p), ("alpha", ctypes.c_float),
                ("K", ctypes.c_int), ("N", ctypes.c_int), ("xo_cols", ctypes.c_int)]


PASS_STATUS_STALE = 1
PASS_STATUS_TIMEOUT = 2


PASS_FORMATS = {"w4": 0, "w8": 1, "w4_i8": 2}


class SvSampling(ctypes.Structure):
    """C struct sv_sampling: temperature (0 = greedy), top_k (0 = off), top_p (1 = off)."""
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int),
                ("top_p", ctypes.c_float)]


class SvError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)}")


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is missing: build it with `python -c 'import __graft_entry__ as g; "
            f"g.build()'` (hipcc, gfx950).  There is no CPU fallback.")
    L = ctypes.CDLL(lib_path)
    vp, i32, u32, u64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32,
                             ctypes.c_uint64, ctypes.c_size_t)
    sig = {
        "sv_status_str": (ctypes.c_char_p, [i32]),
        "sv_version": (i32, []),
        "sv_qgemm_w4": (i32, [vp, i32, i32, vp, vp, vp, i32, i32, vp, vp]),
        "sv_qgemm_w8": (i32, [vp, i32, i32, vp, vp, i32, vp, vp]),
        "sv_hadamard_i8": (i32, [vp, i32, i32, vp, i32, vp, vp, vp]),
        "sv_qgemm_w4_i8": (i32, [vp, vp, i32, i32, vp, vp, vp, i32, i32, vp, vp]),
        "sv_verify_accept_workspace_bytes": (sz, [i32, i32, i32]),
        "sv_verify_accept": (i32, [vp, vp, vp, i32, i32, i32, u64, u32, vp, vp, vp, vp, vp,
                                   vp, vp, sz, vp]),
        "sv_verify_accept_stats": (i32, [vp, vp, vp, vp, i32, i32, i32, u64, u32, vp, vp, vp,
                                         vp, vp, vp, vp, sz, vp]),
        "sv_verify_accept_noalloc_max_bytes": (sz, []),
        "sv_verify_accept_noalloc": (i32, [vp, vp, vp, i32, i32, i32, u64, u32, vp, vp, vp, vp,
                                           vp, vp, vp]),
        "sv_philox4x32_10": (i32, [vp, vp, vp, i32, vp]),
        "sv_read_probe_sink_words": (i32, []),
        "sv_read_bandwidth_probe": (i32, [vp, sz, vp, vp]),
        "sv_w4_packed_codes_bytes": (sz, [i32, i32]),
        "sv_w4_packed_sz_bytes": (sz, [i32, i32, i32]),
        "sv_w4_pack": (i32, [vp, vp, vp, i32, i32, i32, vp, vp, vp]),
        "sv_qgemm_w4_packed": (i32, [vp, i32, i32, vp, vp, i32, i32, vp, vp]),
        "sv_w8_pack": (i32, [vp, i32, i32, vp, vp]),
        "sv_pass_plan_bytes": (sz, [i32, ctypes.POINTER(SvPassGemm), i32, i32]),
        "sv_pass_plan": (i32, [i32, ctypes.POINTER(SvPassGemm), i32, i32, i32, vp, sz,
                               ctypes.POINTER(SvPass), vp]),
        "sv_pass_run": (i32, [ctypes.POINTER(SvPass), vp]),
        "sv_pass_status": (i32, [ctypes.POINTER(SvPass), ctypes.POINTER(u32), vp]),
        "sv_pass_chain_bytes": (sz, [i32, ctypes.POINTER(SvPassLink), i32, i32]),
        "sv_pass_chain_image": (i32, [i32, ctypes.POINTER(SvPassLink), i32, i32, i32, i32, vp,
                                      sz, ctypes.POINTER(i32)]),
        "sv_pass_chain_plan": (i32, [i32, ctypes.POINTER(SvPassLink), i32, i32, i32, vp, sz,
                                     ctypes.POINTER(SvPass), vp]),
        "sv_verify_sampled_workspace_bytes": (sz, [i32, i32, i32]),
        "sv_verify_sampled": (i32, [vp, vp, vp, i32, i32, i32, ctypes.POINTER(SvSampling), u64,
                                    u32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "sv_verify_coupled_workspace_bytes": (sz, [i32, i32, i32]),
        "sv_verify_coupled": (i32, [vp, vp, i32, i32, i32, u64, u32, vp, vp, vp, vp, vp, sz,
                                    vp]),
        "sv_verify_tree_workspace_bytes": (sz, [i32, i32, i32]),
        "sv_verify_tree": (i32, [vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise SvError(fn, status)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def sv_status_str(status):
    return lib.sv_status_str(int(status)).decode()


def sv_version():
    return lib.sv_version()


def sv_qgemm_w4(x, codes, scales, zeros, y=None, group=64, stream=None):
    """Y = X @ dequant_w4(codes, scales, zeros).T  (x bf16 [m, K] -> y f32 [m, N])."""
    m, K = x.shape
    N = codes.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(codes, "codes", torch.uint8, (N, K // 2))
    _need(scales, "scales", torch.float16, (N, K // group))
    _need(zeros, "zeros", torch.float16, (N, K // group))
    if y is None:
        y = torch.empty((m, N), dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32, (m, N))
    _check("sv_qgemm_w4", lib.sv_qgemm_w4(_ptr(x), m, K, _ptr(codes), _ptr(scales), _ptr(zeros),
                                          N, group, _ptr(y), _stream(stream)))
    return y


def sv_w4_pack(codes, scales, zeros, group=64, stream=None):
    """Row-major W4 (codes [N, K/2], scales/zeros [N, K/group]) -> packed layout.

    Returns (packed_codes uint8 [N*K/2], packed_sz fp16 [N*(K/group)*2]).
    """
    N, half = codes.shape
    K = 2 * half
    _need(codes, "codes", torch.uint8, (N, K // 2))
    _need(scales, "scales", torch.float16, (N, K // group))
    _need(zeros, "zeros", torch.float16, (N, K // group))
    pc = torch.empty((int(lib.sv_w4_packed_codes_bytes(N, K)),), dtype=torch.uint8,
                     device=codes.device)
    ps = torch.empty((int(lib.sv_w4_packed_sz_bytes(N, K, group)) // 2,), dtype=torch.float16,
                     device=codes.device)
    _check("sv_w4_pack", lib.sv_w4_pack(_ptr(codes), _ptr(scales), _ptr(zeros), N, K, group,
                                        _ptr(pc), _ptr(ps), _stream(stream)))
    return pc, ps


def sv_qgemm_w4_packed(x, packed_codes, packed_sz, N, y=None, group=64, stream=None):
    """Y = X @ W.T over packed W4 weights (x bf16 [m, K] -> y f32 [m, N])."""
    m, K = x.shape
    _need(x, "x", torch.bfloat16)
    _need(packed_codes, "packed_codes", torch.uint8, (N * K // 2,))
    _need(packed_sz, "packed_sz", torch.float16, (N * (K // group) * 2,))
    if y is None:
        y = torch.empty((m, N), dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32, (m, N))
    _check("sv_qgemm_w4_packed", lib.sv_qgemm_w4_packed(
        _ptr(x), m, K, _ptr(packed_codes), _ptr(packed_sz), N, group, _ptr(y), _stream(stream)))
    return y


def sv_w8_pack(codes, stream=None):
    """Row-major W8 codes int8 [N, K] -> packed streaming layout (uint8 [N*K])."""
    N, K = codes.shape
    _need(codes, "codes", torch.int8, (N, K))
    out = torch.empty((N * K,), dtype=torch.uint8, device=codes.device)
    _check("sv_w8_pack", lib.sv_w8_pack(_ptr(codes), N, K, _ptr(out), _stream(stream)))
    return out


class Pass:
    """A planned verify pass: the device plan, its host descriptor and the
    tensors it points to (kept alive as long as the plan)."""

    def __init__(self, plan, info, tensors):
        self.plan = plan
        self.info = info
        self._tensors = tensors

    @property
    def grid(self):
        return self.info.grid

    @property
    def items(self):
        return self.info.items


def _pass_gemms(fmt, gemms, group):
    arr = (SvPassGemm * len(gemms))()
    m = None
    keep = []
    for i, g in enumerate(gemms):
        base = 6 if fmt == "w4_i8" else 5
        stats = g[base] if len(g) > base else None
        if fmt == "w4_i8":
            x, xscale, codes, sc, N, y = g[:base]
        else:
            x, codes, sc, N, y = g[:base]
            xscale = None
        mm, K = x.shape
        m = mm if m is None else m
        if mm != m:
            raise ValueError("every GEMM of a pass has the same number of rows m")
        if fmt == "w8":
            _need(x, "x", torch.bfloat16)
            _need(codes, "packed_codes", torch.uint8, (N * K,))
            _need(sc, "scales", torch.float16, (N,))
        else:
            _need(x, "x", torch.int8 if fmt == "w4_i8" else torch.bfloat16)
            _need(codes, "packed_codes", torch.uint8, (N * K // 2,))
            _need(sc, "packed_sz", torch.float16, (N * (K // group) * 2,))
        if xscale is not None:
            _need(xscale, "xscale", torch.float32, (m,))
        _need(y, "y", torch.float32, (m, N))
        if stats is not None:
            _need(stats, "stats", torch.float32, (m, (N + 63) // 64, 2))
        arr[i] = SvPassGemm(x.data_ptr(), None if xscale is None else xscale.data_ptr(),
                            codes.data_ptr(), sc.data_ptr(), y.data_ptr(), K, N,
                            None if stats is None else stats.data_ptr())
        keep += [t for t in (x, xscale, codes, sc, y, stats) if t is not None]
    return arr, m, keep


def sv_pass_plan(fmt, gemms, group=64, stream=None, plan=None):
    """Plan one verify pass; `fmt` is "w4", "w8" or "w4_i8".

    gemms: sequence of
      w4:    (x bf16 [m, K], packed_codes, packed_sz, N, y f32 [m, N])
      w8:    (x bf16 [m, K], packed_codes (sv_w8_pack), scales f16 [N], N, y)
      w4_i8: (xq int8 [m, K], xscale f32 [m], packed_codes, packed_sz, N, y)
    each optionally followed by stats f32 [m, ceil(N/64), 2], which receives
    the softmax statistics (max, sum of exp) of every 64 outputs of a row.
    `plan`: an optional uint8 device buffer to plan into (e.g. one that held
    an earlier plan).  Returns a Pass for sv_pass_run.  Synchronizes `stream`.
    """
    if fmt not in PASS_FORMATS:
        raise ValueError(f"unknown pass format {fmt!r}")
    if len(gemms) == 0:
        raise ValueError("a pass needs at least one GEMM")
    arr, m, keep = _pass_gemms(fmt, gemms, group)
    f = PASS_FORMATS[fmt]
    nbytes = int(lib.sv_pass_plan_bytes(f, arr, len(gemms), m))
    if nbytes == 0:
        raise SvError("sv_pass_plan_bytes", 2)
    if plan is None:
        plan = torch.empty((nbytes,), dtype=torch.uint8, device=keep[0].device)
    else:
        _need(plan, "plan", torch.uint8)
        nbytes = plan.numel()
    info = SvPass()
    _check("sv_pass_plan", lib.sv_pass_plan(f, arr, len(gemms), m, group, _ptr(plan), nbytes,
                                            ctypes.byref(info), _stream(stream)))
    return Pass(plan, info, keep)


def sv_pass_run(p, stream=None):
    """Run every GEMM of a planned pass (or every link of a chain) in one launch."""
    _check("sv_pass_run", lib.sv_pass_run(ctypes.byref(p.info), _stream(stream)))


def sv_pass_status(p, stream=None):
    """The plan's status word (PASS_STATUS_* bits; 0 = ok).  Synchronizes."""
    v = ctypes.c_uint32(0)
    _check("sv_pass_status", lib.sv_pass_status(ctypes.byref(p.info), ctypes.byref(v),
                                                _stream(stream)))
    return int(v.value)


def _chain_links(links, group, fmt="w4"):
    """links: sequence of (x bf16 [m, K], packed_codes, packed_sz, N, y f32 [m, N],
    xo bf16 [m, xo_cols] or None, alpha); for "w8" the codes are sv_w8_pack's
    and packed_sz is the f16 [N] channel scales."""
    arr = (SvPassLink * len(links))()
    m, keep = None, []
    for i, (x, codes, sc, N, y, xo, alpha) in enumerate(links):
        mm, K = x.shape
        m = mm if m is None else m
        if mm != m:
            raise ValueError("every link of a chain has the same number of rows m")
        _need(x, "x", torch.bfloat16)
        if fmt == "w8":
            _need(codes, "packed_codes", torch.uint8, (N * K,))
            _need(sc, "scales", torch.float16, (N,))
        else:
            _need(codes, "packed_codes", torch.uint8, (N * K // 2,))
            _need(sc, "packed_sz", torch.float16, (N * (K // group) * 2,))
        _need(y, "y", torch.float32, (m, N))
        xo_cols = 0
        if xo is not None:
            _need(xo, "xo", torch.bfloat16)
            if xo.dim() != 2 or xo.shape[0] != m:
                raise ValueError("xo must be bf16 [m, xo_cols]")
            xo_cols = xo.shape[1]
        arr[i] = SvPassLink(x.data_ptr(), codes.data_ptr(), sc.data_ptr(), y.data_ptr(),
                            None if xo is None else xo.data_ptr(), float(alpha), K, N, xo_cols)
        keep += [t for t in (x, codes, sc, y, xo) if t is not None]
    return arr, m, keep


def sv_pass_chain_plan(links, group=64, stream=None, plan=None, fmt="w4"):
    """Plan a verify pass in model order (fmt "w4" or "w8").  links: sequence of
    (x, packed_codes, packed_sz, N, y, xo, alpha) -- see _chain_links; a link
    whose x is an earlier link's xo waits for every earlier link.  `plan`: an
    optional uint8 device buffer to plan into (256-byte aligned), e.g. one
    that held an earlier plan.  Returns a Pass for sv_pass_run.
    Synchronizes `stream`."""
    if len(links) == 0:
        raise ValueError("a chain needs at least one link")
    if fmt not in ("w4", "w8"):
        raise ValueError("a chain runs the w4 or w8 format")
    arr, m, keep = _chain_links(links, group, fmt)
    nbytes = int(lib.sv_pass_chain_bytes(PASS_FORMATS[fmt], arr, len(links), m))
    if nbytes == 0:
        raise SvError("sv_pass_chain_bytes", 2)
    if plan is None:
        # 256-byte aligned plan buffer
        raw = torch.empty((nbytes + 256,), dtype=torch.uint8, device=keep[0].device)
        off = (-raw.data_ptr()) % 256
        plan = raw[off:off + nbytes]
    else:
        _need(plan, "plan", torch.uint8)
        raw = plan
        nbytes = plan.numel()
    info = SvPass()
    _check("sv_pass_chain_plan", lib.sv_pass_chain_plan(
        PASS_FORMATS[fmt], arr, len(links), m, group, _ptr(plan), nbytes, ctypes.byref(info),
        _stream(stream)))
    return Pass(raw, info, keep)


def sv_pass_chain_image(fmt, links, m, cus, group=64):
    """Host-only plan image of a chain for a device of `cus` compute units.
    links: sequence of dicts with integer addresses x, codes, scales, y, xo
    (0 = none) and alpha, K, N, xo_cols.  Returns (status, grid, bytes)."""
    arr = (SvPassLink * len(links))()
    for i, d in enumerate(links):
        arr[i] = SvPassLink(d["x"], d["codes"], d["scales"], d["y"], d.get("xo") or None,
                            float(d.get("alpha", 1.0)), d["K"], d["N"], d.get("xo_cols", 0))
    cap = 1 << 24
    buf = (ctypes.c_uint8 * cap)()
    grid = ctypes.c_int(0)
    st = lib.sv_pass_chain_image(PASS_FORMATS[fmt], arr, len(links), m, group, cus, buf, cap,
                                 ctypes.byref(grid))
    return int(st), int(grid.value), bytes(buf) if st == 0 else b""


def sv_qgemm_w8(x, codes, scales, y=None, stream=None):
    m, K = x.shape
    N = codes.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(codes, "codes", torch.int8, (N, K))
    _need(scales, "scales", torch.float16, (N,))
    if y is None:
        y = torch.empty((m, N), dtype=torch.float32, device=x.device)
    _need(y, "y", torch.float32, (m, N))
    _check("sv_qgemm_w8", lib.sv_qgemm_w8(_ptr(x), m, K, _ptr(codes), _ptr(scales), N, _ptr(y),
                                          _stream(stream)))
    return y


def sv_hadamard_i8(x, signs, block, xq=None, xscale=None, stream=None):
    m, K = x.shape
    _need(x, "x", torch.bfloat16)
    _need(signs, "signs", torch.int8, (K,))
    if xq is None:
        xq = torch.empty((m, K), dtype=torch.int8, device=x.device)
    if xscale is None:
        xscale = torch.empty((m,), dtype=torch.float32, device=x.device)
    _need(xq, "xq", torch.int8, (m, K))
    _need(xscale, "xscale", torch.float32, (m,))
    _check("sv_hadamard_i8", lib.sv_hadamard_i8(_ptr(x), m, K, _ptr(signs), int(block), _ptr(xq),
                                                _ptr(xscale), _stream(stream)))
    return xq, xscale


def sv_qgemm_w4_i8(xq, xscale, codes, scales, zeros, y=None, group=64, stream=None):
    m, K = xq.shape
    N = codes.shape[0]
    _need(xq, "xq", torch.int8)
    _need(xscale, "xscale", torch.float32, (m,))
    _need(codes, "codes", torch.uint8, (N, K // 2))
    _need(scales, "scales", torch.float16, (N, K // group))
    _need(zeros, "zeros", torch.float16, (N, K // group))
    if y is None:
        y = torch.empty((m, N), dtype=torch.float32, device=xq.device)
    _need(y, "y", torch.float32, (m, N))
    _check("sv_qgemm_w4_i8", lib.sv_qgemm_w4_i8(_ptr(xq), _ptr(xscale), m, K, _ptr(codes),
                                                _ptr(scales), _ptr(zeros), N, group, _ptr(y),
                                                _stream(stream)))
    return y


def sv_verify_accept_workspace_bytes(B, k, V):
    return int(lib.sv_verify_accept_workspace_bytes(int(B), int(k), int(V)))


def sv_verify_accept(target_logits, draft_logits, draft_tokens, seed, offset=0, out=None,
                     diagnostics=False, workspace=None, stream=None):
    """Accept/correct for B independent trials.

    Returns dict(tokens [B, k+1] int32, n_acc [B], status [B]) plus p_at, q_at
    [B, k] and lse [B, 2k+1] when diagnostics=True.
    """
    B, k1, V = target_logits.shape
    k = k1 - 1
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, (B, k + 1, V))
    _need(draft_logits, "draft_logits", torch.float32, (B, k, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, k))
    if out is None:
        out = {
            "tokens": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
            "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
            "status": torch.empty((B,), dtype=torch.int32, device=dev),
        }
        if diagnostics:
            out["p_at"] = torch.empty((B, k), dtype=torch.float32, device=dev)
            out["q_at"] = torch.empty((B, k), dtype=torch.float32, device=dev)
            out["lse"] = torch.empty((B, 2 * k + 1), dtype=torch.float32, device=dev)
    need = sv_verify_accept_workspace_bytes(B, k, V)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    _check("sv_verify_accept", lib.sv_verify_accept(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), B, k, V,
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), ctypes.c_uint32(int(offset) & 0xFFFFFFFF),
        _ptr(out["tokens"]), _ptr(out["n_acc"]), _ptr(out["status"]), _ptr(out.get("p_at")),
        _ptr(out.get("q_at")), _ptr(out.get("lse")), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return out


def sv_verify_accept_noalloc_max_bytes():
    return int(lib.sv_verify_accept_noalloc_max_bytes())


def sv_verify_accept_noalloc(target_logits, draft_logits, draft_tokens, seed, out, offset=0,
                             stream=None):
    """sv_verify_accept on the library's fixed per-device workspace: no
    device allocation in the library (the caller passes every output in
    `out`: tokens, n_acc, status, and optionally p_at, q_at, lse)."""
    B, k1, V = target_logits.shape
    k = k1 - 1
    _need(target_logits, "target_logits", torch.float32, (B, k + 1, V))
    _need(draft_logits, "draft_logits", torch.float32, (B, k, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, k))
    _need(out["tokens"], "tokens", torch.int32, (B, k + 1))
    _need(out["n_acc"], "n_acc", torch.int32, (B,))
    _need(out["status"], "status", torch.int32, (B,))
    _check("sv_verify_accept_noalloc", lib.sv_verify_accept_noalloc(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), B, k, V,
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), ctypes.c_uint32(int(offset) & 0xFFFFFFFF),
        _ptr(out["tokens"]), _ptr(out["n_acc"]), _ptr(out["status"]), _ptr(out.get("p_at")),
        _ptr(out.get("q_at")), _ptr(out.get("lse")), _stream(stream)))
    return out


def sv_verify_accept_stats(target_logits, target_stats, draft_logits, draft_tokens, seed,
                           offset=0, out=None, diagnostics=False, workspace=None, stream=None):
    """sv_verify_accept with the target rows' softmax statistics taken from
    target_stats f32 [B, k+1, ceil(V/64), 2] (a pass GEMM's stats output)."""
    B, k1, V = target_logits.shape
    k = k1 - 1
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, (B, k + 1, V))
    _need(target_stats, "target_stats", torch.float32, (B, k + 1, (V + 63) // 64, 2))
    _need(draft_logits, "draft_logits", torch.float32, (B, k, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, k))
    if out is None:
        out = {
            "tokens": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
            "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
            "status": torch.empty((B,), dtype=torch.int32, device=dev),
        }
        if diagnostics:
            out["p_at"] = torch.empty((B, k), dtype=torch.float32, device=dev)
            out["q_at"] = torch.empty((B, k), dtype=torch.float32, device=dev)
            out["lse"] = torch.empty((B, 2 * k + 1), dtype=torch.float32, device=dev)
    need = sv_verify_accept_workspace_bytes(B, k, V)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    _check("sv_verify_accept_stats", lib.sv_verify_accept_stats(
        _ptr(target_logits), _ptr(target_stats), _ptr(draft_logits), _ptr(draft_tokens), B, k,
        V, ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        ctypes.c_uint32(int(offset) & 0xFFFFFFFF), _ptr(out["tokens"]), _ptr(out["n_acc"]),
        _ptr(out["status"]), _ptr(out.get("p_at")), _ptr(out.get("q_at")), _ptr(out.get("lse")),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return out


def sv_verify_sampled_workspace_bytes(B, k, V):
    return int(lib.sv_verify_sampled_workspace_bytes(int(B), int(k), int(V)))


def sv_verify_sampled(target_logits, draft_logits, draft_tokens, seed, offset=0,
                      temperature=1.0, top_k=0, top_p=1.0, out=None, diagnostics=False,
                      workspace=None, stream=None):
    """Verification under sampling settings (temperature 0 = greedy) for B trials.

    Returns dict(tokens [B, k+1] int32, n_acc [B], status [B]) plus p_at, q_at
    [B, k] when diagnostics=True.
    """
    B, k1, V = target_logits.shape
    k = k1 - 1
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, (B, k + 1, V))
    _need(draft_logits, "draft_logits", torch.float32, (B, k, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, k))
    if out is None:
        out = {
            "tokens": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
            "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
            "status": torch.empty((B,), dtype=torch.int32, device=dev),
        }
        if diagnostics:
            out["p_at"] = torch.empty((B, k), dtype=torch.float32, device=dev)
            out["q_at"] = torch.empty((B, k), dtype=torch.float32, device=dev)
    need = sv_verify_sampled_workspace_bytes(B, k, V)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    cfg = SvSampling(float(temperature), int(top_k), float(top_p))
    _check("sv_verify_sampled", lib.sv_verify_sampled(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), B, k, V,
        ctypes.byref(cfg), ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF),
        ctypes.c_uint32(int(offset) & 0xFFFFFFFF), _ptr(out["tokens"]), _ptr(out["n_acc"]),
        _ptr(out["status"]), _ptr(out.get("p_at")), _ptr(out.get("q_at")), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return out


def sv_verify_coupled_workspace_bytes(B, k, V):
    return int(lib.sv_verify_coupled_workspace_bytes(int(B), int(k), int(V)))


def sv_verify_coupled(target_logits, draft_tokens, seed, offset=0, out=None, choices=False,
                      workspace=None, stream=None):
    """Gumbel-max coupled verification for B trials.

    Returns dict(tokens [B, k+1] int32, n_acc [B], status [B]) plus the
    target's choices [B, k+1] when choices=True.
    """
    B, k1, V = target_logits.shape
    k = k1 - 1
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, (B, k + 1, V))
    _need(draft_tokens, "draft_tokens", torch.int32, (B, k))
    if out is None:
        out = {
            "tokens": torch.empty((B, k + 1), dtype=torch.int32, device=dev),
            "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
            "status": torch.empty((B,), dtype=torch.int32, device=dev),
        }
        if choices:
            out["choices"] = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    need = sv_verify_coupled_workspace_bytes(B, k, V)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _check("sv_verify_coupled", lib.sv_verify_coupled(
        _ptr(target_logits), _ptr(draft_tokens), B, k, V,
        ctypes.c_uint64(int(seed) & 0xFFFFFFFFFFFFFFFF), ctypes.c_uint32(int(offset) & 0xFFFFFFFF),
        _ptr(out["tokens"]), _ptr(out["n_acc"]), _ptr(out["status"]), _ptr(out.get("choices")),
        _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return out


def sv_verify_tree_workspace_bytes(B, n, V):
    return int(lib.sv_verify_tree_workspace_bytes(int(B), int(n), int(V)))


def sv_verify_tree(target_logits, tokens, parents, out=None, path=False, workspace=None,
                   stream=None):
    """Greedy verification of B draft trees of n nodes.

    Returns dict(tokens [B, n+1] int32, n_acc [B], status [B]) plus the
    accepted node indices path [B, n] when path=True.
    """
    B, n1, V = target_logits.shape
    n = n1 - 1
    dev = target_logits.device
    _need(target_logits, "target_logits", torch.float32, (B, n + 1, V))
    _need(tokens, "tokens", torch.int32, (B, n))
    _need(parents, "parents", torch.int32, (B, n))
    if out is None:
        out = {
            "tokens": torch.empty((B, n + 1), dtype=torch.int32, device=dev),
            "n_acc": torch.empty((B,), dtype=torch.int32, device=dev),
            "status": torch.empty((B,), dtype=torch.int32, device=dev),
        }
        if path:
            out["path"] = torch.empty((B, n), dtype=torch.int32, device=dev)
    need = sv_verify_tree_workspace_bytes(B, n, V)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _check("sv_verify_tree", lib.sv_verify_tree(
        _ptr(target_logits), _ptr(tokens), _ptr(parents), B, n, V, _ptr(out["tokens"]),
        _ptr(out["n_acc"]), _ptr(out["status"]), _ptr(out.get("path")), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(stream)))
    return out


def sv_philox4x32_10(ctr, key, out=None, stream=None):
    n = ctr.shape[0]
    _need(ctr, "ctr", torch.int32, (n, 4))
    _need(key, "key", torch.int32, (n, 2))
    if out is None:
        out = torch.empty((n, 4), dtype=torch.int32, device=ctr.device)
    _check("sv_philox4x32_10", lib.sv_philox4x32_10(_ptr(ctr), _ptr(key), _ptr(out), n,
                                                    _stream(stream)))
    return out


def sv_read_probe_sink_words():
    return int(lib.sv_read_probe_sink_words())


def sv_read_bandwidth_probe(src, sink, nbytes=None, stream=None):
    nbytes = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check("sv_read_bandwidth_probe", lib.sv_read_bandwidth_probe(
        _ptr(src), ctypes.c_size_t(nbytes), _ptr(sink), _stream(stream)))
