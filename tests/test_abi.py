"""The C-ABI library loads and exports every entry point the header declares.

CPU-only: nothing here launches a kernel; the argument checks below return
before any HIP call.
"""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "specverify.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_[a-z0-9_]+)\s*\(", src)))


def test_header_declarations_found():
    names = _declared()
    assert "sv_qgemm_w4" in names and "sv_verify_accept" in names
    assert len(names) >= 11


def test_library_exports_every_declared_symbol():
    import verify_pass_sv_amd as sv
    lib = ctypes.CDLL(sv.lib_path)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, f"missing exports: {missing}"
    assert set(_declared()) == set(sv.EXPORTED_SYMBOLS)


def test_version_and_status_strings():
    import verify_pass_sv_amd as sv
    assert sv.sv_version() == 200
    assert sv.sv_status_str(0) == "SV_OK"
    assert sv.sv_status_str(5) == "SV_ERR_WORKSPACE"
    assert sv.sv_status_str(99) == "SV_ERR_UNKNOWN"


def test_argument_validation_before_launch():
    import verify_pass_sv_amd as sv
    L = sv.lib
    fake = ctypes.c_void_p(0x100000)     # aligned, never dereferenced
    odd = ctypes.c_void_p(0x100002)
    # null pointer
    assert L.sv_qgemm_w4(None, 4, 512, fake, fake, fake, 64, 64, fake, None) == 1
    # unsupported group size
    assert L.sv_qgemm_w4(fake, 4, 512, fake, fake, fake, 64, 32, fake, None) == 4
    # m out of range, N not a multiple of 16, K not a multiple of 64
    assert L.sv_qgemm_w4(fake, 33, 512, fake, fake, fake, 64, 64, fake, None) == 2
    assert L.sv_qgemm_w4(fake, 4, 512, fake, fake, fake, 40, 64, fake, None) == 2
    assert L.sv_qgemm_w8(fake, 4, 100, fake, fake, 64, fake, None) == 2
    # a W8 matrix of 2 GiB or more (32-bit buffer offsets)
    assert L.sv_qgemm_w8(fake, 4, 65536, fake, fake, 32768, fake, None) == 4
    # misaligned pointer
    assert L.sv_qgemm_w4(odd, 4, 512, fake, fake, fake, 64, 64, fake, None) == 3
    # Hadamard block must be a power of two dividing K, at most 4096
    assert L.sv_hadamard_i8(fake, 4, 4096, fake, 48, fake, fake, None) == 2
    assert L.sv_hadamard_i8(fake, 4, 4096, fake, 8192, fake, fake, None) == 2
    assert L.sv_hadamard_i8(fake, 4, 32768, fake, 4096, fake, fake, None) == 2
    # accept: k range, workspace size
    ws = sv.sv_verify_accept_workspace_bytes(4, 8, 1000)
    assert ws > 0 and sv.sv_verify_accept_workspace_bytes(4, 33, 1000) == 0
    args = [fake, fake, fake, 4, 8, 1000, 0, 0, fake, fake, fake, None, None, None]
    assert L.sv_verify_accept(*args, fake, ws - 1, None) == 5
    assert L.sv_verify_accept(*args, None, ws, None) == 5
    bad_k = [fake, fake, fake, 4, 0, 1000, 0, 0, fake, fake, fake, None, None, None]
    assert L.sv_verify_accept(*bad_k, fake, ws, None) == 2


def test_workspace_grows_with_batch():
    import verify_pass_sv_amd as sv
    a = sv.sv_verify_accept_workspace_bytes(1, 32, 152000)
    b = sv.sv_verify_accept_workspace_bytes(64, 32, 152000)
    assert 0 < a < b


def test_pass_plan_validation_before_any_hip_call():
    import verify_pass_sv_amd as sv
    L = sv.lib
    a = 0x100000                                   # aligned, never dereferenced
    W4, W8, I8 = 0, 1, 2

    def gemms(*shapes, x=a, xscale=None):
        arr = (sv.SvPassGemm * len(shapes))()
        for i, (K, N) in enumerate(shapes):
            arr[i] = sv.SvPassGemm(x, xscale, a, a, a, K, N)
        return arr

    good = gemms((4096, 12288), (4096, 4096), (12288, 4096), (128, 16))
    nb = L.sv_pass_plan_bytes(W4, good, 4, 16)
    # header + per-workgroup tables + 64 bytes per 512-channel item
    items = 24 + 8 + 8 + 1
    assert nb >= items * 64 and nb < items * 64 + 64 * 1024
    assert L.sv_pass_plan_bytes(W8, good, 4, 16) == nb
    assert L.sv_pass_plan_bytes(7, good, 4, 16) == 0                  # unknown format
    assert L.sv_pass_plan_bytes(W4, good, 4, 0) == 0
    assert L.sv_pass_plan_bytes(W4, good, 4, 33) == 0
    assert L.sv_pass_plan_bytes(W4, good, 0, 16) == 0
    assert L.sv_pass_plan_bytes(W4, gemms((4096, 40)), 1, 16) == 0     # N % 16
    assert L.sv_pass_plan_bytes(W4, gemms((4032, 64)), 1, 16) == 0     # K % 128 (4-bit)
    assert L.sv_pass_plan_bytes(W8, gemms((4032, 64)), 1, 16) > 0      # K % 64 (8-bit)
    # the int8 path needs row scales, the others must not get any
    assert L.sv_pass_plan_bytes(I8, good, 4, 16) == 0
    assert L.sv_pass_plan_bytes(I8, gemms((4096, 64), xscale=a), 1, 16) > 0
    assert L.sv_pass_plan_bytes(W4, gemms((4096, 64), xscale=a), 1, 16) == 0
    info = sv.SvPass()
    plan = ctypes.c_void_p(a)
    assert L.sv_pass_plan(W4, good, 4, 16, 64, None, nb, ctypes.byref(info), None) == 1
    assert L.sv_pass_plan(W4, good, 4, 16, 64, plan, nb, None, None) == 1
    assert L.sv_pass_plan(W4, good, 4, 16, 32, plan, nb, ctypes.byref(info), None) == 4
    assert L.sv_pass_plan(W4, good, 4, 16, 64, plan, nb - 1, ctypes.byref(info), None) == 5
    assert L.sv_pass_plan(W4, good, 4, 16, 64, ctypes.c_void_p(a + 8), nb,
                          ctypes.byref(info), None) == 3
    assert L.sv_pass_plan(W4, gemms((4096, 64), x=a + 2), 1, 16, 64, plan, nb,
                          ctypes.byref(info), None) == 3
    assert L.sv_pass_plan(W4, gemms((4096, 64), x=0), 1, 16, 64, plan, nb,
                          ctypes.byref(info), None) == 1
    assert L.sv_pass_plan(I8, gemms((4096, 64)), 1, 16, 64, plan, nb,
                          ctypes.byref(info), None) == 1
    # a single matrix with 2 GiB of codes does not fit 32-bit buffer offsets
    assert L.sv_pass_plan_bytes(W4, gemms((65536, 65536)), 1, 1) == 0
    assert L.sv_pass_run(None, None) == 1
    bad = sv.SvPass(plan=a, format=W4, m=0, count=1, grid=256, items=1, max_steps=1)
    assert L.sv_pass_run(ctypes.byref(bad), None) == 2
    bad = sv.SvPass(plan=a, format=W4, m=16, count=1, grid=0, items=1, max_steps=1)
    assert L.sv_pass_run(ctypes.byref(bad), None) == 2
    bad = sv.SvPass(plan=a, format=9, m=16, count=1, grid=1, items=1, max_steps=1)
    assert L.sv_pass_run(ctypes.byref(bad), None) == 2
    # W8 packing arguments
    assert L.sv_w8_pack(None, 64, 64, plan, None) == 1
    assert L.sv_w8_pack(plan, 40, 64, plan, None) == 2
    assert L.sv_w8_pack(plan, 64, 96, plan, None) == 2


def test_build_rejects_scratch_in_counted_kernels():
    # The executor and the packed GEMM wait on exact counts of their own
    # memory operations; the build refuses a kernel of theirs that spills.
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "sv_build", os.path.join(ROOT, "verify_pass_sv_amd", "csrc", "build.py"))
    build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(build)
    ok = ("a.hip:1:1: remark: Function Name: k0 [-R]\n"
          "a.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-R]\n")
    build._check_no_scratch("pass.hip", ok)
    bad = ok + ("a.hip:2:1: remark: Function Name: k1 [-R]\n"
                "a.hip:2:1: remark:     ScratchSize [bytes/lane]: 16 [-R]\n")
    with pytest.raises(RuntimeError, match="k1 uses 16 bytes/lane"):
        build._check_no_scratch("pass.hip", bad)
    assert {"pass.hip", "qgemm_w4_packed.hip"} <= build.NO_SCRATCH


def test_sampled_verification_validation_before_launch():
    import verify_pass_sv_amd as sv
    L = sv.lib
    fake = ctypes.c_void_p(0x100000)     # aligned, never dereferenced
    ws = sv.sv_verify_sampled_workspace_bytes(4, 8, 1000)
    assert ws > 0 and sv.sv_verify_sampled_workspace_bytes(4, 33, 1000) == 0
    assert sv.sv_verify_sampled_workspace_bytes(64, 32, 152000) > ws

    def call(cfg, ws_bytes=ws, workspace=fake, k=8):
        ref = ctypes.byref(cfg) if cfg is not None else None
        return L.sv_verify_sampled(fake, fake, fake, 4, k, 1000, ref, 0, 0, fake, fake, fake,
                                   None, None, workspace, ws_bytes, None)
    S = sv.SvSampling
    assert call(None) == 1
    for bad in [S(-1.0, 0, 1.0), S(float("inf"), 0, 1.0), S(float("nan"), 0, 1.0),
                S(1.0, -1, 1.0), S(1.0, 0, 0.0), S(1.0, 0, 1.5), S(1.0, 0, float("nan"))]:
        assert call(bad) == 2
    assert call(S(1.0, 0, 1.0), k=0) == 2
    assert call(S(0.7, 40, 0.9), ws_bytes=ws - 1) == 5
    assert call(S(0.7, 40, 0.9), workspace=None) == 5


def test_coupled_verification_validation_before_launch():
    import verify_pass_sv_amd as sv
    L = sv.lib
    fake = ctypes.c_void_p(0x100000)     # aligned, never dereferenced
    ws = sv.sv_verify_coupled_workspace_bytes(4, 8, 1000)
    assert ws > 0 and sv.sv_verify_coupled_workspace_bytes(4, 33, 1000) == 0

    def call(k=8, offset=0, ws_bytes=ws, workspace=fake, tokens=fake):
        return L.sv_verify_coupled(fake, tokens, 4, k, 1000, 0, offset, fake, fake, fake, None,
                                   workspace, ws_bytes, None)
    assert call(tokens=None) == 1
    assert call(k=0) == 2 and call(k=33) == 2
    assert call(offset=1 << 24) == 2
    assert call(ws_bytes=ws - 1) == 5 and call(workspace=None) == 5


def test_tree_verification_validation_before_launch():
    import verify_pass_sv_amd as sv
    L = sv.lib
    fake = ctypes.c_void_p(0x100000)     # aligned, never dereferenced
    ws = sv.sv_verify_tree_workspace_bytes(4, 8, 1000)
    assert ws > 0 and sv.sv_verify_tree_workspace_bytes(4, 33, 1000) == 0

    def call(n=8, B=4, ws_bytes=ws, workspace=fake, parents=fake, path=None):
        return L.sv_verify_tree(fake, fake, parents, B, n, 1000, fake, fake, fake, path,
                                workspace, ws_bytes, None)
    assert call(parents=None) == 1
    assert call(n=0) == 2 and call(n=33) == 2 and call(B=0) == 2 and call(B=65536) == 2
    assert call(path=ctypes.c_void_p(0x100004)) == 3
    assert call(ws_bytes=ws - 1) == 5 and call(workspace=None) == 5


def test_softmax_statistics_arguments_before_launch():
    import verify_pass_sv_amd as sv
    L = sv.lib
    a = 0x100000                                   # aligned, never dereferenced
    arr = (sv.SvPassGemm * 1)()
    arr[0] = sv.SvPassGemm(a, None, a, a, a, 4096, 152000, a)
    assert L.sv_pass_plan_bytes(0, arr, 1, 16) > 0
    arr[0] = sv.SvPassGemm(a, None, a, a, a, 4096, 152000, a + 8)   # stats misaligned
    assert L.sv_pass_plan_bytes(0, arr, 1, 16) == 0
    fake = ctypes.c_void_p(a)
    ws = sv.sv_verify_accept_workspace_bytes(1, 4, 1000)

    def call(stats=fake, k=4):
        return L.sv_verify_accept_stats(fake, stats, fake, fake, 1, k, 1000, 0, 0, fake, fake,
                                        fake, None, None, None, fake, ws, None)
    assert call(stats=None) == 1
    assert call(stats=ctypes.c_void_p(a + 4)) == 3
    assert call(k=0) == 2 and call(k=33) == 2
