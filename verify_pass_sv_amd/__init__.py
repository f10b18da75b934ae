"""verify_pass_sv_amd -- Python binding of libspecverify (MI355X / gfx950).

Argument marshalling only: every step of the verify pass runs in the HIP
kernels of libspecverify.so; PyTorch supplies device memory and streams.
The binding is loaded on first use of an `sv_*` name and raises ImportError
if the shared library has not been built -- there is no fallback path.
`verify_pass_sv_amd.synth` (seeded workload generators) needs no library.
"""

_BINDING_NAMES = (
    "SvError", "lib", "lib_path", "sv_status_str", "sv_version", "sv_qgemm_w4", "sv_qgemm_w8",
    "sv_hadamard_i8", "sv_qgemm_w4_i8", "sv_verify_accept", "sv_verify_accept_workspace_bytes",
    "sv_philox4x32_10", "sv_read_bandwidth_probe", "sv_read_probe_sink_words",
    "EXPORTED_SYMBOLS", "SV_MAX_ROWS", "sv_w4_pack", "sv_qgemm_w4_packed",
    "sv_w8_pack", "sv_pass_plan", "sv_pass_run", "Pass", "SvPassGemm", "SvPass",
    "PASS_FORMATS", "sv_verify_sampled", "sv_verify_sampled_workspace_bytes", "SvSampling",
    "sv_verify_coupled", "sv_verify_coupled_workspace_bytes", "sv_verify_tree",
    "sv_verify_tree_workspace_bytes", "sv_verify_accept_stats", "sv_pass_status",
    "sv_pass_chain_plan", "sv_pass_chain_image", "SvPassLink", "PASS_STATUS_STALE",
    "PASS_STATUS_TIMEOUT", "sv_verify_accept_noalloc", "sv_verify_accept_noalloc_max_bytes",
)

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
