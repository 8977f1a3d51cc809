"""MI355X-native dense GEMM: hand-written gfx950 HIP kernels behind a C ABI.

The compute entry points live in ``dense_gemm_engineering_amd.binding``
(thin ctypes marshalling over libdge_gemm.so); they are re-exported here on
first use so that importing the package does not load the GPU library.
"""

_BINDING_NAMES = ("gemm", "gemm_f16", "gemm_bf16", "gemm_f32", "gemm_ex", "dequant_q4_f16",
                  "prefill_q4_f16", "gemm_workspace_size", "gemm_workspace_size_splits",
                  "gemm_status_string", "gemm_init", "GemmError")


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
