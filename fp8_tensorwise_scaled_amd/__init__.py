"""MI355X-native FP8 tensorwise-scaled linear layer, its MLP blocks and LM head.

The compute runs in libfp8mlp.so (hand-written gfx950 HIP kernels behind a C
ABI, include/fp8mlp.h).  This package holds the build script, the ctypes
binding (``api``) and the seeded synthetic inputs (``synth``).  The binding
is imported lazily so that ``synth`` works without torch's GPU runtime.
"""
from __future__ import annotations

_API_NAMES = (
    "fp8_amax_quant", "fp8_linear_fwd", "fp8_linear_dgrad", "fp8_linear_wgrad", "fp8_gated_linear_fwd",
    "relu2_mlp_fwd", "relu2_mlp_bwd", "Relu2MlpSaved", "relu2_mlp_fwd_workspace",
    "relu2_mlp_bwd_workspace", "workspace_layout", "fp8_rmsnorm_quant", "fp8_lm_head_ce",
    "fp8_lm_head_ce_workspace", "lm_head_ce_layout", "swiglu_mlp_fwd", "swiglu_mlp_bwd", "SwigluMlpSaved",
    "swiglu_mlp_workspace", "swiglu_workspace_layout", "bf16_gemm_nt", "bf16_gemm_sym", "muon_newton_schulz", "muon_ns_workspace",
    "E4M3", "E5M2", "ACCUM_FAST", "ACCUM_EXACT",
)

__all__ = list(_API_NAMES)


def __getattr__(name):
    if name in _API_NAMES:
        from . import api

        return getattr(api, name)
    raise AttributeError(name)
