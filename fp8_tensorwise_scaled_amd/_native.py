"""ctypes loader for libfp8mlp.so (the gfx950 HIP library).

Argument marshalling only.  There is no fallback: if the library is missing
or cannot be loaded, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8mlp.so")

E4M3 = 0
E5M2 = 1

# FP8 GEMM accumulation: the FP8 matrix cores (group-truncated sums) or exact
# products with fp32 accumulation (codes decoded to bf16, bf16 matrix cores)
ACCUM_FAST = 0
ACCUM_EXACT = 1

_lock = threading.Lock()
_lib = None

i64, f32p, vp, c_int, szt = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t


class Relu2MlpSaved(ctypes.Structure):
    _fields_ = [("xq", vp), ("uq", vp), ("dq", vp), ("aq", vp), ("h", vp), ("scales", vp)]


class SwigluMlpSaved(ctypes.Structure):
    _fields_ = [("xq", vp), ("wgq", vp), ("wuq", vp), ("wdq", vp), ("aq", vp), ("g", vp), ("u", vp),
                ("scales", vp)]


_PROTOS = {
    "fp8mlp_abi_version": (c_int, []),
    "fp8mlp_status_string": (ctypes.c_char_p, [c_int]),
    "fp8_amax_quant_workspace_bytes": (szt, [i64, i64]),
    "fp8_amax_quant": (c_int, [vp, i64, i64, i64, c_int, vp, i64, vp, i64, vp, vp, vp, szt, vp]),
    "fp8_amax_quant_noalloc": (c_int, [vp, i64, i64, i64, c_int, vp, i64, vp, i64, vp, vp, vp]),
    "fp8_rmsnorm_quant_workspace_bytes": (szt, [i64, i64]),
    "fp8_rmsnorm_quant": (c_int, [vp, vp, ctypes.c_float, i64, i64, i64, c_int, vp, i64, vp, i64, vp, vp, vp, vp,
                                  szt, vp]),
    "fp8_linear_fwd": (c_int, [vp, i64, c_int, vp, vp, i64, c_int, vp, i64, i64, i64, vp, i64, c_int, vp]),
    "fp8_linear_fwd_bf16_workspace_bytes": (szt, [i64, i64, i64]),
    "fp8_linear_fwd_bf16": (c_int, [vp, i64, vp, i64, i64, i64, i64, vp, i64, vp, i64, vp, vp, i64, vp, szt, c_int,
                                    vp]),
    "fp8_linear_dgrad": (c_int, [vp, i64, c_int, vp, vp, i64, c_int, vp, i64, i64, i64, vp, i64, c_int, vp]),
    "fp8_linear_wgrad": (c_int, [vp, i64, c_int, vp, vp, i64, c_int, vp, i64, i64, i64, vp, i64, c_int, vp]),
    "relu2_mlp_fwd_workspace_bytes": (szt, [i64, i64, i64]),
    "relu2_mlp_bwd_workspace_bytes": (szt, [i64, i64, i64]),
    "relu2_mlp_fwd_workspace_layout": (c_int, [i64, i64, i64, ctypes.POINTER(szt), c_int]),
    "relu2_mlp_bwd_workspace_layout": (c_int, [i64, i64, i64, ctypes.POINTER(szt), c_int]),
    "relu2_mlp_fwd": (c_int, [vp, vp, vp, i64, i64, i64, vp, ctypes.POINTER(Relu2MlpSaved), vp, szt, c_int, vp]),
    "relu2_mlp_bwd": (c_int, [vp, ctypes.POINTER(Relu2MlpSaved), i64, i64, i64, vp, vp, vp, vp, vp, szt, c_int,
                              vp]),
    "swiglu_mlp_fwd_workspace_bytes": (szt, [i64, i64, i64]),
    "swiglu_mlp_bwd_workspace_bytes": (szt, [i64, i64, i64]),
    "swiglu_mlp_fwd_workspace_layout": (c_int, [i64, i64, i64, ctypes.POINTER(szt), c_int]),
    "swiglu_mlp_bwd_workspace_layout": (c_int, [i64, i64, i64, ctypes.POINTER(szt), c_int]),
    "swiglu_mlp_fwd": (c_int, [vp, vp, vp, vp, i64, i64, i64, vp, ctypes.POINTER(SwigluMlpSaved), vp, szt, c_int,
                               vp]),
    "swiglu_mlp_bwd": (c_int, [vp, ctypes.POINTER(SwigluMlpSaved), i64, i64, i64, vp, vp, vp, vp, vp, vp, szt,
                               c_int, vp]),
    "fp8_gated_linear_fwd": (c_int, [vp, i64, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, vp, i64, c_int, vp]),
    "bf16_gemm_nt": (c_int, [vp, i64, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_float, vp, i64, vp, i64, vp,
                             i64, vp]),
    "bf16_gemm_sym_workspace_bytes": (szt, [i64, i64]),
    "bf16_gemm_sym": (c_int, [vp, i64, i64, i64, ctypes.c_float, ctypes.c_float, vp, i64, vp, i64, vp, szt, vp]),
    "muon_ns_workspace_bytes": (szt, [i64, i64]),
    "muon_newton_schulz": (c_int, [vp, i64, i64, c_int, vp, ctypes.c_float, vp, vp, vp, szt, vp]),
    "fp8_lm_head_ce_workspace_bytes": (szt, [i64, i64, i64, i64]),
    "fp8_lm_head_ce_workspace_layout": (c_int, [i64, i64, i64, i64, ctypes.POINTER(szt), c_int]),
    "fp8_lm_head_ce": (c_int, [vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, i64, vp, vp, vp, vp, vp, szt,
                               c_int, vp]),
}

EXPORTS = tuple(_PROTOS)


class Fp8MlpError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib():
    """Load libfp8mlp.so (raises if it is not built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    f"{LIB_PATH} is missing: build it with `python -m fp8_tensorwise_scaled_amd.build` "
                    "(there is no CPU fallback)")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _PROTOS.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fp8mlp_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != 0:
        raise Fp8MlpError(fn, status, status_string(status))


def call(name: str, *args) -> None:
    check(name, getattr(lib(), name)(*args))
