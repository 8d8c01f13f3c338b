"""Host-side checks of the C ABI: the library loads, exports every function
declared in include/*.h, and rejects invalid arguments before launching
anything (these calls never reach the GPU)."""
import ctypes
import glob
import os
import re

import pytest

from fp8_tensorwise_scaled_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        with open(h) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\**\s+\**([a-z_][a-z0-9_]*)\s*\(", src, re.M):
            names.add(m.group(1))
    return names


def test_header_exports_all_symbols():
    L = _native.lib()
    decl = declared_functions()
    assert len(decl) >= 12
    for name in decl:
        assert hasattr(L, name), name
    assert decl == set(_native.EXPORTS), decl ^ set(_native.EXPORTS)


def test_abi_version_and_status_strings():
    L = _native.lib()
    assert L.fp8mlp_abi_version() == 3
    for s in range(0, 7):
        assert len(_native.status_string(s)) > 0


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
FAKE_ODD = ctypes.c_void_p(0x10001)


def q(*args):
    return _native.lib().fp8_amax_quant(*args)


def test_quant_validation():
    ws_n = _native.lib().fp8_amax_quant_workspace_bytes(64, 64)
    assert ws_n > 0
    ok = [FAKE, 64, 64, 64, 0, FAKE, 64, None, 0, FAKE, None, FAKE, ws_n, None]
    bad = dict(x=(0, None), rows=(1, -1), cols=(2, -1), ldx=(3, 32), fmt=(4, 7), ldq=(6, 10),
               scale=(9, None))
    for _, (i, v) in bad.items():
        a = list(ok)
        a[i] = v
        assert q(*a) == 1, _
    a = list(ok); a[5] = None                     # neither q nor qt
    assert q(*a) == 1
    a = list(ok); a[5] = FAKE; a[0] = FAKE        # q aliases x
    assert q(*a) == 1
    a = list(ok); a[0] = FAKE_ODD; a[5] = ctypes.c_void_p(0x20000)
    assert q(*a) == 2                             # x not 2-byte aligned
    a = list(ok); a[5] = ctypes.c_void_p(0x20000); a[11] = None
    assert q(*a) == 3                             # no workspace
    a[11] = FAKE; a[12] = ws_n - 1
    assert q(*a) == 3                             # workspace too small
    a = list(ok); a[5] = None; a[7] = ctypes.c_void_p(0x20000); a[8] = 10
    assert q(*a) == 1                             # ldqt < rows


def test_linear_fwd_bf16_validation():
    """Every case below fails validation, so nothing is launched."""
    L = _native.lib()
    P = [ctypes.c_void_p(0x10000 * k) for k in range(1, 8)]  # distinct, never dereferenced
    nws = L.fp8_linear_fwd_bf16_workspace_bytes(32, 48, 64)
    assert nws >= 8 and L.fp8_linear_fwd_bf16_workspace_bytes(-1, 48, 64) == 0
    # x [32,64], w [48,64], xq (ld 64), wq (ld 64), scales, y [32,48], ws
    base = [P[0], 64, P[1], 64, 32, 48, 64, P[2], 64, P[3], 64, P[4], P[5], 48, P[6], nws, 0, None]

    def call(**kw):
        a = list(base)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return L.fp8_linear_fwd_bf16(*a)
    assert call(a11=None) == 1                            # scales missing
    assert call(a11=ctypes.c_void_p(0x10002)) == 2        # scales not 4-byte aligned
    assert call(a1=32) == 1                               # ldx < K
    assert call(a3=32) == 1                               # ldw < K
    assert call(a7=None) == 1                             # xq missing
    assert call(a8=72) == 2                               # ldxq % 16
    assert call(a9=ctypes.c_void_p(0x20008)) == 2         # wq not 16-byte aligned
    assert call(a9=P[2]) == 1                             # xq and wq the same buffer
    assert call(a7=P[0]) == 1                             # xq is x
    assert call(a13=40) == 1                              # ldy < N
    assert call(a16=2) == 1                               # unknown accumulation mode
    assert call(a14=None) == 3                            # no workspace
    assert call(a15=nws - 1) == 3                         # workspace too small
    assert call(a14=ctypes.c_void_p(0x10008)) == 2        # workspace not 16-byte aligned
    assert call(a4=-1) == 1                               # M < 0


def test_gemm_validation():
    L = _native.lib()
    # fwd (NT): A [M,K], B [N,K];  M=32, N=48, K=64
    base = [FAKE, 64, 0, FAKE, FAKE, 64, 0, FAKE, 32, 48, 64, FAKE, 48, 0, None]
    for fn in (L.fp8_linear_fwd,):
        assert fn(*[None] + base[1:]) == 1
        a = list(base); a[8] = -1
        assert fn(*a) == 1                          # M < 0
        a = list(base); a[8] = 0
        assert fn(*a) == 0                          # M = 0: empty output, nothing launched
        a = list(base); a[9] = 0
        assert fn(*a) == 0                          # N = 0
        a = list(base); a[1] = 32
        assert fn(*a) == 1                          # lda < K
        a = list(base); a[1] = 72
        assert fn(*a) == 2                          # lda % 16
        a = list(base); a[0] = ctypes.c_void_p(0x10008)
        assert fn(*a) == 2                          # A not 16-byte aligned
        a = list(base); a[2] = 3
        assert fn(*a) == 1                          # unknown format
        a = list(base); a[12] = 40
        assert fn(*a) == 1                          # ldc < N
        a = list(base); a[13] = 2
        assert fn(*a) == 1                          # unknown accumulation mode
        a = list(base); a[13] = -1
        assert fn(*a) == 1
    # tile offsets are 32-bit: 255 rows of a 2^24-byte leading dimension do not fit
    a = list(base); a[1] = 1 << 24
    assert L.fp8_linear_fwd(*a) == 5
    a = list(base); a[5] = 1 << 24
    assert L.fp8_linear_fwd(*a) == 5
    # the exact edge: with K = 4096, lda = 8,421,488 is the last accepted
    # multiple of 16 (a GPU test runs it); 16 bytes more is refused
    a = list(base); a[10] = 4096; a[1] = a[5] = 8_421_488 + 16
    assert L.fp8_linear_fwd(*a) == 5
    # dgrad (NN): dY [M,N] K-major (ld >= N), W [N,K] MN-major (ld >= K); M=32, N=40, K=64
    d = [FAKE, 48, 1, FAKE, FAKE, 64, 0, FAKE, 32, 40, 64, FAKE, 64, 0, None]
    a = list(d); a[1] = 32
    assert L.fp8_linear_dgrad(*a) == 1              # lddy < N
    a = list(d); a[5] = 48
    assert L.fp8_linear_dgrad(*a) == 1              # ldw < K
    a = list(d); a[5] = 72
    assert L.fp8_linear_dgrad(*a) == 2              # ldw % 16
    a = list(d); a[13] = 5
    assert L.fp8_linear_dgrad(*a) == 1              # unknown accumulation mode
    # MN-major operands span every reduction row: (N + 128) ldw + 256 < 2^31
    a = list(d); a[9] = 4096; a[1] = 4096; a[5] = 2 ** 31 // (4096 + 128) // 16 * 16 + 16
    assert L.fp8_linear_dgrad(*a) == 5
    # wgrad (TN): dY [M,N] and X [M,K] both MN-major; M=40 (reduction), N=48, K=64
    w = [FAKE, 48, 1, FAKE, FAKE, 64, 0, FAKE, 40, 48, 64, FAKE, 64, 0, None]
    a = list(w); a[1] = 32
    assert L.fp8_linear_wgrad(*a) == 1              # lddy < N
    a = list(w); a[5] = 32
    assert L.fp8_linear_wgrad(*a) == 1              # ldx < K
    a = list(w); a[0] = ctypes.c_void_p(0x10008)
    assert L.fp8_linear_wgrad(*a) == 2              # dY codes not 16-byte aligned
    # the exact MN-major edge that a GPU test runs: reduction 272, ld 5,368,704;
    # 16 bytes more is refused
    a = list(w); a[8] = 272; a[1] = a[5] = 5_368_704 + 16
    assert L.fp8_linear_wgrad(*a) == 5


def test_gated_linear_validation():
    L = _native.lib()
    fn = L.fp8_gated_linear_fwd
    base = [FAKE, 64, FAKE, FAKE, FAKE, FAKE, FAKE, 64, 32, 48, 64, FAKE, FAKE, FAKE, 48, 0, None]
    a = list(base); a[6] = None
    assert fn(*a) == 1                              # no up scale
    a = list(base); a[13] = None
    assert fn(*a) == 1                              # no A output
    a = list(base); a[5] = None
    assert fn(*a) == 1                              # no up codes
    a = list(base); a[5] = ctypes.c_void_p(0x10008)
    assert fn(*a) == 2                              # up codes not 16-byte aligned
    a = list(base); a[1] = a[7] = 72
    assert fn(*a) == 2                              # leading dimensions % 16
    a = list(base); a[10] = 40; a[1] = a[7] = 48
    assert fn(*a) == 5                              # K % 16
    a = list(base); a[8] = 0
    assert fn(*a) == 0                              # M = 0: nothing written
    a = list(base); a[14] = 40
    assert fn(*a) == 1                              # ldo < N
    a = list(base); a[15] = 3
    assert fn(*a) == 1                              # unknown accumulation mode


def test_mlp_validation():
    L = _native.lib()
    assert L.relu2_mlp_fwd_workspace_bytes(2048, 768, 3072) > 0
    assert L.relu2_mlp_bwd_workspace_bytes(2048, 768, 3072) > 2048 * 768 + 2048 * 3072 * 3
    assert L.relu2_mlp_fwd_workspace_bytes(100, 768, 3072) == 0      # M % 16
    saved = _native.Relu2MlpSaved(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 0x10000)
    n = L.relu2_mlp_fwd_workspace_bytes(64, 64, 256)
    args = [FAKE, FAKE, FAKE, 64, 64, 256, FAKE, ctypes.byref(saved), FAKE, n - 1, 0, None]
    assert L.relu2_mlp_fwd(*args) == 3
    args[3] = 65
    assert L.relu2_mlp_fwd(*args) == 5
    args = [FAKE, FAKE, FAKE, 64, 64, 256, None, ctypes.byref(saved), FAKE, n, 0, None]
    assert L.relu2_mlp_fwd(*args) == 1                               # y missing with M > 0
    args = [FAKE, FAKE, FAKE, -16, 64, 256, FAKE, ctypes.byref(saved), FAKE, n, 0, None]
    assert L.relu2_mlp_fwd(*args) == 1                               # M < 0
    assert L.relu2_mlp_fwd_workspace_bytes(0, 64, 256) > 0           # M = 0 is a valid shape
    bad_saved = _native.Relu2MlpSaved(0x10000, 0, 0x10000, 0x10000, 0x10000, 0x10000)
    args = [FAKE, FAKE, FAKE, 64, 64, 256, FAKE, ctypes.byref(bad_saved), FAKE, n, 0, None]
    assert L.relu2_mlp_fwd(*args) == 1
    args = [FAKE, FAKE, FAKE, 64, 64, 256, FAKE, ctypes.byref(saved), FAKE, n, 7, None]
    assert L.relu2_mlp_fwd(*args) == 1                               # unknown accumulation mode
    nb = L.relu2_mlp_bwd_workspace_bytes(64, 64, 256)
    args = [FAKE, ctypes.byref(saved), 64, 64, 256, FAKE, FAKE, FAKE, None, FAKE, nb - 1, 0, None]
    assert L.relu2_mlp_bwd(*args) == 3
    args = [FAKE, ctypes.byref(saved), 64, 64, 256, ctypes.c_void_p(0x10008), FAKE, FAKE, None, FAKE, nb, 0, None]
    assert L.relu2_mlp_bwd(*args) == 2
    offs = (ctypes.c_size_t * 6)()
    assert L.relu2_mlp_bwd_workspace_layout(64, 64, 256, offs, 6) == 0
    assert list(offs) == sorted(offs) and offs[0] == 0
    assert L.relu2_mlp_bwd_workspace_layout(64, 64, 256, offs, 5) == 1
    assert L.relu2_mlp_fwd_workspace_layout(64, 64, 256, offs, 4) == 0
    assert L.relu2_mlp_fwd_workspace_layout(64, 64, 256, offs, 3) == 1


def test_lm_head_ce_validation():
    L = _native.lib()
    assert L.fp8_lm_head_ce_workspace_bytes(256, 256, 600, 64) > 256 * 256 + 600 * 256 * 5
    assert L.fp8_lm_head_ce_workspace_bytes(256, 256, 600, 60) == 0        # chunk % 16
    assert L.fp8_lm_head_ce_workspace_bytes(256, 256, 1 << 23, 64) == 0    # vocabulary beyond the limit
    n = L.fp8_lm_head_ce_workspace_bytes(256, 256, 600, 64)
    f = ctypes.c_float
    ok = [FAKE, FAKE, FAKE, 256, 256, 600, 590, f(15.0), 64, FAKE, FAKE, FAKE, None, FAKE, n, 0, None]
    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return L.fp8_lm_head_ce(*a)
    assert call(a6=601) == 1                 # n_classes > V
    assert call(a6=0) == 1                   # no classes
    assert call(a7=f(0.0)) == 1              # softcap must be positive
    assert call(a3=250) == 5                 # M % 16
    assert call(a4=40) == 5                  # K % 16
    assert call(a9=None) == 1                # loss missing
    assert call(a14=n - 1) == 3              # workspace too small
    assert call(a0=ctypes.c_void_p(0x10008)) == 2   # x not 16-byte aligned
    assert call(a15=4) == 1                  # unknown accumulation mode
    offs = (ctypes.c_size_t * 11)()
    assert L.fp8_lm_head_ce_workspace_layout(256, 256, 600, 64, offs, 11) == 0
    assert list(offs) == sorted(offs) and offs[0] == 0


def test_rmsnorm_quant_validation():
    L = _native.lib()
    n = L.fp8_rmsnorm_quant_workspace_bytes(64, 64)
    assert n > 0 and L.fp8_rmsnorm_quant_workspace_bytes(-1, 64) == 0
    f = ctypes.c_float
    ok = [FAKE, None, f(1e-6), 64, 64, 64, 0, ctypes.c_void_p(0x20000), 64, None, 0, FAKE, None, FAKE, FAKE, n,
          None]
    assert L.fp8_rmsnorm_quant(*ok[:7], FAKE, *ok[8:]) == 1   # codes written over x
    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return L.fp8_rmsnorm_quant(*a)
    assert call(a13=None) == 1               # rstd missing
    assert call(a2=f(-1.0)) == 1             # negative eps
    assert call(a5=32) == 1                  # ldx < cols
    assert call(a15=n - 1) == 3              # workspace too small
    assert call(a1=FAKE_ODD) == 2            # gamma not 2-byte aligned


def test_swiglu_mlp_validation():
    L = _native.lib()
    M, d, h = 64, 64, 256
    nf = L.swiglu_mlp_fwd_workspace_bytes(M, d, h)
    nb = L.swiglu_mlp_bwd_workspace_bytes(M, d, h)
    assert nf > M * h * 2 and nb > M * d * 5 + M * h * 6
    assert L.swiglu_mlp_fwd_workspace_bytes(100, d, h) == 0            # M % 16
    assert L.swiglu_mlp_bwd_workspace_bytes(0, d, h) > 0               # M = 0 is a valid shape
    saved = _native.SwigluMlpSaved(*([0x10000] * 8))
    ok = [FAKE, FAKE, FAKE, FAKE, M, d, h, FAKE, ctypes.byref(saved), FAKE, nf, 0, None]
    def fwd(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return L.swiglu_mlp_fwd(*a)
    assert fwd(a10=nf - 1) == 3              # workspace too small
    assert fwd(a4=65) == 5                   # M % 16
    assert fwd(a6=-16) == 1                  # h < 0
    assert fwd(a7=None) == 1                 # y missing with M > 0
    assert fwd(a1=None) == 1                 # w_gate missing
    assert fwd(a2=ctypes.c_void_p(0x10008)) == 2   # w_up not 16-byte aligned
    for i in range(8):
        f = [0x10000] * 8
        f[i] = 0
        bad = _native.SwigluMlpSaved(*f)
        assert fwd(a8=ctypes.byref(bad)) == 1, i
    okb = [FAKE, ctypes.byref(saved), M, d, h, FAKE, FAKE, FAKE, FAKE, None, FAKE, nb, 0, None]
    def bwd(**kw):
        a = list(okb)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return L.swiglu_mlp_bwd(*a)
    assert bwd(a11=nb - 1) == 3
    assert bwd(a5=ctypes.c_void_p(0x10008)) == 2   # dx not 16-byte aligned
    assert bwd(a9=ctypes.c_void_p(0x10002)) == 2   # bwd_scales not 4-byte aligned
    assert bwd(a6=None) == 1                 # dw_gate missing
    for kind, n in (("fwd", 6), ("bwd", 10)):
        offs = (ctypes.c_size_t * n)()
        assert getattr(L, f"swiglu_mlp_{kind}_workspace_layout")(M, d, h, offs, n) == 0
        assert list(offs) == sorted(offs) and offs[0] == 0 and all(o % 256 == 0 for o in offs)
        assert getattr(L, f"swiglu_mlp_{kind}_workspace_layout")(M, d, h, offs, n - 1) == 1


def test_bf16_gemm_and_newton_schulz_validation():
    L = _native.lib()
    f = ctypes.c_float
    ok = [FAKE, 64, FAKE, 64, 32, 48, 64, f(1.0), f(0.0), None, 0, FAKE, 48, None, 0, None]
    def g(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return L.bf16_gemm_nt(*a)
    assert g(a6=60) == 5                     # K % 8
    assert g(a1=32) == 1                     # lda < K
    assert g(a0=ctypes.c_void_p(0x10008)) == 2
    assert g(a12=40) == 1                    # ldc < N
    assert g(a4=-1) == 1
    assert g(a4=0) == 0                      # empty output: nothing to do
    n = L.muon_ns_workspace_bytes(3072, 12288)
    assert n >= 3 * 3072 * 3072 * 2 + 2 * 3072 * 12288 * 2
    assert L.muon_ns_workspace_bytes(100, 64) == 0     # rows % 16
    assert L.muon_ns_workspace_bytes(32768, 32768) == 0  # m beyond the limit
    nb = L.muon_ns_workspace_bytes(64, 128)
    okn = [FAKE, 64, 128, 5, None, f(1e-7), ctypes.c_void_p(0x20000), None, FAKE, nb, None]
    def ns(**kw):
        a = list(okn)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return L.muon_newton_schulz(*a)
    assert ns(a9=nb - 1) == 3
    assert ns(a3=-1) == 1 and ns(a3=101) == 1
    assert ns(a5=f(-1.0)) == 1
    assert ns(a6=FAKE) == 1                  # out overlaps g
    assert ns(a6=ctypes.c_void_p(0x20008)) == 2
    assert ns(a1=0) == 0                     # empty matrix


def test_symmetric_product_validation():
    L = _native.lib()
    f = ctypes.c_float
    n = L.bf16_gemm_sym_workspace_bytes(3072, 12288)
    assert n >= 3072 * 3072 * 4 and L.bf16_gemm_sym_workspace_bytes(100, 64) == 0
    nb = L.bf16_gemm_sym_workspace_bytes(64, 128)
    ok = [FAKE, 128, 64, 128, f(1.0), f(0.0), None, 0, ctypes.c_void_p(0x20000), 64, FAKE, nb, None]
    def sym(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[int(k[1:])] = v
        return L.bf16_gemm_sym(*a)
    assert sym(a11=nb - 1) == 3
    assert sym(a2=60) == 5                   # M % 16
    assert sym(a1=64) == 1                   # lda < K
    assert sym(a9=32) == 1                   # ldc < M
    assert sym(a8=ctypes.c_void_p(0x20008)) == 2
    assert sym(a2=0) == 0
    # empty shapes: valid, with a (small) workspace size
    assert L.bf16_gemm_sym_workspace_bytes(0, 64) > 0 and L.bf16_gemm_sym_workspace_bytes(64, 0) > 0
    assert L.muon_ns_workspace_bytes(0, 64) > 0 and L.muon_ns_workspace_bytes(64, 0) > 0


def test_binding_checks_caller_outputs():
    """The Python binding refuses a caller-supplied output of the wrong
    shape, dtype or layout before anything reaches the library."""
    import torch
    from fp8_tensorwise_scaled_amd import api

    cpu = torch.device("cpu")
    ok = torch.empty((4, 8), dtype=torch.bfloat16)
    assert api._out(ok, (4, 8), torch.bfloat16, cpu, "y") is ok
    assert api._out(None, (4, 8), torch.bfloat16, cpu, "y").shape == (4, 8)
    wide = torch.empty((4, 16), dtype=torch.bfloat16)
    assert api._out(wide[:, :8], (4, 8), torch.bfloat16, cpu, "y").stride() == (16, 1)   # row stride allowed
    for bad in (torch.empty((3, 8), dtype=torch.bfloat16), torch.empty((4, 8), dtype=torch.float32),
                torch.empty((8, 4), dtype=torch.bfloat16).t()):
        with pytest.raises(ValueError):
            api._out(bad, (4, 8), torch.bfloat16, cpu, "y")
    with pytest.raises(ValueError):
        api._out(wide[:, :8], (4, 8), torch.bfloat16, cpu, "y", dense=True)
    with pytest.raises(ValueError):
        api._ws(torch.empty(16, dtype=torch.float32))


def test_no_fallback_without_the_library_or_a_gpu():
    """The product path has no CPU route: without the built library every
    entry point raises ImportError, and host tensors are refused before any
    call."""
    import subprocess
    import sys

    code = (
        "import torch\n"
        "from fp8_tensorwise_scaled_amd import _native, api\n"
        "_native.LIB_PATH = '/nonexistent/libfp8mlp.so'\n"
        "_native._lib = None\n"
        "try:\n"
        "    _native.lib()\n"
        "except ImportError as e:\n"
        "    print('library:', 'no CPU fallback' in str(e))\n"
        "try:\n"
        "    api.fp8_amax_quant(torch.zeros((16, 16), dtype=torch.bfloat16))\n"
        "except ValueError as e:\n"
        "    print('host tensor:', 'no CPU path' in str(e))\n"
        "from fp8_tensorwise_scaled_amd import modules\n"
        "try:\n"
        "    modules.fp8_linear(torch.zeros((16, 16), dtype=torch.bfloat16), torch.zeros((16, 16), dtype=torch.bfloat16))\n"
        "except ValueError as e:\n"
        "    print('module on host:', 'no CPU path' in str(e))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "library: True" in r.stdout and "host tensor: True" in r.stdout, r.stdout + r.stderr
    assert "module on host: True" in r.stdout, r.stdout + r.stderr
