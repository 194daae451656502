"""The C ABI on a host without a GPU: the library loads, exports every symbol
include/fng.h declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re

import pytest

from attention_fng_prenorm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fng.h")


def declared_symbols():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(fng_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for must in ("fng_prenorm_rms_gemm", "fng_gemm_postnorm_ln", "fng_gemm_postnorm_rms",
                 "fng_norm_attention", "fng_rmsnorm", "fng_layernorm", "fng_gemm", "fng_attention",
                 "fng_flash_norm_attention", "fng_jagged_attention", "fng_gemm_postnorm_ln_bwd",
                 "fng_gemm_postnorm_rms_bwd", "fng_prenorm_rms_bwd_dx", "fng_layernorm_bwd", "fng_rmsnorm_bwd"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in declared_symbols():
        assert hasattr(L, name), f"{name} not exported"
    # and the binding wraps each of them under the same name
    assert sorted(B.SIGNATURES) == declared_symbols()
    for name in declared_symbols():
        assert callable(getattr(B, name))


def test_only_fng_symbols_are_exported():
    # the dynamic symbol table should not leak internal C++ names
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    funcs = [ln.split()[-1] for ln in out.splitlines() if " T " in ln]
    assert funcs, "no exported functions"
    leaked = [f for f in funcs if not f.startswith("fng_") and not f.startswith("_init")
              and not f.startswith("_fini")]
    assert not leaked, leaked[:10]


def test_version_and_status_strings():
    assert B.fng_version() >= 1
    assert B.fng_status_string(0) == "ok"
    for s in range(1, 7):
        assert B.fng_status_string(s) not in ("ok", "unknown status")
    assert B.fng_status_string(99) == "unknown status"


def test_workspace_sizes():
    assert B.fng_gemm_postnorm_workspace_bytes(8192, 256, 256, B.FNG_PATH_AUTO) == 0
    assert B.fng_gemm_postnorm_workspace_bytes(8192, 256, 256, B.FNG_PATH_FULLN) == 0
    n = B.fng_gemm_postnorm_workspace_bytes(16384, 4096, 1024, B.FNG_PATH_SPLITN)
    # status + two counter arrays + 64 row blocks x 16 slices x 256 rows x 2 floats
    assert n >= 64 * 16 * 256 * 2 * 4
    assert B.fng_gemm_postnorm_workspace_bytes(0, 4096, 1024, B.FNG_PATH_SPLITN) == 0
    assert B.fng_fulln_max_n() >= 256
    # the automatic path (a workspace is needed exactly when it is not full-N):
    # N = 512 takes full-N at any K once the 128 x 512 tiles apply (M >= 32768),
    # else only while K <= 512; larger N takes split-N
    assert B.fng_gemm_postnorm_workspace_bytes(262144, 512, 2048, B.FNG_PATH_AUTO) == 0
    assert B.fng_gemm_postnorm_workspace_bytes(2048, 512, 512, B.FNG_PATH_AUTO) == 0
    assert B.fng_gemm_postnorm_workspace_bytes(2048, 512, 2048, B.FNG_PATH_AUTO) > 0
    assert B.fng_gemm_postnorm_workspace_bytes(262144, 1024, 64, B.FNG_PATH_AUTO) > 0


# raw C calls with arguments that validation must reject -------------------
L = None
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first
MIS = 0x10008   # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    return B.lib()


def test_prenorm_validation(lib):
    f = lib.fng_prenorm_rms_gemm
    assert f(FAKE, FAKE, None, FAKE, None, 4, 8, 0, 1e-6, None) == B.FNG_ERR_INVALID_ARG   # K = 0
    assert f(FAKE, FAKE, None, FAKE, None, -1, 8, 8, 1e-6, None) == B.FNG_ERR_INVALID_ARG  # M < 0
    assert f(FAKE, FAKE, None, FAKE, None, 4, 8, 8, 0.0, None) == B.FNG_ERR_INVALID_ARG    # eps = 0
    assert f(FAKE, FAKE, None, FAKE, None, 4, 8, 8, float("nan"), None) == B.FNG_ERR_INVALID_ARG
    assert f(None, FAKE, None, FAKE, None, 4, 8, 8, 1e-6, None) == B.FNG_ERR_INVALID_ARG   # NULL X
    assert f(MIS, FAKE, None, FAKE, None, 4, 8, 8, 1e-6, None) == B.FNG_ERR_MISALIGNED
    assert f(FAKE, FAKE, MIS, FAKE, None, 4, 8, 8, 1e-6, None) == B.FNG_ERR_MISALIGNED     # gamma
    assert f(FAKE, FAKE, None, FAKE, None, 4, 8, 12, 1e-6, None) == B.FNG_ERR_MISALIGNED   # K % 8
    assert f(FAKE, FAKE, None, FAKE, None, 4, 12, 8, 1e-6, None) == B.FNG_ERR_MISALIGNED   # N % 8
    assert f(FAKE, FAKE, None, FAKE, None, 4, 1 << 20, 1 << 14, 1e-6, None) == B.FNG_ERR_UNSUPPORTED
    # empty problems are a successful no-op (nothing is enqueued)
    assert f(None, None, None, None, None, 0, 8, 8, 1e-6, None) == B.FNG_OK
    assert f(None, None, None, None, None, 4, 0, 8, 1e-6, None) == B.FNG_OK


def test_postnorm_validation(lib):
    for f, ln in ((lib.fng_gemm_postnorm_ln, True), (lib.fng_gemm_postnorm_rms, False)):
        def call(X, W, Y, M, N, K, eps, ws, wsb, path):
            if ln:
                return f(X, W, Y, None, None, M, N, K, eps, ws, wsb, path, None)
            return f(X, W, Y, None, M, N, K, eps, ws, wsb, path, None)
        assert call(FAKE, FAKE, FAKE, 4, 8, 8, -1.0, None, 0, 0) == B.FNG_ERR_INVALID_ARG
        assert call(FAKE, FAKE, FAKE, 4, 8, 8, 1e-5, None, 0, 7) == B.FNG_ERR_INVALID_ARG     # bad path
        assert call(FAKE, FAKE, FAKE, 4, 8, 10, 1e-5, None, 0, 0) == B.FNG_ERR_MISALIGNED
        # full-N path cannot take N above its limit
        assert call(FAKE, FAKE, FAKE, 4, 4096, 8, 1e-5, None, 0, B.FNG_PATH_FULLN) == B.FNG_ERR_UNSUPPORTED
        # two-pass and split-N need the workspace
        assert call(FAKE, FAKE, FAKE, 4, 4096, 8, 1e-5, None, 0, B.FNG_PATH_TWOPASS) == B.FNG_ERR_WORKSPACE
        assert call(FAKE, FAKE, FAKE, 4, 4096, 8, 1e-5, FAKE, 64, B.FNG_PATH_TWOPASS) == B.FNG_ERR_WORKSPACE
        assert call(FAKE, FAKE, FAKE, 4, 4096, 8, 1e-5, MIS, 1 << 30, B.FNG_PATH_TWOPASS) == B.FNG_ERR_MISALIGNED
        assert call(None, None, None, 0, 4096, 8, 1e-5, None, 0, B.FNG_PATH_SPLITN) == B.FNG_OK


def test_attention_validation(lib):
    na = lib.fng_norm_attention
    a = lib.fng_attention
    args = (FAKE, FAKE, FAKE, FAKE)
    assert na(*args, None, None, None, 1, 8, 8, 2, 64, 0.0, 1e-5, 1e-6, None) == B.FNG_ERR_UNSUPPORTED
    assert na(*args, None, None, None, 1, 8, 0, 2, 128, 0.0, 1e-5, 1e-6, None) == B.FNG_ERR_INVALID_ARG
    assert na(*args, None, None, None, 1, 8, 8, 2, 128, 0.0, 0.0, 1e-6, None) == B.FNG_ERR_INVALID_ARG
    assert na(*args, None, None, None, 1, 8, 8, 2, 128, float("inf"), 1e-5, 1e-6, None) == B.FNG_ERR_INVALID_ARG
    assert na(MIS, FAKE, FAKE, FAKE, None, None, None, 1, 8, 8, 2, 128, 0.0, 1e-5, 1e-6, None) == B.FNG_ERR_MISALIGNED
    assert na(None, FAKE, FAKE, FAKE, None, None, None, 1, 8, 8, 2, 128, 0.0, 1e-5, 1e-6, None) == B.FNG_ERR_INVALID_ARG
    assert na(None, None, None, None, None, None, None, 0, 8, 8, 2, 128, 0.0, 1e-5, 1e-6, None) == B.FNG_OK
    assert a(*args, 1, 8, 8, 2, 96, 0.0, None) == B.FNG_ERR_UNSUPPORTED
    assert a(*args, 1, 1 << 22, 8, 64, 128, 0.0, None) == B.FNG_ERR_UNSUPPORTED
    assert a(None, None, None, None, 2, 0, 8, 2, 128, 0.0, None) == B.FNG_OK


def test_flash_norm_attention_validation(lib):
    f = lib.fng_flash_norm_attention
    j = lib.fng_jagged_attention
    S = B.FNG_ACT_SOFTMAX

    def call(Q=FAKE, off=FAKE, K=FAKE, V=FAKE, O=FAKE, b=2, T=16, L=8, skv=8, H=2, D=128,
             scale=0.0, e1=1e-5, e2=1e-6, act=S):
        return f(Q, off, K, V, O, None, None, None, b, T, L, skv, H, D, scale, e1, e2, act, None)

    assert call(D=64) == B.FNG_ERR_UNSUPPORTED
    assert call(H=3) == B.FNG_ERR_UNSUPPORTED            # heads must be 1, 2, 4 or 8
    assert call(H=16) == B.FNG_ERR_UNSUPPORTED
    assert call(skv=0) == B.FNG_ERR_INVALID_ARG
    assert call(T=-1) == B.FNG_ERR_INVALID_ARG
    assert call(act=2) == B.FNG_ERR_INVALID_ARG
    assert call(e1=0.0) == B.FNG_ERR_INVALID_ARG
    assert call(e2=float("nan")) == B.FNG_ERR_INVALID_ARG
    assert call(scale=float("inf")) == B.FNG_ERR_INVALID_ARG
    assert call(off=None) == B.FNG_ERR_INVALID_ARG
    assert call(Q=None) == B.FNG_ERR_INVALID_ARG
    assert call(Q=MIS) == B.FNG_ERR_MISALIGNED
    assert call(off=FAKE + 2) == B.FNG_ERR_MISALIGNED     # int32 offsets need 4-byte alignment
    assert call(L=1 << 22, H=4) == B.FNG_ERR_UNSUPPORTED  # per-batch query range beyond 32 bits
    assert call(skv=1 << 22, H=4) == B.FNG_ERR_UNSUPPORTED
    # empty problems: nothing enqueued
    assert call(Q=None, off=None, K=None, V=None, O=None, b=0) == B.FNG_OK
    assert call(Q=None, off=None, K=None, V=None, O=None, T=0) == B.FNG_OK
    assert call(Q=None, off=None, K=None, V=None, O=None, L=0) == B.FNG_OK
    assert j(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, 8, 8, 2, 128, 0.0, 5, None) == B.FNG_ERR_INVALID_ARG
    assert j(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 16, 8, 8, 2, 96, 0.0, S, None) == B.FNG_ERR_UNSUPPORTED
    assert j(None, None, None, None, None, 2, 0, 8, 8, 2, 128, 0.0, S, None) == B.FNG_OK


def test_prenorm_ln_validation(lib):
    f = lib.fng_prenorm_ln_gemm
    need = B.fng_prenorm_ln_workspace_bytes(1024, 4096)
    assert need == 8 * 1024 * 4
    assert B.fng_prenorm_ln_workspace_bytes(1024, 100) == 2 * 1024 * 4
    assert f(FAKE, FAKE, FAKE, None, None, 4, 1024, 4096, 1e-5, None, 0, None) == B.FNG_ERR_WORKSPACE
    assert f(FAKE, FAKE, FAKE, None, None, 4, 1024, 4096, 1e-5, FAKE, need - 4, None) == B.FNG_ERR_WORKSPACE
    assert f(FAKE, FAKE, FAKE, None, None, 4, 1024, 4096, 1e-5, MIS, need, None) == B.FNG_ERR_MISALIGNED
    assert f(FAKE, FAKE, FAKE, MIS, None, 4, 1024, 4096, 1e-5, FAKE, need, None) == B.FNG_ERR_MISALIGNED
    assert f(FAKE, FAKE, FAKE, None, None, 4, 1024, 4096, 0.0, FAKE, need, None) == B.FNG_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, None, None, 4, 1024, 12, 1e-5, FAKE, need, None) == B.FNG_ERR_MISALIGNED
    assert f(None, None, None, None, None, 0, 1024, 4096, 1e-5, None, 0, None) == B.FNG_OK


def test_flash_norm_attention_bwd_validation(lib):
    f = lib.fng_flash_norm_attention_bwd
    S = B.FNG_ACT_SOFTMAX
    need = B.fng_flash_norm_attention_bwd_workspace_bytes(16, 2)
    assert need == 16 * 2 * (128 * 2 + 4)
    assert B.fng_flash_norm_attention_bwd_workspace_bytes(0, 2) == 0

    def call(Q=FAKE, off=FAKE, K=FAKE, V=FAKE, O=FAKE, dO=FAKE, st=FAKE, dQ=FAKE, dK=FAKE, dV=FAKE,
             ws=FAKE, wsb=None, b=2, T=16, L=8, skv=8, H=2, D=128, scale=0.0, act=S):
        return f(Q, off, K, V, O, dO, st, st, st, dQ, dK, dV, ws, need if wsb is None else wsb,
                 b, T, L, skv, H, D, scale, act, None)

    assert call(skv=129) == B.FNG_ERR_UNSUPPORTED        # short KV: at most 128 keys
    assert call(D=64) == B.FNG_ERR_UNSUPPORTED
    assert call(H=3) == B.FNG_ERR_UNSUPPORTED
    assert call(H=16) == B.FNG_ERR_UNSUPPORTED
    assert B.fng_flash_norm_attention_bwd_workspace_bytes(16, 8) == 16 * 8 * (128 * 2 + 4)
    assert call(H=8) == B.FNG_ERR_WORKSPACE               # eight heads: the workspace sized for two is too small
    assert call(act=7) == B.FNG_ERR_INVALID_ARG
    assert call(scale=float("nan")) == B.FNG_ERR_INVALID_ARG
    assert call(ws=None) == B.FNG_ERR_WORKSPACE
    assert call(wsb=need - 1) == B.FNG_ERR_WORKSPACE
    assert call(ws=MIS) == B.FNG_ERR_MISALIGNED
    assert call(dO=None) == B.FNG_ERR_INVALID_ARG
    assert call(dK=None) == B.FNG_ERR_INVALID_ARG
    assert call(st=None) == B.FNG_ERR_INVALID_ARG
    assert call(st=FAKE + 2) == B.FNG_ERR_MISALIGNED
    assert call(dV=MIS) == B.FNG_ERR_MISALIGNED
    assert call(dQ=MIS) == B.FNG_ERR_MISALIGNED
    # no batch or no head: nothing to write
    assert call(Q=None, off=None, K=None, V=None, O=None, dO=None, dK=None, dV=None, b=0) == B.FNG_OK
    # no query row: dK, dV still written (zeros), so they and K, V, offsets are checked
    assert call(Q=None, O=None, dO=None, st=None, dQ=None, ws=None, T=0, dK=None) == B.FNG_ERR_INVALID_ARG
    assert call(Q=None, O=None, dO=None, st=None, dQ=None, ws=None, T=0, K=MIS) == B.FNG_ERR_MISALIGNED


def test_backward_validation(lib):
    # (function, whether its N and K name the product's output and reduction
    # sizes in that order: the pre-norm input gradient takes the forward's)
    for f, swap in ((lib.fng_gemm_postnorm_ln_bwd, False), (lib.fng_gemm_postnorm_rms_bwd, False),
                    (lib.fng_prenorm_rms_bwd_dx, True)):
        def call(G=FAKE, Wt=FAKE, H=FAKE, r=FAKE, dZ=FAKE, M=4, N=8, K=8, ws=None, wsb=0, path=0):
            # N = the norm axis, K = the reduction, whatever the entry point calls them
            return f(G, Wt, H, r, dZ, M, K, N, ws, wsb, path, None) if swap else \
                f(G, Wt, H, r, dZ, M, N, K, ws, wsb, path, None)
        assert call(K=0) == B.FNG_ERR_INVALID_ARG
        assert call(path=9) == B.FNG_ERR_INVALID_ARG
        assert call(H=None) == B.FNG_ERR_INVALID_ARG
        assert call(r=None) == B.FNG_ERR_INVALID_ARG
        assert call(H=MIS) == B.FNG_ERR_MISALIGNED
        assert call(r=FAKE + 2) == B.FNG_ERR_MISALIGNED
        assert call(N=12, K=12) == B.FNG_ERR_MISALIGNED                          # rows of whole 16-B vectors
        assert call(path=B.FNG_PATH_TWOPASS) == B.FNG_ERR_UNSUPPORTED            # no two-pass backward
        assert call(M=4, N=4096, K=4096, path=B.FNG_PATH_FULLN) == B.FNG_ERR_UNSUPPORTED
        assert call(M=4, N=4096, K=4096, path=B.FNG_PATH_SPLITN) == B.FNG_ERR_WORKSPACE
        assert call(M=1 << 20, N=4096, K=8) == B.FNG_ERR_UNSUPPORTED            # saved tensor over 2 GiB
        assert call(G=None, Wt=None, H=None, r=None, dZ=None, M=0) == B.FNG_OK
    assert lib.fng_layernorm_bwd(FAKE, FAKE, FAKE, FAKE, 4, 12, None) == B.FNG_ERR_MISALIGNED
    assert lib.fng_layernorm_bwd(FAKE, None, FAKE, FAKE, 4, 8, None) == B.FNG_ERR_INVALID_ARG
    assert lib.fng_rmsnorm_bwd(FAKE, FAKE, FAKE + 1, FAKE, 4, 8, 1, None) == B.FNG_ERR_MISALIGNED
    assert lib.fng_rmsnorm_bwd(FAKE, FAKE, FAKE, FAKE, 4, 0, 0, None) == B.FNG_ERR_INVALID_ARG
    assert lib.fng_rmsnorm_bwd(None, None, None, None, 0, 8, 0, None) == B.FNG_OK


def test_norm_and_gemm_validation(lib):
    assert lib.fng_rmsnorm(FAKE, None, FAKE, None, 4, 12, 1e-6, None) == B.FNG_ERR_MISALIGNED
    assert lib.fng_rmsnorm(FAKE, None, FAKE, None, 4, 0, 1e-6, None) == B.FNG_ERR_INVALID_ARG
    assert lib.fng_rmsnorm(FAKE, None, FAKE, None, 4, 8, 0.0, None) == B.FNG_ERR_INVALID_ARG
    assert lib.fng_rmsnorm(None, None, None, None, 0, 8, 1e-6, None) == B.FNG_OK
    assert lib.fng_layernorm(MIS, FAKE, None, None, 4, 8, 1e-5, None) == B.FNG_ERR_MISALIGNED
    assert lib.fng_layernorm(None, FAKE, None, None, 4, 8, 1e-5, None) == B.FNG_ERR_INVALID_ARG
    assert lib.fng_gemm(FAKE, FAKE, FAKE, 4, 8, 0, None) == B.FNG_ERR_INVALID_ARG
    assert lib.fng_gemm(FAKE, FAKE, MIS, 4, 8, 8, None) == B.FNG_ERR_MISALIGNED
    assert lib.fng_gemm(None, None, None, 0, 8, 8, None) == B.FNG_OK


def test_get_kernel_status_validation(lib):
    assert lib.fng_get_kernel_status(None, 0, None) == B.FNG_ERR_WORKSPACE
    assert lib.fng_get_kernel_status(FAKE, 16, None) == B.FNG_ERR_WORKSPACE
    assert lib.fng_get_kernel_status(MIS, 4096, None) == B.FNG_ERR_MISALIGNED


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        B.fng_gemm(x, torch.zeros(8, 8, dtype=torch.bfloat16), torch.zeros(4, 8, dtype=torch.bfloat16))


def test_weight_gradient_validation(lib):
    f = lib.fng_prenorm_rms_bwd_dw
    # (X, rstd, dY, gamma, dW, M, N, K, stream)
    assert f(FAKE, FAKE, FAKE, None, FAKE, 0, 8, 8, None) == B.FNG_ERR_INVALID_ARG     # empty batch
    assert f(FAKE, FAKE, FAKE, None, FAKE, 4, -1, 8, None) == B.FNG_ERR_INVALID_ARG
    assert f(None, FAKE, FAKE, None, FAKE, 4, 8, 8, None) == B.FNG_ERR_INVALID_ARG     # NULL X
    assert f(FAKE, None, FAKE, FAKE, FAKE, 4, 8, 8, None) == B.FNG_ERR_INVALID_ARG     # gain without rstd
    assert f(FAKE, MIS, FAKE, None, FAKE, 4, 8, 8, None) == B.FNG_ERR_MISALIGNED       # rstd
    assert f(FAKE, FAKE, FAKE, MIS, FAKE, 4, 8, 8, None) == B.FNG_ERR_MISALIGNED       # gamma
    assert f(FAKE, FAKE, FAKE, None, FAKE, 4, 8, 12, None) == B.FNG_ERR_MISALIGNED     # K % 8
    assert f(FAKE, FAKE, FAKE, None, FAKE, 4, 12, 8, None) == B.FNG_ERR_MISALIGNED     # N % 8
    assert f(FAKE, FAKE, FAKE, None, FAKE, 1 << 20, 8, 4096, None) == B.FNG_ERR_UNSUPPORTED  # X over 2 GiB
    assert f(None, None, None, None, None, 4, 0, 8, None) == B.FNG_OK                  # nothing to write
    assert f(None, None, None, None, None, 4, 8, 0, None) == B.FNG_OK


def test_noalloc_validation(lib):
    f = lib.fng_gemm_postnorm_rms_noalloc
    # (X, W, Y, rstd_out, M, N, K, eps, path, stream); every case is rejected
    # before the library's array is looked up
    assert f(FAKE, FAKE, FAKE, None, 4, 8, 8, 0.0, 0, None) == B.FNG_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, None, 4, 8, 8, 1e-6, 7, None) == B.FNG_ERR_INVALID_ARG
    assert f(MIS, FAKE, FAKE, None, 4, 8, 8, 1e-6, 0, None) == B.FNG_ERR_MISALIGNED
    assert f(FAKE, FAKE, FAKE, None, 4, 4096, 8, 1e-6, B.FNG_PATH_FULLN, None) == B.FNG_ERR_UNSUPPORTED
    # split-N workspace of 65536 x 8192 is 16 MiB, above the 8 MiB array
    assert B.fng_gemm_postnorm_workspace_bytes(65536, 8192, 64, B.FNG_PATH_SPLITN) > (8 << 20)
    assert f(FAKE, FAKE, FAKE, None, 65536, 8192, 64, 1e-6, B.FNG_PATH_SPLITN, None) == B.FNG_ERR_WORKSPACE
    assert f(FAKE, FAKE, FAKE, None, 65536, 8192, 64, 1e-6, B.FNG_PATH_TWOPASS, None) == B.FNG_ERR_WORKSPACE
    assert f(None, None, None, None, 0, 8, 8, 1e-6, 0, None) == B.FNG_OK


def test_prenorm_ws_validation(lib):
    f = lib.fng_prenorm_rms_gemm_ws
    # (X, W, gamma, Y, rstd_out, M, N, K, eps, ws, wsb, stream)
    assert f(FAKE, FAKE, None, FAKE, None, 4, 8, 8, 0.0, FAKE, 1 << 20, None) == B.FNG_ERR_INVALID_ARG
    assert f(FAKE, FAKE, MIS, FAKE, None, 4, 8, 8, 1e-6, FAKE, 1 << 20, None) == B.FNG_ERR_MISALIGNED
    assert f(FAKE, FAKE, None, FAKE, None, 4, 8, 8, 1e-6, None, 0, None) == B.FNG_ERR_WORKSPACE
    need = B.fng_prenorm_rms_gemm_workspace_bytes(4096, 14336, 4096, True)
    assert need >= 4096 * 14336 * 2 + 4096 * 4      # rstd + the gain-scaled W
    assert B.fng_prenorm_rms_gemm_workspace_bytes(4096, 14336, 4096, False) == 4096 * 4
    assert B.fng_prenorm_rms_gemm_workspace_bytes(256, 128, 128, True) == 1024   # small tiles: no scaled W
    assert f(FAKE, FAKE, FAKE, FAKE, None, 4096, 14336, 4096, 1e-6, FAKE, need - 16, None) == B.FNG_ERR_WORKSPACE
    assert f(FAKE, FAKE, None, FAKE, None, 4096, 14336, 4096, 1e-6, MIS, need, None) == B.FNG_ERR_MISALIGNED
    assert f(None, None, None, None, None, 0, 8, 8, 1e-6, None, 0, None) == B.FNG_OK
