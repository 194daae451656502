"""Thin Python binding of libfng.so (ctypes): argument marshalling only.

Every function here has the name of the C entry point it calls and does no
arithmetic of its own: it checks tensor dtypes/devices/contiguity, passes raw
device pointers, sizes and the current HIP stream, and raises FngError when the
library returns a non-OK status.  All computation runs in the HIP kernels; if
the library is missing, loading fails loudly (there is no fallback).
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfng.so")

FNG_OK = 0
FNG_ERR_INVALID_ARG = 1
FNG_ERR_UNSUPPORTED = 2
FNG_ERR_MISALIGNED = 3
FNG_ERR_WORKSPACE = 4
FNG_ERR_HIP = 5
FNG_ERR_TIMEOUT = 6

FNG_PATH_AUTO = 0
FNG_PATH_FULLN = 1
FNG_PATH_SPLITN = 2
FNG_PATH_TWOPASS = 3

FNG_ACT_SOFTMAX = 0
FNG_ACT_GELU = 1

_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_vp = ctypes.c_void_p
_int = ctypes.c_int
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/fng.h
SIGNATURES = {
    "fng_prenorm_rms_gemm": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _vp]),
    "fng_gemm_postnorm_workspace_bytes": (_sz, [_i64, _i64, _i64, _int]),
    "fng_prenorm_ln_workspace_bytes": (_sz, [_i64, _i64]),
    "fng_prenorm_rms_gemm_workspace_bytes": (_sz, [_i64, _i64, _i64, _int]),
    "fng_prenorm_rms_gemm_ws": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _vp, _sz, _vp]),
    "fng_prenorm_ln_gemm": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _vp, _sz, _vp]),
    "fng_fulln_max_n": (_i64, []),
    "fng_gemm_postnorm_ln": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _vp, _sz, _int, _vp]),
    "fng_gemm_postnorm_rms": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _vp, _sz, _int, _vp]),
    "fng_get_kernel_status": (_int, [_vp, _sz, _vp]),
    "fng_gemm_postnorm_rms_noalloc": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _vp]),
    "fng_gemm_postnorm_affine": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _f32, _int, _vp, _sz,
                                        _int, _vp]),
    "fng_norm_attention": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                  _f32, _f32, _f32, _vp]),
    "fng_rmsnorm": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp]),
    "fng_layernorm": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _f32, _vp]),
    "fng_gemm": (_int, [_vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fng_attention": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _vp]),
    "fng_gemm_postnorm_ln_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _int, _vp]),
    "fng_gemm_postnorm_rms_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _int, _vp]),
    "fng_prenorm_rms_bwd_dx": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _sz, _int, _vp]),
    "fng_prenorm_rms_bwd_dw": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]),
    "fng_layernorm_bwd": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _vp]),
    "fng_rmsnorm_bwd": (_int, [_vp, _vp, _vp, _vp, _i64, _i64, _int, _vp]),
    "fng_flash_norm_attention": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64,
                                        _i64, _i64, _i64, _f32, _f32, _f32, _int, _vp]),
    "fng_jagged_attention": (_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                    _f32, _int, _vp]),
    "fng_flash_norm_attention_bwd_workspace_bytes": (_sz, [_i64, _i64]),
    "fng_flash_norm_attention_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                            _vp, _sz, _i64, _i64, _i64, _i64, _i64, _i64, _f32, _int, _vp]),
    "fng_jagged_attention_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _i64, _i64, _i64, _i64,
                                        _i64, _i64, _f32, _int, _vp]),
    "fng_status_string": (ctypes.c_char_p, [_int]),
    "fng_version": (_int, []),
}

_lib = None


class FngError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = lib().fng_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: status {status} ({msg})")


def lib():
    """The loaded libfng.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m attention_fng_prenorm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t, dtype=None, what="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _check(fn, status):
    if status != FNG_OK:
        raise FngError(fn, status)


def _bf(t, what):
    return _ptr(t, torch.bfloat16, what)


def _f(t, what):
    return _ptr(t, torch.float32, what)


def fng_prenorm_rms_gemm(X, W, Y, eps, gamma=None, rstd_out=None, stream=None):
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(Y.shape) != (M, N):
        raise ValueError("shapes: X [M,K], W [K,N], Y [M,N]")
    _check("fng_prenorm_rms_gemm", lib().fng_prenorm_rms_gemm(
        _bf(X, "X"), _bf(W, "W"), _bf(gamma, "gamma"), _bf(Y, "Y"), _f(rstd_out, "rstd_out"),
        M, N, K, eps, _stream(stream)))


def fng_prenorm_rms_gemm_workspace_bytes(M, N, K, has_gamma=False):
    return lib().fng_prenorm_rms_gemm_workspace_bytes(M, N, K, 1 if has_gamma else 0)


def fng_prenorm_rms_gemm_ws(X, W, Y, eps, workspace, gamma=None, rstd_out=None, stream=None):
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(Y.shape) != (M, N):
        raise ValueError("shapes: X [M,K], W [K,N], Y [M,N]")
    wp, wb = _ws(workspace)
    _check("fng_prenorm_rms_gemm_ws", lib().fng_prenorm_rms_gemm_ws(
        _bf(X, "X"), _bf(W, "W"), _bf(gamma, "gamma"), _bf(Y, "Y"), _f(rstd_out, "rstd_out"), M, N, K, eps,
        wp, wb, _stream(stream)))


def fng_prenorm_ln_workspace_bytes(N, K):
    return int(lib().fng_prenorm_ln_workspace_bytes(N, K))


def fng_prenorm_ln_gemm(X, W, Y, eps, workspace, mean_out=None, rstd_out=None, stream=None):
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(Y.shape) != (M, N):
        raise ValueError("shapes: X [M,K], W [K,N], Y [M,N]")
    wp, wb = _ws(workspace)
    _check("fng_prenorm_ln_gemm", lib().fng_prenorm_ln_gemm(
        _bf(X, "X"), _bf(W, "W"), _bf(Y, "Y"), _f(mean_out, "mean_out"), _f(rstd_out, "rstd_out"),
        M, N, K, eps, wp, wb, _stream(stream)))


def fng_gemm_postnorm_workspace_bytes(M, N, K, path=FNG_PATH_AUTO):
    return int(lib().fng_gemm_postnorm_workspace_bytes(M, N, K, path))


def fng_fulln_max_n():
    return int(lib().fng_fulln_max_n())


def _ws(workspace):
    if workspace is None:
        return None, 0
    return _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size()


def fng_gemm_postnorm_ln(X, W, Y, eps, workspace=None, path=FNG_PATH_AUTO, mean_out=None,
                         rstd_out=None, stream=None):
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(Y.shape) != (M, N):
        raise ValueError("shapes: X [M,K], W [K,N], Y [M,N]")
    wp, wb = _ws(workspace)
    _check("fng_gemm_postnorm_ln", lib().fng_gemm_postnorm_ln(
        _bf(X, "X"), _bf(W, "W"), _bf(Y, "Y"), _f(mean_out, "mean_out"), _f(rstd_out, "rstd_out"),
        M, N, K, eps, wp, wb, path, _stream(stream)))


def fng_gemm_postnorm_rms(X, W, Y, eps, workspace=None, path=FNG_PATH_AUTO, rstd_out=None,
                          stream=None):
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(Y.shape) != (M, N):
        raise ValueError("shapes: X [M,K], W [K,N], Y [M,N]")
    wp, wb = _ws(workspace)
    _check("fng_gemm_postnorm_rms", lib().fng_gemm_postnorm_rms(
        _bf(X, "X"), _bf(W, "W"), _bf(Y, "Y"), _f(rstd_out, "rstd_out"),
        M, N, K, eps, wp, wb, path, _stream(stream)))


def fng_gemm_postnorm_affine(X, W, Y, eps, gamma, beta=None, ln=True, workspace=None, path=FNG_PATH_AUTO,
                             mean_out=None, rstd_out=None, stream=None):
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(Y.shape) != (M, N):
        raise ValueError("shapes: X [M,K], W [K,N], Y [M,N]")
    wp, wb = _ws(workspace)
    _check("fng_gemm_postnorm_affine", lib().fng_gemm_postnorm_affine(
        _bf(X, "X"), _bf(W, "W"), _bf(gamma, "gamma"), _bf(beta, "beta"), _bf(Y, "Y"),
        _f(mean_out, "mean_out"), _f(rstd_out, "rstd_out"), M, N, K, eps, 1 if ln else 0, wp, wb, path,
        _stream(stream)))


def fng_gemm_postnorm_rms_noalloc(X, W, Y, eps, path=FNG_PATH_AUTO, rstd_out=None, stream=None):
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(Y.shape) != (M, N):
        raise ValueError("shapes: X [M,K], W [K,N], Y [M,N]")
    _check("fng_gemm_postnorm_rms_noalloc", lib().fng_gemm_postnorm_rms_noalloc(
        _bf(X, "X"), _bf(W, "W"), _bf(Y, "Y"), _f(rstd_out, "rstd_out"), M, N, K, eps, path, _stream(stream)))


def fng_get_kernel_status(workspace, stream=None):
    wp, wb = _ws(workspace)
    return int(lib().fng_get_kernel_status(wp, wb, _stream(stream)))


def fng_norm_attention(Q, K, V, out, eps_ln, eps_rms, sm_scale=0.0, ln_mean_out=None,
                       ln_rstd_out=None, rms_rstd_out=None, stream=None):
    B, Sq, H, D = Q.shape
    Skv = K.shape[1]
    if tuple(K.shape) != (B, Skv, H, D) or tuple(V.shape) != (B, Skv, H, D) or out.shape != Q.shape:
        raise ValueError("shapes: Q/out [B,Sq,H,D], K/V [B,Skv,H,D]")
    _check("fng_norm_attention", lib().fng_norm_attention(
        _bf(Q, "Q"), _bf(K, "K"), _bf(V, "V"), _bf(out, "out"), _f(ln_mean_out, "ln_mean_out"),
        _f(ln_rstd_out, "ln_rstd_out"), _f(rms_rstd_out, "rms_rstd_out"),
        B, Sq, Skv, H, D, sm_scale, eps_ln, eps_rms, _stream(stream)))


def fng_rmsnorm(X, Y, eps, gamma=None, rstd_out=None, stream=None):
    M, N = X.shape
    if Y.shape != X.shape:
        raise ValueError("Y must have X's shape")
    _check("fng_rmsnorm", lib().fng_rmsnorm(
        _bf(X, "X"), _bf(gamma, "gamma"), _bf(Y, "Y"), _f(rstd_out, "rstd_out"), M, N, eps,
        _stream(stream)))


def fng_layernorm(X, Y, eps, mean_out=None, rstd_out=None, stream=None):
    M, N = X.shape
    if Y.shape != X.shape:
        raise ValueError("Y must have X's shape")
    _check("fng_layernorm", lib().fng_layernorm(
        _bf(X, "X"), _bf(Y, "Y"), _f(mean_out, "mean_out"), _f(rstd_out, "rstd_out"), M, N, eps,
        _stream(stream)))


def fng_gemm(X, W, Y, stream=None):
    M, K = X.shape
    N = W.shape[1]
    if W.shape[0] != K or tuple(Y.shape) != (M, N):
        raise ValueError("shapes: X [M,K], W [K,N], Y [M,N]")
    _check("fng_gemm", lib().fng_gemm(_bf(X, "X"), _bf(W, "W"), _bf(Y, "Y"), M, N, K,
                                      _stream(stream)))


def fng_attention(Q, K, V, out, sm_scale=0.0, stream=None):
    B, Sq, H, D = Q.shape
    Skv = K.shape[1]
    if tuple(K.shape) != (B, Skv, H, D) or tuple(V.shape) != (B, Skv, H, D) or out.shape != Q.shape:
        raise ValueError("shapes: Q/out [B,Sq,H,D], K/V [B,Skv,H,D]")
    _check("fng_attention", lib().fng_attention(
        _bf(Q, "Q"), _bf(K, "K"), _bf(V, "V"), _bf(out, "out"), B, Sq, Skv, H, D, sm_scale,
        _stream(stream)))


def _bwd(fn, G, Wt, H, rstd, dZ, workspace, path, stream, sizes):
    wp, wb = _ws(workspace)
    _check(fn, getattr(lib(), fn)(_bf(G, "G"), _bf(Wt, "Wt"), _bf(H, "saved tensor"), _f(rstd, "rstd"),
                                  _bf(dZ, "output"), *sizes, wp, wb, path, _stream(stream)))


def fng_gemm_postnorm_ln_bwd(G, Wt, Y, rstd, dZ, workspace=None, path=FNG_PATH_AUTO, stream=None):
    M, K = G.shape
    N = Wt.shape[1]
    if Wt.shape[0] != K or tuple(Y.shape) != (M, N) or tuple(dZ.shape) != (M, N) or tuple(rstd.shape) != (M,):
        raise ValueError("shapes: G [M,K], Wt [K,N], Y/dZ [M,N], rstd [M]")
    _bwd("fng_gemm_postnorm_ln_bwd", G, Wt, Y, rstd, dZ, workspace, path, stream, (M, N, K))


def fng_gemm_postnorm_rms_bwd(G, Wt, Y, rstd, dZ, workspace=None, path=FNG_PATH_AUTO, stream=None):
    M, K = G.shape
    N = Wt.shape[1]
    if Wt.shape[0] != K or tuple(Y.shape) != (M, N) or tuple(dZ.shape) != (M, N) or tuple(rstd.shape) != (M,):
        raise ValueError("shapes: G [M,K], Wt [K,N], Y/dZ [M,N], rstd [M]")
    _bwd("fng_gemm_postnorm_rms_bwd", G, Wt, Y, rstd, dZ, workspace, path, stream, (M, N, K))


def fng_prenorm_rms_bwd_dx(dY, Wt, X, rstd, dX, workspace=None, path=FNG_PATH_AUTO, stream=None):
    M, N = dY.shape
    K = Wt.shape[1]
    if Wt.shape[0] != N or tuple(X.shape) != (M, K) or tuple(dX.shape) != (M, K) or tuple(rstd.shape) != (M,):
        raise ValueError("shapes: dY [M,N], Wt [N,K], X/dX [M,K], rstd [M]")
    _bwd("fng_prenorm_rms_bwd_dx", dY, Wt, X, rstd, dX, workspace, path, stream, (M, N, K))


def fng_prenorm_rms_bwd_dw(X, rstd, dY, dW, gamma=None, stream=None):
    M, K = X.shape
    N = dY.shape[1]
    if dY.shape[0] != M or tuple(dW.shape) != (K, N) or (rstd is not None and tuple(rstd.shape) != (M,)) or (
            gamma is not None and tuple(gamma.shape) != (K,)):
        raise ValueError("shapes: X [M,K], rstd [M], dY [M,N], dW [K,N], gamma [K]")
    _check("fng_prenorm_rms_bwd_dw", lib().fng_prenorm_rms_bwd_dw(
        _bf(X, "X"), _f(rstd, "rstd"), _bf(dY, "dY"), _bf(gamma, "gamma"), _bf(dW, "dW"), M, N, K,
        _stream(stream)))


def fng_layernorm_bwd(G, Y, rstd, dZ, stream=None):
    M, N = G.shape
    if tuple(Y.shape) != (M, N) or tuple(dZ.shape) != (M, N):
        raise ValueError("G, Y, dZ must share one shape")
    _check("fng_layernorm_bwd", lib().fng_layernorm_bwd(_bf(G, "G"), _bf(Y, "Y"), _f(rstd, "rstd"),
                                                        _bf(dZ, "dZ"), M, N, _stream(stream)))


def fng_rmsnorm_bwd(G, H, rstd, dZ, h_is_input=False, stream=None):
    M, N = G.shape
    if tuple(H.shape) != (M, N) or tuple(dZ.shape) != (M, N):
        raise ValueError("G, H, dZ must share one shape")
    _check("fng_rmsnorm_bwd", lib().fng_rmsnorm_bwd(_bf(G, "G"), _bf(H, "H"), _f(rstd, "rstd"),
                                                    _bf(dZ, "dZ"), M, N, int(bool(h_is_input)),
                                                    _stream(stream)))


def _act(act):
    codes = {"softmax": FNG_ACT_SOFTMAX, "gelu": FNG_ACT_GELU}
    return codes[act] if isinstance(act, str) else int(act)


def _jagged_shapes(Q, q_offsets, K, V, out):
    T, H, D = Q.shape
    B, Skv = K.shape[0], K.shape[1]
    if tuple(K.shape) != (B, Skv, H, D) or tuple(V.shape) != (B, Skv, H, D) or out.shape != Q.shape:
        raise ValueError("shapes: Q/out [T,H,D], K/V [B,Skv,H,D]")
    if tuple(q_offsets.shape) != (B + 1,):
        raise ValueError("q_offsets must be [B+1]")
    return T, H, D, B, Skv


def fng_flash_norm_attention(Q, q_offsets, K, V, out, max_len_q, eps_ln, eps_rms, sm_scale=0.0,
                             act="softmax", ln_mean_out=None, ln_rstd_out=None, rms_rstd_out=None,
                             stream=None):
    T, H, D, B, Skv = _jagged_shapes(Q, q_offsets, K, V, out)
    _check("fng_flash_norm_attention", lib().fng_flash_norm_attention(
        _bf(Q, "Q"), _ptr(q_offsets, torch.int32, "q_offsets"), _bf(K, "K"), _bf(V, "V"),
        _bf(out, "out"), _f(ln_mean_out, "ln_mean_out"), _f(ln_rstd_out, "ln_rstd_out"),
        _f(rms_rstd_out, "rms_rstd_out"), B, T, max_len_q, Skv, H, D, sm_scale, eps_ln, eps_rms,
        _act(act), _stream(stream)))


def fng_flash_norm_attention_bwd_workspace_bytes(T, H):
    return int(lib().fng_flash_norm_attention_bwd_workspace_bytes(T, H))


def fng_flash_norm_attention_bwd(Q, q_offsets, K, V, out, dout, ln_mean, ln_rstd, rms_rstd, dQ, dK, dV,
                                 max_len_q, workspace=None, sm_scale=0.0, act="softmax", stream=None):
    T, H, D, B, Skv = _jagged_shapes(Q, q_offsets, K, V, out)
    if dout.shape != Q.shape or dQ.shape != Q.shape or dK.shape != K.shape or dV.shape != V.shape:
        raise ValueError("shapes: dout/dQ like Q, dK/dV like K")
    wp, wb = _ws(workspace)
    _check("fng_flash_norm_attention_bwd", lib().fng_flash_norm_attention_bwd(
        _bf(Q, "Q"), _ptr(q_offsets, torch.int32, "q_offsets"), _bf(K, "K"), _bf(V, "V"),
        _bf(out, "out"), _bf(dout, "dout"), _f(ln_mean, "ln_mean"), _f(ln_rstd, "ln_rstd"),
        _f(rms_rstd, "rms_rstd"), _bf(dQ, "dQ"), _bf(dK, "dK"), _bf(dV, "dV"), wp, wb,
        B, T, max_len_q, Skv, H, D, sm_scale, _act(act), _stream(stream)))


def fng_jagged_attention_bwd(Q, q_offsets, K, V, dout, dQ, dK, dV, max_len_q, workspace=None, sm_scale=0.0,
                             act="softmax", stream=None):
    T, H, D, B, Skv = _jagged_shapes(Q, q_offsets, K, V, dout)
    if dQ.shape != Q.shape or dK.shape != K.shape or dV.shape != V.shape:
        raise ValueError("shapes: dout/dQ like Q, dK/dV like K")
    wp, wb = _ws(workspace)
    _check("fng_jagged_attention_bwd", lib().fng_jagged_attention_bwd(
        _bf(Q, "Q"), _ptr(q_offsets, torch.int32, "q_offsets"), _bf(K, "K"), _bf(V, "V"), _bf(dout, "dout"),
        _bf(dQ, "dQ"), _bf(dK, "dK"), _bf(dV, "dV"), wp, wb, B, T, max_len_q, Skv, H, D, sm_scale, _act(act),
        _stream(stream)))


def fng_jagged_attention(Q, q_offsets, K, V, out, max_len_q, sm_scale=0.0, act="softmax",
                         stream=None):
    T, H, D, B, Skv = _jagged_shapes(Q, q_offsets, K, V, out)
    _check("fng_jagged_attention", lib().fng_jagged_attention(
        _bf(Q, "Q"), _ptr(q_offsets, torch.int32, "q_offsets"), _bf(K, "K"), _bf(V, "V"),
        _bf(out, "out"), B, T, max_len_q, Skv, H, D, sm_scale, _act(act), _stream(stream)))


def fng_status_string(status):
    return lib().fng_status_string(status).decode()


def fng_version():
    return int(lib().fng_version())
