"""The post-RMSNorm GEMM entry point that allocates nothing
(fng_gemm_postnorm_rms_noalloc: its workspace is a fixed device array inside
the library), through the C ABI, against fng_gemm_postnorm_rms with a caller
workspace and against the fp64 oracle: two calls in a row on each path, the
second with a smaller input, then a shape too large for the array."""

import numpy as np
import pytest
import torch

import oracle
from attention_fng_prenorm_amd import binding as B
from attention_fng_prenorm_amd import inputs
from gpu_util import assert_close_stats, assert_parity, dev, empty_bf16, host, log

pytestmark = pytest.mark.gpu

f64 = oracle.bf16_to_f64


def run_pair(M, K, N, path, seed):
    spec, d = inputs.make_inputs("postnorm_rms_largen", M=M, K=K, N=N, seed=seed)
    X, W = dev(d["X"]), dev(d["W"])
    Ya, Yb = empty_bf16(M, N), empty_bf16(M, N)
    ra = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    rb = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    B.fng_gemm_postnorm_rms_noalloc(X, W, Ya, spec["eps"], path=path, rstd_out=ra)
    nb = B.fng_gemm_postnorm_workspace_bytes(M, N, K, path)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    B.fng_gemm_postnorm_rms(X, W, Yb, spec["eps"], workspace=ws, path=path, rstd_out=rb)
    torch.cuda.synchronize()
    return spec, d, Ya, Yb, ra, rb


@pytest.mark.parametrize("path", [B.FNG_PATH_SPLITN, B.FNG_PATH_TWOPASS, B.FNG_PATH_AUTO],
                         ids=["splitn", "twopass", "auto"])
def test_noalloc_matches_workspace_entry_point(path):
    # the second call is smaller, and reuses what the first left in the array
    for M, K, N, seed in ((1100, 520, 4096, 71), (300, 256, 1320, 72)):
        log(f"noalloc post-RMS path={path} M={M} K={K} N={N}")
        spec, d, Ya, Yb, ra, rb = run_pair(M, K, N, path, seed)
        assert torch.equal(Ya.view(torch.int16), Yb.view(torch.int16)), "differs from the workspace entry point"
        assert torch.equal(ra, rb)
        ref, _, rref = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), spec["eps"], "rms")
        assert_parity(host(Ya), ref, f"noalloc post-RMS path {path} {M}x{K}x{N}")
        assert_close_stats(ra.cpu().numpy(), rref, "noalloc rstd")


def test_noalloc_workload_shape():
    # the post-RMSNorm workload itself (16384 x 1024 x 4096, split-N), sampled rows
    spec, d = inputs.make_inputs("postnorm_rms_largen")
    M, K, N = spec["M"], spec["K"], spec["N"]
    log(f"noalloc post-RMS workload {M}x{K}x{N}")
    X, W = dev(d["X"]), dev(d["W"])
    Y = empty_bf16(M, N)
    B.fng_gemm_postnorm_rms_noalloc(X, W, Y, spec["eps"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(12).choice(M, 40, replace=False)]))
    ref, _, _ = oracle.gemm_postnorm(f64(d["X"][rows]), f64(d["W"]), spec["eps"], "rms")
    assert_parity(host(Y[torch.as_tensor(rows, device="cuda")]), ref, "noalloc workload sampled rows")


def test_noalloc_rejects_oversize():
    M, K, N = 65536, 64, 8192   # split-N workspace of 16 MiB: twice the array
    assert B.fng_gemm_postnorm_workspace_bytes(M, N, K, B.FNG_PATH_SPLITN) > (8 << 20)
    X, W, Y = empty_bf16(M, K, poison=False), empty_bf16(K, N, poison=False), empty_bf16(M, N, poison=False)
    with pytest.raises(B.FngError) as e:
        B.fng_gemm_postnorm_rms_noalloc(X, W, Y, 1e-6, path=B.FNG_PATH_SPLITN)
    assert e.value.status == B.FNG_ERR_WORKSPACE
    del X, W, Y
    torch.cuda.empty_cache()
