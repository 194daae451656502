"""GPU parity of the lazy LayerNorm pre-norm GEMM (fng_prenorm_ln_gemm: Y =
layernorm(X) @ W applied as diag(rstd) (X W - mean colsum(W))) against the fp64
oracle, through the C ABI: reduced shapes with ragged tiles, rows far off zero
mean (the rank-1 correction's cancellation), the LLM-MLP shape on sampled rows,
and the unfused LayerNorm + GEMM beside it.

Tolerance: normwise max relative error <= 1e-2 and mean absolute error <= 2e-3
(outputs are unit-scale: W ~ N(0, 1/K)); fp32 statistics within 2e-4 relative."""

import numpy as np
import pytest
import torch

import oracle
from attention_fng_prenorm_amd import binding as B
from attention_fng_prenorm_amd import inputs
from gpu_util import assert_close_stats, assert_parity, dev, empty_bf16, host, log

pytestmark = pytest.mark.gpu


def f64(bits):
    return oracle.bf16_to_f64(bits)


def run(d, eps, M, N, K, ws=None):
    X, W = dev(d["X"]), dev(d["W"])
    Y = empty_bf16(M, N)
    mu = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = torch.empty(B.fng_prenorm_ln_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")
    B.fng_prenorm_ln_gemm(X, W, Y, eps, ws, mean_out=mu, rstd_out=r)
    torch.cuda.synchronize()
    return Y, mu, r


@pytest.mark.parametrize("shape", [(256, 128, 128), (300, 1000, 1000), (1100, 520, 4000), (4000, 264, 14200),
                                   (4096, 264, 16384)],
                         ids=["small", "ragged_small_tile", "ragged_large_tile", "tail_launch", "rounds_split"])
def test_prenorm_ln_reduced(shape):
    M, K, N = shape
    spec, d = inputs.make_inputs("prenorm_ln_mlp", M=M, K=K, N=N, seed=51)
    log(f"lazy LN pre-norm M={M} K={K} N={N}")
    Y, mu, r = run(d, spec["eps"], M, N, K)
    rows = np.arange(M) if M * N <= 4e6 else np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(1).choice(M, 40, replace=False)]))
    ref, rmu, rr = oracle.prenorm_ln_gemm(f64(d["X"][rows]), f64(d["W"]), spec["eps"])
    assert_parity(host(Y)[rows], ref, f"lazy LN {shape}")
    _, amu, ar = oracle.layernorm_rows(f64(d["X"]), spec["eps"])
    assert np.max(np.abs(mu.cpu().numpy() - amu)) <= 2e-4 * np.max(np.abs(amu)) + 1e-6
    assert_close_stats(r.cpu().numpy(), ar, "lazy LN rstd")


@pytest.mark.parametrize("shape", [(512, 1024, 1024), (4096, 256, 8192)], ids=["one_launch", "row_scale_split"])
@pytest.mark.parametrize("shift", [8.0, 32.0])
def test_prenorm_ln_far_off_mean(shift, shape):
    # every row's mean is `shift` spreads away from zero: X W and mean colsum(W)
    # are both `shift` times the result and cancel in the epilogue (at the
    # larger shape in the row-scale launch, from the statistic launch's mean)
    M, K, N = shape
    rng = np.random.Generator(np.random.PCG64(52))
    z = rng.standard_normal((M, K), dtype=np.float32)
    sign = np.where(rng.standard_normal((M, 1)) > 0, 1.0, -1.0).astype(np.float32)
    x = (z + np.float32(shift) * sign) * np.exp(rng.standard_normal((M, 1), dtype=np.float32))
    w = rng.standard_normal((K, N), dtype=np.float32) / np.float32(np.sqrt(K))
    d = {"X": inputs.f32_to_bf16_bits(x), "W": inputs.f32_to_bf16_bits(w)}
    log(f"lazy LN pre-norm, |mean| = {shift} x spread")
    Y, mu, r = run(d, 1e-5, M, N, K)
    rows = np.arange(M) if M * N <= 4e6 else np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(2).choice(M, 40, replace=False)]))
    ref, _, rr = oracle.prenorm_ln_gemm(f64(d["X"][rows]), f64(d["W"]), 1e-5)
    e = assert_parity(host(Y)[rows], ref, f"lazy LN shift {shift}")
    log(f"shift {shift}: {e}")
    assert_close_stats(r.cpu().numpy()[rows], rr, "lazy LN rstd, shifted rows", rtol=2e-3 if shift > 10 else 2e-4)


def test_prenorm_ln_full_size_sampled():
    spec, d = inputs.make_inputs("prenorm_ln_mlp")
    M, K, N = spec["M"], spec["K"], spec["N"]
    log(f"lazy LN pre-norm full size {M}x{K}x{N}")
    Y, mu, r = run(d, spec["eps"], M, N, K)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(8).choice(M, 44, replace=False)]))
    ref, _, _ = oracle.prenorm_ln_gemm(f64(d["X"][rows]), f64(d["W"]), spec["eps"])
    assert_parity(host(Y[torch.as_tensor(rows, device="cuda")]), ref, "lazy LN full size sampled rows")


def test_prenorm_ln_matches_unfused():
    M, K, N = 520, 1024, 2048
    spec, d = inputs.make_inputs("prenorm_ln_mlp", M=M, K=K, N=N, seed=53)
    log("lazy LN vs layernorm + gemm")
    Y, _, _ = run(d, spec["eps"], M, N, K)
    X, W = dev(d["X"]), dev(d["W"])
    xn = empty_bf16(M, K)
    B.fng_layernorm(X, xn, spec["eps"])
    Yu = empty_bf16(M, N)
    B.fng_gemm(xn, W, Yu)
    torch.cuda.synchronize()
    ref, _, _ = oracle.prenorm_ln_gemm(f64(d["X"]), f64(d["W"]), spec["eps"])
    ef = assert_parity(host(Y), ref, "lazy LN fused")
    eu = assert_parity(host(Yu), ref, "layernorm + gemm")
    log(f"fused {ef} unfused {eu}")


def test_prenorm_ln_deterministic_guarded_and_workspace_reuse():
    M, K, N = 520, 256, 2048
    spec, d = inputs.make_inputs("prenorm_ln_mlp", M=M, K=K, N=N, seed=54)
    X, W = dev(d["X"]), dev(d["W"])
    ws = torch.empty(B.fng_prenorm_ln_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")
    guard = 3 * N
    buf = empty_bf16(M * N + guard)
    buf.view(torch.int16).fill_(0x1234)
    Y = buf[: M * N].view(M, N)
    log("lazy LN determinism")
    B.fng_prenorm_ln_gemm(X, W, Y, spec["eps"], ws)
    Y2 = empty_bf16(M, N)
    B.fng_prenorm_ln_gemm(X, W, Y2, spec["eps"], ws)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), "run-to-run difference"
    assert bool((buf[M * N:].view(torch.int16) == 0x1234).all()), "write past the end of Y"
    # the same workspace for a smaller problem afterwards
    spec, d = inputs.make_inputs("prenorm_ln_mlp", M=64, K=128, N=512, seed=55)
    Y3, _, _ = run(d, spec["eps"], 64, 512, 128, ws=ws)
    ref, _, _ = oracle.prenorm_ln_gemm(f64(d["X"]), f64(d["W"]), spec["eps"])
    assert_parity(host(Y3), ref, "lazy LN, reused workspace")
