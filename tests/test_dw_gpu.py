"""GPU parity of the lazy pre-RMSNorm weight gradient (fng_prenorm_rms_bwd_dw,
through the C ABI) against the fp64 oracle: dW = (rmsnorm(X) * gamma)^T dY
with rstd applied along the contraction inside the product (Towards Free
Normalization, section 2's limitations: the normalized input is rebuilt for
the gradients of both operands).

Cases: the small tiles and the 256 x 256 tiles with the tail launch, ragged
contraction lengths (rows of the batch not a multiple of the 32-row K tile),
ragged output rows and columns, with and without the gain, zero rows of X
(rstd = 1/sqrt(eps)), the plain product (rstd NULL), and the LLM-MLP shape
(X [4096, 4096], dY [4096, 14336]) on sampled output rows.  rstd is the
forward kernel's own rstd_out, as in training.

Tolerance: dW sums M products, so it is not unit-scale (mean |dW| is about
sqrt(M)); the agreed gate is applied relative to that scale: normwise max
relative error <= 1e-2, and a mean absolute error within 1e-3 * s of the
bf16 rounding floor of the exact result and never above 2e-3 * s, where
s = mean|dW| / 0.8 (the mean magnitude of a unit normal)."""

import numpy as np
import pytest
import torch

import oracle
from attention_fng_prenorm_amd import binding as B
from attention_fng_prenorm_amd import inputs
from gpu_util import assert_parity_floor, dev, empty_bf16, host, log

import gpu_util


def dw_parity(y, ref, what):
    """The gate relative to dW's scale (see the module docstring)."""
    scale = max(1.0, float(np.mean(np.abs(ref))) / 0.8)
    return assert_parity_floor(y, ref, what, margin=gpu_util.FLOOR_MARGIN * scale)

pytestmark = pytest.mark.gpu

f64 = oracle.bf16_to_f64


def dw_case(M, K, N, seed, gamma, zero_rows=()):
    """The weight-gradient recipe at reduced size, with zero rows of X planted."""
    spec, d = inputs.make_inputs("prenorm_rms_mlp_dw_gamma" if gamma else "prenorm_rms_mlp_dw", M=M, K=K, N=N,
                                 seed=seed)
    x = d["X"].copy()
    for r in zero_rows:
        x[r] = 0
    return spec, x, d["dY"], d["gamma"]


def run_dw(x, dy, g, eps, with_rstd=True):
    M, K = x.shape
    N = dy.shape[1]
    X, dY = dev(x), dev(dy)
    G = dev(g) if g is not None else None
    r = None
    if with_rstd:
        # the forward kernel's rstd output, as a training step keeps it
        Wf = torch.zeros(K, 8, dtype=torch.bfloat16, device="cuda")
        Yf = torch.empty(M, 8, dtype=torch.bfloat16, device="cuda")
        r = torch.empty(M, dtype=torch.float32, device="cuda")
        B.fng_prenorm_rms_gemm(X, Wf, Yf, eps, gamma=G, rstd_out=r)
    dW = empty_bf16(K, N)
    B.fng_prenorm_rms_bwd_dw(X, r, dY, dW, gamma=G)
    torch.cuda.synchronize()
    return dW, (r.cpu().numpy() if r is not None else None)


@pytest.mark.parametrize("gamma", [False, True], ids=["plain", "gamma"])
@pytest.mark.parametrize("shape", [(256, 128, 128), (300, 1104, 4000), (1000, 264, 4104), (33, 2048, 2056)],
                         ids=["small_tiles", "ragged_contraction", "tall_batch", "short_batch"])
def test_dw_reduced(shape, gamma):
    M, K, N = shape
    spec, x, dy, g = dw_case(M, K, N, seed=601, gamma=gamma, zero_rows=(0, M // 2))
    g = g if gamma else None
    log(f"dW M={M} K={K} N={N} gamma={gamma}")
    dW, r = run_dw(x, dy, g, spec["eps"])
    rref = oracle.rms_rstd(f64(x), spec["eps"])
    assert np.max(np.abs(r - rref) / rref) < 2e-4
    ref = oracle.prenorm_rms_backward_dw(f64(x), f64(dy), r, f64(g) if g is not None else None)
    dw_parity(host(dW), ref, f"dW {shape} gamma={gamma}")


def test_dw_plain_product():
    M, K, N = 300, 1104, 4000
    spec, x, dy, _ = dw_case(M, K, N, seed=602, gamma=False)
    log("dW with rstd NULL: the plain X^T dY")
    dW, _ = run_dw(x, dy, None, spec["eps"], with_rstd=False)
    ref = f64(x).T @ f64(dy)
    dw_parity(host(dW), ref, "X^T dY")


def test_dw_matches_unfused_composition():
    """rmsnorm(X) written out by the row-norm kernel, then the plain product:
    the chain the fused call replaces, against the same oracle."""
    M, K, N = 520, 1024, 4096
    spec, x, dy, _ = dw_case(M, K, N, seed=603, gamma=False)
    X, dY = dev(x), dev(dy)
    Xn = empty_bf16(M, K)
    r = torch.empty(M, dtype=torch.float32, device="cuda")
    B.fng_rmsnorm(X, Xn, spec["eps"], rstd_out=r)
    dWu, dWf = empty_bf16(K, N), empty_bf16(K, N)
    B.fng_prenorm_rms_bwd_dw(Xn, None, dY, dWu)
    B.fng_prenorm_rms_bwd_dw(X, r, dY, dWf)
    torch.cuda.synchronize()
    ref = oracle.prenorm_rms_backward_dw(f64(x), f64(dy), r.cpu().numpy())
    # both round one operand of the product to bf16 once: the unfused chain
    # rmsnorm(X), the fused call rstd * dY
    dw_parity(host(dWf), ref, "fused dW")
    dw_parity(host(dWu), ref, "unfused rmsnorm + X^T dY")


def test_dw_deterministic_and_guarded():
    M, K, N = 700, 1104, 4000
    spec, x, dy, _ = dw_case(M, K, N, seed=604, gamma=False)
    X, dY = dev(x), dev(dy)
    r = torch.from_numpy(oracle.rms_rstd(f64(x), spec["eps"]).astype(np.float32)).cuda()
    guard = 3 * N
    buf = empty_bf16(K * N + guard)
    buf.view(torch.int16).fill_(0x1234)
    dW = buf[: K * N].view(K, N)
    B.fng_prenorm_rms_bwd_dw(X, r, dY, dW)
    dW2 = empty_bf16(K, N)
    B.fng_prenorm_rms_bwd_dw(X, r, dY, dW2)
    torch.cuda.synchronize()
    assert torch.equal(dW.view(torch.int16), dW2.view(torch.int16)), "run-to-run difference"
    assert bool((buf[K * N:].view(torch.int16) == 0x1234).all()), "write past the end of dW"


def test_dw_invalid_args():
    x = empty_bf16(0, 64)
    with pytest.raises(B.FngError):
        B.fng_prenorm_rms_bwd_dw(x, None, empty_bf16(0, 64), empty_bf16(64, 64))
    X = empty_bf16(64, 60)   # K not a multiple of 8
    with pytest.raises(B.FngError):
        B.fng_prenorm_rms_bwd_dw(X, None, empty_bf16(64, 64), empty_bf16(60, 64))


@pytest.mark.parametrize("gamma", [False, True], ids=["plain", "gamma"])
def test_dw_llm_mlp_full_size_sampled(gamma):
    spec, d = inputs.make_inputs("prenorm_rms_mlp_dw_gamma" if gamma else "prenorm_rms_mlp_dw")
    M, K, N = spec["M"], spec["K"], spec["N"]
    x, dy, g = d["X"], d["dY"], d["gamma"]
    log(f"dW full size X [{M},{K}] dY [{M},{N}] gamma={gamma}")
    dW, r = run_dw(x, dy, g, spec["eps"])
    rng = np.random.default_rng(9)
    ks = np.unique(np.concatenate([[0, 255, 256, K - 1], rng.choice(K, 44, replace=False)]))
    ref = oracle.prenorm_rms_backward_dw(f64(x[:, ks]), f64(dy), r, f64(g[ks]) if g is not None else None)
    y = host(dW[torch.as_tensor(ks, device="cuda")])
    dw_parity(y, ref, f"dW full size sampled rows gamma={gamma}")
    # the tail launch's columns (the last partial round of 256 x 256 tiles)
    dw_parity(y[:, 12288:], ref[:, 12288:], "dW tail columns")
