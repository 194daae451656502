"""GPU parity: every HIP entry point (called through the C ABI) against the fp64
oracle on the same seeded bf16 inputs, at reduced sizes spanning several tiles
with ragged tails, and at the full workload sizes on sampled output rows.

Tolerance (all outputs are bf16): normwise max relative error <= 1e-2 and mean
absolute error <= 2e-3 against the oracle; fp32 statistics outputs within a
relative 2e-4."""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_fng_prenorm_amd import binding as B
from attention_fng_prenorm_amd import inputs
from gpu_util import assert_close_stats, assert_parity, assert_parity_floor, dev, empty_bf16, host, log

pytestmark = pytest.mark.gpu


def f64(bits):
    return oracle.bf16_to_f64(bits)


# ---------------------------------------------------------------------------
# lazy pre-RMSNorm GEMM
# ---------------------------------------------------------------------------

def run_prenorm(d, eps, M, N, K):
    X, W = dev(d["X"]), dev(d["W"])
    g = dev(d["gamma"]) if d.get("gamma") is not None else None
    Y = empty_bf16(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    B.fng_prenorm_rms_gemm(X, W, Y, eps, gamma=g, rstd_out=r)
    torch.cuda.synchronize()
    return Y, r


@pytest.mark.parametrize("gamma", [False, True])
@pytest.mark.parametrize("shape", [(256, 128, 128), (300, 1000, 1000), (1100, 520, 4000)],
                         ids=["small_workload", "ragged_small_tile", "ragged_large_tile"])
def test_prenorm_reduced(shape, gamma):
    M, K, N = shape
    spec, d = inputs.make_inputs("prenorm_rms_mlp_gamma" if gamma else "prenorm_rms_small",
                                 M=M, K=K, N=N)
    log(f"prenorm M={M} K={K} N={N} gamma={gamma}")
    Y, r = run_prenorm(d, spec["eps"], M, N, K)
    ref, rref = oracle.prenorm_rms_gemm(f64(d["X"]), f64(d["W"]), spec["eps"],
                                        f64(d["gamma"]) if gamma else None)
    assert_parity(host(Y), ref, f"prenorm {shape} gamma={gamma}")
    assert_close_stats(r.cpu().numpy(), rref, "prenorm rstd")


@pytest.fixture(scope="module")
def mlp_inputs():
    spec, d = inputs.make_inputs("prenorm_rms_mlp")
    return spec, d


@pytest.mark.parametrize("gamma", [False, True])
def test_prenorm_full_size_sampled(gamma):
    name = "prenorm_rms_mlp_gamma" if gamma else "prenorm_rms_mlp"
    spec, d = inputs.make_inputs(name)
    M, K, N = spec["M"], spec["K"], spec["N"]
    log(f"prenorm full size {M}x{K}x{N} gamma={gamma}")
    Y, r = run_prenorm(d, spec["eps"], M, N, K)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 44, replace=False)]))
    x = f64(d["X"][rows])
    ref, rref = oracle.prenorm_rms_gemm(x, f64(d["W"]), spec["eps"],
                                        f64(d["gamma"]) if gamma else None)
    assert_parity(host(Y[torch.as_tensor(rows, device="cuda")]), ref, f"{name} sampled rows")
    # rstd of every row: only needs X
    rall = oracle.rms_rstd(f64(d["X"]), spec["eps"])
    assert_close_stats(r.cpu().numpy(), rall, "prenorm rstd (all rows)")


@pytest.mark.parametrize("kind", ["gemm", "prenorm", "prenorm_gamma"])
def test_big_tiles_with_tail_launch(kind):
    # 16 x 56 tiles of 256 x 256 are 3.5 rounds of 256 CUs: the trailing 8 column
    # blocks run as a second launch of 128 x 256 tiles (ragged here: N = 14200)
    M, K, N = 4000, 264, 14200
    spec, d = inputs.make_inputs("prenorm_rms_mlp_gamma" if kind == "prenorm_gamma" else "prenorm_rms_mlp",
                                 M=M, K=K, N=N, seed=17)
    X, W = dev(d["X"]), dev(d["W"])
    g = dev(d["gamma"]) if kind == "prenorm_gamma" else None
    guard = 2 * N
    buf = empty_bf16(M * N + guard)
    buf.view(torch.int16).fill_(0x1234)
    Y = buf[: M * N].view(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    log(f"big tiles + tail {kind} {M}x{K}x{N}")
    if kind == "gemm":
        B.fng_gemm(X, W, Y)
    else:
        B.fng_prenorm_rms_gemm(X, W, Y, spec["eps"], gamma=g, rstd_out=r)
    torch.cuda.synchronize()
    assert bool((buf[M * N:].view(torch.int16) == 0x1234).all()), "write past the end of Y"
    rows = np.unique(np.concatenate([[0, 255, 256, 3839, 3840, M - 1], np.random.default_rng(5).choice(M, 40, replace=False)]))
    x = f64(d["X"][rows])
    if kind == "gemm":
        ref = oracle.gemm(x, f64(d["W"]))
    else:
        ref, _ = oracle.prenorm_rms_gemm(x, f64(d["W"]), spec["eps"], f64(d["gamma"]) if g is not None else None)
        assert_close_stats(r.cpu().numpy(), oracle.rms_rstd(f64(d["X"]), spec["eps"]), "rstd (all rows)")
    y = host(Y[torch.as_tensor(rows, device="cuda")])
    assert_parity(y, ref, f"{kind} sampled rows")
    # the tail columns on their own (the second launch)
    assert_parity(y[:, 12288:], ref[:, 12288:], f"{kind} tail columns")


@pytest.mark.parametrize("shape", [(2048, 264, 16384), (4096, 264, 14336), (2000, 136, 16360)],
                         ids=["two_whole_rounds", "whole_rounds_plus_half", "ragged_two_rounds"])
def test_prenorm_statistic_shared_between_launches(shape):
    """With rstd_out given, the big-tile lazy pre-norm accumulates each row's
    sum of squares in one launch (the half-size tiles of the last partial
    round, or the first round's columns) and the other launch applies the
    rstd it wrote: against the oracle, on both launches' columns, and
    against the call that accumulates the statistic in every tile."""
    M, K, N = shape
    spec, d = inputs.make_inputs("prenorm_rms_mlp", M=M, K=K, N=N, seed=88)
    X, W = dev(d["X"]), dev(d["W"])
    Y, Y2 = empty_bf16(M, N), empty_bf16(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    log(f"lazy pre-norm, statistic shared between launches {M}x{K}x{N}")
    B.fng_prenorm_rms_gemm(X, W, Y, spec["eps"], rstd_out=r)
    B.fng_prenorm_rms_gemm(X, W, Y2, spec["eps"])
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 127, 128, 255, 256, M - 1],
                                     np.random.default_rng(M).choice(M, 40, replace=False)]))
    ref, rref = oracle.prenorm_rms_gemm(f64(d["X"][rows]), f64(d["W"]), spec["eps"])
    y = host(Y[torch.as_tensor(rows, device="cuda")])
    assert_parity(y, ref, "shared statistic, all columns")
    for c0, c1 in ((0, 4096), (N - 2048, N)):
        assert_parity(y[:, c0:c1], ref[:, c0:c1], f"columns {c0}..{c1}")
    assert_close_stats(r.cpu().numpy(), oracle.rms_rstd(f64(d["X"]), spec["eps"]), "rstd (all rows)")
    # the two schemes differ at most by the last bit of rstd
    diff = (Y.float() - Y2.float()).abs().max().item()
    assert diff <= 2.0 ** -7 * Y2.float().abs().max().item(), diff


@pytest.mark.parametrize("gamma", [False, True], ids=["plain", "gamma"])
@pytest.mark.parametrize("shape", [(256, 128, 128), (1100, 520, 4000), (4000, 264, 14200)],
                         ids=["small_tiles", "big_tiles", "big_tiles_tail"])
@pytest.mark.parametrize("with_rstd", [True, False], ids=["rstd_out", "no_rstd_out"])
def test_prenorm_ws(shape, gamma, with_rstd):
    """fng_prenorm_rms_gemm_ws: the gain folded into W by a streaming pass
    into the workspace (then the lazy kernel without a gain), the statistic
    handed between launches through rstd_out or the workspace; against the
    oracle and against fng_prenorm_rms_gemm (the in-loop fold)."""
    M, K, N = shape
    spec, d = inputs.make_inputs("prenorm_rms_mlp_gamma" if gamma else "prenorm_rms_mlp", M=M, K=K, N=N, seed=91)
    X, W = dev(d["X"]), dev(d["W"])
    g = dev(d["gamma"]) if gamma else None
    ws = torch.empty(B.fng_prenorm_rms_gemm_workspace_bytes(M, N, K, gamma), dtype=torch.uint8, device="cuda")
    guard = 2 * N
    buf = empty_bf16(M * N + guard)
    buf.view(torch.int16).fill_(0x1234)
    Y = buf[: M * N].view(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda") if with_rstd else None
    log(f"prenorm ws {shape} gamma={gamma} rstd_out={with_rstd}")
    B.fng_prenorm_rms_gemm_ws(X, W, Y, spec["eps"], ws, gamma=g, rstd_out=r)
    Y2 = empty_bf16(M, N)
    B.fng_prenorm_rms_gemm(X, W, Y2, spec["eps"], gamma=g)
    torch.cuda.synchronize()
    assert bool((buf[M * N:].view(torch.int16) == 0x1234).all()), "write past the end of Y"
    rows = np.unique(np.concatenate([[0, 127, 128, 255, 256, M - 1],
                                     np.random.default_rng(M + N).choice(M, 40, replace=False)]))
    rows = rows[rows < M]
    ref, rref = oracle.prenorm_rms_gemm(f64(d["X"][rows]), f64(d["W"]), spec["eps"], f64(d["gamma"]) if gamma else None)
    assert_parity(host(Y[torch.as_tensor(rows, device="cuda")]), ref, f"prenorm ws {shape} gamma={gamma}")
    if with_rstd:
        assert_close_stats(r.cpu().numpy(), oracle.rms_rstd(f64(d["X"]), spec["eps"]), "rstd (all rows)")
    # same products, the statistic at most one fp32 rounding apart
    diff = (Y.float() - Y2.float()).abs().max().item()
    assert diff <= 2.0 ** -7 * Y2.float().abs().max().item(), diff


def test_prenorm_deterministic_and_guarded():
    spec, d = inputs.make_inputs("prenorm_rms_mlp", M=520, K=256, N=2048)
    M, N, K = 520, 2048, 256
    X, W = dev(d["X"]), dev(d["W"])
    guard = 3 * N
    buf = empty_bf16(M * N + guard)
    buf.view(torch.int16).fill_(0x1234)
    Y = buf[: M * N].view(M, N)
    B.fng_prenorm_rms_gemm(X, W, Y, spec["eps"])
    Y2 = empty_bf16(M, N)
    B.fng_prenorm_rms_gemm(X, W, Y2, spec["eps"])
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16)), "run-to-run difference"
    assert bool((buf[M * N:].view(torch.int16) == 0x1234).all()), "write past the end of Y"


# ---------------------------------------------------------------------------
# GEMM + post-norm
# ---------------------------------------------------------------------------

def run_postnorm(d, eps, M, N, K, ln, path):
    X, W = dev(d["X"]), dev(d["W"])
    Y = empty_bf16(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    mu = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda") if ln else None
    wsb = B.fng_gemm_postnorm_workspace_bytes(M, N, K, path)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda") if wsb else None
    if ln:
        B.fng_gemm_postnorm_ln(X, W, Y, eps, workspace=ws, path=path, mean_out=mu, rstd_out=r)
    else:
        B.fng_gemm_postnorm_rms(X, W, Y, eps, workspace=ws, path=path, rstd_out=r)
    torch.cuda.synchronize()
    if ws is not None:
        assert B.fng_get_kernel_status(ws) == B.FNG_OK
    return Y, mu, r, ws


def test_postnorm_ln_smalln_workload_fulln():
    spec, d = inputs.make_inputs("postnorm_ln_smalln")
    M, K, N = spec["M"], spec["K"], spec["N"]
    assert B.fng_gemm_postnorm_workspace_bytes(M, N, K, B.FNG_PATH_AUTO) == 0
    Y, mu, r, _ = run_postnorm(d, spec["eps"], M, N, K, True, B.FNG_PATH_AUTO)
    ref, mref, rref = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), spec["eps"], "ln")
    assert_parity(host(Y), ref, "post-LN 8192x256x256 full-N")
    assert_close_stats(r.cpu().numpy(), rref, "post-LN rstd")
    assert np.max(np.abs(mu.cpu().numpy() - mref)) < 2e-4


SHORT_K = [8, 32, 72, 96, 136]


@pytest.mark.parametrize("K", SHORT_K, ids=[f"K{k}" for k in SHORT_K])
@pytest.mark.parametrize("kind", ["gemm", "prenorm", "splitn_rms", "twopass_ln", "fulln_tall_ln"])
def test_short_k_loops(kind, K):
    """The 8-wave tiles' ping-pong mainloop keeps three K tiles of copies in
    flight: K loops of 1 to 5 tiles (K tails of 8 and 40 included) exercise its
    prologue, the zero-filled refills past the last tile and the phase barriers,
    on every path that runs it; ragged M and N, a guard band after Y."""
    if kind in ("gemm", "prenorm"):
        M, N = 1100, 4000  # big tiles (M * N above the small-problem size)
    elif kind == "fulln_tall_ln":
        M, N = 65536 + 72, 200  # 256 x 256 full-N tiles from 65536 rows on
    else:
        M, N = 700, 1544
    spec, d = inputs.make_inputs("postnorm_rms_largen", M=M, K=K, N=N, seed=300 + K)
    X, W = dev(d["X"]), dev(d["W"])
    log(f"short K loop {kind} M={M} K={K} N={N}")
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(K).choice(M, 64, replace=False)]))
    x = f64(d["X"][rows])
    if kind in ("gemm", "prenorm"):
        buf = empty_bf16(M * N + 2 * N)
        buf.view(torch.int16).fill_(0x1234)
        Y = buf[: M * N].view(M, N)
        r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
        if kind == "gemm":
            B.fng_gemm(X, W, Y)
            ref = oracle.gemm(x, f64(d["W"]))
        else:
            B.fng_prenorm_rms_gemm(X, W, Y, 1e-6, rstd_out=r)
            ref, rref = oracle.prenorm_rms_gemm(x, f64(d["W"]), 1e-6)
        torch.cuda.synchronize()
        assert bool((buf[M * N:].view(torch.int16) == 0x1234).all()), "write past the end of Y"
        if kind == "prenorm":
            assert_close_stats(r.cpu().numpy()[rows], rref, "rstd sampled")
    else:
        ln = kind.endswith("ln")
        path = {"splitn_rms": B.FNG_PATH_SPLITN, "twopass_ln": B.FNG_PATH_TWOPASS,
                "fulln_tall_ln": B.FNG_PATH_FULLN}[kind]
        eps = 1e-5 if ln else 1e-6
        Y, mu, r, _ = run_postnorm(d, eps, M, N, K, ln, path)
        ref, mref, rref = oracle.gemm_postnorm(x, f64(d["W"]), eps, "ln" if ln else "rms")
        assert_close_stats(r.cpu().numpy()[rows], rref, "rstd sampled")
        if ln:
            assert np.max(np.abs(mu.cpu().numpy()[rows] - mref)) < 2e-4
    assert_parity(host(Y[torch.as_tensor(rows, device="cuda")]), ref, f"{kind} K={K}")


@pytest.mark.parametrize("ln", [True, False])
@pytest.mark.parametrize("path", [B.FNG_PATH_FULLN, B.FNG_PATH_SPLITN, B.FNG_PATH_TWOPASS])
def test_postnorm_paths_ragged(ln, path):
    N = 136 if path == B.FNG_PATH_FULLN else 1544
    M, K = 700, 520
    spec, d = inputs.make_inputs("postnorm_rms_largen", M=M, K=K, N=N, seed=2024)
    log(f"postnorm ln={ln} path={path} M={M} K={K} N={N}")
    Y, mu, r, _ = run_postnorm(d, 1e-5, M, N, K, ln, path)
    ref, mref, rref = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), 1e-5, "ln" if ln else "rms")
    assert_parity(host(Y), ref, f"post-{'LN' if ln else 'RMS'} path {path}")
    assert_close_stats(r.cpu().numpy(), rref, "rstd")
    if ln:
        assert np.max(np.abs(mu.cpu().numpy() - mref)) < 2e-4


SMALL_KN = [(1000, 72, 136), (333, 200, 40), (8200, 256, 256), (64, 8, 8), (97, 256, 248)]


@pytest.mark.parametrize("ln", [True, False], ids=["ln", "rms"])
@pytest.mark.parametrize("M,K,N", SMALL_KN, ids=[f"{m}x{k}x{n}" for m, k, n in SMALL_KN])
def test_postnorm_fulln_small(ln, M, K, N):
    """Full-N with all of W resident in LDS (K, N <= 256, eight waves of 32
    columns): ragged M, K and N (zero-filled copies, partial column blocks,
    waves with no valid column), every element and the statistics outputs."""
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=M, K=K, N=N, seed=M + K + N)
    log(f"postnorm full-N small ln={ln} M={M} K={K} N={N}")
    Y, mu, r, _ = run_postnorm(d, spec["eps"], M, N, K, ln, B.FNG_PATH_FULLN)
    ref, mref, rref = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), spec["eps"], "ln" if ln else "rms")
    assert_parity(host(Y), ref, f"full-N small {M}x{K}x{N} ln={ln}")
    assert_close_stats(r.cpu().numpy(), rref, "rstd")
    if ln:
        assert np.max(np.abs(mu.cpu().numpy() - mref)) < 2e-4


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_postnorm_affine_fulln_small(kind):
    """The affine (gain, with and without the bias) in the resident-W kernel."""
    M, K, N = 1000, 136, 200
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=M, K=K, N=N, seed=63)
    rng = np.random.Generator(np.random.PCG64(64))
    g = inputs.f32_to_bf16_bits(1.0 + 0.3 * rng.standard_normal(N).astype(np.float32))
    b = inputs.f32_to_bf16_bits(0.5 * rng.standard_normal(N).astype(np.float32))
    X, W, G, Bb = dev(d["X"]), dev(d["W"]), dev(g), dev(b)
    Y = empty_bf16(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    for beta in (Bb, None):
        log(f"post-{kind} affine full-N small {M}x{K}x{N} beta={beta is not None}")
        B.fng_gemm_postnorm_affine(X, W, Y, spec["eps"], G, beta, ln=(kind == "ln"), workspace=None,
                                   path=B.FNG_PATH_FULLN, rstd_out=r)
        torch.cuda.synchronize()
        ref, _, rr = oracle.gemm_postnorm_affine(f64(d["X"]), f64(d["W"]), spec["eps"], kind, f64(g),
                                                 f64(b) if beta is not None else None)
        assert_parity_floor(host(Y), ref, f"post-{kind} affine full-N small beta={beta is not None}")
        assert_close_stats(r.cpu().numpy(), rr, "affine rstd")


@pytest.mark.parametrize("ln", [True, False])
@pytest.mark.parametrize("N", [264, 392, 512])
def test_postnorm_fulln_wide(ln, N):
    """Full-N path with one workgroup across 256 < N <= 512 (64 x 512 tiles)."""
    M, K = 700, 520
    assert N <= B.fng_fulln_max_n()
    spec, d = inputs.make_inputs("postnorm_rms_largen", M=M, K=K, N=N, seed=4242)
    log(f"postnorm full-N wide ln={ln} M={M} K={K} N={N}")
    Y, mu, r, _ = run_postnorm(d, 1e-5, M, N, K, ln, B.FNG_PATH_FULLN)
    ref, mref, rref = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), 1e-5, "ln" if ln else "rms")
    assert_parity(host(Y), ref, f"post-{'LN' if ln else 'RMS'} full-N N={N}")
    assert_close_stats(r.cpu().numpy(), rref, "rstd")
    if ln:
        assert np.max(np.abs(mu.cpu().numpy() - mref)) < 2e-4


# the pages' ads-shape sweep (M = 256k rows, K and N from 64 to 2048), here at
# 2048 rows so the oracle runs in seconds; the path is chosen automatically
ADS_KN = [(64, 64), (128, 128), (2048, 64), (64, 512), (512, 512), (2048, 512), (256, 1024), (512, 2048),
          (2048, 2048)]


@pytest.mark.parametrize("K,N", ADS_KN, ids=[f"K{k}_N{n}" for k, n in ADS_KN])
def test_postnorm_ads_shapes(K, N):
    M = 2048
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=M, K=K, N=N, seed=K * 7 + N)
    log(f"ads shape post-LN M={M} K={K} N={N}")
    Y, mu, r, _ = run_postnorm(d, 1e-5, M, N, K, True, B.FNG_PATH_AUTO)
    ref, mref, rref = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), 1e-5, "ln")
    assert_parity(host(Y), ref, f"ads post-LN K={K} N={N}")
    assert_close_stats(r.cpu().numpy(), rref, "rstd")
    assert np.max(np.abs(mu.cpu().numpy() - mref)) < 2e-4


@pytest.mark.parametrize("ln", [True, False])
@pytest.mark.parametrize("N", [40, 64, 104, 200, 264, 512])
def test_postnorm_fulln_tall_tiles(ln, N):
    """Full-N with 256-row tiles (used from 65536 rows on; 128 x 512 tiles for
    N above 256), ragged M, K and N; sampled rows against the oracle plus the
    row property on every row."""
    M, K = 65536 + 72, 136
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=M, K=K, N=N, seed=N + 5)
    log(f"postnorm full-N tall ln={ln} M={M} K={K} N={N}")
    Y, mu, r, _ = run_postnorm(d, 1e-5, M, N, K, ln, B.FNG_PATH_FULLN)
    rng = np.random.default_rng(N)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 73, M - 1], rng.choice(M, 48, replace=False)]))
    ref, mref, rref = oracle.gemm_postnorm(f64(d["X"][rows]), f64(d["W"]), 1e-5, "ln" if ln else "rms")
    assert_parity(host(Y[torch.as_tensor(rows, device="cuda")]), ref, f"full-N tall N={N}")
    assert_close_stats(r.cpu().numpy()[rows], rref, "rstd sampled")
    y = Y.float()
    if ln:
        assert np.max(np.abs(mu.cpu().numpy()[rows] - mref)) < 2e-4
        # zero mean, unit variance per row (up to eps and bf16 rounding)
        assert torch.max(torch.abs(y.mean(dim=1))).item() < 2e-2
        assert torch.max(torch.abs(y.var(dim=1, unbiased=False) - 1.0)).item() < 2e-2
    else:
        assert torch.max(torch.abs(torch.sqrt((y * y).mean(dim=1)) - 1.0)).item() < 1e-2


def test_postnorm_ads_full_rows_sampled():
    """One ads shape at its full 256k rows, sampled rows against the oracle."""
    M, K, N = 262144, 512, 512
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=M, K=K, N=N, seed=262)
    log(f"ads shape full rows post-LN M={M} K={K} N={N}")
    Y, mu, r, _ = run_postnorm(d, 1e-5, M, N, K, True, B.FNG_PATH_AUTO)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 63, 64, M - 1], rng.choice(M, 64, replace=False)]))
    ref, mref, rref = oracle.gemm_postnorm(f64(d["X"][rows]), f64(d["W"]), 1e-5, "ln")
    assert_parity(host(Y[torch.as_tensor(rows, device="cuda")]), ref, "ads full rows sampled")
    assert_close_stats(r.cpu().numpy()[rows], rref, "rstd sampled")
    assert np.max(np.abs(mu.cpu().numpy()[rows] - mref)) < 2e-4


@pytest.mark.parametrize("ln", [True, False])
def test_postnorm_three_paths_agree_at_n256(ln):
    M, K, N = 600, 256, 256
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=M, K=K, N=N, seed=77)
    ref, _, _ = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), 1e-5, "ln" if ln else "rms")
    outs = []
    for path in (B.FNG_PATH_FULLN, B.FNG_PATH_SPLITN, B.FNG_PATH_TWOPASS):
        Y, _, _, _ = run_postnorm(d, 1e-5, M, N, K, ln, path)
        y = host(Y)
        assert_parity(y, ref, f"N=256 path {path}")
        outs.append(y)
    # fused paths see the same fp32 accumulators; two-pass re-rounds once more
    assert np.max(np.abs(outs[0] - outs[1])) <= 2 * 2.0 ** -7 * np.max(np.abs(ref))


@pytest.mark.parametrize("ln", [True, False], ids=["ln", "rms"])
def test_postnorm_splitn_placement_shared_row_blocks(ln):
    """Split-N on 2048 x 4096 outputs: 8 row blocks x 16 column tiles = 128
    tiles in one round, placed as rectangles of 2 row blocks x 8 column tiles
    per XCD, two XCDs sharing each row block (their partials merged across
    XCDs); ragged K; every row against the oracle."""
    M, K, N = 2048, 264, 4096
    spec, d = inputs.make_inputs("postnorm_rms_largen", M=M, K=K, N=N, seed=77)
    eps = 1e-5 if ln else 1e-6
    log(f"split-N placement ln={ln} M={M} K={K} N={N}")
    Y, mu, r, _ = run_postnorm(d, eps, M, N, K, ln, B.FNG_PATH_SPLITN)
    ref, mref, rref = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), eps, "ln" if ln else "rms")
    assert_parity(host(Y), ref, f"split-N placement ln={ln}")
    assert_close_stats(r.cpu().numpy(), rref, "split-N placement rstd")
    if ln:
        assert np.max(np.abs(mu.cpu().numpy() - mref)) < 2e-4


def test_postnorm_ln_splitn_shifted_mean():
    """Rows whose mean is large against their spread (the merge of per-slice
    (count, mean, M2) must not cancel)."""
    M, K, N = 520, 512, 2048
    spec, d = inputs.make_inputs("postnorm_rms_largen", M=M, K=K, N=N, seed=99)
    w = inputs.bf16_bits_to_f32(d["W"]) + np.float32(0.25)
    d = dict(d, W=inputs.f32_to_bf16_bits(w))
    for path in (B.FNG_PATH_SPLITN, B.FNG_PATH_TWOPASS):
        Y, mu, r, _ = run_postnorm(d, 1e-5, M, N, K, True, path)
        ref, mref, rref = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), 1e-5, "ln")
        log(f"shifted mean: |mean|/std ~ {np.mean(np.abs(mref) * rref):.1f}")
        assert_parity(host(Y), ref, f"shifted-mean LN path {path}")


def test_postnorm_rms_largen_full_size_sampled():
    spec, d = inputs.make_inputs("postnorm_rms_largen")
    M, K, N = spec["M"], spec["K"], spec["N"]
    log(f"post-RMS split-N full size {M}x{K}x{N}")
    Y, _, r, ws = run_postnorm(d, spec["eps"], M, N, K, False, B.FNG_PATH_AUTO)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 60, replace=False)]))
    ref, _, rref = oracle.gemm_postnorm(f64(d["X"][rows]), f64(d["W"]), spec["eps"], "rms")
    assert_parity(host(Y[torch.as_tensor(rows, device="cuda")]), ref, "post-RMS full size sampled")
    assert_close_stats(r.cpu().numpy()[rows], rref, "post-RMS rstd sampled")
    # every output row has unit RMS up to eps and bf16 rounding (property at any size)
    y = Y.float()
    rms = torch.sqrt(torch.mean(y * y, dim=1)).cpu().numpy()
    assert np.max(np.abs(rms - 1.0)) < 5e-3


def test_splitn_workspace_reuse_and_determinism():
    ws = None
    shapes = [(1100, 256, 4096), (300, 128, 1024), (1100, 256, 4096)]
    first = None
    for call, (M, K, N) in enumerate(shapes, start=1):
        spec, d = inputs.make_inputs("postnorm_rms_largen", M=M, K=K, N=N, seed=5)
        need = B.fng_gemm_postnorm_workspace_bytes(M, N, K, B.FNG_PATH_SPLITN)
        if ws is None:
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        X, W = dev(d["X"]), dev(d["W"])
        Y = empty_bf16(M, N)
        B.fng_gemm_postnorm_rms(X, W, Y, 1e-6, workspace=ws, path=B.FNG_PATH_SPLITN)
        torch.cuda.synchronize()
        assert B.fng_get_kernel_status(ws) == B.FNG_OK
        ref, _, _ = oracle.gemm_postnorm(f64(d["X"]), f64(d["W"]), 1e-6, "rms")
        assert_parity(host(Y), ref, f"split-N reuse {M}x{K}x{N}")
        if first is None:
            first = Y.clone()
        elif (M, K, N) == shapes[0]:
            assert torch.equal(first.view(torch.int16), Y.view(torch.int16)), "not bitwise reproducible"
        # after every call: timeout flag 0, the epoch word counts the calls on
        # this workspace, the finished-row-block and per-row-block reader
        # counters are back to zero
        head = ws[:256 + 2 * 256].view(torch.int32).cpu()
        assert int(head[0]) == 0 and int(head[1]) == call, head[:4]
        head[1] = 0
        assert int(head.abs().sum()) == 0


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def run_attn(d, norm, eps_ln=1e-5, eps_rms=1e-6, scale=0.0, stats=False):
    Q, K, V = dev(d["Q"]), dev(d["K"]), dev(d["V"])
    Bsz, Sq, H, D = Q.shape
    O = empty_bf16(*Q.shape)
    st = None
    if norm:
        if stats:
            st = [torch.full((Bsz, Sq, H), float("nan"), dtype=torch.float32, device="cuda")
                  for _ in range(3)]
            B.fng_norm_attention(Q, K, V, O, eps_ln, eps_rms, scale, *st)
        else:
            B.fng_norm_attention(Q, K, V, O, eps_ln, eps_rms, scale)
    else:
        B.fng_attention(Q, K, V, O, scale)
    torch.cuda.synchronize()
    return O, st


@pytest.mark.parametrize("shape", [(2, 300, 200, 3), (1, 1, 1000, 2), (1, 130, 1, 1), (1, 64, 64, 4)],
                         ids=["ragged", "one_query", "one_key", "single_tile"])
def test_norm_attention_reduced(shape):
    Bsz, Sq, Skv, H = shape
    spec, d = inputs.make_inputs("norm_attention", B=Bsz, Sq=Sq, Skv=Skv, H=H)
    log(f"norm attention B={Bsz} Sq={Sq} Skv={Skv} H={H}")
    O, st = run_attn(d, True, spec["eps_ln"], spec["eps_rms"], stats=True)
    ref, mu, r1, r2 = oracle.norm_attention(f64(d["Q"]), f64(d["K"]), f64(d["V"]), spec["eps_ln"],
                                            spec["eps_rms"], 1.0 / math.sqrt(128))
    assert_parity(host(O), ref, f"norm attention {shape}")
    assert np.max(np.abs(st[0].cpu().numpy() - mu)) < 1e-4
    assert_close_stats(st[1].cpu().numpy(), r1, "ln rstd")
    assert_close_stats(st[2].cpu().numpy(), r2, "rms rstd", rtol=3e-3)


@pytest.mark.parametrize("shape", [(2, 300, 200, 3), (1, 256, 130, 2)])
def test_attention_baseline_reduced(shape):
    Bsz, Sq, Skv, H = shape
    spec, d = inputs.make_inputs("norm_attention", B=Bsz, Sq=Sq, Skv=Skv, H=H, seed=31)
    O, _ = run_attn(d, False, scale=0.1)
    ref = oracle.attention(f64(d["Q"]), f64(d["K"]), f64(d["V"]), 0.1)
    # plain attention output is not normalized: compare at the output's own scale
    assert_parity(host(O), ref, f"attention {shape}", mae=2e-3 * np.mean(np.abs(ref)) / 0.8)


def test_norm_attention_full_size_sampled():
    spec, d = inputs.make_inputs("norm_attention")
    log("norm attention full size 32x1024x4x128")
    O, _ = run_attn(d, True, spec["eps_ln"], spec["eps_rms"])
    y = host(O)
    for (b, h) in [(0, 0), (17, 2), (31, 3)]:
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        ref, _, _, _ = oracle.norm_attention(f64(d["Q"][sl]), f64(d["K"][sl]), f64(d["V"][sl]),
                                             spec["eps_ln"], spec["eps_rms"], 1.0 / math.sqrt(128))
        assert_parity(y[sl], ref, f"norm attention full size (b={b}, h={h})")
    # every output row has unit RMS over head_dim (up to eps and bf16 rounding)
    rms = torch.sqrt(torch.mean(O.float() ** 2, dim=-1)).cpu().numpy()
    assert np.max(np.abs(rms - 1.0)) < 5e-3


# ---------------------------------------------------------------------------
# unfused baselines
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N", [128, 256, 520, 1000, 4096, 8192, 12000])
@pytest.mark.parametrize("kind", ["rms", "rms_gamma", "ln"])
def test_row_norms(N, kind):
    M = 37
    rng = np.random.default_rng(N)
    x = (rng.standard_normal((M, N)) * rng.lognormal(0, 1, (M, 1)) + (0.5 if kind == "ln" else 0))
    xb = inputs.f32_to_bf16_bits(x.astype(np.float32))
    gb = inputs.f32_to_bf16_bits((1 + 0.3 * rng.standard_normal(N)).astype(np.float32))
    X = dev(xb)
    Y = empty_bf16(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    mu = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    if kind == "ln":
        B.fng_layernorm(X, Y, 1e-5, mean_out=mu, rstd_out=r)
        ref, mref, rref = oracle.layernorm_rows(f64(xb), 1e-5)
    else:
        g = dev(gb) if kind == "rms_gamma" else None
        B.fng_rmsnorm(X, Y, 1e-6, gamma=g, rstd_out=r)
        ref, rref = oracle.rmsnorm_rows(f64(xb), 1e-6, f64(gb) if g is not None else None)
    torch.cuda.synchronize()
    assert_parity(host(Y), ref, f"{kind} N={N}")
    assert_close_stats(r.cpu().numpy(), rref, f"{kind} rstd")
    if kind == "ln":
        assert np.max(np.abs(mu.cpu().numpy() - mref)) < 1e-4


def test_row_norm_in_place():
    spec, d = inputs.make_inputs("prenorm_rms_small", M=64, K=4096, N=8)
    X = dev(d["X"])
    ref, _ = oracle.rmsnorm_rows(f64(d["X"]), 1e-6)
    B.fng_rmsnorm(X, X, 1e-6)
    torch.cuda.synchronize()
    assert_parity(host(X), ref, "in-place rmsnorm")


@pytest.mark.parametrize("shape", [(256, 128, 128), (1100, 520, 4000), (65600, 136, 40), (65600, 72, 120)])
def test_gemm_baseline(shape):
    M, K, N = shape
    spec, d = inputs.make_inputs("prenorm_rms_small", M=M, K=K, N=N, seed=3)
    X, W = dev(d["X"]), dev(d["W"])
    Y = empty_bf16(M, N)
    B.fng_gemm(X, W, Y)
    torch.cuda.synchronize()
    ref = oracle.gemm(f64(d["X"]), f64(d["W"]))
    assert_parity(host(Y), ref, f"gemm {shape}")


def test_fused_matches_unfused_prenorm():
    """Keep fused and split versions side by side and cross-check them."""
    M, K, N = 1100, 520, 4000
    spec, d = inputs.make_inputs("prenorm_rms_mlp", M=M, K=K, N=N)
    X, W = dev(d["X"]), dev(d["W"])
    Yf = empty_bf16(M, N)
    B.fng_prenorm_rms_gemm(X, W, Yf, spec["eps"])
    Xn = empty_bf16(M, K)
    B.fng_rmsnorm(X, Xn, spec["eps"])
    Yu = empty_bf16(M, N)
    B.fng_gemm(Xn, W, Yu)
    torch.cuda.synchronize()
    ref, _ = oracle.prenorm_rms_gemm(f64(d["X"]), f64(d["W"]), spec["eps"])
    assert_parity(host(Yf), ref, "fused pre-RMS")
    assert_parity(host(Yu), ref, "unfused rmsnorm + gemm")


def test_empty_calls_are_noops():
    X = empty_bf16(0, 64)
    W = empty_bf16(64, 64)
    Y = empty_bf16(0, 64)
    B.fng_prenorm_rms_gemm(X, W, Y, 1e-6)
    B.fng_gemm(X, W, Y)
    B.fng_gemm_postnorm_rms(X, W, Y, 1e-6)
    Q = empty_bf16(0, 8, 2, 128)
    B.fng_norm_attention(Q, empty_bf16(0, 8, 2, 128), empty_bf16(0, 8, 2, 128), Q, 1e-5, 1e-6)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# post-norm with its affine (gain and bias per column), every path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("path", [B.FNG_PATH_FULLN, B.FNG_PATH_SPLITN, B.FNG_PATH_TWOPASS],
                         ids=["fulln", "splitn", "twopass"])
@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_postnorm_affine(kind, path):
    M, K, N = 600, 264, 256 if path == B.FNG_PATH_FULLN else 1320
    if path == B.FNG_PATH_FULLN and kind == "rms":
        M, N = 32768 + 40, 392  # the 128 x 512 full-N tile (from 32768 rows on), ragged N
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=M, K=K, N=N, seed=61)
    rng = np.random.Generator(np.random.PCG64(62))
    g = inputs.f32_to_bf16_bits(1.0 + 0.3 * rng.standard_normal(N).astype(np.float32))
    b = inputs.f32_to_bf16_bits(0.5 * rng.standard_normal(N).astype(np.float32))
    X, W, G, Bb = dev(d["X"]), dev(d["W"]), dev(g), dev(b)
    Y = empty_bf16(M, N)
    ws = None
    if path != B.FNG_PATH_FULLN:
        ws = torch.zeros(B.fng_gemm_postnorm_workspace_bytes(M, N, K, path), dtype=torch.uint8, device="cuda")
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    log(f"post-{kind} affine {M}x{K}x{N} path={path}")
    for beta in (Bb, None):
        B.fng_gemm_postnorm_affine(X, W, Y, spec["eps"], G, beta, ln=(kind == "ln"), workspace=ws, path=path,
                                   rstd_out=r)
        torch.cuda.synchronize()
        ref, _, rr = oracle.gemm_postnorm_affine(f64(d["X"]), f64(d["W"]), spec["eps"], kind, f64(g),
                                                 f64(b) if beta is not None else None)
        assert_parity_floor(host(Y), ref, f"post-{kind} affine path {path} beta={beta is not None}")
        assert_close_stats(r.cpu().numpy(), rr, "affine rstd")
