"""GPU parity of the regrouped norm backward (section 3, "What about
backward?"): the norm backward as the epilogue of the GEMM that produces its
upstream gradient (fng_gemm_postnorm_ln_bwd / _rms_bwd, full-N and split-N),
the lazy pre-RMSNorm input gradient with xhat rebuilt from X and rstd
(fng_prenorm_rms_bwd_dx), and the unfused row kernels (fng_layernorm_bwd,
fng_rmsnorm_bwd), all through the C ABI against the fp64 oracle.

Tolerance (gpu_util.assert_parity_floor): normwise max relative error <= 1e-2,
and a mean absolute error within 1e-3 of the bf16 rounding floor of the exact
gradient (the gradients are scaled by the forward rstd, log-normal here, so a
fixed 2e-3 would be loose on some rows and tight on others); the bound is never
looser than 2e-3 times max(1, mean |ref| / 0.8)."""

import numpy as np
import pytest
import torch

import oracle
from attention_fng_prenorm_amd import binding as B
from attention_fng_prenorm_amd import inputs
from gpu_util import assert_parity, assert_parity_floor, dev, empty_bf16, host, log

pytestmark = pytest.mark.gpu


def f64(bits):
    return oracle.bf16_to_f64(bits)


def scaled_parity(y, ref, what):
    return assert_parity_floor(y, ref, what)


def workspace(M, N, K, path):
    nb = B.fng_gemm_postnorm_workspace_bytes(M, N, K, B.FNG_PATH_SPLITN)
    return torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if path != B.FNG_PATH_FULLN else None


def run_postnorm_bwd(d, kind, path):
    G, Wt, H = dev(d["G"]), dev(d["Wt"]), dev(d["H"])
    r = torch.from_numpy(d["rstd"]).to("cuda")
    M, K = G.shape
    N = Wt.shape[1]
    dZ = empty_bf16(M, N)
    ws = workspace(M, N, K, path)
    fn = B.fng_gemm_postnorm_ln_bwd if kind == "ln" else B.fng_gemm_postnorm_rms_bwd
    fn(G, Wt, H, r, dZ, workspace=ws, path=path)
    torch.cuda.synchronize()
    if ws is not None:
        assert B.fng_get_kernel_status(ws) == B.FNG_OK
    return dZ


@pytest.mark.parametrize("path", [B.FNG_PATH_FULLN, B.FNG_PATH_SPLITN], ids=["fulln", "splitn"])
@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("shape", [(300, 136, 200), (520, 264, 512), (70, 72, 64)],
                         ids=["ragged", "n512", "small"])
def test_postnorm_bwd_reduced(shape, kind, path):
    M, K, N = shape
    spec, d = inputs.make_inputs("postnorm_ln_smalln_bwd", M=M, K=K, N=N, seed=41)
    log(f"postnorm bwd {kind} {shape} path={path}")
    dZ = run_postnorm_bwd(d, kind, path)
    ref = oracle.gemm_postnorm_backward(f64(d["G"]), f64(d["Wt"]), f64(d["H"]), d["rstd"], kind)
    scaled_parity(host(dZ), ref, f"{kind} bwd {shape} path {path}")


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_postnorm_bwd_splitn_wide(kind):
    # N over several 256-column tiles with a ragged last one
    M, K, N = 600, 200, 1320
    spec, d = inputs.make_inputs("postnorm_rms_largen_bwd", M=M, K=K, N=N, seed=42)
    log(f"postnorm bwd split-N {kind} {M}x{K}x{N}")
    dZ = run_postnorm_bwd(d, kind, B.FNG_PATH_AUTO)
    ref = oracle.gemm_postnorm_backward(f64(d["G"]), f64(d["Wt"]), f64(d["H"]), d["rstd"], kind)
    scaled_parity(host(dZ), ref, f"{kind} bwd split-N wide")
    # the gradient of a LayerNorm input sums to zero over each row when Y is
    # an exact LayerNorm output; here Y is arbitrary, so check the row sums
    # against the oracle's instead
    if kind == "ln":
        got = host(dZ).sum(axis=1)
        assert np.max(np.abs(got - ref.sum(axis=1))) < 0.05 * N ** 0.5


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_postnorm_bwd_splitn_placement(kind):
    # 2048 x 4096: one round of 8 row blocks x 16 column tiles placed as
    # 2 x 8 rectangles per XCD, two XCDs sharing each row block; all rows
    M, K, N = 2048, 200, 4096
    spec, d = inputs.make_inputs("postnorm_rms_largen_bwd", M=M, K=K, N=N, seed=46)
    log(f"postnorm bwd split-N placement {kind} {M}x{K}x{N}")
    dZ = run_postnorm_bwd(d, kind, B.FNG_PATH_SPLITN)
    ref = oracle.gemm_postnorm_backward(f64(d["G"]), f64(d["Wt"]), f64(d["H"]), d["rstd"], kind)
    scaled_parity(host(dZ), ref, f"{kind} bwd split-N placement")


def test_postnorm_bwd_tall_narrow():
    # tall tiles for >= 65536 rows (N <= 64, 128, 256)
    for N in (40, 104, 200):
        M, K = 65608, 72
        spec, d = inputs.make_inputs("postnorm_ln_smalln_bwd", M=M, K=K, N=N, seed=43)
        log(f"postnorm bwd tall M={M} N={N}")
        dZ = run_postnorm_bwd(d, "ln", B.FNG_PATH_AUTO)
        rows = np.unique(np.concatenate([[0, 255, 256, 65535, 65536, M - 1],
                                         np.random.default_rng(N).choice(M, 60, replace=False)]))
        ref = oracle.gemm_postnorm_backward(f64(d["G"][rows]), f64(d["Wt"]), f64(d["H"][rows]),
                                            d["rstd"][rows], "ln")
        scaled_parity(host(dZ)[rows], ref, f"tall bwd N={N}")


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("N", [328, 512])
@pytest.mark.parametrize("path", [B.FNG_PATH_FULLN, B.FNG_PATH_SPLITN], ids=["fulln", "splitn"])
def test_postnorm_bwd_tall_wide(path, N, kind):
    # whole rows of up to 512 columns per workgroup for >= 65536 rows (the
    # automatic choice there), and split-N on the same rows (a ragged
    # last row block: 65608 = 512 * 128 + 72; a ragged column tile at N = 328)
    M, K = 65608, 72
    spec, d = inputs.make_inputs("postnorm_ln_smalln_bwd", M=M, K=K, N=N, seed=44 + N)
    log(f"postnorm bwd tall {kind} M={M} N={N} path={path}")
    dZ = run_postnorm_bwd(d, kind, path)
    rows = np.unique(np.concatenate([[0, 127, 128, 65535, 65536, M - 73, M - 1],
                                     np.random.default_rng(N).choice(M, 60, replace=False)]))
    ref = oracle.gemm_postnorm_backward(f64(d["G"][rows]), f64(d["Wt"]), f64(d["H"][rows]),
                                        d["rstd"][rows], kind)
    scaled_parity(host(dZ)[rows], ref, f"tall {kind} bwd N={N}")


# the ads shapes of the multi-CTA backward (section 3, "What about backward?"),
# at 2048 rows: the automatic path (full-N up to its width, split-N above)
ADS_BWD_KN = [(64, 64), (2048, 128), (256, 256), (64, 512), (512, 512), (1024, 1024), (256, 2048), (2048, 2048)]


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("K,N", ADS_BWD_KN, ids=[f"K{k}_N{n}" for k, n in ADS_BWD_KN])
def test_postnorm_bwd_ads_shapes(K, N, kind):
    M = 2048
    spec, d = inputs.make_inputs("postnorm_ln_smalln_bwd", M=M, K=K, N=N, seed=K * 11 + N)
    log(f"ads shape post-norm bwd {kind} M={M} K={K} N={N}")
    dZ = run_postnorm_bwd(d, kind, B.FNG_PATH_AUTO)
    ref = oracle.gemm_postnorm_backward(f64(d["G"]), f64(d["Wt"]), f64(d["H"]), d["rstd"], kind)
    scaled_parity(host(dZ), ref, f"ads {kind} bwd K={K} N={N}")
    if 256 < N <= B.fng_fulln_max_n():
        # with a workspace the automatic path took split-N here; without one it
        # keeps the forward's choice (full-N)
        G, Wt, H = dev(d["G"]), dev(d["Wt"]), dev(d["H"])
        r = torch.from_numpy(d["rstd"]).to("cuda")
        dZ2 = empty_bf16(M, N)
        fn = B.fng_gemm_postnorm_ln_bwd if kind == "ln" else B.fng_gemm_postnorm_rms_bwd
        fn(G, Wt, H, r, dZ2, workspace=None, path=B.FNG_PATH_AUTO)
        torch.cuda.synchronize()
        scaled_parity(host(dZ2), ref, f"ads {kind} bwd K={K} N={N} without a workspace")


@pytest.mark.parametrize("path", [B.FNG_PATH_FULLN, B.FNG_PATH_SPLITN], ids=["fulln", "splitn"])
@pytest.mark.parametrize("shape", [(300, 520, 256), (260, 136, 1000)], ids=["k256", "k1000"])
def test_prenorm_bwd_dx_reduced(shape, path):
    M, N, K = shape   # forward sizes: X [M,K], W [K,N]
    if path == B.FNG_PATH_FULLN and K > B.fng_fulln_max_n():
        pytest.skip("full-N covers K <= fng_fulln_max_n()")
    spec, d = inputs.make_inputs("prenorm_rms_mlp_bwd_dx", M=M, K=N, N=K, seed=44)
    dY, Wt, X = dev(d["G"]), dev(d["Wt"]), dev(d["H"])
    r = torch.from_numpy(d["rstd"]).to("cuda")
    dX = empty_bf16(M, K)
    ws = workspace(M, K, N, path)
    log(f"prenorm bwd dx {shape} path={path}")
    B.fng_prenorm_rms_bwd_dx(dY, Wt, X, r, dX, workspace=ws, path=path)
    torch.cuda.synchronize()
    ref = oracle.prenorm_rms_backward_dx(f64(d["G"]), f64(d["Wt"]), f64(d["H"]), d["rstd"])
    scaled_parity(host(dX), ref, f"prenorm dx {shape} path {path}")


@pytest.mark.parametrize("kind", ["ln", "rms", "rms_input"])
@pytest.mark.parametrize("N", [200, 1000, 9000])
def test_row_norm_bwd(kind, N):
    M = 130
    spec, d = inputs.make_inputs("postnorm_ln_smalln_bwd", M=M, K=8, N=N, seed=45,
                                 h_dist="lognormal_rows" if kind == "rms_input" else "normal")
    Gm = dev(d["H"]).flip(0).contiguous()   # any [M, N] bf16 gradient
    H = dev(d["H"])
    r = torch.from_numpy(d["rstd"]).to("cuda")
    dZ = empty_bf16(M, N)
    log(f"row bwd {kind} N={N}")
    if kind == "ln":
        B.fng_layernorm_bwd(Gm, H, r, dZ)
    else:
        B.fng_rmsnorm_bwd(Gm, H, r, dZ, h_is_input=(kind == "rms_input"))
    torch.cuda.synchronize()
    g = f64(d["H"])[::-1]
    xhat = f64(d["H"]) * (d["rstd"][:, None] if kind == "rms_input" else 1.0)
    fn = oracle.layernorm_backward_rows if kind == "ln" else oracle.rmsnorm_backward_rows
    scaled_parity(host(dZ), fn(g, xhat, d["rstd"]), f"row bwd {kind} N={N}")


def test_fused_matches_unfused_bwd():
    M, K, N = 520, 264, 1040
    spec, d = inputs.make_inputs("postnorm_rms_largen_bwd", M=M, K=K, N=N, seed=46)
    G, Wt, H = dev(d["G"]), dev(d["Wt"]), dev(d["H"])
    r = torch.from_numpy(d["rstd"]).to("cuda")
    fused = run_postnorm_bwd(d, "ln", B.FNG_PATH_AUTO)
    g = empty_bf16(M, N)
    B.fng_gemm(G, Wt, g)
    unfused = empty_bf16(M, N)
    B.fng_layernorm_bwd(g, H, r, unfused)
    torch.cuda.synchronize()
    ref = oracle.gemm_postnorm_backward(f64(d["G"]), f64(d["Wt"]), f64(d["H"]), d["rstd"], "ln")
    ef = scaled_parity(host(fused), ref, "fused ln bwd")
    # the unfused chain rounds the GEMM output to bf16 before the norm backward
    # (a baseline, not the fused path: its gate is twice the scaled MAE bound)
    eu = assert_parity(host(unfused), ref, "unfused gemm + ln bwd",
                       mae=2 * 2e-3 * max(1.0, float(np.mean(np.abs(ref))) / 0.8))
    assert ef["mae"] <= eu["mae"] * 1.05


def test_bwd_deterministic_and_workspace_reuse():
    M, K, N = 520, 264, 1040
    spec, d = inputs.make_inputs("postnorm_rms_largen_bwd", M=M, K=K, N=N, seed=47)
    G, Wt, H = dev(d["G"]), dev(d["Wt"]), dev(d["H"])
    r = torch.from_numpy(d["rstd"]).to("cuda")
    ws = workspace(M, N, K, B.FNG_PATH_SPLITN)
    outs = []
    for _ in range(3):
        dZ = empty_bf16(M, N)
        B.fng_gemm_postnorm_rms_bwd(G, Wt, H, r, dZ, workspace=ws, path=B.FNG_PATH_SPLITN)
        outs.append(dZ)
    torch.cuda.synchronize()
    assert B.fng_get_kernel_status(ws) == B.FNG_OK
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))
    assert torch.equal(outs[0].view(torch.int16), outs[2].view(torch.int16))


def test_postnorm_bwd_full_size_sampled():
    spec, d = inputs.make_inputs("postnorm_rms_largen_bwd")
    M, K, N = spec["M"], spec["K"], spec["N"]
    log(f"postnorm rms bwd full size {M}x{K}x{N}")
    dZ = run_postnorm_bwd(d, "rms", B.FNG_PATH_AUTO)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(3).choice(M, 28, replace=False)]))
    ref = oracle.gemm_postnorm_backward(f64(d["G"][rows]), f64(d["Wt"]), f64(d["H"][rows]), d["rstd"][rows], "rms")
    scaled_parity(host(dZ)[rows], ref, "post-RMS bwd full size sampled rows")


def test_prenorm_bwd_dx_full_size_sampled():
    spec, d = inputs.make_inputs("prenorm_rms_mlp_bwd_dx")
    M, Kp, Np = spec["M"], spec["K"], spec["N"]   # product sizes: [M, Kp] @ [Kp, Np]
    dY, Wt, X = dev(d["G"]), dev(d["Wt"]), dev(d["H"])
    r = torch.from_numpy(d["rstd"]).to("cuda")
    dX = empty_bf16(M, Np)
    ws = workspace(M, Np, Kp, B.FNG_PATH_SPLITN)
    log(f"prenorm bwd dx full size dY[{M},{Kp}] Wt[{Kp},{Np}]")
    B.fng_prenorm_rms_bwd_dx(dY, Wt, X, r, dX, workspace=ws)
    torch.cuda.synchronize()
    assert B.fng_get_kernel_status(ws) == B.FNG_OK
    rows = np.array([0, 1, 255, 256, 2047, M - 1])
    ref = oracle.prenorm_rms_backward_dx(f64(d["G"][rows]), f64(d["Wt"]), f64(d["H"][rows]), d["rstd"][rows])
    scaled_parity(host(dX)[rows], ref, "prenorm dx full size sampled rows")
