"""GPU parity on the method's degenerate rows, every fused path, through the C
ABI against the fp64 oracle.

Rows of the normalized tensor are replaced (inputs.plant_rows) by
  zero     -> RMSNorm: rstd = 1/sqrt(eps) and an output of exactly 0;
              LayerNorm: the same (mean 0, variance 0)
  const    -> LayerNorm: the centred row is exactly 0, so the output is 0
              (post-norm, attention) and the softmax over the keys is uniform
  tiny     -> mean square (variance) about eps: eps is not negligible
  shifted  -> |mean| about 24 times the spread (LayerNorm's cancellation case)
  huge     -> entries about 2^12 (scale invariance of the norms)
spread over tile boundaries and ragged tails.  Each case checks the agreed
gate (normwise max relative error <= 1e-2, MAE <= 2e-3, or the bf16 floor
form for outputs that are not unit-scale), finiteness everywhere, the exact
zeros the definitions give, and the statistics outputs on the planted rows.
Towards Free Normalization: section 2 defines rstd with eps inside the root
(so a zero row keeps a finite rstd), section 1/3 the post-norms, section 4
the attention norms."""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_fng_prenorm_amd import binding as B
from attention_fng_prenorm_amd import inputs
from gpu_util import (assert_close_stats, assert_parity, assert_parity_floor, dev, empty_bf16, host,
                      log)

pytestmark = pytest.mark.gpu

f64 = oracle.bf16_to_f64
SCALE = 1.0 / math.sqrt(128)


def planted_rows(M, extra=()):
    """Row indices on and next to 256/128/64/32-row tile edges, the first and
    the last row."""
    rows = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257, M - 2, M - 1, *extra}
    return sorted(r for r in rows if 0 <= r < M)


def assert_planted_floor(y, ref, where, what):
    """The floor form of the gate on each kind of planted row on its own, the
    margin relative to the rows' own magnitude (the huge rows' outputs carry
    the raw query through the residual, about 2^12 in size)."""
    for kind, rows in where.items():
        if rows:
            scale = max(1.0, float(np.mean(np.abs(ref[rows]))) / 0.8)
            assert_parity_floor(y[rows], ref[rows], f"{what}: {kind} rows", margin=1e-3 * scale)


def assert_rows_zero(y, rows, what):
    bad = [r for r in rows if not np.all(y[r] == 0.0)]
    assert not bad, f"{what}: rows {bad[:5]} not exactly zero (max {np.max(np.abs(y[bad[0]]))})"


# ---------------------------------------------------------------------------
# lazy pre-RMSNorm GEMM (+ gamma), small and big tiles, and the lazy LayerNorm
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gamma", [False, True], ids=["plain", "gamma"])
@pytest.mark.parametrize("shape", [(256, 128, 128), (1100, 520, 4000)], ids=["small_tiles", "big_tiles"])
def test_prenorm_degenerate_rows(shape, gamma):
    M, K, N = shape
    spec, d = inputs.make_inputs("prenorm_rms_mlp_gamma" if gamma else "prenorm_rms_small", M=M, K=K, N=N,
                                 seed=501)
    eps = 1e-6
    rows = planted_rows(M, extra=(M // 2, M // 3))
    x, where = inputs.plant_rows(d["X"], rows, inputs.ROW_KINDS, seed=502, eps=eps)
    log(f"prenorm degenerate rows {shape} gamma={gamma}: {where}")
    X, W = dev(x), dev(d["W"])
    g = dev(d["gamma"]) if gamma else None
    Y = empty_bf16(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    B.fng_prenorm_rms_gemm(X, W, Y, eps, gamma=g, rstd_out=r)
    torch.cuda.synchronize()
    ref, rref = oracle.prenorm_rms_gemm(f64(x), f64(d["W"]), eps, f64(d["gamma"]) if gamma else None)
    y = host(Y)
    assert_parity(y, ref, f"prenorm degenerate {shape} gamma={gamma}")
    assert_parity(y[rows], ref[rows], "planted rows only")
    assert_rows_zero(y, where["zero"], "zero X rows")
    rr = r.cpu().numpy()
    assert np.all(np.isfinite(rr))
    assert_close_stats(rr, rref, "rstd (all rows)")
    assert np.allclose(rr[where["zero"]], 1.0 / math.sqrt(eps), rtol=1e-6)


def test_prenorm_ln_degenerate_rows():
    M, K, N = 1100, 520, 4000
    spec, d = inputs.make_inputs("prenorm_ln_mlp", M=M, K=K, N=N, seed=503)
    eps = spec["eps"]
    rows = planted_rows(M, extra=(600,))
    x, where = inputs.plant_rows(d["X"], rows, inputs.ROW_KINDS, seed=504, eps=eps)
    log(f"lazy LayerNorm degenerate rows: {where}")
    X, W = dev(x), dev(d["W"])
    Y = empty_bf16(M, N)
    ws = torch.empty(B.fng_prenorm_ln_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")
    mu = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    B.fng_prenorm_ln_gemm(X, W, Y, eps, ws, mean_out=mu, rstd_out=r)
    torch.cuda.synchronize()
    ref, mref, rref = oracle.prenorm_ln_gemm(f64(x), f64(d["W"]), eps)
    y = host(Y)
    assert_parity(y, ref, "lazy LayerNorm degenerate rows")
    assert_parity(y[rows], ref[rows], "planted rows only")
    assert_rows_zero(y, where["zero"], "zero X rows")
    assert np.max(np.abs(mu.cpu().numpy() - mref)) <= 1e-4 * max(1.0, np.max(np.abs(mref)))
    # rstd: exact to fp32 rounding where the variance is not dominated by
    # cancellation (the kernel's variance is sumsq/K - mean^2 of fp32 sums);
    # on constant rows the exact variance is 0 and rstd = 1/sqrt(eps)
    rr = r.cpu().numpy()
    ok = np.setdiff1d(np.arange(M), where["const"] + where["shifted"])
    assert_close_stats(rr[ok], rref[ok], "rstd (rows without cancellation)")
    assert np.all(np.isfinite(rr)) and np.all(rr[where["const"]] <= 1.0 / math.sqrt(eps) * (1 + 1e-6))


# ---------------------------------------------------------------------------
# GEMM + post-norm: full-N (32-row and 256-row tiles), split-N, two-pass
# ---------------------------------------------------------------------------

def postnorm_case(M, K, N, seed):
    """Seeded inputs whose product has planted zero, constant, tiny, shifted
    and huge rows: row 0 of W is all ones (bf16 exact), so an X row that is
    c at k = 0 and zero elsewhere gives the constant product row c; an X row
    scaled by s gives a product row scaled by s; a shifted product row comes
    from c at k = 0 plus a normal row."""
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=M, K=K, N=N, seed=seed)
    w = d["W"].copy()
    w[0, :] = inputs.f32_to_bf16_bits(np.ones(N, dtype=np.float32))
    rows = planted_rows(M, extra=(M // 2,))
    xb = d["X"].copy()
    where = {k: [] for k in ("zero", "const", "tiny", "shifted", "huge")}
    xf = inputs.bf16_bits_to_f32(xb)
    for i, r in enumerate(rows):
        kind = ("zero", "const", "tiny", "shifted", "huge")[i % 5]
        if kind == "zero":
            xf[r] = 0.0
        elif kind == "const":
            xf[r] = 0.0
            xf[r, 0] = 1.5 if i % 2 else -0.75
        elif kind == "tiny":
            xf[r] *= np.float32(3e-3)     # product variance about 1e-5 (the LN eps), mean square about 9e-6
        elif kind == "shifted":
            xf[r, 0] = np.float32(24.0)   # adds 24 to every column of a unit-variance row
        else:
            xf[r] *= np.float32(4096.0)
        where[kind].append(r)
    xb = inputs.f32_to_bf16_bits(xf)
    return spec, xb, w, rows, where


@pytest.mark.parametrize("ln", [True, False], ids=["ln", "rms"])
@pytest.mark.parametrize("case", ["fulln_c2", "fulln_tall", "fulln_512", "splitn", "twopass"])
def test_postnorm_degenerate_rows(case, ln):
    M, K, N, path = {
        "fulln_c2": (8192, 256, 256, B.FNG_PATH_FULLN),      # 32 x 256 tiles (the small-N workload)
        "fulln_tall": (65536 + 72, 136, 200, B.FNG_PATH_FULLN),  # 256-row tiles
        "fulln_512": (700, 264, 392, B.FNG_PATH_FULLN),     # 64 x 512 tiles
        "splitn": (700, 520, 1320, B.FNG_PATH_SPLITN),
        "twopass": (700, 520, 1320, B.FNG_PATH_TWOPASS),
    }[case]
    eps = 1e-5 if ln else 1e-6
    spec, xb, wb, rows, where = postnorm_case(M, K, N, seed=505 + N)
    log(f"post-{'LN' if ln else 'RMS'} degenerate rows {case} {M}x{K}x{N}: {where}")
    X, W = dev(xb), dev(wb)
    Y = empty_bf16(M, N)
    r = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    mu = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda") if ln else None
    nb = B.fng_gemm_postnorm_workspace_bytes(M, N, K, path)
    ws = torch.zeros(max(nb, 16), dtype=torch.uint8, device="cuda") if nb else None
    if ln:
        B.fng_gemm_postnorm_ln(X, W, Y, eps, workspace=ws, path=path, mean_out=mu, rstd_out=r)
    else:
        B.fng_gemm_postnorm_rms(X, W, Y, eps, workspace=ws, path=path, rstd_out=r)
    torch.cuda.synchronize()
    if ws is not None:
        assert B.fng_get_kernel_status(ws) == B.FNG_OK
    # the oracle on every row for the small shapes, else on the planted rows
    # plus a sample (the tall case has 65608 rows)
    sample = np.arange(M) if M <= 8192 else np.unique(np.concatenate(
        [rows, np.random.default_rng(N).choice(M, 64, replace=False)]))
    ref, mref, rref = oracle.gemm_postnorm(f64(xb[sample]), f64(wb), eps, "ln" if ln else "rms")
    y = host(Y[torch.as_tensor(sample, device="cuda")])
    assert_parity(y, ref, f"{case} {'LN' if ln else 'RMS'} degenerate")
    pos = {int(s): i for i, s in enumerate(sample)}
    pr = [pos[q] for q in rows]
    assert_parity(y[pr], ref[pr], "planted rows only")
    yall = Y.float()
    assert bool(torch.isfinite(yall).all()), "non-finite output"
    assert_rows_zero(y, [pos[q] for q in where["zero"]], "zero rows")
    if ln:
        # a constant product row is centred to exactly 0 (the mean of equal
        # fp32 accumulators is exact)
        assert_rows_zero(y, [pos[q] for q in where["const"]], "constant rows (LayerNorm)")
    rr = r.cpu().numpy()[sample]
    assert np.all(np.isfinite(rr))
    assert_close_stats(rr, rref, "rstd")
    assert np.allclose(r.cpu().numpy()[where["zero"]], 1.0 / math.sqrt(eps), rtol=1e-6)
    if ln:
        assert np.max(np.abs(mu.cpu().numpy()[sample] - mref)) <= 2e-4 * max(1.0, float(np.max(np.abs(mref))))


# ---------------------------------------------------------------------------
# norm-sandwiched attention (per head) and the full FlashNormAttention
# ---------------------------------------------------------------------------

def test_norm_attention_degenerate_rows():
    Bsz, Sq, Skv, H = 2, 300, 200, 3
    spec, d = inputs.make_inputs("norm_attention", B=Bsz, Sq=Sq, Skv=Skv, H=H, seed=511)
    # a row is one (b, s, h) query vector of 128 values
    q3 = d["Q"].reshape(Bsz * Sq * H, 128)
    rows = sorted({0, 1, 3 * 63, 3 * 64 + 1, 3 * 255 + 2, 3 * 256, 3 * 299 + 2, 3 * 300, 3 * 300 + 4,
                   3 * 599 + 1, 3 * 599 + 2, 3 * 450, 3 * 451 + 1})
    q3, where = inputs.plant_rows(q3, rows, inputs.ROW_KINDS, seed=512, eps=spec["eps_ln"])
    q = q3.reshape(d["Q"].shape)
    # and one batch whose keys are all zero: uniform weights for every query
    k = d["K"].copy()
    k[1, :, 2, :] = 0
    log(f"norm attention degenerate query rows {where}; keys of (b=1, h=2) zero")
    Q, K, V = dev(q), dev(k), dev(d["V"])
    O = empty_bf16(*Q.shape)
    st = [torch.full((Bsz, Sq, H), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    B.fng_norm_attention(Q, K, V, O, spec["eps_ln"], spec["eps_rms"], 0.0, *st)
    torch.cuda.synchronize()
    ref, mu, r1, r2 = oracle.norm_attention(f64(q), f64(k), f64(d["V"]), spec["eps_ln"], spec["eps_rms"], SCALE)
    y = host(O)
    assert_parity(y, ref, "norm attention degenerate rows")
    yr, rr = y.reshape(-1, 128), ref.reshape(-1, 128)
    assert_parity(yr[rows], rr[rows], "planted rows only")
    # a constant or zero query row normalizes to exactly 0: uniform weights,
    # out = rmsnorm(mean over keys of V)
    vbar = f64(d["V"]).mean(axis=1)                                     # [B, H, D]
    for rix in where["const"] + where["zero"]:
        b, rem = divmod(rix, Sq * H)
        s, h = divmod(rem, H)
        want, _ = oracle.rmsnorm_rows(vbar[b, h][None, :], spec["eps_rms"])
        assert np.max(np.abs(yr[rix] - want[0])) < 2e-2, (b, s, h)
    assert np.max(np.abs(st[0].cpu().numpy() - mu)) <= 1e-4 * max(1.0, float(np.max(np.abs(mu))))
    assert_close_stats(st[1].cpu().numpy(), r1, "ln rstd")
    assert_close_stats(st[2].cpu().numpy(), r2, "rms rstd", rtol=3e-3)


FNA_LENGTHS = [3, 70, 0, 129, 33, 1]


def fna_planted(H, Skv, seed, dout=False, kinds=inputs.ROW_KINDS, shift=24.0):
    name = "flash_norm_attention_bwd" if dout else "flash_norm_attention"
    spec, d = inputs.make_inputs(name, B=len(FNA_LENGTHS), H=H, Skv=Skv, lengths=FNA_LENGTHS,
                                 max_len=max(FNA_LENGTHS), seed=seed)
    T = int(d["offsets"][-1])
    rows = sorted({0, 1, 2, 3, 31, 32, 33, 72, 73, 100, 104, 105, 201, 202, 232, T - 2, T - 1})
    q, where = inputs.plant_rows(d["Q"], [r for r in rows if r < T], kinds, seed=seed + 1,
                                 eps=spec["eps_ln"], row_dims=2, shift=shift)
    return spec, dict(d, Q=q), rows, where


@pytest.mark.parametrize("act", ["softmax", "gelu"])
@pytest.mark.parametrize("H", [2, 4, 8])
def test_fna_degenerate_rows(H, act):
    spec, d, rows, where = fna_planted(H, 72, seed=520 + H)
    log(f"FlashNormAttention degenerate rows H={H} act={act}: {where}")
    Q, K, V = dev(d["Q"]), dev(d["K"]), dev(d["V"])
    off = torch.from_numpy(np.ascontiguousarray(d["offsets"])).to("cuda")
    O = empty_bf16(*Q.shape)
    T = Q.shape[0]
    st = [torch.full((T,), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3)]
    B.fng_flash_norm_attention(Q, off, K, V, O, spec["max_len"], spec["eps_ln"], spec["eps_rms"], SCALE, act, *st)
    torch.cuda.synchronize()
    ref, mu, r1, r2 = oracle.flash_norm_attention(f64(d["Q"]), d["offsets"], f64(d["K"]), f64(d["V"]),
                                                  spec["eps_ln"], spec["eps_rms"], SCALE, act)
    y = host(O)
    assert np.all(np.isfinite(y))
    assert_parity_floor(y, ref, f"fna degenerate H={H} {act}")
    assert_planted_floor(y, ref, where, "planted")
    assert np.max(np.abs(st[0].cpu().numpy() - mu)) <= 1e-4 * max(1.0, float(np.max(np.abs(mu))))
    assert_close_stats(st[1].cpu().numpy(), r1, "fna ln rstd")
    assert_close_stats(st[2].cpu().numpy(), r2, "fna rms rstd", rtol=3e-3)


@pytest.mark.parametrize("H", [4, 8])
@pytest.mark.parametrize("act", ["softmax", "gelu"])
def test_fna_bwd_degenerate_rows(act, H):
    """Zero, constant, tiny and shifted query rows through the forward and the
    backward.  The backward rebuilds the RMSNorm output as out - Q from the
    bf16 forward output (the page's recompute), which carries out's rounding,
    about |x| 2^-9, into it: the shift is 4 spreads here, and rows of 2^12-size
    entries are left to the forward test (there out - Q keeps no digit of the
    unit-size RMSNorm output)."""
    spec, d, rows, where = fna_planted(H, 72, seed=530, dout=True, kinds=("zero", "const", "tiny", "shifted"),
                                       shift=4.0)
    log(f"FlashNormAttention backward degenerate rows H={H} act={act}: {where}")
    Q, K, V, G = dev(d["Q"]), dev(d["K"]), dev(d["V"]), dev(d["dOut"])
    off = torch.from_numpy(np.ascontiguousarray(d["offsets"])).to("cuda")
    T = Q.shape[0]
    out = empty_bf16(*Q.shape)
    st = [torch.zeros(T, dtype=torch.float32, device="cuda") for _ in range(3)]
    B.fng_flash_norm_attention(Q, off, K, V, out, spec["max_len"], spec["eps_ln"], spec["eps_rms"], SCALE, act, *st)
    dQ, dK, dV = empty_bf16(*Q.shape), empty_bf16(*K.shape), empty_bf16(*V.shape)
    ws = torch.empty(B.fng_flash_norm_attention_bwd_workspace_bytes(T, H), dtype=torch.uint8, device="cuda")
    B.fng_flash_norm_attention_bwd(Q, off, K, V, out, G, st[0], st[1], st[2], dQ, dK, dV, spec["max_len"],
                                   workspace=ws, sm_scale=SCALE, act=act)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.flash_norm_attention_backward(f64(d["Q"]), d["offsets"], f64(d["K"]), f64(d["V"]),
                                                      f64(d["dOut"]), spec["eps_ln"], spec["eps_rms"], SCALE, act)
    yq, yk, yv = host(dQ), host(dK), host(dV)
    for t in (yq, yk, yv):
        assert np.all(np.isfinite(t))
    # the LayerNorm backward of a constant row is rstd (g - mean g) with
    # rstd = 1/sqrt(eps_ln), about 316 (and with GELU the RMSNorm of an exactly
    # zero attention output scales its gradient by 1/sqrt(eps_rms) = 1000), so
    # those rows are compared per kind against their own scale
    planted = sorted(sum(where.values(), []))
    rest = np.setdiff1d(np.arange(T), planted)
    assert_parity_floor(yq[rest], rq[rest], f"bwd degenerate {act} dQ (other rows)")
    assert_planted_floor(yq, rq, where, f"bwd degenerate {act} dQ")
    assert_parity_floor(yk, rk, f"bwd degenerate {act} dK")
    assert_parity_floor(yv, rv, f"bwd degenerate {act} dV")


# ---------------------------------------------------------------------------
# backward by regrouping: zero normalized rows (the forward of a zero or
# constant row saved y = 0 and rstd = 1/sqrt(eps))
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["ln", "rms", "prenorm_dx"])
@pytest.mark.parametrize("path", [B.FNG_PATH_FULLN, B.FNG_PATH_SPLITN], ids=["fulln", "splitn"])
def test_norm_bwd_degenerate_rows(kind, path):
    M, K, N = (600, 264, 256) if path == B.FNG_PATH_FULLN else (600, 200, 1320)
    name = "prenorm_rms_mlp_bwd_dx" if kind == "prenorm_dx" else "postnorm_ln_smalln_bwd"
    spec, d = inputs.make_inputs(name, M=M, K=K, N=N, seed=540)
    eps = 1e-6 if kind != "ln" else 1e-5
    rows = planted_rows(M)
    h = d["H"].copy()
    rstd = d["rstd"].copy()
    for i, r in enumerate(rows):
        if i % 2 == 0:     # a zero (or constant, for LN) forward row
            h[r] = 0
            rstd[r] = np.float32(1.0 / math.sqrt(eps))
        else:              # a forward row of mean square about eps (pre-norm input)
            h[r] = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(h[r]) * np.float32(math.sqrt(eps)))
            if kind == "prenorm_dx":
                rstd[r] = np.float32(1.0 / math.sqrt(eps + float(np.mean(f64(h[r]) ** 2))))
    log(f"norm bwd degenerate {kind} path={path} {M}x{K}x{N}")
    G, Wt, H = dev(d["G"]), dev(d["Wt"]), dev(h)
    r = torch.from_numpy(rstd).to("cuda")
    dZ = empty_bf16(M, N)
    ws = None
    if path != B.FNG_PATH_FULLN:
        ws = torch.zeros(B.fng_gemm_postnorm_workspace_bytes(M, N, K, B.FNG_PATH_SPLITN), dtype=torch.uint8,
                         device="cuda")
    if kind == "ln":
        B.fng_gemm_postnorm_ln_bwd(G, Wt, H, r, dZ, workspace=ws, path=path)
        ref = oracle.gemm_postnorm_backward(f64(d["G"]), f64(d["Wt"]), f64(h), rstd, "ln")
    elif kind == "rms":
        B.fng_gemm_postnorm_rms_bwd(G, Wt, H, r, dZ, workspace=ws, path=path)
        ref = oracle.gemm_postnorm_backward(f64(d["G"]), f64(d["Wt"]), f64(h), rstd, "rms")
    else:
        # the product is dY [M, K] @ Wt [K, N]; the norm axis has N entries
        B.fng_prenorm_rms_bwd_dx(G, Wt, H, r, dZ, workspace=ws, path=path)
        ref = oracle.prenorm_rms_backward_dx(f64(d["G"]), f64(d["Wt"]), f64(h), rstd)
    torch.cuda.synchronize()
    if ws is not None:
        assert B.fng_get_kernel_status(ws) == B.FNG_OK
    y = host(dZ)
    assert np.all(np.isfinite(y))
    # rows with rstd = 1/sqrt(eps) carry gradients hundreds of times larger
    # than the others: each group against its own scale
    big = rows[::2]
    rest = np.setdiff1d(np.arange(M), big)
    assert_parity_floor(y[rest], ref[rest], f"{kind} bwd degenerate (other rows)")
    assert_parity_floor(y[big], ref[big], f"{kind} bwd degenerate (zero rows)",
                        margin=1e-3 * float(np.mean(np.abs(ref[big]))))
