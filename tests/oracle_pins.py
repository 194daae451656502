"""Pins that tie the fp64 oracle to something other than itself.

Each check takes the oracle module (or a planted-mistake copy of it) as its
argument and raises AssertionError when the oracle disagrees with:
  * pure-Python brute force (math module, explicit loops) on tiny inputs,
  * closed forms and invariants the mathematics fixes,
  * special cases that reduce to torch CPU fp64 library routines
    (F.rms_norm, F.layer_norm, F.scaled_dot_product_attention).
They are shared by test_oracle_pins.py (real oracle: all must pass) and
test_oracle_mutants.py (planted mistakes: at least one must fail).

Formulas follow "Towards Free Normalization: Fusing Normalization into GEMM
and Attention Kernels": section 2 (rstd with eps inside the rsqrt, division by
the row length, the row-scale commutation identity), section 3 (post-norm over
the GEMM output rows) and section 4 (LayerNorm before attention, RMSNorm
after it).
"""

import math

import numpy as np


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


# ---------------------------------------------------------------------------
# brute force in plain Python (no numpy arithmetic)
# ---------------------------------------------------------------------------

def bf_rmsnorm(rows, eps, gamma=None):
    out, rs = [], []
    for row in rows:
        n = len(row)
        ss = 0.0
        for v in row:
            ss += v * v
        r = 1.0 / math.sqrt(ss / n + eps)
        y = [v * r for v in row]
        if gamma is not None:
            y = [y[i] * gamma[i] for i in range(n)]
        out.append(y)
        rs.append(r)
    return out, rs


def bf_layernorm(rows, eps):
    out, mus, rs = [], [], []
    for row in rows:
        n = len(row)
        mu = 0.0
        for v in row:
            mu += v
        mu /= n
        var = 0.0
        for v in row:
            var += (v - mu) * (v - mu)
        var /= n
        r = 1.0 / math.sqrt(var + eps)
        out.append([(v - mu) * r for v in row])
        mus.append(mu)
        rs.append(r)
    return out, mus, rs


def bf_matmul(a, b):
    M, K, N = len(a), len(b), len(b[0])
    assert all(len(r) == K for r in a)
    c = [[0.0] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = 0.0
            for k in range(K):
                s += a[i][k] * b[k][j]
            c[i][j] = s
    return c


def bf_softmax(row):
    m = max(row)
    e = [math.exp(v - m) for v in row]
    s = sum(e)
    return [v / s for v in e]


def bf_norm_attention(q, k, v, eps_ln, eps_rms, scale):
    """q[b][s][h][d] nested lists; returns out nested lists."""
    B, Sq, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Skv = len(k[0])
    out = [[[None] * H for _ in range(Sq)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            qrows = [q[b][s][h] for s in range(Sq)]
            qn, _, _ = bf_layernorm(qrows, eps_ln)
            for s in range(Sq):
                sc = []
                for t in range(Skv):
                    acc = 0.0
                    for d in range(D):
                        acc += qn[s][d] * k[b][t][h][d]
                    sc.append(acc * scale)
                p = bf_softmax(sc)
                o = [0.0] * D
                for t in range(Skv):
                    for d in range(D):
                        o[d] += p[t] * v[b][t][h][d]
                y, _ = bf_rmsnorm([o], eps_rms)
                out[b][s][h] = y[0]
    return out


def bf_gelu_erf(x):
    """GELU by its definition x * Phi(x), Phi the standard normal CDF."""
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def bf_flash_norm_attention(q, offsets, k, v, eps_ln, eps_rms, scale, act):
    """Full FlashNormAttention on nested lists: q[t][h][d] jagged rows,
    k, v [b][t][h][d]; act 'softmax' or a Python function applied per score."""
    H, D = len(q[0]), len(q[0][0])
    out = [None] * len(q)
    for b in range(len(offsets) - 1):
        for r in range(offsets[b], offsets[b + 1]):
            x = [q[r][h][d] for h in range(H) for d in range(D)]
            ln, _, _ = bf_layernorm([x], eps_ln)
            ln = ln[0]
            o = []
            for h in range(H):
                sc = []
                for t in range(len(k[b])):
                    acc = 0.0
                    for d in range(D):
                        acc += ln[h * D + d] * k[b][t][h][d]
                    sc.append(acc * scale)
                p = bf_softmax(sc) if act == "softmax" else [act(s) for s in sc]
                for d in range(D):
                    acc = 0.0
                    for t in range(len(k[b])):
                        acc += p[t] * v[b][t][h][d]
                    o.append(acc + ln[h * D + d])
            y, _ = bf_rmsnorm([o], eps_rms)
            out[r] = [[y[0][h * D + d] + x[h * D + d] for d in range(D)] for h in range(H)]
    return out


# ---------------------------------------------------------------------------
# bf16 decoding
# ---------------------------------------------------------------------------

def check_bf16_decode(O):
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x3E80,
                     0x7F80, 0xFF80], dtype=np.uint16)
    want = [1.0, -2.0, 3.140625, 2.0 ** -133, (2.0 - 2.0 ** -7) * 2.0 ** 127, 0.0, -0.0,
            0.25, math.inf, -math.inf]
    got = O.bf16_to_f64(bits)
    for g, w, b in zip(got, want, bits):
        assert g == w, f"bf16 0x{int(b):04x} -> {g!r}, want {w!r}"
    assert math.copysign(1.0, got[6]) == -1.0
    assert np.isnan(O.bf16_to_f64(np.array([0x7FC0], dtype=np.uint16))[0])


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def check_rmsnorm_closed_form(O):
    # x = [3, 4]: mean square 12.5; eps = 0 -> rstd = 1/sqrt(12.5)
    y, r = O.rmsnorm_rows(np.array([[3.0, 4.0]]), 0.0)
    _close(r, [1.0 / math.sqrt(12.5)], 1e-15, "rstd([3,4])")
    _close(y, [[3.0 / math.sqrt(12.5), 4.0 / math.sqrt(12.5)]], 1e-15, "rmsnorm([3,4])")
    # constant row c: y = c / sqrt(c^2 + eps)
    y, _ = O.rmsnorm_rows(np.full((1, 5), 2.0), 0.25)
    _close(y, np.full((1, 5), 2.0 / math.sqrt(4.25)), 1e-15, "rmsnorm(const)")
    # zero row: y = 0, rstd = 1/sqrt(eps)
    y, r = O.rmsnorm_rows(np.zeros((1, 4)), 1e-6)
    _close(y, np.zeros((1, 4)), 0.0, "rmsnorm(0)")
    _close(r, [1e3], 1e-9, "rstd(0)")


def check_rmsnorm_bruteforce(O):
    rng = _rng(11)
    x = rng.standard_normal((5, 7)) * rng.uniform(0.1, 3.0, (5, 1))
    g = rng.standard_normal(7)
    for gamma in (None, g):
        y, r = O.rmsnorm_rows(x, 1e-3, gamma)
        by, br = bf_rmsnorm(x.tolist(), 1e-3, None if gamma is None else gamma.tolist())
        _close(y, by, 1e-13, "rmsnorm vs brute force")
        _close(r, br, 1e-13, "rstd vs brute force")


def check_rmsnorm_invariants(O):
    rng = _rng(12)
    x = rng.standard_normal((64, 48)) * rng.lognormal(0.0, 1.0, (64, 1))
    eps = 1e-6
    y, _ = O.rmsnorm_rows(x, eps)
    ms = np.mean(x * x, axis=1)
    # mean(y^2) = ms / (ms + eps) exactly
    _close(np.mean(y * y, axis=1), ms / (ms + eps), 1e-12, "rms of rmsnorm output")
    # eps = 0: invariant under positive row scaling
    y0, _ = O.rmsnorm_rows(x, 0.0)
    y1, _ = O.rmsnorm_rows(x * 37.5, 0.0)
    _close(y0, y1, 1e-12, "rmsnorm scale invariance")
    _close(np.mean(y0 * y0, axis=1), np.ones(64), 1e-12, "unit rms at eps=0")


def check_rmsnorm_torch(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(13)
    x = rng.standard_normal((33, 96))
    g = rng.standard_normal(96)
    for gamma in (None, g):
        ref = F.rms_norm(torch.from_numpy(x), (96,),
                         None if gamma is None else torch.from_numpy(gamma), eps=1e-5).numpy()
        y, _ = O.rmsnorm_rows(x, 1e-5, gamma)
        _close(y, ref, 1e-12, "rmsnorm vs torch F.rms_norm fp64")


# ---------------------------------------------------------------------------
# LayerNorm
# ---------------------------------------------------------------------------

def check_layernorm_closed_form(O):
    # x = [1,2,3,4]: mu = 2.5, biased var = 1.25
    y, mu, r = O.layernorm_rows(np.array([[1.0, 2.0, 3.0, 4.0]]), 0.0)
    _close(mu, [2.5], 1e-15, "ln mean")
    _close(r, [1.0 / math.sqrt(1.25)], 1e-15, "ln rstd (biased variance)")
    _close(y, [[(v - 2.5) / math.sqrt(1.25) for v in (1, 2, 3, 4)]], 1e-15, "ln([1,2,3,4])")
    # constant row -> exactly 0
    y, mu, r = O.layernorm_rows(np.full((2, 6), -3.5), 1e-5)
    _close(y, np.zeros((2, 6)), 0.0, "ln(const)")
    _close(mu, [-3.5, -3.5], 0.0, "ln mean const")


def check_layernorm_bruteforce(O):
    rng = _rng(21)
    x = rng.standard_normal((6, 5)) * 2.0 + 0.7
    y, mu, r = O.layernorm_rows(x, 1e-2)
    by, bmu, br = bf_layernorm(x.tolist(), 1e-2)
    _close(y, by, 1e-13, "ln vs brute force")
    _close(mu, bmu, 1e-13, "ln mean vs brute force")
    _close(r, br, 1e-13, "ln rstd vs brute force")


def check_layernorm_invariants(O):
    rng = _rng(22)
    x = rng.standard_normal((40, 64)) * 3.0 + 5.0
    eps = 1e-5
    y, mu, r = O.layernorm_rows(x, eps)
    v = np.var(x, axis=1)
    _close(np.mean(y, axis=1), np.zeros(40), 1e-12, "ln output mean")
    _close(np.mean(y * y, axis=1), v / (v + eps), 1e-12, "ln output variance")
    y0, _, _ = O.layernorm_rows(x, 0.0)
    y1, _, _ = O.layernorm_rows(x * 4.25 - 11.0, 0.0)
    _close(y0, y1, 1e-11, "ln affine invariance")


def check_layernorm_torch(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(23)
    x = rng.standard_normal((31, 80)) * 1.5 - 0.5
    ref = F.layer_norm(torch.from_numpy(x), (80,), eps=1e-5).numpy()
    y, _, _ = O.layernorm_rows(x, 1e-5)
    _close(y, ref, 1e-12, "ln vs torch F.layer_norm fp64")


# ---------------------------------------------------------------------------
# norm + GEMM
# ---------------------------------------------------------------------------

def check_prenorm_gemm_bruteforce(O):
    rng = _rng(31)
    M, K, N = 4, 6, 3
    x = rng.standard_normal((M, K)) * 1.7
    w = rng.standard_normal((K, N))
    g = rng.standard_normal(K)
    for gamma in (None, g):
        y, r = O.prenorm_rms_gemm(x, w, 1e-4, gamma)
        xn, br = bf_rmsnorm(x.tolist(), 1e-4, None if gamma is None else gamma.tolist())
        _close(y, bf_matmul(xn, w.tolist()), 1e-13, "prenorm gemm vs brute force")
        _close(r, br, 1e-13, "prenorm rstd vs brute force")


def check_prenorm_gemm_identities(O):
    rng = _rng(32)
    M, K, N = 9, 16, 5
    x = rng.standard_normal((M, K)) * rng.lognormal(0.0, 1.0, (M, 1))
    w = rng.standard_normal((K, N))
    eps = 1e-6
    y, r = O.prenorm_rms_gemm(x, w, eps)
    # lazy form: (diag(rstd) X) W = diag(rstd) (X W), rstd from brute force
    _, br = bf_rmsnorm(x.tolist(), eps)
    lazy = np.array(bf_matmul(x.tolist(), w.tolist())) * np.array(br)[:, None]
    _close(y, lazy, 1e-12, "lazy pre-norm identity")
    # W = I reduces to rmsnorm(X)
    yi, _ = O.prenorm_rms_gemm(x, np.eye(K), eps)
    xn, _ = bf_rmsnorm(x.tolist(), eps)
    _close(yi, xn, 1e-13, "prenorm with W = I")
    # row permutation equivariance
    p = rng.permutation(M)
    yp, _ = O.prenorm_rms_gemm(x[p], w, eps)
    _close(yp, y[p], 1e-13, "prenorm row permutation")


def check_prenorm_gemm_torch(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(33)
    x = rng.standard_normal((20, 64)) * 2.0
    w = rng.standard_normal((64, 24)) / 8.0
    g = 1.0 + 0.3 * rng.standard_normal(64)
    ref = (F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6)
           @ torch.from_numpy(w)).numpy()
    y, _ = O.prenorm_rms_gemm(x, w, 1e-6, g)
    _close(y, ref, 1e-12, "prenorm gemm vs torch fp64")


def check_prenorm_ln_gemm(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(34)
    # brute force on a tiny case
    x = rng.standard_normal((4, 6)) * 1.5 + 0.7
    w = rng.standard_normal((6, 3))
    y, mu, r = O.prenorm_ln_gemm(x, w, 1e-4)
    xn, bmu, br = bf_layernorm(x.tolist(), 1e-4)
    _close(y, bf_matmul(xn, w.tolist()), 1e-13, "lazy LN pre-norm vs brute force")
    _close(mu, bmu, 1e-14, "lazy LN mean")
    _close(r, br, 1e-13, "lazy LN rstd")
    # torch fp64 library routines, rows shifted far from zero mean
    x = rng.standard_normal((20, 64)) * 2.0 + 5.0 * rng.standard_normal((20, 1))
    w = rng.standard_normal((64, 24)) / 8.0
    ref = (F.layer_norm(torch.from_numpy(x), (64,), eps=1e-5) @ torch.from_numpy(w)).numpy()
    y, mu, r = O.prenorm_ln_gemm(x, w, 1e-5)
    _close(y, ref, 1e-12, "lazy LN pre-norm vs torch fp64")
    # the rank-1 form the kernel applies: diag(rstd) (X W - mu colsum(W))
    rank1 = r[:, None] * (x @ w - mu[:, None] * w.sum(axis=0)[None, :])
    _close(y, rank1, 1e-11, "lazy LN pre-norm rank-1 identity")
    # W = I reduces it to the LayerNorm itself
    y, _, _ = O.prenorm_ln_gemm(x[:, :24], np.eye(24), 1e-5)
    _close(y, F.layer_norm(torch.from_numpy(x[:, :24]), (24,), eps=1e-5).numpy(), 1e-12, "lazy LN, W = I")


def check_postnorm_affine(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(44)
    x = rng.standard_normal((9, 40)) + 0.6
    w = rng.standard_normal((40, 24)) / 6.0
    g = 1.0 + 0.3 * rng.standard_normal(24)
    b = 0.5 * rng.standard_normal(24)
    z = torch.from_numpy(x @ w)
    y, _, _ = O.gemm_postnorm_affine(x, w, 1e-5, "ln", g, b)
    _close(y, F.layer_norm(z, (24,), torch.from_numpy(g), torch.from_numpy(b), eps=1e-5).numpy(), 1e-12,
           "post-LN affine vs torch")
    y, _, _ = O.gemm_postnorm_affine(x, w, 1e-6, "rms", g, None)
    _close(y, F.rms_norm(z, (24,), torch.from_numpy(g), eps=1e-6).numpy(), 1e-12, "post-RMS gain vs torch")
    y, _, _ = O.gemm_postnorm_affine(x, w, 1e-6, "rms", g, b)
    _close(y, (F.rms_norm(z, (24,), torch.from_numpy(g), eps=1e-6) + torch.from_numpy(b)).numpy(), 1e-12,
           "post-RMS gain and bias vs torch")
    # gamma = 1, beta = 0 is the plain post-norm
    y0, _, _ = O.gemm_postnorm(x, w, 1e-5, "ln")
    y1, _, _ = O.gemm_postnorm_affine(x, w, 1e-5, "ln", np.ones(24), np.zeros(24))
    _close(y1, y0, 0.0, "identity affine")


def check_postnorm_bruteforce(O):
    rng = _rng(41)
    M, K, N = 3, 5, 6
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((K, N))
    z = bf_matmul(x.tolist(), w.tolist())
    y, mu, r = O.gemm_postnorm(x, w, 1e-3, "ln")
    by, bmu, br = bf_layernorm(z, 1e-3)
    _close(y, by, 1e-13, "post-LN gemm vs brute force")
    _close(mu, bmu, 1e-13, "post-LN mean vs brute force")
    _close(r, br, 1e-13, "post-LN rstd vs brute force")
    y, mu, r = O.gemm_postnorm(x, w, 1e-3, "rms")
    by, br = bf_rmsnorm(z, 1e-3)
    assert mu is None
    _close(y, by, 1e-13, "post-RMS gemm vs brute force")
    _close(r, br, 1e-13, "post-RMS rstd vs brute force")


def check_postnorm_identities(O):
    rng = _rng(42)
    M, K, N = 12, 32, 48
    x = rng.standard_normal((M, K))
    w = rng.standard_normal((K, N)) / math.sqrt(K)
    # W = I (K = N) reduces to the row norm of X
    xs = rng.standard_normal((M, N)) * 2.0 + 1.0
    yi, _, _ = O.gemm_postnorm(xs, np.eye(N), 1e-5, "ln")
    bi, _, _ = bf_layernorm(xs.tolist(), 1e-5)
    _close(yi, bi, 1e-13, "post-LN with W = I")
    yi, _, _ = O.gemm_postnorm(xs, np.eye(N), 1e-6, "rms")
    bi, _ = bf_rmsnorm(xs.tolist(), 1e-6)
    _close(yi, bi, 1e-13, "post-RMS with W = I")
    # output invariants over N
    y, _, _ = O.gemm_postnorm(x, w, 0.0, "ln")
    _close(np.mean(y, axis=1), np.zeros(M), 1e-12, "post-LN row mean")
    _close(np.mean(y * y, axis=1), np.ones(M), 1e-12, "post-LN row variance")
    y, _, _ = O.gemm_postnorm(x, w, 0.0, "rms")
    _close(np.mean(y * y, axis=1), np.ones(M), 1e-12, "post-RMS row rms")
    p = rng.permutation(M)
    ya, _, _ = O.gemm_postnorm(x, w, 1e-6, "rms")
    yb, _, _ = O.gemm_postnorm(x[p], w, 1e-6, "rms")
    _close(yb, ya[p], 1e-13, "post-norm row permutation")


def check_postnorm_torch(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(43)
    x = rng.standard_normal((17, 40))
    w = rng.standard_normal((40, 72)) / 6.0
    z = torch.from_numpy(x) @ torch.from_numpy(w)
    y, _, _ = O.gemm_postnorm(x, w, 1e-5, "ln")
    _close(y, F.layer_norm(z, (72,), eps=1e-5).numpy(), 1e-12, "post-LN vs torch fp64")
    y, _, _ = O.gemm_postnorm(x, w, 1e-6, "rms")
    _close(y, F.rms_norm(z, (72,), eps=1e-6).numpy(), 1e-12, "post-RMS vs torch fp64")


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def check_attention_bruteforce(O):
    rng = _rng(51)
    B, Sq, Skv, H, D = 1, 3, 4, 2, 5
    q = rng.standard_normal((B, Sq, H, D)) * 1.3 + 0.2
    k = rng.standard_normal((B, Skv, H, D))
    v = rng.standard_normal((B, Skv, H, D))
    out, _, _, _ = O.norm_attention(q, k, v, 1e-5, 1e-6, 0.7)
    ref = bf_norm_attention(q.tolist(), k.tolist(), v.tolist(), 1e-5, 1e-6, 0.7)
    _close(out, ref, 1e-12, "norm attention vs brute force")


def check_attention_torch(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(52)
    B, Sq, Skv, H, D = 2, 9, 13, 3, 16
    q = rng.standard_normal((B, Sq, H, D)) * 2.0 - 1.0
    k = rng.standard_normal((B, Skv, H, D))
    v = rng.standard_normal((B, Skv, H, D))
    scale = 1.0 / math.sqrt(D)
    tq = F.layer_norm(torch.from_numpy(q), (D,), eps=1e-5).permute(0, 2, 1, 3).contiguous()
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).contiguous()
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).contiguous()
    o = F.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    ref = F.rms_norm(o, (D,), eps=1e-6).permute(0, 2, 1, 3).numpy()
    out, mu, r1, r2 = O.norm_attention(q, k, v, 1e-5, 1e-6, scale)
    _close(out, ref, 1e-12, "norm attention vs torch fp64 sdpa")
    # plain attention against sdpa too
    o2 = F.scaled_dot_product_attention(torch.from_numpy(q).permute(0, 2, 1, 3).contiguous(),
                                        tk, tv, scale=scale).permute(0, 2, 1, 3).numpy()
    _close(O.attention(q, k, v, scale), o2, 1e-12, "attention vs torch fp64 sdpa")
    _close(mu, np.mean(q, axis=-1), 1e-13, "ln mean output")
    _close(r1, 1.0 / np.sqrt(np.var(q, axis=-1) + 1e-5), 1e-12, "ln rstd output")


def check_attention_closed_forms(O):
    rng = _rng(53)
    B, Sq, H, D = 2, 5, 3, 8
    q = rng.standard_normal((B, Sq, H, D))
    # one key: weights are 1, out = rmsnorm(v) for every query
    k1 = rng.standard_normal((B, 1, H, D))
    v1 = rng.standard_normal((B, 1, H, D))
    out, _, _, _ = O.norm_attention(q, k1, v1, 1e-5, 1e-6, 0.3)
    want, _ = bf_rmsnorm(v1.reshape(-1, D).tolist(), 1e-6)
    want = np.array(want).reshape(B, 1, H, D)
    _close(out, np.broadcast_to(want, out.shape), 1e-13, "single key -> rmsnorm(v)")
    # K = 0: uniform weights, out = rmsnorm(mean_t v)
    Skv = 7
    k0 = np.zeros((B, Skv, H, D))
    v = rng.standard_normal((B, Skv, H, D))
    out, _, _, _ = O.norm_attention(q, k0, v, 1e-5, 1e-6, 0.3)
    mv = np.mean(v, axis=1)
    want, _ = bf_rmsnorm(mv.reshape(-1, D).tolist(), 1e-6)
    want = np.array(want).reshape(B, 1, H, D)
    _close(out, np.broadcast_to(want, out.shape), 1e-13, "K = 0 -> uniform weights")
    # constant query rows: layernorm gives 0 -> uniform weights for any K
    qc = np.full((B, Sq, H, D), 4.0)
    k = rng.standard_normal((B, Skv, H, D))
    out, _, _, _ = O.norm_attention(qc, k, v, 1e-5, 1e-6, 0.3)
    _close(out, np.broadcast_to(want, out.shape), 1e-13, "constant q -> uniform weights")
    # jointly permuting keys and values leaves the output unchanged
    qq = rng.standard_normal((B, Sq, H, D))
    o1, _, _, _ = O.norm_attention(qq, k, v, 1e-5, 1e-6, 0.3)
    p = rng.permutation(Skv)
    o2, _, _, _ = O.norm_attention(qq, k[:, p], v[:, p], 1e-5, 1e-6, 0.3)
    _close(o1, o2, 1e-13, "kv permutation invariance")
    # output rows have rms ms/(ms+eps) -> ~1
    _close(np.mean(o1 * o1, axis=-1), np.ones(o1.shape[:-1]), 1e-3, "output row rms")


def check_gelu(O):
    xs = np.linspace(-8.0, 8.0, 401)
    g = O.gelu_tanh(xs)
    # the tanh form stays within 5e-4 of the exact x * Phi(x) everywhere
    _close(g, [bf_gelu_erf(x) for x in xs], 5e-4, "gelu tanh form vs erf definition")
    # exact identities of the form: odd part x/2, value 0 at 0
    _close(g - O.gelu_tanh(-xs), xs, 1e-12, "gelu(x) - gelu(-x) = x")
    _close(O.gelu_tanh(np.array([0.0])), [0.0], 0.0, "gelu(0)")


def _fna_case(seed, lengths, Skv, H, D, qscale=1.0):
    rng = _rng(seed)
    off = [0]
    for n in lengths:
        off.append(off[-1] + n)
    q = rng.standard_normal((off[-1], H, D)) * qscale + 0.3
    q[:, 0, :] *= 3.0  # heads on different scales: per-head and cross-head norms differ
    k = rng.standard_normal((len(lengths), Skv, H, D))
    v = rng.standard_normal((len(lengths), Skv, H, D))
    return q, np.array(off), k, v


def check_fna_bruteforce(O):
    q, off, k, v = _fna_case(61, [2, 0, 3], 4, 2, 3)
    for act, f in (("softmax", "softmax"), ("gelu", bf_gelu_erf)):
        out, _, _, _ = O.flash_norm_attention(q, off, k, v, 1e-5, 1e-6, 0.6, act)
        ref = bf_flash_norm_attention(q.tolist(), off.tolist(), k.tolist(), v.tolist(), 1e-5, 1e-6, 0.6, f)
        # softmax: exact up to rounding; gelu: the reference uses the erf definition
        _close(out, ref, 1e-12 if act == "softmax" else 2e-3, f"flash norm attention ({act}) vs brute force")


def check_fna_torch(O):
    import torch
    import torch.nn.functional as F
    q, off, k, v = _fna_case(62, [5, 7], 6, 3, 8, qscale=2.0)
    H, D = 3, 8
    out, mu, r1, r2 = O.flash_norm_attention(q, off, k, v, 1e-5, 1e-6, 0.4, "softmax")
    for b in range(2):
        x = torch.from_numpy(q[off[b]:off[b + 1]]).reshape(-1, H * D)
        ln = F.layer_norm(x, (H * D,), eps=1e-5).reshape(-1, H, D)
        tq = ln.permute(1, 0, 2).contiguous()
        tk = torch.from_numpy(k[b]).permute(1, 0, 2).contiguous()
        tv = torch.from_numpy(v[b]).permute(1, 0, 2).contiguous()
        o = F.scaled_dot_product_attention(tq, tk, tv, scale=0.4).permute(1, 0, 2) + ln
        ref = F.rms_norm(o.reshape(-1, H * D), (H * D,), eps=1e-6) + x
        _close(out[off[b]:off[b + 1]].reshape(-1, H * D), ref.numpy(), 1e-12, "fna vs torch fp64")
        _close(mu[off[b]:off[b + 1]], x.numpy().mean(axis=1), 1e-13, "fna ln mean")


def check_fna_closed_forms(O):
    q, off, k, v = _fna_case(63, [3, 4], 5, 2, 4)
    T, H, D = q.shape
    flat = q.reshape(T, H * D).tolist()
    ln, _, _ = bf_layernorm(flat, 1e-5)
    # V = 0: the attention term vanishes, out = rmsnorm(layernorm(x)) + x
    out, _, _, _ = O.flash_norm_attention(q, off, k, np.zeros_like(v), 1e-5, 1e-6, 0.5, "gelu")
    y, _ = bf_rmsnorm(ln, 1e-6)
    _close(out.reshape(T, H * D), np.array(y) + q.reshape(T, H * D), 1e-12, "V = 0")
    # K = 0 with softmax: uniform weights, o_h = mean_t v + ln_h
    out, _, _, _ = O.flash_norm_attention(q, off, np.zeros_like(k), v, 1e-5, 1e-6, 0.5, "softmax")
    o = np.array(ln).reshape(T, H, D).copy()
    for b in range(2):
        o[off[b]:off[b + 1]] += np.mean(v[b], axis=0)[None]
    y, _ = bf_rmsnorm(o.reshape(T, H * D).tolist(), 1e-6)
    _close(out.reshape(T, H * D), np.array(y) + q.reshape(T, H * D), 1e-12, "K = 0 softmax")
    # batches are independent: each batch alone gives the same rows
    full, _, _, _ = O.flash_norm_attention(q, off, k, v, 1e-5, 1e-6, 0.5, "gelu")
    for b in range(2):
        one, _, _, _ = O.flash_norm_attention(q[off[b]:off[b + 1]], np.array([0, off[b + 1] - off[b]]),
                                              k[b:b + 1], v[b:b + 1], 1e-5, 1e-6, 0.5, "gelu")
        _close(full[off[b]:off[b + 1]], one, 0.0, f"batch {b} independent")


def check_jagged_attention(O):
    q, off, k, v = _fna_case(64, [3, 0, 2], 5, 2, 3)
    T, H, D = q.shape
    out = O.jagged_attention(q, off, k, v, 0.7, "gelu")
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    for b in range(3):
        for r in range(off[b], off[b + 1]):
            for h in range(H):
                sc = [0.7 * sum(ql[r][h][d] * kl[b][t][h][d] for d in range(D)) for t in range(5)]
                p = [bf_gelu_erf(s) for s in sc]
                ref = [sum(p[t] * vl[b][t][h][d] for t in range(5)) for d in range(D)]
                _close(out[r, h], ref, 2e-3, "jagged gelu attention vs brute force")
    # softmax on equal lengths is the dense attention, batch by batch
    q, off, k, v = _fna_case(65, [4, 4, 4], 6, 3, 5)
    dense = O.attention(q.reshape(3, 4, 3, 5), k, v, 0.45)
    _close(O.jagged_attention(q, off, k, v, 0.45, "softmax"), dense.reshape(12, 3, 5), 1e-13,
           "jagged softmax attention vs dense")
    # the attention step inside FlashNormAttention: V = 0 leaves only ln + x
    # there, and out here is exactly zero
    assert np.all(O.jagged_attention(q, off, k, np.zeros_like(v), 0.45, "gelu") == 0.0)


# ---------------------------------------------------------------------------
# backward (fusion regrouping)
# ---------------------------------------------------------------------------

def _bwd_case(seed, M=5, N=7, shift=0.4):
    rng = _rng(seed)
    z = rng.standard_normal((M, N)) * (1.0 + np.arange(M)[:, None]) + shift
    g = rng.standard_normal((M, N))
    return z, g


def check_norm_backward_torch(O):
    import torch
    import torch.nn.functional as F
    z, g = _bwd_case(71, 6, 40)
    for kind in ("ln", "rms"):
        zt = torch.from_numpy(z.copy()).requires_grad_(True)
        if kind == "ln":
            F.layer_norm(zt, (40,), eps=1e-5).backward(torch.from_numpy(g))
            y, _, r = O.layernorm_rows(z, 1e-5)
            dz = O.layernorm_backward_rows(g, y, r)
        else:
            F.rms_norm(zt, (40,), eps=1e-6).backward(torch.from_numpy(g))
            y, r = O.rmsnorm_rows(z, 1e-6)
            dz = O.rmsnorm_backward_rows(g, y, r)
        _close(dz, zt.grad.numpy(), 1e-12, f"{kind} backward vs torch autograd fp64")


def check_norm_backward_finite_differences(O):
    # central differences of L(z) = sum(g * norm(z)) with the brute-force forward
    z, g = _bwd_case(72, 2, 5)
    h = 1e-6
    for kind in ("ln", "rms"):
        fwd = (lambda rows: bf_layernorm(rows, 1e-5)[0]) if kind == "ln" else (lambda rows: bf_rmsnorm(rows, 1e-6)[0])
        if kind == "ln":
            y, _, r = O.layernorm_rows(z, 1e-5)
            dz = O.layernorm_backward_rows(g, y, r)
        else:
            y, r = O.rmsnorm_rows(z, 1e-6)
            dz = O.rmsnorm_backward_rows(g, y, r)
        for m in range(2):
            for k in range(5):
                zp = z[m].tolist(); zm = z[m].tolist()
                zp[k] += h; zm[k] -= h
                lp = sum(a * b for a, b in zip(g[m], fwd([zp])[0]))
                lm = sum(a * b for a, b in zip(g[m], fwd([zm])[0]))
                fd = (lp - lm) / (2 * h)
                assert abs(fd - dz[m, k]) <= 1e-7 * (1 + abs(fd)), (kind, m, k, fd, dz[m, k])


def check_norm_backward_invariants(O):
    z, g = _bwd_case(73, 4, 9)
    # eps = 0: the gradient is orthogonal to xhat (norm(a z) = norm(z)); LN's
    # also sums to zero (norm(z + c) = norm(z))
    y, _, r = O.layernorm_rows(z, 0.0)
    dz = O.layernorm_backward_rows(g, y, r)
    _close(np.sum(dz, axis=1), np.zeros(4), 1e-12, "LN backward sums to zero")
    _close(np.sum(dz * y, axis=1), np.zeros(4), 1e-12, "LN backward orthogonal to xhat")
    # a constant upstream gradient has no effect through LN; through RMS it does
    _close(O.layernorm_backward_rows(np.ones_like(z), y, r), np.zeros_like(z), 1e-12, "LN: constant g")
    yr, rr = O.rmsnorm_rows(z, 0.0)
    dr = O.rmsnorm_backward_rows(g, yr, rr)
    _close(np.sum(dr * yr, axis=1), np.zeros(4), 1e-12, "RMS backward orthogonal to xhat")
    assert np.max(np.abs(O.rmsnorm_backward_rows(np.ones_like(z), yr, rr))) > 1e-3
    # g along xhat: no gradient (eps = 0)
    _close(O.layernorm_backward_rows(3.0 * y, y, r), np.zeros_like(z), 1e-12, "LN: g = 3 xhat")
    _close(O.rmsnorm_backward_rows(-2.0 * yr, yr, rr), np.zeros_like(z), 1e-12, "RMS: g = -2 xhat")
    # scaling z by a scales dz by 1/a
    y2, _, r2 = O.layernorm_rows(2.5 * z, 0.0)
    _close(O.layernorm_backward_rows(g, y2, r2), dz / 2.5, 1e-12, "LN backward scaling")


def check_gemm_postnorm_backward_torch(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(74)
    M, N, K2 = 9, 24, 11
    z = rng.standard_normal((M, N)) * 2.0 + 0.5
    W2 = rng.standard_normal((N, K2)) / 4.0      # next layer: out = y @ W2
    dy2 = rng.standard_normal((M, K2))
    for kind in ("ln", "rms"):
        zt = torch.from_numpy(z.copy()).requires_grad_(True)
        yt = F.layer_norm(zt, (N,), eps=1e-5) if kind == "ln" else F.rms_norm(zt, (N,), eps=1e-6)
        (yt @ torch.from_numpy(W2)).backward(torch.from_numpy(dy2))
        if kind == "ln":
            y, _, r = O.layernorm_rows(z, 1e-5)
        else:
            y, r = O.rmsnorm_rows(z, 1e-6)
        dz = O.gemm_postnorm_backward(dy2, W2.T.copy(), y, r, kind)
        _close(dz, zt.grad.numpy(), 1e-12, f"post-{kind} backward (regrouped) vs autograd")


def check_prenorm_backward_torch(O):
    import torch
    import torch.nn.functional as F
    rng = _rng(75)
    M, K, N = 7, 20, 13
    x = rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))
    W = rng.standard_normal((K, N)) / 4.0
    dy = rng.standard_normal((M, N))
    xt = torch.from_numpy(x.copy()).requires_grad_(True)
    (F.rms_norm(xt, (K,), eps=1e-6) @ torch.from_numpy(W)).backward(torch.from_numpy(dy))
    r = O.rms_rstd(x, 1e-6)
    _close(O.prenorm_rms_backward_dx(dy, W.T.copy(), x, r), xt.grad.numpy(), 1e-12,
           "lazy pre-RMS dx vs autograd")


def check_prenorm_backward_dw_torch(O):
    # the weight gradient of (rms_norm(x) * gamma) @ W by fp64 autograd
    # through torch's own rms_norm, with and without the gain
    import torch
    import torch.nn.functional as F
    rng = _rng(76)
    M, K, N = 9, 20, 13
    x = rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))
    x[3] = 0.0                                   # a zero row: rstd = 1/sqrt(eps), no contribution
    W = rng.standard_normal((K, N)) / 4.0
    gamma = 1.0 + 0.3 * rng.standard_normal(K)
    dy = rng.standard_normal((M, N))
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1) + 1e-6)   # the forward's saved statistic
    for g in (None, gamma):
        Wt = torch.from_numpy(W.copy()).requires_grad_(True)
        xn = F.rms_norm(torch.from_numpy(x), (K,), eps=1e-6)
        if g is not None:
            xn = xn * torch.from_numpy(g)
        (xn @ Wt).backward(torch.from_numpy(dy))
        _close(O.prenorm_rms_backward_dw(x, dy, r, g), Wt.grad.numpy(), 1e-12,
               f"lazy pre-RMS dW (gamma={g is not None}) vs autograd")


def check_prenorm_backward_dw_bruteforce(O):
    # dW[k][n] = sum_m x[m][k] * rstd[m] * gamma[k] * dy[m][n], plain loops
    rng = _rng(77)
    M, K, N = 4, 3, 5
    x = rng.standard_normal((M, K)).tolist()
    dy = rng.standard_normal((M, N)).tolist()
    r = (0.5 + rng.random(M)).tolist()
    g = (1.0 + 0.5 * rng.standard_normal(K)).tolist()
    for gam in (None, g):
        want = [[sum(x[m][k] * r[m] * (gam[k] if gam else 1.0) * dy[m][n] for m in range(M))
                 for n in range(N)] for k in range(K)]
        got = O.prenorm_rms_backward_dw(np.array(x), np.array(dy), np.array(r),
                                        np.array(gam) if gam else None)
        _close(got, want, 1e-13, f"lazy pre-RMS dW brute force (gamma={gam is not None})")


def check_prenorm_backward_dw_invariants(O):
    rng = _rng(78)
    M, K, N = 6, 8, 5
    x = rng.standard_normal((M, K))
    dy = rng.standard_normal((M, N))
    r = 0.5 + rng.random(M)
    dw = O.prenorm_rms_backward_dw(x, dy, r)
    # a row scale of x with the matching rstd (x * c, rstd / c) changes nothing
    c = np.exp(rng.standard_normal(M))
    _close(O.prenorm_rms_backward_dw(x * c[:, None], dy, r / c), dw, 1e-12, "dW row-scale invariance")
    # additive over the rows of the batch (the contraction axis)
    a = O.prenorm_rms_backward_dw(x[:2], dy[:2], r[:2]) + O.prenorm_rms_backward_dw(x[2:], dy[2:], r[2:])
    _close(a, dw, 1e-12, "dW sums over rows")
    # a single row gives the outer product of its normalized values and its dy
    one = O.prenorm_rms_backward_dw(x[:1], dy[:1], r[:1])
    _close(one, np.outer(x[0] * r[0], dy[0]), 1e-13, "dW of one row")
    # the gain scales the rows of dW
    gam = 1.0 + rng.random(K)
    _close(O.prenorm_rms_backward_dw(x, dy, r, gam), gam[:, None] * dw, 1e-12, "dW with gain")


def _fna_torch_forward(q, off, k, v, eps_ln, eps_rms, scale, act):
    """FlashNormAttention from torch library routines (fp64), differentiable
    in q, k and v: layer_norm and rms_norm across all heads, softmax or the
    tanh GELU, matrix products."""
    import torch
    import torch.nn.functional as F
    T, H, D = q.shape
    outs = []
    for b in range(len(off) - 1):
        x = q[off[b]:off[b + 1]].reshape(-1, H * D)
        ln = F.layer_norm(x, (H * D,), eps=eps_ln).reshape(-1, H, D)
        heads = []
        for h in range(H):
            s = ln[:, h, :] @ k[b, :, h, :].T * scale
            p = torch.softmax(s, dim=-1) if act == "softmax" else F.gelu(s, approximate="tanh")
            heads.append(p @ v[b, :, h, :])
        o = torch.stack(heads, dim=1) + ln
        outs.append((F.rms_norm(o.reshape(-1, H * D), (H * D,), eps=eps_rms) + x).reshape(-1, H, D))
    return torch.cat(outs)


def check_fna_backward_torch(O):
    import torch
    q, off, k, v = _fna_case(81, [4, 6], 5, 3, 8, qscale=1.7)
    dout = _rng(82).standard_normal(q.shape)
    for act in ("softmax", "gelu"):
        tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
        _fna_torch_forward(tq, off, tk, tv, 1e-5, 1e-6, 0.45, act).backward(torch.from_numpy(dout))
        dq, dk, dv = O.flash_norm_attention_backward(q, off, k, v, dout, 1e-5, 1e-6, 0.45, act)
        _close(dq, tq.grad.numpy(), 1e-11, f"fna backward dq ({act}) vs autograd")
        _close(dk, tk.grad.numpy(), 1e-11, f"fna backward dk ({act}) vs autograd")
        _close(dv, tv.grad.numpy(), 1e-11, f"fna backward dv ({act}) vs autograd")


def _bf_gelu_tanh(x):
    return 0.5 * x * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def check_fna_backward_finite_differences(O):
    # directional derivatives of L = sum(dout * out) with the brute-force forward
    q, off, k, v = _fna_case(83, [2, 3], 3, 2, 3)
    rng = _rng(84)
    dout = rng.standard_normal(q.shape)
    h = 1e-6

    def loss(qq, kk, vv, act):
        f = "softmax" if act == "softmax" else _bf_gelu_tanh
        out = bf_flash_norm_attention(qq.tolist(), off.tolist(), kk.tolist(), vv.tolist(), 1e-5, 1e-6, 0.8, f)
        return sum(dout[r][a][d] * out[r][a][d] for r in range(len(out)) for a in range(2) for d in range(3))

    for act in ("softmax", "gelu"):
        dq, dk, dv = O.flash_norm_attention_backward(q, off, k, v, dout, 1e-5, 1e-6, 0.8, act)
        for _ in range(3):
            eq, ek, ev = (rng.standard_normal(a.shape) for a in (q, k, v))
            fd = (loss(q + h * eq, k + h * ek, v + h * ev, act) - loss(q - h * eq, k - h * ek, v - h * ev, act)) / (2 * h)
            an = float(np.sum(dq * eq) + np.sum(dk * ek) + np.sum(dv * ev))
            assert abs(fd - an) <= 1e-6 * (1.0 + abs(fd)), (act, fd, an)
            # and each input alone, so that a mistake in one gradient cannot hide
            for which, (a, e, g) in enumerate(((q, eq, dq), (k, ek, dk), (v, ev, dv))):
                args_p = [q, k, v]; args_m = [q, k, v]
                args_p[which] = a + h * e; args_m[which] = a - h * e
                fd1 = (loss(*args_p, act) - loss(*args_m, act)) / (2 * h)
                assert abs(fd1 - float(np.sum(g * e))) <= 1e-6 * (1.0 + abs(fd1)), (act, which, fd1)


def _bf_jagged_attention(q, off, k, v, scale, act):
    """Brute force (plain Python loops) of the jagged attention: softmax over
    the keys or the tanh GELU, no norms, no residuals."""
    T, H, D = len(q), len(q[0]), len(q[0][0])
    out = [[[0.0] * D for _ in range(H)] for _ in range(T)]
    for b in range(len(off) - 1):
        for r in range(off[b], off[b + 1]):
            for h in range(H):
                sc = [scale * sum(q[r][h][d] * k[b][t][h][d] for d in range(D)) for t in range(len(k[b]))]
                if act == "softmax":
                    m = max(sc)
                    e = [math.exp(x - m) for x in sc]
                    p = [x / sum(e) for x in e]
                else:
                    p = [_bf_gelu_tanh(x) for x in sc]
                for d in range(D):
                    out[r][h][d] = sum(p[t] * v[b][t][h][d] for t in range(len(k[b])))
    return out


def check_jagged_attention_backward_torch(O):
    import torch
    import torch.nn.functional as F
    q, off, k, v = _fna_case(91, [4, 0, 6], 5, 3, 8, qscale=1.3)
    dout = _rng(92).standard_normal(q.shape)
    for act in ("softmax", "gelu"):
        tq, tk, tv = (torch.from_numpy(a.copy()).requires_grad_(True) for a in (q, k, v))
        outs = []
        for b in range(len(off) - 1):
            heads = []
            for h in range(q.shape[1]):
                sc = tq[off[b]:off[b + 1], h, :] @ tk[b, :, h, :].T * 0.45
                pr = torch.softmax(sc, dim=-1) if act == "softmax" else F.gelu(sc, approximate="tanh")
                heads.append(pr @ tv[b, :, h, :])
            if off[b + 1] > off[b]:
                outs.append(torch.stack(heads, dim=1))
        torch.cat(outs).backward(torch.from_numpy(dout))
        dq, dk, dv = O.jagged_attention_backward(q, off, k, v, dout, 0.45, act)
        _close(dq, tq.grad.numpy(), 1e-11, f"jagged attention backward dq ({act}) vs autograd")
        _close(dk, tk.grad.numpy(), 1e-11, f"jagged attention backward dk ({act}) vs autograd")
        _close(dv, tv.grad.numpy(), 1e-11, f"jagged attention backward dv ({act}) vs autograd")


def check_jagged_attention_backward_finite_differences(O):
    # directional derivatives of L = sum(dout * out), out from the brute force
    q, off, k, v = _fna_case(93, [2, 3], 3, 2, 3)
    rng = _rng(94)
    dout = rng.standard_normal(q.shape)
    h = 1e-6

    def loss(qq, kk, vv, act):
        out = _bf_jagged_attention(qq.tolist(), off.tolist(), kk.tolist(), vv.tolist(), 0.8, act)
        return sum(dout[r][a][d] * out[r][a][d] for r in range(len(out)) for a in range(2) for d in range(3))

    for act in ("softmax", "gelu"):
        grads = O.jagged_attention_backward(q, off, k, v, dout, 0.8, act)
        for which, (a, g) in enumerate(zip((q, k, v), grads)):
            for _ in range(2):
                e = rng.standard_normal(a.shape)
                args_p = [q, k, v]; args_m = [q, k, v]
                args_p[which] = a + h * e; args_m[which] = a - h * e
                fd = (loss(*args_p, act) - loss(*args_m, act)) / (2 * h)
                assert abs(fd - float(np.sum(g * e))) <= 1e-6 * (1.0 + abs(fd)), (act, which, fd)


def check_jagged_attention_backward_invariants(O):
    q, off, k, v = _fna_case(95, [3, 5, 0], 6, 2, 4)
    dout = _rng(96).standard_normal(q.shape)
    for act in ("softmax", "gelu"):
        dq, dk, dv = O.jagged_attention_backward(q, off, k, v, dout, 0.6, act)
        assert np.all(dk[2] == 0.0) and np.all(dv[2] == 0.0)  # the empty batch
        z = O.jagged_attention_backward(q, off, k, v, np.zeros_like(dout), 0.6, act)
        assert all(np.all(a == 0.0) for a in z)
    # softmax: a vector added to every key shifts each score row by a constant,
    # so the key gradients sum to zero; a value row's gradient sums the
    # probabilities of that key times dout, and the probabilities of a row sum
    # to one, so sum over keys of dv = sum over the batch's rows of dout
    dq, dk, dv = O.jagged_attention_backward(q, off, k, v, dout, 0.6, "softmax")
    _close(np.sum(dk, axis=1), np.zeros((3, 2, 4)), 1e-11, "softmax: key gradients sum to zero")
    for b in range(2):
        _close(np.sum(dv[b], axis=0), np.sum(dout[off[b]:off[b + 1]], axis=0), 1e-11,
               "softmax: value gradients sum to the rows' dout")
    # GELU with V = 0: the output is zero whatever q and k, so dq = dk = 0
    dq, dk, dv = O.jagged_attention_backward(q, off, k, np.zeros_like(v), dout, 0.6, "gelu")
    _close(dq, np.zeros_like(dq), 0.0, "V = 0: no query gradient")
    _close(dk, np.zeros_like(dk), 0.0, "V = 0: no key gradient")


def check_fna_backward_invariants(O):
    q, off, k, v = _fna_case(85, [3, 5, 0], 6, 2, 4)
    T, H, D = q.shape
    dout = _rng(86).standard_normal(q.shape)
    x = q.reshape(T, H * D)
    for act in ("softmax", "gelu"):
        dq, dk, dv = O.flash_norm_attention_backward(q, off, k, v, dout, 0.0, 1e-6, 0.6, act)
        # out - x depends on x only through layernorm(x): shifting x by a
        # constant, or scaling it (eps_ln = 0), leaves it unchanged
        dx = (dq - dout).reshape(T, H * D)
        _close(np.sum(dx, axis=1), np.zeros(T), 1e-11, f"{act}: LN part of dq sums to zero")
        _close(np.sum(dx * (x - x.mean(axis=1, keepdims=True)), axis=1), np.zeros(T), 1e-11,
               f"{act}: LN part of dq orthogonal to the centred row")
        # the empty batch gets no key or value gradient
        assert np.all(dk[2] == 0.0) and np.all(dv[2] == 0.0)
        # dout = 0: no gradient anywhere
        z = O.flash_norm_attention_backward(q, off, k, v, np.zeros_like(dout), 0.0, 1e-6, 0.6, act)
        assert all(np.all(a == 0.0) for a in z)
    # softmax: adding one vector to every key shifts each score row by a
    # constant, which softmax ignores, so the key gradients sum to zero
    dq, dk, dv = O.flash_norm_attention_backward(q, off, k, v, dout, 1e-5, 1e-6, 0.6, "softmax")
    _close(np.sum(dk, axis=1), np.zeros((3, H, D)), 1e-11, "softmax: key gradients sum to zero")
    # V = 0 with GELU: the attention output is zero whatever the keys, so dk = 0
    dq, dk, dv = O.flash_norm_attention_backward(q, off, k, np.zeros_like(v), dout, 1e-5, 1e-6, 0.6, "gelu")
    _close(dk, np.zeros_like(dk), 0.0, "V = 0: no key gradient")


def check_compare(O):
    e = O.compare(np.array([1.0, 2.0]), np.array([1.0, 3.0]))
    assert abs(e["normwise_rel"] - 1.0 / 3.0) < 1e-15, e
    assert abs(e["mae"] - 0.5) < 1e-15, e
    assert abs(e["max_abs"] - 1.0) < 1e-15, e


ALL_CHECKS = [
    check_bf16_decode,
    check_rmsnorm_closed_form,
    check_rmsnorm_bruteforce,
    check_rmsnorm_invariants,
    check_rmsnorm_torch,
    check_layernorm_closed_form,
    check_layernorm_bruteforce,
    check_layernorm_invariants,
    check_layernorm_torch,
    check_prenorm_gemm_bruteforce,
    check_prenorm_gemm_identities,
    check_prenorm_gemm_torch,
    check_prenorm_ln_gemm,
    check_postnorm_bruteforce,
    check_postnorm_identities,
    check_postnorm_torch,
    check_postnorm_affine,
    check_attention_bruteforce,
    check_attention_torch,
    check_attention_closed_forms,
    check_gelu,
    check_fna_bruteforce,
    check_fna_torch,
    check_fna_closed_forms,
    check_jagged_attention,
    check_norm_backward_torch,
    check_norm_backward_finite_differences,
    check_norm_backward_invariants,
    check_gemm_postnorm_backward_torch,
    check_prenorm_backward_torch,
    check_prenorm_backward_dw_torch,
    check_prenorm_backward_dw_bruteforce,
    check_prenorm_backward_dw_invariants,
    check_fna_backward_torch,
    check_fna_backward_finite_differences,
    check_fna_backward_invariants,
    check_jagged_attention_backward_torch,
    check_jagged_attention_backward_finite_differences,
    check_jagged_attention_backward_invariants,
    check_compare,
]


def failing_checks(O):
    """Names of the checks that fail for oracle module/namespace O."""
    bad = []
    for chk in ALL_CHECKS:
        try:
            chk(O)
        except AssertionError:
            bad.append(chk.__name__)
        except Exception:  # a mutant may crash a check outright: also a catch
            bad.append(chk.__name__)
    return bad
