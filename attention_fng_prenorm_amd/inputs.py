"""Seeded synthetic inputs for the fused-normalization workloads.

This module only draws random numbers and rounds them to bf16 bit patterns;
it holds none of the normalisation, GEMM or attention arithmetic, so both the
HIP path and the fp64 oracle can consume its output without sharing method
code.

Recipe (all draws from numpy.random.Generator(PCG64(seed)), float32, then
round-to-nearest-even to bf16 on the host; the same bf16 bits feed both
sides).  "N(mu, v)" is mean and *variance*:

  prenorm_rms_small   X[256,128] ~ N(0,1), W[128,128] ~ N(0,1/128), eps 1e-6
  postnorm_ln_smalln  X[8192,256] ~ N(0,1), W[256,256] ~ N(0,1/256), eps 1e-5
  prenorm_rms_mlp     X[4096,4096] = exp(xi_m) * z[m,k], xi, z ~ N(0,1);
                      W[4096,14336] ~ N(0,1/4096), eps 1e-6
  prenorm_rms_mlp_gamma  as above plus gamma[4096] ~ N(1, 0.1)
  prenorm_ln_mlp      lazy LayerNorm pre-norm (an extension, not a page workload):
                      X[4096,4096] = exp(xi_m) * (z[m,k] + mu_m), xi, z ~ N(0,1),
                      mu ~ N(0, 4) (rows off zero mean, |mu|/spread up to ~8);
                      W[4096,14336] ~ N(0,1/4096), eps 1e-5
  postnorm_rms_largen X[16384,1024] ~ N(0,1), W[1024,4096] ~ N(0,1/1024),
                      eps 1e-6
  norm_attention      Q, K, V [32,1024,4,128] (BSHD) ~ N(0,1),
                      eps_ln 1e-5, eps_rms 1e-6, sm_scale 1/sqrt(128)
  flash_norm_attention  768 batches; per-batch query length uniform on
                      1..512 (mean 256.5: the pages' average sparsity 0.5 of
                      the maximum length); Q [sum of lengths, 4, 128] jagged,
                      K, V [768, 128, 4, 128] dense, all ~ N(0,1); eps_ln 1e-5,
                      eps_rms 1e-6, sm_scale 1/sqrt(128), GELU activation
  flash_norm_attention_bwd  as flash_norm_attention (seed 1016), plus the
                      output gradient dOut [T, 4, 128] ~ N(0,1) drawn after V

Backward (section 3's fusion regrouping; shapes of the forward workloads):
  postnorm_ln_smalln_bwd   G[8192,256] ~ N(0,1), Wt[256,256] ~ N(0,1/256),
                           Y[8192,256] ~ N(0,1) (the forward output),
                           rstd[8192] = exp(N(0, 0.25)) (fp32)
  postnorm_rms_largen_bwd  G[16384,1024], Wt[1024,4096] ~ N(0,1/1024),
                           Y[16384,4096], rstd[16384], as above
  prenorm_rms_mlp_bwd_dx   dY[4096,14336] ~ N(0,1), Wt[14336,4096] ~
                           N(0,1/14336), X[4096,4096] with log-normal row
                           scales (as the forward), rstd[4096] as above
  prenorm_rms_mlp_dw       the weight gradient: X[4096,4096] with log-normal
                           row scales, dY[4096,14336] ~ N(0,1) (seed 1033);
                           _gamma adds gamma[4096] ~ N(1, 0.1) (seed 1043);
                           rstd is the forward's, computed from X
  The saved tensors and statistics are drawn independently of each other:
  the backward is a function of them, whatever produced them.

Draw order inside one generator: X (row scales, then row shifts, first when
present), W,
gamma; for attention Q, K, V; for the jagged attention the lengths, then Q,
K, V (then dOut for the backward).
"""

import math

import numpy as np


# Workload table.  "kind" selects the operation; sizes may be overridden for
# reduced-size parity cases (the recipe above stays the same).
WORKLOADS = {
    "prenorm_rms_small": dict(kind="prenorm_rms", M=256, K=128, N=128, eps=1e-6,
                              x_dist="normal", gamma=False, seed=1001),
    "postnorm_ln_smalln": dict(kind="postnorm_ln", M=8192, K=256, N=256, eps=1e-5,
                               x_dist="normal", gamma=False, seed=1002),
    "prenorm_rms_mlp": dict(kind="prenorm_rms", M=4096, K=4096, N=14336, eps=1e-6,
                            x_dist="lognormal_rows", gamma=False, seed=1003),
    "prenorm_rms_mlp_gamma": dict(kind="prenorm_rms", M=4096, K=4096, N=14336, eps=1e-6,
                                  x_dist="lognormal_rows", gamma=True, seed=1013),
    "prenorm_ln_mlp": dict(kind="prenorm_ln", M=4096, K=4096, N=14336, eps=1e-5,
                           x_dist="lognormal_rows_shifted", gamma=False, seed=1024),
    "postnorm_rms_largen": dict(kind="postnorm_rms", M=16384, K=1024, N=4096, eps=1e-6,
                                x_dist="normal", gamma=False, seed=1004),
    "norm_attention": dict(kind="norm_attention", B=32, Sq=1024, Skv=1024, H=4, D=128,
                           eps_ln=1e-5, eps_rms=1e-6, seed=1005),
    "postnorm_ln_smalln_bwd": dict(kind="norm_bwd", M=8192, K=256, N=256, norm="ln", h_dist="normal",
                                   seed=1012),
    "postnorm_rms_largen_bwd": dict(kind="norm_bwd", M=16384, K=1024, N=4096, norm="rms", h_dist="normal",
                                    seed=1014),
    "prenorm_rms_mlp_bwd_dx": dict(kind="norm_bwd", M=4096, K=14336, N=4096, norm="rms",
                                   h_dist="lognormal_rows", seed=1023),
    "prenorm_rms_mlp_dw": dict(kind="prenorm_dw", M=4096, K=4096, N=14336, eps=1e-6, gamma=False, seed=1033),
    "prenorm_rms_mlp_dw_gamma": dict(kind="prenorm_dw", M=4096, K=4096, N=14336, eps=1e-6, gamma=True,
                                     seed=1043),
    "flash_norm_attention": dict(kind="flash_norm_attention", B=768, max_len=512, Skv=128, H=4,
                                 D=128, eps_ln=1e-5, eps_rms=1e-6, act="gelu", seed=1006),
    "flash_norm_attention_bwd": dict(kind="flash_norm_attention", B=768, max_len=512, Skv=128, H=4,
                                     D=128, eps_ln=1e-5, eps_rms=1e-6, act="gelu", dout=True, seed=1016),
}


def f32_to_bf16_bits(a):
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns to float32 (exact); for host-side checks."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _normal(rng, shape, var=1.0, mean=0.0):
    z = rng.standard_normal(size=shape, dtype=np.float32)
    if var != 1.0:
        z *= np.float32(math.sqrt(var))
    if mean != 0.0:
        z += np.float32(mean)
    return z


def workload(name, **overrides):
    """The workload spec for `name`, with sizes or seed overridden."""
    if name not in WORKLOADS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    spec["name"] = name
    return spec


def make_gemm_inputs(spec):
    """Inputs of a norm+GEMM workload as bf16 bit arrays: dict X, W, gamma."""
    rng = np.random.Generator(np.random.PCG64(spec["seed"]))
    M, K, N = spec["M"], spec["K"], spec["N"]
    if spec["x_dist"] == "normal":
        x = _normal(rng, (M, K))
    elif spec["x_dist"] == "lognormal_rows":
        s = np.exp(_normal(rng, (M, 1)))
        x = s * _normal(rng, (M, K))
    elif spec["x_dist"] == "lognormal_rows_shifted":
        s = np.exp(_normal(rng, (M, 1)))
        mu = _normal(rng, (M, 1), var=spec.get("shift_var", 4.0))
        x = s * (_normal(rng, (M, K)) + mu)
    else:
        raise ValueError(spec["x_dist"])
    w = _normal(rng, (K, N), var=1.0 / K)
    out = {"X": f32_to_bf16_bits(x), "W": f32_to_bf16_bits(w), "gamma": None}
    if spec.get("gamma"):
        out["gamma"] = f32_to_bf16_bits(_normal(rng, (K,), var=0.1, mean=1.0))
    return out


def make_attention_inputs(spec):
    """Q, K, V of the attention workload as bf16 bit arrays (BSHD)."""
    rng = np.random.Generator(np.random.PCG64(spec["seed"]))
    B, Sq, Skv, H, D = spec["B"], spec["Sq"], spec["Skv"], spec["H"], spec["D"]
    q = f32_to_bf16_bits(_normal(rng, (B, Sq, H, D)))
    k = f32_to_bf16_bits(_normal(rng, (B, Skv, H, D)))
    v = f32_to_bf16_bits(_normal(rng, (B, Skv, H, D)))
    return {"Q": q, "K": k, "V": v}


def make_jagged_attention_inputs(spec):
    """Jagged queries and dense keys/values: dict Q [T,H,D] bf16 bits, K, V
    [B,Skv,H,D] bf16 bits, offsets [B+1] int32 (row offsets of each batch).
    A spec entry "lengths" (a list) fixes the per-batch lengths instead of
    drawing them."""
    rng = np.random.Generator(np.random.PCG64(spec["seed"]))
    B, Skv, H, D = spec["B"], spec["Skv"], spec["H"], spec["D"]
    if spec.get("lengths") is not None:
        lengths = np.asarray(spec["lengths"], dtype=np.int64)
    else:
        lengths = rng.integers(1, spec["max_len"] + 1, size=B)
    offsets = np.zeros(B + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(lengths)
    T = int(offsets[-1])
    q = f32_to_bf16_bits(_normal(rng, (T, H, D)))
    k = f32_to_bf16_bits(_normal(rng, (B, Skv, H, D)))
    v = f32_to_bf16_bits(_normal(rng, (B, Skv, H, D)))
    out = {"Q": q, "K": k, "V": v, "offsets": offsets}
    if spec.get("dout"):
        out["dOut"] = f32_to_bf16_bits(_normal(rng, (T, H, D)))
    return out


def make_norm_bwd_inputs(spec):
    """Inputs of a regrouped norm backward dZ = norm_bwd(G @ Wt) over N:
    dict G [M,K], Wt [K,N], H [M,N] bf16 bits (the saved forward output, or
    the norm's input for the lazy pre-norm), rstd [M] float32.  Sizes are
    those of the product (for the pre-norm input gradient, K is the forward's
    N and N the forward's K)."""
    rng = np.random.Generator(np.random.PCG64(spec["seed"]))
    M, K, N = spec["M"], spec["K"], spec["N"]
    g = _normal(rng, (M, K))
    w = _normal(rng, (K, N), var=1.0 / K)
    if spec["h_dist"] == "lognormal_rows":
        s = np.exp(_normal(rng, (M, 1)))
        h = s * _normal(rng, (M, N))
    else:
        h = _normal(rng, (M, N))
    rstd = np.exp(_normal(rng, (M,), var=0.25)).astype(np.float32)
    return {"G": f32_to_bf16_bits(g), "Wt": f32_to_bf16_bits(w), "H": f32_to_bf16_bits(h), "rstd": rstd}


def make_dw_inputs(spec):
    """Inputs of the lazy pre-RMSNorm weight gradient: dict X [M,K] bf16 bits
    with log-normal row scales (the forward's recipe), dY [M,N] ~ N(0,1), gamma
    [K] ~ N(1, 0.1) or None."""
    rng = np.random.Generator(np.random.PCG64(spec["seed"]))
    M, K, N = spec["M"], spec["K"], spec["N"]
    s = np.exp(_normal(rng, (M, 1)))
    x = s * _normal(rng, (M, K))
    dy = _normal(rng, (M, N))
    g = _normal(rng, (K,), var=0.1, mean=1.0) if spec.get("gamma") else None
    return {"X": f32_to_bf16_bits(x), "dY": f32_to_bf16_bits(dy),
            "gamma": f32_to_bf16_bits(g) if g is not None else None}


def make_inputs(name, **overrides):
    """Spec and inputs for workload `name` (see the recipe in the header)."""
    spec = workload(name, **overrides)
    if spec["kind"] == "norm_attention":
        return spec, make_attention_inputs(spec)
    if spec["kind"] == "flash_norm_attention":
        return spec, make_jagged_attention_inputs(spec)
    if spec["kind"] == "norm_bwd":
        return spec, make_norm_bwd_inputs(spec)
    if spec["kind"] == "prenorm_dw":
        return spec, make_dw_inputs(spec)
    return spec, make_gemm_inputs(spec)


# Degenerate rows for the edge-case parity tests.  Each kind replaces whole
# rows (the last axis, or the last two for [T, H, D] query tensors, so that a
# "row" is everything one normalization sees) with values drawn from its own
# generator PCG64(seed):
#   zero     all zeros
#   const    one value c ~ N(0, 1) repeated over the row (a nonzero draw)
#   tiny     z * sqrt(eps), z ~ N(0, 1): mean square about eps
#   shifted  z + mu, z ~ N(0, 1), mu = +/- shift (rows far off zero mean)
#   huge     z * 2^12 (mean square about 2^24)
ROW_KINDS = ("zero", "const", "tiny", "shifted", "huge")


def plant_rows(bits, rows, kinds, seed, eps=1e-6, shift=24.0, row_dims=1):
    """Copy of the bf16 bit array `bits` with rows[i] replaced by a row of kind
    kinds[i % len(kinds)] (see ROW_KINDS).  row_dims: how many trailing axes
    form one row.  Returns (new bits, dict kind -> list of row indices)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.array(bits, copy=True)
    lead = out.shape[: out.ndim - row_dims]
    flat = out.reshape(int(np.prod(lead)), -1)
    n = flat.shape[1]
    where = {k: [] for k in ROW_KINDS}
    for i, r in enumerate(rows):
        kind = kinds[i % len(kinds)]
        if kind == "zero":
            v = np.zeros(n, dtype=np.float32)
        elif kind == "const":
            c = np.float32(0.0)
            while c == 0.0:
                c = _normal(rng, ())
            v = np.full(n, c, dtype=np.float32)
        elif kind == "tiny":
            v = _normal(rng, (n,)) * np.float32(math.sqrt(eps))
        elif kind == "shifted":
            v = _normal(rng, (n,)) + np.float32(shift if rng.integers(0, 2) else -shift)
        elif kind == "huge":
            v = _normal(rng, (n,)) * np.float32(4096.0)
        else:
            raise ValueError(kind)
        flat[r] = f32_to_bf16_bits(v)
        where[kind].append(int(r))
    return flat.reshape(out.shape), where
