"""The fp64 oracle against its pins (CPU only)."""

import math

import numpy as np
import pytest

import oracle
import oracle_pins
from attention_fng_prenorm_amd import inputs


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_prenorm_small_full_size_bruteforce():
    """The small pre-RMSNorm workload at its full size (256x128 @ 128x128),
    oracle against pure-Python loops."""
    spec, d = inputs.make_inputs("prenorm_rms_small")
    x = oracle.bf16_to_f64(d["X"])
    w = oracle.bf16_to_f64(d["W"])
    y, r = oracle.prenorm_rms_gemm(x, w, spec["eps"])
    xn, br = oracle_pins.bf_rmsnorm(x.tolist(), spec["eps"])
    wl = w.tolist()
    M, K, N = spec["M"], spec["K"], spec["N"]
    ref = []
    for i in range(M):
        row = xn[i]
        out = [0.0] * N
        for k in range(K):
            a = row[k]
            wk = wl[k]
            for j in range(N):
                out[j] += a * wk[j]
        ref.append(out)
    assert np.max(np.abs(y - np.array(ref))) < 1e-12
    assert np.max(np.abs(r - np.array(br))) < 1e-13


def test_input_rounding_is_rne():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6
    # 1 + 2^-8 + 2^-20 is above halfway -> 1 + 2^-7
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                     -(1.0 + 2.0 ** -8), 0.0, 3.0], dtype=np.float32)
    bits = inputs.f32_to_bf16_bits(vals)
    assert [int(b) for b in bits] == [0x3F80, 0x3F82, 0x3F81, 0xBF80, 0x0000, 0x4040]
    assert np.isnan(oracle.bf16_to_f64(inputs.f32_to_bf16_bits(np.array([np.nan], np.float32)))[0])


@pytest.mark.parametrize("name", ["prenorm_rms_small", "postnorm_ln_smalln"])
def test_input_recipe_moments(name):
    spec, d = inputs.make_inputs(name)
    x = oracle.bf16_to_f64(d["X"])
    w = oracle.bf16_to_f64(d["W"])
    assert x.shape == (spec["M"], spec["K"]) and w.shape == (spec["K"], spec["N"])
    assert abs(np.mean(x)) < 0.02 and abs(np.var(x) - 1.0) < 0.03
    assert abs(np.var(w) * spec["K"] - 1.0) < 0.05


def test_input_recipe_lognormal_rows_and_gamma():
    spec, d = inputs.make_inputs("prenorm_rms_mlp_gamma", M=512, K=1024, N=64)
    x = oracle.bf16_to_f64(d["X"])
    # per-row log-scale: log(rms) ~ N(0, 1)
    lr = np.log(np.sqrt(np.mean(x * x, axis=1)))
    assert abs(np.mean(lr)) < 0.15 and abs(np.std(lr) - 1.0) < 0.1
    g = oracle.bf16_to_f64(d["gamma"])
    assert g.shape == (1024,)
    assert abs(np.mean(g) - 1.0) < 0.05 and abs(np.var(g) - 0.1) < 0.02


def test_inputs_are_deterministic():
    _, a = inputs.make_inputs("norm_attention", B=1, Sq=8, Skv=8, H=2)
    _, b = inputs.make_inputs("norm_attention", B=1, Sq=8, Skv=8, H=2)
    for key in "QKV":
        assert np.array_equal(a[key], b[key])
    assert not np.array_equal(a["Q"], a["K"])
