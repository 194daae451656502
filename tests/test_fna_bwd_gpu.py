"""GPU parity of the FlashNormAttention backward (fng_flash_norm_attention_bwd,
called through the C ABI after the forward kernel, as in training) against
the fp64 oracle's gradients on seeded bf16 inputs: jagged query batches with
empty, single-row, tile-straddling and maximum lengths, key counts that leave
a ragged last key tile, one, two, four and eight heads, softmax and GELU.

The forward's output and statistics come from the forward kernel (the
backward rebuilds the LayerNorm output and the RMSNorm output from them, as
the page does); the oracle recomputes everything from Q, K, V and dOut in
fp64.  The softmax case with a single key is the sharp one: there the exact
dK is zero, so any inconsistency between P, dP and the row term shows.

Tolerance: normwise max relative error <= 1e-2, and a mean absolute error
within GRAD_MARGIN of the bf16 rounding floor of the exact gradient (never
looser than 2e-3 scaled by the gradient's mean magnitude over 0.8: dQ
carries dOut through the second residual, mean |dQ| is about 1.1; GELU's dV
sums O(1) activations over up to 512 rows)."""

import math

import numpy as np
import pytest
import torch

import oracle
from attention_fng_prenorm_amd import binding as B
from attention_fng_prenorm_amd import inputs
from gpu_util import assert_parity_floor, dev, empty_bf16, host, log

pytestmark = pytest.mark.gpu

LENGTHS = [0, 1, 300, 37, 256, 65, 0, 129, 64, 128]
SCALE = 1.0 / math.sqrt(128)
# the mean absolute error may exceed the bf16 rounding floor of the exact
# gradient by at most this much (measured excess on these inputs: dQ up to
# 1e-4, dK and dV up to about 2e-4, more for dK with a single key)
GRAD_MARGIN = 1e-3


def f64(bits):
    return oracle.bf16_to_f64(bits)


def grad_parity(y, ref, what):
    return assert_parity_floor(y, ref, what, margin=GRAD_MARGIN)


def case(H, Skv, lengths=LENGTHS, seed=21):
    spec, d = inputs.make_inputs("flash_norm_attention_bwd", B=len(lengths), H=H, Skv=Skv,
                                 lengths=list(lengths), max_len=max(max(lengths), 1), seed=seed)
    return spec, d


def run(d, max_len, act, eps_ln=1e-5, eps_rms=1e-6, T_extra=0):
    """Forward then backward on the device; returns dQ, dK, dV (dQ rows
    outside the processed batches keep their NaN poison)."""
    Q, K, V, dO = dev(d["Q"]), dev(d["K"]), dev(d["V"]), dev(d["dOut"])
    T, H, D = Q.shape
    if T_extra:
        pad = torch.zeros(T_extra, H, D, dtype=torch.bfloat16, device="cuda")
        Q, dO = torch.cat([Q, pad]), torch.cat([dO, pad])
    off = torch.from_numpy(np.ascontiguousarray(d["offsets"])).to("cuda")
    out = empty_bf16(*Q.shape)
    st = [torch.zeros(Q.shape[0], dtype=torch.float32, device="cuda") for _ in range(3)]
    B.fng_flash_norm_attention(Q, off, K, V, out, max_len, eps_ln, eps_rms, SCALE, act, *st)
    dQ, dK, dV = empty_bf16(*Q.shape), empty_bf16(*K.shape), empty_bf16(*V.shape)
    ws = torch.empty(B.fng_flash_norm_attention_bwd_workspace_bytes(Q.shape[0], H), dtype=torch.uint8,
                     device="cuda")
    B.fng_flash_norm_attention_bwd(Q, off, K, V, out, dO, st[0], st[1], st[2], dQ, dK, dV, max_len,
                                   workspace=ws, sm_scale=SCALE, act=act)
    torch.cuda.synchronize()
    return dQ, dK, dV


def check(d, dQ, dK, dV, act, what, rows=None, eps_ln=1e-5, eps_rms=1e-6):
    off = d["offsets"]
    rq, rk, rv = oracle.flash_norm_attention_backward(f64(d["Q"]), off, f64(d["K"]), f64(d["V"]),
                                                      f64(d["dOut"]), eps_ln, eps_rms, SCALE, act)
    owned = np.concatenate([np.arange(off[b], off[b + 1]) for b in range(len(off) - 1)]).astype(np.int64)
    grad_parity(host(dQ)[owned], rq[owned], f"{what} dQ")
    grad_parity(host(dK), rk, f"{what} dK")
    grad_parity(host(dV), rv, f"{what} dV")


@pytest.mark.parametrize("act", ["softmax", "gelu"])
@pytest.mark.parametrize("H", [1, 2, 4, 8])
def test_fna_bwd_reduced(H, act):
    spec, d = case(H, 72)
    log(f"fna bwd H={H} act={act} lengths={LENGTHS} Skv=72")
    dQ, dK, dV = run(d, spec["max_len"], act)
    check(d, dQ, dK, dV, act, f"fna bwd H={H} {act}")


@pytest.mark.parametrize("Skv", [1, 32, 33, 128])
def test_fna_bwd_key_counts(Skv):
    lengths = [5, 70, 0, 3]
    for act in ("softmax", "gelu"):
        spec, d = case(4, Skv, lengths=lengths, seed=22)
        log(f"fna bwd Skv={Skv} act={act}")
        dQ, dK, dV = run(d, spec["max_len"], act)
        check(d, dQ, dK, dV, act, f"fna bwd Skv={Skv} {act}")


def test_fna_bwd_truncated_and_unowned_rows():
    # rows past offsets[B] and rows a batch owns beyond max_len are not
    # written, and contribute nothing to dK, dV
    lengths = [40, 90, 7]
    spec, d = case(4, 48, lengths=lengths, seed=23)
    log("fna bwd max_len 64 with 5 unowned rows")
    dQ, dK, dV = run(d, 64, "gelu", T_extra=5)
    y = host(dQ)
    off = d["offsets"]
    cut = [min(n, 64) for n in lengths]
    owned = np.zeros(y.shape[0], dtype=bool)
    for b in range(len(lengths)):
        owned[off[b]:off[b] + cut[b]] = True
    assert np.all(np.isnan(y[~owned])), "a row outside the processed batches was written"
    rows = np.concatenate([np.arange(off[b], off[b] + cut[b]) for b in range(len(lengths))])
    d2 = dict(d, Q=d["Q"][rows], dOut=d["dOut"][rows], offsets=np.concatenate([[0], np.cumsum(cut)]))
    rq, rk, rv = oracle.flash_norm_attention_backward(f64(d2["Q"]), d2["offsets"], f64(d["K"]), f64(d["V"]),
                                                      f64(d2["dOut"]), 1e-5, 1e-6, SCALE, "gelu")
    grad_parity(y[rows], rq, "truncated dQ")
    grad_parity(host(dK), rk, "truncated dK")
    grad_parity(host(dV), rv, "truncated dV")


def test_fna_bwd_deterministic():
    spec, d = case(4, 72, seed=24)
    log("fna bwd determinism")
    a = run(d, spec["max_len"], "softmax")
    b = run(d, spec["max_len"], "softmax")
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_fna_bwd_no_rows():
    # no query row at all: dK and dV are still written, as zeros
    K = torch.randn(3, 16, 4, 128, device="cuda").to(torch.bfloat16)
    dK, dV = empty_bf16(*K.shape), empty_bf16(*K.shape)
    Q = empty_bf16(0, 4, 128)
    off = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.zeros(0, dtype=torch.float32, device="cuda")
    log("fna bwd T=0")
    B.fng_flash_norm_attention_bwd(Q, off, K, K, Q, Q, st, st, st, Q, dK, dV, 16, workspace=None)
    torch.cuda.synchronize()
    assert torch.all(dK.float() == 0) and torch.all(dV.float() == 0)


@pytest.fixture(scope="module")
def full_inputs():
    return inputs.make_inputs("flash_norm_attention_bwd")


@pytest.mark.parametrize("act", ["gelu", "softmax"])
def test_fna_bwd_full_size_sampled(full_inputs, act):
    spec, d = full_inputs
    off = d["offsets"]
    log(f"fna bwd full size B={spec['B']} T={off[-1]} Skv={spec['Skv']} H={spec['H']} act={act}")
    dQ, dK, dV = run(d, spec["max_len"], act, spec["eps_ln"], spec["eps_rms"])
    yq, yk, yv = host(dQ), host(dK), host(dV)
    lengths = np.diff(off)
    for b in [0, int(np.argmax(lengths)), int(np.argmin(lengths)), 383, spec["B"] - 1]:
        r0, r1 = int(off[b]), int(off[b + 1])
        rq, rk, rv = oracle.flash_norm_attention_backward(
            f64(d["Q"][r0:r1]), np.array([0, r1 - r0]), f64(d["K"][b:b + 1]), f64(d["V"][b:b + 1]),
            f64(d["dOut"][r0:r1]), spec["eps_ln"], spec["eps_rms"], SCALE, act)
        grad_parity(yq[r0:r1], rq, f"full size batch {b} (len {r1 - r0}) dQ")
        grad_parity(yk[b:b + 1], rk, f"full size batch {b} dK")
        grad_parity(yv[b:b + 1], rv, f"full size batch {b} dV")
    assert np.all(np.isfinite(yq)) and np.all(np.isfinite(yk)) and np.all(np.isfinite(yv))


# ---------------------------------------------------------------------------
# the plain jagged attention's backward (fng_jagged_attention_bwd): the
# unfused chain's attention step, the same kernels without the norm and
# residual terms, against oracle.jagged_attention_backward
# ---------------------------------------------------------------------------

def run_plain(d, max_len, act):
    Q, K, V, dO = dev(d["Q"]), dev(d["K"]), dev(d["V"]), dev(d["dOut"])
    off = torch.from_numpy(np.ascontiguousarray(d["offsets"])).to("cuda")
    dQ, dK, dV = empty_bf16(*Q.shape), empty_bf16(*K.shape), empty_bf16(*V.shape)
    ws = torch.empty(B.fng_flash_norm_attention_bwd_workspace_bytes(Q.shape[0], Q.shape[1]), dtype=torch.uint8,
                     device="cuda")
    B.fng_jagged_attention_bwd(Q, off, K, V, dO, dQ, dK, dV, max_len, workspace=ws, sm_scale=SCALE, act=act)
    torch.cuda.synchronize()
    return dQ, dK, dV


def check_plain(d, dQ, dK, dV, act, what):
    off = d["offsets"]
    rq, rk, rv = oracle.jagged_attention_backward(f64(d["Q"]), off, f64(d["K"]), f64(d["V"]), f64(d["dOut"]),
                                                  SCALE, act)
    owned = np.concatenate([np.arange(off[b], off[b + 1]) for b in range(len(off) - 1)]).astype(np.int64)
    grad_parity(host(dQ)[owned], rq[owned], f"{what} dQ")
    grad_parity(host(dK), rk, f"{what} dK")
    grad_parity(host(dV), rv, f"{what} dV")


@pytest.mark.parametrize("act", ["softmax", "gelu"])
@pytest.mark.parametrize("H", [1, 2, 4, 8])
def test_jagged_attention_bwd_reduced(H, act):
    spec, d = case(H, 72, seed=31)
    log(f"jagged attention bwd H={H} act={act} lengths={LENGTHS} Skv=72")
    dQ, dK, dV = run_plain(d, spec["max_len"], act)
    check_plain(d, dQ, dK, dV, act, f"jagged attention bwd H={H} {act}")


@pytest.mark.parametrize("Skv", [1, 33, 128])
def test_jagged_attention_bwd_key_counts(Skv):
    lengths = [5, 70, 0, 3]
    for act in ("softmax", "gelu"):
        spec, d = case(4, Skv, lengths=lengths, seed=32)
        log(f"jagged attention bwd Skv={Skv} act={act}")
        dQ, dK, dV = run_plain(d, spec["max_len"], act)
        check_plain(d, dQ, dK, dV, act, f"jagged attention bwd Skv={Skv} {act}")
