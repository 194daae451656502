"""Helpers for the GPU parity tests: host<->device copies of bf16 bit arrays and
the agreed tolerance (bf16 outputs within normwise max relative error 1e-2 and
mean absolute error 2e-3 of the fp64 oracle)."""

import sys

import numpy as np
import torch

import oracle

MAX_REL = 1e-2
MAE = 2e-3


def log(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def dev(bits):
    """uint16 bf16 bit array -> contiguous bf16 device tensor."""
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).to("cuda").view(torch.bfloat16)


def host(t):
    """bf16 device tensor -> float64 numpy (exact decode by the oracle)."""
    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.bf16_to_f64(bits)


def empty_bf16(*shape, poison=True):
    t = torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
    if poison:
        t.view(torch.int16).fill_(0x7FC0)  # NaN: an unwritten output element fails the check
    return t


def assert_parity(y, ref, what, max_rel=MAX_REL, mae=MAE):
    e = oracle.compare(y, ref)
    log(f"{what}: normwise_rel={e['normwise_rel']:.3e} mae={e['mae']:.3e} max_abs={e['max_abs']:.3e}")
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert e["normwise_rel"] <= max_rel, (what, e)
    assert e["mae"] <= mae, (what, e)
    return e


def assert_close_stats(got, want, what, rtol=2e-4):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rel = np.max(np.abs(got - want) / np.maximum(np.abs(want), 1e-30))
    log(f"{what}: max rel {rel:.3e}")
    assert rel <= rtol, (what, rel)


def bf16_floor(ref):
    """MAE of the exact result rounded to bf16 (nearest even): what a bf16
    output costs by itself, before any arithmetic error."""
    ref = np.ascontiguousarray(ref, dtype=np.float64)
    r = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    return float(np.mean(np.abs(r - ref)))


FLOOR_MARGIN = 1e-3


def assert_parity_floor(y, ref, what, margin=FLOOR_MARGIN):
    """The agreed gate for outputs that are not unit-scale (gradients,
    residual outputs): normwise max relative error <= 1e-2, and a mean
    absolute error within `margin` of the bf16 rounding floor of the exact
    result, never looser than 2e-3 scaled by the output's mean magnitude over
    0.8 (the mean magnitude of a unit normal)."""
    floor = bf16_floor(ref)
    scaled = MAE * max(1.0, float(np.mean(np.abs(ref))) / 0.8)
    bound = min(scaled, floor + margin)
    e = assert_parity(y, ref, what, mae=bound)
    log(f"{what}: bf16 floor mae={floor:.3e} excess={e['mae'] - floor:.3e} bound={bound:.3e}")
    return e
