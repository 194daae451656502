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
