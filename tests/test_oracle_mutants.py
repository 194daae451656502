"""Planted mistakes in copies of the oracle (CPU only): each must fail a pin.

This shows the pins are strong enough that a plausible slip anywhere in the
oracle (a dropped term, a wrong axis or sign, a transposed operand, eps in the
wrong place, a biased/unbiased mix-up) does not go unnoticed.  The mistakes
live only in these in-memory copies; the real oracle is untouched.
"""

import types

import numpy as np
import pytest

import oracle
import oracle_pins
from oracle import fng_oracle as F


def _ns(**over):
    ns = types.SimpleNamespace(**{n: getattr(F, n) for n in dir(F) if not n.startswith("_")})
    for k, v in over.items():
        setattr(ns, k, v)
    # rebind the composite functions so they use the mutated pieces
    def prenorm_rms_gemm(x, w, eps, gamma=None):
        xn, r = ns.rmsnorm_rows(x, eps, gamma)
        return xn @ np.asarray(w, dtype=np.float64), r

    def gemm_postnorm(x, w, eps, kind):
        z = ns.gemm(x, w)
        if kind == "ln":
            return ns.layernorm_rows(z, eps)
        y, r = ns.rmsnorm_rows(z, eps)
        return y, None, r

    def norm_attention(q, k, v, eps_ln, eps_rms, sm_scale):
        q = np.asarray(q, dtype=np.float64)
        B, Sq, H, D = q.shape
        out = np.empty((B, Sq, H, np.shape(v)[-1]))
        mu_a = np.empty((B, Sq, H)); r1_a = np.empty((B, Sq, H)); r2_a = np.empty((B, Sq, H))
        for b in range(B):
            for h in range(H):
                qn, mu, r1 = ns.layernorm_rows(q[b, :, h, :], eps_ln)
                s = (qn @ np.asarray(k)[b, :, h, :].T) * sm_scale
                o = ns.softmax_rows(s) @ np.asarray(v)[b, :, h, :]
                y, r2 = ns.rmsnorm_rows(o, eps_rms)
                out[b, :, h, :] = y
                mu_a[b, :, h] = mu; r1_a[b, :, h] = r1; r2_a[b, :, h] = r2
        return out, mu_a, r1_a, r2_a

    def flash_norm_attention(q, offsets, k, v, eps_ln, eps_rms, sm_scale, act):
        return _fna(ns, q, offsets, k, v, eps_ln, eps_rms, sm_scale, act)

    def jagged_attention(q, offsets, k, v, sm_scale, act):
        return _jagged(ns, q, offsets, k, v, sm_scale, act)

    def gemm_postnorm_backward(dy2, w, y, rstd, kind):
        g = ns.gemm(dy2, w)
        return (ns.layernorm_backward_rows if kind == "ln" else ns.rmsnorm_backward_rows)(g, y, rstd)

    def prenorm_rms_backward_dx(dy, w, x, rstd):
        r = np.asarray(rstd, dtype=np.float64)
        return ns.rmsnorm_backward_rows(ns.gemm(dy, w), np.asarray(x, dtype=np.float64) * r[..., None], r)

    def gemm_postnorm_affine(x, w, eps, kind, gamma, beta=None):
        y, mu, r = gemm_postnorm(x, w, eps, kind)
        y = y * np.asarray(gamma, dtype=np.float64)[None, :]
        return (y + np.asarray(beta, dtype=np.float64)[None, :] if beta is not None else y), mu, r

    def prenorm_ln_gemm(x, w, eps):
        xn, mu, r = ns.layernorm_rows(x, eps)
        return xn @ np.asarray(w, dtype=np.float64), mu, r

    def activation_backward(s_, p, dp, act):
        if act == "softmax":
            return p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
        return dp * ns.gelu_tanh_grad(s_)

    def flash_norm_attention_backward(q, offsets, k, v, dout, eps_ln, eps_rms, sm_scale, act):
        return _fna_bwd(ns, q, offsets, k, v, dout, eps_ln, eps_rms, sm_scale, act)

    def jagged_attention_backward(q, offsets, k, v, dout, sm_scale, act):
        return _jagged_bwd(ns, q, offsets, k, v, dout, sm_scale, act)

    for name, fn in (("gemm_postnorm_affine", gemm_postnorm_affine), ("prenorm_ln_gemm", prenorm_ln_gemm), ("activation_backward", activation_backward),
                     ("flash_norm_attention_backward", flash_norm_attention_backward),
                     ("jagged_attention_backward", jagged_attention_backward),
                     ("prenorm_rms_gemm", prenorm_rms_gemm), ("gemm_postnorm", gemm_postnorm),
                     ("norm_attention", norm_attention), ("flash_norm_attention", flash_norm_attention),
                     ("jagged_attention", jagged_attention),
                     ("gemm_postnorm_backward", gemm_postnorm_backward),
                     ("prenorm_rms_backward_dx", prenorm_rms_backward_dx)):
        if name not in over:
            setattr(ns, name, fn)
    return ns


def _jagged(ns, q, offsets, k, v, sm_scale, act, kv_batch_shift=0, scale_after=False):
    """The jagged attention from the pieces in ns, with switches that plant
    mistakes: keys/values of another batch, the scale applied after the
    activation."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, H, D = q.shape
    nb = len(offsets) - 1
    out = np.zeros((T, H, v.shape[-1]))
    for b in range(nb):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 <= r0:
            continue
        bk = (b + kv_batch_shift) % nb
        for h in range(H):
            s = q[r0:r1, h, :] @ k[bk, :, h, :].T
            if not scale_after:
                s = s * sm_scale
            p = ns.softmax_rows(s) if act == "softmax" else ns.gelu_tanh(s)
            if scale_after:
                p = p * sm_scale
            out[r0:r1, h, :] = p @ v[bk, :, h, :]
    return out


def _fna(ns, q, offsets, k, v, eps_ln, eps_rms, sm_scale, act, ln_per_head=False, res1=True,
         res2="q", rms_per_head=False):
    """The full FlashNormAttention from the (possibly mutated) pieces in ns,
    with switches that plant structural mistakes."""
    q = np.asarray(q, dtype=np.float64)
    T, H, D = q.shape
    out = np.empty_like(q)
    mu_a, r1_a, r2_a = np.zeros(T), np.zeros(T), np.zeros(T)
    for b in range(len(offsets) - 1):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 <= r0:
            continue
        x = q[r0:r1]
        if ln_per_head:
            ln = np.stack([ns.layernorm_rows(x[:, h, :], eps_ln)[0] for h in range(H)], axis=1)
        else:
            ln, mu_a[r0:r1], r1_a[r0:r1] = ns.layernorm_rows(x.reshape(-1, H * D), eps_ln)
            ln = ln.reshape(-1, H, D)
        o = np.empty_like(ln)
        for h in range(H):
            s = (ln[:, h, :] @ np.asarray(k)[b, :, h, :].T) * sm_scale
            p = ns.softmax_rows(s) if act == "softmax" else ns.gelu_tanh(s)
            o[:, h, :] = p @ np.asarray(v)[b, :, h, :] + (ln[:, h, :] if res1 else 0.0)
        if rms_per_head:
            y = np.stack([ns.rmsnorm_rows(o[:, h, :], eps_rms)[0] for h in range(H)], axis=1)
        else:
            y = ns.rmsnorm_rows(o.reshape(-1, H * D), eps_rms)[0].reshape(-1, H, D)
        out[r0:r1] = y + (x if res2 == "q" else ln if res2 == "ln" else 0.0)
    return out, mu_a, r1_a, r2_a


def _fna_bwd(ns, q, offsets, k, v, dout, eps_ln, eps_rms, sm_scale, act, res1=True, res2=True,
             dk_scaled=True, dp_from_k=False, dv_from_ds=False, rms_xhat_is_o=False, ln_xhat_raw=False):
    """The FlashNormAttention backward from the (possibly mutated) pieces in
    ns, with switches that plant structural mistakes."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    T, H, D = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(offsets) - 1):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 <= r0:
            continue
        L = r1 - r0
        x = q[r0:r1].reshape(L, H * D)
        ln, _, rs1 = ns.layernorm_rows(x, eps_ln)
        ln = ln.reshape(L, H, D)
        s, p, o = [], [], np.empty_like(ln)
        for h in range(H):
            s.append((ln[:, h, :] @ k[b, :, h, :].T) * sm_scale)
            p.append(ns.softmax_rows(s[h]) if act == "softmax" else ns.gelu_tanh(s[h]))
            o[:, h, :] = p[h] @ v[b, :, h, :] + ln[:, h, :]
        y, rs2 = ns.rmsnorm_rows(o.reshape(L, H * D), eps_rms)
        g = dout[r0:r1].reshape(L, H * D)
        do = ns.rmsnorm_backward_rows(g, o.reshape(L, H * D) if rms_xhat_is_o else y, rs2).reshape(L, H, D)
        dln = do.copy() if res1 else np.zeros_like(do)
        for h in range(H):
            dp = do[:, h, :] @ (k if dp_from_k else v)[b, :, h, :].T
            ds = ns.activation_backward(s[h], p[h], dp, act)
            dv[b, :, h, :] = (ds if dv_from_ds else p[h]).T @ do[:, h, :]
            dln[:, h, :] += sm_scale * ds @ k[b, :, h, :]
            dk[b, :, h, :] = (sm_scale if dk_scaled else 1.0) * ds.T @ ln[:, h, :]
        dx = ns.layernorm_backward_rows(dln.reshape(L, H * D), x if ln_xhat_raw else ln.reshape(L, H * D), rs1)
        dq[r0:r1] = ((g if res2 else 0.0) + dx).reshape(L, H, D)
    return dq, dk, dv


def _ln_lazy_no_mean(x, w, eps):
    # the row scale alone, as if LayerNorm were lazy like RMSNorm
    xn, mu, r = F.layernorm_rows(x, eps)
    return (np.asarray(x, dtype=np.float64) * r[:, None]) @ np.asarray(w, dtype=np.float64), mu, r


def _ln_lazy_rank1_unscaled(x, w, eps):
    x = np.asarray(x, dtype=np.float64); w = np.asarray(w, dtype=np.float64)
    xn, mu, r = F.layernorm_rows(x, eps)
    return r[:, None] * (x @ w) - mu[:, None] * w.sum(axis=0)[None, :], mu, r


def _affine_before_norm(x, w, eps, kind, gamma, beta=None):
    # the gain applied to the product before the norm (which then undoes much of it)
    z = F.gemm(x, w) * np.asarray(gamma, dtype=np.float64)[None, :]
    y, mu, r = (F.layernorm_rows(z, eps) if kind == "ln" else (F.rmsnorm_rows(z, eps)[0], None, F.rmsnorm_rows(z, eps)[1]))
    return (y + np.asarray(beta, dtype=np.float64)[None, :] if beta is not None else y), mu, r


def _jagged_bwd(ns, q, offsets, k, v, dout, sm_scale, act, dk_scaled=True, dv_from_ds=False, dq_from_v=False):
    """The plain jagged attention backward from the pieces in ns, with
    switches that plant mistakes: dk without the scale, dv from ds instead of
    p, dq through the values instead of the keys."""
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(offsets) - 1):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 <= r0:
            continue
        for h in range(q.shape[1]):
            qh, kh, vh, gh = q[r0:r1, h, :], k[b, :, h, :], v[b, :, h, :], dout[r0:r1, h, :]
            s_ = (qh @ kh.T) * sm_scale
            p = ns.softmax_rows(s_) if act == "softmax" else ns.gelu_tanh(s_)
            ds = ns.activation_backward(s_, p, gh @ vh.T, act)
            dv[b, :, h, :] = (ds if dv_from_ds else p).T @ gh
            dq[r0:r1, h, :] = (ds * sm_scale) @ (vh if dq_from_v else kh)
            dk[b, :, h, :] = (ds * (sm_scale if dk_scaled else 1.0)).T @ qh
    return dq, dk, dv


def _jagged_bwd_mutant(**switches):
    def f(q, offsets, k, v, dout, sm_scale, act):
        return _jagged_bwd(F, q, offsets, k, v, dout, sm_scale, act, **switches)
    return f


def _fna_bwd_mutant(**switches):
    def f(q, offsets, k, v, dout, eps_ln, eps_rms, sm_scale, act):
        return _fna_bwd(F, q, offsets, k, v, dout, eps_ln, eps_rms, sm_scale, act, **switches)
    return f


def _softmax_bwd_no_row_term(s, p, dp, act):
    if act == "softmax":
        return p * dp
    return F.activation_backward(s, p, dp, act)


def _gelu_grad_first_term_only(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def _fna_mutant(**switches):
    def f(q, offsets, k, v, eps_ln, eps_rms, sm_scale, act):
        return _fna(F, q, offsets, k, v, eps_ln, eps_rms, sm_scale, act, **switches)
    return f


def _gelu_wrong_constant(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.44715 * x ** 3)))


def _rms_eps_outside(x, eps, gamma=None):
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / (np.sqrt(np.mean(x * x, axis=-1)) + eps)
    y = x * r[..., None]
    return (y * gamma if gamma is not None else y), r


def _rms_sum_not_mean(x, eps, gamma=None):
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.sum(x * x, axis=-1) / max(x.shape[-1] - 1, 1) + eps)
    y = x * r[..., None]
    return (y * gamma if gamma is not None else y), r


def _rms_gamma_in_stats(x, eps, gamma=None):
    x = np.asarray(x, dtype=np.float64)
    if gamma is not None:
        x = x * gamma
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * r[..., None], r


def _ln_unbiased(x, eps):
    x = np.asarray(x, dtype=np.float64)
    mu = np.mean(x, axis=-1)
    d = x - mu[..., None]
    var = np.sum(d * d, axis=-1) / (x.shape[-1] - 1)
    r = 1.0 / np.sqrt(var + eps)
    return d * r[..., None], mu, r


def _ln_eps_outside(x, eps):
    x = np.asarray(x, dtype=np.float64)
    mu = np.mean(x, axis=-1)
    d = x - mu[..., None]
    r = 1.0 / (np.sqrt(np.mean(d * d, axis=-1)) + eps)
    return d * r[..., None], mu, r


def _ln_no_center(x, eps):
    x = np.asarray(x, dtype=np.float64)
    mu = np.mean(x, axis=-1)
    d = x - mu[..., None]
    r = 1.0 / np.sqrt(np.mean(d * d, axis=-1) + eps)
    return x * r[..., None], mu, r


def _gemm_transposed(x, w):
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def _softmax_wrong_axis(s):
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=0, keepdims=True))
    return e / np.sum(e, axis=0, keepdims=True)


def _softmax_no_norm(s):
    s = np.asarray(s, dtype=np.float64)
    return np.exp(s - np.max(s, axis=-1, keepdims=True))


def _decode_wrong(bits):
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def _compare_wrong(y, ref):
    err = np.abs(np.asarray(y, np.float64) - np.asarray(ref, np.float64))
    return {"normwise_rel": float(np.max(err)), "mae": float(np.max(err)), "max_abs": float(np.max(err))}


def _attn_scale_divided(base):
    def f(q, k, v, eps_ln, eps_rms, sm_scale):
        return base(q, k, v, eps_ln, eps_rms, 1.0 / sm_scale)
    return f


def _attn_norm_k(q, k, v, eps_ln, eps_rms, sm_scale):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Sq, H, D = q.shape
    out = np.empty(q.shape[:3] + (np.shape(v)[-1],))
    z = np.zeros((B, Sq, H))
    for b in range(B):
        for h in range(H):
            kn, _, _ = F.layernorm_rows(k[b, :, h, :], eps_ln)
            s = (q[b, :, h, :] @ kn.T) * sm_scale
            o = F.softmax_rows(s) @ np.asarray(v)[b, :, h, :]
            out[b, :, h, :], _ = F.rmsnorm_rows(o, eps_rms)
    return out, z, z, z


def _attn_no_out_norm(q, k, v, eps_ln, eps_rms, sm_scale):
    q = np.asarray(q, dtype=np.float64)
    B, Sq, H, D = q.shape
    out = np.empty(q.shape[:3] + (np.shape(v)[-1],))
    z = np.zeros((B, Sq, H))
    for b in range(B):
        for h in range(H):
            qn, _, _ = F.layernorm_rows(q[b, :, h, :], eps_ln)
            s = (qn @ np.asarray(k)[b, :, h, :].T) * sm_scale
            out[b, :, h, :] = F.softmax_rows(s) @ np.asarray(v)[b, :, h, :]
    return out, z, z, z


def _ln_bwd_no_mean(g, xhat, rstd):
    g = np.asarray(g, dtype=np.float64); xhat = np.asarray(xhat, dtype=np.float64)
    return np.asarray(rstd)[..., None] * (g - xhat * np.mean(g * xhat, axis=-1, keepdims=True))


def _ln_bwd_sign(g, xhat, rstd):
    g = np.asarray(g, dtype=np.float64); xhat = np.asarray(xhat, dtype=np.float64)
    return np.asarray(rstd)[..., None] * (g - np.mean(g, axis=-1, keepdims=True) + xhat * np.mean(g * xhat, axis=-1, keepdims=True))


def _rms_bwd_with_mean(g, xhat, rstd):
    return F.layernorm_backward_rows(g, xhat, rstd)


def _rms_bwd_no_rstd(g, xhat, rstd):
    g = np.asarray(g, dtype=np.float64); xhat = np.asarray(xhat, dtype=np.float64)
    return g - xhat * np.mean(g * xhat, axis=-1, keepdims=True)


def _prenorm_dx_raw_xhat(dy, w, x, rstd):
    return F.rmsnorm_backward_rows(F.gemm(dy, w), x, rstd)


def _dw_rstd_on_columns(x, dy, rstd, gamma=None):
    # one scale for the whole batch in place of each row's own rstd
    x = np.asarray(x, dtype=np.float64)
    xg = x * np.asarray(gamma)[None, :] if gamma is not None else x
    return xg.T @ (np.asarray(dy) * np.mean(np.asarray(rstd)))


def _dw_no_rstd(x, dy, rstd, gamma=None):
    x = np.asarray(x, dtype=np.float64)
    xg = x * np.asarray(gamma)[None, :] if gamma is not None else x
    return xg.T @ np.asarray(dy, dtype=np.float64)


def _dw_gamma_on_columns(x, dy, rstd, gamma=None):
    xh = np.asarray(x, dtype=np.float64) * np.asarray(rstd)[:, None]
    out = xh.T @ np.asarray(dy, dtype=np.float64)
    if gamma is not None:
        out = out * np.resize(np.asarray(gamma), out.shape[1])[None, :]
    return out


def _dw_rstd_squared(x, dy, rstd, gamma=None):
    r = np.asarray(rstd, dtype=np.float64)
    return F.prenorm_rms_backward_dw(x, dy, r * r, gamma)


MUTANTS = {
    "dw_rstd_averaged_not_per_row": dict(prenorm_rms_backward_dw=_dw_rstd_on_columns),
    "dw_xhat_not_rebuilt": dict(prenorm_rms_backward_dw=_dw_no_rstd),
    "dw_gamma_on_columns": dict(prenorm_rms_backward_dw=_dw_gamma_on_columns),
    "dw_rstd_squared": dict(prenorm_rms_backward_dw=_dw_rstd_squared),
    "rms_eps_outside_sqrt": dict(rmsnorm_rows=_rms_eps_outside),
    "rms_divides_by_n_minus_1": dict(rmsnorm_rows=_rms_sum_not_mean),
    "rms_gamma_before_stats": dict(rmsnorm_rows=_rms_gamma_in_stats),
    "ln_unbiased_variance": dict(layernorm_rows=_ln_unbiased),
    "ln_eps_outside_sqrt": dict(layernorm_rows=_ln_eps_outside),
    "ln_missing_centering": dict(layernorm_rows=_ln_no_center),
    "gemm_transposed_w": dict(gemm=_gemm_transposed,
                              prenorm_rms_gemm=lambda x, w, eps, gamma=None: (
                                  F.rmsnorm_rows(x, eps, gamma)[0] @ np.asarray(w).T,
                                  F.rms_rstd(x, eps))),
    "softmax_over_queries": dict(softmax_rows=_softmax_wrong_axis),
    "softmax_unnormalised": dict(softmax_rows=_softmax_no_norm),
    "bf16_decode_shift": dict(bf16_to_f64=_decode_wrong),
    "compare_mae_is_max": dict(compare=_compare_wrong),
    "attn_scale_inverted": dict(norm_attention=_attn_scale_divided(F.norm_attention)),
    "attn_normalises_k": dict(norm_attention=_attn_norm_k),
    "attn_missing_out_rmsnorm": dict(norm_attention=_attn_no_out_norm),
    "fna_layernorm_per_head": dict(flash_norm_attention=_fna_mutant(ln_per_head=True)),
    "fna_rmsnorm_per_head": dict(flash_norm_attention=_fna_mutant(rms_per_head=True)),
    "fna_missing_residual_1": dict(flash_norm_attention=_fna_mutant(res1=False)),
    "fna_missing_residual_2": dict(flash_norm_attention=_fna_mutant(res2=None)),
    "fna_residual_2_adds_ln_q": dict(flash_norm_attention=_fna_mutant(res2="ln")),
    "gelu_cubic_constant_x10": dict(gelu_tanh=_gelu_wrong_constant),
    "ln_backward_drops_mean_term": dict(layernorm_backward_rows=_ln_bwd_no_mean),
    "ln_backward_wrong_sign": dict(layernorm_backward_rows=_ln_bwd_sign),
    "rms_backward_subtracts_mean": dict(rmsnorm_backward_rows=_rms_bwd_with_mean),
    "rms_backward_missing_rstd": dict(rmsnorm_backward_rows=_rms_bwd_no_rstd),
    "prenorm_dx_xhat_not_rebuilt": dict(prenorm_rms_backward_dx=_prenorm_dx_raw_xhat),
    "fna_bwd_missing_residual_1": dict(flash_norm_attention_backward=_fna_bwd_mutant(res1=False)),
    "fna_bwd_missing_residual_2": dict(flash_norm_attention_backward=_fna_bwd_mutant(res2=False)),
    "fna_bwd_dk_unscaled": dict(flash_norm_attention_backward=_fna_bwd_mutant(dk_scaled=False)),
    "fna_bwd_dp_from_keys": dict(flash_norm_attention_backward=_fna_bwd_mutant(dp_from_k=True)),
    "fna_bwd_dv_from_ds": dict(flash_norm_attention_backward=_fna_bwd_mutant(dv_from_ds=True)),
    "fna_bwd_rms_xhat_is_its_input": dict(flash_norm_attention_backward=_fna_bwd_mutant(rms_xhat_is_o=True)),
    "fna_bwd_ln_xhat_is_raw_x": dict(flash_norm_attention_backward=_fna_bwd_mutant(ln_xhat_raw=True)),
    "softmax_backward_drops_row_term": dict(activation_backward=_softmax_bwd_no_row_term),
    "jagged_bwd_dk_unscaled": dict(jagged_attention_backward=_jagged_bwd_mutant(dk_scaled=False)),
    "jagged_bwd_dv_from_ds": dict(jagged_attention_backward=_jagged_bwd_mutant(dv_from_ds=True)),
    "jagged_bwd_dq_from_values": dict(jagged_attention_backward=_jagged_bwd_mutant(dq_from_v=True)),
    "ln_lazy_without_mean_correction": dict(prenorm_ln_gemm=_ln_lazy_no_mean),
    "postnorm_affine_before_norm": dict(gemm_postnorm_affine=_affine_before_norm),
    "ln_lazy_rank1_term_unscaled": dict(prenorm_ln_gemm=_ln_lazy_rank1_unscaled),
    "gelu_grad_first_term_only": dict(gelu_tanh_grad=_gelu_grad_first_term_only),
    "jagged_kv_of_next_batch": dict(jagged_attention=lambda q, o, k, v, s, a: _jagged(
        oracle, q, o, k, v, s, a, kv_batch_shift=1)),
    "jagged_scale_after_activation": dict(jagged_attention=lambda q, o, k, v, s, a: _jagged(
        oracle, q, o, k, v, s, a, scale_after=True)),
}


def test_unmutated_copy_passes():
    assert oracle_pins.failing_checks(_ns()) == []
    assert oracle_pins.failing_checks(oracle) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    bad = oracle_pins.failing_checks(_ns(**MUTANTS[name]))
    assert bad, f"planted mistake {name} passed every pin"
