"""Plain fp64 CPU oracle for the fused-normalization hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
and imports nothing from the product package.

Every function is the plain mathematical definition written out in numpy
float64, with no blocking, fusion or reordering: the fused kernels reach the
same real-number result because

  * Lazy Pre-Norm only moves a row scale across a matrix product
    ("Towards Free Normalization: Fusing Normalization into GEMM and Attention
    Kernels", section 2, the row-scale commutation identity and its proof);
  * the multi-CTA / split-N post-norm only re-associates a per-row sum
    (same page, section 3, the reduction/elementwise decomposition);
  * FlashNormAttention only re-orders a normalise -> attend -> normalise chain
    (same page, section 4, the fused short-KV pseudocode).

So the oracle is the definition, evaluated in fp64 on the exact bf16 inputs,
with nothing rounded inside it.

Readings of points the page leaves open (each also listed in the design notes):
  * eps sits inside the square root and is an argument (section 2 writes the
    rstd with eps inside the rsqrt).
  * RMS divides by the length of the normalised axis (section 2 divides by the
    last dimension of A).
  * LayerNorm uses the biased (population) variance and no affine, as
    torch.nn.LayerNorm does (linked from the introduction's note on affines;
    benchmarks there disable affines).
  * lazy LayerNorm pre-norm (an extension the page rules out for lazy
    application): the plain definition layernorm(X) @ W; the kernel applies
    it as the rank-1 correction diag(rstd) (X W - mu colsum(W)).
  * the optional RMSNorm gain gamma multiplies after normalisation
    (y = rmsnorm(x) * gamma), then the product with W follows.
  * attention: per (batch, head) LayerNorm of each query row over head_dim,
    scores scaled by sm_scale after the product, max-subtracted softmax over
    all keys (non-causal, no mask), product with V, then RMSNorm of each output
    row over head_dim; K and V are not normalised; layout BSHD (section 4's
    pseudocode header gives [batch, seq, H, head_dim]).
  * full FlashNormAttention (section 4's fused short-KV kernel as written):
    LayerNorm of each query row across all heads (H*head_dim values), the
    scores of each head scaled by sm_scale after the product (the pseudocode
    shows no scale: sm_scale = 1 reproduces it literally), an activation that
    is either the max-subtracted softmax over the keys or the elementwise GELU
    in its tanh form (the pseudocode names a generic elementwise activation),
    the first residual adds the normalised query to the attention output, the
    RMSNorm runs across all heads, the second residual adds the raw query.
    Query rows are jagged (per-batch lengths given by offsets), keys dense.
  * backward (section 3's fusion regrouping): the norm's input gradient is
    the textbook closed form of the derivative of LayerNorm / RMSNorm (no
    affine), applied row-wise to the upstream gradient, which is the product
    of the next layer's output gradient with that layer's weight; the
    normalized values come from the forward (the norm's output, or for the
    lazy pre-norm rebuilt as x * rstd from its input and statistic).
  * FlashNormAttention backward (section 4, "Backward implementation"): the
    gradients of the forward above with respect to q, k and v, by the chain
    rule (RMSNorm backward, the two residuals, the attention backward with
    the softmax Jacobian or the derivative of the tanh-form GELU, LayerNorm
    backward across all heads).  The page keeps the norm statistics from the
    forward and recomputes the LayerNorm output and the RMSNorm output and
    input; the oracle recomputes the whole forward from q, k and v in fp64.
"""

import numpy as np


# ---------------------------------------------------------------------------
# exact bf16 decoding (input plumbing, not arithmetic of the method)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits):
    """Decode raw bf16 bit patterns (uint16/int16 array) to float64, exactly.

    A bf16 value is the upper 16 bits of an IEEE binary32; widening the bit
    pattern by 16 zero bits gives the identical binary32 value, which converts
    to binary64 without rounding.
    """
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# row normalisations (section 2's rstd; section 3's LayerNorm/RMSNorm)
# ---------------------------------------------------------------------------

def rms_rstd(x, eps):
    """rstd[m] = 1 / sqrt(mean_k x[m,k]^2 + eps)   (section 2, rstd(A))."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1)
    return 1.0 / np.sqrt(ms + eps)


def rmsnorm_rows(x, eps, gamma=None):
    """RMSNorm over the last axis: y = x * rstd[:, None] (* gamma).

    Section 2: rmsnorm(A) = A * rstd(A)[:, None].  gamma is the optional
    elementwise gain (applied after the row scale).
    Returns (y, rstd).
    """
    x = np.asarray(x, dtype=np.float64)
    r = rms_rstd(x, eps)
    y = x * r[..., None]
    if gamma is not None:
        y = y * np.asarray(gamma, dtype=np.float64)
    return y, r


def layernorm_rows(x, eps):
    """LayerNorm over the last axis, no affine, biased variance.

    mu = mean(x); var = mean((x - mu)^2); y = (x - mu) / sqrt(var + eps).
    Returns (y, mean, rstd).
    """
    x = np.asarray(x, dtype=np.float64)
    mu = np.mean(x, axis=-1)
    d = x - mu[..., None]
    var = np.mean(d * d, axis=-1)
    r = 1.0 / np.sqrt(var + eps)
    return d * r[..., None], mu, r


# ---------------------------------------------------------------------------
# norm + GEMM (sections 1-3)
# ---------------------------------------------------------------------------

def prenorm_rms_gemm(x, w, eps, gamma=None):
    """Y = rmsnorm(X) @ W   (section 2, C = rmsnorm(A) @ B).

    X is [M, K], W is [K, N]; the RMS statistic is taken over K from the raw X
    (the gain, if any, is applied after the statistic).  Returns (Y, rstd[M]).
    """
    xn, r = rmsnorm_rows(x, eps, gamma)
    return xn @ np.asarray(w, dtype=np.float64), r


def gemm_postnorm_affine(x, w, eps, kind, gamma, beta=None):
    """Y = norm(X @ W) * gamma + beta over the N axis (the post-norm with its
    affine; section 1 notes the page's benchmarks run the norms without it).
    gamma [N]; beta [N] or None.  Returns (Y, mean[M] or None, rstd[M])."""
    y, mu, r = gemm_postnorm(x, w, eps, kind)
    y = y * np.asarray(gamma, dtype=np.float64)[None, :]
    if beta is not None:
        y = y + np.asarray(beta, dtype=np.float64)[None, :]
    return y, mu, r


def prenorm_ln_gemm(x, w, eps):
    """Y = layernorm(X) @ W over K (no affine; the lazy LayerNorm pre-norm).

    The page keeps lazy application to RMSNorm, whose elementwise part is a
    pure row scale; LayerNorm's subtraction of the row mean is a rank-1 term,
    layernorm(X) W = diag(rstd) (X W - mu 1^T W), which a kernel can apply
    after the product.  The oracle is the plain definition.  Returns
    (Y, mean[M], rstd[M]).
    """
    xn, mu, r = layernorm_rows(x, eps)
    return xn @ np.asarray(w, dtype=np.float64), mu, r


def gemm(x, w):
    """Z = X @ W, X [M, K], W [K, N]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)


def gemm_postnorm(x, w, eps, kind):
    """Y = norm(X @ W) over the N axis  (section 1 naive fusion and section 3
    multi-CTA fusion both compute this; statistics come from the exact
    product, i.e. the fp32 accumulator in a kernel, before output rounding).

    kind is "ln" or "rms".  Returns (Y, mean[M] or None, rstd[M]).
    """
    z = gemm(x, w)
    if kind == "ln":
        return layernorm_rows(z, eps)
    if kind == "rms":
        y, r = rmsnorm_rows(z, eps)
        return y, None, r
    raise ValueError(f"unknown norm kind {kind!r}")


# ---------------------------------------------------------------------------
# backward by fusion regrouping (section 3, "What about backward?")
# ---------------------------------------------------------------------------

def layernorm_backward_rows(g, xhat, rstd):
    """Gradient of LayerNorm (no affine, biased variance) with respect to its
    input, per row of the last axis, from the upstream gradient g, the
    normalized values xhat = (z - mean) * rstd and rstd:
        dz = rstd * (g - mean(g) - xhat * mean(g * xhat)).
    (Differentiate y = (z - mu) * rstd with mu and rstd functions of z.)
    """
    g = np.asarray(g, dtype=np.float64)
    xhat = np.asarray(xhat, dtype=np.float64)
    r = np.asarray(rstd, dtype=np.float64)[..., None]
    return r * (g - np.mean(g, axis=-1, keepdims=True) - xhat * np.mean(g * xhat, axis=-1, keepdims=True))


def rmsnorm_backward_rows(g, xhat, rstd):
    """Gradient of RMSNorm (no gain) with respect to its input, per row:
        dz = rstd * (g - xhat * mean(g * xhat)),  xhat = z * rstd.
    """
    g = np.asarray(g, dtype=np.float64)
    xhat = np.asarray(xhat, dtype=np.float64)
    r = np.asarray(rstd, dtype=np.float64)[..., None]
    return r * (g - xhat * np.mean(g * xhat, axis=-1, keepdims=True))


def gemm_postnorm_backward(dy2, w, y, rstd, kind):
    """The post-norm backward as the page regroups it: the norm's upstream
    gradient is the product of the next layer's output gradient dy2 [M, K]
    with that layer's weight read as w [K, N], and the norm backward (over the
    N axis) is that product's epilogue.  y [M, N] is the forward output of the
    norm (the normalized values), rstd [M] its forward statistic.
    Returns dz [M, N], the gradient at the norm's input.
    """
    g = gemm(dy2, w)
    if kind == "ln":
        return layernorm_backward_rows(g, y, rstd)
    if kind == "rms":
        return rmsnorm_backward_rows(g, y, rstd)
    raise ValueError(kind)


def prenorm_rms_backward_dx(dy, w, x, rstd):
    """Input gradient of the lazy pre-RMSNorm GEMM y = rmsnorm(x) @ W: the
    gradient at rmsnorm's output is dy @ W^T (w [N, K] is W^T read row-major:
    w = W.T), then the RMSNorm backward with xhat rebuilt from x and the
    forward rstd.  Returns dx [M, K].
    """
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(rstd, dtype=np.float64)
    return rmsnorm_backward_rows(gemm(dy, w), x * r[..., None], r)


def prenorm_rms_backward_dw(x, dy, rstd, gamma=None):
    """Weight gradient of the lazy pre-RMSNorm GEMM y = (rmsnorm(x) * gamma) @ W
    (section 2's limitations: rmsnorm(A) must be rebuilt from A and rstd for
    the gradients of both operands).  With xhat = x * rstd[:, None] (* gamma),
    the normalized input rebuilt from x [M, K] and the forward rstd [M]:
        dW = xhat^T @ dy,   dW [K, N], dy [M, N].
    """
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(rstd, dtype=np.float64)
    xhat = x * r[:, None]
    if gamma is not None:
        xhat = xhat * np.asarray(gamma, dtype=np.float64)[None, :]
    return xhat.T @ np.asarray(dy, dtype=np.float64)


# ---------------------------------------------------------------------------
# attention (section 4)
# ---------------------------------------------------------------------------

def softmax_rows(s):
    """Max-subtracted softmax over the last axis."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q, k, v, sm_scale):
    """Plain softmax attention, BSHD: O[b,s,h,:] = softmax(q k^T * scale) v.

    q is [B, Sq, H, D]; k, v are [B, Skv, H, D].  Non-causal, no mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    o = np.empty((B, Sq, H, v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = (q[b, :, h, :] @ k[b, :, h, :].T) * sm_scale
            o[b, :, h, :] = softmax_rows(s) @ v[b, :, h, :]
    return o


def norm_attention(q, k, v, eps_ln, eps_rms, sm_scale):
    """out = rmsnorm(softmax(layernorm(q) k^T * scale) v), per (b, h), BSHD.

    Section 4: ln_q = layernorm(q) before the score product, and an RMSNorm of
    the attention output after it; both norms here run over head_dim of one
    head, softmax replaces the generic activation and there are no residual
    adds (the norm-sandwiched attention workload).  Returns
    (out, ln_mean[B,Sq,H], ln_rstd[B,Sq,H], rms_rstd[B,Sq,H]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    out = np.empty((B, Sq, H, v.shape[-1]), dtype=np.float64)
    ln_mean = np.empty((B, Sq, H))
    ln_rstd = np.empty((B, Sq, H))
    rms_rstd = np.empty((B, Sq, H))
    for b in range(B):
        for h in range(H):
            qn, mu, r1 = layernorm_rows(q[b, :, h, :], eps_ln)
            s = (qn @ k[b, :, h, :].T) * sm_scale
            o = softmax_rows(s) @ v[b, :, h, :]
            y, r2 = rmsnorm_rows(o, eps_rms)
            out[b, :, h, :] = y
            ln_mean[b, :, h] = mu
            ln_rstd[b, :, h] = r1
            rms_rstd[b, :, h] = r2
    return out, ln_mean, ln_rstd, rms_rstd


def gelu_tanh(x):
    """GELU in its tanh form (Hendrycks and Gimpel's approximation):
    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))


def _activation(s, act):
    if act == "softmax":
        return softmax_rows(s)
    if act == "gelu":
        return gelu_tanh(s)
    raise ValueError(act)


def jagged_attention(q, offsets, k, v, sm_scale, act):
    """The attention inside FlashNormAttention without its norms and
    residuals (the unfused baseline's attention step), jagged queries:
    out[r, h, :] = act(q[r, h, :] k[b, :, h, :]^T * sm_scale) v[b, :, h, :]
    for every row r of batch b.  Layouts as in flash_norm_attention.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    T, H, D = q.shape
    out = np.zeros((T, H, v.shape[-1]))
    for b in range(len(offsets) - 1):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 <= r0:
            continue
        for h in range(H):
            s = (q[r0:r1, h, :] @ k[b, :, h, :].T) * sm_scale
            out[r0:r1, h, :] = _activation(s, act) @ v[b, :, h, :]
    return out


def flash_norm_attention(q, offsets, k, v, eps_ln, eps_rms, sm_scale, act):
    """Section 4's FlashNormAttention, fused short-KV form, on jagged queries.

    q: [T, H, D] query rows of all batches back to back, rows offsets[b] ..
    offsets[b+1]-1 belonging to batch b; k, v: [B, Skv, H, D] dense.
    For every query row x (H*D values):
        ln  = layernorm(x) over all H*D                       (norm 1)
        o_h = act(ln_h k[b,:,h,:]^T * sm_scale) v[b,:,h,:] + ln_h   (residual 1)
        out = rmsnorm(o) over all H*D + x                      (norm 2, residual 2)
    act is "softmax" (over the keys) or "gelu" (elementwise, tanh form).
    Returns (out [T,H,D], ln_mean [T], ln_rstd [T], rms_rstd [T]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    T, H, D = q.shape
    out = np.empty_like(q)
    ln_mean = np.empty(T)
    ln_rstd = np.empty(T)
    rms_rstd = np.empty(T)
    for b in range(len(offsets) - 1):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 <= r0:
            continue
        x = q[r0:r1].reshape(r1 - r0, H * D)
        ln, mu, rs1 = layernorm_rows(x, eps_ln)
        ln = ln.reshape(r1 - r0, H, D)
        o = np.empty_like(ln)
        for h in range(H):
            s = (ln[:, h, :] @ k[b, :, h, :].T) * sm_scale
            if act == "softmax":
                p = softmax_rows(s)
            elif act == "gelu":
                p = gelu_tanh(s)
            else:
                raise ValueError(act)
            o[:, h, :] = p @ v[b, :, h, :] + ln[:, h, :]
        y, rs2 = rmsnorm_rows(o.reshape(r1 - r0, H * D), eps_rms)
        out[r0:r1] = (y + x).reshape(r1 - r0, H, D)
        ln_mean[r0:r1] = mu
        ln_rstd[r0:r1] = rs1
        rms_rstd[r0:r1] = rs2
    return out, ln_mean, ln_rstd, rms_rstd


def gelu_tanh_grad(x):
    """Derivative of gelu_tanh: with u = sqrt(2/pi) (x + 0.044715 x^3) and
    t = tanh(u), d/dx [0.5 x (1 + t)] = 0.5 (1 + t) + 0.5 x (1 - t^2) u'(x),
    u'(x) = sqrt(2/pi) (1 + 3 * 0.044715 x^2)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.sqrt(2.0 / np.pi)
    t = np.tanh(a * (x + 0.044715 * x ** 3))
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * a * (1.0 + 3.0 * 0.044715 * x * x)


def activation_backward(s, p, dp, act):
    """Gradient at the scores s of p = act(s), given dp, the gradient at p.
    softmax over the last axis: ds = p * (dp - sum(p * dp)) (the softmax
    Jacobian diag(p) - p p^T applied to dp); GELU, elementwise: dp * gelu'(s).
    """
    if act == "softmax":
        return p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    if act == "gelu":
        return dp * gelu_tanh_grad(s)
    raise ValueError(act)


def flash_norm_attention_backward(q, offsets, k, v, dout, eps_ln, eps_rms, sm_scale, act):
    """Gradients of flash_norm_attention with respect to q, k and v, given the
    gradient dout [T, H, D] at its output (section 4, "Backward
    implementation": the norm statistics come from the forward, the LayerNorm
    output and the RMSNorm input and output are recomputed; here the whole
    forward is recomputed in fp64 from q, k and v).

    The chain, for every query row (x = q, all H*D values):
        forward   ln = layernorm(x); s_h = ln_h k_h^T sm_scale; p_h = act(s_h)
                  o_h = p_h v_h + ln_h; y = rmsnorm(o); out = y + x
        backward  do   = rmsnorm_backward(dout, y, rstd_rms)
                  dln  = do + sum over heads of (d/d ln_h of p_h v_h) . do_h
                         with dp_h = do_h v_h^T, ds_h = act_backward(dp_h),
                         dln_h += sm_scale ds_h k_h
                  dv_h += p_h^T do_h, dk_h += sm_scale ds_h^T ln_h  (summed over
                         the batch's rows)
                  dq   = dout + layernorm_backward(dln, ln, rstd_ln)
    Returns (dq [T, H, D], dk [B, Skv, H, D], dv [B, Skv, H, D]); rows outside
    every batch get dq = 0, batches without rows dk = dv = 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    T, H, D = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(offsets) - 1):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 <= r0:
            continue
        L = r1 - r0
        x = q[r0:r1].reshape(L, H * D)
        ln, _, rs1 = layernorm_rows(x, eps_ln)
        ln = ln.reshape(L, H, D)
        s = np.empty((H, L, k.shape[1]))
        p = np.empty_like(s)
        o = np.empty_like(ln)
        for h in range(H):
            s[h] = (ln[:, h, :] @ k[b, :, h, :].T) * sm_scale
            p[h] = _activation(s[h], act)
            o[:, h, :] = p[h] @ v[b, :, h, :] + ln[:, h, :]
        y, rs2 = rmsnorm_rows(o.reshape(L, H * D), eps_rms)
        g = dout[r0:r1].reshape(L, H * D)
        do = rmsnorm_backward_rows(g, y, rs2).reshape(L, H, D)
        dln = do.copy()                                   # first residual
        for h in range(H):
            dv[b, :, h, :] = p[h].T @ do[:, h, :]
            dp = do[:, h, :] @ v[b, :, h, :].T
            ds = activation_backward(s[h], p[h], dp, act) * sm_scale
            dln[:, h, :] += ds @ k[b, :, h, :]
            dk[b, :, h, :] = ds.T @ ln[:, h, :]
        dx = layernorm_backward_rows(dln.reshape(L, H * D), ln.reshape(L, H * D), rs1)
        dq[r0:r1] = (g + dx).reshape(L, H, D)             # second residual
    return dq, dk, dv


def jagged_attention_backward(q, offsets, k, v, dout, sm_scale, act):
    """Gradients of jagged_attention (the attention step of FlashNormAttention
    without its norms and residuals; the unfused chain's attention backward)
    with respect to q, k and v, given dout [T, H, D] at its output.

    For every batch b and head h, with s = q k^T sm_scale and p = act(s):
        dp = dout v^T,  ds = act_backward(s, p, dp) sm_scale
        dq = ds k,  dk = ds^T q (summed over the batch's rows),  dv = p^T dout
    Returns (dq [T, H, D], dk [B, Skv, H, D], dv [B, Skv, H, D]); rows outside
    every batch get dq = 0, batches without rows dk = dv = 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    offsets = np.asarray(offsets, dtype=np.int64)
    T, H, D = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(len(offsets) - 1):
        r0, r1 = int(offsets[b]), int(offsets[b + 1])
        if r1 <= r0:
            continue
        for h in range(H):
            qh, kh, vh, gh = q[r0:r1, h, :], k[b, :, h, :], v[b, :, h, :], dout[r0:r1, h, :]
            s = (qh @ kh.T) * sm_scale
            p = _activation(s, act)
            dv[b, :, h, :] = p.T @ gh
            ds = activation_backward(s, p, gh @ vh.T, act) * sm_scale
            dq[r0:r1, h, :] = ds @ kh
            dk[b, :, h, :] = ds.T @ qh
    return dq, dk, dv


# ---------------------------------------------------------------------------
# the agreed comparison metric
# ---------------------------------------------------------------------------

def compare(y, ref):
    """Errors of a result y against an fp64 reference.

    Returns a dict with
      normwise_rel = max|y - ref| / max|ref|  (the "max relative error", read
                                               normwise so it is defined when
                                               ref has zeros)
      mae          = mean|y - ref|
      max_abs      = max|y - ref|
    """
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    if y.size == 0:
        return {"normwise_rel": 0.0, "mae": 0.0, "max_abs": 0.0}
    err = np.abs(y - ref)
    scale = float(np.max(np.abs(ref)))
    return {
        "normwise_rel": float(np.max(err)) / scale if scale > 0 else float(np.max(err)),
        "mae": float(np.mean(err)),
        "max_abs": float(np.max(err)),
    }
