"""fp64 CPU oracle (test infrastructure only; see fng_oracle's header)."""

from .fng_oracle import (  # noqa: F401
    attention,
    bf16_to_f64,
    compare,
    gemm,
    gemm_postnorm,
    layernorm_rows,
    norm_attention,
    gelu_tanh,
    flash_norm_attention,
    jagged_attention,
    layernorm_backward_rows,
    rmsnorm_backward_rows,
    gemm_postnorm_backward,
    prenorm_rms_backward_dx,
    prenorm_rms_gemm,
    rms_rstd,
    rmsnorm_rows,
    softmax_rows,
)
