"""Write tests/golden/oracle_regression.json from the fp64 oracle only.

The pages ("Towards Free Normalization: Fusing Normalization into GEMM and
Attention Kernels") print no numeric worked example, so there are no page
values to store.  This fixture instead freezes a few oracle outputs on the
seeded synthetic inputs, so that any later change to the oracle's arithmetic
shows up as a test failure and has to be justified.  Run from the repo root:

    python tests/golden/make_golden.py
"""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from attention_fng_prenorm_amd import inputs  # noqa: E402


def build():
    out = {}
    spec, d = inputs.make_inputs("prenorm_rms_small")
    y, r = oracle.prenorm_rms_gemm(oracle.bf16_to_f64(d["X"]), oracle.bf16_to_f64(d["W"]), spec["eps"])
    out["prenorm_rms_small"] = {"Y[0:3,0:6]": y[0:3, 0:6].tolist(), "rstd[0:6]": r[0:6].tolist(),
                                "sum_abs_Y": float(np.sum(np.abs(y)))}
    spec, d = inputs.make_inputs("postnorm_ln_smalln", M=64)
    y, mu, r = oracle.gemm_postnorm(oracle.bf16_to_f64(d["X"]), oracle.bf16_to_f64(d["W"]), spec["eps"], "ln")
    out["postnorm_ln_smalln[M=64]"] = {"Y[0:3,0:6]": y[0:3, 0:6].tolist(), "mean[0:6]": mu[0:6].tolist(),
                                       "rstd[0:6]": r[0:6].tolist()}
    spec, d = inputs.make_inputs("norm_attention", B=1, Sq=16, Skv=16, H=2)
    o, mu, r1, r2 = oracle.norm_attention(oracle.bf16_to_f64(d["Q"]), oracle.bf16_to_f64(d["K"]),
                                          oracle.bf16_to_f64(d["V"]), spec["eps_ln"], spec["eps_rms"],
                                          1.0 / np.sqrt(spec["D"]))
    out["norm_attention[B=1,S=16,H=2]"] = {"out[0,0:2,1,0:6]": o[0, 0:2, 1, 0:6].tolist(),
                                           "rms_rstd[0,0:4,0]": r2[0, 0:4, 0].tolist()}
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as f:
        json.dump(build(), f, indent=1)
    print("wrote", path)
