"""Tolerance rule for GPU-vs-oracle comparisons — TEST INFRASTRUCTURE ONLY.

The required bounds are a max-abs error of 1e-2 on the bf16 output O and 1e-3
on the fp32 LSE.  A bf16 number carries 8 significant bits, so the exact O
correctly rounded to bf16 already errs by up to half a bf16 ulp: 0.0078 on
[2, 4) and 0.0156 on [4, 8).  Inputs whose large logits make rows nearly
one-hot give |O| ≥ 4, where no bf16 output can meet 1e-2 literally.  The rule
applied here therefore reads 1e-2 as the kernel's own error budget on top of
correct rounding:

    pass  iff  |O_gpu − O_ref| ≤ 1e-2 + ½·ulp_bf16(O_ref)   for every element,
          and  |LSE_gpu − LSE_ref| ≤ 1e-3                      (literal).

The report also carries the literal max-abs error, the rounding floor
max|bf16_RNE(O_ref) − O_ref| and the excess max(|err| − ½ulp) so that the
literal reading can be judged too.
"""

import numpy as np

O_TOL = 1e-2
LSE_TOL = 1e-3


def bf16_ulp(x):
    """ulp of bfloat16 at |x| (8 significant bits), elementwise, float64."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(np.abs(x))           # |x| = f·2^e, f in [0.5, 1)
    return np.ldexp(1.0, e - 8)


def bf16_half_ulp(x):
    """Half a bf16 ulp at |x|: the worst error of round-to-nearest to bf16."""
    return 0.5 * bf16_ulp(x)


def bf16_rne(x):
    """Round float64 values to the nearest bf16 value, ties to even."""
    x = np.asarray(x, dtype=np.float64)
    u = bf16_ulp(x)
    return np.round(x / u) * u            # x/u is exact (power-of-two divisor)


def o_excess(o_gpu, o_ref):
    """Error report for O: literal max-abs, rounding floor, excess over ½ulp."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    half = bf16_half_ulp(o_ref)
    return {
        "max_abs": float(err.max()) if err.size else 0.0,
        "floor": float(np.abs(bf16_rne(o_ref) - o_ref).max()) if err.size else 0.0,
        "excess": float((err - half).max()) if err.size else 0.0,
        "ok": bool(np.all(err <= O_TOL + half)) and bool(np.all(np.isfinite(o_gpu))),
    }


def check_prefill(o_gpu, lse_gpu, o_ref, lse_ref):
    """Apply the rule to one prefill comparison; returns the report dict."""
    rep = o_excess(o_gpu, o_ref)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    lse_ref = np.asarray(lse_ref, dtype=np.float64)
    lerr = np.abs(lse_gpu - lse_ref)
    rep["lse_max_abs"] = float(lerr.max()) if lerr.size else 0.0
    rep["lse_ok"] = bool(np.all(lerr <= LSE_TOL)) and bool(np.all(np.isfinite(lse_gpu)))
    rep["pass"] = rep["ok"] and rep["lse_ok"]
    return rep


check_decode = check_prefill
