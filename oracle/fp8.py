"""Block-wise FP8 quantisation for the FP8 form of attention — TEST
INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

[cicada] §4.4.1 (FlashAttention-3, block-wise quantisation): instead of one
scale factor per tensor, every block of rows that the kernel stages on chip
carries its own scale, so an outlier only coarsens the block it sits in.

Readings taken here (the page fixes neither the format nor the block shapes):

* The 8-bit format is OCP E4M3 "FN": 1 sign bit, 4 exponent bits (bias 7),
  3 mantissa bits, subnormals at exponent field 0, no infinities, the all-ones
  code (either sign) is NaN, so the largest finite magnitude is 1.75·2⁸ = 448.
  It is the 8-bit float with the most precision among the OCP formats, and the
  one gfx950's matrix cores read.
* A block's scale is a power of two, the smallest one that brings its largest
  magnitude to at most 448: s = 2^⌈log2(amax/448)⌉, the exponent clamped to
  the E8M0 range [−127, 127] (s = 1 for an all-zero block), so the largest
  element lands in (224, 448].  Power-of-two scales are
  the ones gfx950's matrix cores apply in the product itself (an E8M0 exponent
  per operand block), and dividing by one is exact.  Elements are divided by s
  and rounded to the nearest E4M3 value, ties to the even code, saturating at
  448.
* Blocks are runs of 64 consecutive rows of one (batch, head) slice, all d
  columns together, for Q, K and V alike (the kernel's key tile, and a
  quarter of its query block).
* The attention that FP8 inputs define is exact attention of the dequantised
  Q̂ = s·q₈, K̂, V̂ (``attention_fp8_ref``).  Rounding the probabilities to FP8
  before the second product is a step of the kernel, not of this definition; its
  error is bounded separately.
"""

import numpy as np

from .ref import as_f64, attention_ref

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6   # smallest normal: 2^-6
_MANT_BITS = 3


def e4m3_decode_table():
    """The value of each of the 256 E4M3FN codes, built from the bit fields
    (sign · 2^(e−7) · (1 + m/8) for e ≥ 1, sign · 2^−6 · m/8 for e = 0, NaN for
    e = 15, m = 7).  Returns a float64 array indexed by the code."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * 2.0 ** _MIN_NORMAL_EXP * (m / 8.0)
        else:
            vals[code] = sign * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return vals


def e4m3_round(x):
    """Round float64 values to the nearest E4M3FN value (ties to even),
    saturating at ±448.  Returns float64 values (exactly representable ones).

    For |x| ≥ 2^−6 the spacing of E4M3 values in [2^e, 2^(e+1)) is 2^(e−3);
    below that it is the subnormal spacing 2^−9.  Dividing by the spacing and
    rounding half to even picks the nearest value with an even mantissa on ties
    (the spacing is a power of two, so the division is exact)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                     # a = f·2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, _MIN_NORMAL_EXP)  # exponent of the binade (subnormals share 2^-6's)
    step = np.ldexp(1.0, e - _MANT_BITS)
    r = np.rint(a / step) * step
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def quantize_blocks(x, block_rows):
    """Block-wise quantisation of x [..., N, d] along its row axis.

    Rows [i·block_rows, (i+1)·block_rows) of each leading slice share one scale
    s = 2^⌈log2(amax/448)⌉ (1 when the block is all zero); the stored value is
    e4m3_round(x / s).  Returns (x8, scales): x8 with x's shape (the E4M3 values,
    as float64) and scales [..., ⌈N/block_rows⌉]; the dequantised tensor is
    x8 · s of each row's block."""
    x = as_f64(x)
    *lead, N, d = x.shape
    nb = -(-N // block_rows)
    x8 = np.empty_like(x)
    scales = np.empty((*lead, nb), dtype=np.float64)
    for b in range(nb):
        blk = x[..., b * block_rows:(b + 1) * block_rows, :]
        amax = np.abs(blk).max(axis=(-2, -1)) if blk.size else np.zeros(lead)
        safe = np.where(amax > 0, amax, E4M3_MAX)
        e = np.ceil(np.log2(safe / E4M3_MAX)).astype(np.int64)
        e = np.where(safe / np.ldexp(1.0, e) > E4M3_MAX, e + 1, e)       # log2 rounding guard
        e = np.where(safe / np.ldexp(1.0, e - 1) <= E4M3_MAX, e - 1, e)
        e = np.clip(e, -127, 127)                                        # the E8M0 range
        s = np.where(amax > 0, np.ldexp(1.0, e), 1.0)
        scales[..., b] = s
        x8[..., b * block_rows:(b + 1) * block_rows, :] = e4m3_round(blk / s[..., None, None])
    return x8, scales


def dequantize_blocks(x8, scales, block_rows):
    """x8 · s row block by row block (the inverse map of quantize_blocks' scaling)."""
    x8 = np.asarray(x8, dtype=np.float64)
    rep = np.repeat(scales, block_rows, axis=-1)[..., :x8.shape[-2]]
    return x8 * rep[..., None]


def attention_fp8_ref(q, k, v, scale, causal, q_block=64, kv_block=64, rows=None):
    """Exact attention of block-quantised inputs: Q, K and V are quantised with
    quantize_blocks (Q in blocks of q_block rows, K and V in blocks of kv_block
    keys), dequantised, and fed to attention_ref.  Returns (O, LSE) as float64
    like attention_ref, for the query rows ``rows`` (all by default)."""
    qh = dequantize_blocks(*quantize_blocks(q, q_block), q_block)
    kh = dequantize_blocks(*quantize_blocks(k, kv_block), kv_block)
    vh = dequantize_blocks(*quantize_blocks(v, kv_block), kv_block)
    return attention_ref(qh, kh, vh, scale, causal, rows=rows)


def fp8_allowance(q, k, v, scale, causal, block=64, rows=None):
    """The parity bound of the FP8 forward, per output row.

    The kernel rounds each probability P̃_i = exp(s_i − m) (m at most the row's
    true max, so P̃_i ≤ 2^8 is the only range it needs) to E4M3 before the second
    product and divides by the fp32 sum ℓ of the unrounded P̃.  E4M3 rounding
    moves a value by at most 2^−4 of itself (3 mantissa bits) or by 2^−10 (half
    the subnormal spacing), whichever is larger; a later rescale by α ≤ 1 only
    shrinks both.  With p_i = P̃_i/ℓ and ℓ ≥ ℓ* = Σ exp(s_i − max s):

        |O − O_ref| ≤ 2^−4·Σ p_i |v̂_i| + 2^−10·Σ |v̂_i| / ℓ*

    per element of O (v̂ the dequantised values of that column).  Returns
    (O_ref, L_ref, allowance) as float64 [B, H, R, d], [B, H, R], [B, H, R, d]
    for the query rows ``rows`` (all by default)."""
    from .ref import scores, safe_softmax
    qh = dequantize_blocks(*quantize_blocks(q, block), block)
    kh = dequantize_blocks(*quantize_blocks(k, block), block)
    vh = dequantize_blocks(*quantize_blocks(v, block), block)
    B, H, N, _ = qh.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    o = np.empty((B, H, rows.size, vh.shape[-1]))
    lse = np.empty((B, H, rows.size))
    allow = np.empty_like(o)
    for b in range(B):
        for h in range(H):
            s = scores(qh[b, h][rows], kh[b, h], scale, causal, rows)
            p, m, l = safe_softmax(s)
            o[b, h] = p @ vh[b, h]
            lse[b, h] = m + np.log(l)
            seen = (p > 0).astype(np.float64)  # keys the row attends to (masked ones carry no rounding)
            allow[b, h] = 2.0 ** -4 * (p @ np.abs(vh[b, h])) + 2.0 ** -10 * (seen @ np.abs(vh[b, h])) / l[:, None]
    return o, lse, allow


# ---- the kernel's rounding step, modelled -----------------------------------------
#
# attention_fp8_ref is the definition.  The FP8 forward reaches it up to one
# step of its own: it rounds the probabilities P̃ to E4M3 before the second
# product, against a reference maximum that it moves only now and then
# (conditional rescaling, [cicada] §5, FlashAttention-4: the reference max of
# a group of rows is moved only when some row of the group outgrows it by more
# than 2^8, which keeps every P̃ below the format's 448).  Which values get
# rounded, and how, depends on that schedule, so a bound that does not know it
# must allow every P̃ its worst rounding (fp8_allowance) — and at long N that
# worst case outgrows O itself.  fp8_step_model carries the step out exactly as
# described, in fp64, on the dequantised inputs, and so predicts the rounded
# output itself; what is left between it and a correct kernel is fp32
# arithmetic, bounded in fp8_step_allowance.

U_F32 = 2.0 ** -24            # unit roundoff of fp32
FP8_RESCALE_LOG2 = 8.0        # growth of a row max (base-2 units) that moves the reference max
FP8_GROUP_ROWS = 32           # query rows that share the decision to move it
FP8_KEY_TILE = 64             # keys per step, in order
LAMBDA_PROB = 10.0            # probabilistic bound's confidence parameter (see fp8_step_allowance)
EXP2_REL = 2.0 ** -21         # relative error allowed for the hardware exp2


def _groups_for(rows, N, group):
    """The aligned groups of ``group`` rows that contain ``rows``."""
    rows = np.arange(N) if rows is None else np.asarray(rows)
    return np.unique(rows // group)


def fp8_step_model(q, k, v, scale, causal, rows=None, block=64, round_p=True, group=FP8_GROUP_ROWS,
                   tile=FP8_KEY_TILE, threshold=FP8_RESCALE_LOG2):
    """The FP8 forward's rounding step, carried out in fp64 (a model, not the definition).

    Inputs are quantised block-wise (``quantize_blocks``, blocks of ``block``
    rows) and dequantised; for every query row, with logits in base-2 units
    t_j = scale·log2(e)·q̂·k̂_j (causal: keys after the row are masked), the
    keys are taken ``tile`` at a time, in order ([15-779 L5] §5.1):

    * a reference max M per row, −∞ at first; the first tile sets M to the
      row's max over it; at a later tile, if any row of the row's group
      (``group`` consecutive rows, aligned) has a tile max more than
      ``threshold`` above its M, every row of the group moves M to
      max(M, tile max) and multiplies ℓ and the accumulator by 2^(M_old − M);
    * P̃_j = 2^(t_j − M), rounded to E4M3 (``round_p``; the slip test turns it
      off), accumulated as Σ round(P̃_j)·v̂_j; ℓ sums the unrounded P̃_j;
    * O = acc / ℓ and L = M·ln 2 + ln ℓ.

    The model also tracks how far a kernel doing the same in fp32 could stray
    from it.  The logits of such a kernel differ by at most γ_d·Σ|q̂_c k̂_jc|
    (fp32 dot products of exact products, d terms), which with the roundings
    of the exponent's arguments and of exp2 bounds |log2 P̃_kernel − log2 P̃|
    by e_j per element.  A P̃_j whose interval P̃_j·2^(±e_j) straddles an
    E4M3 rounding boundary may round either way in the kernel: its largest
    possible change of the rounded value, times |v̂_j| and the later rescales,
    over ℓ, is summed into ``amb``.  A decision to move M that lies within its
    own error bound of the threshold marks the group ``sched_amb`` (the
    kernel may have taken the other branch; such rows are checked against the
    schedule-free bound only).

    Returns a dict of float64 arrays over the query rows of every group that
    contains one of ``rows`` (all rows by default): ``rows`` [R], ``o``
    [B, H, R, d], ``lse`` [B, H, R], ``wabs`` [B, H, R, d] = Σ_j w_j|v̂_j| / ℓ
    (w_j the larger of P̃_j and its rounding, rescaled — the size of the terms
    the kernel's fp32 sums add up), ``amb`` [B, H, R, d], ``ex_max`` [B, H, R]
    (largest e_j of the row), ``sched_amb`` [B, H, R] (bool), ``moves``
    [B, H, R] (how often M moved), ``n_keys`` (keys per row at most).
    """
    with np.errstate(divide="ignore", invalid="ignore"):  # rows past N give 0/0; they are dropped
        return _step_model(q, k, v, scale, causal, rows, block, round_p, group, tile, threshold)


def _step_model(q, k, v, scale, causal, rows, block, round_p, group, tile, threshold):
    qh = dequantize_blocks(*quantize_blocks(q, block), block)
    kh = dequantize_blocks(*quantize_blocks(k, block), block)
    vh = dequantize_blocks(*quantize_blocks(v, block), block)
    B, H, N, d = qh.shape
    c = scale * np.log2(np.e)
    gd = d * U_F32 / (1 - d * U_F32)
    grp = _groups_for(rows, N, group)
    allrows = (grp[:, None] * group + np.arange(group)[None, :]).reshape(-1)
    live = allrows < N                       # rows past N do not exist (and never move M)
    R = int(live.sum())
    G = grp.size
    n_tiles = -(-N // tile)
    out = {k_: np.zeros((B, H, R, d)) for k_ in ("o", "wabs", "amb")}
    for k_ in ("lse", "ex_max", "moves"):
        out[k_] = np.zeros((B, H, R))
    out["sched_amb"] = np.zeros((B, H, R), dtype=bool)
    rowidx = np.minimum(allrows, N - 1).reshape(G, group)
    keys = np.arange(N)
    for b in range(B):
        for h in range(H):
            qg = qh[b, h][rowidx]                              # [G, group, d]
            t = c * np.einsum("grc,nc->grn", qg, kh[b, h])     # logits, base-2 units
            a = np.einsum("grc,nc->grn", np.abs(qg), np.abs(kh[b, h]))
            es = c * gd * a                                    # bound on the fp32 logit error
            vis = np.broadcast_to(live.reshape(G, group)[:, :, None], t.shape).copy()
            if causal:
                vis &= keys[None, None, :] <= rowidx[:, :, None]
            t = np.where(vis, t, -np.inf)
            es_max = np.where(vis, es, 0.0).max(axis=2)        # [G, group]
            m = np.full((G, group), -np.inf)
            ell = np.zeros((G, group))
            acc = np.zeros((G, group, d))
            wab = np.zeros((G, group, d))
            amb = np.zeros((G, group, d))
            exm = np.zeros((G, group))
            mov = np.zeros((G, group))
            samb = np.zeros(G, dtype=bool)
            va = np.abs(vh[b, h])
            for j in range(n_tiles):
                sl = slice(j * tile, min(N, (j + 1) * tile))
                tj, vj = t[:, :, sl], vis[:, :, sl]
                if not vj.any():
                    continue
                tmax = tj.max(axis=2)                           # −∞ where the row sees no key of the tile
                if j == 0:
                    move = np.ones(G, dtype=bool)
                else:
                    with np.errstate(invalid="ignore"):
                        grow = tmax - m - threshold
                        edec = 2 * es_max + 4 * U_F32 * (np.abs(np.where(np.isfinite(tmax), tmax, 0)) + np.abs(m)) \
                            + 2.0 ** -20
                        sure = np.any(grow > edec, axis=1)
                        maybe = np.any(grow >= -edec, axis=1)
                    move = np.any(grow > 0, axis=1)
                    samb |= sure != maybe
                if move.any():
                    mn = np.where(move[:, None], np.fmax(m, tmax), m)
                    with np.errstate(invalid="ignore"):
                        alpha = np.where(np.isneginf(m), 0.0, np.exp2(m - mn))
                    alpha = np.where(move[:, None], alpha, 1.0)
                    ell *= alpha
                    acc *= alpha[:, :, None]
                    wab *= alpha[:, :, None]
                    amb *= alpha[:, :, None]
                    mov += move[:, None] & (mn > m)
                    m = mn
                x = np.where(vj, np.exp2(tj - m[:, :, None]), 0.0)
                xr = e4m3_round(x) if round_p else x
                ell += x.sum(axis=2)
                acc += xr @ vh[b, h][sl]
                wab += np.maximum(x, np.abs(xr)) @ va[sl]
                # how far the kernel's log2 P̃ may lie from this one
                mfin = np.where(np.isfinite(m), m, 0.0)[:, :, None]
                ex = (es[:, :, sl] + es_max[:, :, None] + 3 * U_F32 * np.abs(mfin)
                      + U_F32 * (2 * np.abs(np.where(vj, tj, 0.0)) + np.abs(np.where(vj, tj - mfin, 0.0)))
                      + EXP2_REL / np.log(2.0) + 2.0 ** -24)
                ex = np.where(vj, ex, 0.0)
                exm = np.maximum(exm, ex.max(axis=2))
                lo, hi = e4m3_round(x * np.exp2(-ex)), e4m3_round(x * np.exp2(ex))
                ref = xr if round_p else e4m3_round(x)
                dev = np.maximum(hi - ref, ref - lo)
                amb += dev @ va[sl]
            sel = live.reshape(G, group)
            o = acc / ell[:, :, None]
            out["o"][b, h] = o[sel]
            out["wabs"][b, h] = (wab / ell[:, :, None])[sel]
            out["amb"][b, h] = (amb / ell[:, :, None])[sel]
            out["lse"][b, h] = (m * np.log(2.0) + np.log(ell))[sel]
            out["ex_max"][b, h] = exm[sel]
            out["moves"][b, h] = mov[sel]
            out["sched_amb"][b, h] = np.broadcast_to(samb[:, None], (G, group))[sel]
    out["rows"] = allrows[live]
    out["n_keys"] = N
    return out


def fp8_step_allowance(model):
    """Per-element bound on |O_kernel − O_model| for a kernel that carries out
    fp8_step_model's step in fp32 (before O is rounded to bf16).

    * ``amb``: the E4M3 roundings the kernel may take the other way (see the
      model).
    * The fp32 sums Σ round(P̃_j)·v̂_j and ℓ = Σ P̃_j over n ≤ N terms, the
      rescale products, the reciprocal and the final product: each term passes
      through at most n + 16 roundings.  Bounding that worst case by γ_n
      (n·u) gives 1e-3·|O| at N = 16384, as large as the rounding of P̃ it is
      meant to tell apart, so the probabilistic bound of Higham and Mary ("A
      new approach to probabilistic rounding error analysis", SIAM J. Sci.
      Comput. 41(5), 2019, Theorem 2.4) is used: for independent roundings of
      mean zero, the relative error of a product of n factors (1 + δ_i) stays
      below γ̃_n(λ) = exp(λ·√n·u + n·u²/(1 − u)) − 1 with probability at
      least 1 − 2·exp(−λ²(1 − u)²/2); λ = 10 makes that 1 − 4e−22 per term.
      This acts on Σ w_j|v̂_j|/ℓ (``wabs``, numerator) and |O| (through ℓ).
    * The kernel's P̃ differ from the model's by at most a factor 2^(±e_j),
      which moves ℓ (the sum of unrounded P̃) by the relative 2^e_max − 1.
    """
    n = model["n_keys"] + 16
    g = np.expm1(LAMBDA_PROB * np.sqrt(n) * U_F32 + n * U_F32 ** 2 / (1 - U_F32))
    o = np.abs(model["o"])
    return model["amb"] + g * (model["wabs"] + o) + np.expm1(model["ex_max"] * np.log(2.0))[..., None] * o


def fp8_contract(q, k, v, scale, causal, rows=None, block=64):
    """Everything the FP8 parity check needs, for the rows of every 32-row group
    that contains one of ``rows`` (all rows by default): the model, its
    allowance, and the definition (attention_fp8_ref) with the schedule-free
    bound fp8_allowance on the same rows.  Returns a dict (the model's keys
    plus ``o_ref``, ``lse_ref``, ``allow_def``, ``allow_step``)."""
    model = fp8_step_model(q, k, v, scale, causal, rows=rows, block=block)
    o_ref, lse_ref, allow_def = fp8_allowance(q, k, v, scale, causal, block=block, rows=model["rows"])
    model.update(o_ref=o_ref, lse_ref=lse_ref, allow_def=allow_def, allow_step=fp8_step_allowance(model))
    return model


def check_fp8(o, lse, contract, lse_tol=1e-3):
    """The FP8 forward's parity rule, on the rows of ``contract`` (fp8_contract):

    * step (tight): |O − O_model| ≤ allow_step + ½ulp_bf16(|O_model| + allow_step)
      on every row whose group took no decision near the threshold;
    * definition: |O − O_ref| ≤ allow_def + allow_step + ½ulp_bf16(|O_ref| +
      allow_def + allow_step) on every row — the kernel is exact attention of
      the dequantised inputs within the worst case of rounding P̃ (any schedule);
    * |L − L_ref| ≤ lse_tol (L is taken from the unrounded P̃).

    ``o`` and ``lse``: the kernel's outputs on contract["rows"], [B, H, R, d]
    and [B, H, R].  Returns a report dict with 'pass'."""
    from .compare import bf16_half_ulp
    o = np.asarray(o, np.float64)
    lse = np.asarray(lse, np.float64)
    tight = ~contract["sched_amb"]
    lim_s = contract["allow_step"] + bf16_half_ulp(np.abs(contract["o"]) + contract["allow_step"])
    err_s = np.abs(o - contract["o"])
    ok_s = np.all((err_s <= lim_s) | ~tight[..., None])
    lim_d = contract["allow_def"] + contract["allow_step"]
    lim_d = lim_d + bf16_half_ulp(np.abs(contract["o_ref"]) + lim_d)
    err_d = np.abs(o - contract["o_ref"])
    ok_d = np.all(err_d <= lim_d)
    lerr = np.abs(lse - contract["lse_ref"])
    ok_l = np.all(lerr <= lse_tol) and np.all(np.isfinite(lse))
    ratio_s = float(np.where(tight[..., None], err_s / lim_s, 0.0).max()) if o.size else 0.0
    return {"pass": bool(ok_s and ok_d and ok_l and np.all(np.isfinite(o))),
            "step_ok": bool(ok_s), "def_ok": bool(ok_d), "lse_ok": bool(ok_l),
            "step_ratio": ratio_s, "def_ratio": float((err_d / lim_d).max()) if o.size else 0.0,
            "max_abs": float(err_d.max()) if o.size else 0.0, "step_max_abs": float(err_s.max()) if o.size else 0.0,
            "step_allow_max": float(contract["allow_step"].max()) if o.size else 0.0,
            "lse_max_abs": float(lerr.max()) if o.size else 0.0,
            "sched_amb_rows": int(contract["sched_amb"].sum()), "rows": int(tight.size)}
