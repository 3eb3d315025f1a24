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


def check_fp8(o, lse, o_ref, lse_ref, allow, slack=1e-3, lse_tol=1e-3):
    """|O − O_ref| ≤ allowance + slack + ½ulp_bf16(O_ref) per element (slack: the
    fp32 sums and the hardware exp2) and |L − L_ref| ≤ lse_tol.  Returns a
    report dict with 'pass'."""
    from .compare import bf16_half_ulp
    o = np.asarray(o, np.float64)
    err = np.abs(o - o_ref)
    lim = allow + slack + bf16_half_ulp(o_ref)
    lerr = np.abs(np.asarray(lse, np.float64) - lse_ref)
    return {"pass": bool(np.all(err <= lim) and np.all(lerr <= lse_tol)), "max_abs": float(err.max()),
            "ratio": float((err / lim).max()), "lse_max_abs": float(lerr.max()), "allow_max": float(allow.max())}
