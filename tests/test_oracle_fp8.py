"""Pins of the oracle's block-wise FP8 quantisation (oracle/fp8.py) against
things other than itself: PyTorch's own float8_e4m3fn conversion (a library
routine), the format's bit-level definition, brute-force nearest-value search
over all 256 codes, the rounding-error bound of a 3-bit mantissa, and inputs
that the quantisation must reproduce exactly."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import attention_ref
from oracle.fp8 import (E4M3_MAX, attention_fp8_ref, dequantize_blocks, e4m3_decode_table, e4m3_round,
                        quantize_blocks)

TABLE = e4m3_decode_table()


def test_decode_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    want = codes.view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(TABLE), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(TABLE[ok], want[ok])


def test_decode_table_landmarks():
    assert TABLE[0x38] == 1.0 and TABLE[0xB8] == -1.0
    assert TABLE[0x7E] == E4M3_MAX == 448.0
    assert TABLE[0x01] == 2.0 ** -9 and TABLE[0x08] == 2.0 ** -6 and TABLE[0x07] == 7 * 2.0 ** -9
    assert np.isnan(TABLE[0x7F]) and np.isnan(TABLE[0xFF]) and int(np.isnan(TABLE).sum()) == 2
    pos = TABLE[:0x7F]
    assert np.all(np.diff(pos) > 0)  # codes 0 .. 0x7E increase strictly


def _brute_round(x):
    """Nearest finite table value, ties to the even code, saturating at ±448."""
    fin = np.flatnonzero(~np.isnan(TABLE) & (TABLE >= 0))
    vals = TABLE[fin]
    out = []
    for xi in np.atleast_1d(x):
        a = min(abs(xi), E4M3_MAX)
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        pick = best[0] if len(best) == 1 else [b for b in best if fin[b] % 2 == 0][0]
        out.append(np.copysign(vals[pick], xi))
    return np.array(out)


def test_round_matches_brute_force_on_midpoints_and_random_values():
    pos = TABLE[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(3)
    xs = np.concatenate([pos, mids, -mids, rng.uniform(-448, 448, 2000), rng.uniform(-0.02, 0.02, 2000),
                         np.nextafter(mids, 0), np.nextafter(mids, 1000)])
    assert np.array_equal(e4m3_round(xs), _brute_round(xs))


def test_round_matches_torch_within_range():
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.normal(0, 30, 5000), rng.normal(0, 0.01, 5000),
                         (TABLE[:0x7E] + TABLE[1:0x7F]) / 2])
    xs = xs[np.abs(xs) <= 448]
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(e4m3_round(xs), want)


def test_round_saturates():
    xs = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, -500.0, -1e30])
    assert np.array_equal(e4m3_round(xs), np.array([448, 448, 448, 448, 448, 448, -448, -448], dtype=float))


def test_quantize_blocks_scale_error_and_independence():
    rng = np.random.default_rng(7)
    x = rng.normal(0, 1, (2, 3, 200, 16))
    x[0, 1, 64:128] *= 50.0               # an outlier block
    x[1, 2, 128:192] = 0.0                 # an all-zero block
    x8, s = quantize_blocks(x, 64)
    assert s.shape == (2, 3, 4)
    assert np.all(np.isin(np.abs(x8), np.abs(TABLE[:0x7F])))      # every stored value is an E4M3 value
    amax8 = np.abs(x8.reshape(2, 3, -1, 16)[:, :, :192].reshape(2, 3, 3, 64, 16)).max(axis=(-2, -1))
    assert np.all(((amax8 > 224) & (amax8 <= 448)) | (s[..., :3] == 1.0))
    assert np.all(np.log2(s) == np.round(np.log2(s)))                # powers of two
    amax = np.abs(x.reshape(2, 3, -1, 16)[:, :, :192].reshape(2, 3, 3, 64, 16)).max(axis=(-2, -1))
    nz = amax > 0
    assert np.all(amax[nz] / s[..., :3][nz] <= 448) and np.all(amax[nz] / s[..., :3][nz] > 224)
    assert s[1, 2, 2] == 1.0 and np.all(x8[1, 2, 128:192] == 0)
    xh = dequantize_blocks(x8, s, 64)
    rep = np.repeat(s, 64, axis=-1)[..., :200, None]
    err = np.abs(xh - x)
    # 3 mantissa bits: half a spacing is at most 2^-4 of the magnitude for normal
    # values, and 2^-10 (half of 2^-9) in units of the scale for subnormal ones
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, rep * 2.0 ** -10) * (1 + 1e-12))
    # changing one block leaves the others alone
    y = x.copy()
    y[0, 0, 70] = 1e3
    y8, t = quantize_blocks(y, 64)
    assert np.array_equal(np.delete(y8[0, 0], np.s_[64:128], axis=0), np.delete(x8[0, 0], np.s_[64:128], axis=0))
    assert np.array_equal(np.delete(t[0, 0], 1), np.delete(s[0, 0], 1)) and t[0, 0, 1] != s[0, 0, 1]


def test_quantize_blocks_ragged_tail_and_2d():
    x = np.linspace(-3, 5, 70 * 8).reshape(70, 8)
    x8, s = quantize_blocks(x, 64)
    assert s.shape == (2,)
    assert 224 < np.abs(x8[64:]).max() <= 448 and 224 < np.abs(x8[:64]).max() <= 448
    assert np.allclose(dequantize_blocks(x8, s, 64), x, rtol=2.0 ** -4, atol=s.max() * 2.0 ** -10)


def _representable(rng, shape, block, scales_log2):
    """Values s·c with c drawn from the E4M3 table and each block holding ±448 once,
    s a power of two per block: the block quantisation must give them back exactly."""
    fin = TABLE[~np.isnan(TABLE)]
    c = rng.choice(fin, size=shape)
    B, H, N, d = shape
    out = np.empty(shape)
    for b0 in range(0, N, block):
        c[:, :, b0, 0] = 448.0
        s = 2.0 ** scales_log2[(b0 // block) % len(scales_log2)]
        out[:, :, b0:b0 + block] = c[:, :, b0:b0 + block] * s
    return out


def test_fp8_attention_is_exact_attention_on_representable_inputs():
    rng = np.random.default_rng(11)
    shape = (1, 2, 150, 16)
    q = _representable(rng, shape, 64, [-7, -9])
    k = _representable(rng, shape, 32, [-6, -8, -7])
    v = _representable(rng, shape, 32, [-5, -9])
    for causal in (False, True):
        o, l = attention_fp8_ref(q, k, v, 0.25, causal, q_block=64, kv_block=32)
        ro, rl = attention_ref(q, k, v, 0.25, causal)
        assert np.array_equal(o, ro) and np.array_equal(l, rl)


def test_fp8_attention_moves_away_from_exact_attention_by_the_rounding():
    """On N(0,1) inputs the block-quantised attention differs from exact
    attention, by less than what 2^-4 relative rounding of Q, K and V allows."""
    rng = np.random.default_rng(13)
    q, k, v = (rng.normal(0, 1, (1, 1, 300, 64)) for _ in range(3))
    o, l = attention_fp8_ref(q, k, v, 0.125, True)
    ro, rl = attention_ref(q, k, v, 0.125, True)
    assert 0 < np.abs(o - ro).max() < 0.25 and np.abs(l - rl).max() < 0.5


def _sim_kernel(q, k, v, scale, causal, shift, rng):
    """The FP8 forward's arithmetic on the CPU: P̃ against a reference max below
    the true one by up to `shift` (in natural-log units), rounded to E4M3 for the
    second product, O divided by the sum of the unrounded P̃."""
    from oracle.fp8 import dequantize_blocks, quantize_blocks
    from oracle.ref import scores
    qh, kh, vh = (dequantize_blocks(*quantize_blocks(t, 64), 64) for t in (q, k, v))
    o = np.empty(qh.shape)
    for b in range(qh.shape[0]):
        for h in range(qh.shape[1]):
            s = scores(qh[b, h], kh[b, h], scale, causal)
            m = s.max(axis=1) - rng.uniform(0, shift, s.shape[0])
            pt = np.exp(s - m[:, None])
            o[b, h] = (e4m3_round(pt) @ vh[b, h]) / pt.sum(axis=1)[:, None]
    return o


def test_fp8_allowance_covers_the_kernel_arithmetic():
    """Random stale maxima up to the rescale threshold (2^8) and E4M3 weights:
    the simulated kernel output stays within the bound on every element."""
    from oracle.fp8 import fp8_allowance
    rng = np.random.default_rng(17)
    shape = (1, 2, 200, 128)
    q = rng.normal(0, 1, shape)
    k = rng.normal(0, 1, shape)
    v = rng.normal(0, 1, shape)
    k[:, :, ::37] *= 6.0  # a few dominant keys: weights near 1 next to many subnormal ones
    for causal in (False, True):
        ro, rl, allow = fp8_allowance(q, k, v, 0.125, causal)
        for shift in (0.0, 8 * np.log(2)):
            o = _sim_kernel(q, k, v, 0.125, causal, shift, rng)
            err = np.abs(o - ro)
            assert np.all(err <= allow * (1 + 1e-9)), (causal, shift, float((err / allow).max()))
