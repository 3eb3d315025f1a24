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
    """Inputs whose blocks are E4M3 codes times a power of two, and a scale whose
    base-2 form c = scale·log2(e) is a power of two in fp32 (scale = ln 2 / 4:
    fp32(ln 2 / 4)·fp32(log2 e) rounds to exactly 1/4), so that c·Q is
    representable too: quantising changes nothing and the FP8 attention is exact
    attention, to the last bit."""
    from oracle.fp8 import logit_scale_f32
    rng = np.random.default_rng(11)
    shape = (1, 2, 150, 16)
    q = _representable(rng, shape, 64, [-7, -9])
    k = _representable(rng, shape, 32, [-6, -8, -7])
    v = _representable(rng, shape, 32, [-5, -9])
    scale = LN2 / 4
    assert logit_scale_f32(scale) == np.float32(0.25)
    for causal in (False, True):
        o, l = attention_fp8_ref(q, k, v, scale, causal, q_block=64, kv_block=32)
        ro, rl = attention_ref(q, k, v, scale, causal)
        assert np.array_equal(o, ro) and np.array_equal(l, rl)


def test_fp8_attention_moves_away_from_exact_attention_by_the_rounding():
    """On N(0,1) inputs the block-quantised attention differs from exact
    attention, by less than what 2^-4 relative rounding of Q, K and V allows."""
    rng = np.random.default_rng(13)
    q, k, v = (rng.normal(0, 1, (1, 1, 300, 64)) for _ in range(3))
    o, l = attention_fp8_ref(q, k, v, 0.125, True)
    ro, rl = attention_ref(q, k, v, 0.125, True)
    assert 0 < np.abs(o - ro).max() < 0.25 and np.abs(l - rl).max() < 0.5


def _round_p_blocks(pt, pblock=32):
    """P̃ [R, N] rounded as the FP8 forward rounds it for its second product, in
    plain NumPy: each aligned block of ``pblock`` keys of a row is divided by the
    power of two 2^σ, σ = e − 8 with 2^(e−1) ≤ block sum < 2^e (at least −126),
    rounded to E4M3 and multiplied back."""
    R, N = pt.shape
    nb = -(-N // pblock)
    padded = np.zeros((R, nb * pblock))
    padded[:, :N] = pt
    sums = padded.reshape(R, nb, pblock).sum(axis=2)
    e = np.where(sums > 0, np.floor(np.log2(np.where(sums > 0, sums, 1.0))) + 1, 0)
    sk = np.repeat(2.0 ** np.maximum(e - 8, -126), pblock, axis=1)[:, :N]
    return e4m3_round(pt / sk) * sk


def _sim_kernel(q, k, v, scale, causal, shift, rng):
    """The FP8 forward's arithmetic on the CPU: P̃ against a reference max below
    the true one by up to `shift` (in natural-log units), block-quantised for the
    second product (_round_p_blocks), O divided by the sum of the unrounded P̃."""
    from oracle.fp8 import dequantize_blocks, prescale_q, quantize_blocks
    from oracle.ref import scores
    qh, kh, vh = (dequantize_blocks(*quantize_blocks(t, 64), 64) for t in (prescale_q(q, scale), k, v))
    o = np.empty(qh.shape)
    for b in range(qh.shape[0]):
        for h in range(qh.shape[1]):
            s = scores(qh[b, h], kh[b, h], LN2, causal)  # base-2 logits of c·Q, in natural-log units
            m = s.max(axis=1) - rng.uniform(0, shift, s.shape[0])
            pt = np.exp(s - m[:, None])
            o[b, h] = (_round_p_blocks(pt) @ vh[b, h]) / pt.sum(axis=1)[:, None]
    return o


def test_fp8_allowance_covers_the_kernel_arithmetic():
    """Random stale maxima up to the rescale threshold (2^48) and block-quantised
    E4M3 weights: the simulated kernel output stays within the bound on every
    element."""
    from oracle.fp8 import fp8_allowance
    rng = np.random.default_rng(17)
    shape = (1, 2, 200, 128)
    q = rng.normal(0, 1, shape)
    k = rng.normal(0, 1, shape)
    v = rng.normal(0, 1, shape)
    k[:, :, ::37] *= 6.0  # a few dominant keys: weights near 1 next to many subnormal ones
    for causal in (False, True):
        ro, rl, allow = fp8_allowance(q, k, v, 0.125, causal)
        for shift in (0.0, 8 * np.log(2), 48 * np.log(2)):
            o = _sim_kernel(q, k, v, 0.125, causal, shift, rng)
            err = np.abs(o - ro)
            assert np.all(err <= allow * (1 + 1e-9)), (causal, shift, float((err / allow).max()))


def test_round_p_blocks_pins():
    """The block rounding on hand-made rows: a block summing to 1 is scaled by
    2^-7 (its elements become codes below 2^7); 0.3 + 0.3 in one block (sum 0.6,
    σ = −8) both become 0.3·256 = 76.8 → 80 → 0.3125; a lone weight 2^-40 is
    exact (its block takes σ = −47); an all-zero block stays zero."""
    pt = np.zeros((3, 64))
    pt[0, 0] = 1.0
    pt[1, 0] = pt[1, 1] = 0.3
    pt[2, 40] = 2.0 ** -40
    r = _round_p_blocks(pt)
    assert r[0, 0] == 1.0 and r[2, 40] == 2.0 ** -40
    assert r[1, 0] == r[1, 1] == 0.3125
    assert not r[:, 2:40].any() and not r[0, 1:].any()


# ---- the kernel-step model and the tight FP8 contract ---------------------------------

from oracle.compare import bf16_rne
from oracle.fp8 import check_fp8, fp8_contract, fp8_step_model, mma_runs, v_tile_key

import synth

LN2 = float(np.log(2.0))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 300])
def test_step_model_without_rounding_is_the_definition(N, causal):
    """With P̃ left unrounded and exact matrix products, the model's reference-max
    schedule and the block scales of P̃ change nothing in exact arithmetic
    ([cicada] §5: ℓ and the accumulator share the stale max): O and L equal
    exact attention of the dequantised inputs."""
    w = synth.WORKLOADS[2].with_(B=1, H=2, N=N, causal=causal, boost_frac=0.03, wid=900 + N + causal)
    q, k, v = synth.make_prefill(w)
    # a low threshold, so that the boosted keys move the reference max
    m = fp8_step_model(q, k, v, w.scale, causal, round_p=False, mma_exact=True, threshold=4.0)
    o, l = attention_fp8_ref(q, k, v, w.scale, causal)
    assert np.allclose(m["o"], o, rtol=1e-12, atol=1e-13) and np.allclose(m["lse"], l, rtol=1e-13, atol=1e-12)
    if N >= 300:
        assert m["moves"].max() >= 2  # the boosted keys did move the reference max


def _integer_logit_inputs(N, grow_at=None, grow_row=0, grow=51.0, base=3.0):
    """q̂, k̂ for scale = ln 2 (so the base-2 logits are t = q̂·k̂): t_ij = −(j mod 3);
    from key ``grow_at`` on every row's logits are ``base`` higher, and those of
    row ``grow_row`` ``grow`` higher (grow − base must stay an E4M3 value after
    the K block's scale: 48 with base 3, and 40, 44, 48, 52 with base 4 do)."""
    d = 128
    q = np.zeros((1, 1, N, d))
    k = np.zeros((1, 1, N, d))
    q[0, 0, :, 0] = 1.0
    k[0, 0, :, 0] = -(np.arange(N) % 3)
    q[0, 0, :, 2] = 1.0
    q[0, 0, grow_row, 1] = 1.0
    if grow_at is not None:
        k[0, 0, grow_at:, 2] = base
        k[0, 0, grow_at:, 1] = grow - base
    v = np.random.default_rng(N).normal(0, 1, (1, 1, N, d))
    return q, k, v


def test_step_model_is_exact_on_representable_weights():
    """Logits that are integers in base 2 make every P̃ an exact power of two, and
    so every block-scaled code (a power of two between 2^-2 and 2^7 times the
    block's largest): rounding changes nothing, and with exact matrix products
    the model equals the definition, although the keys at +51 (row 250) move the
    reference max of the row's whole group while the next group, whose rows grow
    by 3 only, keeps its stale max."""
    q, k, v = _integer_logit_inputs(300, grow_at=192, grow_row=250)
    for causal in (False, True):
        m = fp8_step_model(q, k, v, LN2, causal, mma_exact=True)
        o, l = attention_fp8_ref(q, k, v, LN2, causal)
        assert np.allclose(m["o"], o, rtol=1e-13, atol=1e-14) and np.allclose(m["lse"], l, rtol=1e-14, atol=1e-13)
        assert np.all(m["amb"] == 0)  # exact weights sit far from every rounding boundary
        assert np.all(m["moves"][0, 0, 224:256] == 2)          # the group of row 250 moved at the key tile 192
        assert np.all(m["moves"][0, 0, 256:300] == 1)          # growth 3 only: the stale max is kept
        assert np.all(m["moves"][0, 0, :192] == 1)


def test_step_model_schedule():
    """The reference max of a 32-row group moves for every row of the group when
    one row outgrows it by more than 2^48 (growths 56 and 52, E4M3-exact after
    quantisation), not at 44, and a growth within the fp32 error bound of the
    threshold (48 exactly) is flagged.  The scale enters through the quantised
    codes of c·Q, so nudging it by 1e-9 either way leaves c = 1 in fp32 and the
    growth at 48 exactly: not moved, flagged."""
    cases = [(56.0, 1.0, 2, False), (52.0, 1.0, 2, False), (44.0, 1.0, 1, False),
             (48.0, 1.0 + 1e-9, 1, True), (48.0, 1.0 - 1e-9, 1, True), (48.0, 1.0, 1, True)]
    for grow, f, moves, amb in cases:
        q, k, v = _integer_logit_inputs(300, grow_at=128, grow_row=3, grow=grow, base=4.0)
        m = fp8_step_model(q, k, v, LN2 * f, False)
        assert np.all(m["moves"][0, 0, :32] == moves), (grow, f)  # the whole group of row 3
        assert np.all(m["moves"][0, 0, 32:] == 1), (grow, f)      # other groups: only the first tile
        assert np.all(m["sched_amb"][0, 0, :32] == amb) and not m["sched_amb"][0, 0, 32:].any(), (grow, f)


def test_step_model_within_the_schedule_free_bound():
    """The model (a particular schedule, the matrix instruction's truncation)
    stays within fp8_allowance + fp8_mma_allowance, the bounds derived for any
    stale max up to 2^8, any E4M3 rounding of P̃ and any truncation of the
    instruction's runs."""
    w = synth.WORKLOADS[2].with_(B=1, H=2, N=400, causal=True, boost_frac=0.02, wid=931)
    q, k, v = synth.make_prefill(w)
    for causal in (False, True):
        con = fp8_contract(q, k, v, w.scale, causal)
        assert np.all(np.abs(con["o"] - con["o_ref"]) <= (con["allow_def"] + con["allow_mma"]) * (1 + 1e-9))


def _brute_runs(a, b, run=8, keep=13):
    """The matrix instruction's rule product by product, in plain Python."""
    import math
    R, K = a.shape
    C = b.shape[1]
    out = np.zeros((R, K // run, C))
    for r in range(R):
        for c in range(C):
            for g in range(K // run):
                ps = [(float(a[r, k]), float(b[k, c])) for k in range(g * run, (g + 1) * run)]
                es = [max(math.frexp(x)[1] - 1, -6) + max(math.frexp(y)[1] - 1, -6) for x, y in ps if x * y != 0]
                if not es:
                    continue
                q = 2.0 ** (max(es) - keep)
                out[r, g, c] = sum(math.trunc(x * y / q) * q for x, y in ps)
    return out


def test_mma_runs_rule():
    """mma_runs against the rule written out product by product, and the rule's
    own consequences: beside a product 256·1 (exponent sum 8) a small product is
    cut to a multiple of 2^-5, toward zero; 22·56 = 1232 has exponent sum 4 + 5
    = 9, so 0.109375 beside it keeps a multiple of 2^-4 (0.0625); zero products
    do not widen the grid; separate runs do not affect each other."""
    rng = np.random.default_rng(21)
    vals = TABLE[~np.isnan(TABLE)]
    a = rng.choice(vals, (5, 64))
    b = rng.choice(vals, (64, 3))
    a[:, 8:16] *= 0  # a run of zero products
    got, _ = mma_runs(torch.from_numpy(a), torch.from_numpy(b))
    assert np.array_equal(got.numpy(), _brute_runs(a, b))
    a = np.zeros((3, 64))
    b = np.zeros((64, 3))   # case r uses row r of a and column r of b
    a[0, 0], b[0, 0] = 256.0, 1.0
    a[0, 1], b[1, 0] = -TABLE[np.argmin(np.abs(TABLE[:0x7F] - 0.0825))], 1.0   # −0.08203125 → −0.0625
    a[1, 0], b[0, 1] = 22.0, 56.0
    a[1, 1], b[1, 1] = 0.109375, 1.0
    a[1, 3], b[3, 1] = 448.0, 0.0                                                  # a zero product
    a[2, 0], b[0, 2] = 256.0, 1.0
    a[2, 8], b[8, 2] = 0.1171875, 1.0                                              # run 1 is its own
    got, _ = mma_runs(torch.from_numpy(a), torch.from_numpy(b))
    g = got.numpy()
    assert g[0, 0, 0] == 256.0 - 0.0625
    assert g[1, 0, 1] == 1232.0 + 0.0625
    assert g[2, 0, 2] == 256.0 and g[2, 1, 2] == 0.1171875
    exact, _ = mma_runs(torch.from_numpy(a), torch.from_numpy(b), exact=True)
    assert np.allclose(exact.numpy().sum(1), a @ b)


def test_v_tile_key_is_a_permutation():
    keys = [v_tile_key(j) for j in range(64)]
    assert sorted(keys) == list(range(64))
    assert keys[:8] == [0, 1, 2, 3, 8, 9, 10, 11] and keys[32:36] == [4, 5, 6, 7]


def _instr_f32(a, b, acc, run_scale=None):
    """One FP8 matrix instruction in float32, written apart from the oracle's
    mma_runs: for each run of 8 reduction indices the products, each cut toward
    zero to the grid 2^(E−13) of the run's largest exponent sum, are summed (the
    sum is exact in fp32) and times the run's power-of-two operand scale
    (``run_scale`` [R, 8], 1 by default); the eight run sums are then added to
    ``acc`` one by one in float32.  a [R, 64], b [64, C], acc [R, C] float32
    tensors."""
    R, C = a.shape[0], b.shape[1]
    ea = torch.where(a != 0, torch.frexp(a)[1].float() - 1, torch.full_like(a, -1e4)).clamp(min=-6)
    eb = torch.where(b != 0, torch.frexp(b)[1].float() - 1, torch.full_like(b, -1e4)).clamp(min=-6)
    for g in range(8):
        p = a[:, 8 * g:8 * g + 8, None] * b[None, 8 * g:8 * g + 8, :]                  # exact in float32
        e = torch.where(p != 0, ea[:, 8 * g:8 * g + 8, None] + eb[None, 8 * g:8 * g + 8, :],
                        torch.full_like(p, -1e4))
        grid = torch.exp2((e.amax(1) - 13).clamp(min=-126))[:, None, :]
        run = (torch.trunc(p / grid) * grid).sum(1)
        acc = acc + (run if run_scale is None else run * run_scale[:, g:g + 1])
    return acc


def _sim_fp32_kernel(q, k, v, scale, causal, rows, flush=False):
    """A float32 re-enactment of the FP8 forward's arithmetic, written apart from
    the model: logits from two float32 matrix instructions on the E4M3 codes times
    the block scales, exp2 and sums in float32, the reference max of each 32-row
    group moved when one of its rows outgrows it by more than 2^48, P̃ of each
    row's 32-key half tile divided by 2^σ (σ from the float32 sum of the half)
    and rounded to E4M3 by torch's float8_e4m3fn conversion, the second product
    by the instruction on the keys in the V tile order with each run scaled by
    its half's 2^σ, O = acc·(1/ℓ) rounded to bf16, L = (m + log2 ℓ)·ln 2.  Q is
    quantised as c·Q (c = scale·log2 e in fp32), so the logits are base 2; the
    first instruction of a tile starts from −m (m when the tile's products are
    issued, 0 while it is −∞) with the block scales applied to each run, and a
    tile that moves m re-offsets its logits in float32.  ``flush``: exp2 returns
    0 for results below fp32's normal range.  Returns (O, L) on the rows of
    every 32-row group that holds one of ``rows``."""
    from oracle.fp8 import quantize_blocks
    c = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    qc = (torch.as_tensor(q).float().numpy() * c).astype(np.float32)   # c·Q, one float32 rounding
    (q8, qs), (k8, ks), (v8, vs) = (quantize_blocks(t, 64) for t in (qc, k, v))
    B, H, N, d = q8.shape
    order = [32 * ((j >> 4) & 1) + 8 * ((j & 15) >> 2) + 4 * (j >> 5) + (j & 3) for j in range(64)]
    run_half = [order[8 * g] // 32 for g in range(8)]  # the 32-key half tile each run of 8 slots holds
    groups = np.unique(np.asarray(rows) // 32)
    outs_o, outs_l = [], []
    f = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    for g in groups:
        r = np.arange(32 * g, min(N, 32 * g + 32))
        o = np.zeros((B, H, r.size, d), np.float32)
        lse = np.zeros((B, H, r.size), np.float32)
        for b in range(B):
            for h in range(H):
                qr = f(q8[b, h][r])
                sq = np.float32(qs[b, h][r[0] // 64])
                m = np.full(r.size, -np.inf, np.float32)
                ell = np.zeros(r.size, np.float32)
                acc = torch.zeros((r.size, d), dtype=torch.float32)
                mo = np.zeros(r.size, np.float32)      # the offset the tiles' logits start from
                for j in range(0, N, 64):
                    kt = np.zeros((64, d), np.float32)
                    kt[:min(64, N - j)] = k8[b, h][j:j + 64]
                    rs = torch.full((r.size, 8), float(np.float32(sq * np.float32(ks[b, h][j // 64]))))
                    s = torch.from_numpy(np.repeat(-mo[:, None], 64, axis=1))
                    for half in (0, 1):
                        s = _instr_f32(qr[:, 64 * half:64 * half + 64], f(kt[:, 64 * half:64 * half + 64].T), s,
                                       run_scale=rs)
                    s = s.numpy()
                    keys = j + np.arange(64)
                    dead = keys[None, :] >= N
                    if causal:
                        dead = dead | (keys[None, :] > r[:, None])
                    s = np.where(dead, np.float32(-np.inf), s)
                    if not np.isfinite(s).any():
                        continue
                    mt = (s.max(axis=1) + mo).astype(np.float32)       # the tile's row max, base 2
                    with np.errstate(invalid="ignore"):
                        grow = mt - m
                    off = np.zeros(r.size, np.float32)
                    if np.any(grow > np.float32(48.0)):
                        mn = np.fmax(m, mt)
                        with np.errstate(invalid="ignore"):
                            al = np.exp2(m - mn).astype(np.float32)
                        al = np.where(np.isneginf(m), np.float32(0), al)
                        ell, acc, m = ell * al, acc * torch.from_numpy(al)[:, None], mn
                        off = (mo - m).astype(np.float32)
                        mo = m.copy()
                    with np.errstate(invalid="ignore"):
                        x = np.exp2((s + off[:, None]).astype(np.float32)).astype(np.float32)
                    x = np.where(np.isfinite(s), x, np.float32(0))
                    if flush:
                        x = np.where(x < np.float32(2.0 ** -126), np.float32(0), x)
                    half_sum = np.stack([x[:, :32].sum(axis=1, dtype=np.float32),
                                         x[:, 32:].sum(axis=1, dtype=np.float32)], axis=1)
                    sig = np.maximum(np.frexp(half_sum)[1] - 8, -126)
                    sc = np.ldexp(np.float32(1), sig).astype(np.float32)          # [rows, 2]
                    x8 = torch.from_numpy(x / np.repeat(sc, 32, axis=1)).to(torch.float8_e4m3fn).float()
                    vt = np.zeros((64, d), np.float32)
                    vt[:min(64, N - j)] = v8[b, h][j:j + 64]
                    acc = _instr_f32(x8[:, order], f(vt[order] * np.float32(vs[b, h][j // 64])), acc,
                                     run_scale=torch.from_numpy(sc[:, run_half]))
                    ell = (ell + x.sum(axis=1, dtype=np.float32)).astype(np.float32)
                o[b, h] = (acc * torch.from_numpy(np.float32(1) / ell)[:, None]).numpy()
                lse[b, h] = (m + np.log2(ell)) * np.float32(np.log(2.0))
        outs_o.append(o)
        outs_l.append(lse)
    o = torch.from_numpy(np.concatenate(outs_o, axis=2)).to(torch.bfloat16).double().numpy()
    return o, np.concatenate(outs_l, axis=2).astype(np.float64)


# (workload, heads, rows): every FP8 shape the GPU tests use, in small and at full size
FP8_SHAPES = [(synth.WORKLOADS[2].with_(B=1, H=2, N=n, causal=c, boost_frac=0.01, wid=250 + n + c), [0, 1], None)
              for n in (1, 7, 64, 65, 300, 513) for c in (False, True)]
FP8_SHAPES += [(synth.WORKLOADS[2], [17], np.array([0, 40, 2100, 4064, 4095])),      # c3: early and late rows
               (synth.WORKLOADS[3], [3], np.array([64, 16383]))]                      # long non-causal


def _shape_id(s):
    w, _, rows = s
    return f"{w.name}-N{w.N}-{'c' if w.causal else 'nc'}" + ("-sampled" if rows is not None else "")


def _inputs(w, heads):
    q, k, v = synth.make_prefill(w)
    return q[:, heads], k[:, heads], v[:, heads]


@pytest.mark.parametrize("shape", [s for s in FP8_SHAPES if s[0].N in (65, 513, 4096, 16384)], ids=_shape_id)
def test_fp32_kernel_simulation_passes(shape):
    """An fp32 re-enactment of the kernel's arithmetic meets the tight rule: the
    step allowance covers fp32 logits, exp2, sums and the output rounding."""
    w, heads, rows = shape
    q, k, v = _inputs(w, heads)
    con = fp8_contract(q, k, v, w.scale, w.causal, rows=rows)
    o, l = _sim_fp32_kernel(q, k, v, w.scale, w.causal, con["rows"])
    rep = check_fp8(o, l, con)
    assert rep["pass"], rep
    assert rep["sched_amb_rows"] == 0


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_kernel_simulation_with_large_logits(causal):
    """Keys ×64: the logits span hundreds of octaves, the reference max moves
    several times a row and many 32-key blocks sum to far below 2^-100 of it.
    The fp32 re-enactment passes the tight rule whether its exp2 keeps
    subnormal results or flushes them, and no row is left to the loose bound."""
    w = synth.WORKLOADS[2].with_(B=1, H=2, N=600, causal=causal, boost_frac=0.03, boost=64.0, wid=777 + causal)
    q, k, v = synth.make_prefill(w)
    con = fp8_contract(q, k, v, w.scale, causal)
    assert con["moves"].max() >= 4
    for flush in (False, True):
        o, l = _sim_fp32_kernel(q, k, v, w.scale, causal, con["rows"], flush=flush)
        rep = check_fp8(o, l, con)
        assert rep["pass"], (flush, rep)
        assert rep["sched_amb_rows"] == 0


def _slips(q, k, v, w, con):
    """Outputs of planted slips of the kernel step (each a model run on altered
    inputs or without the rounding), on the contract's rows."""
    rows = con["rows"]
    model = lambda q_, k_, v_, **kw: fp8_step_model(q_, k_, v_, w.scale, w.causal, rows=rows, **kw)
    N = q.shape[2]
    out = {"zero O": (np.zeros_like(con["o"]), con["lse"])}
    T = -(-N // 64)
    vpad = torch.zeros((*v.shape[:2], T * 64, v.shape[3]), dtype=v.dtype)
    vpad[:, :, :N] = v  # keys of every V tile in reverse order (the tile padded with zero keys)
    vp = vpad.reshape(*v.shape[:2], T, 64, v.shape[3]).flip(3).reshape(vpad.shape)[:, :, :N].contiguous()
    m = model(q, k, vp)
    out["V keys permuted in a tile"] = (bf16_rne(m["o"]), m["lse"])
    for name in ("q", "k", "v"):  # one block's scale one exponent too large
        x = {"q": q.clone(), "k": k.clone(), "v": v.clone()}
        blk = int(rows[-1]) // 64 if name == "q" else 0
        x[name][:, :, blk * 64:(blk + 1) * 64] *= 2
        m = model(x["q"], x["k"], x["v"])
        out[f"{name} block scale ×2"] = (bf16_rne(m["o"]), m["lse"])
    if N > 1:  # one key: P̃ = 1 is exact, so rounding it cannot be missed or caught
        m = model(q, k, v, round_p=False, mma_exact=True)
        out["P̃ not rounded"] = (bf16_rne(m["o"]), m["lse"])
    return out


@pytest.mark.parametrize("shape", FP8_SHAPES, ids=_shape_id)
def test_fp8_rule_rejects_planted_slips(shape):
    """Each planted slip of the FP8 step fails the rule at every shape the GPU
    tests use, including N = 16384 non-causal and the Llama-3-shaped late rows;
    the faithful model (rounded to bf16) passes."""
    w, heads, rows = shape
    q, k, v = _inputs(w, heads)
    con = fp8_contract(q, k, v, w.scale, w.causal, rows=rows)
    assert check_fp8(bf16_rne(con["o"]), con["lse"], con)["pass"]
    for name, (o, l) in _slips(q, k, v, w, con).items():
        rep = check_fp8(o, l, con)
        assert not rep["pass"], (name, rep)
