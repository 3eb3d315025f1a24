"""Pins for the fp64 oracle: closed forms, brute force, library special cases,
invariants, and the method's algebra (online = two-pass, ⊕ associativity).

Each test ties the oracle to something other than itself, chosen so that a
plausible slip (a dropped scale, a wrong mask direction, a transposed operand,
an LSE without its max) fails at least one of them; ``test_pins_catch_mistakes``
plants exactly those slips in copies of the oracle and checks that they fail.
"""

import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import (attention_block_sparse_ref, attention_bwd_ref, attention_ref, decode_gqa_ref, decode_paged_ref,
                    decode_ref, safe_softmax, scores)
from oracle.compare import bf16_half_ulp, bf16_rne, bwd_allowance, check_bwd, check_prefill
import _method_fp64 as M

GOLD = os.path.join(os.path.dirname(__file__), "golden", "closed_form_4tok.json")


def _fx():
    with open(GOLD) as f:
        return json.load(f)


def _frac_mat(rows):
    return [[Fraction(x) for x in r] for r in rows]


def _fixture_inputs(fx):
    w = np.array([[float(Fraction(x)) for x in r] for r in fx["w"]])
    q = np.log(w)[None, None]
    k = (2.0 * np.eye(4))[None, None]
    v = np.array(fx["v"], dtype=np.float64)[None, None]
    return q, k, v, float(Fraction(fx["scale"]))


# --------------------------------------------------------------------------
# closed form


def test_fixture_is_self_consistent():
    """P rows are the normalised visible weights and O = P·V, in exact rationals."""
    fx = _fx()
    w = _frac_mat(fx["w"])
    v = [[Fraction(x) for x in r] for r in fx["v"]]
    p = _frac_mat(fx["causal"]["p"])
    for i in range(4):
        tot = sum(w[i][: i + 1])
        for j in range(4):
            assert p[i][j] == (w[i][j] / tot if j <= i else 0)
        assert Fraction(fx["causal"]["lse_ln_of"][i]) == tot
    for mode in ("causal", "noncausal"):
        o = _frac_mat(fx[mode]["o"])
        for i in range(4):
            vis = range(i + 1) if mode == "causal" else range(4)
            tot = sum(w[i][j] for j in vis)
            assert Fraction(fx[mode]["lse_ln_of"][i]) == tot
            for c in range(4):
                assert o[i][c] == sum(w[i][j] * v[j][c] for j in vis) / tot


@pytest.mark.parametrize("mode", ["causal", "noncausal"])
def test_oracle_matches_closed_form(mode):
    fx = _fx()
    q, k, v, scale = _fixture_inputs(fx)
    o, lse = attention_ref(q, k, v, scale, causal=(mode == "causal"))
    want_o = np.array([[float(x) for x in r] for r in _frac_mat(fx[mode]["o"])])
    want_l = np.array([math.log(int(x)) for x in fx[mode]["lse_ln_of"]])
    np.testing.assert_allclose(o[0, 0], want_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], want_l, rtol=0, atol=1e-13)
    if mode == "causal":
        p, _, _ = safe_softmax(scores(q[0, 0], k[0, 0], scale, True))
        want_p = np.array([[float(x) for x in r] for r in _frac_mat(fx["causal"]["p"])])
        np.testing.assert_allclose(p, want_p, rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# 50-digit brute force with the naive definition (valid: nothing overflows)


def _decimal_attention(q, k, v, scale, causal):
    getcontext().prec = 50
    n, d = q.shape
    dq = [[Decimal(float(x)) for x in r] for r in q]
    dk = [[Decimal(float(x)) for x in r] for r in k]
    dv = [[Decimal(float(x)) for x in r] for r in v]
    ds = Decimal(scale)
    o = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i in range(n):
        vis = range(i + 1) if causal else range(k.shape[0])
        e = {j: (ds * sum(dq[i][t] * dk[j][t] for t in range(d))).exp() for j in vis}
        tot = sum(e.values())
        for c in range(v.shape[1]):
            o[i, c] = float(sum(e[j] * dv[j][c] for j in vis) / tot)
        lse[i] = float(tot.ln())
    return o, lse


@pytest.mark.parametrize("seed", range(8))
def test_oracle_matches_decimal_bruteforce(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 9))
    d = int(rng.integers(1, 9))
    causal = bool(seed % 2)
    q = rng.standard_normal((1, 1, n, d))
    k = rng.standard_normal((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, d))
    scale = 1.0 / math.sqrt(d)
    o, lse = attention_ref(q, k, v, scale, causal)
    wo, wl = _decimal_attention(q[0, 0], k[0, 0], v[0, 0], scale, causal)
    np.testing.assert_allclose(o[0, 0], wo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], wl, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# special cases that reduce to a library routine or a closed form


@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_give_library_softmax(causal):
    """With V = I the output rows are the softmax rows themselves."""
    rng = np.random.default_rng(7)
    n, d = 11, 5
    q = rng.standard_normal((1, 1, n, d)) * 2
    k = rng.standard_normal((1, 1, n, d)) * 2
    v = np.eye(n)[None, None]
    scale = 0.37
    o, lse = attention_ref(q, k, v, scale, causal)
    logits = scale * (q[0, 0] @ k[0, 0].T)
    if causal:
        logits = np.where(np.triu(np.ones((n, n), bool), 1), -np.inf, logits)
    np.testing.assert_allclose(o[0, 0], scipy.special.softmax(logits, axis=1), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], scipy.special.logsumexp(logits, axis=1), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_give_running_mean(causal):
    """K = 0 makes every visible weight equal: O is a (cumulative) mean of V, L = ln(#visible)."""
    rng = np.random.default_rng(3)
    n, d = 37, 6
    q = rng.standard_normal((1, 1, n, d))
    k = np.zeros((1, 1, n, d))
    v = rng.standard_normal((1, 1, n, d))
    o, lse = attention_ref(q, k, v, 0.5, causal)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    want = np.cumsum(v[0, 0], axis=0) / cnt[:, None] if causal else np.broadcast_to(v[0, 0].mean(0), (n, d))
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], np.log(cnt), rtol=0, atol=1e-14)


def test_huge_logits_stay_finite_and_exact():
    """Logits near 1000 overflow the naive exp; the safe softmax gives the closed form."""
    q = np.array([[[[1000.0, 1000.0 + math.log(3.0)], [5.0, 5.0]]]])
    k = np.eye(2)[None, None]
    v = np.array([[[[4.0, -8.0], [0.0, 12.0]]]])
    with np.errstate(over="ignore"):
        assert not np.isfinite(np.exp(q[0, 0, 0]).sum())      # the naive form overflows
    o, lse = attention_ref(q, k, v, 1.0, causal=False)
    np.testing.assert_allclose(o[0, 0, 0], [1.0, 7.0], rtol=0, atol=1e-12)   # P = [1/4, 3/4]
    np.testing.assert_allclose(lse[0, 0, 0], 1000.0 + math.log(4.0), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# invariants


@pytest.mark.parametrize("causal", [False, True])
def test_probability_invariants(causal):
    rng = np.random.default_rng(11)
    n, d = 50, 16
    q = rng.standard_normal((n, d)) * 3
    k = rng.standard_normal((n, d)) * 3
    s = scores(q, k, 0.25, causal)
    p, m, l = safe_softmax(s)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)
    if causal:
        assert np.all(p[np.triu(np.ones((n, n), bool), 1)] == 0.0)   # masked weights are exactly zero
        assert np.all(np.isneginf(s[np.triu(np.ones((n, n), bool), 1)]))


def test_causal_row0_sees_only_key0():
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((2, 3, 9, 4)) for _ in range(3))
    o, lse = attention_ref(q, k, v, 0.3, causal=True)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), rtol=0, atol=1e-14)


def test_row_subset_equals_full():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 2, 40, 8)) for _ in range(3))
    rows = np.array([0, 3, 17, 39])
    for causal in (False, True):
        o, lse = attention_ref(q, k, v, 0.5, causal)
        os_, ls_ = attention_ref(q, k, v, 0.5, causal, rows=rows)
        np.testing.assert_array_equal(os_, o[:, :, rows])
        np.testing.assert_array_equal(ls_, lse[:, :, rows])


# --------------------------------------------------------------------------
# the method's algebra against the oracle


@pytest.mark.parametrize("seed", range(6))
def test_online_blocked_equals_two_pass(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 200))
    d = int(rng.choice([4, 16, 64]))
    causal = bool(seed % 2)
    br, bc = int(rng.integers(1, 70)), int(rng.integers(1, 70))
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    k[rng.choice(n, size=max(1, n // 20), replace=False)] *= 8.0     # force rescales
    o, lse = attention_ref(q[None, None], k[None, None], v[None, None], 1 / math.sqrt(d), causal)
    bo, bl = M.blocked_forward(q, k, v, 1 / math.sqrt(d), causal, br, bc)
    np.testing.assert_allclose(bo, o[0, 0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(bl, lse[0, 0], rtol=0, atol=1e-13)


def test_merge_is_associative_and_commutative():
    """Four merge orders over 10 000 numbers all equal logsumexp and the weighted sum."""
    rng = np.random.default_rng(2024)
    x = rng.standard_normal(10_000) * 4 + 20
    v = rng.standard_normal((10_000, 3))
    want_lse = scipy.special.logsumexp(x)
    w = np.exp(x - want_lse)
    want_o = w @ v

    def fold(parts):
        acc = parts[0]
        for p in parts[1:]:
            acc = M.merge_mlo(acc, p)
        return acc

    def tree(parts):
        while len(parts) > 1:
            nxt = [M.merge_mlo(parts[i], parts[i + 1]) for i in range(0, len(parts) - 1, 2)]
            if len(parts) % 2:
                nxt.append(parts[-1])
            parts = nxt
        return parts[0]

    singles = [M.summary(x[i:i + 1], v[i:i + 1]) for i in range(0, 10_000, 1)]
    cuts = np.sort(rng.choice(np.arange(1, 10_000), size=6, replace=False))
    edges = [0, *cuts.tolist(), 10_000]
    blocks = [M.summary(x[a:b], v[a:b]) for a, b in zip(edges[:-1], edges[1:])]
    shuffled = [blocks[i] for i in rng.permutation(len(blocks))]
    for res in (fold(singles), fold(blocks), tree(singles), fold(shuffled)):
        m, l, o = res
        assert abs(m + math.log(l) - want_lse) <= 1e-13
        np.testing.assert_allclose(o / l, want_o, rtol=0, atol=1e-13)
    # the (m, ℓ) pair alone merges the same way
    m, l = M.summary(x[:1])
    for i in range(1, 10_000):
        m, l = M.merge_ml((m, l), M.summary(x[i:i + 1]))
    assert abs(m + math.log(l) - want_lse) <= 1e-13


def test_rescale_count_statistic():
    """Max updates over N i.i.d. values average H_N − 1 (7.895 for N = 4096)."""
    rng = np.random.default_rng(77)
    n, trials = 4096, 400
    counts = [M.count_rescales(rng.standard_normal(n)) for _ in range(trials)]
    h = sum(1.0 / i for i in range(2, n + 1))
    var = sum((1.0 / i) * (1 - 1.0 / i) for i in range(2, n + 1))
    assert abs(h - 7.895) < 1e-3
    assert abs(np.mean(counts) - h) < 5 * math.sqrt(var / trials)


# --------------------------------------------------------------------------
# decode


def test_decode_ref_is_the_last_query_row():
    rng = np.random.default_rng(21)
    q = rng.standard_normal((2, 3, 1, 16))
    k, v = rng.standard_normal((2, 3, 70, 16)), rng.standard_normal((2, 3, 70, 16))
    o, lse = decode_ref(q, k, v, 0.25)
    ao, al = attention_ref(q, k, v, 0.25, causal=False)
    np.testing.assert_allclose(o, ao[:, :, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, al[:, :, 0], rtol=0, atol=1e-14)
    # the same query placed last in a causal prefill over the same keys sees them all
    qq = np.concatenate([rng.standard_normal((2, 3, 69, 16)), q], axis=2)
    co, cl = attention_ref(qq, k, v, 0.25, causal=True, rows=np.array([69]))
    np.testing.assert_allclose(o, co[:, :, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, cl[:, :, 0], rtol=0, atol=1e-14)


def test_decode_single_key():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((1, 2, 8)), rng.standard_normal((1, 2, 1, 8)), rng.standard_normal((1, 2, 1, 8))
    o, lse = decode_ref(q, k, v, 0.5)
    np.testing.assert_array_equal(o, v[:, :, 0])
    np.testing.assert_allclose(lse, 0.5 * np.einsum("bhd,bhd->bh", q, k[:, :, 0]), rtol=0, atol=1e-15)


def test_decode_split_merge_equals_decode_ref():
    """Split the keys into segments, summarise each, ⊕-merge: the unsplit result."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal(32)
    k, v = rng.standard_normal((1000, 32)), rng.standard_normal((1000, 32))
    o, lse = decode_ref(q[None, None], k[None, None], v[None, None], 0.2)
    s = 0.2 * (k @ q)
    for nsplit in (1, 3, 64, 1000):
        edges = [(i * 1000) // nsplit for i in range(nsplit + 1)]
        parts = [M.summary(s[a:b], v[a:b]) for a, b in zip(edges[:-1], edges[1:])]
        acc = parts[0]
        for p in parts[1:]:
            acc = M.merge_mlo(acc, p)
        np.testing.assert_allclose(acc[2] / acc[1], o[0, 0], rtol=0, atol=1e-13)
        assert abs(acc[0] + math.log(acc[1]) - lse[0, 0]) < 1e-13


# --------------------------------------------------------------------------
# grouped-query decode with per-sequence key counts


def test_decode_gqa_equals_decode_on_repeated_kv_heads():
    """Query head h reads K/V head h // g: the same as plain decode on K/V whose
    heads are repeated g times in a row (and not h % Hkv, which a transposed
    grouping would give)."""
    rng = np.random.default_rng(31)
    B, Hkv, g, L, d = 2, 3, 4, 50, 16
    q = rng.standard_normal((B, Hkv * g, 1, d))
    k, v = rng.standard_normal((B, Hkv, L, d)), rng.standard_normal((B, Hkv, L, d))
    o, lse = decode_gqa_ref(q, k, v, 0.3)
    ro, rl = decode_ref(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.3)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, rl, rtol=0, atol=1e-14)
    wrong = decode_ref(q, np.tile(k, (1, g, 1, 1)), np.tile(v, (1, g, 1, 1)), 0.3)[0]
    assert np.abs(o - wrong).max() > 1e-3


def test_decode_gqa_seqlens_truncate_the_cache():
    rng = np.random.default_rng(32)
    B, Hkv, g, L, d = 3, 2, 2, 40, 8
    q = rng.standard_normal((B, Hkv * g, d))
    k, v = rng.standard_normal((B, Hkv, L, d)), rng.standard_normal((B, Hkv, L, d))
    lens = np.array([1, 17, 40])
    o, lse = decode_gqa_ref(q, k, v, 0.5, seqlens=lens)
    for b, n in enumerate(lens):
        ro, rl = decode_ref(q[b:b + 1], np.repeat(k[b:b + 1, :, :n], g, axis=1),
                            np.repeat(v[b:b + 1, :, :n], g, axis=1), 0.5)
        np.testing.assert_allclose(o[b], ro[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], rl[0], rtol=0, atol=1e-14)
    # one key: the weight is exactly 1 on it
    np.testing.assert_array_equal(o[0], np.repeat(v[0, :, 0], g, axis=0))


def test_decode_gqa_zero_query_is_the_mean_of_the_visible_values():
    """q = 0: every logit is 0, so O is the plain mean of the first len_b value rows
    and LSE = ln len_b (closed form)."""
    rng = np.random.default_rng(33)
    B, Hkv, g, L, d = 2, 2, 3, 30, 4
    v = rng.standard_normal((B, Hkv, L, d))
    lens = np.array([7, 30])
    o, lse = decode_gqa_ref(np.zeros((B, Hkv * g, d)), rng.standard_normal((B, Hkv, L, d)), v, 1.0, seqlens=lens)
    for b, n in enumerate(lens):
        for h in range(Hkv * g):
            np.testing.assert_allclose(o[b, h], v[b, h // g, :n].mean(axis=0), rtol=0, atol=1e-14)
            assert abs(lse[b, h] - math.log(n)) < 1e-14


def test_decode_gqa_matches_decimal_bruteforce():
    rng = np.random.default_rng(34)
    B, Hkv, g, L, d = 1, 2, 2, 6, 5
    q = rng.standard_normal((B, Hkv * g, d))
    k, v = rng.standard_normal((B, Hkv, L, d)), rng.standard_normal((B, Hkv, L, d))
    lens = np.array([4])
    o, lse = decode_gqa_ref(q, k, v, 0.4, seqlens=lens)
    for h in range(Hkv * g):
        wo, wl = _decimal_attention(q[0, h][None], k[0, h // g, :4], v[0, h // g, :4], 0.4, False)
        np.testing.assert_allclose(o[0, h], wo[0], rtol=0, atol=1e-13)
        assert abs(lse[0, h] - wl[0]) < 1e-13


# --------------------------------------------------------------------------
# backward


def _loss(q, k, v, do, scale, causal):
    return float((attention_ref(q, k, v, scale, causal)[0] * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_central_differences(causal):
    """dQ, dK, dV are the gradients of Σ dO ∘ O: central differences of the
    forward definition (step 1e-5, fp64) agree to 1e-8 on a small problem."""
    rng = np.random.default_rng(41 + causal)
    B, H, N, d = 1, 2, 5, 3
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    scale = 0.7
    dq, dk, dv, _ = attention_bwd_ref(q, k, v, do, scale, causal)
    eps = 1e-5
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = _loss(q, k, v, do, scale, causal)
            x[idx] = keep - eps
            down = _loss(q, k, v, do, scale, causal)
            x[idx] = keep
            num[idx] = (up - down) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-8)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_d_identity_and_shift_invariance(causal):
    """D_i = Σ_j P_ij dP_ij equals dO_i · O_i ([15-779 L5] §7.3); every row of dS
    sums to zero (softmax ignores a shift of its row), so Σ_j dK_j = 0."""
    rng = np.random.default_rng(43 + causal)
    q, k, v, do = (rng.standard_normal((2, 2, 37, 8)) for _ in range(4))
    dq, dk, dv, dd = attention_bwd_ref(q, k, v, do, 0.35, causal)
    o, _ = attention_ref(q, k, v, 0.35, causal)
    np.testing.assert_allclose(dd, (do * o).sum(-1), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_with_stored_output(causal):
    """With the exact O passed in, D from dO · O gives the same gradients; an O
    whose row i is off so that dO_i · O_i moves by c_i shifts dS_ij by −P_ij c_i,
    hence dQ_i by −scale c_i (P K)_i and dK_j by −scale Σ_i c_i P_ij Q_i, and
    leaves dV alone."""
    rng = np.random.default_rng(47 + causal)
    q, k, v, do = (rng.standard_normal((1, 2, 29, 8)) for _ in range(4))
    scale = 0.4
    o, _ = attention_ref(q, k, v, scale, causal)
    base = attention_bwd_ref(q, k, v, do, scale, causal)
    same = attention_bwd_ref(q, k, v, do, scale, causal, o=o)
    for a, b in zip(base, same):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
    c = rng.standard_normal((1, 2, 29))
    o_off = o + c[..., None] * do / (do * do).sum(-1, keepdims=True)
    dq, dk, dv, dd = attention_bwd_ref(q, k, v, do, scale, causal, o=o_off)
    np.testing.assert_allclose(dd, base[3] + c, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, base[2], rtol=0, atol=1e-13)
    for h in range(2):
        p, _, _ = safe_softmax(scores(q[0, h], k[0, h], scale, causal))
        np.testing.assert_allclose(dq[0, h] - base[0][0, h], -scale * c[0, h][:, None] * (p @ k[0, h]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk[0, h] - base[1][0, h], -scale * (p * c[0, h][:, None]).T @ q[0, h], rtol=0, atol=1e-12)


def test_backward_dv_with_constant_do_is_column_sums():
    """dO = 1: dV_j = Σ_i P_ij (the column sums of P) in every column."""
    rng = np.random.default_rng(45)
    q, k, v = (rng.standard_normal((1, 1, 20, 4)) for _ in range(3))
    _, _, dv, _ = attention_bwd_ref(q, k, v, np.ones((1, 1, 20, 4)), 0.5, True)
    p, _, _ = safe_softmax(scores(q[0, 0], k[0, 0], 0.5, True))
    np.testing.assert_allclose(dv[0, 0], np.repeat(p.sum(axis=0)[:, None], 4, axis=1), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# backward of block-sparse attention


def _sparse_loss(q, k, v, do, scale, causal, mask, block):
    return float((attention_block_sparse_ref(q, k, v, scale, causal, mask, block)[0] * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_backward_matches_central_differences(causal):
    """With a block mask (blocks of 2 over N = 7: a partial last block, a row
    block that keeps nothing, kept and dropped blocks mixed), dQ, dK, dV are
    the gradients of Σ dO ∘ O through the block-sparse forward definition:
    central differences (step 1e-5, fp64) agree to 1e-8, and the rows with no
    key get exactly zero dQ."""
    rng = np.random.default_rng(61 + causal)
    B, H, N, d, blk = 1, 2, 7, 3, 2
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    mask = np.array([[1, 0, 1, 0], [0, 0, 0, 0], [1, 1, 0, 1], [0, 1, 1, 1]])
    scale = 0.6
    dq, dk, dv, _ = attention_bwd_ref(q, k, v, do, scale, causal, block_mask=mask, block=blk)
    assert np.all(dq[:, :, 2:4] == 0)
    eps = 1e-5
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = _sparse_loss(q, k, v, do, scale, causal, mask, blk)
            x[idx] = keep - eps
            down = _sparse_loss(q, k, v, do, scale, causal, mask, blk)
            x[idx] = keep
            num[idx] = (up - down) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=1e-8)


def test_block_sparse_backward_special_cases():
    """An all-ones mask is the dense backward; a block-diagonal mask splits the
    problem into independent attentions over the two halves."""
    rng = np.random.default_rng(67)
    q, k, v, do = (rng.standard_normal((1, 2, 16, 4)) for _ in range(4))
    dense = attention_bwd_ref(q, k, v, do, 0.5, True)
    ones = attention_bwd_ref(q, k, v, do, 0.5, True, block_mask=np.ones((2, 2)), block=8)
    for a, b in zip(dense, ones):
        np.testing.assert_allclose(b, a, rtol=0, atol=1e-14)
    diag = attention_bwd_ref(q, k, v, do, 0.5, False, block_mask=np.eye(2), block=8)
    for half in (slice(0, 8), slice(8, 16)):
        part = attention_bwd_ref(q[:, :, half], k[:, :, half], v[:, :, half], do[:, :, half], 0.5, False)
        for a, b in zip(part[:3], diag[:3]):
            np.testing.assert_allclose(b[:, :, half], a, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# the tolerance rule


def test_bf16_rounding_helpers():
    assert bf16_half_ulp(4.5) == 2.0 ** -6          # [4, 8): ulp 2^-5
    assert bf16_half_ulp(3.0) == 2.0 ** -7
    assert bf16_half_ulp(1.0) == 2.0 ** -8
    assert bf16_rne(1.0 + 2.0 ** -8) == 1.0          # tie -> even
    assert bf16_rne(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    x = np.array([0.1, -2.7, 5.3, 100.0])
    assert np.all(np.abs(bf16_rne(x) - x) <= bf16_half_ulp(x))
    r = check_prefill(bf16_rne(x), [0.0], x, [0.0005])
    assert r["pass"] and r["floor"] > 0
    r = check_prefill(x + 0.02, [0.0], x, [0.0])
    assert not r["ok"]


# --------------------------------------------------------------------------
# paged K/V decode


def test_decode_paged_is_the_contiguous_cache_scattered_into_pages():
    """Scatter a contiguous cache into pages under a random page permutation: the
    paged decode must see the same keys in the same order (checked against
    decode_ref head by head, which the gather does not use)."""
    rng = np.random.default_rng(81)
    B, Hq, Hkv, P, d, max_pages = 3, 4, 2, 8, 16, 5
    Lmax = P * max_pages
    k = rng.standard_normal((B, Hkv, Lmax, d))
    v = rng.standard_normal((B, Hkv, Lmax, d))
    q = rng.standard_normal((B, Hq, d))
    n_pages = B * max_pages + 3
    perm = rng.permutation(n_pages)[: B * max_pages].reshape(B, max_pages)
    kp = rng.standard_normal((n_pages, Hkv, P, d))   # pages nobody maps hold noise
    vp = rng.standard_normal((n_pages, Hkv, P, d))
    for b in range(B):
        for i in range(max_pages):
            kp[perm[b, i]] = k[b, :, i * P:(i + 1) * P]
            vp[perm[b, i]] = v[b, :, i * P:(i + 1) * P]
    lens = np.array([Lmax, 1, 29])
    o, l = decode_paged_ref(q, kp, vp, perm, lens, 0.3)
    for b in range(B):
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            ro, rl = decode_ref(q[b:b + 1, h:h + 1], k[b:b + 1, kh:kh + 1, :lens[b]], v[b:b + 1, kh:kh + 1, :lens[b]], 0.3)
            np.testing.assert_allclose(o[b, h], ro[0, 0], rtol=0, atol=1e-13)
            np.testing.assert_allclose(l[b, h], rl[0, 0], rtol=0, atol=1e-13)
    # a page past a sequence's length is never read: poisoning it changes nothing
    kp2 = kp.copy()
    kp2[perm[1, 1]] = np.nan
    o2, _ = decode_paged_ref(q, kp2, vp, perm, lens, 0.3)
    np.testing.assert_array_equal(o2[1], o[1])


# --------------------------------------------------------------------------
# block-sparse attention ([FA-1拆解] "块稀疏扩展")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_all_ones_is_dense(causal):
    q, k, v = (_rand((1, 2, 70, 8), 61 + i) for i in range(3))
    o, l = attention_block_sparse_ref(q, k, v, 0.3, causal, np.ones((3, 3)), block=32)
    ro, rl = attention_ref(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-13)


def test_block_sparse_lower_triangle_with_causal_is_causal():
    """Blocks wholly above the diagonal hold only keys after every query of the
    block, so switching them off changes nothing under the causal mask."""
    q, k, v = (_rand((1, 1, 100, 8), 64 + i) for i in range(3))
    o, l = attention_block_sparse_ref(q, k, v, 0.3, True, np.tril(np.ones((4, 4))), block=32)
    ro, rl = attention_ref(q, k, v, 0.3, True)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-13)


def test_block_sparse_block_diagonal_is_independent_blocks():
    q, k, v = (_rand((2, 1, 90, 8), 67 + i) for i in range(3))
    o, l = attention_block_sparse_ref(q, k, v, 0.3, False, np.eye(3), block=32)
    for lo, hi in ((0, 32), (32, 64), (64, 90)):
        ro, rl = attention_ref(q[:, :, lo:hi], k[:, :, lo:hi], v[:, :, lo:hi], 0.3, False)
        np.testing.assert_allclose(o[:, :, lo:hi], ro, rtol=0, atol=1e-14)
        np.testing.assert_allclose(l[:, :, lo:hi], rl, rtol=0, atol=1e-13)


def test_block_sparse_dropped_key_blocks_are_gone():
    """Switching key block j off for every query block equals attention over the
    remaining keys; with causal, query rows keep their own positions."""
    q, k, v = (_rand((1, 1, 96, 8), 70 + i) for i in range(3))
    mask = np.ones((3, 3))
    mask[:, 1] = 0
    keep = np.r_[0:32, 64:96]
    o, l = attention_block_sparse_ref(q, k, v, 0.3, False, mask, block=32)
    ro, rl = attention_ref(q, k[:, :, keep], v[:, :, keep], 0.3, False)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l, rl, rtol=0, atol=1e-13)


def test_block_sparse_empty_rows_and_per_head_masks():
    q, k, v = (_rand((1, 2, 64, 8), 73 + i) for i in range(3))
    m0 = np.array([[1, 0], [0, 0]])   # head 0: the second query block sees nothing
    m1 = np.array([[0, 1], [1, 1]])   # head 1: the first query block sees only key block 1
    o, l = attention_block_sparse_ref(q, k, v, 0.3, False, np.stack([m0, m1]), block=32)
    assert np.all(o[0, 0, 32:] == 0) and np.all(np.isneginf(l[0, 0, 32:]))
    o0, l0 = attention_block_sparse_ref(q[:, :1], k[:, :1], v[:, :1], 0.3, False, m0, block=32)
    np.testing.assert_array_equal(o[:, :1], o0)
    ro, rl = attention_ref(q[:, 1:, :32], k[:, 1:, 32:], v[:, 1:, 32:], 0.3, False)
    np.testing.assert_allclose(o[:, 1:, :32], ro, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l[:, 1:, :32], rl, rtol=0, atol=1e-13)
    # causal + a mask that leaves the first rows of a block without keys
    o, l = attention_block_sparse_ref(q, k, v, 0.3, True, np.array([[0, 0], [1, 1]]), block=32)
    assert np.all(o[0, :, :32] == 0) and np.all(np.isneginf(l[0, :, :32]))
    ro, rl = attention_ref(q, k, v, 0.3, True, rows=np.arange(32, 64))
    np.testing.assert_allclose(o[:, :, 32:], ro, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# the backward allowance: wide enough for a faithful bf16-operand backward,
# narrow enough to fail plausible slips


def _sim_bwd(q, k, v, do, o, lse, scale, causal, slip=None, mask=None, block=128):
    """A bf16-operand, fp32-accumulating backward in numpy float32 (the arithmetic
    bwd_allowance describes), with an optional planted slip and block mask."""
    f = np.float32
    c = f(scale * math.log2(math.e))
    out = [np.empty(q.shape, np.float64) for _ in range(3)]
    N = q.shape[2]
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            qq, kk, vv, dd_o, oo = (np.asarray(x[b, h], dtype=f) for x in (q, k, v, do, o))
            l2 = np.asarray(lse[b, h], dtype=f) * f(math.log2(math.e))
            s = qq @ kk.T
            p = np.exp2(s * c - (l2[:, None] if slip != "no_lse" else f(0)))
            if causal and slip != "no_mask":
                p[np.triu_indices(N, 1)] = 0
            if mask is not None and slip != "no_block_mask":
                idx = np.arange(N) // block
                p = np.where(np.asarray(mask)[idx[:, None], idx[None, :]] != 0, p, f(0))
            dp = dd_o @ vv.T
            dvec = (dd_o * oo).sum(axis=1)
            ds = p * (dp - (dvec[:, None] if slip != "no_d" else f(0)))
            pb = bf16_rne(p).astype(f)
            sb = bf16_rne(ds).astype(f)
            sc = f(1.0) if slip == "no_scale" else f(scale)
            out[2][b, h] = bf16_rne((pb if slip == "dv_untransposed" else pb.T) @ dd_o)
            out[1][b, h] = bf16_rne(sc * (sb.T @ qq))
            out[0][b, h] = bf16_rne(sc * (sb @ kk))
    return out


def _bwd_case(causal, seed, N=48, d=16):
    rng = np.random.default_rng(seed)
    q, k, v, do = (bf16_rne(rng.standard_normal((1, 2, N, d))) for _ in range(4))
    scale = float(np.float32(1 / math.sqrt(d)))
    o, lse = attention_ref(q, k, v, scale, causal)
    return q, k, v, do, bf16_rne(o), np.asarray(lse, dtype=np.float32), scale


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_allowance_admits_a_faithful_bf16_backward(causal):
    q, k, v, do, o, lse, scale = _bwd_case(causal, 51 + causal)
    ref, allow = bwd_allowance(q, k, v, do, scale, causal, o=o)
    rep = check_bwd(_sim_bwd(q, k, v, do, o, lse, scale, causal), ref, allow)
    assert rep["pass"], rep
    # and it is not vacuous: the limits are a small fraction of the gradients' size
    for r, a in zip(ref, allow):
        assert np.median(a) < 0.05 * np.median(np.abs(r))


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_allowance_covers_forward_then_backward(causal):
    """O and L from a float32 forward that rounds its weights to bf16, fed to the
    simulated backward, against the exact reference: within the o_from_fwd limits."""
    q, k, v, do, _, _, scale = _bwd_case(causal, 55 + causal, N=64, d=32)
    f = np.float32
    o = np.empty(q.shape)
    lse = np.empty(q.shape[:3], dtype=f)
    for h in range(q.shape[1]):
        s = np.asarray(q[0, h], dtype=f) @ np.asarray(k[0, h], dtype=f).T * f(scale)
        if causal:
            s[np.triu_indices(q.shape[2], 1)] = -np.inf
        m = s.max(axis=1, keepdims=True)
        pt = np.exp(s - m)
        pb = bf16_rne(pt).astype(f)
        o[0, h] = bf16_rne((pb @ np.asarray(v[0, h], dtype=f)) / pb.sum(axis=1, keepdims=True))
        lse[0, h] = m[:, 0] + np.log(pt.sum(axis=1))
    ref, allow = bwd_allowance(q, k, v, do, scale, causal, o_from_fwd=True)
    rep = check_bwd(_sim_bwd(q, k, v, do, o, lse, scale, causal), ref, allow)
    assert rep["pass"], rep


@pytest.mark.parametrize("slip", [None, "no_block_mask"])
def test_bwd_allowance_block_sparse(slip):
    """The rule with a block mask (blocks of 16 over N = 48, one row block that
    keeps only a far key block): the float32 simulation passes, and one that
    forgets the block mask fails."""
    causal = True
    rng = np.random.default_rng(71)
    q, k, v, do = (bf16_rne(rng.standard_normal((1, 2, 48, 16))) for _ in range(4))
    scale = float(np.float32(0.25))
    mask = np.array([[1, 0, 0], [0, 1, 0], [1, 0, 1]])
    o, lse = attention_block_sparse_ref(q, k, v, scale, causal, mask, 16)
    o, lse = bf16_rne(o), np.asarray(lse, dtype=np.float32)
    ref, allow = bwd_allowance(q, k, v, do, scale, causal, o=o, block_mask=mask, block=16)
    rep = check_bwd(_sim_bwd(q, k, v, do, o, lse, scale, causal, slip=slip, mask=mask, block=16), ref, allow)
    assert rep["pass"] == (slip is None), rep


@pytest.mark.parametrize("slip", ["no_d", "no_mask", "no_scale", "no_lse", "dv_untransposed"])
def test_bwd_allowance_rejects_slips(slip):
    causal = True
    q, k, v, do, o, lse, scale = _bwd_case(causal, 53)
    ref, allow = bwd_allowance(q, k, v, do, scale, causal, o=o)
    rep = check_bwd(_sim_bwd(q, k, v, do, o, lse, scale, causal, slip=slip), ref, allow)
    assert not rep["pass"], (slip, rep)


# --------------------------------------------------------------------------
# the pins are sensitive: plausible slips planted in copies of the oracle fail them


def _mutant(kind):
    def run(q, k, v, scale, causal):
        q, k, v = q[0, 0], k[0, 0], v[0, 0]
        if kind == "no_scale":
            s = q @ k.T
        elif kind == "transposed":
            s = scale * (k @ q.T)
        else:
            s = scale * (q @ k.T)
        if causal:
            n = s.shape[0]
            mask = np.tril(np.ones((n, n), bool), -1) if kind == "mask_flipped" else np.triu(np.ones((n, n), bool), 1)
            s = np.where(mask, -np.inf, s)
        m = s.max(1)
        e = np.exp(s - m[:, None])
        l = e.sum(1)
        o = (e / l[:, None]) @ v
        lse = np.log(l) if kind == "lse_no_max" else m + np.log(l)
        return o[None, None], lse[None, None]
    return run


@pytest.mark.parametrize("kind", ["no_scale", "transposed", "mask_flipped", "lse_no_max"])
def test_pins_catch_mistakes(kind):
    fx = _fx()
    q, k, v, scale = _fixture_inputs(fx)
    failed = False
    for mode in ("causal", "noncausal"):
        o, lse = _mutant(kind)(q, k, v, scale, mode == "causal")
        want_o = np.array([[float(x) for x in r] for r in _frac_mat(fx[mode]["o"])])
        want_l = np.array([math.log(int(x)) for x in fx[mode]["lse_ln_of"]])
        if not (np.allclose(o[0, 0], want_o, atol=1e-9) and np.allclose(lse[0, 0], want_l, atol=1e-9)):
            failed = True
    if kind == "lse_no_max":
        # S = ln w here, so max-free LSE only shows with shifted logits: use the huge-logit case
        q2 = np.array([[[[1000.0, 1000.0 + math.log(3.0)]]]])
        k2 = np.eye(2)[None, None]
        _, l2 = _mutant(kind)(q2, k2, np.ones((1, 1, 2, 1)), 1.0, False)
        failed = failed or abs(l2[0, 0, 0] - (1000.0 + math.log(4.0))) > 1e-9
    assert failed
