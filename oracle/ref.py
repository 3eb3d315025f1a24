"""The oracle: standard attention, computed in fp64 on the CPU, one (b, h) at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Nothing here is fused,
tiled or reordered: the three steps are those of standard attention, and the
method the GPU library implements reaches the same result up to rounding
order ([FA-1拆解] "核心思想：IO 感知" — exact, not an approximation;
[15-779 L5] §5.1 "为什么是精确的").

Steps, as the pages give them:

1. S = scale · Q Kᵀ   ([cicada] §1.2 formula and §1.3 steps one and two;
   [15-779 L5] §2.3).  The scale multiplies S before the max and the exp
   ([15-779 L5] §5.1 pseudo-code writes S_ij = Q_i K_jᵀ / √d).
2. Causal mask: S_ij = −∞ where key j lies after query i ([cicada] §1.3 step
   two; [15-779 L5] §2.3).  Square and top-left aligned: query i sees keys
   0..i.
3. Safe softmax per row: m = max_j S_ij, E = exp(S − m), ℓ = Σ_j E,
   P = E / ℓ ([cicada] §1.3 step three; [15-779 L5] §4.2).
4. O = P V ([cicada] §1.3 step four) and the per-row log-sum-exp
   L = m + ln ℓ ([cicada] §3.2.3 "核心计算 2"; [15-779 L5] §5.1 last line).

Decode is the same definition with a single query row that sees every cached
key ([15-779 L5] §8.1–8.2): no mask and no split — splitting the keys is the
method's speed device ([15-779 L5] §8.4), not part of the result.

Inputs are whatever the caller hands in (numpy arrays, or torch tensors of any
dtype, including bfloat16); they are widened to float64 exactly.  ``scale`` is
used as given (the GPU library receives the same value as an fp32 number,
which a Python float represents exactly).
"""

import numpy as np


def as_f64(x):
    """Widen an array-like (numpy array or torch tensor) to a float64 ndarray."""
    if hasattr(x, "detach"):  # torch tensor: plain CPU conversion, exact for bf16/fp32
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def scores(q, k, scale, causal, rows=None):
    """Steps 1–2 for one (b, h): S = scale · q kᵀ, then the causal mask.

    q: [R, d] float64 query rows; k: [Nk, d] float64 keys.
    rows: the query index of each row of ``q`` (defaults to 0..R-1); it places
    the causal mask, which removes key j from query i when j > i
    ([cicada] §1.3 step two; [15-779 L5] §2.3).
    Returns S as a [R, Nk] float64 array with −∞ in masked slots.
    """
    s = scale * (q @ k.T)
    if causal:
        if rows is None:
            rows = np.arange(q.shape[0])
        rows = np.asarray(rows)
        keys = np.arange(k.shape[0])
        s = np.where(keys[None, :] > rows[:, None], -np.inf, s)
    return s


def safe_softmax(s):
    """Step 3: row-wise safe softmax ([15-779 L5] §4.2; [cicada] §1.3 step three).

    Returns (P, m, ℓ): the probabilities, the row maxima and the row sums of
    exp(S − m).  Masked entries (−∞) get exactly zero weight.
    """
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    p = e / l[:, None]
    return p, m, l


def attention_ref(q, k, v, scale, causal, rows=None):
    """Exact attention forward: O = softmax(scale·QKᵀ [+ causal mask]) V and LSE.

    q, k, v: [B, H, N, d] (v may have its own last dimension d_v).
    rows: optional 1-D array of query indices; only those rows are computed
    (each output row depends on its own query row only, so a subset is the
    same definition evaluated at fewer points).
    Returns (O [B, H, R, d_v], LSE [B, H, R]) as float64 arrays; LSE is the
    natural-log log-sum-exp of the scaled, masked logits of each row.
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    B, H, N, _ = q.shape
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    o = np.empty((B, H, rows.size, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, rows.size), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scores(q[b, h][rows], k[b, h], scale, causal, rows)
            p, m, l = safe_softmax(s)
            o[b, h] = p @ v[b, h]
            lse[b, h] = m + np.log(l)
    return o, lse


def decode_ref(q, k, v, scale):
    """Decode: one new query per sequence attends to all Lkv cached keys.

    q: [B, H, d] or [B, H, 1, d]; k, v: [B, H, Lkv, d].  No mask: the new
    token sees every earlier token ([15-779 L5] §8.1–8.2).  No split.
    Returns (O [B, H, d], LSE [B, H]) in float64.
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, H, _ = q.shape
    o = np.empty((B, H, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            s = scale * (k[b, h] @ q[b, h])          # [Lkv] logits
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            o[b, h] = (e / l) @ v[b, h]
            lse[b, h] = m + np.log(l)
    return o, lse


def decode_gqa_ref(q, k, v, scale, seqlens=None):
    """Grouped-query decode with per-sequence key counts.

    q: [B, Hq, d] or [B, Hq, 1, d]; k, v: [B, Hkv, Lmax, d] with Hq = g·Hkv.
    Query head h attends with K/V head h // g — g query heads share one cached
    head ([15-779 L5] §12, exercise 7) — to keys 0 .. seqlens[b]-1 of
    sequence b (all Lmax when seqlens is None).  The same definition as
    decode_ref, on the selected keys.  Returns (O [B, Hq, d], LSE [B, Hq]).
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    if q.ndim == 4:
        q = q[:, :, 0, :]
    B, Hq, _ = q.shape
    Hkv, Lmax = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0, "query heads must be a multiple of K/V heads"
    g = Hq // Hkv
    lens = [Lmax] * B if seqlens is None else [int(x) for x in np.asarray(seqlens)]
    o = np.empty((B, Hq, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    for b in range(B):
        n = lens[b]
        assert 1 <= n <= Lmax, "each sequence holds between 1 and Lmax keys"
        for h in range(Hq):
            kh = h // g
            s = scale * (k[b, kh, :n] @ q[b, h])     # [n] logits
            m = s.max()
            e = np.exp(s - m)
            l = e.sum()
            o[b, h] = (e / l) @ v[b, kh, :n]
            lse[b, h] = m + np.log(l)
    return o, lse


def decode_paged_ref(q, k_pages, v_pages, block_table, seqlens, scale):
    """Grouped-query decode over a paged K/V cache.

    k_pages, v_pages: [num_pages, Hkv, P, d] — page p of K/V head h holds P
    consecutive keys; block_table: [B, max_pages] page numbers; key t of
    sequence b sits at row t mod P of page block_table[b, ⌊t/P⌋].  Paging is a
    storage layout of the cache (the pages set it beside tiled computation:
    [FA-1拆解], closing section, on paged K/V caches), so the result is that
    of ``decode_gqa_ref`` on the keys gathered in order: the gather is written
    out here and the definition reused.  Returns (O [B, Hq, d], LSE [B, Hq]).
    """
    k_pages = as_f64(k_pages)
    v_pages = as_f64(v_pages)
    table = np.asarray(block_table)
    lens = [int(x) for x in np.asarray(seqlens)]
    B = table.shape[0]
    _, Hkv, P, d = k_pages.shape
    Lmax = table.shape[1] * P
    k = np.zeros((B, Hkv, Lmax, d))
    v = np.zeros((B, Hkv, Lmax, d))
    for b in range(B):
        for t in range(lens[b]):
            page = int(table[b, t // P])
            k[b, :, t] = k_pages[page, :, t % P]
            v[b, :, t] = v_pages[page, :, t % P]
    return decode_gqa_ref(q, k, v, scale, seqlens=lens)


def attention_block_sparse_ref(q, k, v, scale, causal, block_mask, block=128, rows=None):
    """Block-sparse attention ([FA-1拆解] "块稀疏扩展"): standard attention in which
    every score whose (query block, key block) is switched off in the block
    mask is masked like a causal one, i.e. set to −∞ before the softmax.

    block_mask: [T_q, T_k] or [B·H, T_q, T_k] array of 0/1 over blocks of
    ``block`` query rows × ``block`` keys (T_q = T_k = ⌈N/block⌉), one mask for
    all heads or one per (b, h) in b-major order.  Combined with the causal
    mask when ``causal``.  A row left with no key at all has no softmax; its
    output is taken as O = 0 and L = −∞ (the empty sum: ℓ = 0, ln ℓ = −∞).
    Returns (O, LSE) as ``attention_ref`` does.
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    B, H, N, _ = q.shape
    mask = np.asarray(block_mask)
    if rows is None:
        rows = np.arange(N)
    rows = np.asarray(rows)
    keys = np.arange(N)
    o = np.empty((B, H, rows.size, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, rows.size), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            mk = mask if mask.ndim == 2 else mask[b * H + h]
            s = scores(q[b, h][rows], k[b, h], scale, causal, rows)
            on = mk[rows[:, None] // block, keys[None, :] // block] != 0
            s = np.where(on, s, -np.inf)
            empty = np.all(np.isneginf(s), axis=1)
            s_safe = np.where(empty[:, None], 0.0, s)  # any finite row: its result is discarded below
            p, m, l = safe_softmax(s_safe)
            o[b, h] = np.where(empty[:, None], 0.0, p @ v[b, h])
            lse[b, h] = np.where(empty, -np.inf, m + np.log(l))
    return o, lse


def masked_probs(q_bh, k_bh, scale, causal, block_mask_bh=None, block=128):
    """The softmax weights P of one (b, h): P = softmax(S) row by row, S the
    scaled scores with the causal mask and, when ``block_mask_bh`` ([T_q, T_k]
    of 0/1) is given, the switched-off blocks at −∞ ([FA-1拆解] "块稀疏扩展").
    A row with no key left has no softmax; its weights are taken as all zero,
    matching O = 0 for that row."""
    s = scores(q_bh, k_bh, scale, causal)
    if block_mask_bh is None:
        p, _, _ = safe_softmax(s)
        return p
    n = s.shape[0]
    idx = np.arange(n) // block
    s = np.where(np.asarray(block_mask_bh)[idx[:, None], idx[None, :]] != 0, s, -np.inf)
    empty = np.all(np.isneginf(s), axis=1)
    p, _, _ = safe_softmax(np.where(empty[:, None], 0.0, s))
    return np.where(empty[:, None], 0.0, p)


def attention_bwd_ref(q, k, v, do, scale, causal, o=None, block_mask=None, block=128):
    """Exact attention backward: the gradients of Σ dO ∘ O with respect to Q, K, V.

    The chain rule through O = P V and the row softmax P = softmax(S),
    S = scale · Q Kᵀ [+ causal mask] ([15-779 L5] §7.1):
        dV = Pᵀ dO,   dP = dO Vᵀ,   dS = P ∘ (dP − D),   D_i = Σ_j P_ij dP_ij,
        dQ = scale · dS K,   dK = scale · dSᵀ Q.
    (The diag(p) − p pᵀ Jacobian of each softmax row gives dS.)  P is formed
    with steps 1–3 of the standard algorithm, one (b, h) at a time.
    With ``o`` given (a stored forward output [B, H, N, d]), D is taken as
    D_i = Σ_c dO_ic O_ic, the identity of [15-779 L5] §7.3 that lets a
    blockwise backward form D before its loops; it equals Σ_j P_ij dP_ij when
    o is the exact O.
    ``block_mask`` ([T_q, T_k] or [B·H, T_q, T_k], as for
    ``attention_block_sparse_ref``): the backward of block-sparse attention;
    switched-off blocks have P = 0 and so dS = 0, and a row with no key has
    P = 0, O = 0 and zero gradient.
    q, k, v, do: [B, H, N, d].  Returns (dQ, dK, dV, D) as float64 arrays,
    D of shape [B, H, N].
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    do = as_f64(do)
    o = None if o is None else as_f64(o)
    mask = None if block_mask is None else np.asarray(block_mask)
    B, H, N, _ = q.shape
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dd = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            mk = None if mask is None else (mask if mask.ndim == 2 else mask[b * H + h])
            p = masked_probs(q[b, h], k[b, h], scale, causal, mk, block)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            dd[b, h] = (p * dp).sum(axis=1) if o is None else (do[b, h] * o[b, h]).sum(axis=1)
            ds = p * (dp - dd[b, h][:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv, dd
