"""GPU parity: the HIP library, called through the C ABI, against the fp64 oracle
on the same seeded inputs.

Rule (oracle/compare.py): |O − O_ref| ≤ 1e-2 + ½·ulp_bf16(O_ref) per element
and |LSE − LSE_ref| ≤ 1e-3, with the literal max-abs error reported beside.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import exact_attention_31_amd as fa
import synth
from oracle import attention_ref, decode_gqa_ref, decode_ref, check_prefill

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    fa.load_library()  # raise loudly if the HIP library is missing
    yield


def _run_fwd(q, k, v, scale, causal):
    o, lse = fa.fa_fwd(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def _check(name, o, lse, ro, rl):
    rep = check_prefill(o, lse, ro, rl)
    _say(f"[parity] {name}: O max_abs={rep['max_abs']:.3g} floor={rep['floor']:.3g} "
         f"excess={rep['excess']:.3g} LSE max_abs={rep['lse_max_abs']:.3g} pass={rep['pass']}")
    assert rep["pass"], rep
    return rep


# ----------------------------------------------------------------------------
# the five workloads


def test_single_head_n256_d64():
    w = W[0]
    _say("[case] workload", w.name)
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, w.causal)
    ro, rl = attention_ref(q, k, v, w.scale, w.causal)
    _check(w.name, o, lse, ro, rl)


def test_gpt2_small_causal():
    w = W[1]
    _say("[case] workload", w.name)
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, w.causal)
    ro, rl = attention_ref(q, k, v, w.scale, w.causal)
    _check(w.name, o, lse, ro, rl)


def test_llama3_causal_kboost():
    """All 32 heads, every row (the large-logit rows force running-max rescales)."""
    w = W[2]
    _say("[case] workload", w.name)
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, w.causal)
    ro, rl = attention_ref(q, k, v, w.scale, w.causal)
    _check(w.name, o, lse, ro, rl)


def test_long_noncausal_sampled_rows():
    """N = 16384: the oracle evaluates sampled query rows (first, last, random) of 4 heads."""
    w = W[3]
    _say("[case] workload", w.name)
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, w.causal)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, w.N - 1], rng.choice(w.N, 250, replace=False)]))
    heads = [0, 5, 10, 15]
    ro, rl = attention_ref(q[:, heads], k[:, heads], v[:, heads], w.scale, False, rows=rows)
    _check(w.name + " (sampled)", o[:, heads][:, :, rows], lse[:, heads][:, :, rows], ro, rl)


def test_long_noncausal_full():
    """N = 16384, all 16 heads, every row compared with the oracle (one head, 4096
    rows at a time, on the host)."""
    w = W[3]
    _say("[case] workload", w.name, "(every row of every head)")
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, w.causal)
    worst = None
    for h in range(w.H):
        for r0 in range(0, w.N, 4096):
            rows = np.arange(r0, min(w.N, r0 + 4096))
            ro, rl = attention_ref(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], w.scale, False, rows=rows)
            rep = check_prefill(o[:, h:h + 1, rows], lse[:, h:h + 1, rows], ro, rl)
            assert rep["pass"], (h, r0, rep)
            if worst is None or rep["excess"] > worst["excess"]:
                worst = dict(rep, head=h)
        _say(f"  head {h}: ok")
    _say(f"[parity] {w.name} (all 16 x 16384 rows): worst head {worst['head']}: O max_abs={worst['max_abs']:.3g} "
         f"floor={worst['floor']:.3g} excess={worst['excess']:.3g} LSE max_abs={worst['lse_max_abs']:.3g}")


def test_million_keys_causal_sampled_rows():
    """One head of 2^20 + 77 keys, causal, d = 128: the last workgroup streams
    16 385 key tiles, and ℓ, ℓ_b and the accumulator sum over a million keys in
    fp32.  The oracle evaluates sampled rows (the first, the ragged tail, block
    edges, random ones)."""
    n = (1 << 20) + 77
    w = W[2].with_(B=1, H=1, N=n, d=128, causal=True, boost_frac=0.0, wid=200)
    _say("[case] million keys", n)
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, True)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, n - 78, n - 77, n - 2, n - 1], rng.choice(n, 40, replace=False)]))
    ro, rl = attention_ref(q, k, v, w.scale, True, rows=rows)
    _check(f"B1 H1 N={n} causal d128 (sampled)", o[:, :, rows], lse[:, :, rows], ro, rl)


@pytest.mark.parametrize("d", [64, 128])
def test_many_heads_short_sequences(d):
    """B64 H96 (6144 heads) of 70 keys each, causal: a grid of one ragged query
    block per head, far more workgroups than the XCD remap's whole rounds; the
    oracle checks every row of 40 sampled heads."""
    w = W[1].with_(B=64, H=96, N=70, d=d, causal=True, wid=220 + d)
    _say("[case] many heads", d)
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, True)
    rng = np.random.default_rng(d)
    for b, h in zip(rng.choice(w.B, 40), rng.choice(w.H, 40)):
        ro, rl = attention_ref(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], w.scale, True)
        _check(f"many heads d={d} b={b} h={h}", o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], ro, rl)


def test_decode_many_heads():
    """B256 H64 (16 384 heads), 300 keys, 8 splits: 131 072 split workgroups."""
    w = W[4].with_(B=256, H=64, lkv=300, wid=230)
    _say("[case] decode many heads")
    q = synth.make_decode_q(w)
    k, v = synth.make_decode_kv(w, device="cuda")
    o, lse = fa.fa_decode(q.cuda(), k, v, scale=w.scale, num_splits=8)
    torch.cuda.synchronize()
    sel = np.random.default_rng(1).choice(w.B, 12, replace=False)
    idx = torch.from_numpy(sel).cuda()
    ro, rl = decode_ref(q[sel], k[idx].cpu(), v[idx].cpu(), w.scale)
    _check("decode B256 H64 L300 (12 sampled sequences)", o[sel].float().cpu().numpy()[:, :, 0], lse[sel].cpu().numpy(),
           ro, rl)


@pytest.mark.parametrize("n,causal,d", [(4097, True, 128), (4352, True, 64), (4352, False, 64)])
def test_many_blocks_ragged(n, causal, d):
    """H = 32 with ragged N: more than two query blocks per compute unit and an odd
    block count per head; sampled rows cover the block edges and the last row."""
    w = W[2].with_(B=1, H=32, N=n, d=d, causal=causal, boost_frac=0.0, wid=60 + d + (1 if causal else 0))
    _say("[case] many blocks, ragged N", n, causal, d)
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, causal)
    rng = np.random.default_rng(n + d)
    edges = [r for b in range(0, n, 256) for r in (b, b + 31, b + 32, b + 255) if r < n]
    rows = np.unique(np.concatenate([edges, [n - 1], rng.choice(n, 120, replace=False)]))
    heads = [0, 13, 31]
    ro, rl = attention_ref(q[:, heads], k[:, heads], v[:, heads], w.scale, causal, rows=rows)
    _check(f"H32 N={n} causal={causal} d={d} (sampled)", o[:, heads][:, :, rows], lse[:, heads][:, :, rows], ro, rl)


@pytest.mark.parametrize("B,H,n", [(8, 12, 1000), (4, 12, 2048), (10, 12, 1024), (3, 12, 1000)])
def test_cu_pairing_order(B, H, n):
    """d = 64 causal grids that fit the CUs at once, where workgroups are handed out
    heaviest-alone / heaviest-with-lightest (B8 H12 N1000: a ragged last block; B4 H12
    N2048: eight blocks a head; B10 H12: 60 workgroups an XCD), and one whose grid the
    XCD remap does not take (B3 H12 N1000: 18 workgroups an XCD, not whole heads):
    every block of every head against the oracle on sampled rows."""
    w = W[1].with_(B=B, H=H, N=n, wid=70 + n + B)
    _say("[case] CU pairing order", B, H, n)
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, True)
    rng = np.random.default_rng(n + B)
    edges = [r for blk in range(0, n, 256) for r in (blk, blk + 31, blk + 224, blk + 255) if r < n]
    rows = np.unique(np.concatenate([edges, [n - 1], rng.choice(n, 24, replace=False)]))
    for b in range(B):
        ro, rl = attention_ref(q[b:b + 1], k[b:b + 1], v[b:b + 1], w.scale, True, rows=rows)
        _check(f"B{B} H{H} N={n} d64 causal, batch {b} (sampled)", o[b:b + 1][:, :, rows], lse[b:b + 1][:, :, rows],
               ro, rl)


def test_decode_full_size_sampled_heads():
    """B16 H32 Lkv 32768 d128, 64 splits; the oracle recomputes 8 heads unsplit."""
    w = W[4]
    _say("[case] workload", w.name)
    q = synth.make_decode_q(w).cuda()
    k, v = synth.make_decode_kv(w, device="cuda")
    o, lse = fa.fa_decode(q, k, v, scale=w.scale, num_splits=w.num_splits)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()[:, :, 0]
    lse = lse.cpu().numpy()
    picks = [(0, 0), (3, 7), (7, 31), (8, 16), (11, 2), (12, 30), (15, 0), (15, 31)]
    for b, h in picks:
        ro, rl = decode_ref(q[b:b + 1, h:h + 1].cpu(), k[b:b + 1, h:h + 1].cpu(), v[b:b + 1, h:h + 1].cpu(), w.scale)
        _check(f"{w.name} b{b} h{h}", o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], ro, rl)


def test_decode_full_size_every_head():
    """B16 H32 Lkv 32768 d128, 64 splits: all 512 (b, h) heads against the unsplit
    oracle (one sequence's K/V copied to the host at a time)."""
    w = W[4]
    _say("[case] workload", w.name, "(every head)")
    q = synth.make_decode_q(w).cuda()
    k, v = synth.make_decode_kv(w, device="cuda")
    o, lse = fa.fa_decode(q, k, v, scale=w.scale, num_splits=w.num_splits)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()[:, :, 0]
    lse = lse.cpu().numpy()
    qh = q.cpu()
    worst = None
    for b in range(w.B):
        ro, rl = decode_ref(qh[b:b + 1], k[b:b + 1].cpu(), v[b:b + 1].cpu(), w.scale)
        rep = check_prefill(o[b:b + 1], lse[b:b + 1], ro, rl)
        assert rep["pass"], (b, rep)
        if worst is None or rep["excess"] > worst["excess"]:
            worst = dict(rep, b=b)
    _say(f"[parity] {w.name} (all 512 heads): worst sequence {worst['b']}: O max_abs={worst['max_abs']:.3g} "
         f"floor={worst['floor']:.3g} excess={worst['excess']:.3g} LSE max_abs={worst['lse_max_abs']:.3g}")
    del k, v


# ----------------------------------------------------------------------------
# ragged and odd shapes, both head dims, both mask modes


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 2, 7, 8, 63, 65, 129, 200, 1000])
def test_tails(n, causal, d):
    w = W[1].with_(B=2, H=3, N=n, d=d, causal=causal, wid=40 + d)
    _say(f"[case] tails n={n} causal={causal} d={d}")
    q, k, v = synth.make_prefill(w)
    o, lse = _run_fwd(q, k, v, w.scale, causal)
    ro, rl = attention_ref(q, k, v, w.scale, causal)
    _check(f"tails n={n} causal={causal} d={d}", o, lse, ro, rl)


@pytest.mark.parametrize("d", [64, 128])
def test_tail_past_xcd_remap(d):
    """N = 4097 (one row past a tile) with B·H·blocks divisible by 8 and not."""
    for B, H in ((1, 8), (1, 3)):
        w = W[2].with_(B=B, H=H, N=4097, d=d, boost_frac=0.0, wid=60 + d + H)
        _say(f"[case] n=4097 B={B} H={H} d={d}")
        q, k, v = synth.make_prefill(w)
        for causal in (False, True):
            o, lse = _run_fwd(q, k, v, w.scale, causal)
            rows = np.array([0, 1, 2, 127, 128, 2048, 4095, 4096])
            ro, rl = attention_ref(q, k, v, w.scale, causal, rows=rows)
            _check(f"n=4097 B={B} H={H} d={d} causal={causal}", o[:, :, rows], lse[:, :, rows], ro, rl)


# ----------------------------------------------------------------------------
# special cases


@pytest.mark.parametrize("d", [64, 128])
def test_causal_row0_is_v0(d):
    w = W[1].with_(B=1, H=4, N=300, d=d, causal=True, wid=70 + d)
    q, k, v = synth.make_prefill(w)
    o, lse = fa.fa_fwd(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])          # weight exactly 1 on key 0
    want = w.scale * (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1)
    assert torch.allclose(lse[:, :, 0].cpu().double(), want, atol=1e-4, rtol=0)


def test_large_logits_are_stable():
    """Inputs ×16 (logits in the hundreds): finite outputs within the rule."""
    w = W[2].with_(B=1, H=2, N=700, wid=80)
    q, k, v = synth.make_prefill(w)
    q = q * 16
    for causal in (False, True):
        o, lse = _run_fwd(q, k, v, w.scale, causal)
        ro, rl = attention_ref(q, k, v, w.scale, causal)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        _check(f"large logits causal={causal}", o, lse, ro, rl)


@pytest.mark.parametrize("d", [64, 128])
def test_running_max_grows_past_the_rescale_threshold(d):
    """Key rows scaled up along the sequence (×1 … ×40): logits keep growing far
    beyond the first tile's maximum, so the running max is moved (and the
    accumulator rescaled) many times, also on tiles that cross the diagonal."""
    w = W[2].with_(B=1, H=2, N=1000, d=d, boost_frac=0.0, wid=85 + d)
    q, k, v = synth.make_prefill(w)
    ramp = torch.linspace(1.0, 40.0, w.N).view(1, 1, -1, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    for causal in (False, True):
        o, lse = _run_fwd(q, k, v, w.scale, causal)
        ro, rl = attention_ref(q, k, v, w.scale, causal)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        _check(f"growing logits d={d} causal={causal}", o, lse, ro, rl)


# ----------------------------------------------------------------------------
# grouped-query decode with per-sequence key counts


def _gqa_case(B, Hq, Hkv, L, d, wid):
    w = W[4].with_(B=B, H=Hq, hkv=Hkv, lkv=L, d=d, wid=wid)
    q = synth.make_decode_q(w)
    k, v = synth.make_decode_kv(w, device="cuda")
    return w, q, k, v


@pytest.mark.parametrize("B,Hq,Hkv,L,d,ragged,S", [
    (2, 8, 8, 700, 128, False, 5),      # g = 1: multi-head
    (3, 16, 4, 1000, 128, True, 7),     # g = 4
    (2, 16, 2, 513, 64, True, 3),       # g = 8
    (2, 32, 1, 300, 128, True, 64),     # multi-query, g = 32: four groups of 8; empty segments
    (2, 6, 2, 257, 64, True, 1),        # g = 3: one query head per workgroup
    (1, 12, 4, 2000, 128, False, 2000), # one key per segment
])
def test_decode_gqa(B, Hq, Hkv, L, d, ragged, S):
    w, q, k, v = _gqa_case(B, Hq, Hkv, L, d, wid=140 + Hq + Hkv + d)
    lens = synth.make_seqlens(w) if ragged else None
    _say("[case] decode gqa", B, Hq, Hkv, L, d, None if lens is None else lens.tolist(), S)
    o, lse = fa.fa_decode_gqa(q.cuda(), k, v, seqlens=None if lens is None else lens.cuda(), scale=w.scale,
                              num_splits=S)
    torch.cuda.synchronize()
    ro, rl = decode_gqa_ref(q.float(), k.cpu(), v.cpu(), w.scale, seqlens=None if lens is None else lens.numpy())
    _check(f"decode gqa B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} S{S}", o.float().cpu().numpy()[:, :, 0], lse.cpu().numpy(),
           ro, rl)


def test_decode_is_decode_gqa_with_one_query_per_kv_head():
    w, q, k, v = _gqa_case(2, 4, 4, 900, 128, wid=150)
    o1, l1 = fa.fa_decode(q.cuda(), k, v, scale=w.scale, num_splits=9)
    o2, l2 = fa.fa_decode_gqa(q.cuda(), k, v, scale=w.scale, num_splits=9)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_gqa_full_size_sampled_heads():
    """B16 Hq32 Hkv8 Lmax 32768 d128 at the workload's split count, ragged lengths
    (one full, one of a single key); the oracle recomputes 8 query heads of 4
    sequences."""
    w = synth.BY_NAME["decode_gqa_b16hq32hkv8_lkv32768_d128_s8"]
    _say("[case] workload", w.name, "(ragged lengths)")
    q = synth.make_decode_q(w)
    k, v = synth.make_decode_kv(w, device="cuda")
    lens = synth.make_seqlens(w)
    o, lse = fa.fa_decode_gqa(q.cuda(), k, v, seqlens=lens.cuda(), scale=w.scale, num_splits=w.num_splits)
    torch.cuda.synchronize()
    g = w.H // w.kv_heads
    for b in (0, 1, 5, 15):
        heads = [0, 3, 4, 13, 17, 22, 30, 31]
        kh = sorted({h // g for h in heads})
        kb, vb = k[b:b + 1, kh].cpu(), v[b:b + 1, kh].cpu()
        remap = {x: i for i, x in enumerate(kh)}
        # the oracle sees these query heads against their own K/V heads (g = 1 after selection)
        qsel = q[b:b + 1, heads]
        kq = torch.stack([kb[0, remap[h // g]] for h in heads])[None]
        vq = torch.stack([vb[0, remap[h // g]] for h in heads])[None]
        ro, rl = decode_gqa_ref(qsel.float(), kq, vq, w.scale, seqlens=lens[b:b + 1].numpy())
        _check(f"{w.name} b={b} len={int(lens[b])}", o[b:b + 1, heads].float().cpu().numpy()[:, :, 0],
               lse[b:b + 1, heads].cpu().numpy(), ro, rl)
    del k, v


@pytest.mark.parametrize("d", [64, 128])
def test_decode_split_extremes(d):
    """num_splits = 1, = Lkv (one key each), uneven, and the default."""
    w = W[4].with_(B=2, H=3, lkv=1000, d=d, wid=90 + d)
    q = synth.make_decode_q(w)
    k, v = synth.make_decode_kv(w)
    ro, rl = decode_ref(q, k, v, w.scale)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for s in (1, 3, 7, 64, 999, 1000, None):
        o, lse = fa.fa_decode(qd, kd, vd, scale=w.scale, num_splits=s)
        torch.cuda.synchronize()
        _check(f"decode d={d} L=1000 splits={s}", o.float().cpu().numpy()[:, :, 0], lse.cpu().numpy(), ro, rl)


@pytest.mark.parametrize("lkv", [1, 2, 17, 4099])
def test_decode_short_and_ragged(lkv):
    w = W[4].with_(B=1, H=5, lkv=lkv, wid=100)
    q = synth.make_decode_q(w)
    k, v = synth.make_decode_kv(w)
    ro, rl = decode_ref(q, k, v, w.scale)
    o, lse = fa.fa_decode(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, num_splits=min(lkv, 8))
    torch.cuda.synchronize()
    _check(f"decode L={lkv}", o.float().cpu().numpy()[:, :, 0], lse.cpu().numpy(), ro, rl)
    if lkv == 1:
        assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


@pytest.mark.parametrize("splits", [64, 1024])
def test_decode_million_keys(splits):
    """B1 H4 with 2^20 + 5 keys, d = 128: 64 splits of 16 k keys and 1024 of 1 k,
    the ragged last split included."""
    w = W[4].with_(B=1, H=4, lkv=(1 << 20) + 5, wid=210)
    _say("[case] decode million keys", splits)
    q = synth.make_decode_q(w)
    k, v = synth.make_decode_kv(w)
    ro, rl = decode_ref(q, k, v, w.scale)
    o, lse = fa.fa_decode(q.cuda(), k.cuda(), v.cuda(), scale=w.scale, num_splits=splits)
    torch.cuda.synchronize()
    _check(f"decode L={w.lkv} splits={splits}", o.float().cpu().numpy()[:, :, 0], lse.cpu().numpy(), ro, rl)


# ----------------------------------------------------------------------------
# every output element written, nothing outside written, determinism


def test_canaries_and_guard_bands():
    w = W[1].with_(B=2, H=2, N=333, d=128, causal=True, wid=110)
    q, k, v = (t.cuda() for t in synth.make_prefill(w))
    n_o = q.numel()
    guard = 4096
    obuf = torch.full((n_o + 2 * guard,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((w.B * w.H * w.N + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[guard:guard + n_o].view(q.shape)
    lse = lbuf[guard:guard + w.B * w.H * w.N].view(w.B, w.H, w.N)
    fa.fa_fwd(q, k, v, scale=w.scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert torch.isnan(obuf[:guard]).all() and torch.isnan(obuf[guard + n_o:]).all()
    assert torch.isnan(lbuf[:guard]).all() and torch.isnan(lbuf[-guard:]).all()


def _guarded(n, dtype, guard=4096):
    """A NaN-filled device buffer of n elements with ``guard`` NaN elements on either side."""
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=dtype, device="cuda")
    return buf, buf[guard:guard + n], guard


def _intact(buf, guard, n):
    return bool(torch.isnan(buf[:guard]).all()) and bool(torch.isnan(buf[guard + n:]).all())


@pytest.mark.parametrize("splits", [1, 7])
def test_decode_canaries_and_guard_bands(splits):
    """fa_decode (called through the C ABI) writes every element of O and L and
    nothing around them, nor past its workspace (NaN canaries everywhere)."""
    w = W[4].with_(B=3, H=5, lkv=1000, wid=112 + splits)
    q = synth.make_decode_q(w).cuda()
    k, v = synth.make_decode_kv(w, device="cuda")
    n_o, n_l = q.numel(), w.B * w.H
    obuf, o, g = _guarded(n_o, torch.bfloat16)
    lbuf, l, _ = _guarded(n_l, torch.float32)
    need = fa.fa_decode_workspace_bytes(w.B, w.H, w.d, splits)
    wbuf, ws, _ = _guarded(need // 4, torch.float32)
    st = fa.load_library().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(), w.B, w.H,
                                     w.lkv, w.d, w.scale, splits, ws.data_ptr(), need, None)
    torch.cuda.synchronize()
    assert st == fa.FA_OK
    assert torch.isfinite(o).all() and torch.isfinite(l).all()
    assert _intact(obuf, g, n_o) and _intact(lbuf, g, n_l) and _intact(wbuf, g, need // 4)
    ro, rl = decode_ref(q.cpu(), k.cpu(), v.cpu(), w.scale)
    _check(f"decode canaries splits={splits}", o.view(w.B, w.H, w.d).float().cpu().numpy(),
           l.view(w.B, w.H).cpu().numpy(), ro, rl)


@pytest.mark.parametrize("fn", ["fa_bwd", "fa_bwd_atomic"])
def test_bwd_canaries_and_guard_bands(fn):
    """The backward (through the C ABI) writes every element of dQ, dK, dV and
    nothing around them or past its workspace."""
    w = W[1].with_(B=1, H=2, N=333, d=128, causal=True, wid=114)
    q, k, v = (t.cuda() for t in synth.make_prefill(w))
    do = synth.make_prefill_grad(w).cuda()
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    n = q.numel()
    bufs = [_guarded(n, torch.bfloat16) for _ in range(3)]
    need = (fa.fa_bwd_atomic_workspace_bytes(w.B, w.H, w.N, w.d) if fn == "fa_bwd_atomic"
            else fa.fa_bwd_workspace_bytes(w.B, w.H, w.N))
    wbuf, ws, g = _guarded(need // 4, torch.float32)
    st = getattr(fa.load_library(), fn)(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                       lse.data_ptr(), *[b[1].data_ptr() for b in bufs], w.B, w.H, w.N, w.d, w.scale,
                                       1, ws.data_ptr(), need, None)
    torch.cuda.synchronize()
    assert st == fa.FA_OK
    ref = fa.fa_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for (buf, x, gb), r in zip(bufs, ref):
        assert torch.isfinite(x).all() and _intact(buf, gb, n)
        if fn == "fa_bwd":
            assert torch.equal(x.view(r.shape), r)   # deterministic: the binding's call gives the same bits
    assert _intact(wbuf, g, need // 4)


def test_deterministic():
    w = W[2].with_(H=4, N=1500, wid=120)
    q, k, v = (t.cuda() for t in synth.make_prefill(w))
    o1, l1 = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    o2, l2 = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    wd = W[4].with_(B=2, H=4, lkv=5000, wid=121)
    qd = synth.make_decode_q(wd).cuda()
    kd, vd = synth.make_decode_kv(wd, device="cuda")
    a = fa.fa_decode(qd, kd, vd, num_splits=16)
    b = fa.fa_decode(qd, kd, vd, num_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_runs_on_a_side_stream():
    w = W[0]
    q, k, v = (t.cuda() for t in synth.make_prefill(w))
    ref_o, ref_l = fa.fa_fwd(q, k, v, scale=w.scale)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, l = fa.fa_fwd(q, k, v, scale=w.scale)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_binding_rejects_bad_outputs_and_buffers():
    """Caller-supplied out=, lse=, workspace and packed tensors are checked for
    shape, dtype, device and contiguity before the library is called."""
    w = W[0]
    q, k, v = (t.cuda() for t in synth.make_prefill(w))
    B, H, N, d = q.shape
    good_o, good_l = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    bad = [
        (dict(out=torch.empty((B, H, N - 1, d), dtype=torch.bfloat16, device="cuda")), ValueError),
        (dict(out=torch.empty_like(q).float()), TypeError),
        (dict(out=torch.empty_like(q, device="cpu")), ValueError),
        (dict(out=torch.empty((B, H, d, N), dtype=torch.bfloat16, device="cuda").transpose(2, 3)), ValueError),
        (dict(lse=torch.empty((B, H, N - 1), dtype=torch.float32, device="cuda")), ValueError),
        (dict(lse=torch.empty((B, H, N), dtype=torch.float64, device="cuda")), TypeError),
        (dict(lse=torch.empty((B, H, N), dtype=torch.float32)), ValueError),
    ]
    for kw, err in bad:
        args = dict(out=good_o, lse=good_l)
        args.update(kw)
        with pytest.raises(err):
            fa.fa_fwd(q, k, v, scale=w.scale, **args)
    wd = W[4].with_(B=1, H=2, lkv=100, wid=130)
    qd = synth.make_decode_q(wd).cuda()
    kd, vd = synth.make_decode_kv(wd, device="cuda")
    with pytest.raises(ValueError):
        fa.fa_decode(qd, kd, vd, num_splits=4, workspace=torch.empty(1 << 16, dtype=torch.uint8))
    with pytest.raises(fa.FaError):  # too small: the library's own check
        fa.fa_decode(qd, kd, vd, num_splits=4, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    q8, k8, v8 = (t.cuda() for t in synth.make_prefill(W[2].with_(B=1, H=1, N=64, wid=131)))
    packed = fa.fa_quantize_fp8(q8, k8, v8)
    with pytest.raises(fa.FaError):  # the packed buffer is for N = 64, not 128
        fa.fa_fwd_fp8(packed, 1, 1, 128, 128)
    with pytest.raises(ValueError):
        fa.fa_quantize_fp8(q8, k8, v8, packed=torch.empty_like(packed, device="cpu"))
    torch.cuda.synchronize()
