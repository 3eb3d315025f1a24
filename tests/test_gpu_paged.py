"""GPU parity of decode over a paged K/V cache: fa_decode_paged through the C ABI,
bit for bit against fa_decode_gqa on the contiguous cache the page table
describes (same keys, same order, same arithmetic), and against the fp64 oracle
(decode_paged_ref) with the decode rule of oracle/compare.py."""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import exact_attention_31_amd as fa
import synth
from oracle import check_decode, decode_paged_ref

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    fa.load_library()
    yield


def _paged_case(B, Hq, Hkv, max_pages, P, d, seed, spare=5):
    """A contiguous cache [B, Hkv, max_pages·P, d], the same keys scattered into a
    pool of pages under a seeded permutation, and that page table."""
    g = torch.Generator().manual_seed(seed)
    L = max_pages * P
    q = torch.randn(B, Hq, 1, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, Hkv, L, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, Hkv, L, d, generator=g).to(torch.bfloat16)
    n_pages = B * max_pages + spare
    perm = torch.randperm(n_pages, generator=g)[: B * max_pages].reshape(B, max_pages).to(torch.int32)
    kp = torch.randn(n_pages, Hkv, P, d, generator=g).to(torch.bfloat16)   # unmapped pages hold noise
    vp = torch.randn(n_pages, Hkv, P, d, generator=g).to(torch.bfloat16)
    for b in range(B):
        for i in range(max_pages):
            kp[perm[b, i]] = k[b, :, i * P:(i + 1) * P]
            vp[perm[b, i]] = v[b, :, i * P:(i + 1) * P]
    return q, k, v, kp, vp, perm


@pytest.mark.parametrize("B,Hq,Hkv,max_pages,P,d,S", [
    (3, 4, 4, 9, 16, 128, 5),      # multi-head, segments across page edges
    (4, 32, 8, 6, 64, 128, 7),     # Llama-3-like groups
    (2, 8, 1, 3, 256, 64, 4),      # multi-query, large pages
    (5, 16, 2, 40, 1, 64, 16),     # one key per page
    (2, 4, 2, 1, 4096, 128, 64),   # one page per sequence
])
def test_paged_is_the_contiguous_decode_bit_for_bit(B, Hq, Hkv, max_pages, P, d, S):
    _say("[case] paged vs contiguous", B, Hq, Hkv, max_pages, P, d, S)
    q, k, v, kp, vp, tbl = _paged_case(B, Hq, Hkv, max_pages, P, d, seed=B * 100 + P + d)
    L = max_pages * P
    lens = torch.randint(1, L + 1, (B,), generator=torch.Generator().manual_seed(P)).to(torch.int32)
    lens[0] = L
    dev = "cuda"
    o1, l1 = fa.fa_decode_gqa(q.to(dev), k.to(dev), v.to(dev), seqlens=lens.to(dev), scale=0.1, num_splits=S)
    o2, l2 = fa.fa_decode_paged(q.to(dev), kp.to(dev), vp.to(dev), tbl.to(dev), seqlens=lens.to(dev), scale=0.1,
                                num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("P,d", [(16, 128), (64, 64)])
def test_paged_against_oracle(P, d):
    B, Hq, Hkv, max_pages = 3, 8, 2, 7
    _say("[case] paged vs oracle", P, d)
    q, _, _, kp, vp, tbl = _paged_case(B, Hq, Hkv, max_pages, P, d, seed=7 + P)
    lens = torch.tensor([max_pages * P, 1, 3 * P + 5], dtype=torch.int32)
    o, lse = fa.fa_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), tbl.cuda(), seqlens=lens.cuda(), scale=0.09,
                                num_splits=6)
    torch.cuda.synchronize()
    ro, rl = decode_paged_ref(q, kp, vp, tbl.numpy(), lens.numpy(), 0.09)
    rep = check_decode(o[:, :, 0].float().cpu().numpy(), lse.cpu().numpy(), ro, rl)
    _say(f"[parity-paged] P={P} d={d}: O max_abs={rep['max_abs']:.3g} LSE max_abs={rep['lse_max_abs']:.3g}")
    assert rep["pass"], rep


def test_paged_table_entries_are_clamped_into_the_pool():
    """Entries below 0 or past the pool read the first or the last page."""
    B, Hq, Hkv, max_pages, P, d = 2, 4, 2, 4, 16, 64
    _say("[case] paged clamping")
    q, _, _, kp, vp, tbl = _paged_case(B, Hq, Hkv, max_pages, P, d, seed=99, spare=0)
    n_pages = kp.shape[0]
    bad = tbl.clone()
    bad[0, 1] = -7
    bad[1, 2] = n_pages + 3
    o, lse = fa.fa_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), bad.cuda(), scale=0.125, num_splits=3)
    torch.cuda.synchronize()
    ro, rl = decode_paged_ref(q, kp, vp, np.clip(bad.numpy(), 0, n_pages - 1), np.full(B, max_pages * P), 0.125)
    rep = check_decode(o[:, :, 0].float().cpu().numpy(), lse.cpu().numpy(), ro, rl)
    assert rep["pass"], rep


def test_paged_full_size_matches_contiguous():
    """The grouped-query bench workload (B16, 32 over 8 heads, 32768 keys, d128) in
    64-key pages under a seeded permutation: bit-identical to the contiguous call."""
    w = synth.BY_NAME["decode_gqa_b16hq32hkv8_lkv32768_d128_s8"]
    _say("[case] paged full size", w.name)
    q = synth.make_decode_q(w).cuda()
    k, v = synth.make_decode_kv(w, device="cuda")
    kp, vp, tbl = synth.paginate(k, v, 64, seed=5)
    o1, l1 = fa.fa_decode_gqa(q, k, v, scale=w.scale, num_splits=w.num_splits)
    o2, l2 = fa.fa_decode_paged(q, kp, vp, tbl, scale=w.scale, num_splits=w.num_splits)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
