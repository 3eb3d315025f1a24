"""GPU parity of block-sparse attention: fa_fwd_block_sparse through the C ABI
against the fp64 oracle (attention_block_sparse_ref), same rule as the dense
forward (oracle/compare.py), also where the mask keeps everything the dense
call computes (the block-sparse kernel splits every key tile between two
wavefront groups and merges their summaries with ⊕, so it rounds differently
from fa_fwd and is compared with the oracle, like fa_fwd, rather than with
fa_fwd's bits).  Rows the mask leaves without keys
must come back as O = 0 and LSE = −∞.  The backward (fa_bwd_block_sparse),
fed the block-sparse forward's own O and L, is checked against the oracle's
backward with the same mask under bwd_allowance (oracle/compare.py), and is bit
for bit fa_bwd where the mask keeps everything the dense call computes."""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import exact_attention_31_amd as fa
import synth
from oracle import attention_block_sparse_ref, bwd_allowance, check_bwd, check_prefill

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    fa.load_library()
    yield


def _check(name, o, lse, ro, rl):
    empty = np.isneginf(rl)
    assert np.all(np.isneginf(lse[empty])), name
    assert np.all(o[empty] == 0), name
    full = ~empty
    rep = check_prefill(o[full], lse[full], ro[full], rl[full])
    _say(f"[parity-sparse] {name}: empty rows {int(empty.sum())}, O max_abs={rep['max_abs']:.3g} "
         f"excess={rep['excess']:.3g} LSE max_abs={rep['lse_max_abs']:.3g} pass={rep['pass']}")
    assert rep["pass"], rep


def _random_mask(T, heads, density, seed, keep_diag=False):
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand((heads, T, T), generator=g) < density).to(torch.uint8)
    if keep_diag:
        m[:, torch.arange(T), torch.arange(T)] = 1
    return m


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,density,per_head", [(1, 1.0, False), (100, 0.0, False), (129, 0.5, True),
                                                (300, 0.4, False), (513, 0.3, True), (1000, 0.25, True)])
def test_block_sparse_against_oracle(n, density, per_head, causal, d):
    w = W[1].with_(B=2, H=2, N=n, d=d, causal=causal, wid=110 + d // 64 + 4 * causal)
    _say("[case] block sparse", n, density, per_head, causal, d)
    q, k, v = synth.make_prefill(w)
    T = -(-n // 128)
    mask = _random_mask(T, w.B * w.H if per_head else 1, density, n + d + causal)
    o, lse = fa.fa_fwd_block_sparse(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = attention_block_sparse_ref(q, k, v, w.scale, causal, mask.numpy() if per_head else mask[0].numpy())
    _check(f"N={n} density={density} per_head={per_head} causal={causal} d={d}",
           o.float().cpu().numpy(), lse.cpu().numpy(), ro, rl)


@pytest.mark.parametrize("d", [64, 128])
def test_mask_keeping_everything_is_dense_attention(d):
    """All ones (and, with causal, the lower block triangle, whose blocks above
    the diagonal the causal mask removes anyway): the block-sparse call is dense
    attention, checked against the oracle's dense attention like fa_fwd on the
    same inputs (keys ×8 on 1 % of rows, so the reference max moves)."""
    from oracle import attention_ref
    w = W[2].with_(B=1, H=4, N=1100, d=d, boost_frac=0.01, wid=120 + d // 64)
    _say("[case] block sparse vs dense", d)
    q, k, v = synth.make_prefill(w)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    T = -(-w.N // 128)
    for causal, mask in ((False, torch.ones(T, T, dtype=torch.uint8)),
                         (True, torch.tril(torch.ones(T, T, dtype=torch.uint8)))):
        o1, l1 = fa.fa_fwd(qc, kc, vc, scale=w.scale, causal=causal)
        o2, l2 = fa.fa_fwd_block_sparse(qc, kc, vc, mask.cuda(), scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        ro, rl = attention_ref(q, k, v, w.scale, causal)
        for name, o, l in (("fa_fwd", o1, l1), ("fa_fwd_block_sparse", o2, l2)):
            _check(f"all kept, {name}, causal={causal} d={d}", o.float().cpu().numpy(), l.cpu().numpy(), ro, rl)


def test_block_sparse_long_sampled_rows():
    """B1 H16 N16384 d128 with the bench's mask (local + global + 10 % random
    blocks): sampled rows of 3 heads against the oracle."""
    w = W[3]
    _say("[case] block sparse long", w.name)
    q, k, v = synth.make_prefill(w)
    mask = synth.make_block_mask(w, 0.1)
    o, lse = fa.fa_fwd_block_sparse(q.cuda(), k.cuda(), v.cuda(), mask.cuda(), scale=w.scale, causal=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 127, 128, 255, 256, w.N - 1], rng.choice(w.N, 120, replace=False)]))
    heads = [0, 7, 15]
    ro, rl = attention_block_sparse_ref(q[:, heads], k[:, heads], v[:, heads], w.scale, False, mask[0].numpy(),
                                        rows=rows)
    _check("long N16384 (sampled)", o[:, heads][:, :, rows].float().cpu().numpy(),
           lse[:, heads][:, :, rows].cpu().numpy(), ro, rl)


def _bwd_check(name, got, ref, allow):
    rep = check_bwd(got, ref, allow)
    _say(f"[parity-sparse-bwd] {name}: " + " ".join(
        f"{g} max_abs={rep[g + '_max_abs']:.3g} ratio={rep[g + '_ratio']:.3f}" for g in ("dq", "dk", "dv"))
        + f" pass={rep['pass']}")
    assert rep["pass"], rep


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,density,per_head", [(100, 0.0, False), (129, 0.5, True), (300, 0.4, False),
                                                (513, 0.3, True), (700, 0.6, False)])
def test_block_sparse_backward_against_oracle(n, density, per_head, causal, d):
    """fa_fwd_block_sparse then fa_bwd_block_sparse on ragged sizes and random
    masks (rows without keys included) against the oracle's block-sparse backward."""
    w = W[1].with_(B=1, H=2, N=n, d=d, causal=causal, wid=150 + d // 64 + 4 * causal)
    _say("[case] block sparse backward", n, density, per_head, causal, d)
    q, k, v = synth.make_prefill(w)
    do = synth.make_prefill_grad(w)
    T = -(-n // 128)
    mask = _random_mask(T, w.B * w.H if per_head else 1, density, 7 * n + d + causal)
    qc, kc, vc, mc = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    o, lse = fa.fa_fwd_block_sparse(qc, kc, vc, mc, scale=w.scale, causal=causal)
    dq, dk, dv = fa.fa_bwd_block_sparse(qc, kc, vc, o, lse, do.cuda(), mc, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    got = [x.float().cpu().numpy() for x in (dq, dk, dv)]
    m = mask.numpy() if per_head else mask[0].numpy()
    ref, allow = bwd_allowance(q, k, v, do, w.scale, causal, o_from_fwd=True, block_mask=m)
    _bwd_check(f"N={n} density={density} per_head={per_head} causal={causal} d={d}", got, ref, allow)


@pytest.mark.parametrize("d", [64, 128])
def test_block_sparse_backward_keeping_everything_is_the_dense_backward(d):
    """All ones (and, with causal, the lower block triangle): fa_bwd's bits."""
    w = W[2].with_(B=1, H=3, N=1100, d=d, boost_frac=0.01, wid=160 + d // 64)
    _say("[case] block sparse backward vs dense", d)
    q, k, v = (t.cuda() for t in synth.make_prefill(w))
    do = synth.make_prefill_grad(w).cuda()
    T = -(-w.N // 128)
    for causal, mask in ((False, torch.ones(T, T, dtype=torch.uint8)),
                         (True, torch.tril(torch.ones(T, T, dtype=torch.uint8)))):
        o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=causal)
        a = fa.fa_bwd(q, k, v, o, lse, do, scale=w.scale, causal=causal)
        b = fa.fa_bwd_block_sparse(q, k, v, o, lse, do, mask.cuda(), scale=w.scale, causal=causal)
        torch.cuda.synchronize()
        for x, y, name in zip(a, b, ("dq", "dk", "dv")):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), (causal, name)


def test_block_sparse_backward_bench_mask_4096():
    """B1 H4 N4096 d128 with the bench's mask recipe (own + first key block +
    10 % random), non-causal: two heads checked against the oracle."""
    w = W[3].with_(H=4, N=4096, wid=170)
    _say("[case] block sparse backward 4096")
    q, k, v = synth.make_prefill(w)
    do = synth.make_prefill_grad(w)
    mask = synth.make_block_mask(w, 0.1)
    qc, kc, vc, mc = q.cuda(), k.cuda(), v.cuda(), mask.cuda()
    o, lse = fa.fa_fwd_block_sparse(qc, kc, vc, mc, scale=w.scale, causal=False)
    dq, dk, dv = fa.fa_bwd_block_sparse(qc, kc, vc, o, lse, do.cuda(), mc, scale=w.scale, causal=False)
    torch.cuda.synchronize()
    hs = [0, 3]
    got = [x[:, hs].float().cpu().numpy() for x in (dq, dk, dv)]
    ref, allow = bwd_allowance(q[:, hs], k[:, hs], v[:, hs], do[:, hs], w.scale, False, o_from_fwd=True,
                               block_mask=mask[0].numpy())
    _bwd_check("B1 H4 N4096 d128 bench mask, heads [0, 3]", got, ref, allow)
