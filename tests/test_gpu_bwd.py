"""GPU parity of the backward: fa_bwd and fa_bwd_atomic through the C ABI
against the fp64 oracle.

Two ways in:
* on its own — O and L are the oracle forward's, rounded to bf16 and fp32, and
  the oracle backward takes D from the same bf16 O; the limits are
  bwd_allowance(..., o=O_bf16);
* composed — fa_fwd's own O and L feed fa_bwd, and the oracle uses the exact
  O; the limits are bwd_allowance(..., o_from_fwd=True), which adds what a
  bf16-weight forward may differ by.
Either way every element must satisfy |x − x_ref| ≤ allowance + ½ulp_bf16
(oracle/compare.py, check_bwd).  fa_bwd_atomic shares the dK/dV arithmetic of
fa_bwd, so those two must also agree bit for bit; its dQ, summed with atomic
adds in an order that varies, meets the same oracle bound.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import exact_attention_31_amd as fa
import synth
from oracle import attention_ref, bwd_allowance, check_bwd
from oracle.compare import bf16_rne

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


def _inputs(w):
    q, k, v = synth.make_prefill(w)
    return q, k, v, synth.make_prefill_grad(w)


def _oracle_fwd(q, k, v, scale, causal):
    o, lse = attention_ref(q, k, v, scale, causal)
    return torch.from_numpy(bf16_rne(o)).to(torch.bfloat16), torch.from_numpy(lse.astype(np.float32))


IMPLS = {"two-pass": fa.fa_bwd, "atomic": fa.fa_bwd_atomic}


def _bwd(q, k, v, o, lse, do, scale, causal, fn=fa.fa_bwd):
    dq, dk, dv = fn(q.cuda(), k.cuda(), v.cuda(), o.cuda(), lse.cuda(), do.cuda(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    return [x.float().cpu().numpy() for x in (dq, dk, dv)]


def _check(name, got, ref, allow):
    rep = check_bwd(got, ref, allow)
    _say(f"[parity-bwd] {name}: " + " ".join(
        f"{g} max_abs={rep[g + '_max_abs']:.3g} ratio={rep[g + '_ratio']:.3f}" for g in ("dq", "dk", "dv"))
        + f" pass={rep['pass']}")
    assert rep["pass"], rep


def _standalone(w, heads=None, fn=fa.fa_bwd):
    """The backward on the oracle's O and L for all heads; the oracle checks `heads`."""
    q, k, v, do = _inputs(w)
    o, lse = _oracle_fwd(q, k, v, w.scale, w.causal)
    got = _bwd(q, k, v, o, lse, do, w.scale, w.causal, fn)
    hs = list(range(w.H)) if heads is None else heads
    ref, allow = bwd_allowance(q[:, hs], k[:, hs], v[:, hs], do[:, hs], w.scale, w.causal, o=o[:, hs])
    _check(w.name if heads is None else f"{w.name} heads {hs}", [g[:, hs] for g in got], ref, allow)


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 7, 33, 64, 129, 200, 300, 513])
def test_bwd_tails(n, causal, d, impl):
    """Ragged N across the 32-key wavefront slices, the 128-key and 256-row blocks."""
    w = W[1].with_(B=1, H=2, N=n, d=d, causal=causal, wid=80 + d // 64 + 4 * causal)
    _say("[case] bwd tails", impl, n, causal, d)
    _standalone(w, fn=IMPLS[impl])


def test_bwd_single_head_n256_d64():
    _say("[case] bwd", W[0].name)
    _standalone(W[0])


def test_bwd_gpt2_small_causal():
    """B8 H12 N1024 d64 causal: all 96 heads on the GPU, 6 of them checked."""
    w = W[1]
    _say("[case] bwd", w.name)
    q, k, v, do = _inputs(w)
    o, lse = _oracle_fwd(q, k, v, w.scale, w.causal)
    got = _bwd(q, k, v, o, lse, do, w.scale, w.causal)
    for b in (0, 7):
        hs = [0, 5, 11]
        ref, allow = bwd_allowance(q[b:b + 1, hs], k[b:b + 1, hs], v[b:b + 1, hs], do[b:b + 1, hs], w.scale,
                                   w.causal, o=o[b:b + 1, hs])
        _check(f"{w.name} b{b} heads {hs}", [g[b:b + 1, hs] for g in got], ref, allow)


def test_bwd_llama3_full_size_composed():
    """B1 H32 N4096 d128 causal with the ×8 key rows: fa_fwd then fa_bwd on all
    heads, as the bench runs them; the oracle checks three heads exactly."""
    w = W[2]
    _say("[case] bwd composed", w.name)
    q, k, v, do = _inputs(w)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.fa_fwd(qc, kc, vc, scale=w.scale, causal=True)
    dq, dk, dv = fa.fa_bwd(qc, kc, vc, o, lse, doc, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    hs = [0, 17, 31]
    got = [x[:, hs].float().cpu().numpy() for x in (dq, dk, dv)]
    ref, allow = bwd_allowance(q[:, hs], k[:, hs], v[:, hs], do[:, hs], w.scale, True, o_from_fwd=True)
    _check(f"{w.name} heads {hs}", got, ref, allow)


@pytest.mark.parametrize("impl", list(IMPLS))
@pytest.mark.parametrize("n,causal,d", [(700, True, 128), (1000, False, 64), (4097, True, 128)])
def test_bwd_composed(n, causal, d, impl):
    w = W[2].with_(B=1, H=4 if n < 4096 else 2, N=n, d=d, causal=causal, boost_frac=0.0, wid=90 + d // 64 + 4 * causal)
    _say("[case] bwd composed", impl, n, causal, d)
    q, k, v, do = _inputs(w)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.fa_fwd(qc, kc, vc, scale=w.scale, causal=causal)
    got = [x.float().cpu().numpy() for x in IMPLS[impl](qc, kc, vc, o, lse, doc, scale=w.scale, causal=causal)]
    ref, allow = bwd_allowance(q, k, v, do, w.scale, causal, o_from_fwd=True)
    _check(f"{impl} composed N={n} causal={causal} d={d}", got, ref, allow)


def test_bwd_deterministic():
    """No atomics: two calls give the same bits."""
    w = W[1].with_(B=2, H=3, N=777, d=128, causal=True, wid=99)
    _say("[case] bwd deterministic")
    q, k, v, do = (x.cuda() for x in _inputs(w))
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    a = fa.fa_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True)
    b = fa.fa_bwd(q, k, v, o, lse, do, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("n,causal,d", [(777, True, 128), (1000, False, 64), (300, True, 64), (4096, False, 128)])
def test_bwd_atomic_shares_dk_dv_bits(n, causal, d):
    """dK and dV of fa_bwd_atomic are fa_bwd's, bit for bit; dQ agrees to the
    rounding of a reordered fp32 sum (two bf16 ulps, relative to the row's
    largest |dQ|, plus a floor)."""
    w = W[1].with_(B=2, H=2, N=n, d=d, causal=causal, wid=130 + d // 64 + 4 * causal)
    _say("[case] bwd atomic vs two-pass", n, causal, d)
    q, k, v, do = (x.cuda() for x in _inputs(w))
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=causal)
    a = fa.fa_bwd(q, k, v, o, lse, do, scale=w.scale, causal=causal)
    b = fa.fa_bwd_atomic(q, k, v, o, lse, do, scale=w.scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    assert torch.equal(a[2].view(torch.int16), b[2].view(torch.int16))
    x, y = a[0].float(), b[0].float()
    tol = 2 * 2.0 ** -8 * x.abs().amax(dim=-1, keepdim=True) + 1e-6
    assert bool(((x - y).abs() <= tol).all()), float((x - y).abs().max())


def test_bwd_atomic_llama3_full_size_composed():
    """The bench workload (B1 H32 N4096 d128 causal) through fa_bwd_atomic; the
    oracle checks three heads exactly."""
    w = W[2]
    _say("[case] bwd atomic composed", w.name)
    q, k, v, do = _inputs(w)
    qc, kc, vc, doc = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = fa.fa_fwd(qc, kc, vc, scale=w.scale, causal=True)
    dq, dk, dv = fa.fa_bwd_atomic(qc, kc, vc, o, lse, doc, scale=w.scale, causal=True)
    torch.cuda.synchronize()
    hs = [0, 17, 31]
    got = [x[:, hs].float().cpu().numpy() for x in (dq, dk, dv)]
    ref, allow = bwd_allowance(q[:, hs], k[:, hs], v[:, hs], do[:, hs], w.scale, True, o_from_fwd=True)
    _check(f"atomic {w.name} heads {hs}", got, ref, allow)


def test_bwd_atomic_workspace_reuse():
    """The accumulator is cleared by each call: a reused workspace (holding the
    previous call's sums) gives the same gradients as a fresh one."""
    w = W[1].with_(B=1, H=3, N=500, d=64, causal=True, wid=140)
    _say("[case] bwd atomic workspace reuse")
    q, k, v, do = (x.cuda() for x in _inputs(w))
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=True)
    ws = torch.empty(fa.fa_bwd_atomic_workspace_bytes(1, 3, 500, 64), dtype=torch.uint8, device="cuda")
    a = fa.fa_bwd_atomic(q, k, v, o, lse, do, scale=w.scale, causal=True, workspace=ws)
    a = [x.clone() for x in a]
    b = fa.fa_bwd_atomic(q, k, v, o, lse, do, scale=w.scale, causal=True, workspace=ws)
    torch.cuda.synchronize()
    x, y = a[0].float(), b[0].float()
    assert bool(((x - y).abs() <= 2 * 2.0 ** -8 * x.abs().amax(dim=-1, keepdim=True) + 1e-6).all())
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
