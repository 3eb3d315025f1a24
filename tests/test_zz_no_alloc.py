"""fa_decode_noalloc, the allocation-free decode, through the C ABI: on two calls
in a row (the second smaller, so it reuses the scratch the first one filled) its
outputs equal fa_decode's bit for bit, and fa_decode matches the oracle."""

import sys

import pytest

torch = pytest.importorskip("torch")

import exact_attention_31_amd as fa
import synth
from oracle import check_decode, decode_ref

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


def _noalloc(q, k, v, scale, splits):
    B, H, _, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=q.device)
    st = fa.load_library().fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                             B, H, k.shape[2], d, scale, splits,
                                             torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_str(st)
    return o, lse


def test_decode_noalloc_matches_decode_twice():
    cases = [(W.with_(B=4, H=32, lkv=8192, wid=240), 64), (W.with_(B=2, H=3, lkv=1000, wid=241), 7)]
    for w, splits in cases:
        _say("[case] decode noalloc", w.B, w.H, w.lkv, splits)
        q = synth.make_decode_q(w).cuda()
        k, v = synth.make_decode_kv(w, device="cuda")
        o1, l1 = _noalloc(q, k, v, w.scale, splits)
        o2, l2 = fa.fa_decode(q, k, v, scale=w.scale, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.isfinite(o1).all() and torch.isfinite(l1).all()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        b = w.B - 1
        ro, rl = decode_ref(q[b:b + 1].cpu(), k[b:b + 1].cpu(), v[b:b + 1].cpu(), w.scale)
        rep = check_decode(o1[b:b + 1, :, 0].float().cpu().numpy(), l1[b:b + 1].cpu().numpy(), ro, rl)
        assert rep["pass"], rep
        del k, v


def test_decode_noalloc_binding():
    w = W.with_(B=2, H=4, lkv=777, wid=242)
    q = synth.make_decode_q(w).cuda()
    k, v = synth.make_decode_kv(w, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    o1, l1 = fa.fa_decode_noalloc(q, k, v, out, lse, scale=w.scale, num_splits=5)
    o2, l2 = fa.fa_decode(q, k, v, scale=w.scale, num_splits=5)
    torch.cuda.synchronize()
    assert o1.data_ptr() == out.data_ptr() and torch.equal(o1, o2) and torch.equal(l1, l2)
    wb = W.with_(B=1, H=512, lkv=200, wid=243)  # 512 heads × 130 splits: 34.3 MB of partials
    qb = synth.make_decode_q(wb).cuda()
    kb, vb = synth.make_decode_kv(wb, device="cuda")
    assert fa.fa_decode_workspace_bytes(1, 512, 128, 130) > fa.DECODE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(fa.FaError):
        fa.fa_decode_noalloc(qb, kb, vb, torch.empty_like(qb), torch.empty((1, 512), dtype=torch.float32,
                                                                          device="cuda"), num_splits=130)


W = synth.WORKLOADS[4]
