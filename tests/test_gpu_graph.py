"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph over the
library's stream argument): a serving or training loop that replays the same
launches with new inputs copied into the captured buffers.

Every entry point launches kernels only (no allocation, copy, memset or
synchronisation inside the library), so capture records kernel nodes alone; the
binding's output and workspace tensors come from the graph's memory pool.  Each
replay runs after eager work and a synchronisation, with its outputs wiped
first, and must reproduce the eager call on the same inputs bit for bit."""

import sys

import pytest

torch = pytest.importorskip("torch")

import exact_attention_31_amd as fa
import synth

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


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def _inputs(seed):
    """Prefill (B1 H4 N1000 d128 causal), its output gradient, a decode batch
    (B2 H8 Lkv 5000 d128) and a paged grouped-query decode batch, all seeded."""
    w = W[2].with_(B=1, H=4, N=1000, d=128, causal=True, boost_frac=0.0, wid=300 + seed)
    q, k, v = synth.make_prefill(w)
    do = synth.make_prefill_grad(w)
    wd = W[4].with_(B=2, H=8, lkv=5000, wid=320 + seed)
    qd = synth.make_decode_q(wd)
    kd, vd = synth.make_decode_kv(wd)
    g = torch.Generator().manual_seed(seed)
    kp = torch.randn(12, 2, 64, 128, generator=g).to(torch.bfloat16)
    vp = torch.randn(12, 2, 64, 128, generator=g).to(torch.bfloat16)
    qp = torch.randn(2, 8, 1, 128, generator=g).to(torch.bfloat16)
    return dict(q=q, k=k, v=v, do=do, qd=qd, kd=kd, vd=vd, qp=qp, kp=kp, vp=vp), w.scale, wd.scale


def _step(t, scale, dscale, tbl, lens):
    """One pass over the entry points: forward, backward, decode, paged decode, and the FP8
    quantising pass and forward."""
    o, lse = fa.fa_fwd(t["q"], t["k"], t["v"], scale=scale, causal=True)
    g2 = fa.fa_bwd(t["q"], t["k"], t["v"], o, lse, t["do"], scale=scale, causal=True)
    od, ld = fa.fa_decode(t["qd"], t["kd"], t["vd"], scale=dscale, num_splits=16)
    op, lp = fa.fa_decode_paged(t["qp"], t["kp"], t["vp"], tbl, seqlens=lens, scale=dscale, num_splits=5)
    packed = fa.fa_quantize_fp8(t["q"], t["k"], t["v"], scale=scale)
    B, H, N, d = t["q"].shape
    o8, l8 = fa.fa_fwd_fp8(packed, B, H, N, d, causal=True)
    return [o, lse, *g2, od, ld, op, lp, o8, l8]


def test_graph_replays_match_eager_on_new_inputs():
    dev = "cuda"
    tbl = torch.tensor([[3, 7, 1, 10, 0, 5], [2, 11, 4, 9, 8, 6]], dtype=torch.int32, device=dev)
    lens = torch.tensor([384, 301], dtype=torch.int32, device=dev)
    first, scale, dscale = _inputs(0)
    static = {n: x.to(dev) for n, x in first.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture, as torch advises
        _step(static, scale, dscale, tbl, lens)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _step(static, scale, dscale, tbl, lens)
    torch.cuda.synchronize()

    for rep in range(3):
        _say("[case] graph replay", rep)
        fresh, _, _ = _inputs(rep)
        for n, x in fresh.items():
            static[n].copy_(x.to(dev))
        want = [x.clone() for x in _step(static, scale, dscale, tbl, lens)]  # eager, same inputs
        torch.cuda.synchronize()
        for x in outs:
            x.fill_(float("nan") if x.is_floating_point() else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        names = ("o", "lse", "dq", "dk", "dv", "o_decode", "lse_decode", "o_paged", "lse_paged", "o_fp8", "lse_fp8")
        for name, a, b in zip(names, outs, want):
            assert _same(a, b), (rep, name)


def _more_inputs(seed):
    """The prefill batch of _inputs with a seeded block mask, a grouped-query
    decode batch (B2, Hq 8 over Hkv 2, Lmax 700 d128) and the decode batch."""
    t, scale, dscale = _inputs(seed)
    g = torch.Generator().manual_seed(1000 + seed)
    t["qg"] = torch.randn(2, 8, 1, 128, generator=g).to(torch.bfloat16)
    t["kg"] = torch.randn(2, 2, 700, 128, generator=g).to(torch.bfloat16)
    t["vg"] = torch.randn(2, 2, 700, 128, generator=g).to(torch.bfloat16)
    return t, scale, dscale


def _more_step(t, scale, dscale, mask, glens):
    """The entry points _step leaves out: block-sparse forward and backward, the
    atomic backward, grouped-query decode with per-sequence lengths, and decode
    into caller-owned outputs with the library's own scratch."""
    o, lse = fa.fa_fwd_block_sparse(t["q"], t["k"], t["v"], mask, scale=scale, causal=True)
    gs = fa.fa_bwd_block_sparse(t["q"], t["k"], t["v"], o, lse, t["do"], mask, scale=scale, causal=True)
    od, ld = fa.fa_fwd(t["q"], t["k"], t["v"], scale=scale, causal=True)
    ga = fa.fa_bwd_atomic(t["q"], t["k"], t["v"], od, ld, t["do"], scale=scale, causal=True)
    og, lg = fa.fa_decode_gqa(t["qg"], t["kg"], t["vg"], seqlens=glens, scale=dscale, num_splits=4)
    on = torch.empty(t["qd"].shape, dtype=torch.bfloat16, device=t["qd"].device)
    ln = torch.empty(t["qd"].shape[:2], dtype=torch.float32, device=t["qd"].device)
    fa.fa_decode_noalloc(t["qd"], t["kd"], t["vd"], on, ln, scale=dscale, num_splits=16)
    return [o, lse, *gs, *ga, og, lg, on, ln]


def test_graph_replays_more_entry_points():
    """The same replay protocol over the remaining entry points.  The atomic
    backward adds its dQ shares in no fixed order, so its dQ is compared within
    one bf16 step of its largest value; every other output bit for bit."""
    dev = "cuda"
    first, scale, dscale = _more_inputs(0)
    static = {n: x.to(dev) for n, x in first.items()}
    w = W[2].with_(B=1, H=4, N=1000, d=128, causal=True)
    mask = synth.make_block_mask(w, 0.4).to(dev)
    glens = torch.tensor([700, 523], dtype=torch.int32, device=dev)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _more_step(static, scale, dscale, mask, glens)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _more_step(static, scale, dscale, mask, glens)
    torch.cuda.synchronize()

    names = ("o_sparse", "lse_sparse", "dq_sparse", "dk_sparse", "dv_sparse", "dq_atomic", "dk_atomic",
             "dv_atomic", "o_gqa", "lse_gqa", "o_noalloc", "lse_noalloc")
    for rep in range(3):
        _say("[case] graph replay, more entry points", rep)
        fresh, _, _ = _more_inputs(rep)
        for n, x in fresh.items():
            static[n].copy_(x.to(dev))
        want = [x.clone() for x in _more_step(static, scale, dscale, mask, glens)]
        torch.cuda.synchronize()
        for x in outs:
            x.fill_(float("nan") if x.is_floating_point() else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, want):
            if name == "dq_atomic":
                top = b.float().abs().max().item()
                err = (a.float() - b.float()).abs().max().item()
                assert err <= top * 2.0**-7, (rep, name, err, top)
            else:
                assert _same(a, b), (rep, name)
