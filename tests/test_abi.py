"""The C-ABI library on a host without a GPU: it loads, exports every symbol
include/fa.h declares, and rejects bad arguments before any HIP call."""

import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_31_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built (run __graft_entry__.build())")
    return fa.load_library()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("fa_fwd", "fa_decode", "fa_decode_gqa", "fa_decode_workspace_bytes", "fa_status_str",
                 "fa_fwd_tile_pairs", "fa_fwd_tile_shape", "fa_abi_version", "fa_bwd", "fa_bwd_workspace_bytes",
                 "fa_fwd_block_sparse", "fa_decode_paged", "fa_bwd_atomic", "fa_bwd_atomic_workspace_bytes",
                 "fa_bwd_block_sparse"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    assert set(_declared()) <= exported


def test_status_strings_and_version():
    _lib()
    assert fa.fa_abi_version() == 3
    assert fa.fa_status_str(0) == "ok"
    for s in range(1, 9):
        assert fa.fa_status_str(s) not in ("ok", "unknown status")
    assert fa.fa_status_str(99) == "unknown status"


# fake, 16-byte aligned, distinct "device" addresses: every call below must be
# rejected by validation, so nothing ever dereferences them
P = [ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(10)]
MISALIGNED = ctypes.c_void_p(0x10000008)


def _fwd(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, N=16, d=64, scale=0.125, causal=0):
    return _lib().fa_fwd(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), causal, None)


def _dec(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=1, L=16, d=64, scale=0.125, S=4, ws=P[5], wsb=1 << 20):
    return _lib().fa_decode(q, k, v, o, lse, B, H, L, d, ctypes.c_float(scale), S, ws, wsb, None)


def test_fwd_argument_checks():
    assert _fwd(q=None) == 1
    assert _fwd(lse=None) == 1
    assert _fwd(B=0) == 2 and _fwd(H=-1) == 2 and _fwd(N=0) == 2
    assert _fwd(d=96) == 3 and _fwd(d=256) == 3
    assert _fwd(scale=float("nan")) == 5 and _fwd(scale=float("inf")) == 5
    assert _fwd(scale=0.0) == 5 and _fwd(scale=-0.125) == 5
    assert _fwd(o=MISALIGNED) == 4
    assert _fwd(o=P[0]) == 8            # output on top of q
    assert _fwd(lse=ctypes.c_void_p(0x10000000 + 16)) == 8   # LSE inside q's range
    assert _fwd(B=1 << 20, H=1 << 20, N=1 << 20) == 2        # sizes overflow


def test_decode_argument_checks():
    assert _dec(k=None) == 1
    assert _dec(L=0) == 2
    assert _dec(d=32) == 3
    assert _dec(S=0) == 5 and _dec(S=17) == 5 and _dec(scale=float("nan")) == 5 and _dec(scale=-1.0) == 5
    assert _dec(ws=None) == 6
    need = _lib().fa_decode_workspace_bytes(1, 1, 64, 4)
    assert need == 4 * 64 * 4 + 4 * 4
    assert _dec(wsb=need - 1) == 6
    assert _dec(v=MISALIGNED) == 4
    assert _dec(ws=P[0]) == 8            # workspace on top of q
    assert _lib().fa_decode_workspace_bytes(0, 1, 64, 4) == 0
    assert _lib().fa_decode_workspace_bytes(1, 1, 80, 4) == 0


def _gqa(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, Hq=4, Hkv=2, L=16, d=64, seqlens=None, scale=0.125, S=4,
         ws=P[5], wsb=1 << 20):
    return _lib().fa_decode_gqa(q, k, v, o, lse, B, Hq, Hkv, L, d, seqlens, ctypes.c_float(scale), S, ws, wsb, None)


def test_decode_gqa_argument_checks():
    assert _gqa(k=None) == 1
    assert _gqa(Hq=6, Hkv=4) == 2          # query heads not a multiple of K/V heads
    assert _gqa(Hkv=0) == 2 and _gqa(L=0) == 2
    assert _gqa(d=32) == 3
    assert _gqa(S=17) == 5 and _gqa(scale=0.0) == 5
    assert _gqa(ws=None) == 6
    need = _lib().fa_decode_workspace_bytes(1, 4, 64, 4)   # sized by the query heads
    assert _gqa(wsb=need - 1) == 6
    assert _gqa(seqlens=ctypes.c_void_p(0x50000002)) == 4  # int32 lengths must be 4-byte aligned
    assert _gqa(seqlens=P[3]) == 8          # lengths inside the output


def _bsp(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=2, N=300, d=64, scale=0.125, causal=0, mask=P[5],
         mh=1):
    return _lib().fa_fwd_block_sparse(q, k, v, o, lse, B, H, N, d, ctypes.c_float(scale), causal, mask, mh, None)


def test_block_sparse_argument_checks():
    assert _bsp(mask=None) == 1 and _bsp(q=None) == 1
    assert _bsp(mh=3) == 2 and _bsp(mh=0) == 2        # one mask, or one per (b, h) = 2
    assert _bsp(N=1024 * 128 + 1) == 2                # more than 1024 key blocks
    assert _bsp(d=80) == 3
    assert _bsp(scale=-1.0) == 5
    assert _bsp(o=MISALIGNED) == 4
    assert _bsp(mask=ctypes.c_void_p(0x40000000 + 8)) == 8   # mask inside o's range
    assert _bsp(o=P[0]) == 8


def _bwd(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8], B=1, H=2, N=16, d=64,
         scale=0.125, causal=1, ws=P[9], wsb=1 << 20):
    return _lib().fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, ctypes.c_float(scale), causal, ws, wsb, None)


def test_bwd_argument_checks():
    assert _bwd(do=None) == 1 and _bwd(lse=None) == 1 and _bwd(dv=None) == 1
    assert _bwd(B=0) == 2 and _bwd(N=0) == 2
    assert _bwd(B=1 << 12, H=1 << 12, N=1 << 8) == 2       # B·H·N beyond 2^31 rows
    assert _bwd(d=96) == 3
    assert _bwd(scale=float("nan")) == 5 and _bwd(scale=0.0) == 5
    assert _bwd(ws=None) == 6
    need = _lib().fa_bwd_workspace_bytes(1, 2, 16)
    assert need == 2 * 16 * 8                                # one (L, D) pair per row
    assert _bwd(wsb=need - 1) == 6
    assert _bwd(dk=MISALIGNED) == 4
    assert _bwd(dq=P[0]) == 8                               # dQ on top of q
    assert _bwd(dv=P[3]) == 8                               # dV on top of o
    assert _bwd(dk=P[6]) == 8                               # two outputs on one buffer
    assert _bwd(ws=ctypes.c_void_p(0x50000000 + 16)) == 8   # workspace inside dO's range
    assert _lib().fa_bwd_workspace_bytes(0, 1, 1) == 0


def _bwda(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8], B=1, H=2, N=16, d=64,
          scale=0.125, causal=1, ws=P[9], wsb=1 << 20):
    return _lib().fa_bwd_atomic(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, ctypes.c_float(scale), causal, ws, wsb,
                                None)


def test_bwd_atomic_argument_checks():
    """Same checks as fa_bwd; the workspace adds an fp32 [B, H, N, d] accumulator."""
    assert _bwda(q=None) == 1 and _bwda(ws=None) == 6
    assert _bwda(d=96) == 3 and _bwda(scale=float("inf")) == 5
    assert _bwda(B=1 << 12, H=1 << 12, N=1 << 8) == 2
    need = _lib().fa_bwd_atomic_workspace_bytes(1, 2, 16, 64)
    assert need == 256 + 2 * 16 * 64 * 4                       # pairs padded to 256 bytes, then fp32 dQ
    assert _lib().fa_bwd_atomic_workspace_bytes(1, 2, 16, 128) == 256 + 2 * 16 * 128 * 4
    assert _lib().fa_bwd_atomic_workspace_bytes(1, 1, 33, 64) == 512 + 33 * 64 * 4
    assert _bwda(wsb=need - 1) == 6
    assert _bwda(d=128, wsb=need) == 6                          # d = 128 needs the larger buffer
    assert _bwda(dq=P[1]) == 8 and _bwda(ws=ctypes.c_void_p(0x50000000 + 16)) == 8
    assert _bwda(ws=MISALIGNED) == 4
    assert _lib().fa_bwd_atomic_workspace_bytes(1, 1, 1, 80) == 0
    assert _lib().fa_bwd_atomic_workspace_bytes(0, 1, 1, 64) == 0


def _bwds(q=P[0], k=P[1], v=P[2], o=P[3], do=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8], B=1, H=2, N=300, d=64,
          scale=0.125, causal=1, mask=ctypes.c_void_p(0xC0000000), mh=1, ws=P[9], wsb=1 << 20):
    return _lib().fa_bwd_block_sparse(q, k, v, o, do, lse, dq, dk, dv, B, H, N, d, ctypes.c_float(scale), causal,
                                      mask, mh, ws, wsb, None)


def test_bwd_block_sparse_argument_checks():
    """fa_bwd's checks plus the mask's (as for fa_fwd_block_sparse)."""
    assert _bwds(mask=None) == 1 and _bwds(dq=None) == 1
    assert _bwds(mh=3) == 2 and _bwds(mh=0) == 2          # one mask, or one per (b, h) = 2
    assert _bwds(N=1024 * 128 + 1, wsb=1 << 30) == 2     # more than 1024 key blocks
    assert _bwds(d=80) == 3 and _bwds(scale=0.0) == 5
    assert _bwds(ws=None) == 6 and _bwds(wsb=2 * 300 * 8 - 1) == 6
    assert _bwds(dv=MISALIGNED) == 4
    assert _bwds(dq=ctypes.c_void_p(0xC0000000 - 1024)) == 8  # dQ running into the mask
    assert _bwds(ws=ctypes.c_void_p(0xC0000000 - 4096)) == 8  # workspace running into the mask
    assert _bwds(dk=P[0]) == 8


def _paged(q=P[0], kp=P[1], vp=P[2], o=P[3], lse=P[4], B=2, Hq=4, Hkv=2, d=64, ps=16, npg=8, tbl=P[5], mp=4,
           seqlens=None, scale=0.125, S=4, ws=P[6], wsb=1 << 20):
    return _lib().fa_decode_paged(q, kp, vp, o, lse, B, Hq, Hkv, d, ps, npg, tbl, mp, seqlens, ctypes.c_float(scale), S,
                                  ws, wsb, None)


def test_decode_paged_argument_checks():
    assert _paged(tbl=None) == 1 and _paged(kp=None) == 1
    assert _paged(ps=24) == 2 and _paged(ps=0) == 2 and _paged(ps=8192) == 2   # powers of two up to 4096
    assert _paged(npg=0) == 2 and _paged(mp=0) == 2
    assert _paged(npg=1 << 20, Hkv=2, Hq=4, ps=4096) == 2                      # pool of 2^33 rows
    assert _paged(d=80) == 3
    assert _paged(S=65) == 5                                                   # more splits than 4·16 keys
    assert _paged(ws=None) == 6
    assert _paged(tbl=ctypes.c_void_p(0x60000002)) == 4                        # int32 table, 4-byte aligned
    assert _paged(tbl=P[3]) == 8                                               # table inside the output
    assert _paged(o=P[1]) == 8                                                 # output inside the K pool


def test_tile_shape():
    _lib()
    assert fa.fa_fwd_tile_shape(128) == (256, 64)
    assert fa.fa_fwd_tile_shape(64) == (256, 64)
    with pytest.raises(fa.FaError):
        fa.fa_fwd_tile_shape(80)


@pytest.mark.parametrize("d", [64, 128])
def test_causal_tile_skip_counts(d):
    """Square tiles: T(T+1)/2 of T² (query block, key tile) pairs are visited ([15-779 L5] §6.2)."""
    _lib()
    bm, bn = fa.fa_fwd_tile_shape(d)
    for n in (1, 100, 128, 1000, 4096, 16384):
        tq = -(-n // bm)
        tk = -(-n // bn)
        assert fa.fa_fwd_tile_pairs(n, d, False) == tq * tk
        # causal: query block i visits the key tiles up to its last row
        want = sum(-(-min(n, (i + 1) * bm) // bn) for i in range(tq))
        assert fa.fa_fwd_tile_pairs(n, d, True) == want
    if bm == bn:
        for t in (1, 4, 32):
            assert fa.fa_fwd_tile_pairs(t * bm, d, True) == t * (t + 1) // 2
    # the page's numbers: T = 4 visits 10 of 16 pairs; at T = 32 the ratio is 51.6 %
    assert 4 * 5 // 2 == 10 and abs(32 * 33 / 2 / 32 ** 2 - 0.516) < 5e-4
    assert fa.fa_fwd_tile_pairs(0, d, True) == -1


def test_python_binding_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    _lib()
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):          # CPU tensors are refused before any call
        fa.fa_fwd(q, q, q)
    with pytest.raises(TypeError):
        fa.fa_fwd(q.float(), q, q)


def _q8(q=P[0], k=P[1], v=P[2], B=1, H=2, N=300, d=128, scale=0.1, pk=P[3], pkb=1 << 30):
    lib = _lib()
    lib.fa_quantize_fp8.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_void_p,
                                                                                   ctypes.c_size_t, ctypes.c_void_p]
    return lib.fa_quantize_fp8(q, k, v, B, H, N, d, scale, pk, pkb, None)


def _f8(pk=P[3], o=P[4], lse=P[5], B=1, H=2, N=300, d=128, causal=1, pkb=1 << 30):
    lib = _lib()
    lib.fa_fwd_fp8.argtypes = [ctypes.c_void_p, ctypes.c_size_t] + [ctypes.c_void_p] * 2 + [ctypes.c_int] * 5 + \
        [ctypes.c_void_p]
    return lib.fa_fwd_fp8(pk, pkb, o, lse, B, H, N, d, causal, None)


def test_fp8_packed_bytes_follow_the_documented_layout():
    lib = _lib()
    lib.fa_fp8_packed_bytes.argtypes = [ctypes.c_int] * 4
    lib.fa_fp8_packed_bytes.restype = ctypes.c_size_t
    pad = lambda n: (n + 255) // 256 * 256
    B, H, N, d = 2, 3, 300, 128
    T = -(-N // 64)
    want = 2 * pad(B * H * N * d) + pad(B * H * T * d * 64) + 3 * pad(B * H * T * 4)
    assert lib.fa_fp8_packed_bytes(B, H, N, d) == want
    assert lib.fa_fp8_packed_bytes(B, H, N, 64) == 0 and lib.fa_fp8_packed_bytes(B, H, 0, d) == 0


def test_fp8_argument_checks():
    """Every call here fails validation before any HIP call."""
    assert _q8(q=None) == 1 and _q8(pk=None) == 1
    assert _q8(N=0) == 2 and _q8(d=64) == 3
    assert _q8(scale=0.0) == 5 and _q8(scale=float("nan")) == 5 and _q8(scale=-1.0) == 5
    assert _q8(pkb=1000) == 6
    assert _q8(v=MISALIGNED) == 4
    assert _q8(pk=P[0]) == 8  # the buffer over q
    assert _f8(pk=None) == 1 and _f8(lse=None) == 1
    assert _f8(B=0) == 2 and _f8(d=64) == 3
    assert _f8(o=MISALIGNED) == 4
    assert _f8(o=P[3]) == 8  # O over the packed operands
    assert _f8(pkb=1000) == 6  # a packed buffer smaller than the layout needs


def _dn(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=1, H=512, L=128, d=128, scale=0.1, S=64):
    lib = _lib()
    return lib.fa_decode_noalloc(q, k, v, o, lse, B, H, L, d, scale, S, None)


def test_decode_noalloc_argument_checks():
    """The allocation-free decode validates like fa_decode and rejects partials
    beyond its scratch (32 MiB) before any HIP call."""
    assert fa.DECODE_NOALLOC_SCRATCH_BYTES == 32 << 20
    assert _dn(q=None) == 1 and _dn(lse=None) == 1
    assert _dn(B=0) == 2 and _dn(d=96) == 3 and _dn(scale=-1.0) == 5 and _dn(S=0) == 5 and _dn(S=129) == 5
    assert _dn(o=MISALIGNED) == 4
    assert _dn(o=P[0]) == 8  # the output over q
    assert fa.fa_decode_workspace_bytes(16, 32, 128, 64) <= fa.DECODE_NOALLOC_SCRATCH_BYTES
    assert fa.fa_decode_workspace_bytes(1, 512, 128, 128) > fa.DECODE_NOALLOC_SCRATCH_BYTES
    assert _dn(S=128) == 6  # partials of 33.8 MB do not fit (K and V: 16.8 MB each)
