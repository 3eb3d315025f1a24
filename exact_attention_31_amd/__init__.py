"""Python binding of the exact-attention HIP library (``libfa.so``).

Argument marshalling only: the functions below check tensors, allocate the
outputs with torch (device memory and the current stream are all torch is used
for) and call the C ABI declared in ``include/fa.h``.  Every step of the
computation runs in the library's HIP kernels; there is no fallback — if the
library is missing or fails to load, the calls raise.

    fa_fwd(q, k, v, scale=None, causal=False)        -> (o, lse)
    fa_decode(q, k, v, scale=None, num_splits=None)  -> (o, lse)
    fa_decode_gqa(q, k, v, seqlens=None, scale=None, num_splits=None) -> (o, lse)
    fa_decode_paged(q, k_pages, v_pages, block_table, seqlens=None, ...) -> (o, lse)
    fa_decode_noalloc(q, k, v, out, lse, scale=None, num_splits=None) -> (out, lse)
    fa_decode_workspace_bytes(B, H, d, num_splits)   -> int
    fa_fwd_block_sparse(q, k, v, block_mask, scale=None, causal=False) -> (o, lse)
    fa_bwd(q, k, v, o, lse, do, scale=None, causal=False) -> (dq, dk, dv)
    fa_bwd_workspace_bytes(B, H, N)                  -> int
    fa_bwd_atomic(q, k, v, o, lse, do, scale=None, causal=False) -> (dq, dk, dv)
    fa_bwd_block_sparse(q, k, v, o, lse, do, block_mask, scale=None, causal=False) -> (dq, dk, dv)
    fa_bwd_atomic_workspace_bytes(B, H, N, d)        -> int
    fa_fwd_tile_pairs(N, d, causal)                  -> int   (host-only)
    fa_fwd_tile_shape(d)                             -> (block_m, block_n)
    fa_status_str(status)                            -> str
"""

import ctypes
import math
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_UNSUPPORTED", 4: "FA_ERR_ALIGN",
    5: "FA_ERR_VALUE", 6: "FA_ERR_WORKSPACE", 7: "FA_ERR_LAUNCH", 8: "FA_ERR_ALIAS",
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({fa_status_str(status)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m exact_attention_31_amd.build` "
            "(or __graft_entry__.build()) first — there is no non-HIP fallback"
        )
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_decode.restype = i
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    lib.fa_decode_noalloc.restype = i
    lib.fa_decode_gqa.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, f, i, vp, sz, vp]
    lib.fa_decode_gqa.restype = i
    lib.fa_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
    lib.fa_fwd_block_sparse.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_bwd_atomic.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
    lib.fa_bwd_atomic.restype = i
    lib.fa_bwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, sz, vp]
    lib.fa_bwd_block_sparse.restype = i
    lib.fa_bwd_atomic_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_bwd_atomic_workspace_bytes.restype = sz
    lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, i, vp, f, i, vp, sz, vp]
    lib.fa_decode_paged.restype = i
    lib.fa_fp8_packed_bytes.argtypes = [i, i, i, i]
    lib.fa_fp8_packed_bytes.restype = sz
    lib.fa_quantize_fp8.argtypes = [vp, vp, vp, i, i, i, i, f, vp, sz, vp]
    lib.fa_quantize_fp8.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, sz, vp, vp, i, i, i, i, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_fwd_tile_pairs.argtypes = [i, i, i]
    lib.fa_fwd_tile_pairs.restype = ctypes.c_longlong
    lib.fa_fwd_tile_shape.argtypes = [i, ctypes.POINTER(i), ctypes.POINTER(i)]
    lib.fa_fwd_tile_shape.restype = i
    lib.fa_status_str.argtypes = [i]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    _lib = lib
    return lib


def fa_status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


def fa_abi_version() -> int:
    return load_library().fa_abi_version()


def fa_fwd_tile_pairs(N: int, d: int, causal: bool) -> int:
    return int(load_library().fa_fwd_tile_pairs(int(N), int(d), int(bool(causal))))


def fa_fwd_tile_shape(d: int):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    st = load_library().fa_fwd_tile_shape(int(d), ctypes.byref(bm), ctypes.byref(bn))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_tile_shape")
    return bm.value, bn.value


def fa_decode_workspace_bytes(B: int, H: int, d: int, num_splits: int) -> int:
    return int(load_library().fa_decode_workspace_bytes(int(B), int(H), int(d), int(num_splits)))


def fa_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(load_library().fa_bwd_workspace_bytes(int(B), int(H), int(N)))


def fa_bwd_atomic_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(load_library().fa_bwd_atomic_workspace_bytes(int(B), int(H), int(N), int(d)))


def _torch():
    import torch
    return torch


def _check(t, name, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_out(t, name, shape, dtype, device):
    """A caller-supplied output tensor: exactly ``shape`` and ``dtype``, contiguous, on ``device``."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_buffer(t, name, device):
    """A caller-supplied scratch or operand buffer: a contiguous tensor on ``device``;
    returns its size in bytes (the library checks it against what the call needs)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.numel() * t.element_size()


def _stream_ptr(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fa_fwd(q, k, v, scale=None, causal=False, out=None, lse=None):
    """Prefill: O = softmax(scale·QKᵀ [+ causal mask])·V and LSE, q/k/v bf16 [B, H, N, d].

    Returns (o bf16 [B, H, N, d], lse fp32 [B, H, N]).  ``scale`` defaults to
    fp32(1/sqrt(d)).  Runs asynchronously on the current stream.
    """
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, 4)
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, "out", q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_out(lse, "lse", (B, H, N), torch.float32, q.device)
    st = load_library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, N, d, float(scale), int(bool(causal)), _stream_ptr(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")
    return out, lse


SPARSE_BLOCK = 128


def _check_mask(block_mask, BH, T, device):
    """The block mask as a contiguous uint8 [1 or B·H, T, T] tensor on ``device``."""
    torch = _torch()
    m = block_mask
    if not isinstance(m, torch.Tensor) or m.device != device:
        raise ValueError("block_mask must be a tensor on q's device")
    if m.dtype == torch.bool:
        m = m.to(torch.uint8)
    if m.dtype != torch.uint8:
        raise TypeError("block_mask must be uint8 or bool")
    if m.dim() == 2:
        m = m.unsqueeze(0)
    if m.dim() != 3 or m.shape[1:] != (T, T) or m.shape[0] not in (1, BH):
        raise ValueError(f"block_mask must be [T, T] or [B*H, T, T] with T = {T}, got {tuple(block_mask.shape)}")
    return m.contiguous()


def fa_fwd_block_sparse(q, k, v, block_mask, scale=None, causal=False, out=None, lse=None):
    """Block-sparse prefill: fa_fwd with the score blocks whose mask entry is zero set
    to −∞ and skipped.  ``block_mask``: uint8 (or bool) [T, T] or [B·H, T, T] on q's
    device, T = ⌈N/128⌉.  Rows left with no key get O = 0 and LSE = −∞."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, 4)
    if not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v shapes differ")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    T = -(-N // SPARSE_BLOCK)
    m = _check_mask(block_mask, B * H, T, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, "out", q.shape, torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_out(lse, "lse", (B, H, N), torch.float32, q.device)
    st = load_library().fa_fwd_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                            B, H, N, d, float(scale), int(bool(causal)), m.data_ptr(), m.shape[0],
                                            _stream_ptr(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_block_sparse")
    return out, lse


def fa_decode(q, k, v, scale=None, num_splits=None, workspace=None):
    """Split-KV decode: q bf16 [B, H, 1, d], k/v bf16 [B, H, Lkv, d].

    Returns (o bf16 [B, H, 1, d], lse fp32 [B, H]).  ``num_splits`` defaults
    to about 1024 workgroups (``default_splits``); the workspace
    is allocated with torch when not given.  Runs on the current stream.
    """
    torch = _torch()
    _check(q, "q", 4)
    _check(k, "k", 4)
    _check(v, "v", 4)
    B, H, one, d = q.shape
    if one != 1:
        raise ValueError(f"decode takes one query per sequence, q has {one}")
    if k.shape != v.shape or k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    L = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = default_splits(B * H, L)
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    need = fa_decode_workspace_bytes(B, H, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = _check_buffer(workspace, "workspace", q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    st = load_library().fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, H, L, d, float(scale), int(num_splits), workspace.data_ptr(),
                                  wbytes, _stream_ptr(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_decode")
    return o, lse


DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


def fa_decode_noalloc(q, k, v, out, lse, scale=None, num_splits=None):
    """fa_decode for callers that cannot allocate: the caller passes the outputs
    (out bf16 [B, H, 1, d], lse fp32 [B, H]); the split partials go to the
    library's own per-GPU scratch (DECODE_NOALLOC_SCRATCH_BYTES), so nothing is
    allocated.  Calls that may overlap on one GPU race on that scratch.
    Returns (out, lse)."""
    torch = _torch()
    _check(q, "q", 4)
    _check(k, "k", 4)
    _check(v, "v", 4)
    B, H, one, d = q.shape
    if one != 1:
        raise ValueError(f"decode takes one query per sequence, q has {one}")
    if k.shape != v.shape or k.shape[:2] != (B, H) or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    _check_out(out, "out", q.shape, torch.bfloat16, q.device)
    _check_out(lse, "lse", (B, H), torch.float32, q.device)
    L = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = default_splits(B * H, L)
    st = load_library().fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                          B, H, L, d, float(scale), int(num_splits), _stream_ptr(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_decode_noalloc")
    return out, lse


def default_splits(groups: int, L: int) -> int:
    """Segments per (sequence, head group): about 1024 workgroups in all, at least
    512 keys per segment, at most L segments.  With nontemporal loads, fewer and
    longer segments stream faster: at Lkv 32768, B16 H32 runs at 87.7 % of 8 TB/s
    with 4-8 segments against 82.4 % with 64, and B1 with 8 K/V heads at 64
    segments beats 32 and 128."""
    return max(1, min(L, -(-1024 // groups), max(1, L // 512)))


def _group_width(g: int) -> int:
    return 8 if g % 8 == 0 else 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1


def fa_decode_gqa(q, k, v, seqlens=None, scale=None, num_splits=None, workspace=None):
    """Grouped-query split-KV decode: q bf16 [B, Hq, 1, d], k/v bf16 [B, Hkv, Lmax, d]
    with Hq a multiple of Hkv (query head h reads K/V head h // (Hq // Hkv)).

    ``seqlens`` (int32 [B] on the device, or None) gives each sequence's number of
    keys; entries outside [1, Lmax] are clamped by the kernel.  Returns
    (o bf16 [B, Hq, 1, d], lse fp32 [B, Hq]).  Runs on the current stream.
    """
    torch = _torch()
    _check(q, "q", 4)
    _check(k, "k", 4)
    _check(v, "v", 4)
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError(f"decode takes one query per sequence, q has {one}")
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, L = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError(f"query heads {Hq} are not a multiple of K/V heads {Hkv}")
    sl = None
    if seqlens is not None:
        if not isinstance(seqlens, torch.Tensor) or seqlens.dtype != torch.int32 or seqlens.shape != (B,):
            raise TypeError("seqlens must be an int32 tensor of shape [B]")
        if seqlens.device != q.device or not seqlens.is_contiguous():
            raise ValueError("seqlens must be contiguous and on q's device")
        sl = seqlens.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        g = Hq // Hkv
        num_splits = default_splits(B * Hkv * (g // _group_width(g)), L)
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    need = fa_decode_workspace_bytes(B, Hq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = _check_buffer(workspace, "workspace", q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = load_library().fa_decode_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      B, Hq, Hkv, L, d, sl, float(scale), int(num_splits), workspace.data_ptr(),
                                      wbytes, _stream_ptr(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_decode_gqa")
    return o, lse


def _bwd_call(fn, q, k, v, o, lse, do, scale, causal, workspace, block_mask=None):
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (do, "do")):
        _check(t, n, 4)
    if not (q.shape == k.shape == v.shape == o.shape == do.shape):
        raise ValueError("q, k, v, o, do must have one shape")
    if len({t.device for t in (q, k, v, o, do, lse)}) != 1:
        raise ValueError("all tensors must be on one device")
    B, H, N, d = q.shape
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or lse.shape != (B, H, N) \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_bwd_atomic_workspace_bytes(B, H, N, d) if fn == "fa_bwd_atomic" else fa_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = _check_buffer(workspace, "workspace", q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal))]
    if block_mask is not None:
        args += [block_mask.data_ptr(), block_mask.shape[0]]
    st = getattr(load_library(), fn)(*args, workspace.data_ptr(), wbytes, _stream_ptr(q.device))
    if st != FA_OK:
        raise FaError(st, fn)
    return dq, dk, dv


def fa_bwd(q, k, v, o, lse, do, scale=None, causal=False, workspace=None):
    """Backward of fa_fwd: q, k, v, o, do bf16 [B, H, N, d], lse fp32 [B, H, N]
    (o and lse as fa_fwd returned them, do the gradient with respect to o).

    Returns (dq, dk, dv), bf16 [B, H, N, d].  ``scale`` and ``causal`` must be
    the forward's.  The workspace (fa_bwd_workspace_bytes) is allocated with
    torch when not given.  Runs on the current stream.  Deterministic.
    """
    return _bwd_call("fa_bwd", q, k, v, o, lse, do, scale, causal, workspace)


def fa_bwd_block_sparse(q, k, v, o, lse, do, block_mask, scale=None, causal=False, workspace=None):
    """Backward of fa_fwd_block_sparse: as fa_bwd, with the block mask the forward
    used (uint8 [T, T] or [B·H, T, T], T = ⌈N/128⌉, on the device).  o and lse
    must be that forward's outputs."""
    torch = _torch()
    B, H, N, d = q.shape
    T = -(-N // SPARSE_BLOCK)
    m = _check_mask(block_mask, B * H, T, q.device)
    return _bwd_call("fa_bwd_block_sparse", q, k, v, o, lse, do, scale, causal, workspace, block_mask=m)


def fa_bwd_atomic(q, k, v, o, lse, do, scale=None, causal=False, workspace=None):
    """fa_bwd in one key-block pass, dQ added up with atomics: same arguments and
    results up to the order of dQ's fp32 additions (not bit-reproducible).  The
    workspace is fa_bwd_atomic_workspace_bytes(B, H, N, d) bytes."""
    return _bwd_call("fa_bwd_atomic", q, k, v, o, lse, do, scale, causal, workspace)


def fa_decode_paged(q, k_pages, v_pages, block_table, seqlens=None, scale=None, num_splits=None, workspace=None):
    """Grouped-query split-KV decode over a paged cache: q bf16 [B, Hq, 1, d];
    k_pages/v_pages bf16 [num_pages, Hkv, page_size, d]; block_table int32
    [B, max_pages] (device); seqlens int32 [B] (device) or None (all
    max_pages·page_size keys).  Returns (o bf16 [B, Hq, 1, d], lse fp32 [B, Hq])."""
    torch = _torch()
    _check(q, "q", 4)
    _check(k_pages, "k_pages", 4)
    _check(v_pages, "v_pages", 4)
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError(f"decode takes one query per sequence, q has {one}")
    if k_pages.shape != v_pages.shape or k_pages.shape[3] != d:
        raise ValueError("k_pages/v_pages shapes must match and end in d")
    num_pages, Hkv, page_size = k_pages.shape[:3]
    if Hq % Hkv:
        raise ValueError(f"query heads {Hq} are not a multiple of K/V heads {Hkv}")
    t = block_table
    if not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 2 or t.shape[0] != B:
        raise TypeError("block_table must be an int32 tensor [B, max_pages]")
    if t.device != q.device or not t.is_contiguous():
        raise ValueError("block_table must be contiguous and on q's device")
    max_pages = t.shape[1]
    sl = None
    if seqlens is not None:
        if not isinstance(seqlens, torch.Tensor) or seqlens.dtype != torch.int32 or seqlens.shape != (B,):
            raise TypeError("seqlens must be an int32 tensor of shape [B]")
        if seqlens.device != q.device or not seqlens.is_contiguous():
            raise ValueError("seqlens must be contiguous and on q's device")
        sl = seqlens.data_ptr()
    L = max_pages * page_size
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        g = Hq // Hkv
        num_splits = default_splits(B * Hkv * (g // _group_width(g)), L)
    if not (q.device == k_pages.device == v_pages.device):
        raise ValueError("q, k_pages, v_pages must be on one device")
    need = fa_decode_workspace_bytes(B, Hq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    wbytes = _check_buffer(workspace, "workspace", q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = load_library().fa_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), o.data_ptr(),
                                        lse.data_ptr(), B, Hq, Hkv, d, page_size, num_pages, t.data_ptr(), max_pages,
                                        sl, float(scale), int(num_splits), workspace.data_ptr(),
                                        wbytes, _stream_ptr(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_decode_paged")
    return o, lse


def fa_fp8_packed_bytes(B: int, H: int, N: int, d: int) -> int:
    """Bytes of the packed FP8 operand buffer for Q, K, V [B, H, N, d] (0 if unsupported)."""
    return int(load_library().fa_fp8_packed_bytes(B, H, N, d))


def fa_quantize_fp8(q, k, v, scale=None, packed=None):
    """Block-wise FP8 (E4M3) quantisation of bf16 q, k, v [B, H, N, 128] into the
    packed operand buffer of fa_fwd_fp8 (a uint8 tensor; allocated when not given),
    for the softmax scale ``scale`` (default fp32(1/sqrt(d))), which is folded into
    Q.  Runs asynchronously on the current stream; returns the buffer."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, n, 4)
    if not (q.shape == k.shape == v.shape):
        raise ValueError(f"q, k, v shapes differ: {tuple(q.shape)}, {tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_fp8_packed_bytes(B, H, N, d)
    if packed is None:
        packed = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    pbytes = _check_buffer(packed, "packed", q.device)
    st = load_library().fa_quantize_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d, float(scale),
                                        packed.data_ptr(), pbytes, _stream_ptr(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_quantize_fp8")
    return packed


def fa_fwd_fp8(packed, B, H, N, d=128, causal=False, out=None, lse=None):
    """Attention forward on the FP8 operands fa_quantize_fp8 wrote (for the
    softmax scale it was given): returns (o bf16 [B, H, N, d], lse fp32 [B, H, N])."""
    torch = _torch()
    if not isinstance(packed, torch.Tensor) or packed.dtype != torch.uint8:
        raise TypeError("packed must be a uint8 tensor")
    if packed.device.type != "cuda":
        raise ValueError(f"packed must be on a ROCm device, got {packed.device}")
    pbytes = _check_buffer(packed, "packed", packed.device)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=packed.device)
    _check_out(out, "out", (B, H, N, d), torch.bfloat16, packed.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=packed.device)
    _check_out(lse, "lse", (B, H, N), torch.float32, packed.device)
    st = load_library().fa_fwd_fp8(packed.data_ptr(), pbytes, out.data_ptr(), lse.data_ptr(), B, H, N, d,
                                   int(bool(causal)), _stream_ptr(packed.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_fp8")
    return out, lse
