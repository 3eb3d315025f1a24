"""Seeded synthetic inputs and the workload table — shared by tests, bench and smoke.

This module holds none of the attention arithmetic: it only draws numbers.
Both the GPU library's callers and the oracle's callers take their inputs from
here, so the two sides see the same bytes.

Recipe (every tensor is bf16, i.i.d. N(0, 1)):

* Prefill q, k, v, the backward's output gradient dO, and decode q: one
  torch ``Generator`` per (workload, tensor, b, h), seeded with
  ``seed_for(...)``, so any single head can be regenerated on its own.
* ``torch.randn`` in float32, then round-to-nearest-even to bfloat16.
* The Llama-3-8B-shaped workload scales 1 % of the key rows of every (b, h) by
  8: exactly round(0.01·N) distinct rows, chosen by a seeded permutation,
  multiplied after the bf16 rounding (×8 is exact in bf16).  These large
  logits force running-max rescales.
* Decode K/V (8.6 GB at full size) are drawn on the device that will hold them
  (the generator runs where the tensor lives), one generator per (workload,
  tensor, sequence b) covering all heads of b; a CPU draw and a GPU draw with
  the same seed differ, so a GPU test takes the oracle's copy of a head from
  the device tensor itself.
"""

from dataclasses import dataclass, replace
import math

import numpy as np
import torch

BASE_SEED = 31_2026


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" or "decode"
    B: int
    H: int
    N: int               # query length (1 for decode)
    d: int
    causal: bool = False
    lkv: int = 0         # decode: cached keys per sequence
    num_splits: int = 0  # decode: KV splits
    boost_frac: float = 0.0
    boost: float = 1.0
    wid: int = 0         # seed namespace
    hkv: int = 0         # decode: key/value heads (0: as many as query heads)

    @property
    def kv_heads(self) -> int:
        return self.hkv or self.H

    @property
    def scale(self) -> float:
        """fp32(1/sqrt(d)) as a Python float (the value the library receives)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: shapes, distributions and structure of the pages' cases.
WORKLOADS = [
    Workload("single_head_b1h1n256d64", "prefill", 1, 1, 256, 64, False, wid=1),
    Workload("gpt2_small_causal_b8h12n1024d64", "prefill", 8, 12, 1024, 64, True, wid=2),
    Workload("llama3_8b_causal_b1h32n4096d128_kboost", "prefill", 1, 32, 4096, 128, True,
             boost_frac=0.01, boost=8.0, wid=3),
    Workload("long_noncausal_b1h16n16384d128", "prefill", 1, 16, 16384, 128, False, wid=4),
    Workload("decode_b16h32_lkv32768_d128_s64", "decode", 16, 32, 1, 128, False,
             lkv=32768, num_splits=64, wid=5),
]
# Grouped-query decode (Llama-3-8B's 32 query heads over 8 K/V heads), the
# widening of the decode workload above to shared K/V heads.
EXTRA_WORKLOADS = [
    Workload("decode_gqa_b16hq32hkv8_lkv32768_d128_s8", "decode", 16, 32, 1, 128, False,
             lkv=32768, num_splits=8, wid=6, hkv=8),
]
BY_NAME = {w.name: w for w in WORKLOADS + EXTRA_WORKLOADS}

_TENSOR_ID = {"q": 0, "k": 1, "v": 2, "boost": 3, "seqlens": 4, "do": 5, "mask": 6}


def seed_for(w: Workload, tensor: str, b: int, h: int) -> int:
    return BASE_SEED + (((w.wid * 8 + _TENSOR_ID[tensor]) * 4096 + b) * 4096 + h)


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn_bf16(seed: int, shape, device="cpu") -> torch.Tensor:
    """i.i.d. N(0,1) drawn in fp32 with the given seed, rounded to bf16."""
    g = _gen(seed, device)
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)


def boosted_rows(w: Workload, b: int, h: int, n: int) -> torch.Tensor:
    """The round(frac·n) distinct key rows of head (b, h) that get scaled."""
    cnt = int(round(w.boost_frac * n))
    perm = torch.randperm(n, generator=_gen(seed_for(w, "boost", b, h)))
    return perm[:cnt]


def prefill_head(w: Workload, tensor: str, b: int, h: int, n: int | None = None) -> torch.Tensor:
    """One [N, d] head of q, k or v (CPU, bf16)."""
    n = w.N if n is None else n
    x = randn_bf16(seed_for(w, tensor, b, h), (n, w.d))
    if tensor == "k" and w.boost_frac > 0.0:
        x[boosted_rows(w, b, h, n)] *= w.boost
    return x


def make_prefill(w: Workload):
    """q, k, v as CPU bf16 tensors [B, H, N, d]."""
    out = []
    for t in ("q", "k", "v"):
        x = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16)
        for b in range(w.B):
            for h in range(w.H):
                x[b, h] = prefill_head(w, t, b, h)
        out.append(x)
    return tuple(out)


def make_prefill_grad(w: Workload) -> torch.Tensor:
    """The output gradient dO [B, H, N, d] (CPU, bf16, i.i.d. N(0, 1)) for the backward."""
    x = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.bfloat16)
    for b in range(w.B):
        for h in range(w.H):
            x[b, h] = randn_bf16(seed_for(w, "do", b, h), (w.N, w.d))
    return x


def bwd_flops(w: Workload) -> float:
    """The backward's algorithmic FLOPs: five N×N×d products (S, dP, dV, dK, dQ),
    10·N²·d·B·H, halved when causal — 2.5 times the forward's."""
    f = 10.0 * w.N * w.N * w.d * w.B * w.H
    return f / 2 if w.causal else f


def make_decode_q(w: Workload) -> torch.Tensor:
    """The decode queries [B, H, 1, d] (CPU, bf16)."""
    q = torch.empty((w.B, w.H, 1, w.d), dtype=torch.bfloat16)
    for b in range(w.B):
        for h in range(w.H):
            q[b, h, 0] = randn_bf16(seed_for(w, "q", b, h), (w.d,))
    return q


def make_decode_kv(w: Workload, device="cpu"):
    """Decode K, V [B, Hkv, Lkv, d] bf16, drawn on ``device`` one sequence (all heads) at a time."""
    k = torch.empty((w.B, w.kv_heads, w.lkv, w.d), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    for b in range(w.B):
        k[b] = randn_bf16(seed_for(w, "k", b, 0), (w.kv_heads, w.lkv, w.d), device)
        v[b] = randn_bf16(seed_for(w, "v", b, 0), (w.kv_heads, w.lkv, w.d), device)
    return k, v


def paginate(k: torch.Tensor, v: torch.Tensor, page_size: int, seed: int):
    """The cache k, v [B, Hkv, L, d] (L a multiple of page_size) laid out as a pool of
    pages [B·L/page_size, Hkv, page_size, d] in a seeded random order, with the block
    table int32 [B, L/page_size] that maps each sequence's page i to its pool page
    (all on k's device)."""
    B, Hkv, L, d = k.shape
    n = L // page_size
    perm = torch.randperm(B * n, generator=_gen(seed)).to(torch.int32)
    pools = []
    for x in (k, v):
        pages = x.reshape(B, Hkv, n, page_size, d).permute(0, 2, 1, 3, 4).reshape(B * n, Hkv, page_size, d)
        pool = torch.empty_like(pages)
        pool[perm.to(torch.int64).to(x.device)] = pages
        pools.append(pool)
    return pools[0], pools[1], perm.reshape(B, n).to(k.device)


def make_seqlens(w: Workload) -> torch.Tensor:
    """Per-sequence key counts for a ragged decode batch: int32 [B], uniform on
    [1, Lkv] from a seeded generator, with the first sequence at the full Lkv
    and the second at a single key (CPU; move to the device to use)."""
    g = _gen(seed_for(w, "seqlens", 0, 0))
    lens = torch.randint(1, w.lkv + 1, (w.B,), generator=g, dtype=torch.int64)
    lens[0] = w.lkv
    if w.B > 1:
        lens[1] = 1
    return lens.to(torch.int32)


def make_block_mask(w: Workload, density: float, heads: int = 1, block: int = 128) -> torch.Tensor:
    """A seeded block mask uint8 [heads, T, T], T = ⌈N/block⌉: every query block keeps
    its own key block and key block 0 (local and global attention, so no row is
    left empty), and each other block independently with probability ``density``."""
    T = -(-w.N // block)
    g = _gen(seed_for(w, "mask", 0, heads))
    m = (torch.rand((heads, T, T), generator=g) < density).to(torch.uint8)
    idx = torch.arange(T)
    m[:, idx, idx] = 1
    m[:, :, 0] = 1
    return m


def block_sparse_flops(w: Workload, mask: torch.Tensor, block: int = 128) -> float:
    """4·d per (query, key) pair the mask keeps (and, when causal, the causal mask
    keeps), summed over the heads; with one mask it is shared by every (b, h)."""
    n = w.N
    T = mask.shape[-1]
    sizes = torch.tensor([min(block, n - i * block) for i in range(T)], dtype=torch.float64)
    if w.causal:
        # kept pairs of block (r, c): all when c < r, none when c > r, i(i+1)/2 on the diagonal
        pairs = torch.outer(sizes, sizes)
        pairs = torch.tril(pairs, -1) + torch.diag(sizes * (sizes + 1) / 2)
    else:
        pairs = torch.outer(sizes, sizes)
    kept = (mask.to(torch.float64) * pairs).sum().item()
    per_mask_heads = w.B * w.H / mask.shape[0]
    return 4.0 * w.d * kept * per_mask_heads


def prefill_flops(w: Workload) -> float:
    """4·N²·d·B·H, halved when causal (softmax work is not counted)."""
    f = 4.0 * w.N * w.N * w.d * w.B * w.H
    return f / 2 if w.causal else f


def decode_bytes(w: Workload, seqlens=None) -> float:
    """Algorithmic bytes of one decode call: the visible K and V rows once per
    K/V head, q in, O out (bf16), LSE out (fp32)."""
    keys = w.B * w.lkv if seqlens is None else int(sum(int(x) for x in seqlens))
    return float(keys * w.kv_heads * 2 * w.d * 2 + w.B * w.H * (2 * w.d * 2 + 4))


def prefill_bytes(w: Workload) -> float:
    """Algorithmic bytes of one prefill call: Q, K, V in and O out (bf16), LSE out (fp32)."""
    return float(w.B * w.H * (4 * w.N * w.d * 2 + 4 * w.N))
