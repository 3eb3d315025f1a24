// C-ABI entry points: argument checks, kernel-instance choice, grid set-up.
// Every check runs before the first HIP call, so the library can be loaded
// and its error paths exercised on a host without a GPU.

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_fp8.h"
#include "fa_internal.h"

namespace {

constexpr int kAbiVersion = 3;
static_assert(FA_DECODE_NOALLOC_SCRATCH_BYTES == fa::kDecodeScratchBytes, "the header states the scratch size");
constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Element count B·H·N·d with overflow checks; 0 on overflow.
size_t count4(int B, int H, int N, int d) {
  const unsigned long long c = (unsigned long long)B * (unsigned long long)H * (unsigned long long)N *
                               (unsigned long long)d;
  if (c > (1ull << 46)) return 0;  // far beyond any device memory
  return (size_t)c;
}

}  // namespace

extern "C" {

const char* fa_status_str(int s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H, N or Lkv < 1, or the sizes overflow";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (d must be 64 or 128)";
    case FA_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case FA_ERR_VALUE: return "scale not positive and finite, or num_splits outside [1, Lkv]";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ALIAS: return "an output overlaps an input";
    default: return "unknown status";
  }
}

int fa_abi_version(void) { return kAbiVersion; }

fa_status fa_fwd_tile_shape(int d, int* block_m, int* block_n) {
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (block_m) *block_m = fa::kFwdBlockM;
  if (block_n) *block_n = fa::fwd_block_n(d);
  return FA_OK;
}

long long fa_fwd_tile_pairs(int N, int d, int causal) {
  if (N < 1 || (d != 64 && d != 128)) return -1;
  const int nq = fa::ceil_div(N, fa::kFwdBlockM);
  long long pairs = 0;
  for (int qb = 0; qb < nq; ++qb) pairs += fa::fwd_kv_tiles(N, d, causal, qb);
  return pairs;
}

}  // extern "C"

namespace {

fa_status fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   float scale, int causal, const unsigned char* block_mask, int mask_heads, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const size_t elems = count4(B, H, N, d);
  // one head's K (and V) is addressed through a buffer descriptor of N·d·2 bytes
  if (elems == 0 || (unsigned long long)N * d * 2 > 0x7fff0000ull || (unsigned long long)B * H > (1ull << 24) ||
      (unsigned long long)B * H * fa::ceil_div(N, fa::kFwdBlockM) > 0x7fffffffull)
    return FA_ERR_SHAPE;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  const size_t tb = elems * 2, lb = (size_t)B * H * N * 4;
  if (overlap(o, tb, q, tb) || overlap(o, tb, k, tb) || overlap(o, tb, v, tb) || overlap(lse, lb, q, tb) ||
      overlap(lse, lb, k, tb) || overlap(lse, lb, v, tb) || overlap(o, tb, lse, lb))
    return FA_ERR_ALIAS;
  const int nb = fa::ceil_div(N, fa::kSparseBlock);
  if (block_mask) {
    if (nb > fa::kSparseMaxBlocks) return FA_ERR_SHAPE;
    if (mask_heads != 1 && mask_heads != B * H) return FA_ERR_SHAPE;
    const size_t mb = (size_t)mask_heads * nb * nb;
    if (overlap(o, tb, block_mask, mb) || overlap(lse, lb, block_mask, mb)) return FA_ERR_ALIAS;
  }

  fa::FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.BH = B * H;
  p.N = N;
  // block-sparse: one workgroup per query block of the mask (kSparseBlock rows)
  p.n_qblk = block_mask ? nb : fa::ceil_div(N, fa::kFwdBlockM);
  const long long total = (long long)p.BH * p.n_qblk;
  if (total > 0x7fffffffll) return FA_ERR_SHAPE;
  p.xcd_remap = (total % 8 == 0) && ((total / 8) % p.n_qblk == 0);
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  p.block_mask = block_mask;
  p.mask_heads = mask_heads;
  p.mask_tq = nb;
  p.mask_tk = nb;
  if (fa::launch_fwd(p, d, causal ? 1 : 0, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                 int d, float scale, int causal, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, nullptr, 0, stream);
}

fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                              int d, float scale, int causal, const unsigned char* block_mask, int mask_heads,
                              void* stream) {
  if (!block_mask) return FA_ERR_NULL;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, mask_heads, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  const unsigned long long rows = (unsigned long long)B * H * N;
  if (rows > 0x7fffffffull) return 0;
  return (size_t)rows * 8;
}

}  // extern "C"

namespace {

// The dQ accumulator starts on the next 256-byte boundary after the (L, D) pairs.
size_t dqacc_offset(size_t ld_bytes) { return (ld_bytes + 255) & ~(size_t)255; }

fa_status bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
                   size_t workspace_bytes, bool fused, const unsigned char* block_mask, int mask_heads, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const size_t elems = count4(B, H, N, d);
  if (elems == 0 || (unsigned long long)N * d * 2 > 0x7fff0000ull || (unsigned long long)B * H * N > 0x7fffffffull ||
      (unsigned long long)B * H * fa::ceil_div(N, fa::kFwdBlockM) > 0x7fffffffull)
    return FA_ERR_SHAPE;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_VALUE;
  const size_t need = fused ? fa_bwd_atomic_workspace_bytes(B, H, N, d) : fa_bwd_workspace_bytes(B, H, N);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return FA_ERR_ALIGN;
  const size_t tb = elems * 2, lb = (size_t)B * H * N * 4;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const size_t in_bytes[6] = {tb, tb, tb, tb, tb, lb};
  void* outs[4] = {dq, dk, dv, workspace};
  const size_t out_bytes[4] = {tb, tb, tb, need};
  for (int a = 0; a < 4; ++a) {
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[a], out_bytes[a], ins[i], in_bytes[i])) return FA_ERR_ALIAS;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_ALIAS;
  }
  const int nb = fa::ceil_div(N, fa::kSparseBlock);
  if (block_mask) {
    if (nb > fa::kSparseMaxBlocks) return FA_ERR_SHAPE;
    if (mask_heads != 1 && mask_heads != B * H) return FA_ERR_SHAPE;
    const size_t mb = (size_t)mask_heads * nb * nb;
    for (int a = 0; a < 4; ++a)
      if (overlap(outs[a], out_bytes[a], block_mask, mb)) return FA_ERR_ALIAS;
  }

  fa::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.ld = static_cast<float*>(workspace);
  p.dqacc = fused ? reinterpret_cast<float*>(static_cast<char*>(workspace) + dqacc_offset(fa_bwd_workspace_bytes(B, H, N)))
                  : nullptr;
  p.block_mask = block_mask;
  p.mask_heads = mask_heads;
  p.mask_t = nb;
  p.BH = B * H;
  p.N = N;
  p.n_qblk = fa::ceil_div(N, fa::kFwdBlockM);
  p.n_kblk = fa::ceil_div(N, fa::kBwdBlockK);
  const long long tq = (long long)p.BH * p.n_qblk, tk = (long long)p.BH * p.n_kblk;
  p.xcd_remap_q = (tq % 8 == 0) && ((tq / 8) % p.n_qblk == 0);
  p.xcd_remap_k = (tk % 8 == 0) && ((tk / 8) % p.n_kblk == 0);
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  if (fa::launch_bwd(p, d, causal ? 1 : 0, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_atomic_workspace_bytes(int B, int H, int N, int d) {
  const size_t ld = fa_bwd_workspace_bytes(B, H, N);
  if (ld == 0 || (d != 64 && d != 128)) return 0;
  return dqacc_offset(ld) + (size_t)B * H * N * d * 4;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, workspace, workspace_bytes, false,
                  nullptr, 0, stream);
}

fa_status fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                        void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, workspace, workspace_bytes, true,
                  nullptr, 0, stream);
}

fa_status fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
                              int causal, const unsigned char* block_mask, int mask_heads, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!block_mask) return FA_ERR_NULL;
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, workspace, workspace_bytes, false,
                  block_mask, mask_heads, stream);
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits) {
  if (B < 1 || H < 1 || num_splits < 1 || (d != 64 && d != 128)) return 0;
  const size_t parts = (size_t)B * H * num_splits;
  const size_t o_bytes = parts * d * 4;                 // a multiple of 256: LSE part stays aligned
  return o_bytes + parts * 4;
}

}  // extern "C"

namespace {

// Split-KV decode, contiguous (block_table == nullptr: K/V [B, Hkv, Lmax, d])
// or paged (K/V pools [num_pages, Hkv, 2^page_shift, d], Lmax = max_pages << page_shift).
fa_status decode_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Lmax, int d, const int* seqlens, float scale, int num_splits, void* workspace,
                      size_t workspace_bytes, const int* block_table, int max_pages, int page_shift, int num_pages,
                      void* stream, bool check_only = false) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lmax < 1 || Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // bytes of K (and of V): the (b, head) caches, or the page pool
  const size_t kv_elems = block_table ? count4(num_pages, Hkv, 1 << page_shift, d) : count4(B, Hkv, Lmax, d);
  if (kv_elems == 0 || count4(B, Hq, 1, d) == 0 || (unsigned long long)B * Hq * num_splits > 0x7fffffffull)
    return FA_ERR_SHAPE;
  if (block_table && (unsigned long long)num_pages * Hkv << page_shift > 0x7fffffffull) return FA_ERR_SHAPE;
  if (!isfinite(scale) || !(scale > 0.f) || num_splits < 1 || num_splits > Lmax) return FA_ERR_VALUE;
  // check_only: every check except those of the workspace, which the caller
  // supplies afterwards (the allocation-free call's own scratch)
  const size_t need = fa_decode_workspace_bytes(B, Hq, d, num_splits);
  const size_t wb = check_only ? 0 : need;
  if (!check_only && (!workspace || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (!check_only && !aligned16(workspace)) || (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0 ||
      (reinterpret_cast<uintptr_t>(block_table) & 3u) != 0)
    return FA_ERR_ALIGN;
  const size_t qb = (size_t)B * Hq * d * 2, kb = kv_elems * 2, lb = (size_t)B * Hq * 4;
  if (overlap(o, qb, q, qb) || overlap(o, qb, k, kb) || overlap(o, qb, v, kb) || overlap(lse, lb, q, qb) ||
      overlap(lse, lb, k, kb) || overlap(lse, lb, v, kb) || overlap(o, qb, lse, lb) ||
      overlap(workspace, wb, q, qb) || overlap(workspace, wb, k, kb) || overlap(workspace, wb, v, kb) ||
      overlap(workspace, wb, o, qb) || overlap(workspace, wb, lse, lb))
    return FA_ERR_ALIAS;
  if (seqlens) {
    const size_t sb = (size_t)B * 4;
    if (overlap(o, qb, seqlens, sb) || overlap(lse, lb, seqlens, sb) || overlap(workspace, wb, seqlens, sb))
      return FA_ERR_ALIAS;
  }
  if (block_table) {
    const size_t tb = (size_t)B * max_pages * 4;
    if (overlap(o, qb, block_table, tb) || overlap(lse, lb, block_table, tb) || overlap(workspace, wb, block_table, tb))
      return FA_ERR_ALIAS;
  }
  if (check_only) return FA_OK;

  fa::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + (size_t)B * Hq * num_splits * d * 4);
  p.seqlens = seqlens;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.L = Lmax;
  p.S = num_splits;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  p.block_table = block_table;
  p.max_pages = max_pages;
  p.page_shift = page_shift;
  p.num_pages = num_pages;
  if (fa::launch_decode(p, B, d, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_decode_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                        int Lmax, int d, const int* seqlens, float scale, int num_splits, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return decode_impl(q, k, v, o, lse, B, Hq, Hkv, Lmax, d, seqlens, scale, num_splits, workspace, workspace_bytes,
                     nullptr, 0, 0, 0, stream);
}

fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse, int B, int Hq,
                          int Hkv, int d, int page_size, int num_pages, const int* block_table, int max_pages,
                          const int* seqlens, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!block_table) return FA_ERR_NULL;
  if (num_pages < 1 || max_pages < 1 || page_size < 1 || page_size > 4096 || (page_size & (page_size - 1)) != 0)
    return FA_ERR_SHAPE;
  if ((unsigned long long)max_pages * page_size > 0x7fffffffull) return FA_ERR_SHAPE;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  return decode_impl(q, k_pages, v_pages, o, lse, B, Hq, Hkv, max_pages * page_size, d, seqlens, scale, num_splits,
                     workspace, workspace_bytes, block_table, max_pages, shift, num_pages, stream);
}

fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lkv,
                    int d, float scale, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return fa_decode_gqa(q, k, v, o, lse, B, H, H, Lkv, d, nullptr, scale, num_splits, workspace, workspace_bytes,
                       stream);
}

fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Lkv,
                            int d, float scale, int num_splits, void* stream) {
  // every check of fa_decode except the workspace's, then the scratch limit, before any HIP call
  const fa_status pre = decode_impl(q, k, v, o, lse, B, H, H, Lkv, d, nullptr, scale, num_splits, nullptr, 0,
                                    nullptr, 0, 0, 0, stream, /*check_only=*/true);
  if (pre != FA_OK) return pre;
  if (fa_decode_workspace_bytes(B, H, d, num_splits) > fa::kDecodeScratchBytes) return FA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (fa::decode_scratch(&ws) != hipSuccess) return FA_ERR_LAUNCH;
  return decode_impl(q, k, v, o, lse, B, H, H, Lkv, d, nullptr, scale, num_splits, ws, fa::kDecodeScratchBytes,
                     nullptr, 0, 0, 0, stream);
}

}  // extern "C"

// ---- FP8 form of the prefill -------------------------------------------------------

namespace {

// Shape checks shared by the two FP8 calls (d = 128 only).
fa_status fp8_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  if (d != fa::kFp8D) return FA_ERR_UNSUPPORTED;
  const unsigned long long T = (unsigned long long)fa::ceil_div(N, fa::kFp8Block);
  if (count4(B, H, N, d) == 0 || (unsigned long long)N * d * 2 > 0x7fff0000ull ||
      (unsigned long long)B * H > (1ull << 24) || (unsigned long long)B * H * T > 0x7fffffffull ||
      (unsigned long long)B * H * fa::ceil_div(N, fa::kFwdBlockM) > 0x7fffffffull)
    return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_fp8_packed_bytes(int B, int H, int N, int d) {
  if (fp8_shape(B, H, N, d) != FA_OK) return 0;
  return fa::fp8_layout(B, H, N, d).total;
}

fa_status fa_quantize_fp8(const void* q, const void* k, const void* v, int B, int H, int N, int d, float scale,
                          void* packed, size_t packed_bytes, void* stream) {
  if (!q || !k || !v || !packed) return FA_ERR_NULL;
  const fa_status sh = fp8_shape(B, H, N, d);
  if (sh != FA_OK) return sh;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_VALUE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(packed)) return FA_ERR_ALIGN;
  const fa::Fp8Layout L = fa::fp8_layout(B, H, N, d);
  if (packed_bytes < L.total) return FA_ERR_WORKSPACE;
  const size_t tb = count4(B, H, N, d) * 2;
  if (overlap(packed, L.total, q, tb) || overlap(packed, L.total, k, tb) || overlap(packed, L.total, v, tb))
    return FA_ERR_ALIAS;
  fa::Fp8QuantParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.packed = static_cast<unsigned char*>(packed);
  p.L = L;
  p.BH = B * H;
  p.N = N;
  p.T = fa::ceil_div(N, fa::kFp8Block);
  p.qmul = scale * kLog2e;
  if (fa::launch_fp8_quantize(p, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_LAUNCH;
  return FA_OK;
}

fa_status fa_fwd_fp8(const void* packed, size_t packed_bytes, void* o, float* lse, int B, int H, int N, int d,
                     int causal, void* stream) {
  if (!packed || !o || !lse) return FA_ERR_NULL;
  const fa_status sh = fp8_shape(B, H, N, d);
  if (sh != FA_OK) return sh;
  const fa::Fp8Layout L = fa::fp8_layout(B, H, N, d);
  if (packed_bytes < L.total) return FA_ERR_WORKSPACE;
  if (!aligned16(packed) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  const size_t tb = count4(B, H, N, d) * 2, lb = (size_t)B * H * N * 4;
  if (overlap(o, tb, packed, L.total) || overlap(lse, lb, packed, L.total) || overlap(o, tb, lse, lb))
    return FA_ERR_ALIAS;
  fa::Fp8FwdParams p;
  p.packed = static_cast<const unsigned char*>(packed);
  p.L = L;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.BH = B * H;
  p.N = N;
  p.T = fa::ceil_div(N, fa::kFp8Block);
  p.n_qblk = fa::ceil_div(N, fa::kFwdBlockM);
  const long long total = (long long)p.BH * p.n_qblk;
  p.xcd_remap = (total % 8 == 0) && ((total / 8) % p.n_qblk == 0);
  if (fa::launch_fwd_fp8(p, causal ? 1 : 0, static_cast<hipStream_t>(stream)) != hipSuccess) return FA_ERR_LAUNCH;
  return FA_OK;
}

}  // extern "C"
