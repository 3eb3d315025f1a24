/* fa.h — C ABI of the exact-attention library for MI355X (gfx950).
 *
 * Exact attention (the result of standard attention up to rounding order):
 * the forward and decode calls return the output O and the per-row
 * log-sum-exp L; the backward call returns the gradients of Q, K and V:
 *
 *   fa_fwd     prefill: O = softmax(scale · Q Kᵀ [+ causal mask]) V, computed as
 *              one fused, tiled pass with an online softmax, so the N×N score
 *              and probability matrices never exist in device memory.
 *              Definition: [cicada] §1.2–1.3 (scaled dot-product attention and
 *              its steps); the loop order, running (m, ℓ, Õ) state, single
 *              division and L = m + ln ℓ follow [cicada] §3.2.1–3.2.3 and
 *              [15-779 L5] §5.1; skipping of key tiles wholly above the
 *              diagonal follows [15-779 L5] §6.2.
 *   fa_decode  decode: one new query per sequence against Lkv cached keys, with
 *              the keys split into segments whose partial results are merged by
 *              the ⊕ log-sum-exp combine ([15-779 L5] §8.4, §4.4–4.5);
 *              fa_decode_gqa adds grouped query heads (several query heads per
 *              cached K/V head) and per-sequence key counts, fa_decode_paged
 *              reads the cache through a page table.
 *   fa_fwd_block_sparse  fa_fwd with blocks of the score matrix switched off
 *              by a block mask, their work and K/V traffic skipped
 *              ([FA-1拆解] "块稀疏扩展").
 *   fa_bwd     backward of fa_fwd: dQ, dK, dV from the saved O and L, with
 *              the probabilities recomputed rather than stored
 *              ([15-779 L5] §7; [pinghaoyang FA-1] "Backward").
 *   fa_bwd_atomic  the same gradients in one key-block pass with dQ added up
 *              atomically ([15-779 L5] §7.4): not bit-reproducible.
 *   fa_bwd_block_sparse  backward of fa_fwd_block_sparse.
 *   fa_quantize_fp8, fa_fwd_fp8  the forward on FP8 (E4M3) operands with
 *              block-wise scales ([cicada] §4.4.1, FlashAttention-3).
 *
 * Pages cited: [cicada] "已有的几种大模型上下文支持情况" (blog on standard attention
 * and FlashAttention 1–4, cicada.microarchitecture.cn); [15-779 L5] "第 5 讲 ·
 * 案例：Transformer、注意力与 FlashAttention" (CMU 15-779 lecture 5 notes);
 * [pinghaoyang FA-1] "FlashAttention 完全拆解（一）" (pinghaoyang.com.cn).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers owned by the caller; the library
 *   never allocates, frees or retains device memory.
 * - bf16 tensors are raw IEEE bfloat16 (2 bytes), fp32 tensors are IEEE float.
 * - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *   Calls enqueue work and return without synchronising.
 * - Every argument check runs before any HIP call; a failed check returns a
 *   status and enqueues nothing.  A failed launch returns FA_ERR_LAUNCH.  No
 *   exceptions or aborts cross the ABI.
 * - Base pointers must be 16-byte aligned (FA_ERR_ALIGN).
 * - Outputs must not overlap the inputs (FA_ERR_ALIAS).
 * - Supported head dimensions: d ∈ {64, 128} (FA_ERR_UNSUPPORTED otherwise).
 * - Thread safety: calls hold no global mutable state and may be issued from
 *   several host threads; calls on one stream run in stream order.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  FA_ERR_SHAPE = 2,       /* B, H, N or Lkv < 1, or the sizes overflow           */
  FA_ERR_UNSUPPORTED = 3, /* head dimension other than 64 or 128                 */
  FA_ERR_ALIGN = 4,       /* a base pointer is not 16-byte aligned               */
  FA_ERR_VALUE = 5,       /* scale not > 0 and finite, or num_splits outside [1, Lkv] */
  FA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required          */
  FA_ERR_LAUNCH = 7,      /* the HIP runtime rejected a kernel launch            */
  FA_ERR_ALIAS = 8        /* an output overlaps an input                         */
} fa_status;

/* Prefill forward.
 *   q, k, v : bf16 [B, H, N, d], contiguous row-major (d fastest).
 *   o       : bf16 [B, H, N, d], written in full.
 *   lse     : fp32 [B, H, N], natural-log log-sum-exp of each row's scaled,
 *             masked logits: L_i = ln Σ_j exp(scale · q_i·k_j).
 *   scale   : multiplies Q Kᵀ before the softmax (1/sqrt(d) in the usual case);
 *             must be positive and finite (FA_ERR_VALUE otherwise).
 *   causal  : nonzero masks key j from query i when j > i (square, top-left
 *             aligned: query i sees keys 0..i).
 * Any N ≥ 1 is accepted; N need not be a multiple of a tile.  Inputs must be
 * finite, and |v| < 2^56: the kernel keeps the unnormalised softmax weights
 * below 2^48 (a stale running max is only moved when a logit outgrows it by
 * that much), so the fp32 accumulation of weight·v cannot overflow. */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, void* stream);

/* Query rows and keys per block of the fa_fwd_block_sparse mask. */
#define FA_SPARSE_BLOCK 128

/* Block-sparse prefill forward ([FA-1拆解] "块稀疏扩展"): fa_fwd with whole
 * blocks of the score matrix switched off by a mask, their computation and
 * their K/V reads skipped.
 *   block_mask : device uint8 [mask_heads, T, T], T = ⌈N / FA_SPARSE_BLOCK⌉,
 *             row-major; entry (r, c) nonzero keeps the scores of query rows
 *             r·128 … r·128+127 against keys c·128 … c·128+127, zero sets them
 *             to −∞ (like the causal mask, with which it combines when causal
 *             is set).  T ≤ 1024 (N ≤ 131072).
 *   mask_heads : 1 (one mask for every (b, h)) or B·H (mask of (b, h) at
 *             index b·H + h).
 * A query row left with no key at all gets O = 0 and L = −∞.  Other
 * arguments, conventions and errors as for fa_fwd; FA_ERR_NULL for a NULL
 * mask, FA_ERR_SHAPE for T > 1024 or mask_heads not in {1, B·H},
 * FA_ERR_ALIAS when o or lse overlaps the mask. */
fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, int d, float scale, int causal,
                              const unsigned char* block_mask, int mask_heads, void* stream);

/* Bytes of device workspace fa_bwd needs: fp32 pairs [B, H, N, 2].
 * Returns 0 when the sizes are invalid. */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/* Prefill backward: the gradients of the loss through O = fa_fwd(q, k, v).
 *   q, k, v : bf16 [B, H, N, d], the forward's inputs.
 *   o, lse  : the forward's outputs (bf16 [B, H, N, d] and fp32 [B, H, N]);
 *             P is recomputed tile by tile as exp(scale·q_i·k_j − L_i), never
 *             stored ([15-779 L5] §7.2), and D_i = dO_i · O_i is formed from o
 *             once per row ([15-779 L5] §7.3).
 *   dout    : bf16 [B, H, N, d], the gradient of the loss with respect to O.
 *   dq, dk, dv : bf16 [B, H, N, d], written in full:
 *             dV = Pᵀ dO,  dS = P ∘ (dO Vᵀ − D),  dQ = scale · dS K,
 *             dK = scale · dSᵀ Q  ([15-779 L5] §7.1; [pinghaoyang FA-1]
 *             "Backward").  Deterministic: the same inputs give the same bits.
 *   scale, causal : as passed to fa_fwd.
 *   workspace : device buffer of at least fa_bwd_workspace_bytes(B, H, N)
 *             bytes, 16-byte aligned, owned by the caller; contents on entry
 *             ignored, on exit unspecified; calls sharing it must be ordered.
 * Two kernels run in stream order: dQ (query blocks outside), which also forms
 * each row's (L, D) pair into the workspace, then dK and dV (key blocks
 * outside, query tiles inside, [15-779 L5] §7.4), which read the pairs.
 * Errors as for fa_fwd; FA_ERR_WORKSPACE for a missing or
 * short workspace; FA_ERR_ALIAS when an output or the workspace overlaps an
 * input or another output.  B·H·N must stay below 2^31. */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                 float scale, int causal, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace fa_bwd_atomic needs: the pairs of fa_bwd, padded
 * to a multiple of 256 bytes, then an fp32 dQ accumulator [B, H, N, d].
 * Returns 0 when the sizes are invalid. */
size_t fa_bwd_atomic_workspace_bytes(int B, int H, int N, int d);

/* The same backward in the loop order of [15-779 L5] §7.4 alone: one kernel
 * walks the query tiles inside each key block and adds that block's share of
 * dQ, dS K, into an fp32 accumulator with device-scope atomic adds; a last
 * pass scales and rounds it into dq.  Five products per tile instead of seven,
 * but the order of the additions into dQ follows the hardware's scheduling,
 * so dq may differ between calls in its last bits (dk and dv do not).
 * Arguments, layouts and errors as for fa_bwd, except:
 *   workspace : at least fa_bwd_atomic_workspace_bytes(B, H, N, d) bytes,
 *             16-byte aligned, owned by the caller; contents on entry ignored
 *             (the accumulator is cleared by the call), on exit unspecified;
 *             calls sharing it must be ordered. */
fa_status fa_bwd_atomic(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                        float scale, int causal, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of fa_fwd_block_sparse ([FA-1拆解] "块稀疏扩展" applied to the
 * backward of [15-779 L5] §7): the gradients of the loss through
 * O = fa_fwd_block_sparse(q, k, v, block_mask).  Switched-off blocks of the
 * score matrix contribute nothing and their tiles are skipped in both passes
 * (the dK/dV pass walks only the query blocks that keep its key block, the dQ
 * pass only the key blocks its rows keep).  Arguments, layouts, workspace
 * (fa_bwd_workspace_bytes) and errors as for fa_bwd; block_mask and
 * mask_heads as for fa_fwd_block_sparse, and o and lse must be that call's
 * outputs (a row with no key has O = 0, L = −∞ and gets dQ = 0).  FA_ERR_NULL
 * for a missing mask, FA_ERR_ALIAS when an output or the workspace overlaps
 * the mask.  Deterministic. */
fa_status fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                              float scale, int causal, const unsigned char* block_mask, int mask_heads,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace fa_decode needs for these sizes: the per-split
 * partial results, fp32 [B, H, num_splits, d] then fp32 [B, H, num_splits].
 * Returns 0 when the sizes are invalid. */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/* Split-KV decode (one query per sequence, no mask).
 *   q, o    : bf16 [B, H, 1, d].
 *   k, v    : bf16 [B, H, Lkv, d], contiguous per (b, h) (the cached keys and
 *             values, read in place: segments are views, not copies).
 *   lse     : fp32 [B, H].
 *   scale   : as for fa_fwd (positive and finite).
 *   num_splits : number of key segments, 1 ≤ num_splits ≤ Lkv.  Segment s
 *             covers keys [⌊s·Lkv/S⌋, ⌊(s+1)·Lkv/S⌋).
 *   workspace : device buffer of at least fa_decode_workspace_bytes(...) bytes,
 *             16-byte aligned, owned by the caller; its contents on entry are
 *             ignored and on exit are unspecified.  Calls that share one
 *             workspace must be ordered (same stream), or they race.
 * Two kernels run in stream order: the per-segment partials, then the ⊕
 * combine that writes o and lse. */
fa_status fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Lkv, int d, float scale, int num_splits,
                    void* workspace, size_t workspace_bytes, void* stream);

/* fa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments and result without the workspace.  The per-split partials go
 * to a scratch array of FA_DECODE_NOALLOC_SCRATCH_BYTES (32 MiB) that the
 * library keeps in device memory, one per GPU, for the life of the process;
 * the call itself allocates and frees nothing.  Needs
 * fa_decode_workspace_bytes(B, H, d, num_splits) ≤ that size, else
 * FA_ERR_WORKSPACE (the decode workload B16 H32 d128 with 64 splits needs
 * 16.9 MB).  Nothing in the scratch has to start at zero (every partial is
 * written before it is read).  Every call on one GPU shares that GPU's
 * scratch: calls that may overlap on one GPU (different streams, other host
 * threads) race and must be ordered by the caller.  Other errors as for
 * fa_decode; FA_ERR_LAUNCH also when the scratch's address cannot be found. */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
fa_status fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Lkv, int d, float scale, int num_splits, void* stream);

/* Grouped-query split-KV decode with per-sequence key counts.
 *   q, o    : bf16 [B, Hq, 1, d].
 *   k, v    : bf16 [B, Hkv, Lmax, d], contiguous per (b, K/V head).  Hq must
 *             be a multiple of Hkv: with g = Hq/Hkv, query head h attends
 *             with K/V head ⌊h/g⌋ (g query heads share one cached head,
 *             [15-779 L5] §12 exercise 7; g = 1 is multi-head, Hkv = 1
 *             multi-query).
 *   seqlens : device int32 [B] (4-byte aligned) or NULL.  Sequence b attends
 *             to its keys 0 .. seqlens[b]-1; entries outside [1, Lmax] are
 *             clamped into it (the device reads them: no host check is
 *             possible).  NULL: every sequence has Lmax keys.
 *   lse     : fp32 [B, Hq].
 *   num_splits : 1 ≤ S ≤ Lmax.  Sequence b's keys are split into segments
 *             [⌊s·len_b/S⌋, ⌊(s+1)·len_b/S⌋); a segment left empty by a
 *             short sequence contributes nothing.
 *   workspace : at least fa_decode_workspace_bytes(B, Hq, d, num_splits)
 *             bytes, otherwise as for fa_decode.
 * Other arguments, errors and stream behaviour as for fa_decode, which is
 * this call with Hq = Hkv = H and seqlens = NULL. */
fa_status fa_decode_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int Hq, int Hkv, int Lmax, int d, const int* seqlens,
                        float scale, int num_splits, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Grouped-query split-KV decode over a paged K/V cache.
 *   k_pages, v_pages : bf16 [num_pages, Hkv, page_size, d] — a pool of pages;
 *             page p of K/V head h holds page_size consecutive keys of one
 *             sequence, contiguous (page_size·d elements).
 *   block_table : device int32 [B, max_pages] (4-byte aligned): key t of
 *             sequence b is row t mod page_size of page
 *             block_table[b·max_pages + ⌊t/page_size⌋].  Entries outside
 *             [0, num_pages) are clamped into it (the device reads them).
 *   page_size : a power of two, 1 … 4096.
 *   seqlens : as for fa_decode_gqa, with Lmax = max_pages·page_size; NULL:
 *             every sequence holds Lmax keys.
 * The result is fa_decode_gqa's on the cache the table describes (the same
 * keys in the same order, the same arithmetic).  Paging is a layout of the
 * cache, which the pages set beside tiled computation ([FA-1拆解], closing
 * section).  Other arguments, workspace and errors as for fa_decode_gqa;
 * FA_ERR_NULL for a NULL table, FA_ERR_SHAPE for a page size that is not a
 * power of two in range, num_pages or max_pages < 1, or a pool of 2^31 rows
 * or more. */
fa_status fa_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse,
                          int B, int Hq, int Hkv, int d, int page_size, int num_pages,
                          const int* block_table, int max_pages, const int* seqlens, float scale,
                          int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* ---- FP8 form of the prefill ([cicada] §4.4.1: block-wise quantisation) ----
 *
 * fa_quantize_fp8 turns bf16 Q, K, V [B, H, N, d] (d = 128) into the packed FP8
 * operand buffer that fa_fwd_fp8 reads, for the softmax scale `scale` (finite,
 * > 0; fp32(1/√d) is the usual one).  Q is taken as c·Q, c = scale·log2(e)
 * (both factors in fp32, product rounded to fp32, each element's product
 * rounded to fp32): the softmax scale, in base 2, travels in Q's codes, so the
 * forward's logits come out of its first product in base 2.  Every run of 64
 * rows of one (b, h) slice of each tensor (c·Q, K, V) gets its own scale
 * s = 2^e, e the smallest integer with (largest |x| of the block) ≤ 448·2^e,
 * clamped to [−127, 127] (e = 0 for an all-zero block); each element becomes
 * the OCP E4M3FN value nearest to x/s (ties to even).  The buffer holds, each section 256-byte aligned and in this
 * order, with T = ⌈N/64⌉: the codes of Q and of K ([B·H][N][d] bytes each); the
 * codes of V one 64-key tile at a time, transposed, [B·H][T][d][64] bytes, the
 * 64 keys of a row in the order that the forward's second product reads them
 * (byte j holds key 32⌊j/16 mod 2⌋ + 8⌊(j mod 16)/4⌋ + 4⌊j/32⌋ + j mod 4 of the
 * tile; keys past N are zero); then the scales of Q, K and V as int32 E8M0
 * bytes e + 127, [B·H][T] each.  packed_bytes must be at least
 * fa_fp8_packed_bytes(B, H, N, d); the buffer may not overlap q, k or v.
 *
 * fa_fwd_fp8 computes O [B, H, N, d] (bf16) and L [B, H, N] (fp32, natural log)
 * of the attention these operands define, exact attention of the dequantised
 * Q̂' = s·q₈' (≈ c·Q), K̂, V̂ with base-2 logits Q̂'K̂ᵀ (the scale the buffer
 * was quantised for) and causal as for fa_fwd, except that the
 * probabilities enter the second product rounded to E4M3, block-quantised in
 * turn: the probabilities of a row over each aligned half (32 keys) of a
 * 64-key tile are divided by a power of two 2^σ no larger than 2^-7 times their
 * sum before rounding, and the product is scaled back by 2^σ (O is divided by
 * the sum of the unrounded ones).  Both products run on the FP8 matrix cores with
 * the block scales applied inside them.  All pointers are device pointers the
 * caller owns; packed_bytes is the size of the packed buffer, which must be
 * at least fa_fp8_packed_bytes(B, H, N, d) and hold what fa_quantize_fp8 wrote
 * for the same B, H, N.  Status codes as for fa_fwd, FA_ERR_UNSUPPORTED for
 * d ≠ 128, FA_ERR_WORKSPACE for a short buffer. */
size_t fa_fp8_packed_bytes(int B, int H, int N, int d);
fa_status fa_quantize_fp8(const void* q, const void* k, const void* v, int B, int H, int N, int d, float scale,
                          void* packed, size_t packed_bytes, void* stream);
fa_status fa_fwd_fp8(const void* packed, size_t packed_bytes, void* o, float* lse, int B, int H, int N, int d,
                     int causal, void* stream);

/* Number of (query block, key tile) pairs fa_fwd processes for one (b, h),
 * with the block and tile sizes of fa_fwd_tile_shape: ⌈N/BM⌉·⌈N/BN⌉ when not
 * causal; when causal, query block i visits only the key tiles up to its last
 * row, the tiles wholly above the diagonal being skipped ([15-779 L5] §6.2)
 * (T(T+1)/2 of T² for square tiles).
 * Host-only; returns -1 for invalid arguments. */
long long fa_fwd_tile_pairs(int N, int d, int causal);

/* Query-block and key-tile sizes fa_fwd uses for head dimension d (host-only);
 * returns FA_ERR_UNSUPPORTED for other d. */
fa_status fa_fwd_tile_shape(int d, int* block_m, int* block_n);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_str(int status);

/* ABI version of this header (bumped on incompatible changes; 2: fa_fwd_fp8
 * takes the packed buffer's size; 3: the softmax scale moved from fa_fwd_fp8 to
 * fa_quantize_fp8, which folds it into Q). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
