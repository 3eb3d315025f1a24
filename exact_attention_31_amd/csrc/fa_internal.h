// Internal declarations shared by the C-ABI host code and the HIP kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace fa {

// Prefill tiling: a workgroup of 8 wavefronts owns 256 query rows (32 per
// wavefront, split-Q: every row's reductions stay inside one wavefront); key
// tiles hold 64 keys.
constexpr int kFwdWaves = 8;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kFwdBlockM = 32 * kFwdWaves;
// Compute units per XCD of the MI355X (256 CUs in 8 XCDs); it only steers the
// order in which workgroups are handed out, never a result.
constexpr int kCusPerXcd = 32;

__host__ __device__ constexpr int fwd_block_n(int) { return 64; }

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Number of key tiles query block `qb` visits.  Causal: only tiles whose first
// key is not after the block's last query row (tiles wholly above the
// diagonal are never loaded).
__host__ __device__ inline int fwd_kv_tiles(int N, int d, int causal, int qb) {
  const int kv_end = causal ? (N < (qb + 1) * kFwdBlockM ? N : (qb + 1) * kFwdBlockM) : N;
  return ceil_div(kv_end, fwd_block_n(d));
}

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int BH;
  int N;
  int n_qblk;
  int xcd_remap;     // 1: group each head's query blocks on one XCD
  float scale;       // softmax scale (for the LSE)
  float scale_log2;  // scale · log2(e): logits go straight into exp2
  const uint8_t* block_mask;  // null: dense; else [mask_heads, mask_tq, mask_tk] block mask
  int mask_heads;    // 1 (one mask for every head) or BH
  int mask_tq;       // ⌈N / kSparseBlock⌉ query blocks
  int mask_tk;       // ⌈N / kSparseBlock⌉ key blocks
};

// Block-sparse attention: mask blocks of kSparseBlock query rows × keys; at
// most kSparseMaxBlocks key blocks (N ≤ 131072).
constexpr int kSparseBlock = 128;
constexpr int kSparseMaxBlocks = 1024;

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* part_o;     // [B, Hq, S, d] fp32
  float* part_lse;   // [B, Hq, S]    fp32
  const int* seqlens;  // [B] keys per sequence, or null: all L
  int Hq;            // query heads
  int Hkv;           // key/value heads; query head h reads K/V head h / G
  int G;             // Hq / Hkv
  int L;             // key rows per (b, K/V head) in the cache
  int S;
  float scale;
  float scale_log2;
  const int* block_table;  // null: K/V contiguous per (b, K/V head); else [B, max_pages] page numbers
  int max_pages;     // entries per block-table row
  int page_shift;    // keys per page = 2^page_shift
  int num_pages;     // pages in the pool (entries are clamped into it)
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* ld;         // workspace [BH, N] pairs (L·log2 e, D = dO·O)
  float* dqacc;      // null: dQ by its own pass; else workspace fp32 [BH, N, d] for atomic adds
  const uint8_t* block_mask;  // null: dense; else [mask_heads, mask_t, mask_t] of kSparseBlock blocks
  int mask_heads;    // 1 or BH
  int mask_t;        // ceil(N / kSparseBlock)
  int BH;
  int N;
  int n_qblk;        // query blocks of kFwdBlockM rows (dQ kernel)
  int n_kblk;        // key blocks of kBwdBlockK keys (dK/dV kernel)
  int xcd_remap_q;   // 1: group each head's blocks on one XCD
  int xcd_remap_k;
  float scale;
  float scale_log2;
};

// dK/dV kernel: 4 wavefronts (one per SIMD) of 32 keys each.
constexpr int kBwdKvWaves = 4;
constexpr int kBwdKvThreads = 64 * kBwdKvWaves;
constexpr int kBwdBlockK = 32 * kBwdKvWaves;

// Query heads one decode workgroup serves: the largest of 8, 4, 2, 1 that
// divides the group size g = Hq / Hkv.
__host__ __device__ inline int decode_group_width(int g) { return g % 8 == 0 ? 8 : g % 4 == 0 ? 4 : g % 2 == 0 ? 2 : 1; }

// Static LDS beyond the default limit: let `kernel` use the CU's 160 KiB (once per
// instantiation; the static size is read back from the code object).
template <class K>
hipError_t allow_full_lds(K* kernel) {
  const void* fn = reinterpret_cast<const void*>(kernel);
  hipFuncAttributes attr;
  const hipError_t e = hipFuncGetAttributes(&attr, fn);
  if (e != hipSuccess) return e;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - (int)attr.sharedSizeBytes);
}

hipError_t launch_fwd(const FwdParams& p, int d, int causal, hipStream_t stream);
hipError_t launch_bwd(const BwdParams& p, int d, int causal, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int B, int d, hipStream_t stream);

// The allocation-free decode call's scratch: a file-scope device array of
// kDecodeScratchBytes (fa_decode.hip); decode_scratch gives its address on the
// current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace fa
