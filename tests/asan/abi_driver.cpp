// Drives every C-ABI entry point through its argument checks under
// AddressSanitizer and UndefinedBehaviorSanitizer (host code only): bad
// arguments must come back with their status, and a call that passes every
// check must reach the (stub) launcher and report FA_ERR_LAUNCH.  Exit status
// 0 when every expectation holds.
#include <stdint.h>
#include <stdio.h>

#include "fa.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(call, want)                                                            \
  do {                                                                                \
    const int got_ = (int)(call);                                                     \
    if (got_ != (int)(want)) {                                                        \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
              got_, (int)(want));                                                     \
      ++failures;                                                                     \
    }                                                                                 \
  } while (0)

int main() {
  // distinct, 16-byte aligned, far apart fake device addresses (never dereferenced)
  void* P[10];
  for (int i = 0; i < 10; ++i) P[i] = (void*)(uintptr_t)(0x100000000ull * (i + 1));
  void* mis = (void*)(uintptr_t)0x100000008ull;
  float* L = (float*)P[4];
  // prefill
  EXPECT(fa_fwd(nullptr, P[1], P[2], P[3], L, 1, 2, 300, 128, 0.1f, 1, nullptr), FA_ERR_NULL);
  EXPECT(fa_fwd(P[0], P[1], P[2], P[3], L, 0, 2, 300, 128, 0.1f, 1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P[0], P[1], P[2], P[3], L, 1, 2, 300, 96, 0.1f, 1, nullptr), FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(P[0], P[1], P[2], P[3], L, 1, 2, 300, 128, 0.f, 1, nullptr), FA_ERR_VALUE);
  EXPECT(fa_fwd(P[0], P[1], P[2], mis, L, 1, 2, 300, 128, 0.1f, 1, nullptr), FA_ERR_ALIGN);
  EXPECT(fa_fwd(P[0], P[1], P[2], P[0], L, 1, 2, 300, 128, 0.1f, 1, nullptr), FA_ERR_ALIAS);
  EXPECT(fa_fwd(P[0], P[1], P[2], P[3], L, 0x7fffffff, 0x7fffffff, 0x7fffffff, 128, 0.1f, 1, nullptr), FA_ERR_SHAPE);
  EXPECT(fa_fwd(P[0], P[1], P[2], P[3], L, 1, 2, 300, 128, 0.1f, 1, nullptr), FA_ERR_LAUNCH);
  EXPECT(fa_fwd_block_sparse(P[0], P[1], P[2], P[3], L, 1, 2, 300, 128, 0.1f, 0, nullptr, 1, nullptr), FA_ERR_NULL);
  EXPECT(fa_fwd_block_sparse(P[0], P[1], P[2], P[3], L, 1, 2, 300, 128, 0.1f, 0, (unsigned char*)P[5], 3, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_fwd_block_sparse(P[0], P[1], P[2], P[3], L, 1, 2, 300, 128, 0.1f, 0, (unsigned char*)P[5], 2, nullptr),
         FA_ERR_LAUNCH);
  // backward
  const size_t bws = fa_bwd_workspace_bytes(1, 2, 300);
  EXPECT(bws, (size_t)1 * 2 * 300 * 8);
  EXPECT(fa_bwd(P[0], P[1], P[2], P[3], P[4], (float*)P[5], P[6], P[7], P[8], 1, 2, 300, 128, 0.1f, 1, P[9], bws - 1,
                nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(P[0], P[1], P[2], P[3], P[4], (float*)P[5], P[6], P[6], P[8], 1, 2, 300, 128, 0.1f, 1, P[9], bws,
                nullptr), FA_ERR_ALIAS);
  EXPECT(fa_bwd(P[0], P[1], P[2], P[3], P[4], (float*)P[5], P[6], P[7], P[8], 1, 2, 300, 128, 0.1f, 1, P[9], bws,
                nullptr), FA_ERR_LAUNCH);
  const size_t aws = fa_bwd_atomic_workspace_bytes(1, 2, 300, 128);
  EXPECT(fa_bwd_atomic(P[0], P[1], P[2], P[3], P[4], (float*)P[5], P[6], P[7], P[8], 1, 2, 300, 128, 0.1f, 1, P[9],
                       aws, nullptr), FA_ERR_LAUNCH);
  EXPECT(fa_bwd_block_sparse(P[0], P[1], P[2], P[3], P[4], (float*)P[5], P[6], P[7], P[8], 1, 2, 300, 128, 0.1f, 1,
                             nullptr, 1, P[9], bws, nullptr), FA_ERR_NULL);
  // decode
  const size_t dws = fa_decode_workspace_bytes(2, 4, 128, 7);
  EXPECT(fa_decode(P[0], P[1], P[2], P[3], L, 2, 4, 1000, 128, 0.1f, 0, P[9], dws, nullptr), FA_ERR_VALUE);
  EXPECT(fa_decode(P[0], P[1], P[2], P[3], L, 2, 4, 1000, 128, 0.1f, 1001, P[9], dws, nullptr), FA_ERR_VALUE);
  EXPECT(fa_decode(P[0], P[1], P[2], P[3], L, 2, 4, 1000, 128, 0.1f, 7, P[9], dws - 4, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_decode(P[0], P[1], P[2], P[3], L, 2, 4, 1000, 128, 0.1f, 7, P[9], dws, nullptr), FA_ERR_LAUNCH);
  EXPECT(fa_decode_gqa(P[0], P[1], P[2], P[3], L, 2, 6, 4, 1000, 128, nullptr, 0.1f, 7, P[9], dws, nullptr),
         FA_ERR_SHAPE);
  EXPECT(fa_decode_gqa(P[0], P[1], P[2], P[3], L, 2, 8, 4, 1000, 128, (const int*)P[5], 0.1f, 7, P[9],
                       fa_decode_workspace_bytes(2, 8, 128, 7), nullptr), FA_ERR_LAUNCH);
  EXPECT(fa_decode_paged(P[0], P[1], P[2], P[3], L, 2, 8, 4, 128, 48, 64, (const int*)P[5], 20, nullptr, 0.1f, 7,
                         P[9], fa_decode_workspace_bytes(2, 8, 128, 7), nullptr), FA_ERR_SHAPE);  // page size not 2^k
  EXPECT(fa_decode_paged(P[0], P[1], P[2], P[3], L, 2, 8, 4, 128, 64, 64, (const int*)P[5], 20, nullptr, 0.1f, 7,
                         P[9], fa_decode_workspace_bytes(2, 8, 128, 7), nullptr), FA_ERR_LAUNCH);
  EXPECT(fa_decode_noalloc(P[0], P[1], P[2], P[3], L, 1, 512, 128, 128, 0.1f, 128, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_decode_noalloc(P[0], P[1], P[2], P[0], L, 2, 4, 1000, 128, 0.1f, 7, nullptr), FA_ERR_ALIAS);
  EXPECT(fa_decode_noalloc(P[0], P[1], P[2], P[3], L, 2, 4, 1000, 128, 0.1f, 7, nullptr), FA_ERR_LAUNCH);
  // FP8
  const size_t pk = fa_fp8_packed_bytes(1, 2, 300, 128);
  EXPECT(fa_quantize_fp8(P[0], P[1], P[2], 1, 2, 300, 128, 0.1f, P[3], pk - 1, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_quantize_fp8(P[0], P[1], P[2], 1, 2, 300, 128, 0.0f, P[3], pk, nullptr), FA_ERR_VALUE);
  EXPECT(fa_quantize_fp8(P[0], P[1], P[2], 1, 2, 300, 128, 0.1f, P[3], pk, nullptr), FA_ERR_LAUNCH);
  EXPECT(fa_fwd_fp8(P[3], pk - 1, P[4], (float*)P[5], 1, 2, 300, 128, 1, nullptr), FA_ERR_WORKSPACE);
  EXPECT(fa_fwd_fp8(P[3], pk, P[4], (float*)P[5], 1, 2, 300, 128, 1, nullptr), FA_ERR_LAUNCH);
  // host-only helpers
  int bm = 0, bn = 0;
  EXPECT(fa_fwd_tile_shape(128, &bm, &bn), FA_OK);
  EXPECT(fa_fwd_tile_shape(80, &bm, &bn), FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd_tile_pairs(4096, 128, 1) > 0, 1);
  EXPECT(fa_fwd_tile_pairs(0, 128, 1), -1);
  for (int s = -1; s < 12; ++s)
    if (!fa_status_str(s)) ++failures;
  const int launches = 10;
  if (g_launches != launches) {
    fprintf(stderr, "%d calls reached a launcher, expected %d\n", g_launches, launches);
    ++failures;
  }
  printf("%s: %d failures\n", failures ? "FAIL" : "ok", failures);
  return failures ? 1 : 0;
}
