// FP8 (E4M3) form of the prefill: the packed operand buffer that the
// quantising pass writes and the FP8 forward reads, and their launchers.
//
// Block-wise quantisation ([cicada] §4.4.1, FlashAttention-3): every run of
// kFp8Block rows of one (b, h) slice of Q, K and V has its own scale, a power
// of two 2^e with e the smallest integer that brings the block's largest
// magnitude to at most 448 (the largest E4M3 value), clamped to [−127, 127];
// it is stored as the E8M0 byte e + 127 that the matrix cores apply inside
// v_mfma_scale_f32_32x32x64_f8f6f4.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

constexpr int kFp8Block = 64;  // rows per quantisation block = keys per key tile
constexpr int kFp8D = 128;     // the FP8 forward's head dimension

// Byte offsets of the sections of the packed buffer (each 256-byte aligned),
// T = ⌈N / 64⌉ blocks per (b, h):
//   q8  [BH][N][d]      E4M3 codes of Q, rows as in Q
//   k8  [BH][N][d]      E4M3 codes of K
//   vt8 [BH][T][d][64]  E4M3 codes of V, one key tile at a time, transposed:
//                       row i of tile t holds dimension i of its 64 keys, in the
//                       order kFp8VtKey gives (keys past N are zero)
//   qs, ks, vs [BH][T]  int32 E8M0 scale bytes (e + 127) of each block
struct Fp8Layout {
  size_t q8, k8, vt8, qs, ks, vs, total;
};

__host__ __device__ inline size_t fp8_pad256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline Fp8Layout fp8_layout(int B, int H, int N, int d) {
  const size_t bh = (size_t)B * H, T = (size_t)((N + kFp8Block - 1) / kFp8Block);
  Fp8Layout L;
  L.q8 = 0;
  L.k8 = L.q8 + fp8_pad256(bh * N * d);
  L.vt8 = L.k8 + fp8_pad256(bh * N * d);
  L.qs = L.vt8 + fp8_pad256(bh * T * d * kFp8Block);
  L.ks = L.qs + fp8_pad256(bh * T * 4);
  L.vs = L.ks + fp8_pad256(bh * T * 4);
  L.total = L.vs + fp8_pad256(bh * T * 4);
  return L;
}

// Key of byte j (0..63) in a transposed V row of a tile.  The second product
// takes P̃ straight from the Sᵀ accumulators of the tile's two 32-key halves:
// lane half g holds, for key half b, the keys 32b + 8⌊r/4⌋ + 4g + r mod 4
// (r = 0..15), and the matrix core reads a lane's 32 operand bytes as
// reduction indices 32g .. 32g+31 of both operands.  Byte 32g + 16b + r of a
// transposed V row is therefore key 32b + 8⌊r/4⌋ + 4g + r mod 4.
__host__ __device__ inline int kFp8VtKey(int j) {
  const int g = j >> 5, b = (j >> 4) & 1, r = j & 15;
  return 32 * b + 8 * (r >> 2) + 4 * g + (r & 3);
}

struct Fp8QuantParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  unsigned char* packed;
  Fp8Layout L;
  int BH;
  int N;
  int T;
  float qmul;  // c = scale·log2(e): Q is quantised as c·Q
};

struct Fp8FwdParams {
  const unsigned char* packed;
  Fp8Layout L;
  uint16_t* o;
  float* lse;
  int BH;
  int N;
  int T;
  int n_qblk;
  int xcd_remap;
};

hipError_t launch_fp8_quantize(const Fp8QuantParams& p, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int causal, hipStream_t stream);

}  // namespace fa
