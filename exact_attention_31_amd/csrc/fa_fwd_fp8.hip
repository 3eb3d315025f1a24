// FP8 form of the fused attention forward, d = 128 ([cicada] §4.4.1,
// FlashAttention-3's block-wise quantisation), in two kernels:
//
// fa_fp8_quantize_kernel — one workgroup per (tensor, b·h, 64-row block) of Q,
//   K or V: the block's largest magnitude sets its power-of-two scale (see
//   fa_fp8.h), every element is divided by it and rounded to E4M3 (round to
//   nearest even), Q and K keep their row layout, and V is written one key
//   tile at a time transposed, in the key order the second product wants.
//
// fa_fwd_fp8_kernel — the bf16 prefill kernel's schedule (ping-pong of a
//   softmax phase and a matrix phase, K tiles streamed by wavefronts 0-3 and
//   Vᵀ tiles by 4-7, three tiles ahead) on FP8 operands.  Both products run on
//   v_mfma_scale_f32_32x32x64_f8f6f4, whose E8M0 operand scales apply the
//   block scales inside the product: Sᵀ = (s_k K₈)(s_q Q₈)ᵀ comes out as fp32
//   logits of the dequantised inputs, and Oᵀ += (s_v V₈ᵀ)(2^σ P̃₈)ᵀ.  P̃ is
//   computed in fp32 against a reference max that moves only when a row
//   outgrows it by 2^48 (conditional rescaling, [cicada] §5, as in the bf16
//   kernel), and is then block-quantised itself ([cicada] §4.4.1): each row's
//   32-key half of the tile — one scale block of the instruction — takes the
//   power of two 2^σ that brings its sum below 2^8, so its elements land
//   below E4M3's 448 with full precision, whatever the row's offset from the
//   reference max.  O is divided by the fp32 row sum ℓ of the unrounded P̃;
//   L = m + ln ℓ.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_fp8.h"
#include "fa_internal.h"

namespace fa {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float kFp8RescaleLog2 = 48.0f;          // P̃ ≤ 2^48 against the reference max
constexpr float kFp8SumBound = 281474976710656.0f;  // 2^48: a lane's sum at most this bounds its elements
constexpr int kE8M0One = 127;                     // E8M0 encoding of 1
constexpr int kPScaleLog2 = 8;                    // a scaled P̃ block sums to less than 2^8

// ---- quantisation ---------------------------------------------------------------

// The power-of-two exponent of a block with largest magnitude amax: the
// smallest e with amax ≤ 448·2^e, clamped to the E8M0 range; 0 for amax = 0.
__device__ inline int fp8_block_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);  // amax = f·2^E, f in [0.5, 1); 448 = 0.875·2^9
  int e = f <= 0.875f ? E - 9 : E - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__global__ __launch_bounds__(256) void fa_fp8_quantize_kernel(Fp8QuantParams p) {
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) unsigned char vl[kFp8Block * kFp8D];  // V block, E4M3, [key][d]
  const int tensor = blockIdx.y;  // 0 Q, 1 K, 2 V
  const int bh = blockIdx.x / p.T, t = blockIdx.x % p.T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = tid >> 2, c4 = tid & 3;  // row of the block, 32-element quarter of it
  const int row = t * kFp8Block + r;
  const uint16_t* src = tensor == 0 ? p.q : (tensor == 1 ? p.k : p.v);
  const size_t roff = ((size_t)bh * p.N + row) * kFp8D + 32 * c4;
  u32x4_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = row < p.N ? reinterpret_cast<const u32x4_t*>(src + roff)[i] : u32x4_t{0, 0, 0, 0};
  // Q is quantised as c·Q (c = scale·log2 e): the logits of the forward then come
  // out of the first product in base 2 (one fp32 rounding per element here)
  const float mul = tensor == 0 ? p.qmul : 1.f;
  float x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      x[8 * i + 2 * h] = __uint_as_float(w[i][h] << 16) * mul;
      x[8 * i + 2 * h + 1] = __uint_as_float(w[i][h] & 0xffff0000u) * mul;
    }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  if (lane == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int e = fp8_block_exponent(amax);
  uint32_t cw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a0 = __builtin_amdgcn_ldexpf(x[4 * i + 0], -e), a1 = __builtin_amdgcn_ldexpf(x[4 * i + 1], -e);
    const float a2 = __builtin_amdgcn_ldexpf(x[4 * i + 2], -e), a3 = __builtin_amdgcn_ldexpf(x[4 * i + 3], -e);
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, v, true);
    cw[i] = (uint32_t)v;
  }
  const size_t blk = (size_t)bh * p.T + t;
  if (tid == 0) {
    int* sc = reinterpret_cast<int*>(p.packed + (tensor == 0 ? p.L.qs : (tensor == 1 ? p.L.ks : p.L.vs)));
    sc[blk] = e + kE8M0One;
  }
  if (tensor < 2) {
    if (row < p.N) {
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(p.packed + (tensor == 0 ? p.L.q8 : p.L.k8) +
                                                ((size_t)bh * p.N + row) * kFp8D + 32 * c4);
      dst[0] = u32x4_t{cw[0], cw[1], cw[2], cw[3]};
      dst[1] = u32x4_t{cw[4], cw[5], cw[6], cw[7]};
    }
    return;
  }
  // V: through LDS into the transposed, key-permuted tile (rows past N are zeros)
  u32x4_t* vrow = reinterpret_cast<u32x4_t*>(vl + r * kFp8D + 32 * c4);
  vrow[0] = u32x4_t{cw[0], cw[1], cw[2], cw[3]};
  vrow[1] = u32x4_t{cw[4], cw[5], cw[6], cw[7]};
  __syncthreads();
  const int i = tid >> 1, h = tid & 1;  // dimension i, bytes 32h .. 32h+31 of its transposed row
  uint32_t ow[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= (uint32_t)vl[kFp8VtKey(32 * h + 4 * q + b) * kFp8D + i] << (8 * b);
    ow[q] = word;
  }
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(p.packed + p.L.vt8 + blk * (kFp8D * kFp8Block) + i * kFp8Block + 32 * h);
  dst[0] = u32x4_t{ow[0], ow[1], ow[2], ow[3]};
  dst[1] = u32x4_t{ow[4], ow[5], ow[6], ow[7]};
}

// ---- forward ---------------------------------------------------------------------

struct Fp8Tile {
  static constexpr int BN = kFp8Block;         // keys per tile
  static constexpr int KROW = kFp8D;           // bytes per K row
  static constexpr int VROW = kFp8Block;       // bytes per transposed V row
  static constexpr int TILE_BYTES = BN * KROW; // = kFp8D * VROW
  static constexpr int NSUB = BN / 32;         // 32-key sub-tiles of Sᵀ
  static constexpr int KB = kFp8D / 64;        // 64-deep k-blocks of Sᵀ = K Qᵀ
  static constexpr int DSUB = kFp8D / 32;      // 32-row sub-tiles of Oᵀ
  static_assert(TILE_BYTES == 2 * (kFwdWaves / 2) * 1024, "two 1 KiB loads per wavefront of a group fill a tile");
  // XOR swizzles of the 16-byte chunk index: rows of one 8-lane read group hit distinct banks
  __device__ static int k_swz(int r) { return (r >> 1) & 7; }
  __device__ static int v_swz(int r) { return (r >> 2) & 3; }
};

__device__ inline void fp8_decode_work(const Fp8FwdParams& p, int& bh, int& qb) {
  const int x = blockIdx.x;
  const int total = p.BH * p.n_qblk;
  if (p.xcd_remap) {
    const int heads_per_xcd = (total >> 3) / p.n_qblk;
    const int xcd = x & 7, local = x >> 3;
    bh = xcd * heads_per_xcd + local % heads_per_xcd;
    qb = p.n_qblk - 1 - local / heads_per_xcd;
  } else {
    bh = x % p.BH;
    qb = p.n_qblk - 1 - x / p.BH;
  }
}

template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kFwdThreads), amdgpu_waves_per_eu(2)))
void fa_fwd_fp8_kernel(Fp8FwdParams p, const int* __restrict__ ks_all, const int* __restrict__ vs_all) {
  using T = Fp8Tile;
  constexpr int SROW = 2 * kFp8D + 16;  // staging row stride of the bf16 output (bytes)
  // One LDS array with the eight tile buffers first: every tile read then has
  // an address below 64 KiB and takes it as the instruction's immediate offset
  // (placed after the output staging, half of them needed an address add a read).
  __shared__ __attribute__((aligned(16))) unsigned char lds_all[8 * T::TILE_BYTES + kFwdWaves * 32 * SROW];
  unsigned char* const kbufs[4] = {lds_all, lds_all + T::TILE_BYTES, lds_all + 2 * T::TILE_BYTES, lds_all + 3 * T::TILE_BYTES};
  unsigned char* const vbufs[4] = {lds_all + 4 * T::TILE_BYTES, lds_all + 5 * T::TILE_BYTES, lds_all + 6 * T::TILE_BYTES,
                                   lds_all + 7 * T::TILE_BYTES};
  unsigned char* const stg_all = lds_all + 8 * T::TILE_BYTES;

  int bh, qb;
  fp8_decode_work(p, bh, qb);
  const int N = p.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, g = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int q0 = qb * kFwdBlockM;
  const int wq0 = q0 + wave_u * 32;
  const int q_row = wq0 + i32;
  const int grp = wave_u >> 2;
  const int n_tiles = fwd_kv_tiles(N, kFp8D, CAUSAL, qb);

  const unsigned char* const q8 = p.packed + p.L.q8 + (size_t)bh * N * kFp8D;
  const unsigned char* const k8 = p.packed + p.L.k8 + (size_t)bh * N * kFp8D;
  const unsigned char* const vt8 = p.packed + p.L.vt8 + (size_t)bh * p.T * T::TILE_BYTES;
  // The K and V block scales come in as their own read-only kernel arguments, so
  // that their uniform reads become scalar loads: vector loads here would count
  // against the tile loads' vmcnt bookkeeping and make each wait cover a tile more.
  const int* const ksc = ks_all + (size_t)bh * p.T;
  const int* const vsc = vs_all + (size_t)bh * p.T;
  const int qse = __builtin_amdgcn_readfirstlane(
      reinterpret_cast<const int*>(p.packed + p.L.qs)[(size_t)bh * p.T + min(wq0, N - 1) / kFp8Block]);

  // Direct loads: wavefront u of a group, load i, lane L fills 16-byte slot
  // s = (4i + u)·64 + L of the tile.  K (128-byte rows, 8 chunks): row s/8,
  // chunk s%8; Vᵀ (64-byte rows, 4 chunks): row s/4, chunk s%4.  Load i is
  // load 0 moved by 4096 bytes of the global tile in both cases (32 K rows,
  // 64 Vᵀ rows), and the swizzles repeat within that.
  const int u = wave & 3;
  const int rk = (u * 64 + lane) >> 3, ck = lane & 7;
  const int rv = (u * 64 + lane) >> 2, cv = lane & 3;
  const int k_goff = rk * T::KROW + ((ck ^ T::k_swz(rk)) << 4);
  const int v_goff = rv * T::VROW + ((cv ^ T::v_swz(rv)) << 4);
  const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(k8, N * T::KROW);
  const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(vt8, p.T * T::TILE_BYTES);

  // Operand reads (bytes within a tile): K rows i32 (+32 per sub-tile), the two
  // chunks 4kb + 2g, +1; Vᵀ rows i32 (+32 per d sub-tile), chunks 2g, 2g + 1.
  int k_rd[T::KB][2], v_rd[2];
#pragma unroll
  for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h) k_rd[kb][h] = i32 * T::KROW + (((4 * kb + 2 * g + h) ^ T::k_swz(i32)) << 4);
#pragma unroll
  for (int h = 0; h < 2; ++h) v_rd[h] = i32 * T::VROW + (((2 * g + h) ^ T::v_swz(i32)) << 4);

  // Q: B operand of Sᵀ = K Qᵀ, lane: row q_row, bytes 64kb + 32g .. +31.
  i32x8_t qf[T::KB];
#pragma unroll
  for (int kb = 0; kb < T::KB; ++kb) {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(q8 + (size_t)q_row * kFp8D + 64 * kb + 32 * g);
    const u32x4_t a = q_row < N ? qp[0] : u32x4_t{0, 0, 0, 0};
    const u32x4_t b = q_row < N ? qp[1] : u32x4_t{0, 0, 0, 0};
    qf[kb] = __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  auto active = [&](int j) __attribute__((always_inline)) { return !CAUSAL || j * T::BN <= wq0 + 31; };
  auto kscale = [&](int j) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(ksc[j]); };
  auto vscale = [&](int j) __attribute__((always_inline)) { return __builtin_amdgcn_readfirstlane(vsc[j]); };

  // m: the reference max of this lane's row, base 2.  The first logit instruction
  // of a tile starts from −mo (its accumulator input), mo the reference max when
  // the tile's products are issued (0 while m is −∞): the logits come out as
  // t − mo, so while m = mo, P̃ = 2^(t − m) is one exp2 of them.
  float m = -INFINITY, l = 0.f, mo = 0.f;
  f32x16_t moff = {};  // −mo in every element
  f32x16_t acc[T::DSUB];
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds) acc[ds] = f32x16_t{};
  f32x16_t s[T::NSUB];
  i32x8_t pb;      // 2^-σ P̃ of the tile in E4M3, the B operand of the second product
  int psc = kE8M0One;  // E8M0 scale 127 + σ of this lane's block of pb (see below)
  float pe[T::NSUB][16], rsub[T::NSUB];  // P̃ of the tile in fp32 and the lane's sums per sub-tile

  auto softmax = [&](int j, auto clean) __attribute__((always_inline)) {
    const int kv0 = j * T::BN;
    if (!decltype(clean)::value && ((kv0 + T::BN > N) || (CAUSAL && kv0 + T::BN - 1 > wq0))) {
      const int lim = CAUSAL ? min(q_row, N - 1) : N - 1;
#pragma unroll
      for (int sub = 0; sub < T::NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + sub * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key > lim) s[sub][r] = -INFINITY;
        }
    }
    // P̃ = 2^(s + off) in fp32 (off = 0 while m = mo), and the lane's sum over
    // each 32-key sub-tile (the E4M3 conversion follows in the matrix phase,
    // `convert`).  The lane's sum bounds each of its elements, so a sum at most
    // 2^48 proves that no row outgrew m by more.
    float rs;
    auto exps = [&](auto with_off, float off) __attribute__((always_inline)) {
#pragma unroll
      for (int sub = 0; sub < T::NSUB; ++sub) {
        float r2[2];
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            pe[sub][r + t] = __builtin_amdgcn_exp2f(decltype(with_off)::value ? s[sub][r + t] + off : s[sub][r + t]);
          const float q4 = (pe[sub][r] + pe[sub][r + 1]) + (pe[sub][r + 2] + pe[sub][r + 3]);
          r2[(r >> 2) & 1] = r < 8 ? q4 : r2[(r >> 2) & 1] + q4;
        }
        rsub[sub] = r2[0] + r2[1];
      }
      rs = rsub[0] + rsub[1];
    };
    exps(std::false_type{}, 0.f);
    if (__any(!(rs <= kFp8SumBound) || m == -INFINITY)) {  // also taken for inf / NaN sums and the first tile
      float mx[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) mx[t] = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < T::NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx[r & 3] = fmaxf(mx[r & 3], s[sub][r]);
      const float mt = pair_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]))) + mo;  // the tile's row max, base 2
      if (__any(mt - m > kFp8RescaleLog2)) {
        const float m_new = fmaxf(m, mt);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 while m = −∞ (ℓ and acc are 0 then)
        l *= alpha;
#pragma unroll
        for (int ds = 0; ds < T::DSUB; ++ds) acc[ds] *= alpha;
        m = m_new;
        exps(std::true_type{}, mo - m);
        mo = m;  // the next tiles start from the new max
#pragma unroll
        for (int e = 0; e < 16; ++e) moff[e] = -m;
      }
    }
    l += rs;
  };

  auto kop = [&](const unsigned char* kb, int i) __attribute__((always_inline)) {  // i = sub·KB + kb
    const int sub = i / T::KB, kbk = i % T::KB;
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(kb + k_rd[kbk][0] + sub * 32 * T::KROW);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(kb + k_rd[kbk][1] + sub * 32 * T::KROW);
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto vop = [&](const unsigned char* vb, int ds) __attribute__((always_inline)) {
    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(vb + v_rd[0] + ds * 32 * T::VROW);
    const u32x4_t b = *reinterpret_cast<const u32x4_t*>(vb + v_rd[1] + ds * 32 * T::VROW);
    return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto qk_step = [&](const unsigned char* kb, int i, int kse) __attribute__((always_inline)) {
    const int sub = i / T::KB, kbk = i % T::KB;
    s[sub] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop(kb, i), qf[kbk], kbk == 0 ? moff : s[sub], 0, 0, 0, kse,
                                                             0, qse);
  };
  auto pv_step = [&](const unsigned char* vb, int ds, int vse) __attribute__((always_inline)) {
    acc[ds] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop(vb, ds), pb, acc[ds], 0, 0, 0, vse, 0, psc);
  };
  // P̃ of the tile into the E4M3 B operand, a quarter (two words) per call, so
  // that the matrix phase can issue it between the MFMAs of the first product.
  // Sub-tile `sub` of a row is one scale block of the second product (bytes
  // 16·sub .. 16·sub + 15 of the row's two lanes; the lane of the lower half
  // gives the scale of block 0, the upper one that of block 1): both lanes form
  // the block's sum R alike (R = r_lo + r_hi) and take σ = frexp exponent of
  // R − 8, so every element, at most R < 2^(σ+8), scales below 2^8; σ stays at
  // least −126 so that 2^σ is a normal fp32 number and 127 + σ a valid E8M0 code.
  int sig[T::NSUB];
  auto convert = [&](int part) __attribute__((always_inline)) {  // part 0..3: words 2·part, 2·part + 1
    const int sub = part >> 1;
    if ((part & 1) == 0) sig[sub] = max(__builtin_amdgcn_frexp_expf(pair_sum(rsub[sub])) - kPScaleLog2, -126);
    const float sc = __uint_as_float((uint32_t)(sig[sub] + 127) << 23);  // 2^σ
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int w4 = 2 * (part & 1) + h;
      // the two conversions fill the low and the high half of the word; the
      // first is declared as writing the whole register, so that no value is
      // prepared for the half it keeps (the second overwrites that half)
      int w;
      asm("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %3" : "=v"(w) : "v"(pe[sub][4 * w4]), "v"(pe[sub][4 * w4 + 1]), "v"(sc));
      asm("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]"
          : "+v"(w) : "v"(pe[sub][4 * w4 + 2]), "v"(pe[sub][4 * w4 + 3]), "v"(sc));
      pb[4 * sub + w4] = w;
    }
    if (part == 3) psc = kE8M0One + (g ? sig[1] : sig[0]);
  };
  constexpr int NQK = T::NSUB * T::KB;
  constexpr int NPV = T::DSUB;
  static_assert(NQK == NPV, "interleave pairs one MFMA of each product");
  // matrix phase X(j): Sᵀ_{j+1} = K_{j+1} Qᵀ (if do_qk) with P̃_j's conversion issued
  // between its MFMAs, then Oᵀ += Vᵀ_j P̃ᵀ_j (if do_pv)
  auto matrix = [&](const unsigned char* vb, const unsigned char* kb, bool do_pv, bool do_qk, int vse, int kse)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      if (do_qk) qk_step(kb, i, kse);
      if (do_pv) convert(i);
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i)
      if (do_pv) pv_step(vb, i, vse);
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- pipeline: the bf16 kernel's (see fa_fwd.hip) --------------------------------
  auto kbf = [&](int j) { return kbufs[j & 3]; };
  auto vbf = [&](int j) { return vbufs[j & 3]; };
  const __amdgpu_buffer_rsrc_t mrsrc = grp ? vrsrc : krsrc;
  const int m_goff = grp ? v_goff : k_goff;
  const int past_end = grp ? p.T * T::TILE_BYTES : N * T::KROW;  // reads there return zeros
  auto load_tile = [&](int t, unsigned char* dst) __attribute__((always_inline)) {
    const int off = (t >= 0 && t < n_tiles) ? t * T::TILE_BYTES : past_end;
    unsigned char* d = dst + u * 1024;
#pragma unroll
    for (int i = 0; i < 2; ++i) load_lds16(mrsrc, d + i * (kFwdWaves / 2) * 1024, m_goff + off + i * 4096);
  };
#pragma unroll
  for (int t = 0; t < 3; ++t) load_tile(t, grp ? vbufs[t] : kbufs[t]);
  wait_vmcnt<4>();  // tile 0 has landed
#pragma unroll
  for (int kb = 0; kb < T::KB; ++kb) asm volatile("" ::"v"(qf[kb]));
  block_barrier();
  if (grp == 1) block_barrier();
  if (active(0)) matrix(vbf(0), kbf(0), false, true, kE8M0One, kscale(0));
  wait_vmcnt<2>();  // tile 1
  block_barrier();

  auto iter = [&](int j, auto phase, auto clean) __attribute__((always_inline)) {
    constexpr int P = decltype(phase)::value;
    constexpr bool CLEAN = decltype(clean)::value;
    load_tile(j + 3, grp ? vbufs[(P + 3) & 3] : kbufs[(P + 3) & 3]);
    const bool qk_next = j + 1 < n_tiles && active(j + 1);
    const int kse = kscale(qk_next ? j + 1 : 0), vse = vscale(j);
    if (CLEAN)
      softmax(j, std::true_type{});
    else if (active(j))
      softmax(j, std::false_type{});
    wait_vmcnt<4>();  // tile j+1
    block_barrier();
    if (CLEAN)
      matrix(vbf(P), kbf(P + 1), true, true, vse, kse);
    else
      matrix(vbf(P), kbf(P + 1), active(j), qk_next, vse, kse);
    block_barrier();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using Y = std::true_type;
  using G = std::false_type;
  // iteration j is clean when tile j is whole for every row and a tile j+1
  // exists (every wavefront then sees that tile)
  const int n_clean = CAUSAL ? min(N / T::BN, (q0 + 1) / T::BN) : N / T::BN;
  const int n_clean_it = min(n_clean, n_tiles - 1);
  int j = 0;
  for (; j + 4 <= n_clean_it; j += 4) {
    iter(j, I0{}, Y{});
    iter(j + 1, I1{}, Y{});
    iter(j + 2, I2{}, Y{});
    iter(j + 3, I3{}, Y{});
  }
  for (; j < n_tiles; j += 4) {
    iter(j, I0{}, G{});
    if (j + 1 < n_tiles) iter(j + 1, I1{}, G{});
    if (j + 2 < n_tiles) iter(j + 2, I2{}, G{});
    if (j + 3 < n_tiles) iter(j + 3, I3{}, G{});
  }
  if (grp == 0) block_barrier();

  // ---- epilogue: O = acc / ℓ in bf16, staged in LDS and stored as whole rows ------
  wait_vmcnt<0>();
  block_barrier();
  l = pair_sum(l);
  const float inv = 1.f / l;
  unsigned char* const stg = stg_all + wave_u * 32 * SROW;
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = ds * 32 + r4 * 8 + g * 4;
      u32x2_t w;
      w[0] = pack_bf16x2(acc[ds][4 * r4 + 0] * inv, acc[ds][4 * r4 + 1] * inv);
      w[1] = pack_bf16x2(acc[ds][4 * r4 + 2] * inv, acc[ds][4 * r4 + 3] * inv);
      *reinterpret_cast<u32x2_t*>(stg + i32 * SROW + 2 * d0) = w;
    }
  constexpr int CH = 2 * kFp8D / 16;  // 16-byte chunks per bf16 output row
  constexpr int RPI = 64 / CH;        // rows per store instruction
  const int rr0 = lane / CH, cc = lane % CH;
  u32x4_t ow[32 / RPI];
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) ow[it] = *reinterpret_cast<const u32x4_t*>(stg + (it * RPI + rr0) * SROW + cc * 16);
  const size_t obase = (size_t)bh * N * kFp8D;
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it)
    if (wq0 + it * RPI + rr0 < N)
      *reinterpret_cast<u32x4_t*>(p.o + obase + (size_t)(wq0 + it * RPI + rr0) * kFp8D + cc * 8) = ow[it];
  if (q_row < N && g == 0) p.lse[(size_t)bh * N + q_row] = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
}

template <bool CAUSAL>
hipError_t launch_fwd_fp8_t(const Fp8FwdParams& p, hipStream_t stream) {
  static const hipError_t attr = allow_full_lds(&fa_fwd_fp8_kernel<CAUSAL>);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((fa_fwd_fp8_kernel<CAUSAL>), dim3(p.BH * p.n_qblk), dim3(kFwdThreads), 0, stream, p,
                     reinterpret_cast<const int*>(p.packed + p.L.ks), reinterpret_cast<const int*>(p.packed + p.L.vs));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8QuantParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(fa_fp8_quantize_kernel, dim3(p.BH * p.T, 3), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int causal, hipStream_t stream) {
  return causal ? launch_fwd_fp8_t<true>(p, stream) : launch_fwd_fp8_t<false>(p, stream);
}

}  // namespace fa
