// Fused exact-attention forward for CDNA4 (gfx950).
//
// One workgroup owns one (b, h, query block of 128 rows); blocks are
// independent, so the grid runs over (b, h, query block) — the loop order
// with the query block outside and the key/value tiles inside ([cicada]
// §3.2.1–3.2.2; [15-779 L5] §5.1 and §6.3 "parallel over sequence length").
// Per key tile j the workgroup:
//   1. streams K_j, V_j from HBM into LDS (double-buffered: tile j+1 is in
//      flight in registers while tile j is computed),
//   2. computes Sᵀ = K_j Q_iᵀ on bf16 MFMA with fp32 accumulation,
//   3. masks keys after the query on tiles that cross the diagonal and keys
//      past N on the ragged last tile ([15-779 L5] §6.2),
//   4. updates the running max m, running sum ℓ and rescales the output
//      accumulator by exp(m_old − m_new) ([cicada] §3.2.2 steps B–D;
//      [15-779 L5] §4.3–4.5),
//   5. accumulates Oᵀ += V_jᵀ P̃ᵀ on bf16 MFMA,
// and after the last tile divides once by ℓ and writes O and
// L = m + ln ℓ ([cicada] §3.2.3).  Key tiles wholly above the diagonal are
// never visited ([15-779 L5] §6.2).
//
// Pages cited: [cicada] "已有的几种大模型上下文支持情况"; [15-779 L5] "第 5 讲 ·
// 案例：Transformer、注意力与 FlashAttention".
//
// Data layout on chip (per wavefront of 64 lanes, 32 query rows):
// * The products are taken transposed — Sᵀ = K Qᵀ and Oᵀ = Vᵀ P̃ᵀ — so that
//   with v_mfma_f32_32x32x16_bf16 each lane's accumulator column is one query
//   row: the row max and row sum are in-lane plus one exchange between the two
//   32-lane halves, the rescale factor is a per-lane scalar, and the fp32
//   scores of Sᵀ are already laid out as the B operand of the second product
//   (converted to bf16 in place, no LDS round trip).
// * K tile in LDS: row-major [key][d], 16-byte chunks XOR-swizzled by
//   (row & 7) so that MFMA operand reads and the staging writes hit distinct
//   banks.
// * V tile in LDS: transposed to [d][key] while staging (the reduction index
//   of Vᵀ P̃ᵀ is the key), stored in 4-key groups of 8 bytes whose group
//   index is XOR-swizzled by (d + d/16) & 15.
// * exp is computed as exp2 with scale·log2(e) folded into the logits.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int D>
struct Tile {
  static constexpr int BN = fwd_block_n(D);     // keys per tile
  static constexpr int CHUNKS = D / 8;          // 16-byte chunks per K/V row
  static constexpr int ROWS_PER_PASS = kFwdThreads / CHUNKS;
  static constexpr int K_PASSES = BN / ROWS_PER_PASS;  // 16-byte K loads per thread
  static constexpr int NSUB = BN / 32;          // 32-key sub-tiles of Sᵀ
  static constexpr int KS_QK = D / 16;          // MFMA k-steps of Sᵀ = K Qᵀ
  static constexpr int DSUB = D / 32;           // 32-row sub-tiles of Oᵀ
  static constexpr int KS_PV = BN / 16;         // MFMA k-steps of Oᵀ += Vᵀ P̃ᵀ
  static constexpr int K_BYTES = BN * D * 2;
  static constexpr int STAGE_BYTES = 2 * K_BYTES;  // K tile + Vᵀ tile
  static_assert(K_PASSES == 4, "staging assumes four 16-byte K loads per thread");
  static_assert(kFwdThreads / CHUNKS * 4 == BN, "staging assumes 4 V rows per thread");
};

__device__ inline float xor32(float x) { return __shfl_xor(x, 32); }

__device__ inline int k_off(int row, int chunk, int D) {
  return (row * D + ((chunk ^ (row & 7)) << 3)) * 2;  // bytes within the K tile
}

template <int BN>
__device__ inline int vt_off(int d, int grp) {
  return (d * BN + ((grp ^ ((d + (d >> 4)) & 15)) << 2)) * 2;  // bytes within the Vᵀ tile
}

template <int D>
__device__ inline void load_tile(const uint16_t* __restrict__ kbase, const uint16_t* __restrict__ vbase,
                                 int kv0, int N, int tid, u32x4_t (&kr)[4], u32x4_t (&vr)[4]) {
  using T = Tile<D>;
  const int c = tid % T::CHUNKS;
  const int r0 = tid / T::CHUNKS;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = kv0 + r0 + i * T::ROWS_PER_PASS;
    kr[i] = key < N ? *reinterpret_cast<const u32x4_t*>(kbase + (size_t)key * D + c * 8) : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int key = kv0 + 4 * r0 + i;
    vr[i] = key < N ? *reinterpret_cast<const u32x4_t*>(vbase + (size_t)key * D + c * 8) : u32x4_t{0, 0, 0, 0};
  }
}

template <int D>
__device__ inline void store_tile(unsigned char* stage, int tid, const u32x4_t (&kr)[4], const u32x4_t (&vr)[4]) {
  using T = Tile<D>;
  const int c = tid % T::CHUNKS;
  const int r0 = tid / T::CHUNKS;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = r0 + i * T::ROWS_PER_PASS;
    *reinterpret_cast<u32x4_t*>(stage + k_off(row, c, D)) = kr[i];
  }
  // Transpose 4 keys × 8 dims into 8 dims × 4 keys: for dim 8c+e the 8-byte
  // group holds (v[key0][e], v[key1][e], v[key2][e], v[key3][e]).
  unsigned char* vt = stage + T::K_BYTES;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1;
    uint32_t lo, hi;
    if (e & 1) {
      lo = (vr[0][w] >> 16) | (vr[1][w] & 0xffff0000u);
      hi = (vr[2][w] >> 16) | (vr[3][w] & 0xffff0000u);
    } else {
      lo = (vr[0][w] & 0xffffu) | (vr[1][w] << 16);
      hi = (vr[2][w] & 0xffffu) | (vr[3][w] << 16);
    }
    *reinterpret_cast<u32x2_t*>(vt + vt_off<T::BN>(8 * c + e, r0)) = u32x2_t{lo, hi};
  }
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Work index -> (bh, query block).  Workgroups are dealt round-robin to the
// 8 XCDs; with xcd_remap each XCD receives whole heads (so a head's K/V stays
// in one L2), and inside an XCD's share the heaviest query blocks (the last
// ones, for causal) are dispatched first (longest-processing-time-first,
// [15-779 L5] §6.2).
__device__ inline void decode_work(const FwdParams& p, int& bh, int& qb) {
  const int x = blockIdx.x;
  const int total = p.BH * p.n_qblk;
  if (p.xcd_remap) {
    const int per_xcd = total >> 3;
    const int heads_per_xcd = per_xcd / p.n_qblk;
    const int xcd = x & 7;
    const int local = x >> 3;
    bh = xcd * heads_per_xcd + local % heads_per_xcd;
    qb = p.n_qblk - 1 - local / heads_per_xcd;
  } else {
    bh = x % p.BH;
    qb = p.n_qblk - 1 - x / p.BH;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2) void fa_fwd_kernel(FwdParams p) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * T::STAGE_BYTES];

  int bh, qb;
  decode_work(p, bh, qb);
  const int N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i32 = lane & 31;  // query column of Sᵀ / Oᵀ owned by this lane
  const int g = lane >> 5;    // which 32-lane half
  const int q0 = qb * kFwdBlockM;
  const int wq0 = q0 + wave * 32;  // first query row of this wavefront
  const int q_row = wq0 + i32;
  const size_t base = (size_t)bh * N * D;
  const uint16_t* __restrict__ kbase = p.k + base;
  const uint16_t* __restrict__ vbase = p.v + base;

  // Q fragments: the B operand of Sᵀ = K Qᵀ (lane: query q_row, dims 16kk + 8g .. +7).
  bf16x8_t qf[T::KS_QK];
  {
    const u32x4_t* qp = reinterpret_cast<const u32x4_t*>(p.q + base + (size_t)q_row * D);
#pragma unroll
    for (int kk = 0; kk < T::KS_QK; ++kk) {
      const u32x4_t w = q_row < N ? qp[2 * kk + g] : u32x4_t{0, 0, 0, 0};
      qf[kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  const int n_tiles = fwd_kv_tiles(N, D, CAUSAL, qb);
  const float c = p.scale_log2;

  float m = -INFINITY;  // running max of the raw logits q·k (this lane's query row)
  float l = 0.f;        // running Σ exp2((s - m)·c) over this lane's half of the keys
  f32x16_t acc[T::DSUB];
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds) acc[ds] = f32x16_t{};

  u32x4_t kr[4], vr[4];
  load_tile<D>(kbase, vbase, 0, N, tid, kr, vr);
  store_tile<D>(smem, tid, kr, vr);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int kv0 = j * T::BN;
    const bool has_next = j + 1 < n_tiles;
    if (has_next) load_tile<D>(kbase, vbase, kv0 + T::BN, N, tid, kr, vr);

    unsigned char* st_k = smem + (j & 1) * T::STAGE_BYTES;
    unsigned char* st_v = st_k + T::K_BYTES;
    const bool active = !CAUSAL || kv0 <= wq0 + 31;  // else every key of the tile is after every row
    if (active) {
      // ---- Sᵀ = K Qᵀ -------------------------------------------------------
      f32x16_t s[T::NSUB];
#pragma unroll
      for (int st = 0; st < T::NSUB; ++st) {
        s[st] = f32x16_t{};
        const int row = st * 32 + i32;
#pragma unroll
        for (int kk = 0; kk < T::KS_QK; ++kk) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(st_k + k_off(row, 2 * kk + g, D));
          s[st] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qf[kk], s[st], 0, 0, 0);
        }
      }
      // ---- mask: keys after the query (diagonal tiles), keys past N (last tile)
      const bool need_mask = (kv0 + T::BN > N) || (CAUSAL && kv0 + T::BN - 1 > wq0);
      if (need_mask) {
        const int lim = CAUSAL ? min(q_row, N - 1) : N - 1;
#pragma unroll
        for (int st = 0; st < T::NSUB; ++st)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + st * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
            if (key > lim) s[st][r] = -INFINITY;
          }
      }
      // ---- online softmax -----------------------------------------------------
      float mt = -INFINITY;
#pragma unroll
      for (int st = 0; st < T::NSUB; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[st][r]);
      mt = fmaxf(mt, xor32(mt));
      // The first tile holds key 0, visible to every row, so m is finite from
      // then on and m_new never is -inf.
      const float m_new = fmaxf(m, mt);
      const float mc = m_new * c;
      const float alpha = __builtin_amdgcn_exp2f(m * c - mc);
      float rs = 0.f;
#pragma unroll
      for (int st = 0; st < T::NSUB; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(s[st][r], c, -mc));
          s[st][r] = e;
          rs += e;
        }
      l = l * alpha + rs;
      m = m_new;
#pragma unroll
      for (int ds = 0; ds < T::DSUB; ++ds) acc[ds] *= alpha;

      // ---- Oᵀ += Vᵀ P̃ᵀ ---------------------------------------------------------
#pragma unroll
      for (int kk = 0; kk < T::KS_PV; ++kk) {
        const f32x16_t& src = s[kk >> 1];
        const int h8 = (kk & 1) * 8;
        u32x4_t pw;
#pragma unroll
        for (int e = 0; e < 4; ++e) pw[e] = pack_bf16x2(src[h8 + 2 * e], src[h8 + 2 * e + 1]);
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
#pragma unroll
        for (int ds = 0; ds < T::DSUB; ++ds) {
          const int d = ds * 32 + i32;
          const u32x2_t a0 = *reinterpret_cast<const u32x2_t*>(st_v + vt_off<T::BN>(d, 4 * kk + g));
          const u32x2_t a1 = *reinterpret_cast<const u32x2_t*>(st_v + vt_off<T::BN>(d, 4 * kk + 2 + g));
          const u32x4_t a = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
          acc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), pb, acc[ds], 0, 0, 0);
        }
      }
    }

    if (has_next) store_tile<D>(smem + ((j + 1) & 1) * T::STAGE_BYTES, tid, kr, vr);
    __syncthreads();
  }

  // ---- epilogue: one division, one store of O and L ------------------------------
  l += xor32(l);
  if (q_row < N) {
    const float inv = 1.f / l;
    uint16_t* orow = p.o + base + (size_t)q_row * D;
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = ds * 32 + r4 * 8 + g * 4;
        u32x2_t w;
        w[0] = pack_bf16x2(acc[ds][4 * r4 + 0] * inv, acc[ds][4 * r4 + 1] * inv);
        w[1] = pack_bf16x2(acc[ds][4 * r4 + 2] * inv, acc[ds][4 * r4 + 3] * inv);
        *reinterpret_cast<u32x2_t*>(orow + d0) = w;
      }
    if (g == 0) p.lse[(size_t)bh * N + q_row] = m * p.scale + __builtin_amdgcn_logf(l) * 0.69314718055994531f;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  const dim3 grid(p.BH * p.n_qblk);
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL>), grid, dim3(kFwdThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, int causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
  return causal ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
}

}  // namespace fa
