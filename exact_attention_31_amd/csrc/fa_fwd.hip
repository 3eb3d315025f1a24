// Fused exact-attention forward for CDNA4 (gfx950).
//
// One workgroup of 8 wavefronts owns one (b, h, query block of 256 rows);
// blocks are independent, so the grid runs over (b, h, query block) — the
// loop order with the query block outside and the key/value tiles inside
// ([cicada] §3.2.1–3.2.2; [15-779 L5] §5.1 and §6.3 "parallel over sequence
// length").  Each wavefront owns 32 of the rows (split-Q, [15-779 L5] §6.4),
// so every row's max and sums stay inside one wavefront.  Per key tile j of
// 64 keys the workgroup:
//   1. streams K_j, V_j from HBM into LDS: four buffers per tensor, filled by
//      buffer loads that write LDS directly, each issued three iterations
//      before the one that reads it,
//   2. computes Sᵀ = K_j Q_iᵀ on bf16 MFMA with fp32 accumulation,
//   3. masks keys after the query on tiles that cross the diagonal and keys
//      past N on the ragged last tile ([15-779 L5] §6.2),
//   4. keeps the running max m, the running sums ℓ and the output accumulator
//      consistent with each other — when m grows, ℓ and the accumulator are
//      multiplied by exp(m_old − m_new) ([cicada] §3.2.2 steps B–D;
//      [15-779 L5] §4.3–4.5),
//   5. accumulates Oᵀ += V_jᵀ P̃ᵀ on bf16 MFMA,
// and after the last tile divides once by ℓ and writes O and
// L = m + ln ℓ ([cicada] §3.2.3).  Key tiles wholly above the diagonal are
// never visited ([15-779 L5] §6.2).
//
// The reference max m is only moved when some row of the wavefront sees a
// logit more than kRescaleLog2 (in log2 units) above it; otherwise the stale m
// is kept for exponent and sums alike, which changes nothing in exact
// arithmetic (m cancels between ℓ and the accumulator) and bounds every P̃
// by 2^kRescaleLog2.  This is the conditional rescaling of [cicada] §5
// (FlashAttention-4); it removes the accumulator multiply from almost every
// tile.
//
// Pages cited: [cicada] "已有的几种大模型上下文支持情况"; [15-779 L5] "第 5 讲 ·
// 案例：Transformer、注意力与 FlashAttention".
//
// Layout on chip (one wavefront = 64 lanes, 32 query rows; two wavefronts per SIMD):
// * The products are taken transposed — Sᵀ = K Qᵀ and Oᵀ = Vᵀ P̃ᵀ — so that
//   with v_mfma_f32_32x32x16_bf16 each lane's accumulator column is one query
//   row: the row max and row sums are in-lane plus one exchange between the
//   two 32-lane halves (v_permlane32_swap), the rescale factor is a per-lane
//   scalar, and the fp32 scores of Sᵀ are already laid out as the B operand of
//   the second product (converted to bf16 in place, no LDS round trip).
// * K tile in LDS: row-major [key][d] in 16-byte chunks, the chunk index
//   XOR-ed with a function of the row so that the operand reads (16 rows ×
//   one chunk per pass) hit distinct banks; the direct loads write whole
//   1 KiB runs, each lane fetching the global chunk that belongs in its slot.
// * V tile in LDS: row-major [key][d], chunk index XOR-ed likewise; the Vᵀ
//   operand, whose reduction index is the key, is read with the LDS transpose
//   load ds_read_b64_tr_b16, four keys per 16-lane group.
// * The eight tile buffers are separate LDS objects, so the compiler can tell
//   that a direct load into one buffer never aliases reads of another and
//   lets those reads run while the loads are in flight.
// * Software pipeline: while the vector unit turns the scores of tile j into
//   probabilities, the matrix unit already computes the scores of tile j+1;
//   the row max of tile j+1 is taken while Oᵀ += Vᵀ_j P̃ᵀ_j runs.
// * exp is computed as exp2 with scale·log2(e) folded into the logits.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// log2-domain growth of the running max that forces a rescale.
constexpr float kRescaleLog2 = 8.0f;
constexpr int kStages = 4;  // LDS buffers per tensor (the loop is unrolled by this)

template <int D>
struct Tile {
  static constexpr int BN = fwd_block_n(D);       // keys per tile
  static constexpr int CH = D / 8;                // 16-byte chunks per K/V row
  static constexpr int ROW = 2 * D;               // bytes per K/V row in LDS (unpadded)
  static constexpr int TILE_BYTES = BN * ROW;     // one K or V tile
  static constexpr int LOADS = TILE_BYTES / (16 * kFwdThreads);  // 16-byte direct loads per thread per tile
  static constexpr int LDS_BYTES = 2 * kStages * TILE_BYTES;
  static constexpr int NSUB = BN / 32;            // 32-key sub-tiles of Sᵀ
  static constexpr int KS_QK = D / 16;            // MFMA k-steps of Sᵀ = K Qᵀ
  static constexpr int DSUB = D / 32;             // 32-row sub-tiles of Oᵀ
  static constexpr int KS_PV = BN / 16;           // MFMA k-steps of Oᵀ += Vᵀ P̃ᵀ
  static_assert(LOADS * 16 * kFwdThreads == TILE_BYTES, "direct loads cover the tile");
  // XOR swizzles of the 16-byte chunk index within a row (see the file header).
  __device__ static int k_swz(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static int v_swz(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

// Both halves of the wavefront end up with f(x_lo, x_hi) for the lane pair (l, l^32).
__device__ inline float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ inline u32x2_t lds_tr_read(const unsigned char* base, int off) {
  const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(base + off));
  return __builtin_bit_cast(u32x2_t, v);
}

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ... lds):
// lane L's bytes [voff + soff, +16) land at lds + 16·L (lds uniform across the
// wavefront); bytes past the buffer's num_records read as zero.  Kept in a
// non-template function: used directly inside the kernel template, the
// builtin makes the host pass drop the kernel's launch stub.
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Raw buffer descriptor over `bytes` bytes at `base` (word 3: 32-bit data, no swizzle).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// s_waitcnt that waits until at most n vector-memory loads are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at max).
template <int n>
__device__ inline void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
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
__global__ __launch_bounds__(kFwdThreads, 1) void fa_fwd_kernel(FwdParams p) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[T::TILE_BYTES], k_lds1[T::TILE_BYTES],
      k_lds2[T::TILE_BYTES], k_lds3[T::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[T::TILE_BYTES], v_lds1[T::TILE_BYTES],
      v_lds2[T::TILE_BYTES], v_lds3[T::TILE_BYTES];
  unsigned char* const kbufs[4] = {k_lds0, k_lds1, k_lds2, k_lds3};
  unsigned char* const vbufs[4] = {v_lds0, v_lds1, v_lds2, v_lds3};

  int bh, qb;
  decode_work(p, bh, qb);
  const int N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i32 = lane & 31;  // query column of Sᵀ / Oᵀ owned by this lane
  const int g = lane >> 5;    // which 32-lane half
  const int jj = lane & 15;
  const int q0 = qb * kFwdBlockM;
  const int wq0 = q0 + wave * 32;  // first query row of this wavefront
  const int q_row = wq0 + i32;
  const size_t base = (size_t)bh * N * D;

  // Direct global->LDS loads: wavefront `wave`, load i fills LDS chunk slots
  // (i*4 + wave)*64 + lane of the tile; the slot's (row, swizzled chunk) names
  // the global chunk this lane fetches.  Load i covers rows r0 + i*RPL, and
  // both swizzles repeat with that period, so load i is load 0 shifted by
  // i*RPL rows.
  constexpr int RPL = kFwdWaves * 64 / T::CH;  // rows covered by one load across the workgroup
  const int r0 = (wave * 64 + lane) / T::CH;
  const int cpos = lane % T::CH;
  const int k_goff = r0 * T::ROW + ((cpos ^ T::k_swz(r0)) << 4);
  const int v_goff = r0 * T::ROW + ((cpos ^ T::v_swz(r0)) << 4);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave index in a scalar register
  // rows past N lie past the head's bytes and read as zero (their logits are masked)
  const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(p.k + base, N * T::ROW);
  const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.v + base, N * T::ROW);
  auto load_tile = [&](__amdgpu_buffer_rsrc_t rsrc, int goff, int kv0, unsigned char* dst) {
    unsigned char* d = dst + wave_u * 1024;
#pragma unroll
    for (int i = 0; i < T::LOADS; ++i) load_lds16(rsrc, d + i * kFwdWaves * 1024, goff, (kv0 + i * RPL) * T::ROW);
  };

  // Operand-read lane offsets (bytes within a tile).
  int k_rd[T::KS_QK];  // Kᵀ rows i32 (+32 per sub-tile), chunk 2kk + g
#pragma unroll
  for (int kk = 0; kk < T::KS_QK; ++kk) k_rd[kk] = i32 * T::ROW + (((2 * kk + g) ^ T::k_swz(i32)) << 4);
  int v_rd[T::DSUB];   // transpose reads: rows 4g + jj/4 (+16kk, +8), dims 32ds + 16(G&1) + 4(jj&3)
  {
    const int r = 4 * g + (jj >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1);
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds)
      v_rd[ds] = r * T::ROW + (((4 * ds + cl) ^ T::v_swz(r)) << 4) + 8 * (jj & 1);
  }

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
  auto active = [&](int j) { return !CAUSAL || j * T::BN <= wq0 + 31; };  // some row of the wave sees the tile

  float m = -INFINITY;  // reference max of the raw logits q·k (this lane's query row)
  // Two running sums over this lane's half of the keys: ℓ of the fp32 P̃ (for
  // L: rows with few keys need it within 1e-3) and ℓ_b of the bf16-rounded P̃
  // that enter the MFMA (for O: numerator and denominator then use the same
  // weights, so a row dominated by one key returns that key's value exactly).
  float l = 0.f, lb = 0.f;
  f32x16_t acc[T::DSUB];
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds) acc[ds] = f32x16_t{};

  // ---- Sᵀ = K Qᵀ for one tile (the two 32-key sub-tiles interleaved) ----------------
  auto qk = [&](const unsigned char* kb, f32x16_t (&s)[T::NSUB]) {
#pragma unroll
    for (int sub = 0; sub < T::NSUB; ++sub) s[sub] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < T::KS_QK; ++kk)
#pragma unroll
      for (int sub = 0; sub < T::NSUB; ++sub) {
        const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kb + k_rd[kk] + sub * 32 * T::ROW);
        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf), qf[kk], s[sub], 0, 0, 0);
      }
  };

  // ---- mask of one tile's scores: keys after the query (diagonal tiles), keys
  //      past N (last tile); only tiles at the end of the key range need it
  auto mask = [&](int j, f32x16_t (&s)[T::NSUB]) {
    const int kv0 = j * T::BN;
    if ((kv0 + T::BN > N) || (CAUSAL && kv0 + T::BN - 1 > wq0)) {
      const int lim = CAUSAL ? min(q_row, N - 1) : N - 1;
#pragma unroll
      for (int sub = 0; sub < T::NSUB; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + sub * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key > lim) s[sub][r] = -INFINITY;
        }
    }
  };
  // ---- row max of one tile's scores ------------------------------------------------------
  auto rowmax = [&](const f32x16_t (&s)[T::NSUB]) {
    float mt = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < T::NSUB; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[sub][r]);
    return pair_max(mt);
  };
  // ---- move the reference max when some row outgrew it by 2^kRescaleLog2 ----------------
  auto rescale = [&](float mt) {
    // The first tile holds key 0, visible to every row: m is finite after it.
    if (__any((mt - m) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
      l *= alpha;
      lb *= alpha;
#pragma unroll
      for (int ds = 0; ds < T::DSUB; ++ds) acc[ds] *= alpha;
      m = m_new;
    }
  };

  // ---- P̃ = exp2(s·c − m·c) as packed bf16, and the two row sums -------------------------
  auto exps = [&](const f32x16_t (&s)[T::NSUB], u32x4_t (&pw)[T::KS_PV]) {
    const float mc = m * c;
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float rs = 0.f, rsb = 0.f;
#pragma unroll
    for (int kk = 0; kk < T::KS_PV; ++kk) {
      const int h8 = (kk & 1) * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][h8 + 2 * e], c, -mc));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][h8 + 2 * e + 1], c, -mc));
        rs += e0 + e1;
        // The pair goes to dot2 directly: fed from an element of the packed
        // u32x4 instead, hipcc (ROCm 7.2) reads element 0 four times.
        bf16x2_t pe;
        pe[0] = (__bf16)e0;
        pe[1] = (__bf16)e1;
        rsb = __builtin_amdgcn_fdot2_f32_bf16(pe, ones, rsb, false);
        pw[kk][e] = __builtin_bit_cast(uint32_t, pe);
      }
    }
    l += rs;
    lb += rsb;
  };

  // ---- Oᵀ += Vᵀ P̃ᵀ ----------------------------------------------------------------------
  auto pv = [&](const unsigned char* vb, const u32x4_t (&pw)[T::KS_PV]) {
#pragma unroll
    for (int kk = 0; kk < T::KS_PV; ++kk)
#pragma unroll
      for (int ds = 0; ds < T::DSUB; ++ds) {
        const u32x2_t a0 = lds_tr_read(vb, v_rd[ds] + 16 * kk * T::ROW);
        const u32x2_t a1 = lds_tr_read(vb, v_rd[ds] + (16 * kk + 8) * T::ROW);
        const u32x4_t a = u32x4_t{a0[0], a0[1], a1[0], a1[1]};
        acc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                          __builtin_bit_cast(bf16x8_t, pw[kk]), acc[ds], 0, 0, 0);
      }
  };

  // ---- pipeline ---------------------------------------------------------------------
  // Iteration j reads K_{j+1} (for Sᵀ_{j+1}) and V_j, and issues the loads of
  // K_{j+4} into the buffer K_j held and of V_{j+3} into the buffer V_{j-1}
  // held: both were last read before the barrier that ended iteration j-1.
  // Before its closing barrier, iteration j waits only for the loads issued
  // two iterations earlier (K_{j+2}, V_{j+1}: needed next), so every load has
  // about two iterations to arrive.  Within an iteration the MFMAs of Sᵀ_{j+1}
  // are issued between the exp2 / convert / sum instructions of tile j, so the
  // matrix and vector units run side by side; the row max of Sᵀ_{j+1} is taken
  // while Oᵀ += Vᵀ_j P̃ᵀ_j runs.  The loop is unrolled by kStages so that every
  // buffer address is a compile-time offset.
  f32x16_t s0[T::NSUB], s1[T::NSUB];
  auto kb = [&](int j) { return kbufs[j % kStages]; };
  auto vb = [&](int j) { return vbufs[j % kStages]; };
#pragma unroll
  for (int j = 0; j < kStages; ++j)
    if (j < n_tiles) load_tile(krsrc, k_goff, j * T::BN, kb(j));
#pragma unroll
  for (int j = 0; j < kStages - 1; ++j)
    if (j < n_tiles) load_tile(vrsrc, v_goff, j * T::BN, vb(j));
  wait_vmcnt<0>();
  __syncthreads();
  if (active(0)) {
    qk(kb(0), s0);
    mask(0, s0);
    rescale(rowmax(s0));
  }
  __syncthreads();  // every wave is done with K_0 before K_4 lands in its buffer

  // Tiles 0 .. n_clean-1 need no mask for any row of the workgroup (and, when
  // causal, are seen by every wavefront); iterations whose next tile is clean
  // run without mask or activity tests.
  const int n_clean = CAUSAL ? min(N / T::BN, (q0 + 1) / T::BN) : N / T::BN;

  // phase: j mod kStages as a compile-time constant
  auto iteration = [&](int j, auto phase, auto generic) {
    constexpr int P = decltype(phase)::value;
    constexpr bool GENERIC = decltype(generic)::value;
    f32x16_t(&scur)[T::NSUB] = (P & 1) ? s1 : s0;
    f32x16_t(&snext)[T::NSUB] = (P & 1) ? s0 : s1;
    const bool ld_k = j + kStages < n_tiles;
    const bool ld_v = j + kStages - 1 < n_tiles;
    if (ld_k) load_tile(krsrc, k_goff, (j + kStages) * T::BN, kb(P));
    if (ld_v) load_tile(vrsrc, v_goff, (j + kStages - 1) * T::BN, vb(P + kStages - 1));
    const bool next = GENERIC ? (j + 1 < n_tiles && active(j + 1)) : true;
    const bool cur = GENERIC ? active(j) : true;
    if (cur) {
      u32x4_t pw[T::KS_PV];
      if (next) {
        qk(kb(P + 1), snext);
        exps(scur, pw);
        // issue order: K-fragment reads run two MFMAs ahead; each MFMA of
        // Sᵀ_{j+1} is followed by six VALU instructions of tile j's softmax
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < T::KS_QK * T::NSUB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        exps(scur, pw);
      }
      pv(vb(P), pw);
    }
    // (a wavefront that sees no key of tile j sees none of tile j+1 either)
    if (cur && next) {
      if (GENERIC) mask(j + 1, snext);
      rescale(rowmax(snext));
    }
    // loads issued by this iteration and the one before may stay in flight
    const int pending = (ld_k ? 1 : 0) + (ld_v ? 1 : 0) + (j + kStages - 1 < n_tiles ? 1 : 0) +
                        (j + kStages - 2 < n_tiles && j >= 1 ? 1 : 0);
    if (pending >= 4)
      wait_vmcnt<4 * T::LOADS>();
    else if (pending == 3)
      wait_vmcnt<3 * T::LOADS>();
    else if (pending == 2)
      wait_vmcnt<2 * T::LOADS>();
    else if (pending == 1)
      wait_vmcnt<T::LOADS>();
    else
      wait_vmcnt<0>();
    __syncthreads();
  };
  int j = 0;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  static_assert(kStages == 4, "unrolled by four");
  for (; j + 4 < n_clean; j += 4) {
    iteration(j, I0{}, std::false_type{});
    iteration(j + 1, I1{}, std::false_type{});
    iteration(j + 2, I2{}, std::false_type{});
    iteration(j + 3, I3{}, std::false_type{});
  }
  for (; j < n_tiles; j += 4) {
    iteration(j, I0{}, std::true_type{});
    if (j + 1 < n_tiles) iteration(j + 1, I1{}, std::true_type{});
    if (j + 2 < n_tiles) iteration(j + 2, I2{}, std::true_type{});
    if (j + 3 < n_tiles) iteration(j + 3, I3{}, std::true_type{});
  }

  // ---- epilogue: one division, one store of O and L ------------------------------
  l = pair_sum(l);
  lb = pair_sum(lb);
  if (q_row < N) {
    const float inv = 1.f / lb;
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
  using T = Tile<D>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&fa_fwd_kernel<D, CAUSAL>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - T::LDS_BYTES);
  if (attr != hipSuccess) return attr;
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
