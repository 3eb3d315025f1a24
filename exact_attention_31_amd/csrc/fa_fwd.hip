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
//      buffer loads that write LDS directly, about three tiles ahead of use,
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
// (FlashAttention-4), with the threshold set by the range of fp32 and bf16
// rather than by their precision (which is relative, so a stale m costs no
// accuracy).  P̃ is computed against the current m first; a tile row sum
// within 2^kRescaleLog2 proves that no element exceeds it, and only otherwise
// (in practice the first tile, where m = −∞) is the row max taken, m moved
// and P̃ recomputed.
//
// Pages cited: [cicada] "已有的几种大模型上下文支持情况"; [15-779 L5] "第 5 讲 ·
// 案例：Transformer、注意力与 FlashAttention".
//
// Schedule: the work of a tile is split into a softmax phase Y (steps 3–4 and
// P̃: vector ALU only) and a matrix phase X (step 5 for tile j and step 2 for
// tile j+1: MFMAs and LDS reads only).  Each wavefront runs Y(0) X(0) Y(1)
// X(1) ..., one phase per workgroup barrier; wavefronts 4-7 start one barrier
// after wavefronts 0-3.  The two wavefronts that share a SIMD are therefore
// always in opposite phases: while one keeps the matrix core busy, the other
// runs exp2 and the sums on the vector ALU.
//
// Layout on chip (one wavefront = 64 lanes, 32 query rows):
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
// * exp is computed as exp2 with scale·log2(e) folded into the logits.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

// log2-domain growth of the running max that forces a rescale.  P̃ stays
// below 2^48, so the fp32 accumulator holds Σ P̃·v over the at most 2^24 keys
// the library accepts as long as |v| < 2^56.
constexpr float kRescaleLog2 = 48.0f;
// A tile's P̃ row sum at most this bounds each of its elements by 2^kRescaleLog2.
constexpr float kSumBound = 281474976710656.0f;  // 2^48
constexpr int kStages = 4;  // LDS buffers per tensor (the loop is unrolled by this)
constexpr int kOperandLead = 2;  // MFMA pairs by which LDS operand reads run ahead

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

// Work index -> (bh, query block).  Workgroups are dealt round-robin to the
// 8 XCDs; with xcd_remap each XCD receives whole heads (so a head's K/V stays
// in one L2), and inside an XCD's share the heaviest query blocks (the last
// ones, for causal) are dispatched first (longest-processing-time-first,
// [15-779 L5] §6.2): r is the rank of the block in that order.
// PAIR (kernels that fit two workgroups on a CU): when an XCD's share fits its
// CUs at once — C < share ≤ 2C, C = kCusPerXcd — the first C workgroups take
// one CU each and workgroup C + k lands on the CU of workgroup k, so the order
// is arranged for that: the share's heaviest C − P blocks (P = share − C) get
// CUs of their own, and the next P are each paired with one of the P lightest,
// heaviest with lightest, which evens out the work per CU (causal blocks differ
// up to N/256-fold in length).  Only the order changes, not any result.
template <bool PAIR>
__device__ inline void decode_work(const FwdParams& p, int& bh, int& qb) {
  const int x = blockIdx.x;
  const int total = p.BH * p.n_qblk;
  if (p.xcd_remap) {
    const int per_xcd = total >> 3;
    const int heads_per_xcd = per_xcd / p.n_qblk;
    const int xcd = x & 7;
    const int local = x >> 3;
    int r = local;
    if (PAIR && per_xcd > kCusPerXcd && per_xcd <= 2 * kCusPerXcd) {
      const int P = per_xcd - kCusPerXcd;
      r = local < P ? (kCusPerXcd - P) + local                  // paired, heavier of the two
          : local < kCusPerXcd ? local - P                      // alone on its CU: the heaviest
          : per_xcd - 1 - (local - kCusPerXcd);                 // paired, lighter of the two
    }
    bh = xcd * heads_per_xcd + r % heads_per_xcd;
    qb = p.n_qblk - 1 - r / heads_per_xcd;
  } else {
    bh = x % p.BH;
    qb = p.n_qblk - 1 - x / p.BH;
  }
}

// SPARSE: block-sparse attention ([FA-1拆解] "块稀疏扩展"): a mask over blocks
// of kSparseBlock query rows × kSparseBlock keys switches whole score blocks
// off.  A workgroup owns one query block of kSparseBlock rows and streams only
// the key blocks its mask row keeps.  Wavefronts w and w + 4 own the same 32
// rows and take the two 32-key halves of every tile (group 0 the first, group
// 1 the second), so both groups work on every streamed tile; each keeps its own
// running (m, ℓ, accumulator) over its halves, and group 1 hands its summary to
// group 0 through LDS at the end, where the two are merged with ⊕ ([15-779 L5]
// §4.4) before the one division.
//
// Causal d = 64 runs two workgroups per CU (64 KiB of LDS each, registers held
// to 128 a lane): a CU then overlaps one block's prologue and epilogue with
// another's steady state, which pays where causal blocks vary in length
// (−15 % at B1 H32 N8192 d64 causal).  Non-causal d = 64 ran 2 % slower so,
// and d = 128 needs 128 KiB of LDS per workgroup.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kFwdThreads),
                          amdgpu_waves_per_eu(D == 64 && CAUSAL ? 4 : 2)))
void fa_fwd_kernel(FwdParams p) {
  using T = Tile<D>;
  static_assert(kSparseBlock == 2 * T::BN && kSparseBlock == 32 * (kFwdWaves / 2),
                "two tiles per key block; SPARSE: four wavefronts of 32 rows per query block");
  // per wavefront and tile: 32-key sub-tiles of Sᵀ and 16-key k-steps of Oᵀ += Vᵀ P̃ᵀ
  // (SPARSE: one 32-key half of each tile per wavefront group)
  constexpr int NSUB_W = SPARSE ? 1 : T::NSUB;
  constexpr int KSPV_W = SPARSE ? T::KS_PV / 2 : T::KS_PV;
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[T::TILE_BYTES], k_lds1[T::TILE_BYTES],
      k_lds2[T::TILE_BYTES], k_lds3[T::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[T::TILE_BYTES], v_lds1[T::TILE_BYTES],
      v_lds2[T::TILE_BYTES], v_lds3[T::TILE_BYTES];
  unsigned char* const kbufs[4] = {k_lds0, k_lds1, k_lds2, k_lds3};
  unsigned char* const vbufs[4] = {v_lds0, v_lds1, v_lds2, v_lds3};
  // SPARSE: the key blocks the workgroup's query block keeps, in order
  __shared__ uint16_t kblocks[SPARSE ? kSparseMaxBlocks : 1];

  int bh, qb;
  decode_work<D == 64 && CAUSAL && !SPARSE>(p, bh, qb);  // the two-workgroups-per-CU form
  const int N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int i32 = lane & 31;  // query column of Sᵀ / Oᵀ owned by this lane
  const int g = lane >> 5;    // which 32-lane half
  const int jj = lane & 15;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // wave index in a scalar register
  const int grp = wave_u >> 2;  // wavefronts w and w+4 share a SIMD and alternate phases
  const int q0 = qb * (SPARSE ? kSparseBlock : kFwdBlockM);
  const int wq0 = q0 + (SPARSE ? wave_u & 3 : wave_u) * 32;  // first query row of this wavefront (uniform)
  const int q_row = wq0 + i32;
  const int kh = SPARSE ? 32 * grp : 0;  // first key of this wavefront's part of a tile
  const size_t base = (size_t)bh * N * D;

  // Direct global->LDS loads, a tile issued by the four wavefronts of a group
  // (K by group 0, V by group 1): wavefront w (w & 3 = u), load i fills LDS
  // chunk slots (i*4 + u)*64 + lane of the tile; the slot's (row, swizzled
  // chunk) names the global chunk this lane fetches.  Load i covers rows
  // r0 + i*RPL, and both swizzles repeat with that period, so load i is load 0
  // shifted by i*RPL rows.  Rows past N lie past the head's bytes and read as
  // zero (their logits are masked).
  constexpr int RPL = (kFwdWaves / 2) * 64 / T::CH;  // rows covered by one load across a group
  const int r0 = ((wave & 3) * 64 + lane) / T::CH;
  const int cpos = lane % T::CH;
  const int k_goff = r0 * T::ROW + ((cpos ^ T::k_swz(r0)) << 4);
  const int v_goff = r0 * T::ROW + ((cpos ^ T::v_swz(r0)) << 4);
  const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(p.k + base, N * T::ROW);
  const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.v + base, N * T::ROW);

  // Operand-read lane offsets (bytes within a tile).
  int k_rd[T::KS_QK];  // K rows i32 (+32 per sub-tile), chunk 2kk + g
#pragma unroll
  for (int kk = 0; kk < T::KS_QK; ++kk) k_rd[kk] = (kh + i32) * T::ROW + (((2 * kk + g) ^ T::k_swz(i32)) << 4);
  int v_rd[T::DSUB];   // transpose reads: rows 4g + jj/4 (+16kk, +8), dims 32ds + 16(G&1) + 4(jj&3)
  {
    const int r = 4 * g + (jj >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1);
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds)
      v_rd[ds] = (kh + r) * T::ROW + (((4 * ds + cl) ^ T::v_swz(r)) << 4) + 8 * (jj & 1);
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

  int n_tiles;
  if constexpr (SPARSE) {
    // wavefront 0 compacts the key blocks the query block keeps into kblocks
    // (ballot + running count); causal: none past the block's last row
    const uint8_t* m0 = p.block_mask + ((size_t)(p.mask_heads == 1 ? 0 : bh) * p.mask_tq + qb) * p.mask_tk;
    const int kb_end = CAUSAL ? min(p.mask_tk, qb + 1) : p.mask_tk;
    int count = 0;
    if (wave_u == 0) {
      for (int base0 = 0; base0 < kb_end; base0 += 64) {
        const int kbk = base0 + lane;
        const int b0 = kbk < kb_end ? (m0[kbk] != 0) : 0;
        const uint64_t keep = __ballot(b0);
        const int pos = count + __builtin_amdgcn_mbcnt_hi((uint32_t)(keep >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)keep, 0));
        if (b0) kblocks[pos] = (uint16_t)kbk;
        count += __popcll(keep);
      }
    }
    __shared__ int kblock_count;
    if (tid == 0) kblock_count = count;
    __syncthreads();
    n_tiles = 2 * __builtin_amdgcn_readfirstlane(kblock_count);
  } else {
    n_tiles = fwd_kv_tiles(N, D, CAUSAL, qb);
  }
  // first key of tile j (SPARSE: of the j-th tile of the kept blocks)
  auto tile_kv0 = [&](int j) __attribute__((always_inline)) {
    if constexpr (SPARSE)
      return ((int)kblocks[j >> 1] * kSparseBlock) + (j & 1) * T::BN;
    else
      return j * T::BN;
  };
  const float c = p.scale_log2;
  auto active = [&](int j) __attribute__((always_inline)) {  // some row of the wave sees the tile
    if constexpr (SPARSE) {  // ... in this wavefront's half of it, which holds a key below N
      if (j >= n_tiles) return false;
      const int k0 = __builtin_amdgcn_readfirstlane(tile_kv0(j)) + kh;
      return k0 < N && (!CAUSAL || k0 <= wq0 + 31);
    } else {
      return !CAUSAL || j * T::BN <= wq0 + 31;
    }
  };

  float m = -INFINITY;  // reference max of the raw logits q·k (this lane's query row)
  // Two running sums over this lane's half of the keys: ℓ of the fp32 P̃ (for
  // L: rows with few keys need it within 1e-3) and ℓ_b of the bf16-rounded P̃
  // that enter the MFMA (for O: numerator and denominator then use the same
  // weights, so a row dominated by one key returns that key's value exactly).
  float l = 0.f;
  float lb[2] = {0.f, 0.f};  // ℓ_b in two partial sums, accumulated in the matrix phase
  f32x16_t acc[T::DSUB];
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds) acc[ds] = f32x16_t{};
  f32x16_t s[NSUB_W];       // scores of the tile between its QK and its softmax
  bf16x2_t pw[KSPV_W][4];   // P̃ of the tile between its softmax and its PV (bf16 pairs)

  // ---- softmax phase of tile j: mask, row max, rescale, P̃ and the sums ------------
  auto softmax = [&](int j, auto clean) __attribute__((always_inline)) {
    const int kv0 = __builtin_amdgcn_readfirstlane(tile_kv0(j)) + kh;  // first key of the wave's part
    if (!decltype(clean)::value && ((kv0 + 32 * NSUB_W > N) || (CAUSAL && kv0 + 32 * NSUB_W - 1 > wq0))) {
      const int lim = CAUSAL ? min(q_row, N - 1) : N - 1;
#pragma unroll
      for (int sub = 0; sub < NSUB_W; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + sub * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
          if (key > lim) s[sub][r] = -INFINITY;
        }
    }
    // P̃ against the current reference max; the tile sum bounds every element,
    // so a sum at most 2^kRescaleLog2 proves that no row outgrew m by more
    // than that and the row max is not needed.
    float rs;
    auto exps = [&]() __attribute__((always_inline)) {
      // SPARSE: a row may still have no key (m = −∞); 0 then stands in for
      // the offset, which keeps masked logits at weight 0 instead of NaN
      const float mc = (SPARSE && m == -INFINITY) ? 0.f : m * c;
      float r2[2] = {0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KSPV_W; ++kk) {
        const int h8 = (kk & 1) * 8;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][h8 + 2 * e], c, -mc));
          const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kk >> 1][h8 + 2 * e + 1], c, -mc));
          r2[e & 1] += e0 + e1;
          pw[kk][e][0] = (__bf16)e0;
          pw[kk][e][1] = (__bf16)e1;
        }
      }
      rs = r2[0] + r2[1];
    };
    exps();
    if (__any(!(rs <= kSumBound) || (SPARSE && m == -INFINITY))) {  // also taken for inf / NaN sums (first tile: m = -inf)
      // row max: four independent chains, then across the two lane halves
      float mx[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) mx[t] = -INFINITY;
#pragma unroll
      for (int sub = 0; sub < NSUB_W; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx[r & 3] = fmaxf(mx[r & 3], s[sub][r]);
      const float mt = pair_max(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
      // move the reference max only when some row outgrew it by 2^kRescaleLog2;
      // the first tile holds key 0, visible to every row, so m is finite after it
      if (__any((mt - m) * c > kRescaleLog2)) {
        const float m_new = fmaxf(m, mt);
        const float alpha = (SPARSE && m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((m - m_new) * c);
        l *= alpha;
        lb[0] *= alpha;
        lb[1] *= alpha;
#pragma unroll
        for (int ds = 0; ds < T::DSUB; ++ds) acc[ds] *= alpha;
        m = m_new;
        exps();
      }
    }
    l += rs;
  };

  // ---- matrix phase: Oᵀ += Vᵀ_j P̃ᵀ_j and Sᵀ_{j+1} = K_{j+1} Qᵀ, MFMAs interleaved ------
  auto qk_step = [&](const unsigned char* kb, int i) __attribute__((always_inline)) {
    const int kk = i / NSUB_W, sub = i % NSUB_W;
    const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kb + k_rd[kk] + sub * 32 * T::ROW);
    s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf), qf[kk], s[sub], 0, 0, 0);
  };
  // ℓ_b += the bf16 P̃ of k-step kk.  v_dot2 shares the matrix core's pipe: in
  // the softmax phase each one would wait for the other wavefront's MFMA, here
  // it queues behind this wavefront's own.  ℓ_b and the accumulator take the
  // same tile in the same phase, so a later rescale treats them alike.
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  // (The pairs are kept as bf16x2 values: taken as elements of a packed u32x4,
  // hipcc (ROCm 7.2) feeds all four dot2 of a k-step from element 0.)
  auto lb_step = [&](int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) lb[e & 1] = __builtin_amdgcn_fdot2_f32_bf16(pw[kk][e], ones, lb[e & 1], false);
  };
  auto pv_read = [&](const unsigned char* vb, int i) __attribute__((always_inline)) {
    const int kk = i / T::DSUB, ds = i % T::DSUB;
    const u32x2_t a0 = lds_tr_read(vb, v_rd[ds] + 16 * kk * T::ROW);
    const u32x2_t a1 = lds_tr_read(vb, v_rd[ds] + (16 * kk + 8) * T::ROW);
    return u32x4_t{a0[0], a0[1], a1[0], a1[1]};
  };
  u32x4_t vpre[2];  // the first two Vᵀ operands of a clean matrix phase, read before its barrier
  auto pv_mma = [&](int i, const u32x4_t& a) __attribute__((always_inline)) {
    const int kk = i / T::DSUB, ds = i % T::DSUB;
    const bf16x8_t pb = __builtin_shufflevector(__builtin_shufflevector(pw[kk][0], pw[kk][1], 0, 1, 2, 3),
                                                __builtin_shufflevector(pw[kk][2], pw[kk][3], 0, 1, 2, 3), 0, 1, 2,
                                                3, 4, 5, 6, 7);
    acc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), pb, acc[ds], 0, 0, 0);
    if (ds == T::DSUB - 1) lb_step(kk);
  };
  auto pv_step = [&](const unsigned char* vb, int i) __attribute__((always_inline)) { pv_mma(i, pv_read(vb, i)); };
  constexpr int NQK = T::KS_QK * NSUB_W;  // MFMAs of one Sᵀ tile (of the wave's part)
  constexpr int NPV = KSPV_W * T::DSUB;   // MFMAs of one Oᵀ update
  auto matrix_clean = [&](const unsigned char* vb, const unsigned char* kb) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);  // the matrix-phase wavefront wins issue ties
    // Lane offsets opaque to loop-invariant code motion: addresses are formed
    // here as offset + constant, the constant going into the instruction.
#pragma unroll
    for (int kk = 0; kk < T::KS_QK; ++kk) asm volatile("" : "+v"(k_rd[kk]));
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds) asm volatile("" : "+v"(v_rd[ds]));
#pragma unroll
    for (int sub = 0; sub < NSUB_W; ++sub) s[sub] = f32x16_t{};
    static_assert(NQK == NPV, "interleave pairs one MFMA of each product");
    // PV(0), PV(1) from the operands read before the barrier, then QK(i) with
    // PV(i+2): the K reads the first QK waits for run under two MFMAs
    pv_mma(0, vpre[0]);
    pv_mma(1, vpre[1]);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      qk_step(kb, i);
      if (i + 2 < NPV) pv_step(vb, i + 2);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 3 * kOperandLead - 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    asm volatile("" : "+v"(lb[0]), "+v"(lb[1]));  // the dot2 stay in this phase
    __builtin_amdgcn_s_setprio(0);
  };
  auto matrix = [&](const unsigned char* vb, const unsigned char* kb, bool do_pv, bool do_qk) __attribute__((always_inline)) {
    if (do_qk) {
#pragma unroll
      for (int sub = 0; sub < NSUB_W; ++sub) s[sub] = f32x16_t{};
#pragma unroll
      for (int i = 0; i < NQK; ++i) qk_step(kb, i);
    }
    if (do_pv) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) pv_step(vb, i);
      asm volatile("" : "+v"(lb[0]), "+v"(lb[1]));
    }
  };

  // ---- pipeline -------------------------------------------------------------------
  // Every wavefront runs the same sequence of phases, each closed by a
  // workgroup barrier:  QK(0) | Y(0) | X(0) | Y(1) | X(1) | ... | Y(n-1) | X(n-1)
  // with Y(j) the softmax of tile j and X(j) the matrix phase Oᵀ += Vᵀ_j P̃ᵀ_j,
  // Sᵀ_{j+1} = K_{j+1} Qᵀ.  Group 1 (wavefronts 4-7) starts one barrier later
  // than group 0, so the two wavefronts of a SIMD are always in opposite
  // phases: one feeds the matrix core while the other runs the softmax.
  // The K tiles stream through group 0 and the V tiles through group 1, each
  // issuing its loads at the start of its softmax phases, so the matrix
  // phases never issue or wait for a load.  With T the global phase (group
  // 0's phase index; group 1's plus one), Y(j) loads tile j+3: group 0's at
  // T = 2j+1 puts K_{j+3} where K_{j-1} was (last read at T = 2j-1), group 1's
  // at T = 2j+2 puts V_{j+3} where V_{j-1} was (last read at T = 2j+1).  At
  // the end of Y(j) a wavefront waits for its tile j+1, which the matrix
  // phases read from T = 2j+2 (K) and T = 2j+4 (V) on.  Tiles outside
  // [0, n_tiles) are loaded from past the end of K and V (zeros, no memory
  // traffic) into buffers nobody reads again, so every wavefront keeps the
  // same number of loads in flight.
  auto kb = [&](int j) { return kbufs[j & 3]; };
  auto vb = [&](int j) { return vbufs[j & 3]; };
  const __amdgpu_buffer_rsrc_t mrsrc = grp ? vrsrc : krsrc;
  const int m_goff = grp ? v_goff : k_goff;
  auto load_tile = [&](int t, unsigned char* dst) __attribute__((always_inline)) {  // this group's tile t
    const int kv0 = (t >= 0 && t < n_tiles) ? __builtin_amdgcn_readfirstlane(tile_kv0(t)) : N;
    unsigned char* d = dst + (wave_u & 3) * 1024;
#pragma unroll
    for (int i = 0; i < 2 * T::LOADS; ++i)
      load_lds16(mrsrc, d + i * (kFwdWaves / 2) * 1024, m_goff + (kv0 + i * RPL) * T::ROW);
  };
#pragma unroll
  for (int t = 0; t < 3; ++t) load_tile(t, grp ? vbufs[t] : kbufs[t]);
  wait_vmcnt<4 * T::LOADS>();  // tile 0 has landed
  // The Q loads were issued before the tile loads, so they are complete now;
  // a use here settles the compiler's load tracking for those registers once,
  // instead of a full wait for all loads at their first use inside the loop.
#pragma unroll
  for (int kk = 0; kk < T::KS_QK; ++kk) asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, qf[kk])));
  block_barrier();
  if (grp == 1) block_barrier();
  if (active(0)) matrix(vb(0), kb(0), false, true);
  wait_vmcnt<2 * T::LOADS>();  // tile 1
  block_barrier();

  auto iter = [&](int j, auto phase, auto clean) __attribute__((always_inline)) {
    constexpr int P = decltype(phase)::value;  // j mod 4
    constexpr bool CLEAN = decltype(clean)::value;
    // Y(j), with this group's tile j+3
    load_tile(j + 3, grp ? vbufs[(P + 3) & 3] : kbufs[(P + 3) & 3]);
    if (CLEAN)
      softmax(j, std::true_type{});
    else if (active(j))
      softmax(j, std::false_type{});
    wait_vmcnt<4 * T::LOADS>();  // tile j+1
    // The first two Vᵀ operands of X(j) are read now, ahead of the barrier: V_j
    // has been visible since the barrier that closed group 1's Y(j-1), which
    // both groups have passed, and its buffer is refilled only after X(j).
    if (CLEAN) {
      vpre[0] = pv_read(vb(P), 0);
      vpre[1] = pv_read(vb(P), 1);
    }
    block_barrier();
    // X(j)
    if (CLEAN)
      matrix_clean(vb(P), kb(P + 1));
    else
      matrix(vb(P), kb(P + 1), active(j), j + 1 < n_tiles && active(j + 1));
    block_barrier();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using Y = std::true_type;
  using G = std::false_type;
  // Tiles 0 .. n_clean-1 are seen whole by every row of the workgroup.
  // Iteration j is clean when tile j is and a tile j+1 exists: that tile's
  // first key is then at most the workgroup's first row + 1, so every
  // wavefront sees it and computes its Sᵀ in either form.  SPARSE: with N a
  // multiple of the mask block every kept tile is whole, and every row sees all
  // of its keys when non-causal, those of the blocks before its own when causal
  // (the list is in key order, so only its last block can be the query block's
  // own); a wavefront that does not see tile j+1 computes its Sᵀ for nothing.
  int n_clean;
  if constexpr (SPARSE) {
    const int nb = n_tiles >> 1;
    const int own_last = nb > 0 ? __builtin_amdgcn_readfirstlane((int)kblocks[nb - 1]) == qb : 0;
    n_clean = N % kSparseBlock != 0 ? 0 : !CAUSAL ? n_tiles : 2 * (nb - own_last);
  } else {
    n_clean = CAUSAL ? min(N / T::BN, (q0 + 1) / T::BN) : N / T::BN;
  }
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

  // ---- epilogue: one division, one store of O and L ------------------------------
  // O leaves the accumulators as 8-byte pieces of 32 different rows per
  // instruction; written to HBM like that, each row segment is a separate
  // partial-line write.  The wavefront stages its 32 rows in LDS instead (a K
  // or V buffer: every wavefront is past its last read of them and every load
  // has landed) and writes them back as whole rows, 16 bytes a lane.
  wait_vmcnt<0>();  // the loads past the last tile write tile buffers too
  block_barrier();
  l = pair_sum(l);
  float lbs = pair_sum(lb[0] + lb[1]);
  if constexpr (SPARSE) {
    // Wavefront w + 4 holds the same rows as w over the other key half of every
    // tile: it leaves its (m, ℓ, ℓ_b, accumulator) in LDS (K and V buffer w & 3:
    // every load has landed and every read is done) and w merges the two with ⊕.  Each value
    // goes to [element][lane], so the stores and loads are conflict-free.
    const int u = wave_u & 3;
    float* const xacc = reinterpret_cast<float*>(u == 0 ? k_lds0 : u == 1 ? k_lds1 : u == 2 ? k_lds2 : k_lds3);
    float* const xrow = reinterpret_cast<float*>(u == 0 ? v_lds0 : u == 1 ? v_lds1 : u == 2 ? v_lds2 : v_lds3);
    static_assert(T::DSUB * 16 * 64 * 4 <= T::TILE_BYTES, "the accumulator fits one tile buffer");
    if (grp == 1) {
#pragma unroll
      for (int ds = 0; ds < T::DSUB; ++ds)
#pragma unroll
        for (int r = 0; r < 16; ++r) xacc[(ds * 16 + r) * 64 + lane] = acc[ds][r];
      xrow[lane] = m;
      xrow[64 + lane] = l;
      xrow[128 + lane] = lbs;
    }
    block_barrier();
    if (grp == 1) return;  // no barrier follows
    const float m2 = xrow[lane];
    const float mm = fmaxf(m, m2);  // −∞: neither half of the row saw a key
    const float f1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mm) * c);
    const float f2 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m2 - mm) * c);
    l = l * f1 + xrow[64 + lane] * f2;
    lbs = lbs * f1 + xrow[128 + lane] * f2;
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ds][r] = acc[ds][r] * f1 + xacc[(ds * 16 + r) * 64 + lane] * f2;
    m = mm;
  }
  const float inv = (SPARSE && lbs == 0.f) ? 0.f : 1.f / lbs;  // SPARSE: a row with no key writes O = 0, L = −∞
  constexpr int SROW = 2 * D + 16;  // padded row stride of the staging tile (bytes)
  static_assert(32 * SROW <= T::TILE_BYTES, "a wavefront's rows fit one tile buffer");
  unsigned char* const stg = wave_u == 0 ? k_lds0 : wave_u == 1 ? k_lds1 : wave_u == 2 ? k_lds2 : wave_u == 3 ? k_lds3
                           : wave_u == 4 ? v_lds0 : wave_u == 5 ? v_lds1 : wave_u == 6 ? v_lds2 : v_lds3;
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
  constexpr int RPI = 64 / T::CH;  // rows per store instruction
  const int rr0 = lane / T::CH, cc = lane % T::CH;
  u32x4_t ow[32 / RPI];
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) ow[it] = *reinterpret_cast<const u32x4_t*>(stg + (it * RPI + rr0) * SROW + cc * 16);
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it)
    if (wq0 + it * RPI + rr0 < N)
      *reinterpret_cast<u32x4_t*>(p.o + base + (size_t)(wq0 + it * RPI + rr0) * D + cc * 8) = ow[it];
  if (q_row < N && g == 0) p.lse[(size_t)bh * N + q_row] = m * p.scale + __builtin_amdgcn_logf(l) * 0.69314718055994531f;
}

template <int D, bool CAUSAL, bool SPARSE>
hipError_t launch_fwd_t(const FwdParams& p, hipStream_t stream) {
  static const hipError_t attr = allow_full_lds(&fa_fwd_kernel<D, CAUSAL, SPARSE>);
  if (attr != hipSuccess) return attr;
  const dim3 grid(p.BH * p.n_qblk);
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, SPARSE>), grid, dim3(kFwdThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool SPARSE>
hipError_t launch_fwd_s(const FwdParams& p, int d, int causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_fwd_t<64, true, SPARSE>(p, stream) : launch_fwd_t<64, false, SPARSE>(p, stream);
  return causal ? launch_fwd_t<128, true, SPARSE>(p, stream) : launch_fwd_t<128, false, SPARSE>(p, stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, int causal, hipStream_t stream) {
  return p.block_mask ? launch_fwd_s<true>(p, d, causal, stream) : launch_fwd_s<false>(p, d, causal, stream);
}

}  // namespace fa
