// Exact-attention backward for CDNA4 (gfx950): dQ, dK, dV from Q, K, V, the
// forward output O, its log-sum-exp L and the output gradient dO.
//
// The N×N probabilities are never stored: every kernel recomputes the tile
// it needs as P = exp(scale·Q Kᵀ − L) from the saved L, which already holds
// each row's normalisation, so no online softmax is needed here
// ([15-779 L5] §7.2; [cicada] §3.2.3 keeps L for exactly this).  With
// D_i = dO_i · O_i formed once per row before the loops ([15-779 L5] §7.3),
// each tile's gradient of the scores is local:
//     dP = dO Vᵀ,   dS = P ∘ (dP − D),
//     dV = Σ Pᵀ dO,   dK = scale · Σ dSᵀ Q,   dQ = scale · Σ dS K.
// ([15-779 L5] §7.1; [pinghaoyang FA-1] "Backward".)
//
// The kernels:
//   fa_bwd_prep   per row: (L·log2 e, D) into the workspace;
//   fa_bwd_dkdv   key/value blocks outside, query tiles inside — the loop
//                 order of [15-779 L5] §7.4: a workgroup keeps dK and dV of
//                 its 128 keys in registers and writes them once (by default
//                 fa_bwd_dkdv_pair, eight wavefronts in pairs; the atomic and
//                 block-sparse forms use fa_bwd_dkdv, four wavefronts);
//   fa_bwd_dq     query blocks outside, key/value tiles inside, as in the
//                 forward: dQ of 256 query rows stays in registers.
// Stream order: by default fa_bwd_dq (which forms the per-row pairs itself,
// as fa_bwd_prep would, and writes them) then fa_bwd_dkdv_pair; the
// block-sparse form runs prep, dkdv, dq; the atomic form prep, dkdv<FUSED>,
// then fa_bwd_dq_finish.
// By default dQ is not accumulated with atomic adds from the key-block kernel
// (the scheme of [15-779 L5] §7.4); its own pass recomputes S and dP instead,
// which costs two more tile products (seven in all, against five) but keeps
// the result deterministic and needs no fp32 dQ buffer or atomic traffic.
// The atomic scheme is built too (fa_bwd_dkdv<FUSED>, then fa_bwd_dq_finish):
// each key block adds its dQ share into an fp32 buffer, and every key block
// of a head adds into all of the head's later query rows, so the atomic
// traffic is about N/128 times the size of dQ in fp32.  On this chip those
// device-scope fp32 adds, not the products, bound it: at 4096 keys the atomic
// form takes about twice as long as the two-pass form.
//
// Layout on chip (64-lane wavefronts, v_mfma_f32_32x32x16_bf16):
// * dkdv (four-wavefront form): each wavefront owns 32 keys.  The products
//   are taken so that a lane's accumulator column is one key: S = Q Kᵀ and
//   dP = dO Vᵀ with the key rows of K and V held in registers as the B
//   operands; P and dS then sit in the layout of the B operand of
//   dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS, whose A operands are read from the Q and
//   dO tiles in LDS with the transpose load ds_read_b64_tr_b16.
// * dkdv_pair: the same products split over two wavefronts per 32 keys
//   (layout at the kernel).
// * dq: each wavefront owns 32 query rows, lane = query column as in the
//   forward: Sᵀ = K Qᵀ and dPᵀ = V dOᵀ with Q and dO rows in registers, so
//   L and D are one scalar per lane; dSᵀ feeds dQᵀ += Kᵀ dSᵀ directly, Kᵀ
//   again read with the transpose load.
// * Tiles in LDS are row-major with the 16-byte chunk index XOR-ed with a
//   function of the row that keeps both the 16-byte row reads (16 rows, one
//   chunk) and the transpose reads (4 rows, 64 bytes each) on distinct banks.
//   Tiles are filled by buffer loads that write LDS directly, two stages
//   ahead of use; rows past N read as zero.
//
// Pages cited: [15-779 L5] "第 5 讲 · 案例：Transformer、注意力与 FlashAttention";
// [cicada] "已有的几种大模型上下文支持情况"; [pinghaoyang FA-1] "FlashAttention
// 完全拆解（一）".

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <int D>
struct BwdTile {
  static constexpr int CH = D / 8;        // 16-byte chunks per row
  static constexpr int ROW = 2 * D;       // bytes per row in LDS (unpadded)
  static constexpr int RPR = 1024 / ROW;  // rows filled by one wavefront-wide 16-byte direct load
  static constexpr int KS = D / 16;       // MFMA k-steps over d
  static constexpr int DSUB = D / 32;     // 32-wide sub-tiles over d
  // Chunk swizzle, period 16 rows.  D = 128 (16 chunks a row): 16 consecutive
  // rows take 16 distinct values (row reads), and the 4 rows of an aligned
  // group differ in bits 2-3 (transpose reads touch 4 chunks of each of 4
  // rows).  D = 64 (8 chunks): the same for rows of equal parity, whose bank
  // halves coincide.
  __device__ static int swz(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
};

// Buffer loads into registers; bytes at or past num_records read as zero.
__device__ inline u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

__device__ inline float2 buffer_load8(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
}

// Lane offsets into a tile of BwdTile<D> rows.
template <int D>
struct TileReads {
  using T = BwdTile<D>;
  int row[T::KS];    // 16-byte row reads: row i32 (+32 per sub-tile), chunk 2kk + g
  int tr0[T::DSUB];  // transpose reads, rows 4g + jj/4 (+16 per k-step)
  int tr8[T::DSUB];  // the same 8 rows further on (the swizzle has period 16)
  // offsets of the transpose reads of d sub-tile ds (rows 4g + jj/4 and 8 on)
  __device__ static int tr_off(int lane, int ds, int plus8) {
    const int jj = lane & 15;
    const int r = 4 * (lane >> 5) + (jj >> 2) + 8 * plus8;
    const int cl = 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1);
    return r * T::ROW + (((4 * ds + cl) ^ T::swz(r)) << 4) + 8 * (jj & 1);
  }
  __device__ void init(int lane) {
    const int i32 = lane & 31, g = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < T::KS; ++kk) row[kk] = i32 * T::ROW + (((2 * kk + g) ^ T::swz(i32)) << 4);
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds) {
      tr0[ds] = tr_off(lane, ds, 0);
      tr8[ds] = tr_off(lane, ds, 1);
    }
  }
  // A operand of one k-step (16 rows) of a product whose reduction index is the row,
  // from the offsets of its two halves.
  __device__ static bf16x8_t tr_at(const unsigned char* b, int o0, int o8, int kk) {
    const u32x2_t a0 = lds_tr_read(b, o0 + 16 * kk * T::ROW);
    const u32x2_t a1 = lds_tr_read(b, o8 + 16 * kk * T::ROW);
    return __builtin_bit_cast(bf16x8_t, u32x4_t{a0[0], a0[1], a1[0], a1[1]});
  }
  __device__ bf16x8_t tr(const unsigned char* b, int ds, int kk) const { return tr_at(b, tr0[ds], tr8[ds], kk); }
  // A operand of one k-step (16 of d) for the 32 rows of sub-tile `sub`.
  __device__ bf16x8_t rows(const unsigned char* b, int kk, int sub) const {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(b + row[kk] + sub * 32 * T::ROW));
  }
};

// Direct loads of a tile: wavefront-wide load x fills LDS bytes [1024x, +1024),
// i.e. rows x·RPR .. +RPR-1 with their chunks swizzled.  `goff` is the global
// offset of the lane's chunk for run x0; runs x0 + 16/RPR·i share it up to a
// shift of the tile offset (the swizzle repeats every 16 rows).
template <int D>
__device__ inline int run_goff(int x0, int lane) {
  using T = BwdTile<D>;
  const int r = x0 * T::RPR + lane / T::CH;
  return r * T::ROW + (((lane % T::CH) ^ T::swz(r)) << 4);
}

// Writes a wavefront's 32 output rows, held as fp32 accumulators whose lane is
// the row (a[ds] element r: column 32·ds + 8·(r/4) + 4·g + r%4), scaled by
// `mul` and rounded to bf16.  Stored straight from that layout, every store
// instruction would write 8-byte pieces of 32 rows; instead the rows go
// through `stg` (32·2D bytes of LDS that nothing else uses meanwhile; 16-byte
// chunks XOR-swizzled by the row) and leave as whole rows, 16 bytes a lane.
// Rows at or past `valid` are not written.
template <int D>
__device__ inline void store_rows_staged(const f32x16_t (&a)[D / 32], float mul, unsigned char* stg,
                                         uint16_t* out, int valid, int lane) {
  constexpr int CH = D / 8, ROW = 2 * D, RPI = 64 / CH;
  const int i32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      u32x2_t w;
      w[0] = pack_bf16x2(a[ds][4 * r4 + 0] * mul, a[ds][4 * r4 + 1] * mul);
      w[1] = pack_bf16x2(a[ds][4 * r4 + 2] * mul, a[ds][4 * r4 + 3] * mul);
      *reinterpret_cast<u32x2_t*>(stg + i32 * ROW + (((4 * ds + r4) ^ (i32 % CH)) << 4) + 8 * g) = w;
    }
  const int rr0 = lane / CH, cc = lane % CH;
  u32x4_t ow[32 / RPI];
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int rr = it * RPI + rr0;
    ow[it] = *reinterpret_cast<const u32x4_t*>(stg + rr * ROW + ((cc ^ (rr % CH)) << 4));
  }
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it)
    if (it * RPI + rr0 < valid) *reinterpret_cast<u32x4_t*>(out + (size_t)(it * RPI + rr0) * D + cc * 8) = ow[it];
}

// ---- per-row statistics: (L·log2 e, D = dO·O) ---------------------------------------
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_prep_kernel(BwdParams p) {
  constexpr int CH = D / 8;
  const int rows_total = p.BH * p.N;
  const int row = blockIdx.x * (256 / CH) + threadIdx.x / CH;
  const int c = threadIdx.x % CH;
  float acc = 0.f;
  if (row < rows_total) {
    const u32x4_t o = reinterpret_cast<const u32x4_t*>(p.o + (size_t)row * D)[c];
    const u32x4_t g = reinterpret_cast<const u32x4_t*>(p.dout + (size_t)row * D)[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(o[e] << 16), __uint_as_float(g[e] << 16), acc);
      acc = fmaf(__uint_as_float(o[e] & 0xffff0000u), __uint_as_float(g[e] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int w = CH / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, CH);
  if (row < rows_total && c == 0)
    reinterpret_cast<float2*>(p.ld)[row] = make_float2(p.lse[row] * 1.4426950408889634f, acc);
  if (p.dqacc && row < rows_total) {  // the fused backward's dQ accumulator starts at zero
    float4* z = reinterpret_cast<float4*>(p.dqacc + (size_t)row * D + 8 * c);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// dQ = scale · the fp32 accumulator, as bf16 (8 elements per thread)
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_dq_finish_kernel(BwdParams p) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= (size_t)p.BH * p.N * D) return;
  const float4 a = *reinterpret_cast<const float4*>(p.dqacc + i);
  const float4 b = *reinterpret_cast<const float4*>(p.dqacc + i + 4);
  u32x4_t w;
  w[0] = pack_bf16x2(a.x * p.scale, a.y * p.scale);
  w[1] = pack_bf16x2(a.z * p.scale, a.w * p.scale);
  w[2] = pack_bf16x2(b.x * p.scale, b.y * p.scale);
  w[3] = pack_bf16x2(b.z * p.scale, b.w * p.scale);
  *reinterpret_cast<u32x4_t*>(p.dq + i) = w;
}

// ---- dK, dV: key blocks outside, query tiles inside ------------------------------
__device__ inline void decode_kblock(const BwdParams& p, int& bh, int& kb) {
  const int x = blockIdx.x;
  if (p.xcd_remap_k) {  // whole heads per XCD; within an XCD the heaviest blocks (first keys) first
    const int per_xcd = (p.BH * p.n_kblk) >> 3;
    const int heads_per_xcd = per_xcd / p.n_kblk;
    const int local = x >> 3;
    bh = (x & 7) * heads_per_xcd + local % heads_per_xcd;
    kb = local / heads_per_xcd;
  } else {
    bh = x % p.BH;
    kb = x / p.BH;
  }
}

// One wavefront per SIMD: the dK and dV accumulators (32 keys × d each),
// the K and V rows and two 32-row score tiles need more than the 256
// registers a lane has when two wavefronts share a SIMD.
// FUSED: also dQ, by the loop order of [15-779 L5] §7.4 — each step's dS goes
// through LDS ([key][query] bf16), the next step multiplies it by the block's
// K tile (kept in LDS) and adds the block's share of dQ to an fp32 buffer with
// atomic adds.  Every wait then covers all outstanding memory operations.
// SPARSE: the backward of block-sparse attention; the workgroup lists the
// query blocks (kSparseBlock rows) whose mask keeps its key block and steps
// through those only.
template <int D, bool CAUSAL, bool FUSED, bool SPARSE>
__global__ __launch_bounds__(kBwdKvThreads, 1) void fa_bwd_dkdv_kernel(BwdParams p) {
  static_assert(!(FUSED && SPARSE), "the block-sparse backward takes the two-pass form");
  static_assert(kBwdBlockK == kSparseBlock, "one key block is one mask block");
  using T = BwdTile<D>;
  using TS = BwdTile<64>;  // the dS tile: 64 query columns (128-byte rows) per key
  constexpr int W = kBwdKvWaves;
  constexpr int BM = 64;              // query rows per step (two 32-row sub-tiles)
  constexpr int QT = BM * T::ROW;     // bytes of one Q (or dO) stage
  constexpr int R = BM / T::RPR;      // direct loads per tensor per stage
  static_assert(2 * R % W == 0 && (W * T::RPR) % 16 == 0, "stage loads spread evenly, one lane offset");
  constexpr int PER = 2 * R / W;      // tile loads per wavefront per stage
  __shared__ __attribute__((aligned(16))) unsigned char q_lds0[QT], q_lds1[QT], q_lds2[QT];
  __shared__ __attribute__((aligned(16))) unsigned char o_lds0[QT], o_lds1[QT], o_lds2[QT];
  __shared__ __attribute__((aligned(16))) float l_lds0[2 * BM], l_lds1[2 * BM], l_lds2[2 * BM];
  unsigned char* const qbufs[3] = {q_lds0, q_lds1, q_lds2};
  unsigned char* const obufs[3] = {o_lds0, o_lds1, o_lds2};
  float* const lbufs[3] = {l_lds0, l_lds1, l_lds2};
  // FUSED: the block's K tile (tr reads give the B operand of dQ = dS K) and dS
  __shared__ __attribute__((aligned(16))) unsigned char kt_lds[FUSED ? kBwdBlockK * T::ROW : 16];
  __shared__ __attribute__((aligned(16))) unsigned char ds_lds[FUSED ? kBwdBlockK * BM * 2 : 16];

  int bh, kb;
  decode_kblock(p, bh, kb);
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i32 = lane & 31, g = lane >> 5;
  const int k0 = kb * kBwdBlockK;
  const int kw = k0 + 32 * wave_u;  // first key of this wavefront
  const int key = kw + i32;         // the key of this lane's accumulator column
  const size_t base = (size_t)bh * N * D;
  const __amdgpu_buffer_rsrc_t qrsrc = make_rsrc(p.q + base, N * T::ROW);
  const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(p.dout + base, N * T::ROW);
  const __amdgpu_buffer_rsrc_t lrsrc = make_rsrc(p.ld + (size_t)bh * N * 2, N * 8);

  // K and V rows of this lane's key: the B operands of S = Q Kᵀ and dP = dO Vᵀ.
  bf16x8_t kf[T::KS], vf[T::KS];
  {
    const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(p.k + base, N * T::ROW);
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.v + base, N * T::ROW);
#pragma unroll
    for (int kk = 0; kk < T::KS; ++kk) {
      kf[kk] = __builtin_bit_cast(bf16x8_t, buffer_load16(krsrc, key * T::ROW + (2 * kk + g) * 16));
      vf[kk] = __builtin_bit_cast(bf16x8_t, buffer_load16(vrsrc, key * T::ROW + (2 * kk + g) * 16));
    }
  }

  TileReads<D> rd;
  rd.init(lane);
  // FUSED: this wavefront's share of dQ = dS K is d columns 32·dq_ds on, for
  // both 32-query halves (d = 128) or for half dq_u0 (d = 64); the lane
  // offsets of its transpose reads of K and dS (uniform indexes, computed once)
  constexpr int DQ_NU = T::DSUB == 4 ? 2 : 1;
  const int dq_ds = T::DSUB == 4 ? wave_u : wave_u >> 1;
  const int dq_u0 = T::DSUB == 4 ? 0 : wave_u & 1;
  int kt_o0 = 0, kt_o8 = 0, dso0[DQ_NU] = {}, dso8[DQ_NU] = {};
  if constexpr (FUSED) {
    kt_o0 = TileReads<D>::tr_off(lane, dq_ds, 0);
    kt_o8 = TileReads<D>::tr_off(lane, dq_ds, 1);
#pragma unroll
    for (int iu = 0; iu < DQ_NU; ++iu) {
      dso0[iu] = TileReads<64>::tr_off(lane, dq_u0 + iu, 0);
      dso8[iu] = TileReads<64>::tr_off(lane, dq_u0 + iu, 1);
    }
    // the K rows of the block into kt_lds, swizzled like every tile
    constexpr int RK = kBwdBlockK / T::RPR;  // 1 KiB runs
    const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(p.k + base, N * T::ROW);
    const int kgoff = run_goff<D>(wave_u % (16 / T::RPR), lane);
#pragma unroll
    for (int x = wave_u; x < RK; x += W)
      load_lds16(krsrc, kt_lds + x * 1024, kgoff + k0 * T::ROW + (x - wave_u % (16 / T::RPR)) * 1024);
  }

  const int first = CAUSAL ? k0 / BM : 0;  // query tiles before the block's first key see none of it
  // SPARSE: the kept query blocks in ascending order (causal: from the key
  // block's own on), compacted by wavefront 0 with a ballot over the mask column
  __shared__ uint16_t qblocks[SPARSE ? kSparseMaxBlocks : 1];
  int n_steps;
  if constexpr (SPARSE) {
    const uint8_t* col = p.block_mask + (size_t)(p.mask_heads == 1 ? 0 : bh) * p.mask_t * p.mask_t + kb;
    int count = 0;
    if (wave_u == 0) {
      for (int b0 = CAUSAL ? kb : 0; b0 < p.mask_t; b0 += 64) {
        const int qbk = b0 + lane;
        const int keep = qbk < p.mask_t ? (col[(size_t)qbk * p.mask_t] != 0) : 0;
        const uint64_t bal = __ballot(keep);
        const int pos = count + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (keep) qblocks[pos] = (uint16_t)qbk;
        count += __popcll(bal);
      }
    }
    __shared__ int qblock_count;
    if (threadIdx.x == 0) qblock_count = count;
    __syncthreads();
    n_steps = 2 * __builtin_amdgcn_readfirstlane(qblock_count);
  } else {
    n_steps = ceil_div(N, BM) - first;
  }
  // first query row of step s; at or past N for the steps past the last
  auto step_row = [&](int s) __attribute__((always_inline)) {
    if constexpr (SPARSE)
      return s < n_steps ? (int)__builtin_amdgcn_readfirstlane(qblocks[s >> 1]) * kSparseBlock + (s & 1) * BM : N;
    else
      return (first + s) * BM;
  };
  // Stage loads: wavefront w issues loads w, w + W, ... of the 2R runs (Q
  // runs first, then dO); the lane's offset is the same for all of them.
  const int x0 = wave_u % R;
  const int goff = run_goff<D>(x0, lane);
  // Stages past the last one are loaded all the same: their rows lie past N
  // and read as zeros into a buffer nobody reads again, and every step then
  // keeps the same number of loads in flight.
  auto issue_tile = [&](int s, auto buf, int i) __attribute__((always_inline)) {  // load i < PER of stage s
    constexpr int B = decltype(buf)::value;
    const int toff = step_row(s) * T::ROW;  // byte offset of the stage's first row
    const int x = wave_u + i * W;           // i < R / W exactly when x < R (W divides R)
    if (i * W < R)
      load_lds16(qrsrc, qbufs[B] + x * 1024, goff + toff + (x - x0) * 1024);
    else
      load_lds16(orsrc, obufs[B] + (x - R) * 1024, goff + toff + (x - R - x0) * 1024);
  };
  auto issue_ld = [&](int s, auto buf) __attribute__((always_inline)) {  // the stage's (L, D) pairs
    constexpr int B = decltype(buf)::value;
    if (wave_u == 0) load_lds4(lrsrc, lbufs[B], lane * 4 + step_row(s) * 8);
    if (wave_u == 1) load_lds4(lrsrc, lbufs[B] + 64, lane * 4 + step_row(s) * 8 + 256);
  };
  auto issue = [&](int s, auto buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER; ++i) issue_tile(s, buf, i);
    issue_ld(s, buf);
  };
  static_assert(R % W == 0, "a load's tensor does not depend on the wavefront");
  auto wait_stage = [&]() {  // own loads of the oldest stage in flight have landed
    if (FUSED)
      wait_vmcnt<0>();
    else if (wave_u <= 1)
      wait_vmcnt<PER + 1>();
    else
      wait_vmcnt<PER>();
  };

  f32x16_t dk[T::DSUB], dv[T::DSUB];
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds) dk[ds] = dv[ds] = f32x16_t{};
  const float c = p.scale_log2;

  // One step = the 64 query rows of a stage, as two 32-row sub-tiles u, in
  // four phases of 2·d/16 MFMAs each:
  //   A  S(0), dP(0)                     (S = Q Kᵀ, dP = dO Vᵀ; Q, dO rows from LDS)
  //   B  S(1), dP(1)   + softmax of u = 0 (P, dS as bf16 operands)
  //   C  dV, dK(0)     + softmax of u = 1 (dVᵀ += dOᵀ P, dKᵀ += Qᵀ dS; transpose reads)
  //   D  dV, dK(1)
  // With one wavefront per SIMD nothing else hides latency, so the order is
  // fixed by hand: each MFMA is followed by the LDS read of the operand it
  // needs LA (or LC) MFMAs later and by one element of the vector work, and
  // a scheduling fence after each such group keeps the compiler from
  // regrouping them.
  constexpr int LA = 6;  // 16-byte operand reads in flight in phases A and B
  constexpr int LC = 4;  // transpose-read operands in flight in phases C and D
  constexpr int NA = 2 * T::KS;    // MFMAs per sub-tile in A and B (S and dP, KS k-steps each)
  constexpr int NC = 4 * T::DSUB;  // MFMAs per sub-tile in C and D (dV and dK, 2 k-steps × DSUB)
  static_assert(16 % NA == 0 && 16 % NC == 0 && LA <= NA && LC <= NC, "phase shapes");
  f32x16_t sacc[2], dpacc[2];
  u32x4_t pw[4], sw[4];  // bf16 P and dS: the B operands of the four k-steps
  // issue_next(i): tile load i of the stage two steps ahead, one after each
  // of the first PER MFMAs (the matrix core keeps running while they issue)
  auto step_body = [&](const unsigned char* qb, const unsigned char* ob, const float* lb, int qs0,
                       auto masked, auto issue_next) __attribute__((always_inline)) {
    // operand j of A/B: sub-tile j / NA, k-step (j % NA) / 2, Q (even j) or dO (odd j)
    auto op_a = [&](int j) __attribute__((always_inline)) {
      return rd.rows((j & 1) ? ob : qb, (j % NA) >> 1, j / NA);
    };
    auto mfma_a = [&](int j, bf16x8_t a) __attribute__((always_inline)) {
      const int u = j / NA, kk = (j % NA) >> 1;
      if (j & 1)
        dpacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[kk], dpacc[u], 0, 0, 0);
      else
        sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[kk], sacc[u], 0, 0, 0);
    };
    // operand m of C/D: sub-tile u = m / NC, k-step 2u + (m % NC) / (2·DSUB),
    // d sub-tile (m / 2) % DSUB, dO for dV (even m) or Q for dK (odd m)
    auto op_c = [&](int m) __attribute__((always_inline)) {
      return rd.tr((m & 1) ? qb : ob, (m >> 1) % T::DSUB, 2 * (m / NC) + (m % NC) / (2 * T::DSUB));
    };
    auto mfma_c = [&](int m, bf16x8_t a) __attribute__((always_inline)) {
      const int kk = 2 * (m / NC) + (m % NC) / (2 * T::DSUB), ds = (m >> 1) % T::DSUB;
      if (m & 1)
        dk[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, sw[kk]), dk[ds], 0, 0, 0);
      else
        dv[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, pw[kk]), dv[ds], 0, 0, 0);
    };
    float4 ldq[2][8];  // (L·log2 e, D) of rows 32u + 8t + 4g + (0..3): t-th pair of float4
    auto read_ld = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ldq[u][2 * t] = *reinterpret_cast<const float4*>(lb + 2 * (32 * u + 8 * t + 4 * g));
        ldq[u][2 * t + 1] = *reinterpret_cast<const float4*>(lb + 2 * (32 * u + 8 * t + 4 * g + 2));
      }
    };
    float pr[2], dsr[2];
    // element r of sub-tile u (accumulator row 32u + 8(r/4) + 4g + r%4)
    auto soft_el = [&](int u, int r) __attribute__((always_inline)) {
      const float4 q4 = ldq[u][2 * (r >> 2) + ((r >> 1) & 1)];
      const float l2 = (r & 1) ? q4.z : q4.x, dd = (r & 1) ? q4.w : q4.y;
      float e = __builtin_amdgcn_exp2f(fmaf(sacc[u][r], c, -l2));
      if (decltype(masked)::value && key > qs0 + 32 * u + 8 * (r >> 2) + 4 * g + (r & 3)) e = 0.f;
      pr[r & 1] = e;
      dsr[r & 1] = e * (dpacc[u][r] - dd);
      if (r & 1) {
        pw[2 * u + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(pr[0], pr[1]);
        sw[2 * u + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(dsr[0], dsr[1]);
      }
    };

#pragma unroll
    for (int u = 0; u < 2; ++u) sacc[u] = dpacc[u] = f32x16_t{};
    bf16x8_t ra[LA], rc[LC];
    read_ld(0);
#pragma unroll
    for (int j = 0; j < LA; ++j) ra[j] = op_a(j);
    __builtin_amdgcn_sched_barrier(0);
    static_assert(PER <= NA, "the stage loads fit phase A");
#pragma unroll
    for (int j = 0; j < NA; ++j) {  // A
      mfma_a(j, ra[j % LA]);
      ra[j % LA] = op_a(j + LA);
      if (j < PER) issue_next(j);
      if (j == NA - 1) read_ld(1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = NA; j < 2 * NA; ++j) {  // B
      mfma_a(j, ra[j % LA]);
      if (j + LA < 2 * NA)
        ra[j % LA] = op_a(j + LA);
      else if (j + LA - 2 * NA < LC)
        rc[j + LA - 2 * NA] = op_c(j + LA - 2 * NA);
#pragma unroll
      for (int r = (j - NA) * (16 / NA); r < (j - NA + 1) * (16 / NA); ++r) soft_el(0, r);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < NC; ++m) {  // C
      mfma_c(m, rc[m % LC]);
      rc[m % LC] = op_c(m + LC);
#pragma unroll
      for (int r = m * (16 / NC); r < (m + 1) * (16 / NC); ++r) soft_el(1, r);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = NC; m < 2 * NC; ++m) {  // D
      mfma_c(m, rc[m % LC]);
      if (m + LC < 2 * NC) rc[m % LC] = op_c(m + LC);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (FUSED) {  // dS of the step into ds_lds: this lane's key row, 4 queries per write
      const int krow = 32 * wave_u + i32;
      unsigned char* rowp = ds_lds + krow * TS::ROW;
      const int sz = TS::swz(krow);
      // keys past N: their K rows read as zero, but P = exp(−L) there need not
      // be finite, so their dS is cleared rather than multiplied by zero
      const unsigned keep = key < N ? ~0u : 0u;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          *reinterpret_cast<u32x2_t*>(rowp + (((4 * u + t) ^ sz) << 4) + 8 * g) =
              u32x2_t{sw[2 * u + (t >> 1)][2 * (t & 1)] & keep, sw[2 * u + (t >> 1)][2 * (t & 1) + 1] & keep};
    }
  };
  // FUSED: dQ rows of step s_prev (64 queries × d) += dS K over the block's keys;
  // the wavefront takes 32 columns of d for both (d = 128) or one (d = 64) of
  // the 32-row halves, then adds them into the fp32 buffer.
  auto dq_phase = [&](int s_prev) __attribute__((always_inline)) {
    f32x16_t a2[DQ_NU];
#pragma unroll
    for (int iu = 0; iu < DQ_NU; ++iu) a2[iu] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < kBwdBlockK / 16; ++kk) {
      const bf16x8_t kb8 = TileReads<D>::tr_at(kt_lds, kt_o0, kt_o8, kk);
#pragma unroll
      for (int iu = 0; iu < DQ_NU; ++iu)
        a2[iu] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(TileReads<64>::tr_at(ds_lds, dso0[iu], dso8[iu], kk), kb8,
                                                         a2[iu], 0, 0, 0);
    }
    const int qs = step_row(s_prev);
    float* dst = p.dqacc + ((size_t)bh * N) * D + dq_ds * 32 + i32;
#pragma unroll
    for (int iu = 0; iu < DQ_NU; ++iu)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = qs + 32 * (dq_u0 + iu) + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row < N) __hip_atomic_fetch_add(dst + (size_t)row * D, a2[iu][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  };
  // CLEAN: every query of the step comes at or after every key of the block.
  auto step = [&](int s, auto buf, auto clean) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    const int qs0 = step_row(s);
    auto issue_next = [&](int i) __attribute__((always_inline)) {
      issue_tile(s + 2, std::integral_constant<int, (B + 2) % 3>{}, i);
    };
    // lane offsets opaque here: addresses are formed as offset + constant
#pragma unroll
    for (int kk = 0; kk < T::KS; ++kk) asm volatile("" : "+v"(rd.row[kk]));
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds) asm volatile("" : "+v"(rd.tr0[ds]), "+v"(rd.tr8[ds]));
    if (decltype(clean)::value) {
      step_body(qbufs[B], obufs[B], lbufs[B], qs0, std::false_type{}, issue_next);
    } else if (qs0 + BM - 1 >= kw) {  // else every query of the step precedes this wavefront's keys
      step_body(qbufs[B], obufs[B], lbufs[B], qs0, std::true_type{}, issue_next);
    } else {                          // ... (the stage loads are still this wavefront's share)
#pragma unroll
      for (int i = 0; i < PER; ++i) issue_next(i);
      if constexpr (FUSED) {          // ... and its dS rows are zero
        unsigned char* rowp = ds_lds + (32 * wave_u + i32) * TS::ROW;
#pragma unroll
        for (int x = 0; x < 8; ++x) *reinterpret_cast<u32x4_t*>(rowp + 16 * x) = u32x4_t{0, 0, 0, 0};
      }
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using Y = std::true_type;
  using G = std::false_type;
  issue(0, I0{});
  issue(1, I1{});
  wait_stage();
  // K and V were loaded before the stages, so they are in: settle the
  // compiler's load tracking for them once, outside the loop.
#pragma unroll
  for (int kk = 0; kk < T::KS; ++kk)
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, kf[kk])), "v"(__builtin_bit_cast(u32x4_t, vf[kk])));
  auto body = [&](int s, auto buf, auto clean) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    wait_stage();
    block_barrier();  // stage s is in LDS for everyone; stage s-1's buffers are free
    issue_ld(s + 2, std::integral_constant<int, (B + 2) % 3>{});  // its tiles: during the step
    if constexpr (FUSED) {
      if (s > 0) {
        dq_phase(s - 1);
        block_barrier();  // everyone has read dS of step s-1 before step s writes its own
      }
    }
    step(s, buf, clean);
  };
  auto loop = [&](int s0, auto phase) __attribute__((always_inline)) {
    constexpr int P = decltype(phase)::value;  // s0 mod 3
    for (int s = s0; s < n_steps; s += 3) {
      body(s, phase, Y{});
      if (s + 1 < n_steps) body(s + 1, std::integral_constant<int, (P + 1) % 3>{}, Y{});
      if (s + 2 < n_steps) body(s + 2, std::integral_constant<int, (P + 2) % 3>{}, Y{});
    }
  };
  if constexpr (CAUSAL) {
    // The block's keys are 128 from a multiple of 128, its steps 64 queries
    // from the first key on: the first two steps hold the diagonal (masked),
    // and from the third on every query follows every key of the block.
    // SPARSE: so when the diagonal block is kept (it is then the first);
    // otherwise every listed query follows every key of the block.
    static_assert(kBwdBlockK == 2 * BM, "two diagonal steps");
    if (!SPARSE || (n_steps > 0 && step_row(0) == k0)) {
      body(0, I0{}, G{});
      if (n_steps > 1) body(1, I1{}, G{});
      loop(2, I2{});
    } else {
      loop(0, I0{});
    }
  } else {
    loop(0, I0{});
  }
  if constexpr (FUSED) {
    wait_vmcnt<0>();
    block_barrier();  // dS of the last step is complete
    dq_phase(n_steps - 1);
  }

  // ---- epilogue: dK = scale · Σ dSᵀ Q, dV = Σ Pᵀ dO, one store each ------------------
  // staged in the Q and dO stage buffers, free once every wavefront is past
  // its last step and the loads past the last stage have landed: 32 rows ×
  // 2D bytes per region, two regions per buffer
  wait_vmcnt<0>();
  block_barrier();
  {
    constexpr int RG = 32 * T::ROW;
    static_assert(2 * RG == QT, "two staging regions per stage buffer");
    unsigned char* const kst = wave_u == 0 ? q_lds0 : wave_u == 1 ? q_lds0 + RG : wave_u == 2 ? q_lds1 : q_lds1 + RG;
    unsigned char* const vst = wave_u == 0 ? q_lds2 : wave_u == 1 ? q_lds2 + RG : wave_u == 2 ? o_lds0 : o_lds0 + RG;
    const int valid = min(32, N - kw);
    store_rows_staged<D>(dk, p.scale, kst, p.dk + base + (size_t)kw * D, valid, lane);
    store_rows_staged<D>(dv, 1.f, vst, p.dv + base + (size_t)kw * D, valid, lane);
  }
}

// ---- dK, dV by wavefront pairs: key blocks outside, query tiles inside ------------
// The same loop order as fa_bwd_dkdv_kernel ([15-779 L5] §7.4), with eight
// wavefronts, two per SIMD, so that one wavefront's waits are covered by the
// other's work.  The workgroup's 128 keys go to four pairs of 32; a pair's
// products are split so that each wavefront fits the 256 registers a lane
// has when two wavefronts share a SIMD:
// * the score wavefront (0-3) holds the pair's K and V rows and, per step of
//   64 queries, takes Sᵀ = K Qᵀ and dPᵀ = V dOᵀ with the query as the
//   accumulator column (Q and dO rows read from LDS; L and D are then one
//   pair of scalars per lane, loaded straight into registers), forms
//   P = exp(scale·S − L) and dS = P ∘ (dP − D) in fp32 and writes both as
//   bf16 to an LDS tile [query][key];
// * the gradient wavefront (4-7) holds dK and dV of the pair's keys and, one
//   step behind, adds dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS, every operand read with
//   the transpose load: dOᵀ and Qᵀ from the stage tiles, P and dS from the
//   pair's tiles.  Their 8-byte chunks are XOR-swizzled by (query row / 2)
//   mod 8: an 8-byte LDS write goes through in four passes of 16 consecutive
//   lanes over 32 four-byte banks (measured with the conflict counter), and
//   the score wavefront's 16 lanes of a pass write 16 rows, two per swizzle
//   value; the transpose reads stay conflict-free too.
// One barrier per step t: the score wavefronts take query tile t, the
// gradient wavefronts tile t − 1 and issue the direct loads of tile t + 1 into
// the buffers tile t − 2 has left (three stages of Q and dO, two of P and dS:
// 160 KiB of LDS at d = 128).  P and dS are rounded at the same point, from
// the same fp32 values, as in fa_bwd_dkdv_kernel.
constexpr int kBwdPairThreads = 512;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdPairThreads, 1) void fa_bwd_dkdv_pair_kernel(BwdParams p) {
  using T = BwdTile<D>;
  constexpr int BM = 64;            // query rows per step
  constexpr int QT = BM * T::ROW;   // bytes of one Q (or dO) stage
  constexpr int R = BM / T::RPR;    // direct loads per tensor per stage
  constexpr int NG = 4;             // gradient wavefronts; they issue the stage loads
  static_assert(R % NG == 0 && (NG * T::RPR) % 16 == 0, "stage loads spread evenly, one lane offset");
  constexpr int PER = 2 * R / NG;   // stage loads per gradient wavefront
  constexpr int XT = BM * 64;       // one P (or dS) tile: 64 queries × 32 keys, bf16
  static_assert(kBwdBlockK == 4 * 32, "four pairs of 32 keys");
  __shared__ __attribute__((aligned(16))) unsigned char q_lds0[QT], q_lds1[QT], q_lds2[QT];
  __shared__ __attribute__((aligned(16))) unsigned char o_lds0[QT], o_lds1[QT], o_lds2[QT];
  __shared__ __attribute__((aligned(16))) unsigned char x_lds[2 * 4 * 2 * XT];  // [step parity][pair][P, dS]
  unsigned char* const qbufs[3] = {q_lds0, q_lds1, q_lds2};
  unsigned char* const obufs[3] = {o_lds0, o_lds1, o_lds2};

  int bh, kb;
  decode_kblock(p, bh, kb);
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pair = wave_u & 3;
  const int i32 = lane & 31, g = lane >> 5, jj = lane & 15;
  const int k0 = kb * kBwdBlockK;
  const int kw = k0 + 32 * pair;  // first key of the pair
  const size_t base = (size_t)bh * N * D;
  const int first = CAUSAL ? k0 / BM : 0;  // query tiles before the block's first key see none of it
  const int n_steps = ceil_div(N, BM) - first;
  auto step_row = [&](int s) __attribute__((always_inline)) { return (first + s) * BM; };
  // causal: the block's first two steps hold the diagonal; a pair whose keys
  // all follow every query of a step skips it (both wavefronts alike)
  auto skipped = [&](int s) __attribute__((always_inline)) { return CAUSAL && step_row(s) + BM - 1 < kw; };
  unsigned char* const xpair = x_lds + pair * 2 * XT;  // + parity · 8·XT: P, then dS
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  if (wave_u < 4) {
    // ---------------- score wavefront ----------------
    const __amdgpu_buffer_rsrc_t lrsrc = make_rsrc(p.ld + (size_t)bh * N * 2, N * 8);
    bf16x8_t kf[T::KS], vf[T::KS];  // A operands: the K and V rows of key kw + i32
    {
      const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(p.k + base, N * T::ROW);
      const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.v + base, N * T::ROW);
#pragma unroll
      for (int kk = 0; kk < T::KS; ++kk) {
        kf[kk] = __builtin_bit_cast(bf16x8_t, buffer_load16(krsrc, (kw + i32) * T::ROW + (2 * kk + g) * 16));
        vf[kk] = __builtin_bit_cast(bf16x8_t, buffer_load16(vrsrc, (kw + i32) * T::ROW + (2 * kk + g) * 16));
      }
    }
    // (L·log2 e, D) of the lane's query in each 32-row half of a step
    float2 ldc[2], ldn[2];
    auto load_ld = [&](int s, float2(&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < 2; ++u) dst[u] = buffer_load8(lrsrc, (step_row(s) + 32 * u + i32) * 8);
    };
    load_ld(0, ldc);
    int row[T::KS];  // 16-byte row reads of Q and dO: row i32 (+32 per half), chunk 2kk + g
#pragma unroll
    for (int kk = 0; kk < T::KS; ++kk) row[kk] = i32 * T::ROW + (((2 * kk + g) ^ T::swz(i32)) << 4);
    int xw[4];  // P/dS writes: query row i32 (+32 per half), keys 8t + 4g .. +3
#pragma unroll
    for (int t = 0; t < 4; ++t) xw[t] = i32 * 64 + 8 * ((2 * t + g) ^ ((i32 >> 1) & 7));
    const float c = p.scale_log2;
    wait_vmcnt<0>();
    block_barrier();  // stage 0 is in

    auto score = [&](int s, auto buf, auto masked) __attribute__((always_inline)) {
      constexpr int B = decltype(buf)::value;
      constexpr bool MASKED = decltype(masked)::value;
      if (MASKED && skipped(s)) return;
      const unsigned char* qb = qbufs[B];
      const unsigned char* ob = obufs[B];
      unsigned char* const xp = xpair + (s & 1) * 8 * XT;
      unsigned char* const xs = xp + XT;
      const int qs0 = step_row(s);
#pragma unroll
      for (int kk = 0; kk < T::KS; ++kk) asm volatile("" : "+v"(row[kk]));
      constexpr int NA = 2 * T::KS;  // MFMAs per 32-query half (S and dP, KS k-steps each)
      constexpr int LA = 6;          // operand reads in flight
      static_assert(16 % NA == 0 && LA <= NA, "phase shapes");
      f32x16_t sacc[2], dpacc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) sacc[u] = dpacc[u] = f32x16_t{};
      // operand j: half j / NA, k-step (j % NA) / 2, a Q row (even j) or a dO row (odd j)
      auto op = [&](int j) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(((j & 1) ? ob : qb) + row[(j % NA) >> 1] +
                                                                             (j / NA) * 32 * T::ROW));
      };
      auto mfma = [&](int j, bf16x8_t b) __attribute__((always_inline)) {
        const int u = j / NA, kk = (j % NA) >> 1;
        if (j & 1)
          dpacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kk], b, dpacc[u], 0, 0, 0);
        else
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], b, sacc[u], 0, 0, 0);
      };
      // element r of half u: key kw + 8(r/4) + 4g + r%4, query qs0 + 32u + i32
      float pe[4], se[4];
      auto soft_el = [&](int u, int r) __attribute__((always_inline)) {
        float e = __builtin_amdgcn_exp2f(fmaf(sacc[u][r], c, -ldc[u].x));
        if (MASKED && kw + 8 * (r >> 2) + 4 * g + (r & 3) > qs0 + 32 * u + i32) e = 0.f;
        pe[r & 3] = e;
        se[r & 3] = e * (dpacc[u][r] - ldc[u].y);
        if ((r & 3) == 3) {
          const int o = u * 32 * 64 + xw[r >> 2];
          *reinterpret_cast<u32x2_t*>(xp + o) = u32x2_t{pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3])};
          *reinterpret_cast<u32x2_t*>(xs + o) = u32x2_t{pack_bf16x2(se[0], se[1]), pack_bf16x2(se[2], se[3])};
        }
      };
      bf16x8_t ra[LA];
#pragma unroll
      for (int j = 0; j < LA; ++j) ra[j] = op(j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NA; ++j) {  // S, dP of half 0
        mfma(j, ra[j % LA]);
        ra[j % LA] = op(j + LA);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = NA; j < 2 * NA; ++j) {  // S, dP of half 1 with P, dS of half 0
        mfma(j, ra[j % LA]);
        if (j + LA < 2 * NA) ra[j % LA] = op(j + LA);
#pragma unroll
        for (int r = (j - NA) * (16 / NA); r < (j - NA + 1) * (16 / NA); ++r) soft_el(0, r);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) soft_el(1, r);  // P, dS of half 1
    };
    auto phase = [&](int t, auto buf, auto masked) __attribute__((always_inline)) {
      load_ld(t + 1, ldn);
      if (t < n_steps) score(t, buf, masked);
      wait_vmcnt<0>();
      block_barrier();  // tile t + 1 is in; P and dS of tile t are complete
#pragma unroll
      for (int u = 0; u < 2; ++u) ldc[u] = ldn[u];
    };
    if (CAUSAL) {
      phase(0, I0{}, std::true_type{});
      phase(1, I1{}, std::true_type{});
    } else {
      phase(0, I0{}, std::false_type{});
      phase(1, I1{}, std::false_type{});
    }
    for (int t = 2; t <= n_steps; t += 3) {
      phase(t, I2{}, std::false_type{});
      if (t + 1 <= n_steps) phase(t + 1, I0{}, std::false_type{});
      if (t + 2 <= n_steps) phase(t + 2, I1{}, std::false_type{});
    }
    return;
  }

  // ---------------- gradient wavefront ----------------
  const int gw = wave_u - 4;
  const __amdgpu_buffer_rsrc_t qrsrc = make_rsrc(p.q + base, N * T::ROW);
  const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(p.dout + base, N * T::ROW);
  // Stage loads: gradient wavefront gw issues loads gw, gw + NG, ... of the 2R
  // runs (Q runs first, then dO); the lane's offset is the same for all of
  // them.  Stages past the last read zeros into a buffer nobody reads.
  const int x0 = gw % R;
  const int goff = run_goff<D>(x0, lane);
  auto issue = [&](int s, auto buf) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    const int toff = step_row(s) * T::ROW;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = gw + i * NG;
      if (i * NG < R)
        load_lds16(qrsrc, qbufs[B] + x * 1024, goff + toff + (x - x0) * 1024);
      else
        load_lds16(orsrc, obufs[B] + (x - R) * 1024, goff + toff + (x - R - x0) * 1024);
    }
  };
  int tr0[T::DSUB], tr8[T::DSUB];  // transpose reads of the stage tiles
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds) {
    tr0[ds] = TileReads<D>::tr_off(lane, ds, 0);
    tr8[ds] = TileReads<D>::tr_off(lane, ds, 1);
  }
  // transpose reads of a P/dS tile, k-step kk: rows 16kk + 4g + jj/4 (+8),
  // keys 16·((lane/16) mod 2) + 4·(jj mod 4) .. +3
  int xr[2];
#pragma unroll
  for (int pl = 0; pl < 2; ++pl)
    xr[pl] = (4 * g + (jj >> 2) + 8 * pl) * 64 + 8 * ((4 * ((lane >> 4) & 1) + (jj & 3)) ^ (2 * g + (jj >> 3) + 4 * pl));
  f32x16_t dk[T::DSUB], dv[T::DSUB];
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds) dk[ds] = dv[ds] = f32x16_t{};
  issue(0, I0{});
  wait_vmcnt<0>();
  block_barrier();  // stage 0 is in

  auto grad = [&](int s, auto buf, auto masked) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    if (decltype(masked)::value && skipped(s)) return;
    const unsigned char* qb = qbufs[B];
    const unsigned char* ob = obufs[B];
    const unsigned char* xp = xpair + (s & 1) * 8 * XT;
    const unsigned char* xs = xp + XT;
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds) asm volatile("" : "+v"(tr0[ds]), "+v"(tr8[ds]));
    constexpr int NC = 2 * T::DSUB;  // MFMAs per k-step (dV and dK of each 32-wide d sub-tile)
    constexpr int NM = 4 * NC;       // MFMAs per step (four k-steps of 16 queries)
    constexpr int LC = 4;            // operand reads in flight
    auto xop = [&](const unsigned char* x, int kk) __attribute__((always_inline)) {
      const u32x2_t a0 = lds_tr_read(x, xr[0] + kk * 16 * 64);
      const u32x2_t a1 = lds_tr_read(x, xr[1] + kk * 16 * 64);
      return __builtin_bit_cast(bf16x8_t, u32x4_t{a0[0], a0[1], a1[0], a1[1]});
    };
    // MFMA m: k-step m / NC, d sub-tile (m / 2) mod DSUB; dV (even m: dOᵀ, P) or dK (odd m: Qᵀ, dS)
    auto op = [&](int m) __attribute__((always_inline)) {
      return TileReads<D>::tr_at((m & 1) ? qb : ob, tr0[(m >> 1) % T::DSUB], tr8[(m >> 1) % T::DSUB], m / NC);
    };
    bf16x8_t pop[2], sop[2];  // B operands of the current and the next k-step
    bf16x8_t ra[LC];
    pop[0] = xop(xp, 0);
    sop[0] = xop(xs, 0);
#pragma unroll
    for (int m = 0; m < LC; ++m) ra[m] = op(m);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int kk = m / NC, ds = (m >> 1) % T::DSUB;
      if (m & 1)
        dk[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[m % LC], sop[kk & 1], dk[ds], 0, 0, 0);
      else
        dv[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[m % LC], pop[kk & 1], dv[ds], 0, 0, 0);
      if (m + LC < NM) ra[m % LC] = op(m + LC);
      if (m % NC == 0 && kk + 1 < 4) {
        pop[(kk + 1) & 1] = xop(xp, kk + 1);
        sop[(kk + 1) & 1] = xop(xs, kk + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto phase = [&](int t, auto buf, auto masked) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;  // t mod 3: tile t − 1 is in buffer B + 2, tile t + 1 goes to B + 1
    issue(t + 1, std::integral_constant<int, (B + 1) % 3>{});
    if (t >= 1) grad(t - 1, std::integral_constant<int, (B + 2) % 3>{}, masked);
    wait_vmcnt<0>();
    block_barrier();
  };
  if (CAUSAL) {
    phase(0, I0{}, std::true_type{});
    phase(1, I1{}, std::true_type{});
  } else {
    phase(0, I0{}, std::false_type{});
    phase(1, I1{}, std::false_type{});
  }
  for (int t = 2; t <= n_steps; t += 3) {
    phase(t, I2{}, std::false_type{});
    if (t + 1 <= n_steps) phase(t + 1, I0{}, std::false_type{});
    if (t + 2 <= n_steps) phase(t + 2, I1{}, std::false_type{});
  }

  // ---- epilogue: dK = scale · Σ dSᵀ Q, dV = Σ Pᵀ dO, staged in the (now free)
  // Q and dO stage buffers: region 2·gw for dK, 2·gw + 1 for dV
  {
    constexpr int RG = 32 * T::ROW;
    static_assert(2 * RG == QT, "two staging regions per stage buffer");
    unsigned char* const kst = gw == 0 ? q_lds0 : gw == 1 ? q_lds1 : gw == 2 ? q_lds2 : o_lds0;
    const int valid = min(32, N - kw);
    store_rows_staged<D>(dk, p.scale, kst, p.dk + base + (size_t)kw * D, valid, lane);
    store_rows_staged<D>(dv, 1.f, kst + RG, p.dv + base + (size_t)kw * D, valid, lane);
  }
}

// ---- dQ: query blocks outside, key/value tiles inside -----------------------------
__device__ inline void decode_qblock(const BwdParams& p, int& bh, int& qb) {
  const int x = blockIdx.x;
  if (p.xcd_remap_q) {  // whole heads per XCD; the heaviest blocks (last rows, when causal) first
    const int per_xcd = (p.BH * p.n_qblk) >> 3;
    const int heads_per_xcd = per_xcd / p.n_qblk;
    const int local = x >> 3;
    bh = (x & 7) * heads_per_xcd + local % heads_per_xcd;
    qb = p.n_qblk - 1 - local / heads_per_xcd;
  } else {
    bh = x % p.BH;
    qb = p.n_qblk - 1 - x / p.BH;
  }
}

// SPARSE: the workgroup's 256 rows span two mask rows; it lists the key
// blocks either of them keeps (as the block-sparse forward does) and each
// wavefront skips the tiles its own mask row drops.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(kFwdThreads, 1) void fa_bwd_dq_kernel(BwdParams p) {
  using T = BwdTile<D>;
  constexpr int BN = 64;              // keys per tile
  constexpr int KT = BN * T::ROW;     // bytes of one K (or V) stage
  constexpr int R = BN / T::RPR;      // direct loads per tensor per stage
  static_assert(2 * R % kFwdWaves == 0 && (kFwdWaves * T::RPR) % 16 == 0, "stage loads share one lane offset");
  constexpr int PER = 2 * R / kFwdWaves;
  __shared__ __attribute__((aligned(16))) unsigned char k_lds0[KT], k_lds1[KT], k_lds2[KT];
  __shared__ __attribute__((aligned(16))) unsigned char v_lds0[KT], v_lds1[KT], v_lds2[KT];
  unsigned char* const kbufs[3] = {k_lds0, k_lds1, k_lds2};
  unsigned char* const vbufs[3] = {v_lds0, v_lds1, v_lds2};

  int bh, qb;
  decode_qblock(p, bh, qb);
  const int N = p.N;
  const int lane = threadIdx.x & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i32 = lane & 31, g = lane >> 5;
  const int q0 = qb * kFwdBlockM;
  const int wq0 = q0 + 32 * wave_u;
  const int q_row = wq0 + i32;
  const size_t base = (size_t)bh * N * D;
  const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(p.k + base, N * T::ROW);
  const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(p.v + base, N * T::ROW);

  // Q and dO rows of this lane's query: the B operands of Sᵀ = K Qᵀ, dPᵀ = V dOᵀ.
  bf16x8_t qf[T::KS], of[T::KS];
  float2 ld;
  {
    const __amdgpu_buffer_rsrc_t qrsrc = make_rsrc(p.q + base, N * T::ROW);
    const __amdgpu_buffer_rsrc_t orsrc = make_rsrc(p.dout + base, N * T::ROW);
#pragma unroll
    for (int kk = 0; kk < T::KS; ++kk) {
      qf[kk] = __builtin_bit_cast(bf16x8_t, buffer_load16(qrsrc, q_row * T::ROW + (2 * kk + g) * 16));
      of[kk] = __builtin_bit_cast(bf16x8_t, buffer_load16(orsrc, q_row * T::ROW + (2 * kk + g) * 16));
    }
    if constexpr (SPARSE) {
      ld = buffer_load8(make_rsrc(p.ld + (size_t)bh * N * 2, N * 8), q_row * 8);
    } else {
      // (L·log2 e, D = dO·O) of this lane's row formed here and written to the
      // workspace for the dK/dV kernel, which runs after this one.  The per-row
      // kernel's arithmetic in its order — each 16-byte chunk's eight products
      // in turn, then the chunks pairwise at index distance 8, 4, 2, 1 (the lane
      // holds the even or the odd chunks) — so D is the same bit for bit as in
      // the backward forms that keep that kernel.
      const __amdgpu_buffer_rsrc_t o_rsrc = make_rsrc(p.o + base, N * T::ROW);
      float part[T::KS];
#pragma unroll
      for (int kk = 0; kk < T::KS; ++kk) {
        const u32x4_t o = buffer_load16(o_rsrc, q_row * T::ROW + (2 * kk + g) * 16);
        const u32x4_t d = __builtin_bit_cast(u32x4_t, of[kk]);
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a = fmaf(__uint_as_float(o[e] << 16), __uint_as_float(d[e] << 16), a);
          a = fmaf(__uint_as_float(o[e] & 0xffff0000u), __uint_as_float(d[e] & 0xffff0000u), a);
        }
        part[kk] = a;
      }
#pragma unroll
      for (int w = T::KS / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) part[i] = part[i] + part[i + w];
      const float lse = q_row < N ? p.lse[(size_t)bh * N + q_row] : 0.f;
      ld = make_float2(lse * 1.4426950408889634f, pair_sum(part[0]));
      if (g == 0 && q_row < N) reinterpret_cast<float2*>(p.ld)[(size_t)bh * N + q_row] = ld;
    }
  }

  TileReads<D> rd;
  rd.init(lane);

  // SPARSE: kept key blocks, bits 0-13 the block, bit 14 (15) set when the
  // first (second) mask row of the workgroup keeps it
  __shared__ uint16_t kblocks[SPARSE ? kSparseMaxBlocks : 1];
  int n_tiles;
  if constexpr (SPARSE) {
    static_assert(kSparseBlock == 2 * BN && kFwdBlockM == 2 * kSparseBlock, "two tiles per key block, two mask rows");
    const int rb0 = q0 / kSparseBlock;
    const bool two = rb0 + 1 < p.mask_t;
    const uint8_t* m0 = p.block_mask + ((size_t)(p.mask_heads == 1 ? 0 : bh) * p.mask_t + rb0) * p.mask_t;
    const int kb_end = CAUSAL ? min(p.mask_t, ceil_div(min(N, q0 + kFwdBlockM), kSparseBlock)) : p.mask_t;
    int count = 0;
    if (wave_u == 0) {
      for (int b0 = 0; b0 < kb_end; b0 += 64) {
        const int kbk = b0 + lane;
        const int k0b = kbk < kb_end ? (m0[kbk] != 0) : 0;
        const int k1b = (kbk < kb_end && two) ? (m0[p.mask_t + kbk] != 0) : 0;
        const uint64_t bal = __ballot(k0b | k1b);
        const int pos = count + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (k0b | k1b) kblocks[pos] = (uint16_t)(kbk | (k0b << 14) | (k1b << 15));
        count += __popcll(bal);
      }
    }
    __shared__ int kblock_count;
    if (threadIdx.x == 0) kblock_count = count;
    __syncthreads();
    n_tiles = 2 * __builtin_amdgcn_readfirstlane(kblock_count);
  } else {
    n_tiles = fwd_kv_tiles(N, D, CAUSAL, qb);
  }
  // first key of tile j (SPARSE: of the j-th tile of the kept blocks)
  auto tile_kv0 = [&](int j) __attribute__((always_inline)) {
    if constexpr (SPARSE)
      return (int)(__builtin_amdgcn_readfirstlane(kblocks[j >> 1]) & 0x3fff) * kSparseBlock + (j & 1) * BN;
    else
      return j * BN;
  };
  auto kept = [&](int j) __attribute__((always_inline)) {  // SPARSE: this wavefront's mask row keeps tile j
    if constexpr (SPARSE)
      return ((__builtin_amdgcn_readfirstlane(kblocks[j >> 1]) >> (14 + (wave_u >> 2))) & 1) != 0;
    else
      return true;
  };
  const int goff = run_goff<D>(wave_u % R, lane);
  // Tiles past the last are loaded all the same, from past the end of K and V
  // (zeros, no memory traffic) into a buffer nobody reads again, and every
  // step then keeps the same number of loads in flight.
  auto issue_tile = [&](int j, auto buf, int i) __attribute__((always_inline)) {  // load i < PER of tile j
    constexpr int B = decltype(buf)::value;
    const int toff = j < n_tiles ? tile_kv0(j) * T::ROW : N * T::ROW;  // byte offset of the tile's first row
    const int x = wave_u + i * kFwdWaves;  // i < R / 8 exactly when x < R (8 divides R)
    if (i * kFwdWaves < R)
      load_lds16(krsrc, kbufs[B] + x * 1024, goff + toff + (x - wave_u % R) * 1024);
    else
      load_lds16(vrsrc, vbufs[B] + (x - R) * 1024, goff + toff + (x - R - wave_u % R) * 1024);
  };
  static_assert(R % kFwdWaves == 0, "a load's tensor does not depend on the wavefront");
  auto issue = [&](int j, auto buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PER; ++i) issue_tile(j, buf, i);
  };
  auto wait_stage = [&]() { wait_vmcnt<PER>(); };  // the oldest tile in flight has landed

  f32x16_t dq[T::DSUB];
#pragma unroll
  for (int ds = 0; ds < T::DSUB; ++ds) dq[ds] = f32x16_t{};
  const float c = p.scale_log2;
  const int lim = CAUSAL ? min(q_row, N - 1) : N - 1;  // last key this row sees

  // CLEAN: every row of the workgroup sees every key of the tile (no mask, no skip)
  // issue_next(i): load i of the tile two steps ahead, one after each of the
  // first PER MFMAs of a clean step (before the step otherwise)
  auto step = [&](int j, auto buf, auto clean) __attribute__((always_inline)) {
    constexpr int B = decltype(buf)::value;
    constexpr bool CLEAN = decltype(clean)::value;
    auto issue_next = [&](int i) __attribute__((always_inline)) {
      issue_tile(j + 2, std::integral_constant<int, (B + 2) % 3>{}, i);
    };
    const int kv0 = tile_kv0(j);
    if (!CLEAN) {  // tiles with a mask or a skip: the loads go out first
#pragma unroll
      for (int i = 0; i < PER; ++i) issue_next(i);
      if (CAUSAL && kv0 > wq0 + 31) return;  // the tile lies wholly after this wavefront's rows
      if (!kept(j)) return;                  // SPARSE: this wavefront's mask row drops it
    }
    const unsigned char* kb = kbufs[B];
    const unsigned char* vb = vbufs[B];
    // lane offsets opaque here: addresses are formed as offset + constant
#pragma unroll
    for (int kk = 0; kk < T::KS; ++kk) asm volatile("" : "+v"(rd.row[kk]));
#pragma unroll
    for (int ds = 0; ds < T::DSUB; ++ds) asm volatile("" : "+v"(rd.tr0[ds]), "+v"(rd.tr8[ds]));
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) s[sub] = dp[sub] = f32x16_t{};
    const bool edge = !CLEAN && ((kv0 + BN > N) || (CAUSAL && kv0 + BN - 1 > wq0));
    // A: S, dP of key sub-tile 0; B: those of sub-tile 1 with the vector work of
    // sub-tile 0; C: dQ of sub-tile 0's keys with that of sub-tile 1; D: the rest
    constexpr int NA = 2 * T::KS;      // MFMAs of S and dP per 32-key sub-tile
    constexpr int NC = 2 * T::DSUB;    // dQ MFMAs per 32 keys (two k-steps)
    constexpr int LA = SPARSE ? 3 : 4, LC = 2;  // SPARSE: one read fewer in flight (registers)
    auto op_a = [&](int j2) __attribute__((always_inline)) {  // j2: sub-tile j2 / NA, k-step (j2 % NA) / 2, K or V
      return rd.rows((j2 & 1) ? vb : kb, (j2 % NA) >> 1, j2 / NA);
    };
    auto mfma_a = [&](int j2, bf16x8_t a) __attribute__((always_inline)) {
      const int sub = j2 / NA, kk = (j2 % NA) >> 1;
      if (j2 & 1)
        dp[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, of[kk], dp[sub], 0, 0, 0);
      else
        s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[sub], 0, 0, 0);
    };
    u32x4_t sw[4];
    float dsr2[2];
    auto soft_el = [&](int sub, int r) __attribute__((always_inline)) {
      float e = __builtin_amdgcn_exp2f(fmaf(s[sub][r], c, -ld.x));
      if (edge && kv0 + sub * 32 + 8 * (r >> 2) + 4 * g + (r & 3) > lim) e = 0.f;
      dsr2[r & 1] = e * (dp[sub][r] - ld.y);
      if (r & 1) sw[2 * sub + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(dsr2[0], dsr2[1]);
    };
    auto op_c = [&](int m) __attribute__((always_inline)) {  // m: k-step m / DSUB, d sub-tile m % DSUB
      return rd.tr(kb, m % T::DSUB, m / T::DSUB);
    };
    auto mfma_c = [&](int m, bf16x8_t a) __attribute__((always_inline)) {
      dq[m % T::DSUB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, sw[m / T::DSUB]),
                                                              dq[m % T::DSUB], 0, 0, 0);
    };
    bf16x8_t ra[LA], rc[LC];
#pragma unroll
    for (int t = 0; t < LA; ++t) ra[t] = op_a(t);
    __builtin_amdgcn_sched_barrier(0);
    static_assert(PER <= NA, "the tile loads fit phase A");
#pragma unroll
    for (int t = 0; t < NA; ++t) {  // A
      mfma_a(t, ra[t % LA]);
      ra[t % LA] = op_a(t + LA);
      if (CLEAN && t < PER) issue_next(t);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = NA; t < 2 * NA; ++t) {  // B
      mfma_a(t, ra[t % LA]);
      if (t + LA < 2 * NA)
        ra[t % LA] = op_a(t + LA);
      else if (t + LA - 2 * NA < LC)
        rc[t + LA - 2 * NA] = op_c(t + LA - 2 * NA);
#pragma unroll
      for (int r = (t - NA) * (16 / NA); r < (t - NA + 1) * (16 / NA); ++r) soft_el(0, r);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int m = 0; m < 2 * NC; ++m) {  // C and D
      mfma_c(m, rc[m % LC]);
      if (m + LC < 2 * NC) rc[m % LC] = op_c(m + LC);
      if (m < NC) {
#pragma unroll
        for (int r = m * (16 / NC); r < (m + 1) * (16 / NC); ++r) soft_el(1, r);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  issue(0, I0{});
  issue(1, I1{});
  wait_stage();
#pragma unroll
  for (int kk = 0; kk < T::KS; ++kk)
    asm volatile("" ::"v"(__builtin_bit_cast(u32x4_t, qf[kk])), "v"(__builtin_bit_cast(u32x4_t, of[kk])));
  asm volatile("" ::"v"(ld.x), "v"(ld.y));
  auto body = [&](int j, auto buf, auto clean) __attribute__((always_inline)) {
    wait_stage();
    block_barrier();  // tile j is in LDS for everyone; tile j-1's buffers are free
    step(j, buf, clean);
  };
  using Y = std::true_type;
  using G = std::false_type;
  // tiles 0 .. n_clean-1 are whole and before the diagonal of every row of the block
  const int n_clean = SPARSE ? 0 : CAUSAL ? min(N / BN, (q0 + 1) / BN) : N / BN;
  int j = 0;
  for (; j + 3 <= n_clean; j += 3) {
    body(j, I0{}, Y{});
    body(j + 1, I1{}, Y{});
    body(j + 2, I2{}, Y{});
  }
  for (; j < n_tiles; j += 3) {
    body(j, I0{}, G{});
    if (j + 1 < n_tiles) body(j + 1, I1{}, G{});
    if (j + 2 < n_tiles) body(j + 2, I2{}, G{});
  }

  // dQ staged in the K/V stage buffers (free once every wavefront is past its
  // last tile and the loads past the last tile have landed), two 32-row
  // regions per buffer
  wait_vmcnt<0>();
  block_barrier();
  {
    constexpr int RG = 32 * T::ROW;
    static_assert(2 * RG == KT, "two staging regions per stage buffer");
    unsigned char* const st = wave_u == 0 ? k_lds0 : wave_u == 1 ? k_lds0 + RG : wave_u == 2 ? k_lds1
                            : wave_u == 3 ? k_lds1 + RG : wave_u == 4 ? k_lds2 : wave_u == 5 ? k_lds2 + RG
                            : wave_u == 6 ? v_lds0 : v_lds0 + RG;
    if (wq0 < N) store_rows_staged<D>(dq, p.scale, st, p.dq + base + (size_t)wq0 * D, min(32, N - wq0), lane);
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  const long long rows = (long long)p.BH * p.N;
  if (!p.block_mask && !p.dqacc) {
    // the default form: the dQ kernel forms the per-row (L, D) itself and
    // writes them for the dK/dV kernel, which therefore runs second
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, false>), dim3(p.BH * p.n_qblk), dim3(kFwdThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    static const hipError_t pattr = allow_full_lds(&fa_bwd_dkdv_pair_kernel<D, CAUSAL>);
    if (pattr != hipSuccess) return pattr;
    hipLaunchKernelGGL((fa_bwd_dkdv_pair_kernel<D, CAUSAL>), dim3(p.BH * p.n_kblk), dim3(kBwdPairThreads), 0, stream,
                       p);
    return hipGetLastError();
  }
  const int rows_per_block = 256 / (D / 8);
  hipLaunchKernelGGL((fa_bwd_prep_kernel<D>), dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)), dim3(256),
                     0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.block_mask) {
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, false, true>), dim3(p.BH * p.n_kblk), dim3(kBwdKvThreads), 0,
                       stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, true>), dim3(p.BH * p.n_qblk), dim3(kFwdThreads), 0, stream, p);
    return hipGetLastError();
  }
  static const hipError_t attr = allow_full_lds(&fa_bwd_dkdv_kernel<D, CAUSAL, true, false>);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, true, false>), dim3(p.BH * p.n_kblk), dim3(kBwdKvThreads), 0,
                     stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n8 = rows * D / 8;
  hipLaunchKernelGGL((fa_bwd_dq_finish_kernel<D>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, int causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_bwd_t<64, true>(p, stream) : launch_bwd_t<64, false>(p, stream);
  return causal ? launch_bwd_t<128, true>(p, stream) : launch_bwd_t<128, false>(p, stream);
}

}  // namespace fa
