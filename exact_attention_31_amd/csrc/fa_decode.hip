// Split-KV decode for CDNA4 (gfx950): one new query per (b, query head)
// against the cached keys of its sequence.
//
// Decode has one query row per sequence, so a grid over (b, h) alone leaves
// most compute units idle; the keys are therefore split into S segments, each
// segment is reduced by its own workgroup to a partial (O_s, LSE_s), and a
// small second kernel re-weights the partials by their LSE ([15-779 L5] §8.4,
// Flash-Decoding).  Re-weighting is the ⊕ merge of (m, ℓ, o) summaries, which
// is associative and commutative ([15-779 L5] §4.4–4.5), so the split count
// does not change the result beyond rounding.
//
// Grouped queries ([15-779 L5] §12, exercise 7): g = Hq/Hkv query heads share
// one K/V head (g = 1: multi-head; Hkv = 1: multi-query).  A workgroup serves
// GQ of the g query heads of its K/V head, so every K/V byte it streams feeds
// GQ dot products and GQ accumulators: the arithmetic intensity rises by GQ.
// Sequences may hold fewer keys than the cache's row count (per-sequence
// lengths); each sequence's keys are split into its own S segments, and a
// segment left empty (a sequence shorter than S) contributes weight 0.
//
// Pages cited: [15-779 L5] "第 5 讲 · 案例：Transformer、注意力与 FlashAttention".
//
// The work is a stream of K and V (a few multiply-adds per byte pair), so it
// is bound by HBM bandwidth ([15-779 L5] §8.3): the kernel reads each key row
// with 16-byte loads by d/8 adjacent lanes (a wavefront instruction covers
// 1 KiB of contiguous cache), keeps several such loads of K and of V in
// flight per lane, marks them nontemporal (every cached byte is read exactly
// once per call, so it should not displace other lines: 7-8 % more bandwidth
// than plain loads on this chip), and does the arithmetic on the vector ALUs — q·k as
// bf16-pair dot products (v_dot2_f32_bf16) summed across the d/8 lanes of a
// row on the DPP lane network, P̃·v in fp32 — as a matrix-core formulation
// would not help a matrix-vector product.
//
// Lane roles inside a wavefront: lane = slot·(d/8) + chunk; `chunk` selects 8
// dims of the row, `slot` selects one of 64/(d/8) keys per instruction.  Each
// slot keeps its own running (m, ℓ, o[8]) per query over the keys it sees;
// the slots, then the 4 wavefronts, are merged with ⊕ at the end of the
// segment.

#include <hip/hip_runtime.h>

#include <mutex>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
// wavefront instructions of K (and of V) in flight per lane: fewer when each
// key feeds more queries (more registers per key, more arithmetic per byte)
__host__ __device__ constexpr int dec_unroll(int gq) { return gq >= 8 ? 4 : 8; }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Σ over the `lanes` adjacent lanes (a power of two, at most 16, aligned) that
// share a key row, left in every one of them: butterfly steps on the DPP lane
// network (quad permutations, then mirrors within 8 and 16 lanes), each a
// plain vector add with a permuted operand — no LDS crossbar round trip.
template <int lanes>
__device__ inline float row_sum(float t) {
  t += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0xB1, 0xF, 0xF, true));   // [1,0,3,2]
  if (lanes > 2)
    t += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0x4E, 0xF, 0xF, true)); // [2,3,0,1]
  if (lanes > 4)
    t += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0x141, 0xF, 0xF, true)); // half mirror
  if (lanes > 8)
    t += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, t), 0x140, 0xF, 0xF, true)); // mirror
  return t;
}

__device__ inline uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// exp2 scale of a max that may still be -inf (no key seen yet): such a
// summary carries weight exactly 0 after the merge.
__device__ inline float safe_mc(float m, float c) { return m == -INFINITY ? 0.f : m * c; }

// Paged K/V (PAGED): the cache is a pool of pages, page × K/V head holding
// 2^page_shift consecutive keys; a sequence's keys follow its row of the block
// table.  The workgroup copies the page numbers of its segment into LDS
// (clamped into the pool) in chunks of kPageChunk and maps each key to its row
// through them; the streaming and the arithmetic are unchanged.
constexpr int kPageChunk = 1024;

template <int D, int GQ, bool PAGED>
__global__ __launch_bounds__(kDecThreads) void fa_decode_split_kernel(DecodeParams p) {
  constexpr int LPK = D / 8;        // lanes per key row
  constexpr int KPI = 64 / LPK;     // keys per wavefront instruction
  constexpr int STEP = kDecWaves * KPI;
  constexpr int UNR = dec_unroll(GQ);

  // workgroup -> (segment s, query group qg of K/V head (b, hk))
  const int s = blockIdx.x % p.S;   // consecutive workgroups walk one head's segments
  const int rest = blockIdx.x / p.S;
  const int n_qg = p.G / GQ;
  const int qg = rest % n_qg;
  const int bk = rest / n_qg;       // b·Hkv + hk
  const int b = bk / p.Hkv;
  const int hq0 = (bk % p.Hkv) * p.G + qg * GQ;  // first of the GQ query heads
  const size_t bq0 = (size_t)b * p.Hq + hq0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = lane % LPK;
  const int slot = lane / LPK;
  int len = p.L;
  if (p.seqlens) {
    const int x = p.seqlens[b];
    len = x < 1 ? 1 : (x > p.L ? p.L : x);
  }
  const int k_begin = (int)(((long long)s * len) / p.S);
  const int k_end = (int)(((long long)(s + 1) * len) / p.S);
  const float c = p.scale_log2;

  // q stays in bf16 pairs: q·k takes one v_dot2_f32_bf16 per pair of dims
  uint32_t qw[GQ][4];
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p.q + (bq0 + i) * D + chunk * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) qw[i][e] = w[e];
  }
  // row r of the (b, K/V head) cache, or of the page pool when PAGED
  const uint16_t* __restrict__ kb = p.k + (PAGED ? 0 : (size_t)bk * p.L * D) + chunk * 8;
  const uint16_t* __restrict__ vb = p.v + (PAGED ? 0 : (size_t)bk * p.L * D) + chunk * 8;

  float m[GQ], l[GQ], acc[GQ][8];
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }

  __shared__ int page_row[PAGED ? kPageChunk : 1];  // first pool row of each page of the chunk
  const int hk = bk % p.Hkv;
  // keys [c_begin, c_end) of the segment; PAGED: pages from page0 on are in page_row
  auto run = [&](int c_begin, int c_end, int page0) __attribute__((always_inline)) {
  for (int k0 = c_begin; k0 < c_end; k0 += UNR * STEP) {
    u32x4_t kr[UNR], vr[UNR];
    int key[UNR];
    size_t row[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      key[u] = k0 + (u * kDecWaves + wave) * KPI + slot;
      if (PAGED)
        row[u] = key[u] < c_end ? (size_t)page_row[(key[u] >> p.page_shift) - page0] + (key[u] & ((1 << p.page_shift) - 1)) : 0;
      else
        row[u] = (size_t)key[u];
      kr[u] = key[u] < c_end ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kb + row[u] * D)) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      vr[u] = key[u] < c_end ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vb + row[u] * D)) : u32x4_t{0, 0, 0, 0};

#pragma unroll
    for (int i = 0; i < GQ; ++i) {
      float sc[UNR];
      float bm = -INFINITY;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          t = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qw[i][e]),
                                              __builtin_bit_cast(bf16x2_t, (uint32_t)kr[u][e]), t, false);
        t = row_sum<LPK>(t);
        sc[u] = key[u] < c_end ? t : -INFINITY;
        bm = fmaxf(bm, sc[u]);
      }
      const float m_new = fmaxf(m[i], bm);
      const float mc = safe_mc(m_new, c);
      const float alpha = __builtin_amdgcn_exp2f(m[i] * c - mc);
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] *= alpha;
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const float pu = __builtin_amdgcn_exp2f(fmaf(sc[u], c, -mc));
        l[i] += pu;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[i][2 * e] = fmaf(pu, bf_lo(vr[u][e]), acc[i][2 * e]);
          acc[i][2 * e + 1] = fmaf(pu, bf_hi(vr[u][e]), acc[i][2 * e + 1]);
        }
      }
      m[i] = m_new;
    }
  }
  };
  if (!PAGED) {
    run(k_begin, k_end, 0);
  } else if (k_end > k_begin) {
    const int sh = p.page_shift;
    const int first_page = k_begin >> sh, last_page = (k_end - 1) >> sh;
    const int* tbl = p.block_table + (size_t)b * p.max_pages;
    for (int pc = first_page; pc <= last_page; pc += kPageChunk) {
      const int np = min(kPageChunk, last_page - pc + 1);
      __syncthreads();  // the previous chunk's rows are no longer read
      for (int i = tid; i < np; i += kDecThreads) {
        int pg = tbl[pc + i];
        pg = pg < 0 ? 0 : (pg >= p.num_pages ? p.num_pages - 1 : pg);
        page_row[i] = (pg * p.Hkv + hk) << sh;
      }
      __syncthreads();
      run(max(k_begin, pc << sh), min(k_end, (pc + np) << sh), pc);
    }
  }

  // ⊕-merge the slots of this wavefront (lanes that share a chunk).
#pragma unroll
  for (int i = 0; i < GQ; ++i) {
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m[i], off);
      const float l2 = __shfl_xor(l[i], off);
      const float mm = fmaxf(m[i], m2);
      const float mmc = safe_mc(mm, c);
      const float fa = __builtin_amdgcn_exp2f(m[i] * c - mmc);
      const float fb = __builtin_amdgcn_exp2f(m2 * c - mmc);
      l[i] = l[i] * fa + l2 * fb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a2 = __shfl_xor(acc[i][e], off);
        acc[i][e] = acc[i][e] * fa + a2 * fb;
      }
      m[i] = mm;
    }
  }

  // ⊕-merge the wavefronts through LDS and write the segment's (O_s, LSE_s);
  // an empty segment (a sequence shorter than S) writes O_s = 0, LSE_s = -inf.
  __shared__ float sm_m[GQ][kDecWaves], sm_l[GQ][kDecWaves];
  __shared__ float sm_o[GQ][kDecWaves][D];
  if (slot == 0) {
#pragma unroll
    for (int i = 0; i < GQ; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sm_o[i][wave][chunk * 8 + e] = acc[i][e];
      if (chunk == 0) {
        sm_m[i][wave] = m[i];
        sm_l[i][wave] = l[i];
      }
    }
  }
  __syncthreads();
  for (int x = tid; x < GQ * D; x += kDecThreads) {
    const int i = x / D, dd = x % D;
    float M = sm_m[i][0];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, sm_m[i][w]);
    const float Mc = safe_mc(M, c);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm_m[i][w] * c - Mc);
      L = fmaf(sm_l[i][w], f, L);
      o = fmaf(sm_o[i][w][dd], f, o);
    }
    const size_t part = (bq0 + i) * p.S + s;
    const bool empty = !(L > 0.f);
    p.part_o[part * D + dd] = empty ? 0.f : o / L;
    if (dd == 0) p.part_lse[part] = empty ? -INFINITY : M * p.scale + __builtin_amdgcn_logf(L) * 0.69314718055994531f;
  }
}

// O = Σ_s w_s O_s / Σ_s w_s and LSE = M + ln Σ_s w_s with w_s = exp(LSE_s − M),
// M = max_s LSE_s: the ⊕ merge written on normalised partials (an empty
// segment has LSE_s = -inf, weight 0, and O_s = 0).  One workgroup per
// (b, query head): the max over segments is a block reduction, then
// groups of threads take interleaved segments (16-byte loads of O_s, d/4
// threads per segment) and the groups' partial sums meet in LDS.
constexpr int kCombThreads = 256;

template <int D>
__global__ __launch_bounds__(kCombThreads) void fa_decode_combine_kernel(DecodeParams p) {
  constexpr int C4 = D / 4;                    // float4 chunks per partial row
  constexpr int G = kCombThreads / C4;         // segment groups
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  __shared__ float red[kCombThreads / 64];
  __shared__ f32x4_t part[G][C4];
  __shared__ float wsum[G];

  const int bh = blockIdx.x;  // b·Hq + query head
  const int t = threadIdx.x;
  const float* __restrict__ pl = p.part_lse + (size_t)bh * p.S;
  const f32x4_t* __restrict__ po = reinterpret_cast<const f32x4_t*>(p.part_o + (size_t)bh * p.S * D);

  float mx = -INFINITY;
  for (int s = t; s < p.S; s += kCombThreads) mx = fmaxf(mx, pl[s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kCombThreads / 64; ++w) M = fmaxf(M, red[w]);

  const int c = t % C4, gi = t / C4;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  for (int s = gi; s < p.S; s += G) {
    const float w = __builtin_amdgcn_exp2f((pl[s] - M) * 1.4426950408889634f);
    W += w;
    o += w * po[(size_t)s * C4 + c];
  }
  part[gi][c] = o;
  if (c == 0) wsum[gi] = W;
  __syncthreads();
  if (t < C4) {
    f32x4_t sum = part[0][t];
    float Wt = wsum[0];
#pragma unroll
    for (int q = 1; q < G; ++q) {
      sum += part[q][t];
      Wt += wsum[q];
    }
    const float inv = 1.f / Wt;
    uint32_t w0 = (uint32_t)to_bf16(sum[0] * inv) | ((uint32_t)to_bf16(sum[1] * inv) << 16);
    uint32_t w1 = (uint32_t)to_bf16(sum[2] * inv) | ((uint32_t)to_bf16(sum[3] * inv) << 16);
    *reinterpret_cast<u32x2_t*>(p.o + (size_t)bh * D + 4 * t) = u32x2_t{w0, w1};
    if (t == 0) p.lse[bh] = M + __builtin_amdgcn_logf(Wt) * 0.69314718055994531f;
  }
}

template <int D, int GQ>
hipError_t launch_decode_t(const DecodeParams& p, int B, hipStream_t stream) {
  const long long groups = (long long)B * p.Hkv * (p.G / GQ);
  if (p.block_table)
    hipLaunchKernelGGL((fa_decode_split_kernel<D, GQ, true>), dim3((unsigned)(groups * p.S)), dim3(kDecThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((fa_decode_split_kernel<D, GQ, false>), dim3((unsigned)(groups * p.S)), dim3(kDecThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fa_decode_combine_kernel<D>, dim3(B * p.Hq), dim3(kCombThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& p, int B, hipStream_t stream) {
  switch (decode_group_width(p.G)) {
    case 8: return launch_decode_t<D, 8>(p, B, stream);
    case 4: return launch_decode_t<D, 4>(p, B, stream);
    case 2: return launch_decode_t<D, 2>(p, B, stream);
    default: return launch_decode_t<D, 1>(p, B, stream);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int B, int d, hipStream_t stream) {
  return d == 64 ? launch_decode_d<64>(p, B, stream) : launch_decode_d<128>(p, B, stream);
}

// Scratch of the allocation-free decode call (fa_decode_noalloc): the split
// partials live in this file-scope device array, one copy per GPU, held until
// the process ends.  In host code the name stands for a host-side shadow, not
// a device address; the device address is looked up once per device with
// hipGetSymbolAddress and kept.
static __device__ __attribute__((aligned(256))) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!dev_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
