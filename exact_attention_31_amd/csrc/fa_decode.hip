// Split-KV decode for CDNA4 (gfx950): one query per (b, h) against Lkv keys.
//
// Decode has one query row per sequence, so a grid over (b, h) alone leaves
// most compute units idle; the keys are therefore split into S segments, each
// segment is reduced by its own workgroup to a partial (O_s, LSE_s), and a
// small second kernel re-weights the partials by their LSE ([15-779 L5] §8.4,
// Flash-Decoding).  Re-weighting is the ⊕ merge of (m, ℓ, o) summaries, which
// is associative and commutative ([15-779 L5] §4.4–4.5), so the split count
// does not change the result beyond rounding.
//
// Pages cited: [15-779 L5] "第 5 讲 · 案例：Transformer、注意力与 FlashAttention".
//
// The work is a pure stream of K and V (one multiply-add per byte pair), so it
// is bound by HBM bandwidth ([15-779 L5] §8.3): the kernel reads each key row
// with 16-byte loads by d/8 adjacent lanes (a wavefront instruction covers
// 1 KiB of contiguous cache), keeps eight such loads of K and eight of V in
// flight per lane, and does the arithmetic in fp32 on the vector ALUs —
// a matrix-core formulation would not help a matrix-vector product.
//
// Lane roles inside a wavefront: lane = slot·(d/8) + chunk; `chunk` selects 8
// dims of the row, `slot` selects one of 64/(d/8) keys per instruction.  Each
// slot keeps its own running (m, ℓ, o[8]) over the keys it sees; the slots,
// then the 4 wavefronts, are merged with ⊕ at the end of the segment.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kUnroll = 8;  // wavefront instructions of K (and of V) in flight per lane

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// exp2 scale of a max that may still be -inf (no key seen yet): such a
// summary carries weight exactly 0 after the merge.
__device__ inline float safe_mc(float m, float c) { return m == -INFINITY ? 0.f : m * c; }

template <int D>
__global__ __launch_bounds__(kDecThreads) void fa_decode_split_kernel(DecodeParams p) {
  constexpr int LPK = D / 8;        // lanes per key row
  constexpr int KPI = 64 / LPK;     // keys per wavefront instruction
  constexpr int STEP = kDecWaves * KPI;

  const int s = blockIdx.x % p.S;   // consecutive workgroups walk one head's segments
  const int bh = blockIdx.x / p.S;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = lane % LPK;
  const int slot = lane / LPK;
  const int k_begin = (int)(((long long)s * p.L) / p.S);
  const int k_end = (int)(((long long)(s + 1) * p.L) / p.S);
  const float c = p.scale_log2;

  float qf[8];
  {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p.q + (size_t)bh * D + chunk * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[2 * e] = bf_lo(w[e]);
      qf[2 * e + 1] = bf_hi(w[e]);
    }
  }
  const uint16_t* __restrict__ kb = p.k + (size_t)bh * p.L * D + chunk * 8;
  const uint16_t* __restrict__ vb = p.v + (size_t)bh * p.L * D + chunk * 8;

  float m = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;

  for (int k0 = k_begin; k0 < k_end; k0 += kUnroll * STEP) {
    u32x4_t kr[kUnroll], vr[kUnroll];
    int key[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      key[u] = k0 + (u * kDecWaves + wave) * KPI + slot;
      kr[u] = key[u] < k_end ? *reinterpret_cast<const u32x4_t*>(kb + (size_t)key[u] * D) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      vr[u] = key[u] < k_end ? *reinterpret_cast<const u32x4_t*>(vb + (size_t)key[u] * D) : u32x4_t{0, 0, 0, 0};

    float sc[kUnroll];
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t = fmaf(qf[2 * e], bf_lo(kr[u][e]), t);
        t = fmaf(qf[2 * e + 1], bf_hi(kr[u][e]), t);
      }
#pragma unroll
      for (int off = 1; off < LPK; off <<= 1) t += __shfl_xor(t, off);
      sc[u] = key[u] < k_end ? t : -INFINITY;
      bm = fmaxf(bm, sc[u]);
    }
    const float m_new = fmaxf(m, bm);
    const float mc = safe_mc(m_new, c);
    const float alpha = __builtin_amdgcn_exp2f(m * c - mc);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float pu = __builtin_amdgcn_exp2f(fmaf(sc[u], c, -mc));
      l += pu;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(pu, bf_lo(vr[u][e]), acc[2 * e]);
        acc[2 * e + 1] = fmaf(pu, bf_hi(vr[u][e]), acc[2 * e + 1]);
      }
    }
    m = m_new;
  }

  // ⊕-merge the slots of this wavefront (lanes that share a chunk).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float mm = fmaxf(m, m2);
    const float mmc = safe_mc(mm, c);
    const float fa = __builtin_amdgcn_exp2f(m * c - mmc);
    const float fb = __builtin_amdgcn_exp2f(m2 * c - mmc);
    l = l * fa + l2 * fb;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float a2 = __shfl_xor(acc[e], off);
      acc[e] = acc[e] * fa + a2 * fb;
    }
    m = mm;
  }

  // ⊕-merge the wavefronts through LDS and write the segment's (O_s, LSE_s).
  __shared__ float sm_m[kDecWaves], sm_l[kDecWaves];
  __shared__ float sm_o[kDecWaves][D];
  if (slot == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[wave][chunk * 8 + e] = acc[e];
    if (chunk == 0) {
      sm_m[wave] = m;
      sm_l[wave] = l;
    }
  }
  __syncthreads();
  if (tid < D) {
    float M = sm_m[0];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, sm_m[w]);
    const float Mc = safe_mc(M, c);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm_m[w] * c - Mc);
      L = fmaf(sm_l[w], f, L);
      o = fmaf(sm_o[w][tid], f, o);
    }
    const size_t part = (size_t)bh * p.S + s;
    p.part_o[part * D + tid] = o / L;
    if (tid == 0) p.part_lse[part] = M * p.scale + __builtin_amdgcn_logf(L) * 0.69314718055994531f;
  }
}

// O = Σ_s w_s O_s / Σ_s w_s and LSE = M + ln Σ_s w_s with w_s = exp(LSE_s − M),
// M = max_s LSE_s: the ⊕ merge written on normalised partials.  One
// workgroup per (b, h): the max over segments is a block reduction, then
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

  const int bh = blockIdx.x;
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

template <int D>
hipError_t launch_decode_t(const DecodeParams& p, int B, hipStream_t stream) {
  const int BH = B * p.H;
  hipLaunchKernelGGL(fa_decode_split_kernel<D>, dim3(BH * p.S), dim3(kDecThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fa_decode_combine_kernel<D>, dim3(BH), dim3(kCombThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int B, int d, hipStream_t stream) {
  return d == 64 ? launch_decode_t<64>(p, B, stream) : launch_decode_t<128>(p, B, stream);
}

}  // namespace fa
