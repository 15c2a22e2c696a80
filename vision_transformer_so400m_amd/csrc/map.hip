// MAP head probe attention with the K/V projection folded away.
//
// The MAP head ([SLB] intro and mermaid figure: one learned probe, its query
// projection, one fused K/V projection of the final-LN tokens Z, softmax
// attention per head, output projection) needs, per image b and head h,
//   scores_t = q_h . K_{t,h} = Z_t . (W_k,h q_h) + b_k,h . q_h
//   o_h      = sum_t p_t V_{t,h} = (sum_t p_t Z_t) W_v,h + b_v,h
// (p sums to one). The probe is shared by every image ([SLB]: each batch uses
// the same learned probe), so u_h = W_k,h q_h is computed once at create, and
// the constant b_k,h . q_h cancels in the softmax. That replaces the
// [M, width] x [width, 2 width] K/V GEMM (3.9 GFLOP per image) by one pass
// over Z for the scores, one for the probability-weighted sum of Z, and a
// per-head [width] x [width, head_dim] product: the same real numbers, about
// 70x fewer operations, and no e4m3 rounding of K and V.
//
//  * map_scores: S[b][h][t] = (Z[b T + t,:] . u_h) * scale * log2(e), F32, by
//    v_mfma_f32_16x16x32_f16 on 16-token x 16-head tiles. u is held as two
//    F16 parts (u = hi + lo), so the scores carry F32-level accuracy.
//  * map_pool: per image and 64-column block, the softmax over the tokens
//    (max, exp2, sum in F32, probabilities in LDS) and zbar_h = sum_t p_t Z_t.
//  * map_vproj: o[b, h*D + d] = zbar_h . W_v[:, h*D + d] + b_v, written as the
//    operand type of the MAP output projection (F16 or e4m3 codes).
//
// map_attn (the explicit K/V option): probe attention, one query per (image,
// head) against the T encoder tokens' projected K and V; memory-bound, it
// reads K and V once (2 x T x 72 x 2 bytes per head).
#include "common.h"

#include <algorithm>

namespace siglip {
namespace {

constexpr int kMapHeads = 16;  // head slots of a score row (heads beyond H are zero)

// A 16 x 16 tile of scores (tokens t0..t0+15 on the MFMA rows, head slots on
// the columns) per workgroup: wave w sums the width/4 columns
// [w width/4, (w+1) width/4) in K steps of 32, lane (i, g) = (lane % 16,
// lane / 16) loading Z[t0+i][k0 + 8g .. +7] and the same columns of u for
// head slot i; the four partial tiles are added in LDS.
__global__ __launch_bounds__(256) void map_scores_kernel(const f16* __restrict__ z, int64_t ldz,
                                                         const f16* __restrict__ u_hi,
                                                         const f16* __restrict__ u_lo, int width,
                                                         float* __restrict__ s, int rows, int T, float sl2) {
  __shared__ f32x4 part[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int i = lane & 15;
  const int g = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const int row = min(t0 + i, rows - 1);  // rows past the end re-read the last row; never stored
  const int quarter = width >> 2;
  const int kb = wave * quarter + 8 * g;
  const f16* zr = z + (int64_t)row * ldz + kb;
  const f16* uh = u_hi + (int64_t)i * width + kb;
  const f16* ul = u_lo + (int64_t)i * width + kb;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 9
  for (int k0 = 0; k0 < quarter; k0 += 32) {
    const f16x8 a = *reinterpret_cast<const f16x8*>(zr + k0);
    const f16x8 h = *reinterpret_cast<const f16x8*>(uh + k0);
    const f16x8 l = *reinterpret_cast<const f16x8*>(ul + k0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, h, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, l, acc, 0, 0, 0);
  }
  part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    const f32x4 sum = (part[0][lane] + part[1][lane]) + (part[2][lane] + part[3][lane]);
    // lane holds rows t0 + 4g + r (r = 0..3) of head slot i; scores are
    // stored per image and head: s[(b * 16 + i) * T + t] for row b * T + t
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = t0 + 4 * g + r;
      if (m < rows) {
        const int b = m / T;
        s[((int64_t)b * kMapHeads + i) * T + (m - b * T)] = sum[r] * sl2;
      }
    }
  }
}

// Sum of v over the four 16-lane rows of a wave, in every lane
// (v_permlane16_swap / v_permlane32_swap exchanges; second operands made
// opaque so the compiler keeps the two results of each swap apart).
__device__ __forceinline__ float row4_sum(float v) {
  unsigned a = __builtin_bit_cast(unsigned, v), b = a;
  asm volatile("" : "+v"(b));
  const auto s16 = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  const unsigned x0 = s16[0], x1 = s16[1];
  v = __builtin_bit_cast(float, x0) + __builtin_bit_cast(float, x1);  // rows (0+1, 0+1, 2+3, 2+3)
  a = __builtin_bit_cast(unsigned, v);
  b = a;
  asm volatile("" : "+v"(b));
  const auto s32 = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  const unsigned y0 = s32[0], y1 = s32[1];
  return __builtin_bit_cast(float, y0) + __builtin_bit_cast(float, y1);
}

// One workgroup of 512 threads (8 waves) per (64-column block, image).
// Thread (c, q) = (tid / 16, tid % 16) takes the tokens t = c (mod 32) and
// columns c0 + 4q .. +3 for all 16 head slots (64 accumulators): one 8-byte
// load of Z per token, kRound tokens per round, the next round's loads in
// flight while the current one is summed. The first round is issued before
// the softmax: each wave takes two heads, holds a lane's share of the scores
// in registers (all loads issued together), then max, exp2 and sum in F32;
// the probabilities go to LDS as rows of kPStride floats per token (16 head
// slots, padded so that the column writes spread over the banks). The four
// token slices of a wave are summed by lane exchanges, the 8 waves through
// LDS.
constexpr int kPoolThreads = 512;
constexpr int kPoolWaves = kPoolThreads / 64;
constexpr int kPoolSlices = kPoolThreads / 16;
constexpr int kPoolRound = 8;                            // tokens per thread per round
constexpr int kPoolStep = kPoolRound * kPoolSlices;      // tokens per round per workgroup
constexpr int kPStride = 20;                             // floats per probability row
constexpr int kMaxTokens = 1024;
constexpr int kScorePerLane = kMaxTokens / 64;

__global__ __launch_bounds__(kPoolThreads) void map_pool_kernel(const f16* __restrict__ z, int64_t ldz,
                                                        const float* __restrict__ s, int T, int heads,
                                                        float* __restrict__ zbar, int width) {
  extern __shared__ float p[];  // [T][kPStride]; reused for the wave partials [waves][16][64]
  __shared__ float inv_l[kMapHeads];
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int c = tid >> 4;
  const int q = tid & 15;
  const f16* zc = z + (int64_t)b * T * ldz + blockIdx.x * 64 + 4 * q;

  f16x4 zv[kPoolRound];
#pragma unroll
  for (int j = 0; j < kPoolRound; ++j) {
    const int t = c + kPoolSlices * j;
    zv[j] = t < T ? *reinterpret_cast<const f16x4*>(zc + (int64_t)t * ldz) : f16x4{0, 0, 0, 0};
  }

  {
    const int wave = tid >> 6, lane = tid & 63;
    const int h0 = 2 * wave;  // heads h0 and h0 + 1
    const float* s0 = s + ((int64_t)b * kMapHeads + h0) * T;
    float v0[kScorePerLane], v1[kScorePerLane];
#pragma unroll
    for (int i = 0; i < kScorePerLane; ++i) {
      const int t = lane + 64 * i;
      v0[i] = t < T ? s0[t] : -__builtin_inff();
      v1[i] = t < T ? s0[T + t] : -__builtin_inff();
    }
    float m0 = v0[0], m1 = v1[0];
#pragma unroll
    for (int i = 1; i < kScorePerLane; ++i) {
      m0 = fmaxf(m0, v0[i]);
      m1 = fmaxf(m1, v1[i]);
    }
    m0 = wave_max(m0);
    m1 = wave_max(m1);
    float l0 = 0.f, l1 = 0.f;
#pragma unroll
    for (int i = 0; i < kScorePerLane; ++i) {
      const int t = lane + 64 * i;
      const float e0 = __builtin_amdgcn_exp2f(v0[i] - m0);  // exactly 0 past the end
      const float e1 = __builtin_amdgcn_exp2f(v1[i] - m1);
      if (t < T) *reinterpret_cast<float2*>(p + t * kPStride + h0) = float2{e0, e1};
      l0 += e0;
      l1 += e1;
    }
    l0 = wave_sum(l0);
    l1 = wave_sum(l1);
    if (lane == 0) {
      inv_l[h0] = 1.0f / l0;
      inv_l[h0 + 1] = 1.0f / l1;
    }
  }
  __syncthreads();

  float acc[kMapHeads][4];
#pragma unroll
  for (int h = 0; h < kMapHeads; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = 0.f;
  for (int t0 = c; t0 < T; t0 += kPoolStep) {
    f16x4 zn[kPoolRound];
#pragma unroll
    for (int j = 0; j < kPoolRound; ++j) {
      const int t = t0 + kPoolStep + kPoolSlices * j;
      zn[j] = t < T ? *reinterpret_cast<const f16x4*>(zc + (int64_t)t * ldz) : f16x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < kPoolRound; ++j) {
      const int t = min(t0 + kPoolSlices * j, T - 1);  // tokens past the end carry Z = 0
      const f32x4* pt = reinterpret_cast<const f32x4*>(p + t * kPStride);
      float zf[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) zf[e] = (float)zv[j][e];
#pragma unroll
      for (int h4 = 0; h4 < kMapHeads / 4; ++h4) {
        const f32x4 pv = pt[h4];
#pragma unroll
        for (int hh = 0; hh < 4; ++hh)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * h4 + hh][e] = fmaf(pv[hh], zf[e], acc[4 * h4 + hh][e]);
      }
    }
#pragma unroll
    for (int j = 0; j < kPoolRound; ++j) zv[j] = zn[j];
  }
  // lanes q, q+16, q+32, q+48 of a wave hold the four token slices of column quad q
#pragma unroll
  for (int h = 0; h < kMapHeads; ++h)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[h][e] = row4_sum(acc[h][e]);
  __syncthreads();  // every thread is done reading p: reuse it for the wave partials
  const int wave = tid >> 6, lane = tid & 63;
  f32x4* part = reinterpret_cast<f32x4*>(p);  // [waves][16 heads][16 quads]
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < kMapHeads; ++h)
      part[(wave * kMapHeads + h) * 16 + lane] = f32x4{acc[h][0], acc[h][1], acc[h][2], acc[h][3]};
  }
  __syncthreads();
  if (tid < kMapHeads * 16) {
    const int h = tid >> 4, qq = tid & 15;
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kPoolWaves; ++w) sum += part[(w * kMapHeads + h) * 16 + qq];
    if (h < heads) {
      const float inv = inv_l[h];
      *reinterpret_cast<f32x4*>(zbar + ((int64_t)b * kMapHeads + h) * width + blockIdx.x * 64 + 4 * qq) =
          f32x4{sum[0] * inv, sum[1] * inv, sum[2] * inv, sum[3] * inv};
    }
  }
}

// One workgroup per (head, quarter of the head's D outputs, group of 4
// images). wvt holds W_v transposed per head: wvt[(h*D + d) * width + k] =
// W_v[k][h*D + d]. Thread (kc, d) = (tid / (D/4), tid % (D/4)) sums the K
// chunk [kc width/32, (kc+1) width/32) for the 4 images (zbar rows staged in
// LDS); the 32 chunks are added in LDS in chunk order. Short per-thread
// chains and 4x the workgroups of one per head: at batch 1 the launch is
// bound by the latency of each thread's chain of loads.
constexpr int kVprojImages = 4;
constexpr int kVprojChunks = 32;
constexpr int kVprojSplit = 4;  // output groups per head

template <bool OUT_FP8>
__global__ __launch_bounds__(1024) void map_vproj_kernel(const float* __restrict__ zbar, const float* __restrict__ wvt,
                                                         const float* __restrict__ bv, int width, int D, int batch,
                                                         void* __restrict__ o, int64_t ldo, float out_scale) {
  extern __shared__ float sm[];  // zbar rows [kVprojImages][width], then partials [kVprojChunks][kVprojImages][DD]
  const int h = blockIdx.x / kVprojSplit;
  const int DD = D / kVprojSplit;  // outputs of this workgroup: dims dg*DD .. dg*DD + DD - 1 of head h
  const int dg = blockIdx.x - h * kVprojSplit;
  const int b0 = blockIdx.y * kVprojImages;
  const int nb = min(kVprojImages, batch - b0);
  for (int i = threadIdx.x; i < kVprojImages * width; i += blockDim.x) {
    const int bi = i / width;
    sm[i] = bi < nb ? zbar[((int64_t)(b0 + bi) * kMapHeads + h) * width + (i - bi * width)] : 0.f;
  }
  __syncthreads();
  const int kc = threadIdx.x / DD;
  const int d = threadIdx.x - kc * DD;
  const int chunk = width / kVprojChunks;
  float acc[kVprojImages] = {0.f, 0.f, 0.f, 0.f};
  if (kc < kVprojChunks) {
    const float* wr = wvt + (int64_t)(h * D + dg * DD + d) * width + kc * chunk;
    const float* zr = sm + kc * chunk;
#pragma unroll 4
    for (int k = 0; k < chunk; k += 4) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(wr + k);
#pragma unroll
      for (int bi = 0; bi < kVprojImages; ++bi) {
        const f32x4 zv = *reinterpret_cast<const f32x4*>(zr + bi * width + k);
        acc[bi] = fmaf(w[0], zv[0], fmaf(w[1], zv[1], fmaf(w[2], zv[2], fmaf(w[3], zv[3], acc[bi]))));
      }
    }
  }
  float* red = sm + kVprojImages * width;
  if (kc < kVprojChunks)
#pragma unroll
    for (int bi = 0; bi < kVprojImages; ++bi) red[(kc * kVprojImages + bi) * DD + d] = acc[bi];
  __syncthreads();
  if (threadIdx.x < kVprojImages * DD) {
    const int bi = threadIdx.x / DD, dd = threadIdx.x - bi * DD;
    if (bi < nb) {
      float v = bv[h * D + dg * DD + dd];
#pragma unroll
      for (int c = 0; c < kVprojChunks; ++c) v += red[(c * kVprojImages + bi) * DD + dd];
      const int64_t at = (int64_t)(b0 + bi) * ldo + h * D + dg * DD + dd;
      if constexpr (OUT_FP8)
        reinterpret_cast<uint8_t*>(o)[at] = (uint8_t)(cvt_pk_e4m3(v * out_scale, 0.f, 0u, false) & 0xFF);
      else
        reinterpret_cast<f16*>(o)[at] = (f16)v;
    }
  }
}

// ---- create-time constants of the fold (one launch each, F32 arithmetic).
// q[n] = bq[n] + sum_k probe[k] Wq[k][n]; also kept as F16 for inspection.
__global__ __launch_bounds__(256) void map_query_kernel(const float* __restrict__ probe, const float* __restrict__ wq,
                                                        const float* __restrict__ bq, int width, float* __restrict__ q,
                                                        f16* __restrict__ q16) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= width) return;
  float acc = bq[n];
  for (int k = 0; k < width; ++k) acc = fmaf(probe[k], wq[(int64_t)k * width + n], acc);
  q[n] = acc;
  q16[n] = (f16)acc;
}

// u_h[k] = sum_d W_k[k][h D + d] q[h D + d] for head slots h < heads (slots
// up to kMapHeads are zero), split into F16 parts hi = f16(u), lo = f16(u - hi).
// W_k is the first width columns of the fused [width, 2 width] K/V weight.
__global__ __launch_bounds__(256) void map_u_kernel(const float* __restrict__ wkv, const float* __restrict__ q,
                                                    int width, int heads, int head_dim, f16* __restrict__ u_hi,
                                                    f16* __restrict__ u_lo) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= kMapHeads * width) return;
  const int h = i / width, k = i - h * width;
  float u = 0.f;
  if (h < heads) {
    const float* wr = wkv + (int64_t)k * 2 * width + h * head_dim;
    const float* qh = q + h * head_dim;
    for (int d = 0; d < head_dim; ++d) u = fmaf(wr[d], qh[d], u);
  }
  const f16 hi = (f16)u;
  u_hi[i] = hi;
  u_lo[i] = (f16)(u - (float)hi);
}

// wvt[n][k] = W_v[k][n] = wkv[k][width + n] (32 x 32 tiles through LDS)
__global__ __launch_bounds__(256) void map_wv_transpose_kernel(const float* __restrict__ wkv, int width,
                                                               float* __restrict__ wvt) {
  __shared__ float tile[32][33];
  const int k0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int j = 0; j < 32; j += 8) {
    const int k = k0 + ty + j, n = n0 + tx;
    tile[ty + j][tx] = (k < width && n < width) ? wkv[(int64_t)k * 2 * width + width + n] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 32; j += 8) {
    const int n = n0 + ty + j, k = k0 + tx;
    if (n < width && k < width) wvt[(int64_t)n * width + k] = tile[tx][ty + j];
  }
}

constexpr int kMapMaxT = 4096;

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

template <bool OUT_FP8>
__global__ __launch_bounds__(256) void map_attn_kernel(
    const f16* __restrict__ q, const f16* __restrict__ kv, int64_t ldkv, int64_t voff,
    void* __restrict__ o, int64_t ldo, int T, int D, float sl2, float out_scale) {
  __shared__ float sq[80];
  __shared__ float sp[kMapMaxT];
  __shared__ float red[4];
  __shared__ float part[32][80];

  const int t = threadIdx.x;
  const int hc = blockIdx.x * D;
  const int b = blockIdx.y;
  const f16* base = kv + (int64_t)b * T * ldkv + hc;
  if (t < D) sq[t] = (float)q[hc + t] * sl2;
  __syncthreads();

  const int nch = D >> 3;
  float lmax = -__builtin_inff();
  for (int key = t; key < T; key += 256) {
    const f16* kr = base + (int64_t)key * ldkv;
    float s = 0.0f;
    for (int ch = 0; ch < nch; ++ch) {
      const f16x8 x = *reinterpret_cast<const f16x8*>(kr + 8 * ch);
#pragma unroll
      for (int i = 0; i < 8; ++i) s += (float)x[i] * sq[8 * ch + i];
    }
    sp[key] = s;
    lmax = fmaxf(lmax, s);
  }
  const float M = block_max(lmax, red);
  float lsum = 0.0f;
  for (int key = t; key < T; key += 256) {
    const float p = __builtin_amdgcn_exp2f(sp[key] - M);
    sp[key] = p;
    lsum += p;
  }
  const float L = block_sum(lsum, red);  // includes a barrier: sp[] complete

  const int ng = min(256 / nch, 32);
  const int grp = t / nch, ch = t % nch;
  if (grp < ng) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int key = grp; key < T; key += ng) {
      const f16x8 x = *reinterpret_cast<const f16x8*>(base + (int64_t)key * ldkv + voff + 8 * ch);
      const float p = sp[key];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += p * (float)x[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[grp][8 * ch + i] = acc[i];
  }
  __syncthreads();
  if (t < D) {
    float s = 0.0f;
    for (int g = 0; g < ng; ++g) s += part[g][t];
    const float r = s / L;
    if constexpr (OUT_FP8) {
      reinterpret_cast<uint8_t*>(o)[(int64_t)b * ldo + hc + t] =
          (uint8_t)(cvt_pk_e4m3(r * out_scale, 0.0f, 0u, false) & 0xFF);
    } else {
      reinterpret_cast<f16*>(o)[(int64_t)b * ldo + hc + t] = (f16)r;
    }
  }
}

}  // namespace

bool map_fold_supported(int width, int heads, int head_dim, int tokens) {
  return heads >= 1 && heads <= kMapHeads && width % 128 == 0 && width <= 4096 && tokens >= 1 &&
         tokens <= kMaxTokens && head_dim >= 4 && head_dim % kVprojSplit == 0 &&
         head_dim / kVprojSplit * kVprojChunks <= 1024 &&
         heads * head_dim == width;
}

hipError_t launch_map_fold(const f16* z, int64_t ldz, const f16* u_hi, const f16* u_lo, const float* wvt,
                           const float* bv, float* scores, float* zbar, int batch, int tokens, int heads,
                           int head_dim, int width, float scale, bool out_fp8, float out_scale, void* o,
                           int64_t ldo, hipStream_t s, int phase) {
  if (!map_fold_supported(width, heads, head_dim, tokens) || batch < 1 || batch > 65535 || ldz < width ||
      (ldz & 7) || ldo < width)
    return hipErrorInvalidValue;
  const int rows = batch * tokens;
  if (phase == 0) {
    const float sl2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL(map_scores_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, s, z, ldz, u_hi, u_lo,
                       width, scores, rows, tokens, sl2);
    return hipGetLastError();
  }
  // probabilities [tokens][kPStride] F32, reused for waves x 16 x 16 partial sums of 16 bytes
  const size_t pool_lds = std::max<size_t>((size_t)kPStride * tokens * sizeof(float), kPoolWaves * kMapHeads * 16 * 16);
  hipLaunchKernelGGL(map_pool_kernel, dim3((unsigned)(width / 64), (unsigned)batch), dim3(kPoolThreads), pool_lds, s, z, ldz,
                     scores, tokens, heads, zbar, width);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)(heads * kVprojSplit), (unsigned)((batch + kVprojImages - 1) / kVprojImages));
  const dim3 block((unsigned)(head_dim / kVprojSplit * kVprojChunks));
  const size_t lds =
      ((size_t)kVprojImages * width + (size_t)kVprojChunks * kVprojImages * (head_dim / kVprojSplit)) * sizeof(float);
  if (out_fp8)
    hipLaunchKernelGGL(map_vproj_kernel<true>, grid, block, lds, s, zbar, wvt, bv, width, head_dim, batch, o, ldo,
                       out_scale);
  else
    hipLaunchKernelGGL(map_vproj_kernel<false>, grid, block, lds, s, zbar, wvt, bv, width, head_dim, batch, o, ldo,
                       out_scale);
  return hipGetLastError();
}

hipError_t launch_map_fold_prepare(const float* probe, const float* wq, const float* bq, const float* wkv, int width,
                                   int heads, int head_dim, float* q, f16* q16, f16* u_hi, f16* u_lo, float* wvt,
                                   hipStream_t s) {
  if (width < 1 || width > 4096 || heads < 1 || heads > kMapHeads || head_dim < 1 || heads * head_dim != width)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(map_query_kernel, dim3((unsigned)((width + 255) / 256)), dim3(256), 0, s, probe, wq, bq, width, q,
                     q16);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(map_u_kernel, dim3((unsigned)((kMapHeads * width + 255) / 256)), dim3(256), 0, s, wkv, q, width,
                     heads, head_dim, u_hi, u_lo);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((width + 31) / 32), (unsigned)((width + 31) / 32));
  hipLaunchKernelGGL(map_wv_transpose_kernel, grid, dim3(256), 0, s, wkv, width, wvt);
  return hipGetLastError();
}

hipError_t launch_map_attention(const f16* q, const f16* kv, int64_t ldkv, int64_t v_offset, void* o,
                                int64_t ldo, int batch, int heads, int tokens, int head_dim,
                                float scale, bool out_fp8, float out_scale, hipStream_t s) {
  if (batch < 1 || heads < 1 || tokens < 1 || tokens > kMapMaxT || head_dim < 8 || head_dim > 80 ||
      (head_dim & 7) || (ldkv & 7) || (v_offset & 7) || batch > 65535)
    return hipErrorInvalidValue;
  const float sl2 = scale * 1.4426950408889634f;
  dim3 grid(heads, batch);
  if (out_fp8)
    hipLaunchKernelGGL(map_attn_kernel<true>, grid, dim3(256), 0, s, q, kv, ldkv, v_offset, o, ldo, tokens, head_dim, sl2, out_scale);
  else
    hipLaunchKernelGGL(map_attn_kernel<false>, grid, dim3(256), 0, s, q, kv, ldkv, v_offset, o, ldo, tokens, head_dim, sl2, out_scale);
  return hipGetLastError();
}

}  // namespace siglip
