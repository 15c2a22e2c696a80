// LayerNorm over rows of the F16 residual stream (HBM-bound).
//
// Page "Single-layer SigLIP vision benchmark", intro: layernorm with
// epsilon 1e-6 and affine parameters, F32 statistics computed in separate
// sum, centered-variance and affine passes. Here one 64-lane wavefront owns
// one row: the row is read once from HBM into registers with coalesced
// loads, the two F32 reductions run across the wavefront's lanes (DPP and
// lane-swap steps in the kernel for the So400m width, which gives every
// lane 18 values; shuffles in the generic one, whose lane i takes 8-value
// chunks i, i+64, ...), 1/sqrt(var + eps) comes from the hardware reciprocal
// square root (within 1 ulp of F32; a correctly rounded square root and
// division took about 12 of the ~150 instructions per row), and the
// normalised row is written once,
// as F16 or, when it feeds an FP8 GEMM, as e4m3 codes of y * 2^-exp (the
// producer writes the quantized operand; page "FP8 attention and resident
// image/embedding transfers", "Full 27-layer ViT", names producer-written
// FP8 as the way to keep the FP8 gain). Traffic per row: 2*width bytes in,
// 2*width (F16) or width (e4m3) bytes out.
#include "common.h"

#include <algorithm>

namespace siglip {
namespace {

constexpr int kMaxChunks = 4;  // 16-byte chunks per lane: width <= 64 * 8 * 4 = 2048

// WIDTH > 0 fixes the row width at compile time (the chunk bounds then fold
// into the unrolled loops); WIDTH = 0 takes it from the argument.
template <bool OUT_FP8, int WIDTH>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const f16* __restrict__ x, int64_t ldx, void* __restrict__ y, int64_t ldy,
    const float* __restrict__ gamma, const float* __restrict__ beta, int rows,
    int width_arg, float eps, float out_scale) {
  const int width = WIDTH > 0 ? WIDTH : width_arg;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int chunks = width >> 3;  // 8 values per chunk; chunk c of the row is lane c % 64, slot c / 64
  const f16x8* xr = reinterpret_cast<const f16x8*>(x + (int64_t)row * ldx);

  float v[kMaxChunks][8];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < chunks) {
      const f16x8 h = xr[c];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[i][e] = (float)h[e];
        s += v[i][e];
      }
    }
  }
  const float inv_w = 1.0f / (float)width;
  const float mean = wave_sum(s) * inv_w;
  float cs = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    if (lane + 64 * i < chunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[i][e] - mean;
        cs += d * d;
      }
    }
  }
  const float var = wave_sum(cs) * inv_w;
  const float rstd = __builtin_amdgcn_rsqf(var + eps);
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int c = lane + 64 * i;
    if (c < chunks) {
      const f32x4 g0 = reinterpret_cast<const f32x4*>(gamma)[2 * c];
      const f32x4 g1 = reinterpret_cast<const f32x4*>(gamma)[2 * c + 1];
      const f32x4 b0 = reinterpret_cast<const f32x4*>(beta)[2 * c];
      const f32x4 b1 = reinterpret_cast<const f32x4*>(beta)[2 * c + 1];
      float o[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (v[i][e] - mean) * rstd * g0[e] + b0[e];
        o[e + 4] = (v[i][e + 4] - mean) * rstd * g1[e] + b1[e];
      }
      if constexpr (OUT_FP8) {
        uint32_t w0 = pack4_e4m3(o[0] * out_scale, o[1] * out_scale, o[2] * out_scale, o[3] * out_scale);
        uint32_t w1 = pack4_e4m3(o[4] * out_scale, o[5] * out_scale, o[6] * out_scale, o[7] * out_scale);
        reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(y) + (int64_t)row * ldy)[c] = make_uint2(w0, w1);
      } else {
        f16x8 ov;
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = (f16)o[e];
        reinterpret_cast<f16x8*>(reinterpret_cast<f16*>(y) + (int64_t)row * ldy)[c] = ov;
      }
    }
  }
}

// Sum over the 64 lanes, every lane receiving the same total, without LDS:
// four DPP steps make every 16-lane row uniform (partners at lane distance
// 1 and 2 within quads, then the 8- and 16-lane mirrors), then
// v_permlane16_swap pairs rows 0/1 and 2/3 and v_permlane32_swap the two
// halves. Each step adds two partial sums in the same order on both
// partners, so all lanes end bit-identical.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int p = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
  return v + __builtin_bit_cast(float, p);
}
__device__ __forceinline__ float wave_sum_lanes(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v = dpp_add<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  v = dpp_add<0x140>(v);  // row_mirror
  unsigned a = __builtin_bit_cast(unsigned, v), b = a;
  asm volatile("" : "+v"(b));  // two distinct operands (see half_swap)
  const auto sw = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  const unsigned even = sw[0], odd = sw[1];  // rows 0/2 and rows 1/3 of each pair
  v = __builtin_bit_cast(float, even) + __builtin_bit_cast(float, odd);
  float lo, hi;
  half_swap(v, &lo, &hi);
  return lo + hi;
}

// a * b rounded to F32 on its own: the product is never fused with the
// operation that consumes it
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// The same LayerNorm for a compile-time width WIDTH = 512 NF + 64 TW, with
// waves that stay resident and walk rows r, r + (waves in the grid), ....
// Every lane holds 8 NF + TW values of a row: NF 16-byte chunks (chunk
// lane + 64 i) and TW values of the tail at 512 NF + TW lane, so no lane idles
// (1152 = 2 x 512 + 128: 18 values per lane). gamma and beta stay in
// registers; two register sets alternate so the next row's loads are in
// flight while the current row is reduced and written. The centred values
// are kept for the output, and the power-of-two e4m3 scale is applied to
// rstd and beta (exact), so y = fma((x - mean) rstd, gamma, beta) before
// scaling, as in layernorm_kernel; the row sums run in another order. The
// mean is rounded before the values are centred (not fused into the
// subtraction), so x - mean can be recomputed from the stored mean.
//
// STATS: the same kernel writes only each row's statistics, {mean, rstd *
// out_scale} as two floats at y + 8 row bytes, for a GEMM that normalizes
// its A operand itself (gemm.hip, LayerNorm-folded operand): it computes
// fma((x - mean) * rs, gamma, beta * out_scale) per element, the arithmetic
// below, so its operand equals this kernel's output bit for bit.
template <bool OUT_FP8, int WIDTH, bool STATS = false>
__global__ __launch_bounds__(256) void layernorm_rows_kernel(
    const f16* __restrict__ x, int64_t ldx, void* __restrict__ y, int64_t ldy,
    const float* __restrict__ gamma, const float* __restrict__ beta, int rows, float eps, float out_scale) {
  constexpr int NF = WIDTH / 512;
  constexpr int TW = (WIDTH % 512) / 64;
  constexpr int NV = 8 * NF + TW;
  static_assert(WIDTH % 64 == 0 && (TW == 0 || TW == 2) && NF >= 1 && NF <= 3, "row width");
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;  // waves in the grid
  const float sc = (OUT_FP8 || STATS) ? out_scale : 1.0f;
  float gm[NV], bt[NV];
  if constexpr (!STATS) {  // (the statistics kernel takes no gamma or beta)
#pragma unroll
    for (int i = 0; i < NF; ++i) {
      const int c = lane + 64 * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gm[8 * i + e] = gamma[8 * c + e];
        bt[8 * i + e] = beta[8 * c + e] * sc;
      }
    }
#pragma unroll
    for (int e = 0; e < TW; ++e) {
      gm[8 * NF + e] = gamma[512 * NF + TW * lane + e];
      bt[8 * NF + e] = beta[512 * NF + TW * lane + e] * sc;
    }
  }
  struct Raw {
    f16x8 f[NF];
    f16x2 t;
  };
  auto load = [&](Raw& r, int row) {
    const f16* xr = x + (int64_t)row * ldx;
#pragma unroll
    for (int i = 0; i < NF; ++i) r.f[i] = reinterpret_cast<const f16x8*>(xr)[lane + 64 * i];
    if constexpr (TW == 2) r.t = reinterpret_cast<const f16x2*>(xr + 512 * NF)[lane];
  };
  auto process = [&](const Raw& r, int row) {
    float v[NV];
#pragma unroll
    for (int i = 0; i < NF; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * i + e] = (float)r.f[i][e];
#pragma unroll
    for (int e = 0; e < TW; ++e) v[8 * NF + e] = (float)r.t[e];
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) s += v[k];
    const float inv_w = 1.0f / (float)WIDTH;
    const float mean = mul_rn(wave_sum_lanes(s), inv_w);
    float cs = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      v[k] -= mean;
      cs += v[k] * v[k];
    }
    const float var = wave_sum_lanes(cs) * inv_w;
    const float rs = __builtin_amdgcn_rsqf(var + eps) * sc;
    if constexpr (STATS) {
      if (lane == 0) reinterpret_cast<float2*>(y)[row] = make_float2(mean, rs);
      return;
    }
    float o[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) o[k] = fmaf(v[k] * rs, gm[k], bt[k]);
    if constexpr (OUT_FP8) {
      uint8_t* yr = reinterpret_cast<uint8_t*>(y) + (int64_t)row * ldy;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        const float* q = o + 8 * i;
        reinterpret_cast<uint2*>(yr)[lane + 64 * i] =
            make_uint2(pack4_e4m3(q[0], q[1], q[2], q[3]), pack4_e4m3(q[4], q[5], q[6], q[7]));
      }
      if constexpr (TW == 2)
        reinterpret_cast<uint16_t*>(yr + 512 * NF)[lane] = (uint16_t)cvt_pk_e4m3(o[8 * NF], o[8 * NF + 1], 0u, false);
    } else {
      f16* yr = reinterpret_cast<f16*>(y) + (int64_t)row * ldy;
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        f16x8 ov;
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = (f16)o[8 * i + e];
        reinterpret_cast<f16x8*>(yr)[lane + 64 * i] = ov;
      }
      if constexpr (TW == 2)
        reinterpret_cast<f16x2*>(yr + 512 * NF)[lane] = f16x2{(f16)o[8 * NF], (f16)o[8 * NF + 1]};
    }
  };
  Raw ra, rb;
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row < rows) load(ra, row);
  for (; row < rows; row += 2 * stride) {
    const int r1 = row + stride;
    if (r1 < rows) load(rb, r1);
    process(ra, row);
    if (r1 >= rows) break;
    const int r2 = r1 + stride;
    if (r2 < rows) load(ra, r2);
    process(rb, r1);
  }
}

// Resident grid for layernorm_rows_kernel: 16 workgroups of 4 waves per CU
// at most.
constexpr int kRowsGridMax = 4096;

}  // namespace

hipError_t launch_layernorm(const f16* x, int64_t ldx, void* y, int64_t ldy,
                            const float* gamma, const float* beta, int rows,
                            int width, float eps, bool out_fp8, float out_scale,
                            hipStream_t s) {
  if (rows < 1 || width < 8 || (width & 7) || width > 8 * 64 * kMaxChunks || ldx < width || ldy < width ||
      (ldx & 7) || (ldy & 7))
    return hipErrorInvalidValue;
  dim3 grid((rows + 3) / 4);
  if (width == 1152) {  // the So400m width
    const dim3 rgrid(std::min((rows + 3) / 4, kRowsGridMax));
    if (out_fp8)
      hipLaunchKernelGGL((layernorm_rows_kernel<true, 1152>), rgrid, dim3(256), 0, s, x, ldx, y, ldy, gamma, beta, rows, eps, out_scale);
    else
      hipLaunchKernelGGL((layernorm_rows_kernel<false, 1152>), rgrid, dim3(256), 0, s, x, ldx, y, ldy, gamma, beta, rows, eps, out_scale);
  } else if (out_fp8) {
    hipLaunchKernelGGL((layernorm_kernel<true, 0>), grid, dim3(256), 0, s, x, ldx, y, ldy, gamma, beta, rows, width, eps, out_scale);
  } else {
    hipLaunchKernelGGL((layernorm_kernel<false, 0>), grid, dim3(256), 0, s, x, ldx, y, ldy, gamma, beta, rows, width, eps, out_scale);
  }
  return hipGetLastError();
}

hipError_t launch_layernorm_stats(const f16* x, int64_t ldx, float* stats, int rows, int width, float eps,
                                  float scale, hipStream_t s) {
  if (rows < 1 || width != 1152 || ldx < width || (ldx & 7) || !stats || (reinterpret_cast<uintptr_t>(stats) & 7))
    return hipErrorInvalidValue;
  const dim3 rgrid(std::min((rows + 3) / 4, kRowsGridMax));
  hipLaunchKernelGGL((layernorm_rows_kernel<false, 1152, true>), rgrid, dim3(256), 0, s, x, ldx, stats, 0,
                     nullptr, nullptr, rows, eps, scale);
  return hipGetLastError();
}

}  // namespace siglip
