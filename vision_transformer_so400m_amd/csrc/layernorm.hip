// LayerNorm over rows of the F16 residual stream (HBM-bound).
//
// Page "Single-layer SigLIP vision benchmark", intro: layernorm with
// epsilon 1e-6 and affine parameters, F32 statistics computed in separate
// sum, centered-variance and affine passes. Here one 64-lane wavefront owns
// one row: the row is read once from HBM into registers with coalesced
// 16-byte loads (lane i takes 8-value chunks i, i+64, i+128), the two F32
// reductions are wavefront shuffles, and the normalised row is written once,
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
  const float rstd = 1.0f / sqrtf(var + eps);
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

// The same arithmetic for a compile-time width, with waves that stay
// resident and walk rows r, r + (waves in the grid), ...: gamma and beta are
// loaded once per lane, and the next row's loads are in flight while the
// current row is reduced and written. Each row's sums run in the same order
// as in layernorm_kernel, so the output is bit-identical.
template <bool OUT_FP8, int WIDTH>
__global__ __launch_bounds__(256) void layernorm_rows_kernel(
    const f16* __restrict__ x, int64_t ldx, void* __restrict__ y, int64_t ldy,
    const float* __restrict__ gamma, const float* __restrict__ beta, int rows, float eps, float out_scale) {
  constexpr int CH = WIDTH / 8;            // 8-value chunks per row
  constexpr int NS = (CH + 63) / 64;       // chunk slots per lane
  static_assert(WIDTH % 8 == 0 && NS <= kMaxChunks, "row width");
  const int lane = threadIdx.x & 63;
  const int stride = gridDim.x * 4;        // waves in the grid
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  f32x4 g[NS][2], b[NS][2];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int c = lane + 64 * i;
    if (c < CH) {
      g[i][0] = reinterpret_cast<const f32x4*>(gamma)[2 * c];
      g[i][1] = reinterpret_cast<const f32x4*>(gamma)[2 * c + 1];
      b[i][0] = reinterpret_cast<const f32x4*>(beta)[2 * c];
      b[i][1] = reinterpret_cast<const f32x4*>(beta)[2 * c + 1];
    }
  }
  f16x8 cur[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int c = lane + 64 * i;
    if (c < CH && row < rows) cur[i] = reinterpret_cast<const f16x8*>(x + (int64_t)row * ldx)[c];
  }
  for (; row < rows; row += stride) {
    const int next = row + stride;
    f16x8 nxt[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int c = lane + 64 * i;
      if (c < CH && next < rows) nxt[i] = reinterpret_cast<const f16x8*>(x + (int64_t)next * ldx)[c];
    }
    float v[NS][8];
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (lane + 64 * i < CH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[i][e] = (float)cur[i][e];
          s += v[i][e];
        }
      }
    }
    const float inv_w = 1.0f / (float)WIDTH;
    const float mean = wave_sum(s) * inv_w;
    float cs = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (lane + 64 * i < CH) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = v[i][e] - mean;
          cs += d * d;
        }
      }
    }
    const float var = wave_sum(cs) * inv_w;
    const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int c = lane + 64 * i;
      if (c < CH) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = (v[i][e] - mean) * rstd * g[i][0][e] + b[i][0][e];
          o[e + 4] = (v[i][e + 4] - mean) * rstd * g[i][1][e] + b[i][1][e];
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
#pragma unroll
    for (int i = 0; i < NS; ++i) cur[i] = nxt[i];
  }
}

// Resident grid for layernorm_rows_kernel: 16 workgroups of 4 waves per CU
// at most (measured at 46,656 rows: 30.5 us against 32 us for one row per
// wave; a copy of the same bytes takes 24 us).
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

}  // namespace siglip
