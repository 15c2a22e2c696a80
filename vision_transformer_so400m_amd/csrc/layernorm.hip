// LayerNorm over rows of the F16 residual stream (HBM-bound).
//
// Page "Single-layer SigLIP vision benchmark", intro: layernorm with
// epsilon 1e-6 and affine parameters, F32 statistics computed in separate
// sum, centered-variance and affine passes. Here one 64-lane wavefront owns
// one row: the row is read once from HBM into registers with coalesced
// 4-byte loads (lane i takes elements 2i, 2i+1, 2i+128, ...), the two F32
// reductions are wavefront shuffles, and the normalised row is written once,
// as F16 or, when it feeds an FP8 GEMM, as e4m3 codes of y * 2^-exp (the
// producer writes the quantized operand; page "FP8 attention and resident
// image/embedding transfers", "Full 27-layer ViT", names producer-written
// FP8 as the way to keep the FP8 gain). Traffic per row: 2*width bytes in,
// 2*width (F16) or width (e4m3) bytes out.
#include "common.h"

namespace siglip {
namespace {

constexpr int kMaxPairs = 16;  // width <= 2 * 64 * 16 = 2048

template <bool OUT_FP8>
__global__ __launch_bounds__(256) void layernorm_kernel(
    const f16* __restrict__ x, int64_t ldx, void* __restrict__ y, int64_t ldy,
    const float* __restrict__ gamma, const float* __restrict__ beta, int rows,
    int width, float eps, float out_scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int pairs = width >> 1;
  const f16x2* xr = reinterpret_cast<const f16x2*>(x + (int64_t)row * ldx);

  float v0[kMaxPairs], v1[kMaxPairs];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPairs; ++i) {
    const int p = lane + 64 * i;
    if (p < pairs) {
      f16x2 h = xr[p];
      v0[i] = (float)h[0];
      v1[i] = (float)h[1];
    } else {
      v0[i] = 0.0f;
      v1[i] = 0.0f;
    }
    s += v0[i] + v1[i];
  }
  const float inv_w = 1.0f / (float)width;
  const float mean = wave_sum(s) * inv_w;
  float c = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPairs; ++i) {
    if (lane + 64 * i < pairs) {
      const float d0 = v0[i] - mean, d1 = v1[i] - mean;
      c += d0 * d0 + d1 * d1;
    }
  }
  const float var = wave_sum(c) * inv_w;
  const float rstd = 1.0f / sqrtf(var + eps);
#pragma unroll
  for (int i = 0; i < kMaxPairs; ++i) {
    const int p = lane + 64 * i;
    if (p < pairs) {
      const float2 g = reinterpret_cast<const float2*>(gamma)[p];
      const float2 b = reinterpret_cast<const float2*>(beta)[p];
      const float o0 = (v0[i] - mean) * rstd * g.x + b.x;
      const float o1 = (v1[i] - mean) * rstd * g.y + b.y;
      if constexpr (OUT_FP8) {
        uint32_t w = cvt_pk_e4m3(o0 * out_scale, o1 * out_scale, 0u, false);
        reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(y) + (int64_t)row * ldy)[p] = (uint16_t)w;
      } else {
        f16x2 o = {(f16)o0, (f16)o1};
        reinterpret_cast<f16x2*>(reinterpret_cast<f16*>(y) + (int64_t)row * ldy)[p] = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_layernorm(const f16* x, int64_t ldx, void* y, int64_t ldy,
                            const float* gamma, const float* beta, int rows,
                            int width, float eps, bool out_fp8, float out_scale,
                            hipStream_t s) {
  if (rows < 1 || width < 2 || (width & 1) || width > 2 * 64 * kMaxPairs || ldx < width || ldy < width)
    return hipErrorInvalidValue;
  dim3 grid((rows + 3) / 4);
  if (out_fp8)
    hipLaunchKernelGGL(layernorm_kernel<true>, grid, dim3(256), 0, s, x, ldx, y, ldy, gamma, beta, rows, width, eps, out_scale);
  else
    hipLaunchKernelGGL(layernorm_kernel<false>, grid, dim3(256), 0, s, x, ldx, y, ldy, gamma, beta, rows, width, eps, out_scale);
  return hipGetLastError();
}

}  // namespace siglip
