// Layout and precision conversions around the GEMMs.
//
//  * pad_convert: the caller's patch rows [M, 588] F16 (1,176-byte rows, only
//    8-byte aligned) become K-padded rows [M, 640] of the GEMM operand type,
//    zeros in columns 588..639, so the patch GEMM reads whole aligned 128-byte
//    K slices and never a byte past a row (page "Layout and barrier
//    diagnosis", "Padding, SRAM placement and paired transfers": padding is
//    read by the products, so it must hold zeros, never stale data).
//  * weight_transpose: create-time F32 [K, N] -> [N_pad, K_pad] F16 or e4m3,
//    K-contiguous in 64-byte K panels (panel p holds bytes 64p..64p+63 of
//    every row, rows consecutive), zero padding; staged through LDS so both
//    the F32 reads and the narrow writes are coalesced.
//  * f32_convert: create-time F32 rows -> padded F16/e4m3 rows (the probe).
//  * vt_transpose: V [batch, tokens, width] -> V^T per image ([b width + c]
//    rows of tokens, zero past the last token), the layout the streaming
//    attention kernel reads, for attention calls that receive V row-major.
//  * fill_u16: workspace poisoning for the padding tests.
#include "common.h"

namespace siglip {
namespace {

template <bool OUT_FP8>
__global__ __launch_bounds__(256) void pad_convert_kernel(const f16* __restrict__ x, int64_t ldx,
                                                          void* __restrict__ y, int rows, int cols,
                                                          int cols_pad, float scale) {
  // one thread per 4 output columns
  const int quads = cols_pad >> 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * quads) return;
  const int r = (int)(idx / quads);
  const int c = (int)(idx % quads) * 4;
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  if (c + 4 <= cols) {
    const f16x4 h = *reinterpret_cast<const f16x4*>(x + (int64_t)r * ldx + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (float)h[i];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (c + i < cols) v[i] = (float)x[(int64_t)r * ldx + c + i];
  }
  if constexpr (OUT_FP8) {
    reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(y) + (int64_t)r * cols_pad)[c >> 2] =
        pack4_e4m3(v[0] * scale, v[1] * scale, v[2] * scale, v[3] * scale);
  } else {
    f16x4 o = {(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
    *reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(y) + (int64_t)r * cols_pad + c) = o;
  }
}

// 32x32 tile transpose; block 32x8 threads.
template <bool OUT_FP8>
__global__ __launch_bounds__(256) void weight_transpose_kernel(const float* __restrict__ w, int K, int N,
                                                               void* __restrict__ wt, int K_pad, int N_pad,
                                                               float scale) {
  __shared__ float tile[32][33];
  const int k0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
  for (int j = 0; j < 32; j += 8) {
    const int k = k0 + ty + j, n = n0 + tx;
    tile[ty + j][tx] = (k < K && n < N) ? w[(int64_t)k * N + n] : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 32; j += 8) {
    const int n = n0 + ty + j, k = k0 + tx;
    if (n < N_pad && k < K_pad) {
      const float v = tile[tx][ty + j] * scale;
      if constexpr (OUT_FP8) {  // 64 codes per panel row
        const uint32_t c = cvt_pk_e4m3(v, 0.0f, 0u, false);
        reinterpret_cast<uint8_t*>(wt)[((int64_t)(k >> 6) * N_pad + n) * 64 + (k & 63)] = (uint8_t)(c & 0xFF);
      } else {  // 32 F16 values per panel row
        reinterpret_cast<f16*>(wt)[((int64_t)(k >> 5) * N_pad + n) * 32 + (k & 31)] = (f16)v;
      }
    }
  }
}

template <bool OUT_FP8>
__global__ __launch_bounds__(256) void f32_convert_kernel(const float* __restrict__ x, int rows, int cols,
                                                          void* __restrict__ y, int cols_pad, float scale) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * cols_pad) return;
  const int r = (int)(idx / cols_pad), c = (int)(idx % cols_pad);
  const float v = c < cols ? x[(int64_t)r * cols + c] * scale : 0.0f;
  if constexpr (OUT_FP8) {
    reinterpret_cast<uint8_t*>(y)[idx] = (uint8_t)(cvt_pk_e4m3(v, 0.0f, 0u, false) & 0xFF);
  } else {
    reinterpret_cast<f16*>(y)[idx] = (f16)v;
  }
}

// 64 tokens x 64 columns per workgroup through LDS: 16-byte reads along V
// rows, 16-byte writes along V^T rows. The LDS row pitch of 66 halfs (33
// words) puts the 8 rows one column read touches in distinct banks.
__global__ __launch_bounds__(256) void vt_transpose_kernel(const f16* __restrict__ v, int64_t ld, int T, int width,
                                                           f16* __restrict__ vt, int64_t vt_ld) {
  constexpr int P = 66;
  __shared__ uint32_t tile[64 * P / 2];
  f16* th = reinterpret_cast<f16*>(tile);
  const int b = blockIdx.z, t0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int r = i >> 3, ch = i & 7;
    const int tok = t0 + r, col = c0 + 8 * ch;
    i32x4 x = {0, 0, 0, 0};
    if (tok < T && col < width) x = *reinterpret_cast<const i32x4*>(v + ((int64_t)b * T + tok) * ld + col);
    uint32_t* d = tile + (r * P + 8 * ch) / 2;
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = (uint32_t)x[e];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 512; i += 256) {
    const int cc = i >> 3, ch = i & 7;
    const int col = c0 + cc;
    if (col >= width) continue;
    f16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = th[(8 * ch + e) * P + cc];
    *reinterpret_cast<f16x8*>(vt + ((int64_t)b * width + col) * vt_ld + t0 + 8 * ch) = y;
  }
}

__global__ __launch_bounds__(256) void zero_cols_kernel(f16* __restrict__ p, int64_t rows, int64_t ld, int c0, int w) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * w) return;
  p[(i / w) * ld + c0 + (i % w)] = (f16)0.0f;
}

__global__ __launch_bounds__(256) void zero_cols_u8_kernel(uint8_t* __restrict__ p, int64_t rows, int64_t ld, int c0,
                                                           int w) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * w) return;
  p[(i / w) * ld + c0 + (i % w)] = 0;  // e4m3 code of +0
}

__global__ __launch_bounds__(256) void fill_u16_kernel(uint16_t* __restrict__ p, size_t n, uint16_t v) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t j = i; j < n; j += stride) p[j] = v;
}

}  // namespace

hipError_t launch_pad_convert(const f16* x, int64_t ldx, void* y, int rows, int cols, int cols_pad,
                              bool out_fp8, float scale, hipStream_t s) {
  if (rows < 1 || cols < 1 || cols_pad < cols || (cols_pad & 3) || (cols & 3) || ldx < cols || (ldx & 3))
    return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * (cols_pad / 4);
  dim3 grid((unsigned)((n + 255) / 256));
  if (out_fp8)
    hipLaunchKernelGGL(pad_convert_kernel<true>, grid, dim3(256), 0, s, x, ldx, y, rows, cols, cols_pad, scale);
  else
    hipLaunchKernelGGL(pad_convert_kernel<false>, grid, dim3(256), 0, s, x, ldx, y, rows, cols, cols_pad, scale);
  return hipGetLastError();
}

hipError_t launch_weight_transpose(const float* w, int K, int N, void* wt, int K_pad, int N_pad,
                                   bool out_fp8, float scale, hipStream_t s) {
  if (K < 1 || N < 1 || K_pad < K || N_pad < N || (K_pad * (out_fp8 ? 1 : 2)) % 64) return hipErrorInvalidValue;
  dim3 grid((K_pad + 31) / 32, (N_pad + 31) / 32);
  if (out_fp8)
    hipLaunchKernelGGL(weight_transpose_kernel<true>, grid, dim3(256), 0, s, w, K, N, wt, K_pad, N_pad, scale);
  else
    hipLaunchKernelGGL(weight_transpose_kernel<false>, grid, dim3(256), 0, s, w, K, N, wt, K_pad, N_pad, scale);
  return hipGetLastError();
}

hipError_t launch_f32_convert(const float* x, int rows, int cols, void* y, int cols_pad, bool out_fp8,
                              float scale, hipStream_t s) {
  if (rows < 1 || cols < 1 || cols_pad < cols) return hipErrorInvalidValue;
  const int64_t n = (int64_t)rows * cols_pad;
  dim3 grid((unsigned)((n + 255) / 256));
  if (out_fp8)
    hipLaunchKernelGGL(f32_convert_kernel<true>, grid, dim3(256), 0, s, x, rows, cols, y, cols_pad, scale);
  else
    hipLaunchKernelGGL(f32_convert_kernel<false>, grid, dim3(256), 0, s, x, rows, cols, y, cols_pad, scale);
  return hipGetLastError();
}

hipError_t launch_vt_transpose(const f16* v, int64_t ld, int batch, int tokens, int width, f16* vt, int64_t vt_ld,
                               hipStream_t s) {
  auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (batch < 1 || batch > 65535 || tokens < 1 || width < 8 || (width & 7) || ld < width || (ld & 7) ||
      vt_ld < tokens || (vt_ld & 63) || !a16(v) || !a16(vt))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)((width + 63) / 64), (unsigned)(vt_ld / 64), (unsigned)batch);
  hipLaunchKernelGGL(vt_transpose_kernel, grid, dim3(256), 0, s, v, ld, tokens, width, vt, vt_ld);
  return hipGetLastError();
}

hipError_t launch_zero_cols(f16* p, int64_t rows, int64_t ld, int c0, int c1, hipStream_t s) {
  if (rows < 0 || c0 < 0 || c1 > ld || c1 < c0) return hipErrorInvalidValue;
  const int64_t n = rows * (c1 - c0);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_cols_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, rows, ld, c0, c1 - c0);
  return hipGetLastError();
}

hipError_t launch_zero_cols_u8(uint8_t* p, int64_t rows, int64_t ld, int c0, int c1, hipStream_t s) {
  if (rows < 0 || c0 < 0 || c1 > ld || c1 < c0) return hipErrorInvalidValue;
  const int64_t n = rows * (c1 - c0);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_cols_u8_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, rows, ld, c0, c1 - c0);
  return hipGetLastError();
}

hipError_t launch_fill_u16(void* p, size_t n, uint16_t value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_u16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint16_t*)p, n, value);
  return hipGetLastError();
}

}  // namespace siglip
