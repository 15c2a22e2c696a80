// Weight GEMMs of the encoder with fused epilogues, on gfx950 MFMA.
//
// Every projection on the page "Single-layer SigLIP vision benchmark"
// (intro: patch embedding + bias + positional embedding, fused QKV + bias,
// output projection + residual, MLP up + bias + GELU, MLP down + residual;
// "Fused encoder QKV and MAP KV") is one launch of this kernel. The bias,
// positional-embedding and residual additions and the GELU the page runs as
// separate Add/pointwise kernels ("Performance follow-up": bias-add cost grows
// with batch) are applied to the F32 accumulators before the single F16 (or
// e4m3) rounding of the output.
//
// Operands: A [M, K] activations and Wt [N, K] weights, both K-contiguous, both
// F16 (v_mfma_f32_32x32x16_f16) or both OCP e4m3 codes
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales; the power-of-two
// operand scale is folded into acc_scale). F32 accumulation.
//
// Tiling: a workgroup of 4 waves owns a BM x BN output tile and walks K in
// 128-byte slices (64 F16 or 128 e4m3 values per row). Slices are staged
// global -> registers -> LDS, double-buffered so the loads of slice k+1 are in
// flight while slice k is multiplied. LDS rows are 128 bytes with the 16-byte
// chunk index XOR-swizzled by (row & 7), so the 32 lanes that read one chunk
// column of 32 consecutive rows hit distinct banks.
//
// The MFMA is issued with the weight fragment as its first operand, so the
// hardware's 32x32 result holds, per lane, one activation row m and four
// consecutive output columns n per register quad: the epilogue reads bias
// and residual and writes the output 4 columns (8 bytes F16) at a time.
#include "common.h"

namespace siglip {
namespace {

constexpr int kRowBytes = 128;  // K bytes of one LDS tile row

template <int BM, int BN, int WM, int WN>
struct Tile {
  static constexpr int WAVES_N = BN / WN;
  static constexpr int WAVES_M = BM / WM;
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  static constexpr int TM = WM / 32;
  static constexpr int TN = WN / 32;
  static constexpr int A_LOADS = BM / 32;  // 16-byte global loads per thread
  static constexpr int W_LOADS = BN / 32;
  static constexpr int STAGE = (BM + BN) * kRowBytes;
};

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <int BM, int BN, int WM, int WN, bool FP8, int EPI, bool OUT_FP8>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  using T = Tile<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * T::STAGE];

  constexpr int E = FP8 ? 1 : 2;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int nk = (g.K * E) / kRowBytes;

  // ---- global -> register staging assignment: 8 threads per 128-byte row
  const int lr = t >> 3;
  const int lc = t & 7;
  const uint8_t* abase = reinterpret_cast<const uint8_t*>(g.a) + lc * 16;
  const uint8_t* wbase = reinterpret_cast<const uint8_t*>(g.w) + lc * 16;
  uint32_t aoff[T::A_LOADS];
  uint32_t woff[T::W_LOADS];
#pragma unroll
  for (int i = 0; i < T::A_LOADS; ++i) {
    int row = min(m0 + lr + 32 * i, g.M - 1);  // rows past M re-read row M-1; never stored
    aoff[i] = (uint32_t)((int64_t)row * g.lda * E);
  }
#pragma unroll
  for (int i = 0; i < T::W_LOADS; ++i)
    woff[i] = (uint32_t)((int64_t)(n0 + lr + 32 * i) * g.ldw * E);
  const int lds_st = lr * kRowBytes + swz(lr, lc) * 16;  // + 32*i rows keeps (row & 7)

  i32x4 ra[T::A_LOADS], rw[T::W_LOADS];
  auto gload = [&](int kt) {
    const int kb = kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i)
      ra[i] = *reinterpret_cast<const i32x4*>(abase + aoff[i] + kb);
#pragma unroll
    for (int i = 0; i < T::W_LOADS; ++i)
      rw[i] = *reinterpret_cast<const i32x4*>(wbase + woff[i] + kb);
  };
  auto sstore = [&](int buf) {
    uint8_t* sa = smem + buf * T::STAGE;
    uint8_t* sw = sa + BM * kRowBytes;
#pragma unroll
    for (int i = 0; i < T::A_LOADS; ++i)
      *reinterpret_cast<i32x4*>(sa + lds_st + 32 * i * kRowBytes) = ra[i];
#pragma unroll
    for (int i = 0; i < T::W_LOADS; ++i)
      *reinterpret_cast<i32x4*>(sw + lds_st + 32 * i * kRowBytes) = rw[i];
  };

  f32x16 acc[T::TM][T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int fr = lane & 31;  // fragment row inside a 32-row MFMA tile
  const int fg = lane >> 5;  // lane group: which K chunk(s) of a step
  int arow[T::TM], wrow[T::TN];
#pragma unroll
  for (int i = 0; i < T::TM; ++i) arow[i] = wm * WM + i * 32 + fr;
#pragma unroll
  for (int j = 0; j < T::TN; ++j) wrow[j] = wn * WN + j * 32 + fr;

  auto compute = [&](int buf) {
    const uint8_t* sa = smem + buf * T::STAGE;
    const uint8_t* sw = sa + BM * kRowBytes;
    if constexpr (!FP8) {
      // 4 steps of K=16: lane group fg takes chunk 2*s + fg of each row
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f16x8 af[T::TM], wf[T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
          af[i] = *reinterpret_cast<const f16x8*>(sa + arow[i] * kRowBytes + swz(arow[i], 2 * s + fg) * 16);
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          wf[j] = *reinterpret_cast<const f16x8*>(sw + wrow[j] * kRowBytes + swz(wrow[j], 2 * s + fg) * 16);
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
          for (int j = 0; j < T::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[j], af[i], acc[i][j], 0, 0, 0);
      }
    } else {
      // 2 steps of K=64: lane group fg takes chunks 4*s + 2*fg and +1. The
      // same K permutation is applied to both operands, so the sum is exact.
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        i32x8 af[T::TM], wf[T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
          i32x4 lo = *reinterpret_cast<const i32x4*>(sa + arow[i] * kRowBytes + swz(arow[i], 4 * s + 2 * fg) * 16);
          i32x4 hi = *reinterpret_cast<const i32x4*>(sa + arow[i] * kRowBytes + swz(arow[i], 4 * s + 2 * fg + 1) * 16);
          af[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
          i32x4 lo = *reinterpret_cast<const i32x4*>(sw + wrow[j] * kRowBytes + swz(wrow[j], 4 * s + 2 * fg) * 16);
          i32x4 hi = *reinterpret_cast<const i32x4*>(sw + wrow[j] * kRowBytes + swz(wrow[j], 4 * s + 2 * fg + 1) * 16);
          wf[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
          for (int j = 0; j < T::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                wf[j], af[i], acc[i][j], 0, 0, 0, 127, 0, 127);
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    compute(cur);
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds row m = tile row + fr, columns 8q + 4fg + (0..3)
#pragma unroll
  for (int i = 0; i < T::TM; ++i) {
    const int m = m0 + wm * WM + i * 32 + fr;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * fg;
        const f32x4 b = *reinterpret_cast<const f32x4*>(g.bias + n);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r] * g.acc_scale + b[r];
        if constexpr (EPI == EPI_BIAS_POS) {
          const f32x4 p = *reinterpret_cast<const f32x4*>(g.pos + (int64_t)(m % g.pos_rows) * g.ldpos + n);
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += p[r];
        }
        if constexpr (EPI == EPI_BIAS_RES) {
          const f16x4 rr = *reinterpret_cast<const f16x4*>(g.res + (int64_t)m * g.ldres + n);
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] += (float)rr[r];
        }
        if constexpr (EPI == EPI_BIAS_GELU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = gelu_tanh(v[r]);
        }
        if constexpr (OUT_FP8) {
          uint32_t w4 = pack4_e4m3(v[0] * g.out_scale, v[1] * g.out_scale,
                                   v[2] * g.out_scale, v[3] * g.out_scale);
          *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(g.c) + (int64_t)m * g.ldc + n) = w4;
        } else {
          f16x4 o = {(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
          *reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(g.c) + (int64_t)m * g.ldc + n) = o;
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, bool FP8, int EPI, bool OUT_FP8>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  dim3 grid(g.N / BN, (g.M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, FP8, EPI, OUT_FP8>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

template <bool FP8, int EPI, bool OUT_FP8>
hipError_t launch_sized(const GemmArgs& g, hipStream_t s) {
  const long tiles_l = (long)((g.M + 255) / 256) * (g.N / 128);
  const long tiles_m = (long)((g.M + 127) / 128) * (g.N / 128);
  if (tiles_l >= 1024) return launch_cfg<256, 128, 128, 64, FP8, EPI, OUT_FP8>(g, s);
  if (tiles_m >= 512) return launch_cfg<128, 128, 64, 64, FP8, EPI, OUT_FP8>(g, s);
  return launch_cfg<64, 64, 32, 32, FP8, EPI, OUT_FP8>(g, s);
}

template <bool FP8>
hipError_t launch_epi(const GemmArgs& g, int epi, bool out_fp8, hipStream_t s) {
  switch (epi) {
    case EPI_BIAS: return launch_sized<FP8, EPI_BIAS, false>(g, s);
    case EPI_BIAS_POS: return launch_sized<FP8, EPI_BIAS_POS, false>(g, s);
    case EPI_BIAS_RES: return launch_sized<FP8, EPI_BIAS_RES, false>(g, s);
    case EPI_BIAS_GELU:
      return out_fp8 ? launch_sized<FP8, EPI_BIAS_GELU, true>(g, s)
                     : launch_sized<FP8, EPI_BIAS_GELU, false>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, int epi, bool in_fp8, bool out_fp8, hipStream_t s) {
  // shape contract (checked here so no launch can index out of bounds)
  const int E = in_fp8 ? 1 : 2;
  if (g.M < 1 || g.N < 64 || g.N % 128 != 0 || g.K < 1 || (g.K * E) % kRowBytes != 0)
    return hipErrorInvalidValue;
  if (g.lda < g.K || g.ldw < g.K || g.ldc < g.N) return hipErrorInvalidValue;
  if ((int64_t)g.M * g.lda * E >= (int64_t)1 << 31 || (int64_t)g.N * g.ldw * E >= (int64_t)1 << 31)
    return hipErrorInvalidValue;
  if (out_fp8 && epi != EPI_BIAS_GELU) return hipErrorInvalidValue;
  return in_fp8 ? launch_epi<true>(g, epi, out_fp8, s) : launch_epi<false>(g, epi, out_fp8, s);
}

}  // namespace siglip
