// Internal declarations shared by the HIP sources of libsiglip (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

namespace siglip {

constexpr float kE4m3Max = 448.0f;

// Two floats -> two OCP e4m3fn codes (round to nearest even) packed into the
// low (hi=false) or high (hi=true) 16 bits of `old`. Inputs are clamped to
// +-448 first so out-of-range values saturate instead of becoming NaN.
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old, bool hi) {
  a = __builtin_amdgcn_fmed3f(a, -kE4m3Max, kE4m3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4m3Max, kE4m3Max);
  return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
            : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}

__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  uint32_t w = cvt_pk_e4m3(a, b, 0u, false);
  return cvt_pk_e4m3(c, d, w, true);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Exchange with the lane 32 positions away (l <-> l ^ 32) by
// v_permlane32_swap, no LDS round trip. The second operand is passed through
// an empty asm so that the compiler sees two distinct values: given the same
// value twice it folds the two results of the swap into one.
__device__ __forceinline__ void half_swap(float v, float* lo_half, float* hi_half) {
  unsigned a = __builtin_bit_cast(unsigned, v), b = a;
  asm volatile("" : "+v"(b));
  const auto sw = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  // (elements copied out by value first: a bit cast applied to a vector
  // element expression reinterprets element 0)
  const unsigned x0 = sw[0], x1 = sw[1];
  *lo_half = __builtin_bit_cast(float, x0);  // every lane: value of lane l % 32
  *hi_half = __builtin_bit_cast(float, x1);  // every lane: value of lane l % 32 + 32
}
__device__ __forceinline__ float half_swap_max(float v) {
  float lo, hi;
  half_swap(v, &lo, &hi);
  return fmaxf(lo, hi);
}
__device__ __forceinline__ float half_other(float v) {
  float lo, hi;
  half_swap(v, &lo, &hi);
  return __lane_id() < 32 ? hi : lo;
}

// GELU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). Since
// 0.5 (1 + tanh(z)) = 1 / (1 + exp(-2z)), this is x / (1 + exp(-2z)) with
// z = sqrt(2/pi) x (1 + 0.044715 x^2): one exp2 and one reciprocal (both
// hardware approximations, ~1 ulp of F32), no IEEE division. Large negative x
// gives exp2 -> inf and x * rcp(inf) = -0; large positive x gives x.
//
// gelu_tanh_scaled takes xs = sc * x for a power of two sc (the e4m3 output
// scale, or 1) and returns sc * gelu(x): with the exponent -2 z log2(e)
// written as xs * (k1 + k3 xs^2), k1 = -2 sqrt(2/pi) log2(e) / sc and
// k3 = k1 * 0.044715 / sc^2, the scale costs no instruction per element.
constexpr float kGeluExp2K = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
constexpr float kGeluCubic = 0.044715f;

struct GeluConsts {
  float k1, k3;
};
__device__ __forceinline__ GeluConsts gelu_consts(float sc) {
  const float k1 = kGeluExp2K / sc;
  return {k1, k1 * kGeluCubic / (sc * sc)};
}
__device__ __forceinline__ float gelu_tanh_scaled(float xs, GeluConsts k) {
  const float e = __builtin_amdgcn_exp2f(xs * fmaf(k.k3, xs * xs, k.k1));
  return xs * __builtin_amdgcn_rcpf(1.0f + e);
}

// ------------------------------------------------------------------ GEMM
// C[M, N] = epilogue(A[M, K] . Wt[N, K]^T). A and Wt are K-contiguous, either
// both F16 or both e4m3 codes. K is a multiple of 128 bytes of A row, N a
// multiple of the chosen column tile (weights are padded at create time).
enum GemmEpi : int {
  EPI_BIAS = 0,      // acc*s + bias[n]
  EPI_BIAS_POS = 1,  // acc*s + bias[n] + pos[m % pos_rows][n]
  EPI_BIAS_RES = 2,  // acc*s + bias[n] + res[m][n]
  EPI_BIAS_GELU = 3, // gelu(acc*s + bias[n])
  EPI_QKV = 4,       // acc*s + bias[n]; columns >= vt_col0 (the V part) go to
                     // vt transposed per head instead of to c (as F16, or as
                     // e4m3 codes of value*out_scale when out_fp8 is set)
  EPI_QKV8 = 5       // as EPI_QKV, with the columns < vt_col0 (Q and K) written
                     // as e4m3 codes into the head slots of qk8 instead of to c
};

struct GemmArgs {
  const void* a; int64_t lda;     // elements
  // Wt [N, K] in 64-byte K panels: byte b of row n (b = k * element size) at
  // ((b / 64) * ldw + n) * 64 + b % 64; ldw = rows per panel (>= N)
  const void* w; int64_t ldw;
  void* c; int64_t ldc;           // elements of the output type
  const float* bias;              // [N]
  const float* pos; int pos_rows; int64_t ldpos;
  const f16* res; int64_t ldres;
  int M, N, K;                    // K in elements
  float acc_scale;                // 1 (F16) or 2^(2*exp) (FP8)
  float out_scale;                // for e4m3 outputs: 2^-exp
  // EPI_QKV: V^T[(b*vt_heads + h)*vt_dim + d][t] at vt + row*vt_ld + t, for
  // output row m = b*vt_tokens + t and column vt_col0 + h*vt_dim + d; vt and
  // vt_ld count elements of the V^T type (F16, or bytes for e4m3)
  f16* vt; int vt_col0, vt_tokens, vt_heads, vt_dim; int64_t vt_ld;
  float vt_inv_dim;  // 1 / vt_dim
  int group_m;       // tile-order band height in row blocks (<= 0: N-fastest)
  // EPI_QKV8: column n < vt_col0 (head slot n / vt_dim: Q heads, then K
  // heads) is written as the e4m3 code of value*qk8_scale at byte
  // qk8 + m*qk8_ld + (n / vt_dim)*qk8_pitch + n % vt_dim
  uint8_t* qk8; int64_t qk8_ld; int qk8_pitch; float qk8_scale;
  // LayerNorm folded into the A operand (ln_stats != nullptr): a is the F16
  // residual [M, K] (lda in elements) and row m is normalized on its way into
  // LDS as fma((x - mean) * rs, ln_gamma[k], ln_beta[k] * ln_scale), with
  // {mean, rs} the two floats at ln_stats + 2m (launch_layernorm_stats), then
  // rounded to the operand type.
  const float* ln_stats; const float* ln_gamma; const float* ln_beta; float ln_scale;
};

hipError_t launch_gemm(const GemmArgs& g, int epi, bool in_fp8, bool out_fp8,
                       hipStream_t s);

// ------------------------------------------------------------- LayerNorm
hipError_t launch_layernorm(const f16* x, int64_t ldx, void* y, int64_t ldy,
                            const float* gamma, const float* beta, int rows,
                            int width, float eps, bool out_fp8, float out_scale,
                            hipStream_t s);

// Row statistics of the LayerNorm above for width 1152 only: {mean, rstd *
// scale} per row as two floats at stats + 2 row, the values
// launch_layernorm computes for the same row (hipErrorInvalidValue for
// another width).
hipError_t launch_layernorm_stats(const f16* x, int64_t ldx, float* stats, int rows, int width, float eps,
                                  float scale, hipStream_t s);

// ------------------------------------------------------------- attention
hipError_t launch_flash_attention(const f16* q, const f16* k, const f16* v,
                                  int64_t ld, void* o, int64_t ldo, int batch,
                                  int heads, int tokens, int head_dim,
                                  float scale, bool out_fp8, float out_scale,
                                  hipStream_t s);

// Encoder attention with V given transposed per head: vt row (b*heads + h)*
// head_dim + d holds keys 0..tokens-1 of that (image, head, dim), row stride
// vt_ld >= round_up(tokens, 64), zeros in columns tokens..vt_ld-1. head_dim
// must be 64, 72 or 80. With qk8_pitch = 0, q and k are F16 as for
// launch_flash_attention (ld in elements). With qk8_pitch = 80, they are
// e4m3 codes of 2^4 times the values: token row t at q + t*ld bytes, head h
// at byte h*80 (bytes head_dim..79 of a slot are never used in a product),
// ld a multiple of 16, q and k 16-byte aligned.
hipError_t launch_flash_attention_vt(const void* q, const void* k, int64_t ld, int qk8_pitch, const f16* vt,
                                     int64_t vt_ld, void* o, int64_t ldo, int batch, int heads, int tokens,
                                     int head_dim, float scale, bool out_fp8, float out_scale, hipStream_t s);

// The same streaming attention with V row-major: q, k and v F16 with one row
// stride ld (elements; a multiple of 8), head h at column h * head_dim of
// each, v 16-byte aligned; head_dim 64, 72 or 80. The kernel reads V rows
// and transposes them in its LDS reads, so no V^T buffer is needed.
hipError_t launch_flash_attention_vrow(const f16* q, const f16* k, const f16* v, int64_t ld, void* o, int64_t ldo,
                                       int batch, int heads, int tokens, int head_dim, float scale, bool out_fp8,
                                       float out_scale, hipStream_t s);

// The same with the PV product in e4m3: vt holds codes of v * v_scale (bytes,
// row stride vt_ld, a multiple of 16, zero codes in columns tokens..vt_ld-1;
// only each head's head_dim rows are read), the probabilities are quantized
// to e4m3(p * 2^4) in registers. v_scale is a power of two in (0, 256].
hipError_t launch_flash_attention_vt8(const void* q, const void* k, int64_t ld, int qk8_pitch, const uint8_t* vt,
                                      int64_t vt_ld, void* o, int64_t ldo, int batch, int heads, int tokens,
                                      int head_dim, float scale, bool out_fp8, float out_scale, float v_scale,
                                      hipStream_t s);
bool flash_attention_vt_supported(int head_dim);

hipError_t launch_map_attention(const f16* q, const f16* kv, int64_t ldkv,
                                int64_t v_offset, void* o, int64_t ldo,
                                int batch, int heads, int tokens, int head_dim,
                                float scale, bool out_fp8, float out_scale,
                                hipStream_t s);

// MAP head with the K/V projection folded (map.hip). phase 0: scores
// [batch, 16, tokens] F32 = (Z . u_h) * scale * log2(e); phase 1: softmax per
// (image, head), zbar [batch, 16, width] F32 = sum_t p_t Z_t, then
// o[b, h*head_dim + d] = zbar_h . W_v[:, h*head_dim + d] + bv (F16, or e4m3
// codes of o*out_scale). u_hi/u_lo: [16, width] F16, rows >= heads zero;
// wvt: W_v transposed, wvt[(h*head_dim + d) * width + k] = W_v[k][h*head_dim + d].
bool map_fold_supported(int width, int heads, int head_dim, int tokens);
hipError_t launch_map_fold(const f16* z, int64_t ldz, const f16* u_hi, const f16* u_lo, const float* wvt,
                           const float* bv, float* scores, float* zbar, int batch, int tokens, int heads,
                           int head_dim, int width, float scale, bool out_fp8, float out_scale, void* o,
                           int64_t ldo, hipStream_t s, int phase);

// Create-time constants of the folded MAP head from the F32 blob tensors on
// the device: q = probe Wq + bq (F32, and F16 in q16), u_hi/u_lo [16, width]
// as for launch_map_fold, wvt [width, width] = W_v transposed. wkv is the
// fused [width, 2 width] K/V weight.
hipError_t launch_map_fold_prepare(const float* probe, const float* wq, const float* bq, const float* wkv, int width,
                                   int heads, int head_dim, float* q, f16* q16, f16* u_hi, f16* u_lo, float* wvt,
                                   hipStream_t s);

// ------------------------------------------------------------ conversion
// F16 [rows, cols] (row stride ldx) -> [rows, cols_pad] F16 or e4m3 codes of
// x*scale, columns cols..cols_pad-1 set to zero.
hipError_t launch_pad_convert(const f16* x, int64_t ldx, void* y, int rows,
                              int cols, int cols_pad, bool out_fp8, float scale,
                              hipStream_t s);

// F32 weight [K, N] -> Wt [N_pad, K_pad] (F16 or e4m3 codes of w*scale,
// zero in the padding) in 64-byte K panels: byte b of row n at
// ((b / 64) * N_pad + n) * 64 + b % 64 (K_pad * element size a multiple of
// 64), so that any 64-byte-aligned K slice of consecutive rows is one
// contiguous run per panel.
hipError_t launch_weight_transpose(const float* w, int K, int N, void* wt,
                                   int K_pad, int N_pad, bool out_fp8,
                                   float scale, hipStream_t s);

// F32 [rows, cols] -> [rows, cols_pad] F16 or e4m3 codes of x*scale.
hipError_t launch_f32_convert(const float* x, int rows, int cols, void* y,
                              int cols_pad, bool out_fp8, float scale,
                              hipStream_t s);

// V [batch, tokens, width] F16 (row stride ld elements, a multiple of 8) ->
// vt [batch * width, vt_ld]: row b * width + c holds column c of image b for
// tokens 0..tokens-1 and zeros in columns tokens..vt_ld-1 (vt_ld a multiple
// of 64). With width = heads * head_dim, row (b heads + h) head_dim + d is
// the V^T row of launch_flash_attention_vt. 16-byte aligned v and vt.
hipError_t launch_vt_transpose(const f16* v, int64_t ld, int batch, int tokens, int width, f16* vt, int64_t vt_ld,
                               hipStream_t s);

// Zero columns c0..c1-1 of every row of an F16 [rows, ld] matrix.
hipError_t launch_zero_cols(f16* p, int64_t rows, int64_t ld, int c0, int c1, hipStream_t s);
// The same for a byte matrix (e4m3 codes): columns [c0, c1) of rows rows.
hipError_t launch_zero_cols_u8(uint8_t* p, int64_t rows, int64_t ld, int c0, int c1, hipStream_t s);

// Fill n 16-bit words.
hipError_t launch_fill_u16(void* p, size_t n, uint16_t value, hipStream_t s);

}  // namespace siglip
