// Attention kernels.
//
// flash_attn: encoder self-attention, softmax(Q K^T * scale) V per image and
// head, T = 729 tokens, head width 72 (page "Single-layer SigLIP vision
// benchmark", intro). Softmax state (running maximum, denominator) and the
// accumulator stay F32 and the result is converted to F16 once (same page,
// precision paragraph); the blocked/online merge of the pages' attention
// (page "Capacity-first baseline", "Correctness fixes": running maximum and
// denominator kept with each accumulator row) is done here in registers, so
// no probability or score tensor is ever written to memory.
//
// Padding: head width 72 is padded to 80 for the QK contraction and to 96
// for the PV output, keys to a multiple of 64, queries to a multiple of 128.
// Every pad value is a zero written by this kernel into registers or LDS,
// keys past T are masked to -inf before the maximum, so no data past token
// T-1 of an image or column 71 of a head is ever read (the pages' PV-padding
// NaN came from reading stale statistics as F16: page "SigLIP optimized
// execution and PV padding", "Cause and fix").
//
// Work split: a workgroup of 4 waves takes 128 queries of one (image, head);
// each wave owns 32 queries. Per block of 64 keys the workgroup stages K
// [64 x 80] and V transposed [96 x 64] in LDS; each wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_f16 (keys on the MFMA rows, so every
// lane holds 16 scores of ONE query and the row max / sum need one
// cross-half shuffle), rescales, and computes O^T += V^T P^T where the P
// fragment is the F32 score registers converted to F16 in place (the K
// order inside a 16-key step is chosen to match the score layout, and V^T
// is read in that same order). The small-batch kernel's row-major V form
// (VROW) reads V in its token rows and transposes it in the LDS reads
// instead, with the same products in the same order.
//
// Padding work that is skipped: a wave whose queries all lie past T only
// helps move K and V into LDS, and a last key block whose second 32-key half
// lies past T leaves that half out (its probabilities would be exact zeros).
#include "common.h"

#include <type_traits>

namespace siglip {
namespace {

constexpr int QB = 128;   // queries per workgroup
constexpr int KB = 64;    // keys per block
constexpr int KST = 88;   // K tile row stride in halfs (176 B: conflict-free 16-B reads)
constexpr int VROWS = 96; // padded head width of the PV output (3 x 32)
constexpr int VST = 68;   // V^T tile row stride in halfs (136 B)
constexpr float kNegInf = -__builtin_inff();

// One 16-byte global -> LDS transfer per lane (global_load_lds_dwordx4): the
// wave writes 64 x 16 bytes contiguously from lds_wave_base, lane i at +16 i.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// Linear workgroup id -> logical block, XCD-aware: workgroups are dispatched
// round-robin over the 8 XCDs; the remap gives each XCD a contiguous range of
// logical blocks, so the query blocks of one (image, head) share an L2 and
// read that head's K and V from HBM once.
__device__ __forceinline__ int xcd_block(int id, int total) {
  const int total8 = total & ~7;
  return id < total8 ? (id & 7) * (total8 >> 3) + (id >> 3) : id;
}

template <bool OUT_FP8>
__global__ __launch_bounds__(256, 2) void flash_attn_kernel(
    const f16* __restrict__ q, const f16* __restrict__ k, const f16* __restrict__ v, int64_t ld,
    void* __restrict__ o, int64_t ldo, int T, int D, int H, int nqb, float c, float out_scale) {
  __shared__ __attribute__((aligned(16))) f16 Ks[2][KB * KST];
  __shared__ __attribute__((aligned(16))) f16 Vt[2][VROWS * VST];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int fr = lane & 31;
  const int fg = lane >> 5;
  const int L = xcd_block(blockIdx.x, gridDim.x);
  const int qb = L % nqb;
  const int bh = L / nqb;
  const int h = bh % H;
  const int b = bh / H;
  const int hc = h * D;
  const int64_t img = (int64_t)b * T;
  const int qi = qb * QB + wave * 32 + fr;  // this lane's query

  // Q fragments: query qi, head dims 16s + 8fg .. +7 (zero past D and T)
  f16x8 qf[5];
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const int d0 = 16 * s + 8 * fg;
    if (qi < T && d0 < D)
      qf[s] = *reinterpret_cast<const f16x8*>(q + (img + qi) * ld + hc + d0);
    else
      qf[s] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  // V^T rows D..95 stay zero for the whole kernel (both buffers)
  for (int i = t; i < 2 * (VROWS - D) * VST; i += 256) {
    const int bsel = i / ((VROWS - D) * VST), r = i % ((VROWS - D) * VST);
    Vt[bsel][D * VST + r] = (f16)0.0f;
  }

  // ---- staging of one 64-key block into registers, then into LDS.
  // K: 64 keys x 10 chunks of 8 dims (zero past D), 3 chunks per thread.
  // V: thread t < 8*nvc owns 8 consecutive keys x one 8-dim chunk and writes
  //    it transposed (8 rows of V^T, 8 keys each).
  const int nvc = D >> 3;
  const bool vown = t < 8 * nvc;
  const int vkg = t / max(nvc, 1), vc = t % max(nvc, 1);
  i32x4 kr[3];
  f16x8 vr[8];
  auto gload = [&](int key0) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int cidx = t + 256 * i;
      const int key = cidx / 10, ch = cidx % 10;
      const int kk = key0 + key;
      kr[i] = i32x4{0, 0, 0, 0};
      if (cidx < KB * 10 && kk < T && ch * 8 < D)
        kr[i] = *reinterpret_cast<const i32x4*>(k + (img + kk) * ld + hc + ch * 8);
    }
    if (vown) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int kk = key0 + 8 * vkg + j;
        vr[j] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (kk < T) vr[j] = *reinterpret_cast<const f16x8*>(v + (img + kk) * ld + hc + 8 * vc);
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int cidx = t + 256 * i;
      if (cidx < KB * 10) {
        const int key = cidx / 10, ch = cidx % 10;
        *reinterpret_cast<i32x4*>(&Ks[buf][key * KST + ch * 8]) = kr[i];
      }
    }
    if (vown) {
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const f16x4 lo = {vr[0][dd], vr[1][dd], vr[2][dd], vr[3][dd]};
        const f16x4 hi = {vr[4][dd], vr[5][dd], vr[6][dd], vr[7][dd]};
        f16* row = &Vt[buf][(8 * vc + dd) * VST + 8 * vkg];
        *reinterpret_cast<f16x4*>(row) = lo;
        *reinterpret_cast<f16x4*>(row + 4) = hi;
      }
    }
  };

  float m_run = kNegInf, l_run = 0.0f;
  f32x16 oacc[3];
#pragma unroll
  for (int dt = 0; dt < 3; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;

  const int nkb = (T + KB - 1) / KB;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int buf = kb & 1;
    const int key0 = kb * KB;
    if (kb + 1 < nkb) gload(key0 + KB);  // next block in flight during this one

    // S^T[key][query] (raw dot products) for keys key0 + 32kt + (8(r/4) + 4fg + r%4)
    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.0f;
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        const f16x8 kf = *reinterpret_cast<const f16x8*>(&Ks[buf][(32 * kt + fr) * KST + 16 * s + 8 * fg]);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[s], sacc[kt], 0, 0, 0);
      }
    }
    if (key0 + KB > T) {  // only the last block holds keys past T
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + 32 * kt + 8 * (r >> 2) + 4 * fg + (r & 3) >= T) sacc[kt][r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kt][r]);
    mx = half_swap_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float mc = m_new * c;
    float ls = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], c, -mc));  // exp(scale (s - m))
        sacc[kt][r] = p;
        ls += p;
      }
    ls += half_other(ls);
    if (!__all(m_new == m_run)) {  // some row's maximum moved: rescale the state
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 3; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
    }
    l_run += ls;
    m_run = m_new;

    // O^T[d][query] += V^T[d][keys] P^T[keys][query], 16 keys per step; the
    // lane group fg slots hold keys 16s + 4fg + (0..3) then 16s + 8 + 4fg + (0..3)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kt = s >> 1, base = 8 * (s & 1);
      f16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = (f16)sacc[kt][base + e];
#pragma unroll
      for (int dt = 0; dt < 3; ++dt) {
        const f16* vrow = &Vt[buf][(32 * dt + fr) * VST + 16 * s + 4 * fg];
        const f16x4 lo = *reinterpret_cast<const f16x4*>(vrow);
        const f16x4 hi = *reinterpret_cast<const f16x4*>(vrow + 8);
        const f16x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf, oacc[dt], 0, 0, 0);
      }
    }
    if (kb + 1 < nkb) sstore(buf ^ 1);  // the other buffer was last read in block kb-1
    __syncthreads();
  }

  if (qi >= T) return;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int dt = 0; dt < 3; ++dt)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = 32 * dt + 8 * qd + 4 * fg;
      if (d0 >= D) continue;
      const float a0 = oacc[dt][4 * qd + 0] * inv, a1 = oacc[dt][4 * qd + 1] * inv;
      const float a2 = oacc[dt][4 * qd + 2] * inv, a3 = oacc[dt][4 * qd + 3] * inv;
      if constexpr (OUT_FP8) {
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(o) + (img + qi) * ldo + hc + d0) =
            pack4_e4m3(a0 * out_scale, a1 * out_scale, a2 * out_scale, a3 * out_scale);
      } else {
        const f16x4 ov = {(f16)a0, (f16)a1, (f16)a2, (f16)a3};
        *reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(o) + (img + qi) * ldo + hc + d0) = ov;
      }
    }
}

// ---------------------------------------------------------------------------
// Encoder attention with V already transposed per head (written that way by
// the QKV GEMM epilogue). Both operands of a 64-key block then stream
// global -> LDS with global_load_lds_dwordx4 into a 3-stage ring, exactly as
// the GEMM operands do: no register staging and no transposition here.
//
// LDS stage (bytes): K [64 rows x 176] (11 chunks of 16 B per key: 9 chunks of
// dims, then copies of the last dim chunk, which meet the zero Q padding), then
// V^T [96 dims x 128] (64 keys per row, 16-byte chunk index XOR-swizzled as in
// the GEMM; row D is ones and rows D+1..95 zeros, written once). Keys past T
// read token T-1 (finite, masked to -inf); V^T columns past T are zeros in
// memory.
//
// K rows are stored permuted within each 16-row group (rows 4..7 hold keys
// 8..11 and rows 8..11 keys 4..7). The S^T result puts tile rows
// 16s + 8(e/4) + 4g + e%4 in element e of lane group g; with the permutation
// those are keys 16s + 8g + e, eight consecutive keys, so each V^T fragment
// of the PV product is one 16-byte LDS read.
constexpr int VK_PITCH = 176;
constexpr int VK_BYTES = KB * VK_PITCH;          // 11 x 1 KiB
constexpr int VV_PITCH = 128;
constexpr int VT_STAGE = VK_BYTES + VROWS * VV_PITCH;
constexpr int VT_STAGES_DEFAULT = 2;  // 48 KiB per workgroup: three workgroups per CU
// e4m3 Q and K (QK8): a key's codes sit in a head slot of kQK8Pitch bytes (dims
// 0..D-1, the rest not read into an MFMA operand); the K stage holds 64 such
// rows, and each 32-key score tile takes two 32x32x64 e4m3 MFMAs (dims 0..63,
// then dims 64..D-1 with zero-filled operand bytes above D).
constexpr int kQK8Pitch = 80;
constexpr int VK8_BYTES = KB * kQK8Pitch;        // 5 x 1 KiB

// i32x8 fragment of 32 e4m3 codes at p (two 16-byte reads)
__device__ __forceinline__ i32x8 load32b(const uint8_t* p) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// second K-step fragment of a D-dim row (dims 64..95 for lane group 0, zero
// for lane group 1): only the D - 64 real code bytes at p + 64 are read
template <int D>
__device__ __forceinline__ i32x8 load_tail8(const uint8_t* p, int fg) {
  static_assert(D == 64 || D == 72 || D == 80, "head width");
  i32x8 f = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (D == 72) {
    const uint2 w = *reinterpret_cast<const uint2*>(p + 64);
    if (fg == 0) { f[0] = (int)w.x; f[1] = (int)w.y; }
  } else if constexpr (D == 80) {
    const i32x4 w = *reinterpret_cast<const i32x4*>(p + 64);
    if (fg == 0) { f[0] = w[0]; f[1] = w[1]; f[2] = w[2]; f[3] = w[3]; }
  }
  return f;
}

// key held by K tile row i (see the permutation above)
__device__ __forceinline__ int key_of_row(int i) {
  const int x = i & 15;
  return (i & ~15) + ((x >= 4 && x < 8) ? x + 4 : (x >= 8 && x < 12) ? x - 4 : x);
}
__device__ __forceinline__ int vswz_key(int d) { return (d & 7) ^ ((d >> 3) & 1); }

template <int N>
__device__ __forceinline__ void attn_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Row-major V (VROW). A stage's V part holds the block's 64 key rows, in key
// order, kVRowPitch bytes each: dims 0..D-1 of the key, then the chunk
// {1, 0, ..., 0} at dim D (the PV product then also yields each query's
// probability sum) and zero chunks up to dim 95. The padding chunks are
// written once per stage (vrow_pad); the transfer lanes that would land on
// them are masked off.
// Transposing LDS reads (ds_read_b64_tr_b16) give the PV A operand: within
// each 16-lane group, lane a + 4r reads four dims of key k + r, and lane
// 4a + b receives dim b of those four keys. With a 192-byte pitch, four
// consecutive rows start in four distinct 64-byte bank ranges.
constexpr int kVRowPitch = 192;
constexpr int VR_BYTES = KB * kVRowPitch;  // 12 KiB

// the padding chunks (NDC .. 11) of the 64 V rows of `stages` stages of
// `stage_bytes` whose V part starts at vbase; threads t = 0 .. nthreads - 1
template <int NDC>
__device__ __forceinline__ void vrow_pad(uint8_t* smem, int stages, int stage_bytes, int vbase, int t, int nthreads) {
  constexpr int PC = kVRowPitch / 16 - NDC;  // padding chunks per row
  for (int i = t; i < stages * KB * PC; i += nthreads) {
    const int c = i % PC, r = (i / PC) % KB, st = i / (PC * KB);
    const int one = c == 0 ? 0x3C00 : 0;  // F16 1 in the first dim of the first padding chunk
    *reinterpret_cast<i32x4*>(smem + st * stage_bytes + vbase + r * kVRowPitch + (NDC + c) * 16) =
        i32x4{one, 0, 0, 0};
  }
}

// four F16 of four consecutive rows (see above), as one half of an f16x8 operand
__device__ __forceinline__ f16x4 ds_read_tr4(const uint8_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<uint8_t*>(p)));
  return __builtin_bit_cast(f16x4, r);
}
__device__ __forceinline__ f16x8 cat8(f16x4 lo, f16x4 hi) {
  return f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// QK8: q and k are e4m3 codes (head h of a token row at byte h * kQK8Pitch,
// ld in bytes), their products scaled into c by the caller.
template <int D, bool OUT_FP8, int VT_STAGES = VT_STAGES_DEFAULT, int MIN_WG = 3, int QT = 1, bool QK8 = false>
__global__ __launch_bounds__(256, MIN_WG) void flash_attn_vt_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv, int64_t ld, const f16* __restrict__ vt,
    int64_t vt_ld, void* __restrict__ o, int64_t ldo, int T, int H, int nqb, float c, float out_scale) {
  static_assert(D % 8 == 0 && D <= 80 && D >= 64, "head width");
  static_assert(QT == 1 || QT == 2, "query tiles per wave");
  static_assert(!QK8 || QT == 1, "e4m3 Q/K with one query tile per wave");
  constexpr int QWG = 4 * 32 * QT;               // queries per workgroup
  constexpr int NDC = D / 8;                     // 16-byte dim chunks per key
  constexpr int KBYTES = QK8 ? VK8_BYTES : VK_BYTES;
  constexpr int STAGE = KBYTES + VROWS * VV_PITCH;
  constexpr int NK = KBYTES / 1024;              // 1 KiB transfers for K per stage
  static_assert(KBYTES % 1024 == 0, "whole K transfers");
  constexpr int NDMA = NK + D / 8;               // 1 KiB transfers per stage
  constexpr int PER_WAVE = (NDMA + 3) / 4;       // every wave issues the same count
  constexpr int RL = (D - 64) / 2;               // oacc[.][2] register holding O^T row D (lane group 0)
  constexpr float kTau = 8.0f;                   // rescale only when a row max grows by > 2^8
  __shared__ __attribute__((aligned(1024))) uint8_t smem[VT_STAGES * STAGE + 1024];
  uint8_t* trash = smem + VT_STAGES * STAGE;     // target of the padding transfers
  const f16* q = static_cast<const f16*>(qv);
  const f16* k = static_cast<const f16*>(kv);
  const uint8_t* kb8 = static_cast<const uint8_t*>(kv);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int fr = lane & 31;
  const int fg = lane >> 5;
  const int L = xcd_block(blockIdx.x, gridDim.x);
  const int qb = L % nqb;
  const int bh = L / nqb;
  const int h = bh % H;
  const int b = bh / H;
  const int hc = h * D;
  const int64_t img = (int64_t)b * T;
  int qi[QT];
#pragma unroll
  for (int u = 0; u < QT; ++u) qi[u] = qb * QWG + (wave * QT + u) * 32 + fr;
  const f16* vth = vt + (int64_t)bh * D * vt_ld;  // this head's V^T rows

  f16x8 qf[QT][5];
  i32x8 q8[2];
  if constexpr (QK8) {
    const uint8_t* qrow = static_cast<const uint8_t*>(qv) + (img + qi[0]) * ld + h * kQK8Pitch;
    q8[0] = q8[1] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (qi[0] < T) {
      q8[0] = load32b(qrow + 32 * fg);
      q8[1] = load_tail8<D>(qrow, fg);
    }
  } else {
#pragma unroll
    for (int u = 0; u < QT; ++u)
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        const int d0 = 16 * s + 8 * fg;
        if (qi[u] < T && d0 < D)
          qf[u][s] = *reinterpret_cast<const f16x8*>(q + (img + qi[u]) * ld + hc + d0);
        else
          qf[u][s] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
  }
  // The Q fragments must be complete before the block loop: an explicit,
  // compiler-visible wait here keeps the compiler from inserting a full
  // vmcnt(0) before the first MFMA of every block, which would also drain
  // the transfers prefetching later blocks.
  __builtin_amdgcn_s_waitcnt(0);
  // constant V^T rows of every stage: row D = 1 (the PV product then also
  // yields each query's sum of the F16 probabilities it used), rows D+1..95 = 0
  constexpr int ZCH = (VROWS - D) * VV_PITCH / 16;
  for (int i = t; i < VT_STAGES * ZCH; i += 256) {
    const int r = i % ZCH;
    uint8_t* z = smem + (i / ZCH) * STAGE + KBYTES + D * VV_PITCH + r * 16;
    const int one = 0x3C003C00;  // two F16 ones
    *reinterpret_cast<i32x4*>(z) = r < VV_PITCH / 16 ? i32x4{one, one, one, one} : i32x4{0, 0, 0, 0};
  }
  __syncthreads();

  // ---- transfer slots (slot j of this wave: global index jg = wave + 4 j).
  // Sources are kept without the block offset: a K slot advances by key0 rows,
  // a V^T slot by key0 columns, a padding slot not at all.
  const f16* src[PER_WAVE];
  int kkey[PER_WAVE], kdc[PER_WAVE];
  const int vd_lo = lane >> 3;
  const int vchunk = lane & 7;
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int jg = wave + 4 * j;
    const int off = jg * 1024 + 16 * lane;
    if constexpr (QK8) {  // K row of kQK8Pitch code bytes: 5 chunks of 16
      kkey[j] = key_of_row(off / kQK8Pitch);
      kdc[j] = (off % kQK8Pitch) / 16;
    } else {
      kkey[j] = key_of_row(off / VK_PITCH);
      kdc[j] = min((off % VK_PITCH) / 16, NDC - 1);
    }
    if (jg < NK) {
      if constexpr (QK8)
        src[j] = reinterpret_cast<const f16*>(kb8 + (img + kkey[j]) * ld + h * kQK8Pitch + 16 * kdc[j]);
      else
        src[j] = k + (img + kkey[j]) * ld + hc + 8 * kdc[j];
    } else if (jg < NDMA) {
      const int d = 8 * (jg - NK) + vd_lo;
      src[j] = vth + (int64_t)d * vt_ld + 8 * (vchunk ^ vswz_key(d));
    } else {
      src[j] = vth;
    }
  }
  // bytes a slot's source advances per key (uniform): K rows by ld, V^T
  // columns by one F16, padding slots not at all
  int64_t kstep[PER_WAVE];
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int jg = wave + 4 * j;
    kstep[j] = jg < NK ? (QK8 ? ld : 2 * ld) : jg < NDMA ? 2 : 0;
  }
  auto issue = [&](int kb) {
    const int key0 = kb * KB;
    uint8_t* st = smem + (kb % VT_STAGES) * STAGE;
    const bool tail = key0 + KB > T;  // keys past T re-read token T-1
    if (!tail) {
      // every slot lands at its KiB of the stage (the V^T part starts at
      // NK KiB), padding slots in the trash KiB: no per-slot branches
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int jg = wave + 4 * j;
        dma16(reinterpret_cast<const uint8_t*>(src[j]) + key0 * kstep[j], jg < NDMA ? st + jg * 1024 : trash);
      }
      return;
    }
    // the last block: K rows past T re-read token T-1 (V^T columns past T
    // are zeros in memory)
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int jg = wave + 4 * j;
      if (jg < NK) {
        if constexpr (QK8)
          dma16(kb8 + (img + min(key0 + kkey[j], T - 1)) * ld + h * kQK8Pitch + 16 * kdc[j], st + jg * 1024);
        else
          dma16(k + (img + min(key0 + kkey[j], T - 1)) * ld + hc + 8 * kdc[j], st + jg * 1024);
      } else {
        dma16(reinterpret_cast<const uint8_t*>(src[j]) + key0 * kstep[j], jg < NDMA ? st + jg * 1024 : trash);
      }
    }
  };

  // per-lane LDS byte offsets of the fragments inside a stage
  const int koff = fr * VK_PITCH + fg * 16;                      // + kt*32*176 + s*32
  int voff[4];                                                   // + dt*32*128
#pragma unroll
  for (int s = 0; s < 4; ++s) voff[s] = KBYTES + fr * VV_PITCH + 16 * ((2 * s + fg) ^ vswz_key(fr));

  float m_run[QT];
  f32x16 oacc[QT][3];
#pragma unroll
  for (int u = 0; u < QT; ++u) {
    m_run[u] = kNegInf;
#pragma unroll
    for (int dt = 0; dt < 3; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[u][dt][r] = 0.0f;
  }

  // One 64-key block. NKT: 32-key score tiles that hold a key below T (2,
  // or 1 for a last block whose second half is all padding: its scores
  // would be -inf, its probabilities 0 and its products exact zeros, so
  // leaving that half out gives the same bits).
  auto block = [&](const uint8_t* st, int key0, auto nkt_tag, auto tail_tag) {
    constexpr int NKT = decltype(nkt_tag)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;  // the last block: keys past T masked
    // S^T for every query tile; each K fragment read feeds QT MFMAs
    f32x16 sacc[QT][NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int u = 0; u < QT; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[u][kt][r] = 0.0f;
      if constexpr (QK8) {
        const uint8_t* kr = st + (kt * 32 + fr) * kQK8Pitch;
        sacc[0][kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(load32b(kr + 32 * fg), q8[0], sacc[0][kt],
                                                                      0, 0, 0, 127, 0, 127);
        if constexpr (D > 64)
          sacc[0][kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(load_tail8<D>(kr, fg), q8[1], sacc[0][kt],
                                                                        0, 0, 0, 127, 0, 127);
      } else {
#pragma unroll
        for (int s = 0; s < 5; ++s) {
          const f16x8 kf = *reinterpret_cast<const f16x8*>(st + koff + kt * 32 * VK_PITCH + s * 32);
#pragma unroll
          for (int u = 0; u < QT; ++u)
            sacc[u][kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[u][s], sacc[u][kt], 0, 0, 0);
        }
      }
    }
    if (TAIL && key0 + KB > T) {
#pragma unroll
      for (int u = 0; u < QT; ++u)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + key_of_row(32 * kt + 8 * (r >> 2) + 4 * fg + (r & 3)) >= T) sacc[u][kt][r] = kNegInf;
    }
    float mc[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      float a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a[i] = fmaxf(sacc[u][0][i], sacc[u][0][i + 8]);
        if constexpr (NKT == 2) a[i] = fmaxf(a[i], fmaxf(sacc[u][NKT - 1][i], sacc[u][NKT - 1][i + 8]));
      }
      float mx = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7])));
      mx = half_swap_max(mx);
      // Probabilities are exp(scale (s - m_run)) with a running reference
      // m_run that only moves when a row maximum exceeds it by more than 2^8
      // in exp2 units, so they stay <= 2^8; the final division by the row sum
      // makes the result independent of the reference.
      if (__any((mx - m_run[u]) * c > kTau)) {
        const float m_new = fmaxf(m_run[u], mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run[u] - m_new) * c);
#pragma unroll
        for (int dt = 0; dt < 3; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[u][dt][r] *= alpha;
        m_run[u] = m_new;
      }
      mc[u] = m_run[u] * c;
    }

#pragma unroll
    for (int s = 0; s < 2 * NKT; ++s) {
      const int kt = s >> 1, base = 8 * (s & 1);
      f16x8 pf[QT];
#pragma unroll
      for (int u = 0; u < QT; ++u)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          typedef float f32x2 __attribute__((ext_vector_type(2)));
          const f32x2 pp = {__builtin_amdgcn_exp2f(fmaf(sacc[u][kt][base + e], c, -mc[u])),
                            __builtin_amdgcn_exp2f(fmaf(sacc[u][kt][base + e + 1], c, -mc[u]))};
          const f16x2 ph = __builtin_convertvector(pp, f16x2);
          pf[u][e] = ph[0];
          pf[u][e + 1] = ph[1];
        }
#pragma unroll
      for (int dt = 0; dt < 3; ++dt) {  // keys 16s + 8fg + (0..7) of dim row 32dt + fr
        const f16x8 vf = *reinterpret_cast<const f16x8*>(st + voff[s] + dt * 32 * VV_PITCH);
#pragma unroll
        for (int u = 0; u < QT; ++u)
          oacc[u][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[u], oacc[u][dt], 0, 0, 0);
      }
    }
  };

  // A wave whose queries all lie past T only moves K/V^T for the others.
  // The last block (keys past T masked, possibly only its first half) runs
  // after the loop, so the loop holds one form of the block.
  const bool active = qb * QWG + wave * QT * 32 < T;
  const int nkb = (T + KB - 1) / KB;
  using full = std::integral_constant<int, 2>;
  using half = std::integral_constant<int, 1>;
  using yes = std::true_type;
  using no = std::false_type;
#pragma unroll
  for (int p = 0; p < VT_STAGES - 1; ++p)
    if (p < nkb) issue(p);
  for (int kb = 0; kb < nkb - 1; ++kb) {
    if (kb + VT_STAGES - 2 < nkb)
      attn_wait_vmcnt<(VT_STAGES - 2) * PER_WAVE>();
    else
      attn_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kb + VT_STAGES - 1 < nkb) issue(kb + VT_STAGES - 1);  // into the stage block kb-1 used
    if (active) block(smem + (kb % VT_STAGES) * STAGE, kb * KB, full(), no());
  }
  {
    const int kb = nkb - 1, key0 = kb * KB;
    attn_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const uint8_t* st = smem + (kb % VT_STAGES) * STAGE;
    if (active) {
      if (key0 + 32 >= T)
        block(st, key0, half(), yes());
      else
        block(st, key0, full(), yes());
    }
  }

#pragma unroll
  for (int u = 0; u < QT; ++u) {
    // the row sum sits in O^T row D, register RL of lane group 0
    const float lsum0 = oacc[u][2][RL];
    const float lsum1 = half_other(lsum0);
    if (qi[u] >= T) continue;
    const float inv = 1.0f / (fg ? lsum1 : lsum0);
#pragma unroll
    for (int dt = 0; dt < 3; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * dt + 8 * qd + 4 * fg;
        if (d0 >= D) continue;
        const float a0 = oacc[u][dt][4 * qd + 0] * inv, a1 = oacc[u][dt][4 * qd + 1] * inv;
        const float a2 = oacc[u][dt][4 * qd + 2] * inv, a3 = oacc[u][dt][4 * qd + 3] * inv;
        if constexpr (OUT_FP8) {
          *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(o) + (img + qi[u]) * ldo + hc + d0) =
              pack4_e4m3(a0 * out_scale, a1 * out_scale, a2 * out_scale, a3 * out_scale);
        } else {
          const f16x4 ov = {(f16)a0, (f16)a1, (f16)a2, (f16)a3};
          *reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(o) + (img + qi[u]) * ldo + hc + d0) = ov;
        }
      }
  }
}

// ---------------------------------------------------------------------------
// e4m3 PV product (page "FP8 attention and resident image/embedding
// transfers": F143 operands at scale -4 for the PV product, with the softmax,
// its F32 state and the output precision unchanged; "Full 27-layer ViT": a
// profitable form has the producers write the quantized operands). Here the
// QKV GEMM epilogue writes V^T as e4m3 codes of v * 2^-exp and the
// probabilities are quantized in registers as e4m3 codes of p * 2^4, so no
// cast pass exists; one v_mfma_scale_f32_32x32x64_f8f6f4 per 32 head dims
// covers a whole 64-key block (four F16 MFMAs otherwise). QK stays F16.
//
// Same work split and K streaming as flash_attn_vt_kernel, with another K row
// order: tile kt row i holds key 32 ((i >> 2) & 1) + 16 kt + 4 (i >> 3) + (i & 3),
// so lane group g of a score tile holds the keys 32 g + 16 kt + r (r = 0..15)
// and its 32 probabilities of the block are keys 32 g .. 32 g + 31 in order:
// the P^T fragment of the MFMA, and the matching V^T fragment is bytes
// 32 g .. 32 g + 31 of a V^T row (two 16-byte LDS reads).
//
// V^T stage: 80 rows of 64 key bytes, 16-byte chunks swizzled by
// (row >> 2) & 3 (16 consecutive rows read one chunk without bank conflicts).
// The transfers fill whole 16-row groups, so rows D..79 are copies of the
// head's row D-1 (the source row is clamped: nothing outside the head's D
// rows is read); they reach only rows D..79 of O^T, which are never read.
// Row 80 holds e4m3(2^-exp), so the
// same MFMA yields each query's sum of its quantized probabilities (the scales
// 2^4 and 2^-exp cancel in the division); rows 81..95 are zero.
//
// The probabilities stay <= 2^4: the running reference moves when a block's
// maximum exceeds it by more than 4 in exp2 units, so 2^4 p <= 256 < 448 and
// the codes never saturate.
constexpr int VV8_ROWS_DMA = 80;                 // V^T rows streamed per block
constexpr int VV8_PITCH = 64;                    // bytes per V^T row of a block
constexpr int VT8_STAGE = VK_BYTES + VROWS * VV8_PITCH;

__device__ __forceinline__ int key_of_row8(int row) {
  const int kt = row >> 5, i = row & 31;
  return 32 * ((i >> 2) & 1) + 16 * kt + 4 * (i >> 3) + (i & 3);
}
__device__ __forceinline__ int vswz8(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

template <int D, bool OUT_FP8, bool QK8 = false>
__global__ __launch_bounds__(256, 3) void flash_attn_vt8_kernel(
    const void* __restrict__ qv, const void* __restrict__ kv, int64_t ld, const uint8_t* __restrict__ vt,
    int64_t vt_ld, void* __restrict__ o, int64_t ldo, int T, int H, int nqb, float c, float out_scale,
    float v_scale) {
  static_assert(D % 8 == 0 && D <= 80 && D >= 64, "head width");
  constexpr int STAGES = 2;
  constexpr int QWG = 4 * 32;                    // queries per workgroup
  constexpr int NDC = D / 8;                     // 16-byte dim chunks per key (F16 K)
  constexpr int KBYTES = QK8 ? VK8_BYTES : VK_BYTES;
  constexpr int STAGE = KBYTES + VROWS * VV8_PITCH;
  constexpr int NK = KBYTES / 1024;              // 1 KiB transfers for K per stage
  constexpr int NV = VV8_ROWS_DMA * VV8_PITCH / 1024;  // 1 KiB transfers for V^T per stage
  constexpr int NDMA = NK + NV;
  constexpr int PER_WAVE = (NDMA + 3) / 4;
  constexpr int RL = 8;                          // oacc[2] register holding O^T row 80 (lane group 0)
  constexpr float kTau = 4.0f;                   // probabilities stay <= 2^4
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE + 1024];
  uint8_t* trash = smem + STAGES * STAGE;
  const f16* q = static_cast<const f16*>(qv);
  const f16* k = static_cast<const f16*>(kv);
  const uint8_t* kb8 = static_cast<const uint8_t*>(kv);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int fr = lane & 31;
  const int fg = lane >> 5;
  const int L = xcd_block(blockIdx.x, gridDim.x);
  const int qb = L % nqb;
  const int bh = L / nqb;
  const int h = bh % H;
  const int b = bh / H;
  const int hc = h * D;
  const int64_t img = (int64_t)b * T;
  const int qi = qb * QWG + wave * 32 + fr;
  const uint8_t* vth = vt + (int64_t)bh * D * vt_ld;

  f16x8 qf[5];
  i32x8 q8[2];
  if constexpr (QK8) {
    const uint8_t* qrow = static_cast<const uint8_t*>(qv) + (img + qi) * ld + h * kQK8Pitch;
    q8[0] = q8[1] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (qi < T) {
      q8[0] = load32b(qrow + 32 * fg);
      q8[1] = load_tail8<D>(qrow, fg);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 5; ++s) {
      const int d0 = 16 * s + 8 * fg;
      if (qi < T && d0 < D)
        qf[s] = *reinterpret_cast<const f16x8*>(q + (img + qi) * ld + hc + d0);
      else
        qf[s] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  // constant V^T rows 80..95 of every stage: row 80 = e4m3(2^-exp), the rest 0
  {
    const uint32_t one = cvt_pk_e4m3(v_scale, v_scale, 0u, false) & 0xFFFF;
    const uint32_t one4 = one | (one << 16);
    constexpr int ZCH = (VROWS - VV8_ROWS_DMA) * VV8_PITCH / 16;
    for (int i = t; i < STAGES * ZCH; i += 256) {
      const int r = i % ZCH;
      uint8_t* z = smem + (i / ZCH) * STAGE + KBYTES + VV8_ROWS_DMA * VV8_PITCH + r * 16;
      *reinterpret_cast<i32x4*>(z) =
          r < VV8_PITCH / 16 ? i32x4{(int)one4, (int)one4, (int)one4, (int)one4} : i32x4{0, 0, 0, 0};
    }
  }
  __syncthreads();

  // transfer slots (slot j of this wave: global index jg = wave + 4 j); a
  // V^T transfer fills 16 rows of 64 bytes, lane i row i / 4, physical
  // chunk i % 4
  const uint8_t* ksrc[PER_WAVE];  // byte addresses (F16 or e4m3 K)
  const uint8_t* vsrc[PER_WAVE];
  int kkey[PER_WAVE], kdc[PER_WAVE];
  // byte offset of a key's row start and of a 16-byte chunk of it
  const int64_t krow = QK8 ? ld : 2 * ld;
  const int64_t kcol = QK8 ? (int64_t)h * kQK8Pitch : 2 * (int64_t)hc;
  constexpr int KCH_BYTES = 16;
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int jg = wave + 4 * j;
    kkey[j] = 0;
    kdc[j] = 0;
    ksrc[j] = kb8 + img * krow + kcol;
    vsrc[j] = vth;
    if (jg < NK) {
      const int off = jg * 1024 + 16 * lane;
      if constexpr (QK8) {
        kkey[j] = key_of_row8(off / kQK8Pitch);
        kdc[j] = (off % kQK8Pitch) / 16;
      } else {
        kkey[j] = key_of_row8(off / VK_PITCH);
        kdc[j] = min((off % VK_PITCH) / 16, NDC - 1);
      }
      ksrc[j] = kb8 + (img + kkey[j]) * krow + kcol + KCH_BYTES * kdc[j];
    } else if (jg < NDMA) {
      // LDS row vr takes logical chunk vswz8(vr, lane & 3) of V^T row vr;
      // rows D..79 take row D-1 instead, so nothing past the head is read
      const int vr = 16 * (jg - NK) + (lane >> 2);
      vsrc[j] = vth + (int64_t)min(vr, D - 1) * vt_ld + 16 * vswz8(vr, lane & 3);
    }
  }
  auto issue = [&](int kb) {
    const int key0 = kb * KB;
    uint8_t* st = smem + (kb % STAGES) * STAGE;
    const bool tail = key0 + KB > T;  // keys past T re-read token T-1
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int jg = wave + 4 * j;
      if (jg < NK) {
        const uint8_t* p = tail ? kb8 + (img + min(key0 + kkey[j], T - 1)) * krow + kcol + KCH_BYTES * kdc[j]
                                : ksrc[j] + (int64_t)key0 * krow;
        dma16(p, st + jg * 1024);
      } else if (jg < NDMA) {
        dma16(vsrc[j] + key0, st + KBYTES + (jg - NK) * 1024);
      } else {
        dma16(ksrc[0], trash);
      }
    }
  };

  const int koff = fr * VK_PITCH + fg * 16;
  // V^T fragment of rows 32 dt + fr, key bytes 32 fg .. +31: chunks 2 fg, 2 fg + 1
  int voff[3][2];
#pragma unroll
  for (int dt = 0; dt < 3; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int row = 32 * dt + fr;
      voff[dt][h2] = KBYTES + row * VV8_PITCH + 16 * vswz8(row, 2 * fg + h2);
    }

  float m_run = kNegInf;
  f32x16 oacc[3];
#pragma unroll
  for (int dt = 0; dt < 3; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;

  // a wave whose queries all lie past T only moves K/V^T for the others
  const bool active = qb * QWG + wave * 32 < T;
  const int nkb = (T + KB - 1) / KB;
  issue(0);
  for (int kb = 0; kb < nkb; ++kb) {
    attn_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (kb + 1 < nkb) issue(kb + 1);  // into the stage block kb-1 used
    if (!active) continue;
    const uint8_t* st = smem + (kb % STAGES) * STAGE;
    const int key0 = kb * KB;

    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.0f;
      if constexpr (QK8) {
        const uint8_t* kr = st + (kt * 32 + fr) * kQK8Pitch;
        sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(load32b(kr + 32 * fg), q8[0], sacc[kt], 0, 0, 0,
                                                                   127, 0, 127);
        if constexpr (D > 64)
          sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(load_tail8<D>(kr, fg), q8[1], sacc[kt], 0, 0, 0,
                                                                     127, 0, 127);
      } else {
#pragma unroll
        for (int s = 0; s < 5; ++s) {
          const f16x8 kf = *reinterpret_cast<const f16x8*>(st + koff + kt * 32 * VK_PITCH + s * 32);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[s], sacc[kt], 0, 0, 0);
        }
      }
    }
    if (key0 + KB > T) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + 32 * fg + 16 * kt + r >= T) sacc[kt][r] = kNegInf;
    }
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      a[i] = fmaxf(fmaxf(sacc[0][i], sacc[0][i + 8]), fmaxf(sacc[1][i], sacc[1][i + 8]));
    float mx = fmaxf(fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])), fmaxf(fmaxf(a[4], a[5]), fmaxf(a[6], a[7])));
    mx = half_swap_max(mx);
    if (__any((mx - m_run) * c > kTau)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
#pragma unroll
      for (int dt = 0; dt < 3; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_run = m_new;
    }
    // 2^4 p = exp2(s c - (m_run c - 4)): the code scale rides in the exponent
    const float mc = fmaf(m_run, c, -4.0f);
    // P^T fragment: byte 16 kt + r = e4m3(2^4 p) of key 32 fg + 16 kt + r
    i32x8 pf;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kt = w >> 2, r0 = 4 * (w & 3);
      float e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r0 + u], c, -mc));
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], word, true);
      pf[w] = word;
    }
#pragma unroll
    for (int dt = 0; dt < 3; ++dt) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(st + voff[dt][0]);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(st + voff[dt][1]);
      const i32x8 vf = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      oacc[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vf, pf, oacc[dt], 0, 0, 0, 127, 0, 127);
    }
  }

  // the row sum sits in O^T row 80, register RL of lane group 0
  const float lsum0 = oacc[2][RL];
  const float lsum1 = half_other(lsum0);
  if (qi >= T) return;
  const float inv = 1.0f / (fg ? lsum1 : lsum0);
#pragma unroll
  for (int dt = 0; dt < 3; ++dt)
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int d0 = 32 * dt + 8 * qd + 4 * fg;
      if (d0 >= D) continue;
      const float a0 = oacc[dt][4 * qd + 0] * inv, a1 = oacc[dt][4 * qd + 1] * inv;
      const float a2 = oacc[dt][4 * qd + 2] * inv, a3 = oacc[dt][4 * qd + 3] * inv;
      if constexpr (OUT_FP8) {
        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(o) + (img + qi) * ldo + hc + d0) =
            pack4_e4m3(a0 * out_scale, a1 * out_scale, a2 * out_scale, a3 * out_scale);
      } else {
        const f16x4 ov = {(f16)a0, (f16)a1, (f16)a2, (f16)a3};
        *reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(o) + (img + qi) * ldo + hc + d0) = ov;
      }
    }
}

// ---------------------------------------------------------------------------
// The same attention for one-round grids (small batches): 16 queries per
// wave with v_mfma_f32_16x16x32_f16, four waves (64 queries) per
// workgroup, so a batch-1 grid of 729 tokens x 16 heads is 192 workgroups of
// one wave per SIMD. Per query it does the same products, exponentials and
// rescales in the same order as flash_attn_vt_kernel, so its outputs are
// bit-identical (tested); each wave's chain of dependent steps per key block
// is half as long, which is what a grid of one round waits on, while a full
// grid runs faster on the 32-query kernel, whose waves read each K/V^T
// fragment once for twice the queries.
//
// K rows are stored permuted within each 32-key half: LDS row
// 32h + 16t + 4g + i holds key 32h + 8g + 4t + i, so lane group g of score
// tiles 2h and 2h + 1 (16x16 result: lane group g holds tile rows 4g..4g+3)
// holds keys 32h + 8g .. 32h + 8g + 7, exactly the P^T operand of PV k-step
// h. A K row has D/8 (made odd) 16-byte chunks: conflict-free fragment reads
// of 16 consecutive rows; dims past D read the last real chunk, against zero
// Q padding. V^T rows D (ones: the probability sum) .. 16 NT - 1 (zeros) are
// written once. VROW: vt is V row-major (rows of stride ld, head h at column
// h * D, as q and k), read through the transposing LDS reads; vt_ld is not
// used.
//
// NS > 1 (key split, as in split-KV decoding): the workgroup holds NS groups
// of the four query waves, group s taking key blocks [s nkb / NS, (s + 1)
// nkb / NS) through a K/V ring of its own, so a grid of one round runs NS
// waves per SIMD instead of one. Groups 1 .. NS-1 then leave their O^T
// partial sums (with the probability-sum row) and references in LDS, and
// group 0 rescales each to the largest reference and adds them in group
// order: the same bits for every batch, not those of NS = 1.
template <int D, bool OUT_FP8, bool VROW = false, int NS = 1>
__global__ __launch_bounds__(256 * NS, NS == 1 ? 2 : 1) void flash_attn_vt16_kernel(
    const f16* __restrict__ q, const f16* __restrict__ k, int64_t ld, const f16* __restrict__ vt,
    int64_t vt_ld, void* __restrict__ o, int64_t ldo, int T, int H, int nqb, float c, float out_scale) {
  static_assert(D % 8 == 0 && D >= 64 && D <= 80, "head width");
  constexpr int NW = 4;
  constexpr int QWG = NW * 16;
  constexpr int NDC = D / 8;                       // 16-byte dim chunks of a key
  constexpr int KP = 16 * (NDC | 1);               // K LDS row pitch (odd chunk count)
  constexpr int KBYTES = KB * KP;
  static_assert(KBYTES % 1024 == 0, "whole K transfers");
  constexpr int NKS = (D + 31) / 32;               // QK k-steps of 32 dims
  constexpr int NT = (D + 1 + 15) / 16;            // PV dim tiles: D dims and the ones row
  constexpr int VR = 16 * NT;                      // V^T LDS rows
  static_assert(!VROW || VR <= kVRowPitch / 2, "row-major V rows hold the PV dim tiles");
  constexpr int STAGE = KBYTES + (VROW ? VR_BYTES : VR * VV_PITCH);
  constexpr int NK = KBYTES / 1024;                // 1 KiB transfers for K per stage
  constexpr int NDMA = NK + (VROW ? VR_BYTES / 1024 : D / 8);  // and for V (V^T: 8 rows of 128 bytes each)
  constexpr int PER_WAVE = (NDMA + NW - 1) / NW;
  constexpr float kTau = 8.0f;                     // rescale only when a row max grows by > 2^8
  constexpr int STAGES = 2;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGES * STAGE + 1024];
  uint8_t* trash = smem + NS * STAGES * STAGE;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane((t >> 6) % NW);  // query wave
  const int sp = __builtin_amdgcn_readfirstlane((t >> 6) / NW);    // key split: its own ring
  uint8_t* const ring = smem + sp * STAGES * STAGE;
  const int fq = lane & 15;  // query of the wave (MFMA column)
  const int g = lane >> 4;   // lane group
  const int L = xcd_block(blockIdx.x, gridDim.x);
  const int qb = L % nqb;
  const int bh = L / nqb;
  const int h = bh % H;
  const int b = bh / H;
  const int hc = h * D;
  const int64_t img = (int64_t)b * T;
  const int qi = qb * QWG + wave * 16 + fq;
  const f16* vth = vt + (int64_t)bh * D * vt_ld;

  // Q^T operand of k-step ks: dims 32 ks + 8 g .. + 7 of query qi (zero past D or T)
  f16x8 qf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int d0 = 32 * ks + 8 * g;
    if (qi < T && d0 < D)
      qf[ks] = *reinterpret_cast<const f16x8*>(q + (img + qi) * ld + hc + d0);
    else
      qf[ks] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  __builtin_amdgcn_s_waitcnt(0);  // as in flash_attn_vt_kernel: Q complete before the block loop
  if constexpr (VROW) vrow_pad<NDC>(smem, NS * STAGES, STAGE, KBYTES, t, NS * NW * 64);
  constexpr int ZCH = VROW ? 0 : (VR - D) * VV_PITCH / 16;
  for (int i = t; i < NS * STAGES * ZCH; i += NS * NW * 64) {
    const int r = i % ZCH;
    uint8_t* z = smem + (i / ZCH) * STAGE + KBYTES + D * VV_PITCH + r * 16;
    const int one = 0x3C003C00;  // two F16 ones
    *reinterpret_cast<i32x4*>(z) = r < VV_PITCH / 16 ? i32x4{one, one, one, one} : i32x4{0, 0, 0, 0};
  }
  __syncthreads();

  // transfer slots (global index jg = wave + 8 j): K LDS bytes jg KiB .. (row off / KP, chunk),
  // V^T rows 8 (jg - NK) .., padding transfers into the trash KiB
  const f16* src[PER_WAVE];
  int kkey[PER_WAVE], kdc[PER_WAVE];
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int jg = wave + NW * j;
    const int off = jg * 1024 + 16 * lane;
    const int r = off / KP;
    const int x = r & 31;
    kkey[j] = (r & ~31) + 8 * ((x >> 2) & 3) + 4 * (x >> 4) + (x & 3);
    kdc[j] = min((off % KP) / 16, NDC - 1);
    if (VROW && jg >= NK && jg < NDMA) {  // V row kkey, chunk kdc (>= NDC: padding, not transferred)
      const int vo = off - NK * 1024;
      kkey[j] = vo / kVRowPitch;
      kdc[j] = (vo % kVRowPitch) / 16;
      src[j] = vt + (img + kkey[j]) * ld + hc + 8 * min(kdc[j], NDC - 1);
    } else if (jg < NK) {
      src[j] = k + (img + kkey[j]) * ld + hc + 8 * kdc[j];
    } else if (jg < NDMA) {
      const int d = 8 * (jg - NK) + (lane >> 3);
      src[j] = vth + (int64_t)d * vt_ld + 8 * ((lane & 7) ^ vswz_key(d));
    } else {
      src[j] = vth;
    }
  }
  // per slot: bytes its source advances per key (uniform) and whether this
  // lane transfers (row-major V lanes that would land on padding do not)
  int64_t kstep[PER_WAVE];
  bool lon[PER_WAVE];
#pragma unroll
  for (int j = 0; j < PER_WAVE; ++j) {
    const int jg = wave + NW * j;
    kstep[j] = jg < NK ? 2 * ld : jg < NDMA ? (VROW ? 2 * ld : 2) : 0;
    lon[j] = !(VROW && jg >= NK && jg < NDMA && kdc[j] >= NDC);
  }
  auto issue = [&](int kb) {
    const int key0 = kb * KB;
    uint8_t* st = ring + (kb % STAGES) * STAGE;
    const bool tail = key0 + KB > T;  // keys past T re-read token T-1
    if (!tail) {
      // every slot lands at its KiB of the stage (the V part starts at NK
      // KiB), padding slots in the trash KiB: no per-slot branches
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int jg = wave + NW * j;
        if (lon[j])
          dma16(reinterpret_cast<const uint8_t*>(src[j]) + key0 * kstep[j], jg < NDMA ? st + jg * 1024 : trash);
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int jg = wave + NW * j;
      if (jg < NK) {
        const f16* p = tail ? k + (img + min(key0 + kkey[j], T - 1)) * ld + hc + 8 * kdc[j]
                            : src[j] + (int64_t)key0 * ld;
        dma16(p, st + jg * 1024);
      } else if (jg < NDMA) {
        if constexpr (VROW) {
          const f16* p = tail ? vt + (img + min(key0 + kkey[j], T - 1)) * ld + hc + 8 * kdc[j]
                              : src[j] + (int64_t)key0 * ld;
          if (kdc[j] < NDC) dma16(p, st + jg * 1024);
        } else {
          dma16(src[j] + key0, st + KBYTES + (jg - NK) * 1024);
        }
      } else {
        dma16(src[j], trash);
      }
    }
  };
  // VROW: lane a + 4r of lane group g reads dims 4a .. 4a + 3 of key 8g + r
  // (+ 32 hh + 4 t for PV k-step hh, half t; + 16 dt dims): lane 4a + b then
  // holds dim fq of keys 32 hh + 8 g + 4 t + 0..3
  const int vrb = KBYTES + (8 * g + ((lane & 15) >> 2)) * kVRowPitch + 8 * (lane & 3);

  int koff[NKS];  // K fragment: row fq of a tile, chunk 4 ks + g (the last real chunk past D)
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = fq * KP + min(4 * ks + g, NDC - 1) * 16;

  float m_run = kNegInf;
  f32x4 oacc[NT];  // O^T rows 16 dt + 4 g + (0..3), column fq
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One 64-key block; NKT: 32-key halves that hold a key below T (a last
  // block's all-padding second half would add exact zeros: left out, the
  // same bits)
  auto block = [&](const uint8_t* st, int key0, auto nkt_tag, auto tail_tag) {
    constexpr int NKT = decltype(nkt_tag)::value;
    constexpr bool TAIL = decltype(tail_tag)::value;  // the last block: keys past T masked
    f32x4 sacc[2 * NKT];  // S^T tile tt: LDS rows 16 tt + 4 g + i, query fq
#pragma unroll
    for (int tt = 0; tt < 2 * NKT; ++tt) {
      sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const f16x8 kf = *reinterpret_cast<const f16x8*>(st + tt * 16 * KP + koff[ks]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ks], sacc[tt], 0, 0, 0);
      }
    }
    if (TAIL && key0 + KB > T) {
#pragma unroll
      for (int tt = 0; tt < 2 * NKT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + 32 * (tt >> 1) + 8 * g + 4 * (tt & 1) + i >= T) sacc[tt][i] = kNegInf;
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    if constexpr (NKT == 2)
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(sacc[NKT][0], sacc[NKT][1]), fmaxf(sacc[NKT][2], sacc[NKT][3])),
                           fmaxf(fmaxf(sacc[2 * NKT - 1][0], sacc[2 * NKT - 1][1]),
                                 fmaxf(sacc[2 * NKT - 1][2], sacc[2 * NKT - 1][3]))));
    {  // over the four lane groups of query fq: lane rows 0/1 and 2/3, then the halves
      unsigned a = __builtin_bit_cast(unsigned, mx), bb = a;
      asm volatile("" : "+v"(bb));  // two distinct operands (see half_swap)
      const auto sw = __builtin_amdgcn_permlane16_swap(a, bb, false, false);
      const unsigned e0 = sw[0], e1 = sw[1];
      mx = half_swap_max(fmaxf(__builtin_bit_cast(float, e0), __builtin_bit_cast(float, e1)));
    }
    // lazy running reference, as in flash_attn_vt_kernel
    if (__any((mx - m_run) * c > kTau)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) oacc[dt] *= alpha;
      m_run = m_new;
    }
    const float mc = m_run * c;
#pragma unroll
    for (int hh = 0; hh < NKT; ++hh) {  // PV k-step: keys 32 hh + 8 g .. + 7 of this lane group
      f16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const int tt = 2 * hh + (e >> 2), i = e & 3;
        const f32x2 pp = {__builtin_amdgcn_exp2f(fmaf(sacc[tt][i], c, -mc)),
                          __builtin_amdgcn_exp2f(fmaf(sacc[tt][i + 1], c, -mc))};
        const f16x2 ph = __builtin_convertvector(pp, f16x2);
        pf[e] = ph[0];
        pf[e + 1] = ph[1];
      }
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        f16x8 vf;
        if constexpr (VROW) {
          const uint8_t* pv = st + vrb + 32 * hh * kVRowPitch + 32 * dt;
          vf = cat8(ds_read_tr4(pv), ds_read_tr4(pv + 4 * kVRowPitch));
        } else {
          const int vr = 16 * dt + fq;
          vf = *reinterpret_cast<const f16x8*>(st + KBYTES + vr * VV_PITCH + 16 * ((4 * hh + g) ^ vswz_key(vr)));
        }
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf, oacc[dt], 0, 0, 0);
      }
    }
  };

  // a wave whose queries all lie past T only moves K/V for the others; the
  // last block (keys past T masked, possibly only its first half) runs
  // after the loop, so the loop holds one form of the block
  const bool active = qb * QWG + wave * 16 < T;
  const int nkb = (T + KB - 1) / KB;
  // key split sp: blocks kb0 .. kb0 + ns - 1; the last split has the most
  // (nmax) and the masked last block. Every split steps through nmax rounds
  // so that all waves meet the same barriers.
  const int kb0 = sp * nkb / NS, ns = (sp + 1) * nkb / NS - kb0, nmax = (nkb + NS - 1) / NS;
  using full = std::integral_constant<int, 2>;
  using half = std::integral_constant<int, 1>;
  using yes = std::true_type;
  using no = std::false_type;
  // every issue() is PER_WAVE transfer instructions of this wave (each slot
  // has real lanes), so at most (STAGES - 2) blocks' worth may stay in flight
#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p)
    if (p < ns) issue(kb0 + p);
  for (int i = 0; i < nmax - 1; ++i) {
    const int kb = kb0 + i;
    if (i + STAGES - 2 < ns)
      attn_wait_vmcnt<(STAGES - 2) * PER_WAVE>();
    else
      attn_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();  // block kb in LDS; block kb-1's stage free
    if (i + STAGES - 1 < ns) issue(kb + STAGES - 1);
    if (active && i < ns) block(ring + (kb % STAGES) * STAGE, kb * KB, full(), no());
  }
  {
    // round nmax - 1: the last block of the splits that have nmax blocks
    // (masking is a no-op but for the last split's)
    const int kb = kb0 + nmax - 1, key0 = kb * KB;
    attn_wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const uint8_t* st = ring + (kb % STAGES) * STAGE;
    if (active && nmax == ns) {
      if (key0 + 32 >= T)
        block(st, key0, half(), yes());
      else
        block(st, key0, full(), yes());
    }
  }
  if constexpr (NS > 1) {
    // splits 1 .. NS-1 leave their O^T partial sums (the probability-sum row
    // included) and references in LDS; split 0 rescales every split to the
    // largest reference and adds them in split order
    constexpr int PB = NT * 1024 + 256;  // bytes per (split, query wave)
    static_assert((NS - 1) * NW * PB <= NS * STAGES * STAGE, "partials fit in the rings");
    __syncthreads();  // every wave is done with the rings
    if (sp > 0 && active) {
      uint8_t* pp = smem + ((sp - 1) * NW + wave) * PB;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) *reinterpret_cast<f32x4*>(pp + dt * 1024 + 16 * lane) = oacc[dt];
      *reinterpret_cast<float*>(pp + NT * 1024 + 4 * lane) = m_run;
    }
    __syncthreads();
    if (sp > 0 || !active) return;
    float mref = m_run;  // query fq's largest reference over the splits
#pragma unroll
    for (int s2 = 1; s2 < NS; ++s2)
      mref = fmaxf(mref, *reinterpret_cast<const float*>(smem + ((s2 - 1) * NW + wave) * PB + NT * 1024 + 4 * lane));
    const float a0 = __builtin_amdgcn_exp2f((m_run - mref) * c);
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) oacc[dt] *= a0;
#pragma unroll
    for (int s2 = 1; s2 < NS; ++s2) {
      const uint8_t* pp = smem + ((s2 - 1) * NW + wave) * PB;
      const float a = __builtin_amdgcn_exp2f((*reinterpret_cast<const float*>(pp + NT * 1024 + 4 * lane) - mref) * c);
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(pp + dt * 1024 + 16 * lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[dt][r] = fmaf(a, v[r], oacc[dt][r]);
      }
    }
  }
  // the probability sum sits in O^T row D: tile D / 16, lane group (D % 16) / 4, register D % 4
  const float lsum = __shfl(oacc[D / 16][D % 4], ((D % 16) / 4) * 16 + fq, 64);
  if (qi >= T) return;
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) {
    const int d0 = 16 * dt + 4 * g;
    if (d0 >= D) continue;
    const float a0 = oacc[dt][0] * inv, a1 = oacc[dt][1] * inv, a2 = oacc[dt][2] * inv, a3 = oacc[dt][3] * inv;
    if constexpr (OUT_FP8) {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(o) + (img + qi) * ldo + hc + d0) =
          pack4_e4m3(a0 * out_scale, a1 * out_scale, a2 * out_scale, a3 * out_scale);
    } else {
      const f16x4 ov = {(f16)a0, (f16)a1, (f16)a2, (f16)a3};
      *reinterpret_cast<f16x4*>(reinterpret_cast<f16*>(o) + (img + qi) * ldo + hc + d0) = ov;
    }
  }
}

template <int D, bool QK8, bool VROW = false>
hipError_t launch_vt_d(const void* q, const void* k, int64_t ld, const f16* vt, int64_t vt_ld, void* o, int64_t ldo,
                       int batch, int heads, int tokens, float sl2, bool out_fp8, float out_scale, hipStream_t s) {
  const int nqb = (tokens + QB - 1) / QB;
  const int64_t blocks = (int64_t)nqb * heads * batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  // One round of workgroups (batch 1 and 2 at 729 tokens x 16 heads): the
  // 16-query kernel, the same bits (729 tokens, 16 heads, head dim 72, batch
  // 1 / 2: 20.2 -> 19.3 us, 21.5 -> 20.4 us with eight waves per workgroup;
  // four waves, one per SIMD, 18.9 -> 16.4 us at batch 1; deeper K/V rings
  // did not help; from batch 3 on the 32-query kernel is as fast or faster).
  // With row-major V, three key splits per workgroup: 16.5 -> 14.0 us at
  // batch 1 (splits over workgroups, combined by the last to arrive, took
  // 81 us: each agent-scope release and acquire writes back and invalidates
  // an XCD's L2)
  if constexpr (!QK8) {
    if (blocks <= 256) {
      const int nq16 = (tokens + 63) / 64;
      const unsigned nb = (unsigned)(nq16 * heads * batch);
      const f16* q16 = static_cast<const f16*>(q);
      const f16* k16 = static_cast<const f16*>(k);
      if constexpr (VROW) {
        // row-major V (the encoder's one-round calls): three key splits per
        // workgroup when one image's grid is at most one workgroup per CU,
        // whatever the batch, so every batch adds the same partials
        if (nq16 * heads <= 256) {
          if (out_fp8)
            hipLaunchKernelGGL((flash_attn_vt16_kernel<D, true, true, 3>), dim3(nb), dim3(768), 0, s, q16, k16, ld,
                               vt, vt_ld, o, ldo, tokens, heads, nq16, sl2, out_scale);
          else
            hipLaunchKernelGGL((flash_attn_vt16_kernel<D, false, true, 3>), dim3(nb), dim3(768), 0, s, q16, k16, ld,
                               vt, vt_ld, o, ldo, tokens, heads, nq16, sl2, out_scale);
          return hipGetLastError();
        }
      }
      if (out_fp8)
        hipLaunchKernelGGL((flash_attn_vt16_kernel<D, true, VROW>), dim3(nb), dim3(256), 0, s, q16, k16, ld, vt, vt_ld,
                           o, ldo, tokens, heads, nq16, sl2, out_scale);
      else
        hipLaunchKernelGGL((flash_attn_vt16_kernel<D, false, VROW>), dim3(nb), dim3(256), 0, s, q16, k16, ld, vt, vt_ld,
                           o, ldo, tokens, heads, nq16, sl2, out_scale);
      return hipGetLastError();
    }
  }
  if constexpr (VROW) {
    return hipErrorInvalidValue;  // row-major V: one-round grids only (the 16-query kernel)
  } else {
    if (out_fp8)
      hipLaunchKernelGGL((flash_attn_vt_kernel<D, true, VT_STAGES_DEFAULT, 3, 1, QK8>), dim3((unsigned)blocks),
                         dim3(256), 0, s, q, k, ld, vt, vt_ld, o, ldo, tokens, heads, nqb, sl2, out_scale);
    else
      hipLaunchKernelGGL((flash_attn_vt_kernel<D, false, VT_STAGES_DEFAULT, 3, 1, QK8>), dim3((unsigned)blocks),
                         dim3(256), 0, s, q, k, ld, vt, vt_ld, o, ldo, tokens, heads, nqb, sl2, out_scale);
    return hipGetLastError();
  }
}

}  // namespace

hipError_t launch_flash_attention(const f16* q, const f16* k, const f16* v, int64_t ld, void* o,
                                  int64_t ldo, int batch, int heads, int tokens, int head_dim,
                                  float scale, bool out_fp8, float out_scale, hipStream_t s) {
  if (batch < 1 || heads < 1 || tokens < 1 || head_dim < 8 || head_dim > 80 || (head_dim & 7) ||
      ld < (int64_t)heads * head_dim || (ld & 7) || ldo < (int64_t)heads * head_dim || (ldo & 3))
    return hipErrorInvalidValue;
  if (batch > 65535 || heads > 65535) return hipErrorInvalidValue;
  const float sl2 = scale * 1.4426950408889634f;
  const int nqb = (tokens + QB - 1) / QB;
  const int64_t blocks = (int64_t)nqb * heads * batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks);
  if (out_fp8)
    hipLaunchKernelGGL(flash_attn_kernel<true>, grid, dim3(256), 0, s, q, k, v, ld, o, ldo, tokens, head_dim, heads,
                       nqb, sl2, out_scale);
  else
    hipLaunchKernelGGL(flash_attn_kernel<false>, grid, dim3(256), 0, s, q, k, v, ld, o, ldo, tokens, head_dim, heads,
                       nqb, sl2, out_scale);
  return hipGetLastError();
}

bool flash_attention_vt_supported(int head_dim) { return head_dim == 64 || head_dim == 72 || head_dim == 80; }

namespace {
// Q/K operand checks shared by the V^T launchers: F16 rows of ld elements, or
// e4m3 code rows of ld bytes with head slots of kQK8Pitch bytes (16-byte
// aligned rows and slots, every slot of a row inside ld).
bool qk_args_ok(const void* q, const void* k, int64_t ld, int heads, int head_dim, int qk8_pitch) {
  if (qk8_pitch == 0) return ld >= (int64_t)heads * head_dim && (ld & 7) == 0;
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  return qk8_pitch == kQK8Pitch && head_dim <= kQK8Pitch && ld >= (int64_t)heads * kQK8Pitch && (ld & 15) == 0 &&
         a16(q) && a16(k);
}
}  // namespace

hipError_t launch_flash_attention_vt(const void* q, const void* k, int64_t ld, int qk8_pitch, const f16* vt,
                                     int64_t vt_ld, void* o, int64_t ldo, int batch, int heads, int tokens,
                                     int head_dim, float scale, bool out_fp8, float out_scale, hipStream_t s) {
  if (batch < 1 || heads < 1 || tokens < 1 || !flash_attention_vt_supported(head_dim) ||
      !qk_args_ok(q, k, ld, heads, head_dim, qk8_pitch) || ldo < (int64_t)heads * head_dim || (ldo & 3) ||
      vt_ld < (int64_t)(tokens + KB - 1) / KB * KB || (vt_ld & 7))
    return hipErrorInvalidValue;
  // e4m3 Q and K codes carry 2^4 each: their products are 2^8 times the scores
  const float sl2 = scale * 1.4426950408889634f * (qk8_pitch ? 1.0f / 256.0f : 1.0f);
  switch (head_dim * 2 + (qk8_pitch ? 1 : 0)) {
    case 128: return launch_vt_d<64, false>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
    case 144: return launch_vt_d<72, false>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
    case 160: return launch_vt_d<80, false>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
    case 129: return launch_vt_d<64, true>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
    case 145: return launch_vt_d<72, true>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
    case 161: return launch_vt_d<80, true>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_flash_attention_vrow(const f16* q, const f16* k, const f16* v, int64_t ld, void* o, int64_t ldo,
                                       int batch, int heads, int tokens, int head_dim, float scale, bool out_fp8,
                                       float out_scale, hipStream_t s) {
  if (batch < 1 || heads < 1 || tokens < 1 || !flash_attention_vt_supported(head_dim) ||
      !qk_args_ok(q, k, ld, heads, head_dim, 0) || (reinterpret_cast<uintptr_t>(v) & 15) ||
      ldo < (int64_t)heads * head_dim || (ldo & 3))
    return hipErrorInvalidValue;
  const float sl2 = scale * 1.4426950408889634f;
  switch (head_dim) {
    case 64: return launch_vt_d<64, false, true>(q, k, ld, v, 0, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
    case 72: return launch_vt_d<72, false, true>(q, k, ld, v, 0, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
    case 80: return launch_vt_d<80, false, true>(q, k, ld, v, 0, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, s);
  }
  return hipErrorInvalidValue;
}

namespace {
template <int D, bool QK8>
hipError_t launch_vt8_d(const void* q, const void* k, int64_t ld, const uint8_t* vt, int64_t vt_ld, void* o,
                        int64_t ldo, int batch, int heads, int tokens, float sl2, bool out_fp8, float out_scale,
                        float v_scale, hipStream_t s) {
  const int nqb = (tokens + QB - 1) / QB;
  const int64_t blocks = (int64_t)nqb * heads * batch;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (out_fp8)
    hipLaunchKernelGGL((flash_attn_vt8_kernel<D, true, QK8>), dim3((unsigned)blocks), dim3(256), 0, s, q, k, ld, vt,
                       vt_ld, o, ldo, tokens, heads, nqb, sl2, out_scale, v_scale);
  else
    hipLaunchKernelGGL((flash_attn_vt8_kernel<D, false, QK8>), dim3((unsigned)blocks), dim3(256), 0, s, q, k, ld, vt,
                       vt_ld, o, ldo, tokens, heads, nqb, sl2, out_scale, v_scale);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_flash_attention_vt8(const void* q, const void* k, int64_t ld, int qk8_pitch, const uint8_t* vt,
                                      int64_t vt_ld, void* o, int64_t ldo, int batch, int heads, int tokens,
                                      int head_dim, float scale, bool out_fp8, float out_scale, float v_scale,
                                      hipStream_t s) {
  if (batch < 1 || heads < 1 || tokens < 1 || !flash_attention_vt_supported(head_dim) ||
      !qk_args_ok(q, k, ld, heads, head_dim, qk8_pitch) || ldo < (int64_t)heads * head_dim || (ldo & 3) ||
      vt_ld < (int64_t)(tokens + KB - 1) / KB * KB || (vt_ld & 15) ||
      (reinterpret_cast<uintptr_t>(vt) & 15) || !(v_scale > 0.0f) || v_scale > 256.0f)
    return hipErrorInvalidValue;
  const float sl2 = scale * 1.4426950408889634f * (qk8_pitch ? 1.0f / 256.0f : 1.0f);
  switch (head_dim * 2 + (qk8_pitch ? 1 : 0)) {
    case 128: return launch_vt8_d<64, false>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, v_scale, s);
    case 144: return launch_vt8_d<72, false>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, v_scale, s);
    case 160: return launch_vt8_d<80, false>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, v_scale, s);
    case 129: return launch_vt8_d<64, true>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, v_scale, s);
    case 145: return launch_vt8_d<72, true>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, v_scale, s);
    case 161: return launch_vt8_d<80, true>(q, k, ld, vt, vt_ld, o, ldo, batch, heads, tokens, sl2, out_fp8, out_scale, v_scale, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace siglip
