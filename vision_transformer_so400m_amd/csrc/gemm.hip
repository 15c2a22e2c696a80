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
// Operands: A [M, K] activations, K-contiguous rows, and Wt [N, K] weights,
// K-contiguous in 64-byte K panels (consecutive rows of one 64-byte piece of
// K are contiguous, so every K slice of a weight tile is one run of memory
// per panel: 64-byte slices cost half-line row fetches otherwise); both
// F16 (v_mfma_f32_32x32x16_f16) or both OCP e4m3 codes
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales; the power-of-two
// operand scale is folded into acc_scale). F32 accumulation.
//
// LayerNorm-folded A operand (an option): A is the F16 residual stream and
// each row is normalized with its precomputed statistics on its way into LDS
// (page "FP8 attention and resident image/embedding transfers", "Full
// 27-layer ViT": producers and consumers handle the quantized operand
// themselves instead of separate passes), the per-element arithmetic of the
// LayerNorm kernel, so the products are those of LayerNorm + GEMM.
//
// Tiling: a workgroup of 4 to 12 waves owns a BM x BN output tile and walks K in
// 128-byte slices (64 F16 or 128 e4m3 values per row; 64-byte slices for the
// MLP-up tile, 256-byte slices for one-round small grids with a long K).
// Slices go global -> LDS directly (global_load_lds_dwordx4) into a ring of
// STAGES buffers, so the loads of the next slices are in flight while one is
// multiplied. The 16-byte chunk index of each LDS row is XOR-swizzled (swz
// below), so the 16 lanes that read one chunk of 16 consecutive rows hit
// distinct banks.
//
// The MFMA is issued with the weight fragment as its first operand, so the
// hardware's 32x32 result holds, per lane, one activation row m and four
// consecutive output columns n per register quad. The epilogue stages these
// values through the idle LDS ring and writes whole 16-byte chunks of output
// rows (the V^T columns of the QKV projection are stored transposed straight
// from registers).
#include "common.h"

#include <type_traits>



namespace siglip {
namespace {

constexpr int kRowBytes = 128;  // K bytes of one LDS tile row (the default K slice)

// RB: K bytes of one LDS tile row (one K slice): 128, or 64 for tiles that
// need a deeper ring in less LDS.
template <int BM, int BN, int WM, int WN, int RB = kRowBytes>
struct Tile {
  static constexpr int WAVES_N = BN / WN;
  static constexpr int WAVES_M = BM / WM;
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static_assert(WAVES == 4 || WAVES == 8 || WAVES == 12, "four, eight or twelve waves per workgroup");
  static_assert(RB == 64 || RB == 128 || RB == 256, "64-, 128- or 256-byte K slices");
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int TM = WM / 32;
  static constexpr int TN = WN / 32;
  static constexpr int RPW = 1024 / RB;             // tile rows one wave's 1 KiB transfer fills
  static constexpr int ROWS_PER_ROUND = RPW * WAVES;  // tile rows one DMA round fills
  static_assert(BM % ROWS_PER_ROUND == 0 && BN % ROWS_PER_ROUND == 0, "whole DMA rounds");
  static_assert(ROWS_PER_ROUND % 16 == 0, "a round's rows share their swizzle keys");
  static constexpr int STAGE = (BM + BN) * RB;
};

// 16-byte chunk swizzle of an LDS row. A fragment read has 16 lanes reading
// one logical chunk of 16 consecutive rows; 64 banks of 4 bytes span 256
// bytes. 128-byte rows: two rows span all banks, so (row & 1) picks the half
// and the chunk must differ across the 8 rows of each parity: chunk ^ (row &
// 7) ^ ((row >> 3) & 1). 64-byte rows: four rows span all banks, so the chunk
// must differ across rows r, r+4, r+8, r+12: chunk ^ ((row >> 2) & 3).
// 256-byte rows: one row spans all banks, so the chunk must differ across the
// 16 rows: chunk ^ (row & 15). All are bijections on the chunks of any row.
template <int RB = kRowBytes>
__device__ __forceinline__ int swz_key(int row) {
  if constexpr (RB == 256) return row & 15;
  else if constexpr (RB == 128) return (row & 7) ^ ((row >> 3) & 1);
  else return (row >> 2) & 3;
}
template <int RB = kRowBytes>
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ swz_key<RB>(row); }

// Element type of the output tile staged in LDS: F32 while a residual is
// still to be added (one rounding), else the output type (for EPI_QKV the Q
// and K columns are F16 either way; OUT_FP8 there makes V^T e4m3).
template <int EPI, bool OUT_FP8>
struct StageType {
  typedef typename std::conditional<
      EPI == EPI_BIAS_RES, float,
      typename std::conditional<(OUT_FP8 && EPI != EPI_QKV) || EPI == EPI_QKV8, uint8_t, f16>::type>::type type;
};

// Linear workgroup id -> output tile. Workgroups are dispatched round-robin
// over the 8 XCDs (id % 8), each with its own 4 MB L2. The remap gives every
// XCD a contiguous range L of tile numbers. Within it, tiles run in bands of
// gm row blocks: a band is walked column by column (row block fastest), so
// the workgroups resident on one XCD at a time share a few row blocks of A
// and a few column blocks of Wt, and both stay in L2 instead of the whole
// weight matrix streaming past once per row block. gm <= 0 numbers tiles
// N-fastest over the whole range.
__device__ __forceinline__ void tile_of(int id, int ntm, int ntn, int gm, int* tm, int* tn) {
  const int total = ntm * ntn;
  const int total8 = total & ~7;
  const int L = id < total8 ? (id & 7) * (total8 >> 3) + (id >> 3) : id;
  if (gm <= 0) {
    *tm = L / ntn;
    *tn = L - *tm * ntn;
    return;
  }
  const int band = L / (gm * ntn);
  const int r = L - band * gm * ntn;
  const int first = band * gm;
  const int rows = min(gm, ntm - first);  // the last band may be shorter; r < rows * ntn
  *tn = r / rows;
  *tm = first + (r - *tn * rows);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One 16-byte global -> LDS transfer per lane (global_load_lds_dwordx4): the
// wave writes 64 x 16 bytes contiguously from lds_wave_base, lane i at +16 i.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gsrc,
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// MINW: waves per SIMD the register allocation must allow (the second
// __launch_bounds__ argument): 2 for the four-wave tiles that rely on two
// workgroups sharing a CU, 4 for eight-wave ones.
// LNA: the A operand is LayerNorm-folded (GemmArgs::ln_stats): A rows are
// the F16 residual, normalized in registers and written to LDS as operand
// values; only the weight rows stream by DMA.
template <int BM, int BN, int WM, int WN, int STAGES, bool FP8, int EPI, bool OUT_FP8, int RB = kRowBytes,
          int MINW = 1, bool LNA = false>
__global__ __launch_bounds__(64 * (BM / WM) * (BN / WN), MINW) void gemm_kernel(GemmArgs g) {
  using T = Tile<BM, BN, WM, WN, RB>;
  static_assert(STAGES >= 2, "at least double buffering");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * T::STAGE];

  constexpr int E = FP8 ? 1 : 2;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / T::WAVES_N;
  const int wn = wave % T::WAVES_N;
  const int ntn = g.N / BN;
  const int ntm = (g.M + BM - 1) / BM;
  int tm, tn;
  tile_of(blockIdx.x, ntm, ntn, g.group_m, &tm, &tn);
  const int m0 = tm * BM;
  const int n0 = tn * BN;
  const int nk = (g.K * E) / RB;

  // ---- global -> LDS transfer assignment. A stage holds BM rows of A then
  // BN rows of Wt, RB bytes each, chunk-swizzled. Transfer j of wave w fills
  // tile rows R j + RPW w .. +RPW-1 (R = RPW x waves); lane i lands at row
  // R j + RPW w + i / CPR, physical chunk i % CPR (CPR = RB / 16 chunks per
  // row), so it fetches logical chunk swz(row, i % CPR). R j is a multiple of
  // 16, so the swizzle key depends on RPW w + i / CPR only.
  constexpr int R = T::ROWS_PER_ROUND;
  constexpr int CPR = RB / 16;
  constexpr int CH = (BM + BN) / R;  // transfers per thread per stage
  const int rr = lane / CPR;
  const int lchunk = swz<RB>(T::RPW * wave + rr, lane % CPR);
  const uint8_t* src[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int row = R * j + T::RPW * wave + rr;
    if (R * j < BM) {
      const int am = min(m0 + row, g.M - 1);  // rows past M re-read row M-1; never stored
      src[j] = LNA ? nullptr : reinterpret_cast<const uint8_t*>(g.a) + (int64_t)am * g.lda * E + lchunk * 16;
    } else {
      // weight rows in 64-byte K panels: chunk c of the slice lies in panel c / 4
      src[j] = reinterpret_cast<const uint8_t*>(g.w) + ((int64_t)(lchunk >> 2) * g.ldw + n0 + row - BM) * 64 +
               (lchunk & 3) * 16;
    }
  }
  auto issue = [&](int kt) {
    uint8_t* st = smem + (kt % STAGES) * T::STAGE + T::RPW * wave * RB;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (LNA && R * j < BM) continue;  // the A rows are written by anorm
      // a slice further: RB bytes along an A row, RB / 64 panels of the weight
      dma16(src[j] + (R * j < BM ? (int64_t)kt * RB : (int64_t)kt * RB * g.ldw), st + R * j * RB);
    }
  };

  // ---- LayerNorm-folded A operand. Each thread normalizes, per slice, NA
  // chunks of 8 K-values: chunk column lcol of tile rows (t + i THREADS) /
  // CPRA. The residual chunks, gamma and beta of slice kt + 1 are loaded
  // while slice kt is multiplied. Per element the arithmetic is that of the
  // LayerNorm kernel (fma((x - mean) rs, gamma, beta scale), then the
  // operand rounding), so the LDS tile holds exactly what the LayerNorm
  // kernel would have written.
  constexpr int KV = RB / E;                            // K values per slice
  constexpr int CPRA = KV / 8;                          // 8-value chunks per A row and slice
  constexpr int NA = LNA ? BM * CPRA / T::THREADS : 1;  // chunks per thread and slice
  static_assert(!LNA || (STAGES == 2 && (BM * CPRA) % T::THREADS == 0 && T::THREADS % CPRA == 0),
                "LayerNorm-folded operand: two stages, whole chunks per thread");
  const int lcol = t % CPRA;
  const f16* asrc[NA];
  float amean[NA], ars[NA];
  f16x8 areg[NA];
  f32x4 lgam[2], lbet[2];
  if constexpr (LNA) {
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int am = min(m0 + (t + i * T::THREADS) / CPRA, g.M - 1);  // rows past M: never stored
      const float2 st = reinterpret_cast<const float2*>(g.ln_stats)[am];
      amean[i] = st.x;
      ars[i] = st.y;
      asrc[i] = reinterpret_cast<const f16*>(g.a) + (int64_t)am * g.lda + lcol * 8;
    }
  }
  auto aload = [&](int kt) {
    if constexpr (LNA) {
#pragma unroll
      for (int i = 0; i < NA; ++i) areg[i] = *reinterpret_cast<const f16x8*>(asrc[i] + kt * KV);
      const int k0 = kt * KV + lcol * 8;
      lgam[0] = *reinterpret_cast<const f32x4*>(g.ln_gamma + k0);
      lgam[1] = *reinterpret_cast<const f32x4*>(g.ln_gamma + k0 + 4);
      lbet[0] = *reinterpret_cast<const f32x4*>(g.ln_beta + k0);
      lbet[1] = *reinterpret_cast<const f32x4*>(g.ln_beta + k0 + 4);
    }
  };
  auto anorm = [&](int kt) {
    if constexpr (LNA) {
      uint8_t* st = smem + (kt % STAGES) * T::STAGE;
      float gm[8], bt[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gm[e] = lgam[0][e];
        gm[e + 4] = lgam[1][e];
        bt[e] = lbet[0][e] * g.ln_scale;
        bt[e + 4] = lbet[1][e] * g.ln_scale;
      }
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int r = (t + i * T::THREADS) / CPRA;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(((float)areg[i][e] - amean[i]) * ars[i], gm[e], bt[e]);
        if constexpr (FP8) {  // 8 codes: half of 16-byte chunk lcol / 2
          *reinterpret_cast<uint2*>(st + r * RB + swz<RB>(r, lcol >> 1) * 16 + (lcol & 1) * 8) =
              make_uint2(pack4_e4m3(o[0], o[1], o[2], o[3]), pack4_e4m3(o[4], o[5], o[6], o[7]));
        } else {  // 8 F16 values: chunk lcol
          f16x8 ov;
#pragma unroll
          for (int e = 0; e < 8; ++e) ov[e] = (f16)o[e];
          *reinterpret_cast<f16x8*>(st + r * RB + swz<RB>(r, lcol) * 16) = ov;
        }
      }
    }
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
    const uint8_t* sw = sa + BM * RB;
    if constexpr (!FP8) {
      // RB / 32 steps of K=16: lane group fg takes chunk 2*s + fg of each row
#pragma unroll
      for (int s = 0; s < RB / 32; ++s) {
        f16x8 af[T::TM], wf[T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
          af[i] = *reinterpret_cast<const f16x8*>(sa + arow[i] * RB + swz<RB>(arow[i], 2 * s + fg) * 16);
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          wf[j] = *reinterpret_cast<const f16x8*>(sw + wrow[j] * RB + swz<RB>(wrow[j], 2 * s + fg) * 16);
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
#pragma unroll
          for (int j = 0; j < T::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[j], af[i], acc[i][j], 0, 0, 0);
      }
    } else {
      // RB / 64 steps of K=64: lane group fg takes chunks 4*s + 2*fg and +1.
      // The same K permutation is applied to both operands, so the sum is exact.
#pragma unroll
      for (int s = 0; s < RB / 64; ++s) {
        i32x8 af[T::TM], wf[T::TN];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
          i32x4 lo = *reinterpret_cast<const i32x4*>(sa + arow[i] * RB + swz<RB>(arow[i], 4 * s + 2 * fg) * 16);
          i32x4 hi = *reinterpret_cast<const i32x4*>(sa + arow[i] * RB + swz<RB>(arow[i], 4 * s + 2 * fg + 1) * 16);
          af[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
          i32x4 lo = *reinterpret_cast<const i32x4*>(sw + wrow[j] * RB + swz<RB>(wrow[j], 4 * s + 2 * fg) * 16);
          i32x4 hi = *reinterpret_cast<const i32x4*>(sw + wrow[j] * RB + swz<RB>(wrow[j], 4 * s + 2 * fg + 1) * 16);
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

  using SType = typename StageType<EPI, OUT_FP8>::type;
  constexpr int SB = sizeof(SType);
  constexpr int SROW = BN * SB;  // staged bytes per row
  constexpr int SCH = SROW / 16;
  // chunk swizzle mask: the largest power of two <= 16 that divides the
  // row's chunk count, so a swizzled chunk stays inside its row (a 384-byte
  // e4m3 row has 24 chunks: mask 7)
  constexpr int SWZ = (SCH % 16 == 0 ? 16 : SCH % 8 == 0 ? 8 : SCH % 4 == 0 ? 4 : SCH % 2 == 0 ? 2 : 1) - 1;
  static_assert(SCH % (SWZ + 1) == 0, "swizzled chunks stay inside the row");
  // A tile whose staged form exceeds the ring (the F32 residual tile of the
  // widest tiles) is staged and stored in PASSES bands of PR rows; every
  // 32-row block of a wave falls in one band.
  constexpr int RING = STAGES * T::STAGE;
  constexpr int PASSES = (BM * SROW + RING - 1) / RING;
  constexpr int PR = BM / PASSES;
  static_assert(BM % PASSES == 0 && PR % 32 == 0 && PR * SROW <= RING, "the staged bands fit the LDS ring");
  constexpr int OB = SB == 1 ? 1 : 2;
  constexpr int OCH = BN * OB / 16;  // 16-byte output chunks per row
  constexpr int VPC = 16 / OB;       // values per output chunk
  // Residual prefetch: where the residual tile is stored in one pass with at
  // most four 16-byte chunks per thread (the 128x128 and smaller residual
  // tiles), the residual chunks this thread adds in the epilogue are loaded
  // here, so their latency hides behind the main loop instead of following
  // it. The residual rows are read and written by this workgroup only, so
  // reading them early is safe in place too. These loads are older than every
  // slice transfer, so the slice waits below also cover them.
  constexpr int NPF = (EPI == EPI_BIAS_RES && PASSES == 1 && (PR * OCH) % T::THREADS == 0 &&
                       PR * OCH / T::THREADS <= 4) ? PR * OCH / T::THREADS : 0;
  f16x8 rpf[NPF > 0 ? NPF : 1];
  if constexpr (NPF > 0) {
#pragma unroll
    for (int i = 0; i < NPF; ++i) {
      const int u = t + i * T::THREADS;
      const int rs = u / OCH;
      const int m = m0 + rs;
      if (m < g.M) rpf[i] = *reinterpret_cast<const f16x8*>(g.res + (int64_t)m * g.ldres + n0 + (u - rs * OCH) * VPC);
    }
  }

  // Residual tiles whose F32 staged form takes more than one pass (the
  // 192x384 tile) but whose F16 form fits the two-stage ring (RES_LDS): the
  // F16 residual tile comes into the ring by DMA as 16-byte chunks, swizzled
  // by row like the staged tiles of the epilogue. Half h of its rows fills
  // stage h: the half whose stage is free while the last K slice is
  // multiplied goes then, the other after the main loop. The residual rows
  // are read and written by this workgroup only, so the early read is safe
  // in place.
  constexpr bool RES_LDS = EPI == EPI_BIAS_RES && STAGES == 2 && !LNA &&
                           BM * BN * 8 > STAGES * T::STAGE && BM * BN * 2 == STAGES * T::STAGE;
  constexpr int RROW = BN * 2;  // F16 bytes per residual tile row
  constexpr int RCH = RROW / 16;
  constexpr int RSWZ = (RCH % 16 == 0 ? 16 : RCH % 8 == 0 ? 8 : RCH % 4 == 0 ? 4 : RCH % 2 == 0 ? 2 : 1) - 1;
  static_assert(RCH % (RSWZ + 1) == 0, "swizzled chunks stay inside the row");
  auto raddr = [&](int r, int byte) -> uint8_t* {
    return smem + r * RROW + ((((byte >> 4) ^ (r & RSWZ)) << 4) | (byte & 15));
  };
  constexpr int RDMA = BM / 2 * RCH / (64 * T::WAVES);  // 1 KiB transfers per wave and half
  static_assert(!RES_LDS || (BM / 2 * RCH) % (64 * T::WAVES) == 0, "whole residual transfers");
  auto res_dma = [&](int h) {
#pragma unroll
    for (int j = 0; j < RDMA; ++j) {
      const int kib = (h * RDMA + j) * T::WAVES + wave;
      const int slot = kib * 64 + lane;                    // LDS chunk this lane fills
      const int r = slot / RCH;
      const int c = (slot - r * RCH) ^ (r & RSWZ);          // the logical chunk kept there
      const int m = min(m0 + r, g.M - 1);                    // rows past M: read, never stored
      dma16(g.res + (int64_t)m * g.ldres + n0 + c * 8, smem + kib * 1024);
    }
  };

  if constexpr (LNA) {
    // Two stages. Iteration kt writes the A part of stage kt % 2, last read
    // by slice kt - 2's products, which every wave finished before the
    // previous barrier; the barrier here makes the A rows and the weight
    // transfers of slice kt visible, and slice kt - 1's stage free for the
    // transfers of slice kt + 1.
    aload(0);
    issue(0);
    for (int kt = 0; kt < nk; ++kt) {
      wait_vmcnt<0>();
      anorm(kt);
      __syncthreads();
      if (kt + 1 < nk) {
        aload(kt + 1);
        issue(kt + 1);
      }
      compute(kt % STAGES);
    }
  } else {
    // prologue: the first STAGES-1 slices in flight
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (p < nk) issue(p);
    for (int kt = 0; kt < nk; ++kt) {
      // this thread's transfers of slice kt are done when at most the newer
      // slices' transfers remain; the barrier then makes every wave's visible
      // and guarantees that slice kt-1's buffer is no longer being read
      if (kt + STAGES - 2 < nk)
        wait_vmcnt<(STAGES - 2) * CH>();
      else
        wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1);
      else if (RES_LDS && kt == nk - 1) res_dma(nk % 2);  // the stage slice kt-1 held
      compute(kt % STAGES);
    }
  }

  // ---- epilogue: lane holds row m = tile row + fr, columns 8q + 4fg + (0..3)
  if constexpr (EPI == EPI_QKV || EPI == EPI_QKV8) {
    if (n0 + wn * WN >= g.vt_col0) {
      // V columns (whole tiles: vt_col0 is a multiple of the tile width): 4 consecutive
      // dims of one head written transposed. The 32 lanes of a half-wave hold
      // 32 consecutive tokens, so each store covers 64 (F16) or 32 (e4m3)
      // contiguous bytes of a V^T row.
      using VT = typename std::conditional<OUT_FP8, uint8_t, f16>::type;
#pragma unroll
      for (int i = 0; i < T::TM; ++i) {
        const int m = m0 + wm * WM + i * 32 + fr;
        if (m >= g.M) continue;
        const int bb = m / g.vt_tokens, tt = m - bb * g.vt_tokens;
        VT* vrow0 = reinterpret_cast<VT*>(g.vt) + (int64_t)bb * g.vt_heads * g.vt_dim * g.vt_ld + tt;
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int n = n0 + wn * WN + j * 32 + 8 * qq + 4 * fg;
            const f32x4 bv = *reinterpret_cast<const f32x4*>(g.bias + n);
            const int hd = n - g.vt_col0;  // head*dim + d; the 4 dims never cross a head (dim % 4 == 0)
            const int hh = (int)(((float)hd + 0.5f) * g.vt_inv_dim);  // exact: hd < 2^20, dim <= 2^10
            const int dd = hd - hh * g.vt_dim;
            VT* dst = vrow0 + ((int64_t)hh * g.vt_dim + dd) * g.vt_ld;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = acc[i][j][4 * qq + r] * g.acc_scale + bv[r];
              if constexpr (OUT_FP8)
                dst[r * g.vt_ld] = (uint8_t)(cvt_pk_e4m3(v * g.out_scale, 0.f, 0u, false) & 0xFF);
              else
                dst[r * g.vt_ld] = (f16)v;
            }
          }
        }
      }
      return;
    }
  }
  // Residual tiles whose F32 staged form takes more than one pass: the
  // residual tile is in LDS (res_dma); each lane adds its accumulators to the
  // residual values of its rows in registers and writes the F16 sums back in
  // place (the same arithmetic as the staged path: acc * acc_scale is exact,
  // then + bias, + residual, one F16 rounding), and the workgroup stores
  // whole 16-byte row chunks.
  if constexpr (RES_LDS) {
    __syncthreads();  // every wave is done with the ring
    res_dma(1 - nk % 2);  // the half the last slice's stage held
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * WN + j * 32 + 8 * q + 4 * fg;
        const f32x4 b = *reinterpret_cast<const f32x4*>(g.bias + n0 + c);
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
          f16x4* p = reinterpret_cast<f16x4*>(raddr(wm * WM + i * 32 + fr, 2 * c));
          const f16x4 rv = *p;
          f16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (f16)((acc[i][j][4 * q + e] * g.acc_scale + b[e]) + (float)rv[e]);
          *p = o;
        }
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int u = t; u < BM * RCH; u += T::THREADS) {
      const int rs = u / RCH;
      const int c = (u - rs * RCH) * 8;
      const int m = m0 + rs;
      if (m >= g.M) continue;
      *reinterpret_cast<i32x4*>(reinterpret_cast<f16*>(g.c) + (int64_t)m * g.ldc + n0 + c) =
          *reinterpret_cast<const i32x4*>(raddr(rs, 2 * c));
    }
    return;
  }
  // Output through LDS. The MFMA layout gives each lane 4-column pieces of
  // 32 different rows, so direct stores write 4 or 8 bytes per row per
  // instruction. Instead every wave puts its values (bias, positional
  // embedding and GELU applied; with a residual still to come, kept F32) into
  // the tile staged in the now idle LDS ring, then the workgroup writes whole
  // 16-byte chunks of output rows, consecutive threads covering consecutive
  // chunks, adding the residual there from 16-byte loads. Staged rows are
  // swizzled in 16-byte chunks by row so the column-wise writes of 16 rows
  // hit distinct banks.
  auto saddr = [&](int r, int byte) -> uint8_t* {
    return smem + r * SROW + ((((byte >> 4) ^ (r & SWZ)) << 4) | (byte & 15));
  };
  // The GELU epilogue with e4m3 output applies its power-of-two output scale
  // to the GELU input (exactly) and to the GELU constants instead of to
  // every output.
  constexpr bool GELU8 = EPI == EPI_BIAS_GELU && SB == 1;
  const float pre = GELU8 ? g.out_scale : 1.0f;
  const float vscale = g.acc_scale * pre;
  const GeluConsts gk = gelu_consts(pre);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    // every wave is done with the ring (no transfer is outstanding), or with
    // the previous band's stores
    __syncthreads();
    // column pieces outermost so each lane's bias quad is loaded (and
    // scaled) once for all its row blocks
#pragma unroll
    for (int j = 0; j < T::TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * WN + j * 32 + 8 * q + 4 * fg;
        const int n = n0 + c;
        f32x4 b = *reinterpret_cast<const f32x4*>(g.bias + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] *= pre;
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
          const int r = wm * WM + i * 32 + fr;  // tile row
          if ((wm * WM + i * 32) / PR != pass) continue;
          const int rs = r - pass * PR;  // row of the staged band
          const int m = m0 + r;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] * vscale + b[e];
          if constexpr (EPI == EPI_BIAS_POS) {
            const f32x4 p = *reinterpret_cast<const f32x4*>(g.pos + (int64_t)(m % g.pos_rows) * g.ldpos + n);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += p[e];
          }
          if constexpr (EPI == EPI_BIAS_GELU) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu_tanh_scaled(v[e], gk);
          }
          if constexpr (SB == 4) {
            *reinterpret_cast<f32x4*>(saddr(rs, 4 * c)) = f32x4{v[0], v[1], v[2], v[3]};
          } else if constexpr (SB == 2) {
            *reinterpret_cast<f16x4*>(saddr(rs, 2 * c)) = f16x4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
          } else if constexpr (GELU8) {
            *reinterpret_cast<uint32_t*>(saddr(rs, c)) = pack4_e4m3(v[0], v[1], v[2], v[3]);
          } else {
            const float sc = EPI == EPI_QKV8 ? g.qk8_scale : g.out_scale;
            *reinterpret_cast<uint32_t*>(saddr(rs, c)) = pack4_e4m3(v[0] * sc, v[1] * sc, v[2] * sc, v[3] * sc);
          }
        }
      }
    }
    __syncthreads();
    if constexpr (EPI == EPI_QKV8) {
      // e4m3 Q/K codes into head slots: 8 consecutive columns never cross a
      // head (vt_dim % 8 == 0, n0 % 8 == 0), so each 8-byte group of a staged
      // row is one 8-byte store; consecutive threads take consecutive groups
      constexpr int G = BN / 8;
#pragma unroll 4
      for (int u = t; u < PR * G; u += T::THREADS) {
        const int rs = u / G;
        const int c = (u - rs * G) * 8;
        const int m = m0 + pass * PR + rs;
        if (m >= g.M) continue;
        const int n = n0 + c;
        const int hh = (int)(((float)n + 0.5f) * g.vt_inv_dim);  // exact: n < 2^20, dim <= 2^10
        const int dd = n - hh * g.vt_dim;
        *reinterpret_cast<uint2*>(g.qk8 + (int64_t)m * g.qk8_ld + hh * g.qk8_pitch + dd) =
            *reinterpret_cast<const uint2*>(saddr(rs, c));
      }
    } else if constexpr (NPF > 0) {
      // the residual tile with its prefetched chunks (PASSES == 1, every
      // thread owns NPF whole chunks)
#pragma unroll
      for (int i = 0; i < NPF; ++i) {
        const int u = t + i * T::THREADS;
        const int rs = u / OCH;
        const int c = (u - rs * OCH) * VPC;
        const int m = m0 + rs;
        if (m >= g.M) continue;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(saddr(rs, 4 * c));
        const f32x4 hi = *reinterpret_cast<const f32x4*>(saddr(rs, 4 * c + 16));
        f16x8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = (f16)(lo[e] + (float)rpf[i][e]);
          o[e + 4] = (f16)(hi[e] + (float)rpf[i][e + 4]);
        }
        *reinterpret_cast<f16x8*>(reinterpret_cast<f16*>(g.c) + (int64_t)m * g.ldc + n0 + c) = o;
      }
    } else {
#pragma unroll 4
      for (int u = t; u < PR * OCH; u += T::THREADS) {
        const int rs = u / OCH;
        const int c = (u - rs * OCH) * VPC;
        const int m = m0 + pass * PR + rs;
        if (m >= g.M) continue;
        uint8_t* dst = reinterpret_cast<uint8_t*>(g.c) + ((int64_t)m * g.ldc + n0 + c) * OB;
        if constexpr (SB == 4) {  // F32 staged, residual added here, F16 out
          const f32x4 lo = *reinterpret_cast<const f32x4*>(saddr(rs, 4 * c));
          const f32x4 hi = *reinterpret_cast<const f32x4*>(saddr(rs, 4 * c + 16));
          const f16x8 rr = *reinterpret_cast<const f16x8*>(g.res + (int64_t)m * g.ldres + n0 + c);
          f16x8 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = (f16)(lo[e] + (float)rr[e]);
            o[e + 4] = (f16)(hi[e] + (float)rr[e + 4]);
          }
          *reinterpret_cast<f16x8*>(dst) = o;
        } else {
          *reinterpret_cast<i32x4*>(dst) = *reinterpret_cast<const i32x4*>(saddr(rs, c * SB));
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, bool FP8, int EPI, bool OUT_FP8, int RB = kRowBytes,
          int MINW = 1, bool LNA = false>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  if (g.N % BN != 0 || (g.K * (FP8 ? 1 : 2)) % RB != 0) return hipErrorInvalidValue;  // whole tiles and slices
  dim3 grid((g.N / BN) * ((g.M + BM - 1) / BM));
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, STAGES, FP8, EPI, OUT_FP8, RB, MINW, LNA>), grid,
                     dim3(Tile<BM, BN, WM, WN, RB>::THREADS), 0, s, g);
  return hipGetLastError();
}

template <bool FP8, int EPI, bool OUT_FP8>
hipError_t launch_sized(const GemmArgs& g, hipStream_t s) {
  // Tile choice measured on the batch-64 shapes (M = 46,656): the GELU
  // epilogue takes 128x256 tiles (256x128 where N % 256 != 0), residual,
  // long-K and wide QKV GEMMs 192x384 where N divides by 384,
  // other N divisible by 256 256x256 tiles of eight waves (128x64 each, one
  // workgroup per CU), the rest 128x128 tiles of eight waves (64x32 each)
  // with two LDS stages, two workgroups per CU. Small M falls back to
  // smaller tiles that still fill the 256 CUs.
  const long tiles_128 = (long)((g.M + 127) / 128) * (g.N / 128);
  // LayerNorm-folded A operand (the epilogues of the projections that
  // follow a LayerNorm): one tile shape at every size, 128x128 of eight
  // waves, two stages
  if constexpr (EPI == EPI_BIAS || EPI == EPI_QKV || EPI == EPI_QKV8 || EPI == EPI_BIAS_GELU) {
    if (g.ln_stats) {
      GemmArgs b = g;
      if (b.group_m == 0 && tiles_128 >= 1024) b.group_m = 8;
      // two workgroups per CU where the registers allow it without spills (the
      // GELU epilogue: 128 VGPRs; 864 -> 600 us at 46,656 x 4,352 x 1,152)
      constexpr int LW = EPI == EPI_BIAS_GELU && (OUT_FP8 || !FP8) ? 4 : 1;
      return launch_cfg<128, 128, 64, 32, 2, FP8, EPI, OUT_FP8, kRowBytes, LW, true>(b, s);
    }
  } else {
    if (g.ln_stats) return hipErrorInvalidValue;
  }
  if (tiles_128 >= 1024) {
    // Large grids walk tiles in bands of row blocks (tile_of) unless the
    // caller chose a band: 4 row blocks for 256x256 tiles, 8 for the others
    // (measured at 46,656 rows: 1-3% over row-block-major order).
    GemmArgs b = g;
    // 256x256 tiles: not for the residual epilogue (its F32 staged tile
    // would not fit the LDS ring) nor the V-transposing one (a tile must not
    // straddle the V column boundary)
    // GELU epilogue (MLP up): tiles of four waves with a 3-stage ring of
    // 64-byte K slices, 72 KiB of LDS, so two workgroups share a CU and one's
    // VALU-heavy epilogue (bias, GELU, e4m3) runs beside the other's MFMA
    // main loop (measured at 46,656 x 4,352 x 1,152: 2-7% faster than one
    // 256x256 workgroup per CU, the same bits; slower for the residual and
    // QKV epilogues). With N % 256 == 0, 128x256 tiles (waves of 64x128): the
    // larger share of each slice is weight rows, which the 64-byte K panels
    // make contiguous, so the activation rows' half-line fetches weigh less
    // (255-273 against 267-287 us on two boxes, the same bits); else 256x128.
    if constexpr (EPI == EPI_BIAS_GELU) {
      if (b.group_m == 0) b.group_m = 8;
      if (g.N % 256 == 0) return launch_cfg<128, 256, 64, 128, 3, FP8, EPI, OUT_FP8, 64, 2>(b, s);
      return launch_cfg<256, 128, 128, 64, 3, FP8, EPI, OUT_FP8, 64, 2>(b, s);
    }
    // Long K (MLP down, K = 4352), wide N (the fused QKV projection, 3456;
    // the explicit MAP K/V, 2304) or a residual: 192x384 tiles, 2 stages, 144 KiB of LDS.
    // Per flop they move half the operand bytes of 128x128 tiles from L2
    // into LDS (A is re-read for 3 column blocks of 1152 instead of 9), which
    // is what bounds these GEMMs: at 46,656 rows MLP down 280 -> 245 us and a
    // 3456-wide projection 235-251 -> 222 us with eight waves of 96x96, the
    // same bits. Twelve waves of 96x64 (164-167 VGPRs, three waves per SIMD
    // instead of two, to cover the slice waits and the epilogue) take a
    // 3456-wide projection from 221-231 to 207-215 us and MLP down from
    // ~248 to 233-251 us, the same bits. The residual tile comes into the
    // ring by DMA, half of it during the last K slice, and is added in
    // registers (RES_LDS; MLP down 234 -> 225 us against the F32 tile
    // staged in two bands, 233 -> 229 us for the half issued early, the
    // same bits). The out-projection (K = 1152) takes them too since its
    // residual is added that way: 95.8 -> 91.3 us per launch (with the F32
    // tile in two bands it was 98 -> 105-113 us). A V-transposing tile must
    // not straddle the V columns.
    if constexpr (EPI == EPI_BIAS_RES || EPI == EPI_BIAS || EPI == EPI_QKV || EPI == EPI_QKV8) {
      constexpr bool qkv = EPI == EPI_QKV || EPI == EPI_QKV8;
      const bool fits = g.N % 384 == 0 && (!qkv || g.vt_col0 % 384 == 0);
      if (fits && ((int64_t)g.K * (FP8 ? 1 : 2) >= 2048 || g.N >= 2304 || EPI == EPI_BIAS_RES)) {
        if (b.group_m == 0) b.group_m = 8;
        return launch_cfg<192, 384, 96, 64, 2, FP8, EPI, OUT_FP8>(b, s);
      }
    }
    if constexpr (EPI != EPI_BIAS_RES && EPI != EPI_QKV && EPI != EPI_QKV8)
      if (g.N % 256 == 0) {
        if (b.group_m == 0) b.group_m = 4;
        return launch_cfg<256, 256, 128, 64, 2, FP8, EPI, OUT_FP8>(b, s);
      }
    if (b.group_m == 0) b.group_m = 8;
    return launch_cfg<128, 128, 64, 32, 2, FP8, EPI, OUT_FP8>(b, s);
  }
  if (tiles_128 >= 384) return launch_cfg<128, 128, 64, 64, 2, FP8, EPI, OUT_FP8>(g, s);
  // Fewer 64x64 tiles than two per CU (729 rows x 1152 columns: 216): each
  // workgroup's run of K slices is the critical path, so a fourth stage
  // keeps one more slice in flight (measured: 15.0 -> 13.4 us for 729 x 1152
  // x 4352, 6.0 -> 5.6 us for K = 1152; larger grids gain nothing from it).
  const long tiles_64 = (long)((g.M + 63) / 64) * (g.N / 64);
  // A grid of at most one 64x64 workgroup per CU with a long K (MLP down at
  // batch 1, K = 4352) takes 256-byte slices: half the slices, and with them
  // half the per-slice waits and barriers that make up its critical path
  // (729 x 1152 x 4352: e4m3 16.4 -> 14.8 us, F16 27.0 -> 24.9 us, the same
  // bits: the K order of every output is unchanged). Their 128 KiB ring
  // leaves room for one workgroup per CU, so larger grids (1458 rows: 20.4
  // -> 24.6 us) and short K (1152: up to 30% slower) keep 128-byte slices.
  if (tiles_64 < 512) {
    const int64_t kb = (int64_t)g.K * (FP8 ? 1 : 2);
    if (tiles_64 <= 256 && kb >= 4096 && kb % 256 == 0)
      return launch_cfg<64, 64, 32, 32, 4, FP8, EPI, OUT_FP8, 256>(g, s);
    return launch_cfg<64, 64, 32, 32, 4, FP8, EPI, OUT_FP8>(g, s);
  }
  // Between the two: 128x64 tiles of four waves (64x32 each), three stages.
  // Measured with every launch reading its weights cold from HBM (as the
  // layers of one small-batch call do), against 64x64 tiles with three
  // stages: 729 x 4352 x 1152 14.5 -> 11.3 us, 729 x 3456 x 1152 10.4 ->
  // 9.9 us, 2916 x 1152 x 4352 34.7 -> 24.7 us, 2916 x 1152 x 1152 12.6 ->
  // 10.3 us.
  return launch_cfg<128, 64, 64, 32, 3, FP8, EPI, OUT_FP8>(g, s);
}

template <bool FP8>
hipError_t launch_epi(const GemmArgs& g, int epi, bool out_fp8, hipStream_t s) {
  switch (epi) {
    case EPI_BIAS: return launch_sized<FP8, EPI_BIAS, false>(g, s);
    case EPI_BIAS_POS: return launch_sized<FP8, EPI_BIAS_POS, false>(g, s);
    case EPI_BIAS_RES: return launch_sized<FP8, EPI_BIAS_RES, false>(g, s);
    case EPI_QKV:
      return out_fp8 ? launch_sized<FP8, EPI_QKV, true>(g, s) : launch_sized<FP8, EPI_QKV, false>(g, s);
    case EPI_QKV8:
      return out_fp8 ? launch_sized<FP8, EPI_QKV8, true>(g, s) : launch_sized<FP8, EPI_QKV8, false>(g, s);
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
  const int EA = g.ln_stats ? 2 : E;  // a LayerNorm-folded A operand is the F16 residual
  if (g.M < 1 || g.N < 64 || g.N % 128 != 0 || g.K < 1 || (g.K * E) % kRowBytes != 0)
    return hipErrorInvalidValue;
  if (g.lda < g.K || g.ldw < g.N || g.ldc < g.N) return hipErrorInvalidValue;
  if ((int64_t)g.M * g.lda * EA >= (int64_t)1 << 31 || (int64_t)g.K * E * g.ldw >= (int64_t)1 << 31)
    return hipErrorInvalidValue;
  if (g.ln_stats && (!g.ln_gamma || !g.ln_beta || (reinterpret_cast<uintptr_t>(g.ln_stats) & 7) ||
                     (reinterpret_cast<uintptr_t>(g.ln_gamma) & 15) || (reinterpret_cast<uintptr_t>(g.ln_beta) & 15)))
    return hipErrorInvalidValue;
  // e4m3 output: the GELU epilogue's output, or V^T of the QKV epilogue
  const bool qkv = epi == EPI_QKV || epi == EPI_QKV8;
  if (out_fp8 && epi != EPI_BIAS_GELU && !qkv) return hipErrorInvalidValue;
  // 16-byte transfers: operand rows, output rows and residual rows aligned
  const int OB = (out_fp8 && !qkv) ? 1 : 2;
  auto misaligned = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; };
  if (misaligned(g.a) || misaligned(g.w) || misaligned(g.c) || (g.lda * EA) % 16 ||
      (g.ldc * OB) % 16)
    return hipErrorInvalidValue;
  if (epi == EPI_BIAS_RES && (!g.res || misaligned(g.res) || g.ldres % 8 || g.ldres < g.N))
    return hipErrorInvalidValue;
  if (qkv && (!g.vt || g.vt_dim < 4 || g.vt_dim % 4 || g.vt_dim > 1024 || g.vt_col0 % 128 ||
              g.vt_tokens < 1 || g.vt_ld < g.vt_tokens || g.N >= (1 << 20) ||
              (g.N - g.vt_col0) != g.vt_heads * g.vt_dim))
    return hipErrorInvalidValue;
  if (epi == EPI_QKV8 && (!g.qk8 || g.vt_dim % 8 || g.vt_col0 % g.vt_dim || g.qk8_pitch < g.vt_dim ||
                          g.qk8_pitch % 16 || g.qk8_ld < (int64_t)(g.vt_col0 / g.vt_dim) * g.qk8_pitch ||
                          g.qk8_ld % 16 || misaligned(g.qk8)))
    return hipErrorInvalidValue;
  return in_fp8 ? launch_epi<true>(g, epi, out_fp8, s) : launch_epi<false>(g, epi, out_fp8, s);
}

}  // namespace siglip
