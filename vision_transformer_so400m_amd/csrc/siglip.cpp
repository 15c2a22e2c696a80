// libsiglip: C ABI, weight-blob parsing, resident weights, workspace and the
// per-call kernel sequence of the SigLIP So400m/14 image encoder on one
// gfx950 GPU. The sequence follows the page "Single-layer SigLIP vision
// benchmark" (intro and mermaid figure):
//
//   X [B*T, 588] --pad/convert--> Xp [B*T, 640]
//   H = Xp Wpe + bpe + pos[t]                      (GEMM, EPI_BIAS_POS)
//   per layer:  A = LN1(H)                         (layernorm)
//               QKV = A Wqkv + b                   (GEMM, EPI_QKV: V transposed)
//               O = attention(Q, K, V^T)           (streaming flash attention)
//               H = O Wo + bo + H                  (GEMM, EPI_BIAS_RES, in place)
//               A = LN2(H)
//               U = gelu(A W1 + b1)                (GEMM, EPI_BIAS_GELU)
//               H = U W2 + b2 + H                  (GEMM, EPI_BIAS_RES)
//   Z = LN(H); o = probe attention of q over K = Z Wk + bk, V = Z Wv + bv
//   y = o Wo' + bo'; out = gelu(LN(y) W1' + b1') W2' + b2' + y
//
// The probe is the same for every image (same page, intro: one learned probe
// shared by the whole batch), so its query q = probe Wq + bq is a model
// constant. By default the MAP K/V projection is folded away: create computes
// q, u_h = W_k,h q_h and W_v transposed with small GPU kernels, and each call
// computes the scores Z u_h and (sum_t p_t Z_t) W_v,h + b_v,h (map.hip). With
// the explicit K/V option, q comes from the projection GEMM at create and
// every call runs the K/V GEMM and the probe attention.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <climits>
#include <exception>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/siglip.h"
#include "../../include/siglip_test_hooks.h"
#include "common.h"

using namespace siglip;

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

struct HipFail {
  hipError_t err;
  std::string where;
};

void hip_check(hipError_t e, const char* where) {
  if (e != hipSuccess) throw HipFail{e, where};
}

struct BadBlob {
  std::string msg;
};

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

constexpr int kKAlign = 128;  // K padding (elements): whole 128-byte slices for both F16 and e4m3
constexpr int kNAlign = 128;  // N padding: the widest GEMM column tile
constexpr int kQK8SlotBytes = 80;  // e4m3 Q/K head slot: 16-byte aligned rows for the attention's transfers

struct Gemm {
  void* w = nullptr;      // [n_pad, k_pad] F16 or e4m3, K-contiguous in 64-byte K panels
  float* bias = nullptr;  // [n_pad]
  int k = 0, n = 0, k_pad = 0, n_pad = 0;
};

struct Layer {
  float *ln1_g, *ln1_b, *ln2_g, *ln2_b;
  Gemm qkv, out, mlp1, mlp2;
  Gemm q, k, v;  // the three column blocks of qkv (separate-projection option only)
};

struct BlobHeader {
  char magic[4];
  uint32_t version, width, depth, heads, head_dim, mlp, tokens, patch_dim, dtype;
  uint64_t total_bytes;
  uint8_t reserved[16];
};
static_assert(sizeof(BlobHeader) == 64, "blob header is 64 bytes");

struct TensorRef {
  const float* host;
  int64_t rows, cols;
};

// Walks the blob in canonical order, checking bounds.
class BlobReader {
 public:
  BlobReader(const uint8_t* base, size_t size) : base_(base), size_(size), off_(64) {}
  TensorRef next(const char* name, int64_t rows, int64_t cols) {
    off_ = (size_t)round_up((int64_t)off_, 64);
    const size_t n = (size_t)(rows * cols) * 4;
    if (off_ + n > size_) throw BadBlob{std::string("blob truncated at tensor ") + name};
    TensorRef r{reinterpret_cast<const float*>(base_ + off_), rows, cols};
    off_ += n;
    return r;
  }
  size_t end() const { return (size_t)round_up((int64_t)off_, 64); }

 private:
  const uint8_t* base_;
  size_t size_;
  size_t off_;
};

}  // namespace

struct siglip_model {
  int device = 0;
  int width = 0, depth = 0, layers = 0, heads = 0, head_dim = 0, mlp = 0, tokens = 0, patch_dim = 0;
  int max_batch = 0;
  bool fp8 = false;
  int scale_exp = 0;
  float op_scale = 1.0f;   // operand quantization multiplier 2^-exp
  float acc_scale = 1.0f;  // product rescale 2^(2 exp)
  int patch_pad = 0, mlp_pad = 0;
  bool vt_path = false;  // streaming attention (head dims 64, 72, 80): V^T buffer in the workspace
  bool vrow_ok = false;  // F16 attention products: one-round calls read V row-major instead (vrow_call)
  bool attn_fp8 = false; // PV product in e4m3: V^T as e4m3 codes of v * attn_v_scale
  bool attn_qk8 = false; // QK product in e4m3: Q and K as e4m3 codes of x * attn_v_scale in the
                         // QKV buffer's bytes, head h of a token row at byte h * 80 (K after Q)
  float attn_v_scale = 1.0f;
  int tokens_pad = 0;    // V^T row length: tokens rounded up to the 64-key block

  std::vector<void*> allocs;
  Gemm embed;
  float* pos = nullptr;
  std::vector<Layer> L;
  float *lnf_g = nullptr, *lnf_b = nullptr;
  Gemm mq, mkv, mout, mmlp1, mmlp2;
  Gemm mk, mv;  // the two column blocks of mkv (separate-projection option only)
  bool separate_qkv = false;
  // LayerNorms 1 and 2 folded into the QKV and MLP-up GEMMs: a statistics
  // kernel writes {mean, rstd * scale} per row and the GEMMs normalize the
  // F16 residual rows themselves
  bool ln_fold = false;
  // MAP head with the K/V projection folded: u_h = W_k,h q_h in two F16
  // parts, W_v transposed per head [width (h, d), width (k)] and b_v F32
  bool map_fold = false;
  f16 *u_hi = nullptr, *u_lo = nullptr;
  float *wv = nullptr, *bv = nullptr;
  float *mln_g = nullptr, *mln_b = nullptr;
  f16* map_q = nullptr;  // [width]

  // workspace
  void* ws = nullptr;
  size_t ws_bytes = 0;
  void* xp = nullptr;   // [M, patch_pad] operand type
  f16* h = nullptr;     // [M, width]
  void* a = nullptr;    // [M, width] operand type
  f16* qkv = nullptr;   // [M, 3 width] (also the MAP KV [M, 2 width])
  void* o = nullptr;    // [M, width] operand type
  void* u = nullptr;    // [M, mlp_pad] operand type
  void* mo = nullptr;   // [B, width] operand type
  f16* my = nullptr;    // [B, width]
  void* ma = nullptr;   // [B, width] operand type
  void* mu = nullptr;   // [B, mlp_pad] operand type
  f16* vt = nullptr;    // [B*heads*head_dim, tokens_pad] (vt_path only)
  float* mscores = nullptr;  // [B, 16, tokens] F32 (map_fold only)
  float* zbar = nullptr;     // [B, 16, width] F32 (map_fold only)
  float* lnst = nullptr;     // [M, 2] F32 LayerNorm row statistics (ln_fold only)

  // diagnostics
  int capture_layer = -1;
  bool captured = false;
  int captured_batch = 0;
  void* cap[SIGLIP_STAGE_COUNT] = {};
  size_t cap_bytes[SIGLIP_STAGE_COUNT] = {};

  // two half-batches on two streams (images are independent): a second
  // stream of default priority and the events that fork it from the
  // caller's stream and join it back
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;

  // per-launch timing: event pairs recorded around launches, resolved on read
  uint32_t timing_mask = 0;               // classes whose launches are timed
  std::vector<hipEvent_t> ev_pool;        // 2 events per pending launch
  std::vector<int> ev_class;              // class of each pending pair
  size_t ev_used = 0;                     // pairs in use
  bool timing_lost = false;               // an end event failed to record
  double t_ms[SIGLIP_K_COUNT] = {};
  int64_t t_n[SIGLIP_K_COUNT] = {};

  ~siglip_model() {
    for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
    if (fork_ev) (void)hipEventDestroy(fork_ev);
    if (join_ev) (void)hipEventDestroy(join_ev);
    if (side) (void)hipStreamDestroy(side);
    for (void* p : allocs) (void)hipFree(p);
  }

  int esz() const { return fp8 ? 1 : 2; }

  void* dalloc(size_t bytes) {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, std::max<size_t>(bytes, 256));
    if (e != hipSuccess) throw HipFail{e, "hipMalloc"};
    allocs.push_back(p);
    return p;
  }
};

namespace {

float* upload_f32(siglip_model* m, const TensorRef& t, int64_t pad_to = 0) {
  const int64_t n = t.rows * t.cols;
  const int64_t np = std::max(n, pad_to);
  float* d = static_cast<float*>(m->dalloc((size_t)np * 4));
  if (np > n) hip_check(hipMemset(d, 0, (size_t)np * 4), "hipMemset");
  hip_check(hipMemcpy(d, t.host, (size_t)n * 4, hipMemcpyHostToDevice), "hipMemcpy");
  return d;
}

// weight [k, n] F32 (host) -> resident [n_pad, k_pad] operand type + F32 bias
Gemm make_gemm(siglip_model* m, const TensorRef& w, const TensorRef& b, float* staging) {
  Gemm g;
  g.k = (int)w.rows;
  g.n = (int)w.cols;
  g.k_pad = (int)round_up(g.k, kKAlign);
  g.n_pad = (int)round_up(g.n, kNAlign);
  g.w = m->dalloc((size_t)g.n_pad * g.k_pad * m->esz());
  hip_check(hipMemcpy(staging, w.host, (size_t)g.k * g.n * 4, hipMemcpyHostToDevice), "hipMemcpy");
  hip_check(launch_weight_transpose(staging, g.k, g.n, g.w, g.k_pad, g.n_pad, m->fp8, m->fp8 ? m->op_scale : 1.0f, nullptr),
            "weight_transpose");
  hip_check(hipDeviceSynchronize(), "weight_transpose sync");
  g.bias = upload_f32(m, b, g.n_pad);
  return g;
}

// Columns c0 .. c0+n-1 of a host [rows, cols] tensor (a weight [in, out] or
// a bias [1, out]) as a contiguous copy in buf.
TensorRef column_block(const TensorRef& t, int64_t c0, int64_t n, std::vector<float>& buf) {
  buf.resize((size_t)(t.rows * n));
  for (int64_t r = 0; r < t.rows; ++r)
    std::memcpy(buf.data() + r * n, t.host + r * t.cols + c0, (size_t)n * 4);
  return TensorRef{buf.data(), t.rows, n};
}

// make_gemm of columns c0 .. c0+n-1 of a fused projection
Gemm make_gemm_block(siglip_model* m, const TensorRef& w, const TensorRef& b, int64_t c0, int64_t n, float* staging) {
  std::vector<float> wb, bb;
  const TensorRef ws = column_block(w, c0, n, wb);
  const TensorRef bs = column_block(b, c0, n, bb);
  return make_gemm(m, ws, bs, staging);
}

// Constants of the folded MAP head, computed on the device from the F32 blob
// tensors (map.hip, launch_map_fold_prepare): q = probe Wq + bq (kept as F16
// for the MAP_Q checkpoint), u_h = W_k,h q_h as F16 hi + lo parts in 16 head
// rows, W_v transposed per head; b_v is the V half of the fused bias.
void make_map_fold(siglip_model* m, const TensorRef& probe, const TensorRef& qw, const TensorRef& qb,
                   const TensorRef& kvw, const TensorRef& kvb) {
  const int W = m->width;
  m->map_q = static_cast<f16*>(m->dalloc((size_t)W * 2));
  m->u_hi = static_cast<f16*>(m->dalloc((size_t)16 * W * 2));
  m->u_lo = static_cast<f16*>(m->dalloc((size_t)16 * W * 2));
  m->wv = static_cast<float*>(m->dalloc((size_t)W * W * 4));
  m->bv = static_cast<float*>(m->dalloc((size_t)W * 4));
  hip_check(hipMemcpy(m->bv, kvb.host + W, (size_t)W * 4, hipMemcpyHostToDevice), "hipMemcpy");
  // the blob tensors the constants come from, for the duration of the call
  float* tmp = nullptr;
  const size_t nf = (size_t)W + (size_t)W * W + W + (size_t)W * 2 * W + W;  // probe, Wq, bq, Wkv, q
  hip_check(hipMalloc(&tmp, nf * 4), "hipMalloc");
  float* d_probe = tmp;
  float* d_wq = d_probe + W;
  float* d_bq = d_wq + (size_t)W * W;
  float* d_wkv = d_bq + W;
  float* d_q = d_wkv + (size_t)W * 2 * W;
  hipError_t e = hipMemcpy(d_probe, probe.host, (size_t)W * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(d_wq, qw.host, (size_t)W * W * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(d_bq, qb.host, (size_t)W * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(d_wkv, kvw.host, (size_t)W * 2 * W * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = launch_map_fold_prepare(d_probe, d_wq, d_bq, d_wkv, W, m->heads, m->head_dim, d_q, m->map_q, m->u_hi,
                                m->u_lo, m->wv, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipFree(tmp);
  hip_check(e, "MAP fold constants");
}

// The activation buffers of the images [b0, ...) of a call: every buffer is
// image-major, so a half-batch works on row (or image) ranges of the same
// workspace.
struct Acts {
  void* xp;
  f16* h;
  void* a;
  f16* qkv;
  void* o;
  void* u;
  void* mo;
  f16* my;
  void* ma;
  void* mu;
  void* vt;  // F16, or e4m3 codes with the e4m3 PV product
  float* mscores;
  float* zbar;
  float* lnst;
};

Acts acts_at(const siglip_model* m, int b0) {
  const int64_t r0 = (int64_t)b0 * m->tokens;  // first token row
  const int64_t W = m->width, es = m->esz();
  auto at = [](void* p, int64_t bytes) -> void* { return p ? static_cast<uint8_t*>(p) + bytes : nullptr; };
  Acts A;
  A.xp = at(m->xp, r0 * m->patch_pad * es);
  A.h = m->h + r0 * W;
  A.a = at(m->a, r0 * W * es);
  A.qkv = m->qkv + r0 * 3 * W;
  A.o = at(m->o, r0 * W * es);
  A.u = at(m->u, r0 * m->mlp_pad * es);
  A.mo = at(m->mo, b0 * W * es);
  A.my = m->my + b0 * W;
  A.ma = at(m->ma, b0 * W * es);
  A.mu = at(m->mu, b0 * m->mlp_pad * es);
  A.vt = at(m->vt, (int64_t)b0 * W * m->tokens_pad * (m->attn_fp8 ? 1 : 2));
  A.mscores = m->mscores ? m->mscores + r0 * 16 : nullptr;
  A.zbar = m->zbar ? m->zbar + (int64_t)b0 * 16 * W : nullptr;
  A.lnst = m->lnst ? m->lnst + r0 * 2 : nullptr;
  return A;
}

// A LayerNorm folded into a GEMM's A operand: the rows' statistics and the
// LayerNorm's affine parameters (a is then the F16 residual)
struct LnFold {
  const float* stats;
  const float* gamma;
  const float* beta;
  float scale;
};

void set_ln(GemmArgs& args, const LnFold* ln) {
  if (!ln) return;
  args.ln_stats = ln->stats;
  args.ln_gamma = ln->gamma;
  args.ln_beta = ln->beta;
  args.ln_scale = ln->scale;
}

void gemm(siglip_model* m, const Gemm& g, const void* a, int64_t lda, int M, void* c, int64_t ldc, int epi,
          bool out_fp8, const f16* res, int64_t ldres, hipStream_t s, const LnFold* ln = nullptr) {
  GemmArgs args{};
  args.a = a;
  args.lda = lda;
  args.w = g.w;
  args.ldw = g.n_pad;  // rows per 64-byte K panel
  args.c = c;
  args.ldc = ldc;
  args.bias = g.bias;
  args.pos = m->pos;
  args.pos_rows = m->tokens;
  args.ldpos = m->width;
  args.res = res;
  args.ldres = ldres;
  args.M = M;
  args.N = g.n_pad;
  args.K = g.k_pad;
  args.acc_scale = m->acc_scale;
  args.out_scale = m->op_scale;
  set_ln(args, ln);
  hip_check(launch_gemm(args, epi, m->fp8, out_fp8, s), "gemm launch");
}

// QKV-epilogue arguments of one projection whose columns from vt_col0 on are
// V (written transposed into vt) and whose columns before it are Q and/or K
// (written into c, or as e4m3 codes into head slots of the QKV buffer's bytes
// from qk8 on when the QK product is e4m3).
GemmArgs qkv_args(siglip_model* m, const Gemm& g, const void* a, f16* c, void* vt, int vt_col0, uint8_t* qk8,
                  int M, const LnFold* ln) {
  GemmArgs args{};
  args.a = a;
  args.lda = m->width;
  args.w = g.w;
  args.ldw = g.n_pad;  // rows per 64-byte K panel
  args.c = c;
  args.ldc = 3 * m->width;
  args.bias = g.bias;
  args.M = M;
  args.N = g.n_pad;
  args.K = g.k_pad;
  args.acc_scale = m->acc_scale;
  args.out_scale = m->attn_fp8 ? m->attn_v_scale : m->op_scale;
  args.vt = static_cast<f16*>(vt);
  args.vt_col0 = vt_col0;
  args.vt_tokens = m->tokens;
  args.vt_heads = (g.n_pad - vt_col0) / m->head_dim;
  args.vt_dim = m->head_dim;
  args.vt_ld = m->tokens_pad;
  args.vt_inv_dim = 1.0f / (float)m->head_dim;
  if (m->attn_qk8) {
    args.qk8 = qk8;
    args.qk8_ld = 6LL * m->width;  // bytes of one F16 row of the QKV buffer
    args.qk8_pitch = kQK8SlotBytes;
    args.qk8_scale = m->attn_v_scale;
  }
  set_ln(args, ln);
  return args;
}

// The fused QKV projection: Q and K row-major into qkv (or as e4m3 codes in
// its bytes), V transposed per head into vt when the streaming attention is
// used.
void gemm_qkv(siglip_model* m, const Layer& Ly, const void* a, f16* qkv, void* vt, int M, hipStream_t s,
              const LnFold* ln, bool vrow) {
  const Gemm& g = Ly.qkv;
  const int W = m->width;
  uint8_t* qk8 = reinterpret_cast<uint8_t*>(qkv);
  if (m->separate_qkv) {
    // Q and K into their columns of the fused row (or their e4m3 head slots);
    // V as its own projection, transposed per head (all its columns are V)
    if (m->attn_qk8) {
      hip_check(launch_gemm(qkv_args(m, Ly.q, a, qkv, vt, W, qk8, M, ln), EPI_QKV8, m->fp8, m->attn_fp8, s),
                "q gemm launch");
      hip_check(launch_gemm(qkv_args(m, Ly.k, a, qkv + W, vt, W, qk8 + (int64_t)m->heads * kQK8SlotBytes, M, ln),
                            EPI_QKV8, m->fp8, m->attn_fp8, s),
                "k gemm launch");
    } else {
      gemm(m, Ly.q, a, W, M, qkv, 3 * W, EPI_BIAS, false, nullptr, 0, s, ln);
      gemm(m, Ly.k, a, W, M, qkv + W, 3 * W, EPI_BIAS, false, nullptr, 0, s, ln);
    }
    if (!m->vt_path || vrow) {
      gemm(m, Ly.v, a, W, M, qkv + 2 * W, 3 * W, EPI_BIAS, false, nullptr, 0, s, ln);
      return;
    }
    // c is not written: every column goes to vt
    hip_check(launch_gemm(qkv_args(m, Ly.v, a, qkv + 2 * W, vt, 0, nullptr, M, ln), EPI_QKV, m->fp8, m->attn_fp8, s),
              "v gemm launch");
    return;
  }
  if (!m->vt_path || vrow) {
    gemm(m, g, a, W, M, qkv, 3 * W, EPI_BIAS, false, nullptr, 0, s, ln);
    return;
  }
  GemmArgs args = qkv_args(m, g, a, qkv, vt, 2 * W, qk8, M, ln);
  // 3456-wide weight (4 MB e4m3, 8 MB F16) exceeds an XCD's L2 next to the
  // activations: walk tiles in bands of 8 row blocks (measured ~12% faster
  // at 46,656 rows than row-block-major order)
  args.group_m = 8;
  hip_check(launch_gemm(args, m->attn_qk8 ? EPI_QKV8 : EPI_QKV, m->fp8, m->attn_fp8, s), "qkv gemm launch");
}

void capture(siglip_model* m, int stage, const void* src, size_t bytes, hipStream_t s) {
  if (m->capture_layer < 0 || !m->cap[stage]) return;
  hip_check(hipMemcpyAsync(m->cap[stage], src, bytes, hipMemcpyDeviceToDevice, s), "capture copy");
}

// Whether a call of `batch` images reads V row-major: with F16 attention
// products, when the attention grid is one round (the 16-query kernel). V
// then stays in the QKV rows and no V^T is written; larger grids run faster
// on V^T (the 32-query kernel's transposing V reads cost more than the V^T
// stores save). Both give the same bits.
bool vrow_call(const siglip_model* m, int batch) {
  return m->vrow_ok && (int64_t)((m->tokens + 127) / 128) * m->heads * batch <= 256;
}

void stage_shape(const siglip_model* m, int stage, int batch, int64_t* rows, int64_t* cols, int64_t* ld,
                 int32_t* eb) {
  const int64_t M = (int64_t)batch * m->tokens;
  const int e = m->esz();
  int64_t r = M, c = m->width, l = m->width;
  int32_t b = 2;
  switch (stage) {
    case SIGLIP_STAGE_EMBED: case SIGLIP_STAGE_H_ATTN: case SIGLIP_STAGE_H_OUT: break;
    case SIGLIP_STAGE_LN1: case SIGLIP_STAGE_ATTN: case SIGLIP_STAGE_LN2: b = e; break;
    case SIGLIP_STAGE_FINAL_LN: b = m->map_fold ? 2 : e; break;
    case SIGLIP_STAGE_QKV:
      if (m->attn_qk8) {  // e4m3 Q then K head slots, in the bytes of the F16 rows
        l = 6LL * m->width;
        c = 2LL * m->heads * kQK8SlotBytes;
        b = 1;
      } else {
        l = 3LL * m->width;
        c = m->vt_path && !vrow_call(m, batch) ? 2LL * m->width : l;
      }
      break;
    case SIGLIP_STAGE_V_T:
      r = m->vt_path && !vrow_call(m, batch) ? (int64_t)batch * m->heads * m->head_dim : 0;
      c = m->tokens;
      l = m->tokens_pad;
      b = m->attn_fp8 ? 1 : 2;
      break;
    case SIGLIP_STAGE_MLP_HIDDEN: c = m->mlp; l = m->mlp_pad; b = e; break;
    case SIGLIP_STAGE_MAP_KV: c = l = 2LL * m->width; r = m->map_fold ? 0 : M; break;
    case SIGLIP_STAGE_MAP_ATTN: case SIGLIP_STAGE_MAP_LN: r = batch; b = e; break;
    case SIGLIP_STAGE_MAP_Y: r = batch; break;
    case SIGLIP_STAGE_MAP_HIDDEN: r = batch; c = m->mlp; l = m->mlp_pad; b = e; break;
    case SIGLIP_STAGE_MAP_Q: r = 1; break;
  }
  if (rows) *rows = r;
  if (cols) *cols = c;
  if (ld) *ld = l;
  if (eb) *eb = b;
}

// Brackets one launch with a pair of events when timing is on.
class LaunchTimer {
 public:
  LaunchTimer(siglip_model* m, int kclass, hipStream_t s)
      : m_(m), s_(s), on_(((m->timing_mask >> kclass) & 1u) != 0) {
    if (!on_) return;
    if (m_->ev_used * 2 + 2 > m_->ev_pool.size()) {
      for (int i = 0; i < 2; ++i) {
        hipEvent_t e;
        hip_check(hipEventCreate(&e), "hipEventCreate");
        m_->ev_pool.push_back(e);
      }
      m_->ev_class.push_back(kclass);
    }
    pair_ = m_->ev_used++;
    m_->ev_class[pair_] = kclass;
    hip_check(hipEventRecord(m_->ev_pool[2 * pair_], s_), "hipEventRecord");
  }
  ~LaunchTimer() {
    // never throws: a failed record only loses this sample (the launch
    // itself reports its own error)
    if (on_ && hipEventRecord(m_->ev_pool[2 * pair_ + 1], s_) != hipSuccess) m_->timing_lost = true;
  }

 private:
  siglip_model* m_;
  hipStream_t s_;
  bool on_;
  size_t pair_ = 0;
};

void encode_part(siglip_model* m, const Acts& A, const f16* x, int B, f16* out, hipStream_t s, bool vrow) {
  const int M = B * m->tokens;
  const int W = m->width;
  const int e = m->esz();
  const bool q8 = m->fp8;
  const bool cap = m->capture_layer >= 0;
  auto cb = [&](int stage) {
    int64_t r, c, l;
    int32_t b;
    stage_shape(m, stage, B, &r, &c, &l, &b);
    return (size_t)(r * l * b);
  };

  {
    LaunchTimer lt(m, SIGLIP_K_INPUT, s);
    hip_check(launch_pad_convert(x, m->patch_dim, A.xp, M, m->patch_dim, m->patch_pad, q8, q8 ? m->op_scale : 1.0f, s),
              "pad_convert");
  }
  {
    LaunchTimer lt(m, SIGLIP_K_EMBED, s);
    gemm(m, m->embed, A.xp, m->patch_pad, M, A.h, W, EPI_BIAS_POS, false, nullptr, 0, s);
  }
  if (m->vt_path && !vrow && m->tokens_pad > m->tokens) {
    // V^T columns past the last token are read by the last key block: zeros
    LaunchTimer lt(m, SIGLIP_K_INPUT, s);
    const int64_t vrows = (int64_t)B * m->heads * m->head_dim;
    if (m->attn_fp8)
      hip_check(launch_zero_cols_u8(static_cast<uint8_t*>(A.vt), vrows, m->tokens_pad, m->tokens, m->tokens_pad, s),
                "zero V^T tail");
    else
      hip_check(launch_zero_cols(static_cast<f16*>(A.vt), vrows, m->tokens_pad, m->tokens, m->tokens_pad, s),
                "zero V^T tail");
  }
  if (cap) capture(m, SIGLIP_STAGE_EMBED, A.h, cb(SIGLIP_STAGE_EMBED), s);

  const float attn_scale = 1.0f / std::sqrt((float)m->head_dim);
  for (int i = 0; i < m->layers; ++i) {
    const Layer& Ly = m->L[i];
    const bool ci = cap && i == m->capture_layer;
    // LayerNorm 1: its output operand, or (folded) the row statistics the
    // QKV GEMM normalizes the residual rows with
    const LnFold ln1{A.lnst, Ly.ln1_g, Ly.ln1_b, q8 ? m->op_scale : 1.0f};
    {
      LaunchTimer lt(m, SIGLIP_K_LAYERNORM, s);
      if (m->ln_fold)
        hip_check(launch_layernorm_stats(A.h, W, A.lnst, M, W, 1e-6f, ln1.scale, s), "ln1 statistics");
      else
        hip_check(launch_layernorm(A.h, W, A.a, W, Ly.ln1_g, Ly.ln1_b, M, W, 1e-6f, q8, m->op_scale, s), "ln1");
    }
    if (ci && !m->ln_fold) capture(m, SIGLIP_STAGE_LN1, A.a, cb(SIGLIP_STAGE_LN1), s);
    {
      LaunchTimer lt(m, SIGLIP_K_QKV, s);
      if (m->ln_fold)
        gemm_qkv(m, Ly, A.h, A.qkv, A.vt, M, s, &ln1, vrow);
      else
        gemm_qkv(m, Ly, A.a, A.qkv, A.vt, M, s, nullptr, vrow);
    }
    if (ci) capture(m, SIGLIP_STAGE_QKV, A.qkv, cb(SIGLIP_STAGE_QKV), s);
    if (ci && m->vt_path && !vrow) capture(m, SIGLIP_STAGE_V_T, A.vt, cb(SIGLIP_STAGE_V_T), s);
    {
      LaunchTimer lt(m, SIGLIP_K_ATTENTION, s);
      // Q and K: F16 columns of the QKV rows, or e4m3 head slots in their bytes
      const uint8_t* qb8 = reinterpret_cast<const uint8_t*>(A.qkv);
      const void* aq = m->attn_qk8 ? static_cast<const void*>(qb8) : A.qkv;
      const void* ak = m->attn_qk8 ? static_cast<const void*>(qb8 + (int64_t)m->heads * kQK8SlotBytes)
                                   : static_cast<const void*>(A.qkv + W);
      const int64_t ald = m->attn_qk8 ? 6LL * W : 3LL * W;
      const int apitch = m->attn_qk8 ? kQK8SlotBytes : 0;
      if (m->attn_fp8)
        hip_check(launch_flash_attention_vt8(aq, ak, ald, apitch, static_cast<const uint8_t*>(A.vt), m->tokens_pad,
                                             A.o, W, B, m->heads, m->tokens, m->head_dim, attn_scale, q8,
                                             m->op_scale, m->attn_v_scale, s),
                  "attention");
      else if (vrow)
        hip_check(launch_flash_attention_vrow(A.qkv, A.qkv + W, A.qkv + 2 * W, 3 * W, A.o, W, B, m->heads, m->tokens,
                                              m->head_dim, attn_scale, q8, m->op_scale, s),
                  "attention");
      else if (m->vt_path)
        hip_check(launch_flash_attention_vt(aq, ak, ald, apitch, static_cast<const f16*>(A.vt), m->tokens_pad,
                                            A.o, W, B, m->heads, m->tokens, m->head_dim, attn_scale, q8,
                                            m->op_scale, s),
                  "attention");
      else
        hip_check(launch_flash_attention(A.qkv, A.qkv + W, A.qkv + 2 * W, 3 * W, A.o, W, B, m->heads, m->tokens,
                                         m->head_dim, attn_scale, q8, m->op_scale, s),
                  "attention");
    }
    if (ci) capture(m, SIGLIP_STAGE_ATTN, A.o, cb(SIGLIP_STAGE_ATTN), s);
    {
      LaunchTimer lt(m, SIGLIP_K_OUT_PROJ, s);
      gemm(m, Ly.out, A.o, W, M, A.h, W, EPI_BIAS_RES, false, A.h, W, s);
    }
    if (ci) capture(m, SIGLIP_STAGE_H_ATTN, A.h, cb(SIGLIP_STAGE_H_ATTN), s);
    const LnFold ln2{A.lnst, Ly.ln2_g, Ly.ln2_b, q8 ? m->op_scale : 1.0f};
    {
      LaunchTimer lt(m, SIGLIP_K_LAYERNORM, s);
      if (m->ln_fold)
        hip_check(launch_layernorm_stats(A.h, W, A.lnst, M, W, 1e-6f, ln2.scale, s), "ln2 statistics");
      else
        hip_check(launch_layernorm(A.h, W, A.a, W, Ly.ln2_g, Ly.ln2_b, M, W, 1e-6f, q8, m->op_scale, s), "ln2");
    }
    if (ci && !m->ln_fold) capture(m, SIGLIP_STAGE_LN2, A.a, cb(SIGLIP_STAGE_LN2), s);
    {
      LaunchTimer lt(m, SIGLIP_K_MLP_UP, s);
      if (m->ln_fold)
        gemm(m, Ly.mlp1, A.h, W, M, A.u, m->mlp_pad, EPI_BIAS_GELU, q8, nullptr, 0, s, &ln2);
      else
        gemm(m, Ly.mlp1, A.a, W, M, A.u, m->mlp_pad, EPI_BIAS_GELU, q8, nullptr, 0, s);
    }
    if (ci) capture(m, SIGLIP_STAGE_MLP_HIDDEN, A.u, cb(SIGLIP_STAGE_MLP_HIDDEN), s);
    {
      LaunchTimer lt(m, SIGLIP_K_MLP_DOWN, s);
      gemm(m, Ly.mlp2, A.u, m->mlp_pad, M, A.h, W, EPI_BIAS_RES, false, A.h, W, s);
    }
    if (ci) capture(m, SIGLIP_STAGE_H_OUT, A.h, cb(SIGLIP_STAGE_H_OUT), s);
  }

  if (m->map_fold) {
    // Z in F16 (the QKV buffer is free now), then the folded MAP attention
    f16* z = A.qkv;
    {
      LaunchTimer lt(m, SIGLIP_K_LAYERNORM, s);
      hip_check(launch_layernorm(A.h, W, z, W, m->lnf_g, m->lnf_b, M, W, 1e-6f, false, 1.0f, s), "final ln");
    }
    if (cap) capture(m, SIGLIP_STAGE_FINAL_LN, z, cb(SIGLIP_STAGE_FINAL_LN), s);
    {
      LaunchTimer lt(m, SIGLIP_K_MAP_KV, s);
      hip_check(launch_map_fold(z, W, m->u_hi, m->u_lo, m->wv, m->bv, A.mscores, A.zbar, B, m->tokens, m->heads,
                                m->head_dim, W, attn_scale, q8, m->op_scale, A.mo, W, s, 0),
                "map scores");
    }
    {
      LaunchTimer lt(m, SIGLIP_K_MAP_ATTENTION, s);
      hip_check(launch_map_fold(z, W, m->u_hi, m->u_lo, m->wv, m->bv, A.mscores, A.zbar, B, m->tokens, m->heads,
                                m->head_dim, W, attn_scale, q8, m->op_scale, A.mo, W, s, 1),
                "map pool");
    }
  } else {
  {
    LaunchTimer lt(m, SIGLIP_K_LAYERNORM, s);
    hip_check(launch_layernorm(A.h, W, A.a, W, m->lnf_g, m->lnf_b, M, W, 1e-6f, q8, m->op_scale, s), "final ln");
  }
  if (cap) capture(m, SIGLIP_STAGE_FINAL_LN, A.a, cb(SIGLIP_STAGE_FINAL_LN), s);
  f16* kv = A.qkv;  // [M, 2W]
  {
    LaunchTimer lt(m, SIGLIP_K_MAP_KV, s);
    if (m->separate_qkv) {
      gemm(m, m->mk, A.a, W, M, kv, 2 * W, EPI_BIAS, false, nullptr, 0, s);
      gemm(m, m->mv, A.a, W, M, kv + W, 2 * W, EPI_BIAS, false, nullptr, 0, s);
    } else {
      gemm(m, m->mkv, A.a, W, M, kv, 2 * W, EPI_BIAS, false, nullptr, 0, s);
    }
  }
  if (cap) capture(m, SIGLIP_STAGE_MAP_KV, kv, cb(SIGLIP_STAGE_MAP_KV), s);
  {
    LaunchTimer lt(m, SIGLIP_K_MAP_ATTENTION, s);
    hip_check(launch_map_attention(m->map_q, kv, 2 * W, W, A.mo, W, B, m->heads, m->tokens, m->head_dim, attn_scale,
                                   q8, m->op_scale, s),
              "map attention");
  }
  }
  if (cap) capture(m, SIGLIP_STAGE_MAP_ATTN, A.mo, cb(SIGLIP_STAGE_MAP_ATTN), s);
  {
    LaunchTimer lt(m, SIGLIP_K_MAP_TAIL, s);
    gemm(m, m->mout, A.mo, W, B, A.my, W, EPI_BIAS, false, nullptr, 0, s);
  }
  if (cap) capture(m, SIGLIP_STAGE_MAP_Y, A.my, cb(SIGLIP_STAGE_MAP_Y), s);
  {
    LaunchTimer lt(m, SIGLIP_K_LAYERNORM, s);
    hip_check(launch_layernorm(A.my, W, A.ma, W, m->mln_g, m->mln_b, B, W, 1e-6f, q8, m->op_scale, s), "map ln");
  }
  if (cap) capture(m, SIGLIP_STAGE_MAP_LN, A.ma, cb(SIGLIP_STAGE_MAP_LN), s);
  {
    LaunchTimer lt(m, SIGLIP_K_MAP_TAIL, s);
    gemm(m, m->mmlp1, A.ma, W, B, A.mu, m->mlp_pad, EPI_BIAS_GELU, q8, nullptr, 0, s);
  }
  if (cap) capture(m, SIGLIP_STAGE_MAP_HIDDEN, A.mu, cb(SIGLIP_STAGE_MAP_HIDDEN), s);
  {
    LaunchTimer lt(m, SIGLIP_K_MAP_TAIL, s);
    gemm(m, m->mmlp2, A.mu, m->mlp_pad, B, out, W, EPI_BIAS_RES, false, A.my, W, s);
  }
  if (cap) {
    m->captured = true;
    m->captured_batch = B;
  }
}

// One call: the whole batch on the caller's stream, or (batches of two or
// more, no stage capture or launch timing) the first half there and the
// second half on the side stream, forked from and joined back into the
// caller's stream. The halves share no buffer rows, and the kernels of one
// can fill the CUs the other leaves idle (the last partial wave of a GEMM's
// tiles, an attention or LayerNorm phase next to a GEMM).
void encode_impl(siglip_model* m, const f16* x, int B, f16* out, hipStream_t s) {
  const bool split = B >= 2 && m->side && m->capture_layer < 0 && m->timing_mask == 0;
  // V row-major in the QKV rows (no V^T) and the key-split attention: chosen
  // for the whole call, so both halves run the attention form of the
  // one-stream run
  const bool vrow = vrow_call(m, B);
  if (!split) {
    encode_part(m, acts_at(m, 0), x, B, out, s, vrow);
    return;
  }
  const int B0 = (B + 1) / 2;
  hip_check(hipEventRecord(m->fork_ev, s), "fork record");
  hip_check(hipStreamWaitEvent(m->side, m->fork_ev, 0), "fork wait");
  encode_part(m, acts_at(m, 0), x, B0, out, s, vrow);
  encode_part(m, acts_at(m, B0), x + (int64_t)B0 * m->tokens * m->patch_dim, B - B0, out + (int64_t)B0 * m->width,
              m->side, vrow);
  hip_check(hipEventRecord(m->join_ev, m->side), "join record");
  hip_check(hipStreamWaitEvent(s, m->join_ev, 0), "join wait");
}

int validate_header(const BlobHeader& h, size_t blob_bytes, std::string* why) {
  if (std::memcmp(h.magic, "SGLP", 4) != 0) return (*why = "bad magic (expected \"SGLP\")", SIGLIP_E_BAD_BLOB);
  if (h.version != 1) return (*why = "unsupported blob version " + std::to_string(h.version), SIGLIP_E_BAD_BLOB);
  if (h.dtype != 0) return (*why = "unsupported blob dtype (only 0 = F32)", SIGLIP_E_BAD_BLOB);
  if (h.width == 0 || h.depth == 0 || h.heads == 0 || h.head_dim == 0 || h.mlp == 0 || h.tokens == 0 ||
      h.patch_dim == 0)
    return (*why = "zero dimension in blob header", SIGLIP_E_BAD_BLOB);
  if (h.width > 16384 || h.depth > 1024 || h.mlp > 65536 || h.tokens > 65536 || h.patch_dim > 65536)
    return (*why = "implausible dimension in blob header", SIGLIP_E_BAD_BLOB);
  if ((uint64_t)h.heads * h.head_dim != h.width)
    return (*why = "width != heads * head_dim", SIGLIP_E_BAD_BLOB);
  if (h.total_bytes != blob_bytes)
    return (*why = "blob size " + std::to_string(blob_bytes) + " != header total_bytes " +
                   std::to_string(h.total_bytes), SIGLIP_E_BAD_BLOB);
  return SIGLIP_OK;
}

int check_supported(const BlobHeader& h, std::string* why) {
  // activation rows are GEMM operands read in whole 128-element K slices
  if (h.width % 128) return (*why = "width must be a multiple of 128", SIGLIP_E_UNSUPPORTED);
  if (h.width > 2048) return (*why = "width above 2048", SIGLIP_E_UNSUPPORTED);
  if (h.head_dim % 8 || h.head_dim > 80) return (*why = "head_dim must be a multiple of 8 and <= 80", SIGLIP_E_UNSUPPORTED);
  if (h.mlp % 8) return (*why = "mlp must be a multiple of 8", SIGLIP_E_UNSUPPORTED);
  if (h.patch_dim % 4) return (*why = "patch_dim must be a multiple of 4", SIGLIP_E_UNSUPPORTED);
  if (h.tokens > 4096) return (*why = "more than 4096 tokens", SIGLIP_E_UNSUPPORTED);
  return SIGLIP_OK;
}

int create_impl(const void* blob, size_t blob_bytes, const siglip_options* opt, siglip_model** out) {
  if (!out) return fail(SIGLIP_E_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (!blob || !opt) return fail(SIGLIP_E_INVALID_ARG, "blob or opt is NULL");
  if (opt->max_batch < 1 || opt->max_batch > 4096) return fail(SIGLIP_E_INVALID_ARG, "max_batch must be 1..4096");
  if (opt->gemm_precision != 0 && opt->gemm_precision != 1)
    return fail(SIGLIP_E_INVALID_ARG, "gemm_precision must be 0 (F16) or 1 (FP8)");
  if (opt->gemm_precision == 1 && (opt->fp8_scale_exp < -8 || opt->fp8_scale_exp > 8))
    return fail(SIGLIP_E_INVALID_ARG, "fp8_scale_exp must be in -8..8");
  if (opt->separate_qkv != 0 && opt->separate_qkv != 1)
    return fail(SIGLIP_E_INVALID_ARG, "separate_qkv must be 0 or 1");
  if (opt->map_explicit_kv != 0 && opt->map_explicit_kv != 1)
    return fail(SIGLIP_E_INVALID_ARG, "map_explicit_kv must be 0 or 1");
  if (opt->attention_fp8 < 0 || opt->attention_fp8 > 3)
    return fail(SIGLIP_E_INVALID_ARG, "attention_fp8 must be 0..3 (bit 0: PV product, bit 1: QK product)");
  if (opt->attention_fp8 != 0 && (opt->fp8_scale_exp < -8 || opt->fp8_scale_exp > 8))
    return fail(SIGLIP_E_INVALID_ARG, "fp8_scale_exp must be in -8..8");
  if (opt->layernorm_fold != 0 && opt->layernorm_fold != 1)
    return fail(SIGLIP_E_INVALID_ARG, "layernorm_fold must be 0 or 1");
  if (blob_bytes < sizeof(BlobHeader)) return fail(SIGLIP_E_BAD_BLOB, "blob shorter than its 64-byte header");
  BlobHeader h;
  std::memcpy(&h, blob, sizeof h);
  std::string why;
  int st = validate_header(h, blob_bytes, &why);
  if (st != SIGLIP_OK) return fail(st, why);
  if (opt->layers < 0 || (uint32_t)opt->layers > h.depth)
    return fail(SIGLIP_E_INVALID_ARG, "layers must be 0 (all) or 1..depth");
  st = check_supported(h, &why);
  if (st != SIGLIP_OK) return fail(st, why);
  if (opt->layernorm_fold == 1 && h.width != 1152)
    return fail(SIGLIP_E_UNSUPPORTED, "layernorm_fold needs width 1152 (the statistics kernel's row layout)");

  // Walk the whole blob once on the CPU before touching the GPU.
  const int W = (int)h.width, F = (int)h.mlp, T = (int)h.tokens, P = (int)h.patch_dim;
  BlobReader rd(static_cast<const uint8_t*>(blob), blob_bytes);
  struct LayerRefs {
    TensorRef ln1g, ln1b, qkvw, qkvb, outw, outb, ln2g, ln2b, m1w, m1b, m2w, m2b;
  };
  std::vector<LayerRefs> lr;
  TensorRef ew, eb, pos, lfg, lfb, probe, qw, qb, kvw, kvb, ow, ob, mlg, mlb, m1w, m1b, m2w, m2b;
  try {
    ew = rd.next("embed.w", P, W);
    eb = rd.next("embed.b", 1, W);
    pos = rd.next("pos", T, W);
    for (uint32_t i = 0; i < h.depth; ++i) {
      LayerRefs r;
      r.ln1g = rd.next("ln1.g", 1, W);
      r.ln1b = rd.next("ln1.b", 1, W);
      r.qkvw = rd.next("qkv.w", W, 3 * W);
      r.qkvb = rd.next("qkv.b", 1, 3 * W);
      r.outw = rd.next("out.w", W, W);
      r.outb = rd.next("out.b", 1, W);
      r.ln2g = rd.next("ln2.g", 1, W);
      r.ln2b = rd.next("ln2.b", 1, W);
      r.m1w = rd.next("mlp1.w", W, F);
      r.m1b = rd.next("mlp1.b", 1, F);
      r.m2w = rd.next("mlp2.w", F, W);
      r.m2b = rd.next("mlp2.b", 1, W);
      lr.push_back(r);
    }
    lfg = rd.next("final_ln.g", 1, W);
    lfb = rd.next("final_ln.b", 1, W);
    probe = rd.next("map.probe", 1, W);
    qw = rd.next("map.q.w", W, W);
    qb = rd.next("map.q.b", 1, W);
    kvw = rd.next("map.kv.w", W, 2 * W);
    kvb = rd.next("map.kv.b", 1, 2 * W);
    ow = rd.next("map.out.w", W, W);
    ob = rd.next("map.out.b", 1, W);
    mlg = rd.next("map.ln.g", 1, W);
    mlb = rd.next("map.ln.b", 1, W);
    m1w = rd.next("map.mlp1.w", W, F);
    m1b = rd.next("map.mlp1.b", 1, F);
    m2w = rd.next("map.mlp2.w", F, W);
    m2b = rd.next("map.mlp2.b", 1, W);
  } catch (const BadBlob& b) {
    return fail(SIGLIP_E_BAD_BLOB, b.msg);
  }
  if (rd.end() != blob_bytes) return fail(SIGLIP_E_BAD_BLOB, "blob has trailing bytes beyond its last tensor");

  // Device checks.
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SIGLIP_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(SIGLIP_E_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(SIGLIP_E_UNSUPPORTED, std::string("device is ") + prop.gcnArchName + ", the library is built for gfx950 only");

  siglip_model* m = new (std::nothrow) siglip_model();
  if (!m) return fail(SIGLIP_E_OUT_OF_MEMORY, "host allocation failed");
  try {
    m->device = dev;
    m->width = W;
    m->depth = (int)h.depth;
    m->layers = opt->layers == 0 ? (int)h.depth : opt->layers;
    m->heads = (int)h.heads;
    m->head_dim = (int)h.head_dim;
    m->mlp = F;
    m->tokens = T;
    m->patch_dim = P;
    m->max_batch = opt->max_batch;
    m->fp8 = opt->gemm_precision == 1;
    m->scale_exp = m->fp8 ? opt->fp8_scale_exp : 0;
    m->op_scale = std::ldexp(1.0f, -m->scale_exp);
    m->acc_scale = std::ldexp(1.0f, 2 * m->scale_exp);
    m->patch_pad = (int)round_up(P, kKAlign);
    m->mlp_pad = (int)round_up(F, kNAlign);  // U is both an N (MLP up) and a K (MLP down) dimension
    m->tokens_pad = (int)round_up(T, 64);
    m->separate_qkv = opt->separate_qkv == 1;
    m->ln_fold = opt->layernorm_fold == 1;
    m->attn_fp8 = (opt->attention_fp8 & 1) != 0;
    m->attn_qk8 = (opt->attention_fp8 & 2) != 0;
    // The streaming attention kernels take head widths 64, 72 and 80: with F16
    // products they read V in the QKV rows; the e4m3 forms read V^T, which
    // the QKV GEMM then writes.
    const bool streaming = flash_attention_vt_supported(m->head_dim);
    if ((m->attn_fp8 || m->attn_qk8) && !streaming) {
      delete m;
      return fail(SIGLIP_E_UNSUPPORTED, "attention_fp8 needs head_dim 64, 72 or 80");
    }
    m->vt_path = streaming;
    m->vrow_ok = streaming && !m->attn_fp8 && !m->attn_qk8;
    m->attn_v_scale = std::ldexp(1.0f, -opt->fp8_scale_exp);
    m->map_fold = opt->map_explicit_kv == 0 && map_fold_supported(W, m->heads, m->head_dim, T);

    const size_t staging_floats = (size_t)std::max<int64_t>({(int64_t)P * W, 3LL * W * W, (int64_t)W * F, (int64_t)T * W});
    float* staging = static_cast<float*>(m->dalloc(staging_floats * 4));

    m->embed = make_gemm(m, ew, eb, staging);
    m->pos = upload_f32(m, pos);
    for (int i = 0; i < m->layers; ++i) {
      const LayerRefs& r = lr[i];
      Layer Ly;
      Ly.ln1_g = upload_f32(m, r.ln1g);
      Ly.ln1_b = upload_f32(m, r.ln1b);
      Ly.ln2_g = upload_f32(m, r.ln2g);
      Ly.ln2_b = upload_f32(m, r.ln2b);
      if (m->separate_qkv) {
        Ly.q = make_gemm_block(m, r.qkvw, r.qkvb, 0, W, staging);
        Ly.k = make_gemm_block(m, r.qkvw, r.qkvb, W, W, staging);
        Ly.v = make_gemm_block(m, r.qkvw, r.qkvb, 2 * W, W, staging);
      } else {
        Ly.qkv = make_gemm(m, r.qkvw, r.qkvb, staging);
      }
      Ly.out = make_gemm(m, r.outw, r.outb, staging);
      Ly.mlp1 = make_gemm(m, r.m1w, r.m1b, staging);
      Ly.mlp2 = make_gemm(m, r.m2w, r.m2b, staging);
      m->L.push_back(Ly);
    }
    m->lnf_g = upload_f32(m, lfg);
    m->lnf_b = upload_f32(m, lfb);
    if (m->map_fold) {
      make_map_fold(m, probe, qw, qb, kvw, kvb);
    } else {
      m->mq = make_gemm(m, qw, qb, staging);
      if (m->separate_qkv) {
        m->mk = make_gemm_block(m, kvw, kvb, 0, W, staging);
        m->mv = make_gemm_block(m, kvw, kvb, W, W, staging);
      } else {
        m->mkv = make_gemm(m, kvw, kvb, staging);
      }
    }
    m->mout = make_gemm(m, ow, ob, staging);
    m->mmlp1 = make_gemm(m, m1w, m1b, staging);
    m->mmlp2 = make_gemm(m, m2w, m2b, staging);
    m->mln_g = upload_f32(m, mlg);
    m->mln_b = upload_f32(m, mlb);

    // workspace
    const int64_t M = (int64_t)m->max_batch * T;
    const int64_t B = m->max_batch;
    const int es = m->esz();
    struct Part { void** dst; int64_t bytes; };
    std::vector<Part> parts = {
        {&m->xp, M * m->patch_pad * es}, {(void**)&m->h, M * W * 2}, {&m->a, M * W * es},
        {(void**)&m->qkv, M * 3 * W * 2}, {&m->o, M * W * es}, {&m->u, M * m->mlp_pad * es},
        {&m->mo, B * W * es}, {(void**)&m->my, B * W * 2}, {&m->ma, B * W * es}, {&m->mu, B * m->mlp_pad * es},
        // V^T: F16, or e4m3 codes with the e4m3 PV product
        {(void**)&m->vt, m->vt_path ? B * W * m->tokens_pad * (m->attn_fp8 ? 1 : 2) : 0},
        {(void**)&m->mscores, m->map_fold ? M * 16 * 4 : 0},
        {(void**)&m->zbar, m->map_fold ? B * 16 * W * 4 : 0},
        {(void**)&m->lnst, m->ln_fold ? M * 2 * 4 : 0},
    };
    size_t total = 0;
    for (auto& p : parts) total += (size_t)round_up(p.bytes, 256);
    m->ws = m->dalloc(total);
    m->ws_bytes = total;
    size_t off = 0;
    for (auto& p : parts) {
      *p.dst = static_cast<uint8_t*>(m->ws) + off;
      off += (size_t)round_up(p.bytes, 256);
    }

    hip_check(hipStreamCreateWithFlags(&m->side, hipStreamNonBlocking), "hipStreamCreate");
    hip_check(hipEventCreateWithFlags(&m->fork_ev, hipEventDisableTiming), "hipEventCreate");
    hip_check(hipEventCreateWithFlags(&m->join_ev, hipEventDisableTiming), "hipEventCreate");

    // probe query, once: q = probe Wq + bq (same GEMM as every projection;
    // the folded path computed it with the fold constants)
    if (!m->map_fold) {
    void* probe_op = m->dalloc((size_t)m->mq.k_pad * es);
    hip_check(hipMemcpy(staging, probe.host, (size_t)W * 4, hipMemcpyHostToDevice), "hipMemcpy");
    hip_check(launch_f32_convert(staging, 1, W, probe_op, m->mq.k_pad, m->fp8, m->fp8 ? m->op_scale : 1.0f, nullptr),
              "probe convert");
    m->map_q = static_cast<f16*>(m->dalloc((size_t)m->mq.n_pad * 2));
    gemm(m, m->mq, probe_op, m->mq.k_pad, 1, m->map_q, m->mq.n_pad, EPI_BIAS, false, nullptr, 0, nullptr);
    }
    hip_check(hipDeviceSynchronize(), "create sync");
  } catch (const HipFail& f) {
    delete m;
    const int code = (f.err == hipErrorOutOfMemory || f.err == hipErrorMemoryAllocation) ? SIGLIP_E_OUT_OF_MEMORY
                                                                                           : SIGLIP_E_HIP;
    return fail(code, f.where + ": " + hipGetErrorString(f.err));
  } catch (const std::bad_alloc&) {
    delete m;
    return fail(SIGLIP_E_OUT_OF_MEMORY, "host allocation failed");
  }
  *out = m;
  return SIGLIP_OK;
}

// Library-owned V^T staging of siglip_attention, one buffer per device,
// grown on demand (the call that needs more than any before it allocates)
// and kept until the process ends.
std::mutex g_vt_mu;
constexpr int kMaxDevices = 64;
void* g_vt_buf[kMaxDevices] = {};
size_t g_vt_bytes[kMaxDevices] = {};

int vt_staging(size_t need, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SIGLIP_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SIGLIP_E_UNSUPPORTED, "device ordinal above 63");
  std::lock_guard<std::mutex> lock(g_vt_mu);
  if (g_vt_bytes[dev] < need) {
    if (g_vt_buf[dev]) (void)hipFree(g_vt_buf[dev]);
    g_vt_buf[dev] = nullptr;
    g_vt_bytes[dev] = 0;
    e = hipMalloc(&g_vt_buf[dev], need);
    if (e != hipSuccess) {
      g_vt_buf[dev] = nullptr;
      return fail(e == hipErrorOutOfMemory ? SIGLIP_E_OUT_OF_MEMORY : SIGLIP_E_HIP,
                  std::string("V^T staging: ") + hipGetErrorString(e));
    }
    g_vt_bytes[dev] = need;
  }
  *out = g_vt_buf[dev];
  return SIGLIP_OK;
}

// Scratch of siglip_attention_noalloc: a fixed device array, so that entry
// point allocates nothing. Every GPU the library runs on holds its own copy
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: host code uses only the per-device address that
// hipGetSymbolAddress returns (static_scratch below).
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
int static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SIGLIP_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SIGLIP_E_UNSUPPORTED, "device ordinal above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SIGLIP_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SIGLIP_OK;
}

// Standalone attention. Head widths the streaming kernel takes (64, 72, 80)
// run the encoder's own kernel: V is first transposed per image into V^T
// rows (zeros past the last token), in stage_buf (a device address of
// stage_bytes) when the caller supplies one, else in the library's staging
// buffer. Other head widths run the register-staged kernel, which needs no
// staging.
int attention_impl(const void* q, const void* k, const void* v, int64_t ld, void* o, int32_t batch, int32_t heads,
                   int32_t tokens, int32_t head_dim, float scale, void* hip_stream, void* stage_buf,
                   size_t stage_bytes) {
  if (!q || !k || !v || !o) return fail(SIGLIP_E_INVALID_ARG, "null q, k, v or o");
  if (batch < 1 || heads < 1 || tokens < 1 || batch > 65535 || heads > 65535)
    return fail(SIGLIP_E_INVALID_ARG, "batch, heads and tokens must be >= 1 (batch, heads <= 65535)");
  if (head_dim < 8 || head_dim > 80 || head_dim % 8)
    return fail(SIGLIP_E_UNSUPPORTED, "head_dim must be a multiple of 8 in 8..80");
  if (ld < (int64_t)heads * head_dim || ld % 8)
    return fail(SIGLIP_E_INVALID_ARG, "row_stride_elems must be >= heads*head_dim and a multiple of 8");
  for (const void* p : {q, k, v, (const void*)o})
    if (reinterpret_cast<uintptr_t>(p) & 15) return fail(SIGLIP_E_INVALID_ARG, "pointers must be 16-byte aligned");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(SIGLIP_E_INVALID_ARG, "scale must be finite and > 0");
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  const int64_t width = (int64_t)heads * head_dim;
  if (width > INT32_MAX) return fail(SIGLIP_E_INVALID_ARG, "heads*head_dim too large");
  hipError_t e;
  if (flash_attention_vt_supported(head_dim)) {
    const int64_t vt_ld = round_up(tokens, 64);
    const size_t need = (size_t)batch * (size_t)width * (size_t)vt_ld * 2;
    void* vt = stage_buf;
    if (!vt) {
      const int st = vt_staging(need, &vt);
      if (st != SIGLIP_OK) return st;
    } else if (need > stage_bytes) {
      return fail(SIGLIP_E_INVALID_ARG, "V^T staging needs " + std::to_string(need) + " bytes, the buffer holds " +
                                            std::to_string(stage_bytes));
    }
    e = launch_vt_transpose(static_cast<const f16*>(v), ld, batch, tokens, (int)width, static_cast<f16*>(vt), vt_ld,
                            s);
    if (e == hipSuccess)
      e = launch_flash_attention_vt(q, k, ld, 0, static_cast<const f16*>(vt), vt_ld, o, width, batch, heads, tokens,
                                    head_dim, scale, false, 1.0f, s);
  } else {
    e = launch_flash_attention(static_cast<const f16*>(q), static_cast<const f16*>(k), static_cast<const f16*>(v), ld,
                               o, width, batch, heads, tokens, head_dim, scale, false, 1.0f, s);
  }
  if (e != hipSuccess) return fail(SIGLIP_E_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  return SIGLIP_OK;
}

}  // namespace

extern "C" {

SIGLIP_API int siglip_create(const void* blob, size_t blob_bytes, const siglip_options* opt, siglip_model** out) {
  try {
    g_last_error.clear();
    return create_impl(blob, blob_bytes, opt, out);
  } catch (const std::exception& ex) {
    return fail(SIGLIP_E_HIP, std::string("unexpected: ") + ex.what());
  } catch (...) {
    return fail(SIGLIP_E_HIP, "unexpected exception");
  }
}

SIGLIP_API int siglip_encode(siglip_model* m, const void* pixels_f16, int32_t batch, void* out_f16, void* hip_stream) {
  if (!m || !pixels_f16 || !out_f16) return fail(SIGLIP_E_INVALID_ARG, "null model, input or output pointer");
  if (batch < 1 || batch > m->max_batch)
    return fail(SIGLIP_E_INVALID_ARG, "batch " + std::to_string(batch) + " outside 1..max_batch (" +
                                          std::to_string(m->max_batch) + ")");
  if ((reinterpret_cast<uintptr_t>(pixels_f16) & 7) || (reinterpret_cast<uintptr_t>(out_f16) & 15))
    return fail(SIGLIP_E_INVALID_ARG, "input must be 8-byte and output 16-byte aligned");
  try {
    encode_impl(m, static_cast<const f16*>(pixels_f16), batch, static_cast<f16*>(out_f16),
                static_cast<hipStream_t>(hip_stream));
  } catch (const HipFail& f) {
    return fail(SIGLIP_E_HIP, f.where + ": " + hipGetErrorString(f.err));
  } catch (...) {
    return fail(SIGLIP_E_HIP, "unexpected exception");
  }
  return SIGLIP_OK;
}

SIGLIP_API int siglip_attention(const void* q, const void* k, const void* v, int64_t row_stride_elems, void* o,
                                int32_t batch, int32_t heads, int32_t tokens, int32_t head_dim, float scale,
                                void* hip_stream) {
  return attention_impl(q, k, v, row_stride_elems, o, batch, heads, tokens, head_dim, scale, hip_stream, nullptr, 0);
}

SIGLIP_API int siglip_attention_noalloc(const void* q, const void* k, const void* v, int64_t row_stride_elems,
                                        void* o, int32_t batch, int32_t heads, int32_t tokens, int32_t head_dim,
                                        float scale, void* hip_stream) {
  // the same argument checks as siglip_attention come first, so a bad call
  // fails before the scratch is looked up
  if (!q || !k || !v || !o) return fail(SIGLIP_E_INVALID_ARG, "null q, k, v or o");
  if (batch < 1 || heads < 1 || tokens < 1 || batch > 65535 || heads > 65535)
    return fail(SIGLIP_E_INVALID_ARG, "batch, heads and tokens must be >= 1 (batch, heads <= 65535)");
  if (head_dim < 8 || head_dim > 80 || head_dim % 8)
    return fail(SIGLIP_E_UNSUPPORTED, "head_dim must be a multiple of 8 in 8..80");
  if (flash_attention_vt_supported(head_dim)) {
    const size_t need = (size_t)batch * (size_t)heads * head_dim * (size_t)round_up(tokens, 64) * 2;
    if (need > kStaticScratchBytes)
      return fail(SIGLIP_E_INVALID_ARG, "batch*heads*head_dim*round_up(tokens,64)*2 = " + std::to_string(need) +
                                            " bytes exceeds the 64 MiB static scratch of siglip_attention_noalloc");
  }
  void* p = nullptr;
  const int st = static_scratch(&p);
  if (st != SIGLIP_OK) return st;
  return attention_impl(q, k, v, row_stride_elems, o, batch, heads, tokens, head_dim, scale, hip_stream, p,
                        kStaticScratchBytes);
}

SIGLIP_API int siglip_destroy(siglip_model* m) {
  if (!m) return SIGLIP_OK;
  (void)hipDeviceSynchronize();
  delete m;
  return SIGLIP_OK;
}

SIGLIP_API const char* siglip_status_string(int status) {
  switch (status) {
    case SIGLIP_OK: return "SIGLIP_OK";
    case SIGLIP_E_INVALID_ARG: return "SIGLIP_E_INVALID_ARG";
    case SIGLIP_E_BAD_BLOB: return "SIGLIP_E_BAD_BLOB";
    case SIGLIP_E_UNSUPPORTED: return "SIGLIP_E_UNSUPPORTED";
    case SIGLIP_E_OUT_OF_MEMORY: return "SIGLIP_E_OUT_OF_MEMORY";
    case SIGLIP_E_HIP: return "SIGLIP_E_HIP";
  }
  return "SIGLIP_E_UNKNOWN";
}

SIGLIP_API const char* siglip_last_error(void) { return g_last_error.c_str(); }

SIGLIP_API int siglip_model_info(const siglip_model* m, int32_t* width, int32_t* layers, int32_t* heads,
                                 int32_t* head_dim, int32_t* mlp, int32_t* tokens, int32_t* patch_dim,
                                 int32_t* max_batch, int32_t* gemm_precision) {
  if (!m) return fail(SIGLIP_E_INVALID_ARG, "null model");
  if (width) *width = m->width;
  if (layers) *layers = m->layers;
  if (heads) *heads = m->heads;
  if (head_dim) *head_dim = m->head_dim;
  if (mlp) *mlp = m->mlp;
  if (tokens) *tokens = m->tokens;
  if (patch_dim) *patch_dim = m->patch_dim;
  if (max_batch) *max_batch = m->max_batch;
  if (gemm_precision) *gemm_precision = m->fp8 ? 1 : 0;
  return SIGLIP_OK;
}

#ifdef SIGLIP_TEST_HOOKS
SIGLIP_API int siglip_debug_capture(siglip_model* m, int32_t layer) {
  if (!m) return fail(SIGLIP_E_INVALID_ARG, "null model");
  if (layer >= m->layers) return fail(SIGLIP_E_INVALID_ARG, "capture layer beyond the model's layers");
  m->captured = false;
  if (layer < 0) {
    m->capture_layer = -1;
    return SIGLIP_OK;
  }
  try {
    for (int s = 0; s < SIGLIP_STAGE_COUNT; ++s) {
      if (m->cap[s]) continue;
      int64_t r, c, l;
      int32_t b;
      stage_shape(m, s, m->max_batch, &r, &c, &l, &b);
      m->cap_bytes[s] = (size_t)(r * l * b);
      m->cap[s] = m->dalloc(m->cap_bytes[s]);
    }
    // the probe query is computed at create time; snapshot it now
    hip_check(hipMemcpy(m->cap[SIGLIP_STAGE_MAP_Q], m->map_q, (size_t)m->width * 2, hipMemcpyDeviceToDevice),
              "capture map_q");
  } catch (const HipFail& f) {
    return fail(SIGLIP_E_OUT_OF_MEMORY, f.where + ": " + hipGetErrorString(f.err));
  }
  m->capture_layer = layer;
  return SIGLIP_OK;
}

SIGLIP_API int siglip_debug_stage_info(const siglip_model* m, int32_t stage, int64_t* rows, int64_t* cols,
                                       int64_t* ld, int32_t* elem_bytes) {
  if (!m || stage < 0 || stage >= SIGLIP_STAGE_COUNT) return fail(SIGLIP_E_INVALID_ARG, "bad model or stage");
  stage_shape(m, stage, m->captured ? m->captured_batch : m->max_batch, rows, cols, ld, elem_bytes);
  return SIGLIP_OK;
}

SIGLIP_API int siglip_debug_stage(const siglip_model* m, int32_t stage, void* dst, size_t dst_bytes) {
  if (!m || !dst || stage < 0 || stage >= SIGLIP_STAGE_COUNT) return fail(SIGLIP_E_INVALID_ARG, "bad arguments");
  if (!m->captured && stage != SIGLIP_STAGE_MAP_Q) return fail(SIGLIP_E_INVALID_ARG, "no capturing encode yet");
  if (!m->cap[stage]) return fail(SIGLIP_E_INVALID_ARG, "capture is off");
  int64_t r, c, l;
  int32_t b;
  stage_shape(m, stage, m->captured ? m->captured_batch : 1, &r, &c, &l, &b);
  const size_t n = (size_t)(r * l * b);
  if (dst_bytes < n) return fail(SIGLIP_E_INVALID_ARG, "dst too small: need " + std::to_string(n) + " bytes");
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(dst, m->cap[stage], n, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SIGLIP_E_HIP, std::string("stage copy: ") + hipGetErrorString(e));
  return SIGLIP_OK;
}

#endif  // SIGLIP_TEST_HOOKS

SIGLIP_API int siglip_debug_timing(siglip_model* m, uint32_t class_mask) {
  if (!m) return fail(SIGLIP_E_INVALID_ARG, "null model");
  if (class_mask >> SIGLIP_K_COUNT) return fail(SIGLIP_E_INVALID_ARG, "class_mask selects unknown classes");
  m->timing_mask = class_mask;
  m->ev_used = 0;
  m->timing_lost = false;
  for (int k = 0; k < SIGLIP_K_COUNT; ++k) {
    m->t_ms[k] = 0.0;
    m->t_n[k] = 0;
  }
  return SIGLIP_OK;
}

SIGLIP_API int siglip_debug_timing_read(siglip_model* m, int32_t kernel_class, double* total_ms, int64_t* launches) {
  if (!m || kernel_class < 0 || kernel_class >= SIGLIP_K_COUNT) return fail(SIGLIP_E_INVALID_ARG, "bad model or class");
  // fold every pending pair into the totals, then recycle the events
  for (size_t i = 0; i < m->ev_used; ++i) {
    hipError_t e = hipEventSynchronize(m->ev_pool[2 * i + 1]);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, m->ev_pool[2 * i], m->ev_pool[2 * i + 1]);
    if (e != hipSuccess) return fail(SIGLIP_E_HIP, std::string("timing read: ") + hipGetErrorString(e));
    m->t_ms[m->ev_class[i]] += ms;
    m->t_n[m->ev_class[i]] += 1;
  }
  m->ev_used = 0;
  if (m->timing_lost) return fail(SIGLIP_E_HIP, "an end-of-launch event failed to record");
  if (total_ms) *total_ms = m->t_ms[kernel_class];
  if (launches) *launches = m->t_n[kernel_class];
  return SIGLIP_OK;
}

#ifdef SIGLIP_TEST_HOOKS
SIGLIP_API int siglip_debug_fill_workspace(siglip_model* m, uint16_t pattern) {
  if (!m) return fail(SIGLIP_E_INVALID_ARG, "null model");
  hipError_t e = launch_fill_u16(m->ws, m->ws_bytes / 2, pattern, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(SIGLIP_E_HIP, std::string("fill: ") + hipGetErrorString(e));
  return SIGLIP_OK;
}
#endif  // SIGLIP_TEST_HOOKS

}  // extern "C"
