/*
 * siglip.h -- C ABI of the MI355X (gfx950) SigLIP So400m/14 image encoder.
 *
 * The library runs the image-encoder forward pass described on the page
 * "Single-layer SigLIP vision benchmark" (intro and mermaid figure): a
 * 588->1152 patch-embedding GEMM with bias and learned positional
 * embedding, pre-norm encoder layers (layernorm eps 1e-6, fused QKV
 * projection, 16x72 multi-head self-attention, output projection and
 * residual, GELU MLP 1152->4304->1152 and residual), a final layernorm and
 * the MAP pooling head, returning [batch, 1, 1152].
 *
 * Conventions for every function below:
 *   - extern "C", never throws, never aborts; returns a siglip_status.
 *   - On failure, siglip_last_error() returns a thread-local message.
 *   - "device" pointers are HIP device memory on the current device;
 *     "host" pointers are ordinary CPU memory.
 *   - hip_stream is a hipStream_t passed as void*; NULL means the null stream.
 *   - Compute calls enqueue work on hip_stream and return without a host
 *     synchronisation; results are valid once the stream has reached them.
 */
#ifndef SIGLIP_H_
#define SIGLIP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SIGLIP_API __attribute__((visibility("default")))

typedef enum {
  SIGLIP_OK = 0,
  SIGLIP_E_INVALID_ARG = -1,   /* null pointer, size out of range, bad option */
  SIGLIP_E_BAD_BLOB = -2,      /* weight blob malformed, truncated or inconsistent */
  SIGLIP_E_UNSUPPORTED = -3,   /* valid request this library cannot run (dims, device) */
  SIGLIP_E_OUT_OF_MEMORY = -4, /* device allocation failed */
  SIGLIP_E_HIP = -5            /* a HIP runtime call or kernel launch failed */
} siglip_status;

typedef struct siglip_model siglip_model; /* opaque; owned by the library */

/* Options for siglip_create. */
typedef struct {
  /* Encoder layers to run: 0 = every layer in the blob, else 1..depth.
   * The page's single-layer benchmark reduces depth 27 to one. */
  int32_t layers;
  /* Largest batch siglip_encode will accept; the workspace is sized for it. */
  int32_t max_batch;
  /* 0 = F16 GEMM operands; 1 = OCP e4m3 FP8 operands for every weight GEMM
   * (page "Single-layer SigLIP vision benchmark", intro: "--fp8-scale=-4";
   * both operands of a product share the scale, page "FP8 attention and
   * resident image/embedding transfers", intro). Accumulation is F32 in
   * both modes; attention products, layernorm, residuals and GELU stay
   * F16 storage with F32 arithmetic. */
  int32_t gemm_precision;
  /* Power-of-two operand scale exponent for FP8 (the page uses -4): an
   * operand x is stored as e4m3(x * 2^-exp), saturating at +-448, and each
   * product is rescaled by 2^(2*exp). Ignored for F16. Range -8..8. */
  int32_t fp8_scale_exp;
  /* 0 = one fused Q/K/V projection per layer and one fused MAP K/V
   * projection (the default); 1 = separate projections of width columns
   * each (three per layer, two in the MAP head). Page "Single-layer SigLIP
   * vision benchmark", "Fused encoder QKV and MAP KV", compares the two
   * forms. Each output element is computed with the same operands and the
   * same summation order either way, so the results are identical. */
  int32_t separate_qkv;
  /* 0 = MAP head with its K/V projection folded away (the default where
   * supported: heads <= 16, width a multiple of 64, tokens <= 1024): the
   * probe's scores are Z . (W_k,h q_h) and each head's output is
   * (sum_t p_t Z_t) W_v,h + b_v,h, the same real numbers as projecting every
   * token (page "Single-layer SigLIP vision benchmark", intro: one fused K/V
   * projection and one shared probe), computed from the F16 final-LN
   * output with F32 accumulation in both precision modes.
   * 1 = the explicit K/V projection of every token (an e4m3 GEMM in FP8
   * mode) followed by the probe attention. */
  int32_t map_explicit_kv;
  /* Encoder attention products in OCP e4m3 (page "FP8 attention and
   * resident image/embedding transfers": F143 operands at scale -4, PV and
   * QK selected independently, softmax state and the attention output
   * precision unchanged). 0 = both F16 (the default). Bit 0 (1) = PV: the
   * QKV projection writes V^T as e4m3 codes of v * 2^-fp8_scale_exp and the
   * probabilities are quantized to e4m3(p * 2^4) in registers. Bit 1 (2) =
   * QK: the QKV projection writes Q and K as e4m3 codes of x *
   * 2^-fp8_scale_exp. 3 = both. No separate cast runs (the same page, "Full
   * 27-layer ViT": producer-written operands). Independent of
   * gemm_precision; needs head_dim 64, 72 or 80 (UNSUPPORTED otherwise).
   * fp8_scale_exp must then be in -8..8. */
  int32_t attention_fp8;
  /* 0 = each layer's two LayerNorms write their normalized output (F16, or
   * e4m3 in FP8 mode) for the next GEMM (the default). 1 = LayerNorms 1 and
   * 2 are folded into the GEMMs that consume them (the QKV and MLP-up
   * projections): a statistics kernel writes each row's mean and rstd, and
   * those GEMMs normalize the F16 residual rows as they load them, with the
   * LayerNorm's per-element arithmetic, so the results are bitwise those of
   * the default (page "FP8 attention and resident image/embedding
   * transfers", "Full 27-layer ViT": operands prepared by the kernels that
   * use them rather than by separate passes). Slower on MI355X: every
   * column tile normalizes its rows again. Needs width 1152 (UNSUPPORTED
   * otherwise). The final and MAP LayerNorms are unchanged; the test
   * build's LN1 and LN2 stage captures are not produced. */
  int32_t layernorm_fold;
} siglip_options;

/*
 * Parse a weight blob, upload and convert the weights once, allocate the
 * workspace for opt->max_batch images. Parameters stay resident until
 * siglip_destroy (page "SigLIP optimized execution and PV padding",
 * "Full-model results": parameters uploaded once, inference calls repeat).
 *
 * blob:       host memory, blob_bytes long, read during the call only (the
 *             caller may free it afterwards). Format, little-endian:
 *             64-byte header {char magic[4]="SGLP"; u32 version=1; u32 width,
 *             depth, heads, head_dim, mlp, tokens, patch_dim, dtype(0=F32);
 *             u64 total_bytes; u8 reserved[16]}, then every parameter as
 *             float32 at 64-byte aligned offsets in this order: embed.w
 *             [patch_dim,width], embed.b [width], pos [tokens,width]; per
 *             layer ln1.g, ln1.b [width], qkv.w [width,3*width], qkv.b,
 *             out.w [width,width], out.b, ln2.g, ln2.b, mlp1.w [width,mlp],
 *             mlp1.b [mlp], mlp2.w [mlp,width], mlp2.b; final_ln.g, .b;
 *             map.probe [1,width], map.q.w [width,width], map.q.b,
 *             map.kv.w [width,2*width], map.kv.b, map.out.w, map.out.b,
 *             map.ln.g, map.ln.b, map.mlp1.w, map.mlp1.b, map.mlp2.w,
 *             map.mlp2.b. Matrices are [in,out] row-major (y = x W).
 * opt:        host pointer, read during the call.
 * out:        receives the new model; set to NULL on failure.
 * Errors: INVALID_ARG (null pointer, bad options), BAD_BLOB (checked on the
 * CPU before any HIP call), UNSUPPORTED (dims this library cannot run: width
 * != heads*head_dim, width % 128, head_dim > 80 or % 8, mlp % 8,
 * patch_dim % 4, tokens > 4096, or a device that is not gfx950),
 * OUT_OF_MEMORY, HIP. Blocks until the upload and conversion are complete.
 */
SIGLIP_API int siglip_create(const void* blob, size_t blob_bytes,
                             const siglip_options* opt, siglip_model** out);

/*
 * Forward pass: patch-ordered F16 pixels to F16 embeddings.
 *
 * pixels_f16: device, [batch, tokens, patch_dim] F16 contiguous, in
 *             [batch, patch_y, patch_x, y, x, channel] order (page
 *             "Single-layer SigLIP vision benchmark", intro). Read only;
 *             8-byte aligned.
 * batch:      1..max_batch.
 * out_f16:    device, [batch, 1, width] F16 contiguous (page "Single-layer
 *             SigLIP vision benchmark", intro: the probe axis is kept);
 *             16-byte aligned (rows are written in 16-byte chunks).
 * hip_stream: stream to enqueue on.
 * A batch of two or more images runs as two half-batches: the first half on
 * hip_stream, the second on a stream the model owns (default priority),
 * which waits for hip_stream's earlier work and which hip_stream waits for
 * before its later work, so the call behaves as one ordered unit of
 * hip_stream. Images are independent, each output row is computed by the
 * same kernels in the same order either way, and the results are bitwise
 * identical. Launch timing (siglip_debug_timing) and, in the test build,
 * stage capture run the batch on hip_stream alone.
 * The model's workspace is shared by its calls: calls on one model must be
 * ordered (one stream, or explicit synchronisation). Results are bitwise
 * deterministic run to run. The call enqueues kernel launches and event
 * records/waits only (no allocation, memset or host synchronisation), so it
 * may be captured into a HIP graph by stream capture on hip_stream and the
 * graph replayed; a replay reads and writes the pointers given at capture.
 * Errors: INVALID_ARG, HIP.
 */
SIGLIP_API int siglip_encode(siglip_model* m, const void* pixels_f16,
                             int32_t batch, void* out_f16, void* hip_stream);

/*
 * Multi-head scaled dot-product attention alone, the encoder's attention
 * step: for each image b and head h, o = softmax(q k^T * scale) v with F32
 * softmax state (running maximum, denominator) and F32 accumulation; the
 * result is rounded to F16 (page "Single-layer SigLIP vision benchmark",
 * intro: attention explicitly converts its result back to F16; page
 * "Capacity-first baseline", blocked attention keeps running max and
 * denominator).
 *
 * q, k, v:     device F16; row r of image b starts at
 *              ptr + (b*tokens + r)*row_stride_elems; head h occupies the
 *              head_dim columns from h*head_dim. They may be three views
 *              into one fused [.., 3*heads*head_dim] QKV buffer.
 * o:           device F16 [batch, tokens, heads*head_dim] contiguous.
 * Requires head_dim % 8 == 0, head_dim <= 80, row_stride_elems % 8 == 0
 * and >= heads*head_dim, 16-byte aligned pointers, tokens >= 1. No data
 * past token tokens-1 of an image or past column head_dim-1 of a head is
 * read.
 * Head widths 64, 72 and 80 run the encoder's own streaming kernel: V is
 * first transposed per image into a staging buffer of
 * batch * heads*head_dim * round_up(tokens, 64) * 2 bytes that the library
 * owns, one per device, allocated by the first call that needs more than
 * any call before it (hipMalloc; that call is then not capturable into a
 * HIP graph) and kept until the process ends. Calls on one device share
 * it: calls that overlap in time on one device (different streams, no
 * ordering) race. Other head widths use a register-staged kernel and no
 * staging. Errors: INVALID_ARG, UNSUPPORTED, OUT_OF_MEMORY, HIP.
 */
SIGLIP_API int siglip_attention(const void* q, const void* k, const void* v,
                                int64_t row_stride_elems, void* o,
                                int32_t batch, int32_t heads, int32_t tokens,
                                int32_t head_dim, float scale, void* hip_stream);

/*
 * siglip_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, the same kernels and the same results,
 * but the V^T staging lives in a fixed 64 MiB device array of the library
 * (a file-scope __device__ array, one per GPU, held until the process
 * ends) instead of a buffer it allocates. The call makes no hipMalloc,
 * hipFree or other allocating call; the first call on a device looks up
 * the array's device address (hipGetSymbolAddress) once.
 * Limit: batch * heads*head_dim * round_up(tokens, 64) * 2 <= 64 MiB for
 * head widths 64, 72 and 80 (the attention workload [32, 729, 16 x 72]
 * needs 56.6 MB); larger calls fail with INVALID_ARG before any launch.
 * Every call on a GPU shares that GPU's array and leaves its contents
 * behind: calls that overlap in time on one GPU (different streams, no
 * ordering) race. Each call writes every staging byte it reads (V^T and its
 * zero padding) before reading it. Errors: INVALID_ARG, UNSUPPORTED, HIP.
 */
SIGLIP_API int siglip_attention_noalloc(const void* q, const void* k, const void* v,
                                        int64_t row_stride_elems, void* o,
                                        int32_t batch, int32_t heads, int32_t tokens,
                                        int32_t head_dim, float scale, void* hip_stream);

/* Free the model's device memory. Synchronises the device first. NULL is a
 * no-op returning SIGLIP_OK. */
SIGLIP_API int siglip_destroy(siglip_model* m);

/* Static string naming a status code; never NULL. */
SIGLIP_API const char* siglip_status_string(int status);

/* Thread-local detail of the last failure on this thread ("" if none). */
SIGLIP_API const char* siglip_last_error(void);

/* Model dimensions as created: width, depth used, heads, head_dim, mlp,
 * tokens, patch_dim, max_batch, gemm_precision (any pointer may be NULL). */
SIGLIP_API int siglip_model_info(const siglip_model* m, int32_t* width,
                                 int32_t* layers, int32_t* heads,
                                 int32_t* head_dim, int32_t* mlp,
                                 int32_t* tokens, int32_t* patch_dim,
                                 int32_t* max_batch, int32_t* gemm_precision);

/* ---------------------------------------------------------------------
 * Measurement: per-launch timing of the kernel classes of siglip_encode
 * (used by the benchmark for per-kernel times and the roofline figure).
 * ------------------------------------------------------------------- */
/* Kernel classes of one siglip_encode call, for per-launch timing. */
typedef enum {
  SIGLIP_K_INPUT = 0,       /* patch rows -> padded GEMM operand          */
  SIGLIP_K_EMBED = 1,       /* patch GEMM + bias + positional embedding   */
  SIGLIP_K_LAYERNORM = 2,   /* every encoder, final and MAP layernorm     */
  SIGLIP_K_QKV = 3,         /* fused QKV GEMM + bias                      */
  SIGLIP_K_ATTENTION = 4,   /* encoder flash attention                    */
  SIGLIP_K_OUT_PROJ = 5,    /* output projection + bias + residual        */
  SIGLIP_K_MLP_UP = 6,      /* MLP up GEMM + bias + GELU                  */
  SIGLIP_K_MLP_DOWN = 7,    /* MLP down GEMM + bias + residual            */
  SIGLIP_K_MAP_KV = 8,      /* MAP fused KV GEMM + bias                   */
  SIGLIP_K_MAP_ATTENTION = 9, /* MAP probe attention                      */
  SIGLIP_K_MAP_TAIL = 10,   /* MAP output projection and MLP GEMMs        */
  SIGLIP_K_COUNT = 11
} siglip_kernel_class;

/* Per-launch timing of later siglip_encode calls on this model, and reset of
 * the totals. class_mask bit k (1 << siglip_kernel_class) selects the
 * launches of class k; 0 turns timing off. Each selected launch is bracketed
 * by two HIP events recorded on the call's stream, so its duration is the
 * time between them on the GPU; unselected launches are not perturbed.
 * While timing is on, siglip_encode runs the whole batch on the call's
 * stream (no half-batch split), so a launch's duration is its own.
 * Errors: INVALID_ARG. */
SIGLIP_API int siglip_debug_timing(siglip_model* m, uint32_t class_mask);

/* Totals since timing was turned on for one kernel class: summed launch
 * durations in milliseconds and the number of launches. Waits for the
 * recorded events. Errors: INVALID_ARG, HIP. */
SIGLIP_API int siglip_debug_timing_read(siglip_model* m, int32_t kernel_class,
                                        double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* SIGLIP_H_ */
