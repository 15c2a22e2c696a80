/*
 * siglip_test_hooks.h -- test-build entry points of libsiglip.
 *
 * Per-stage checkpoints, the analogue of the operator checkpoints the pages
 * validate against a host reference (page "Single-layer SigLIP vision
 * benchmark", "Performance follow-up": operator checkpoints compared with
 * the host reference), and workspace poisoning for the padding tests. They
 * are exported only by the test build of the library (libsiglip_test.so,
 * compiled with SIGLIP_TEST_HOOKS); the product library (libsiglip.so)
 * exports siglip.h alone. Conventions as in siglip.h.
 */
#ifndef SIGLIP_TEST_HOOKS_H_
#define SIGLIP_TEST_HOOKS_H_

#include "siglip.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SIGLIP_STAGE_EMBED = 0,      /* [M, width]   F16  patch GEMM + bias + pos   */
  SIGLIP_STAGE_LN1 = 1,        /* [M, width]   F16 | e4m3 code (FP8 mode)     */
  SIGLIP_STAGE_QKV = 2,        /* [M, 3*width] F16                            */
  SIGLIP_STAGE_ATTN = 3,       /* [M, width]   F16 | e4m3 code                */
  SIGLIP_STAGE_H_ATTN = 4,     /* [M, width]   F16  after attention residual  */
  SIGLIP_STAGE_LN2 = 5,        /* [M, width]   F16 | e4m3 code                */
  SIGLIP_STAGE_MLP_HIDDEN = 6, /* [M, mlp_pad] F16 | e4m3 code (post-GELU)    */
  SIGLIP_STAGE_H_OUT = 7,      /* [M, width]   F16  after MLP residual        */
  SIGLIP_STAGE_FINAL_LN = 8,   /* [M, width]   F16 | e4m3 code (F16 whenever
                                  the MAP K/V projection is folded)           */
  SIGLIP_STAGE_MAP_KV = 9,     /* [M, 2*width] F16 (explicit MAP K/V only;
                                  0 rows when folded)                         */
  SIGLIP_STAGE_MAP_ATTN = 10,  /* [B, width]   F16 | e4m3 code                */
  SIGLIP_STAGE_MAP_Y = 11,     /* [B, width]   F16  MAP output projection     */
  SIGLIP_STAGE_MAP_LN = 12,    /* [B, width]   F16 | e4m3 code                */
  SIGLIP_STAGE_MAP_HIDDEN = 13,/* [B, mlp_pad] F16 | e4m3 code (post-GELU)    */
  SIGLIP_STAGE_MAP_Q = 14,     /* [1, width]   F16  probe query (create time) */
  SIGLIP_STAGE_V_T = 15,       /* [B*heads*head_dim, round_up(tokens,64)] F16
                                  (e4m3 codes of v * 2^-fp8_scale_exp with
                                  the e4m3 PV product): V of each (image,
                                  head) transposed (dims x tokens, zeros past
                                  tokens); when present, the QKV stage holds
                                  only the Q and K columns; with the e4m3 QK
                                  product the QKV stage is [M, 2*heads*80]
                                  e4m3 codes, head slots of 80 bytes (Q heads,
                                  then K heads; bytes head_dim..79 of a slot
                                  unused), row stride 6*width bytes           */
  SIGLIP_STAGE_COUNT = 16
} siglip_stage;

/* Capture stage outputs on later siglip_encode calls: layer-local stages
 * (LN1..H_OUT) of encoder layer `layer` (0-based) and every other stage.
 * layer < 0 turns capture off. Allocates the capture buffers (sized for
 * max_batch) on first use. Errors: INVALID_ARG, OUT_OF_MEMORY. */
SIGLIP_API int siglip_debug_capture(siglip_model* m, int32_t layer);

/* Describe a captured stage of the last capturing encode: rows, columns
 * holding data, row stride in elements and bytes per element (2 = F16,
 * 1 = e4m3 code of x * 2^-fp8_scale_exp). Any pointer may be NULL. */
SIGLIP_API int siglip_debug_stage_info(const siglip_model* m, int32_t stage,
                                       int64_t* rows, int64_t* cols,
                                       int64_t* ld, int32_t* elem_bytes);

/* Copy a captured stage (rows*ld*elem_bytes bytes) to host memory dst of
 * dst_bytes; synchronises the device. Errors: INVALID_ARG (capture off,
 * stage out of range, dst too small), HIP. */
SIGLIP_API int siglip_debug_stage(const siglip_model* m, int32_t stage,
                                  void* dst, size_t dst_bytes);

/* Fill the whole workspace (every activation buffer, including row and
 * column padding) with a 16-bit pattern, e.g. 0x7E00 (F16 NaN), to show
 * that siglip_encode never reads data it did not write in the same call
 * (page "Layout and barrier diagnosis", "Padding, SRAM placement and paired
 * transfers": padding is read, so unwritten tails must not be). Synchronous. */
SIGLIP_API int siglip_debug_fill_workspace(siglip_model* m, uint16_t pattern);

#ifdef __cplusplus
}
#endif

#endif /* SIGLIP_TEST_HOOKS_H_ */
