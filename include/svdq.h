/*
 * svdq.h -- C ABI of libsvdq, an MI355X (gfx950) implementation of the
 * SVDQuant W4A4 linear layer with its 16-bit low-rank branch, and of the
 * AWQ-style W4A16 linear used for modulation layers.
 *
 * Method.  "Bringing Nunchaku 4-bit diffusion inference to Diffusers"
 * (Vietnamese edition, section "Bối cảnh: SVDQuant và Nunchaku"; Korean
 * edition, section "SVDQuant 및 Nunchaku 엔진"): activation outliers are
 * migrated into the weights by per-channel smoothing, the hardest part of
 * each smoothed weight is kept as a small 16-bit low-rank branch, and the
 * remaining residual runs on 4-bit weights against 4-bit activations.  With
 * X [M,K] bf16, W [N,K] bf16 (nn.Linear layout) and b [N]:
 *
 *   Y = Q4(X diag(iota)) Q4(R)^T (group scales) + (X L1s) L2 + b
 *   R = W diag(lambda) - (diag(lambda) L1s L2)^T,   iota = 1/lambda
 *
 * Q4 is symmetric INT4 (codes -7..7) per group of 64 consecutive input
 * channels with float32 scales s = a/7, a the group's max |value|.
 * The same pages (Korean edition, same section) place the low-rank
 * down-projection next to activation quantisation and the up-projection in
 * the 4-bit GEMM; this library does the same with two device kernels.
 *
 * Conventions for every entry point
 *   - Every function returns svdq_status_t; nothing throws across the ABI.
 *     svdq_last_error() returns a thread-local message for the last failure.
 *   - All validation is synchronous and happens before any HIP call.
 *   - Ownership: the caller owns every host and device buffer.  The library
 *     never allocates device memory; device scratch is the caller's
 *     `workspace` (size from svdq_workspace_bytes).
 *   - Device entry points are asynchronous: they enqueue on `hip_stream`
 *     (a hipStream_t; NULL = the null stream) and never synchronise.  Launch
 *     failures return SVDQ_ERR_HIP; faults surface at the caller's next sync.
 *   - Device check: the first device call on a device checks that it is a
 *     gfx950 part and caches the answer; any other device gets
 *     SVDQ_ERR_UNSUPPORTED_DEVICE rather than a wrong result (the pages'
 *     "Hỗ trợ phần cứng" section: the quantiser refuses unsupported GPUs at
 *     load time with a clear error).
 *   - Device pointers must be 16-byte aligned.
 *   - Shapes: K % 64 == 0; M, N >= 1 (ragged tails are masked); rank in
 *     [0, min(N, K)] and rank <= 256.
 *   - bf16 / fp16 values are passed as uint16_t bit patterns on the host.
 */
#ifndef SVDQ_H_
#define SVDQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVDQ_ABI_VERSION 1
#define SVDQ_GROUP_SIZE 64
#define SVDQ_MAX_RANK 256

typedef enum {
  SVDQ_OK = 0,
  SVDQ_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad enum, misaligned pointer */
  SVDQ_ERR_UNSUPPORTED_SHAPE = 2,  /* K % 64 != 0, rank out of range, M/N/K < 1, too large */
  SVDQ_ERR_NO_DEVICE = 3,          /* no HIP device visible */
  SVDQ_ERR_UNSUPPORTED_DEVICE = 4, /* the current device is not gfx950 */
  SVDQ_ERR_WORKSPACE_TOO_SMALL = 5,
  SVDQ_ERR_NUMERICAL = 6,          /* non-finite input to an offline step */
  SVDQ_ERR_HIP = 7                 /* a HIP runtime call or launch failed */
} svdq_status_t;

typedef enum { SVDQ_BF16 = 0, SVDQ_FP16 = 1, SVDQ_FP32 = 2 } svdq_dtype_t;

/* Output epilogue of svdq_linear_forward. */
typedef enum {
  SVDQ_EPILOGUE_NONE = 0,
  /* Y = gelu_tanh(linear(X)): the activation between the two projections of
   * a diffusion-transformer MLP, fused into the store (Vietnamese edition,
   * section "Giới thiệu Nunchaku Lite", which credits fused GELU/MLP paths
   * for part of the original engine's speed). */
  SVDQ_EPILOGUE_GELU_TANH = 1
} svdq_epilogue_t;

int svdq_abi_version(void);
const char *svdq_status_string(svdq_status_t s);
/* Thread-local description of the most recent failure on this thread. */
const char *svdq_last_error(void);

/* Checks the current HIP device once and caches the answer.  Returns
 * SVDQ_OK on gfx950, SVDQ_ERR_NO_DEVICE or SVDQ_ERR_UNSUPPORTED_DEVICE
 * otherwise.  Called implicitly by every device entry point. */
svdq_status_t svdq_device_check(void);

/* ======================================================== offline, host only */

/* Host-side prepared weights.  Every pointer is caller-owned; sizes in bytes
 * come from svdq_host_weights_sizes (order: inv_lambda, l1s, l2, qweight,
 * wscales, bias). */
typedef struct {
  int32_t N, K, rank, group_size; /* group_size is always 64 */
  float *inv_lambda;   /* [K]       fp32 iota_j = fl32(1/lambda_j) */
  uint16_t *l1s;       /* [K, rank] bf16, = bf16(diag(iota) V_r S_r^(1/2)) */
  uint16_t *l2;        /* [rank, N] bf16, = bf16(S_r^(1/2) U_r^T) */
  uint8_t *qweight;    /* [N, K/2]  residual codes, canonical packing: byte j of a
                          row = code 2j (low nibble) | code 2j+1 (high nibble),
                          two's complement, codes in [-7, 7] */
  float *wscales;      /* [N, K/64] fp32 group scales of the residual */
  float *bias;         /* [N]       fp32 (zeros when no bias) */
} svdq_host_weights_t;

svdq_status_t svdq_host_weights_sizes(int N, int K, int rank, size_t sizes_out[6]);

/* Per-channel max |x| over `rows` calibration rows of bf16 activations
 * X_bf16 [rows, K] -> absmax_out [K] fp32.  Host only. */
svdq_status_t svdq_calibration_absmax(const uint16_t *X_bf16, int rows, int K,
                                      float *absmax_out);

/* Offline preparation of one linear layer (host, multi-threaded):
 *   1. smoothing factors lambda_j = fl32(sqrt(fl32(max(ax_j,1e-5)/max(aw_j,1e-5))))
 *      from act_absmax (ax) and the weight column maxima (aw); act_absmax ==
 *      NULL means no smoothing (lambda = 1).  Activation outliers move into
 *      the weights (Vietnamese edition, "Bối cảnh: SVDQuant và Nunchaku").
 *   2. W_hat = W diag(lambda) (float64), top-`rank` singular triplets of W_hat
 *      (Gram matrix of the smaller side, Householder tridiagonalisation,
 *      bisection and inverse iteration), split as L1 = V S^(1/2),
 *      L2 = S^(1/2) U^T, stored bf16 with iota folded into L1.
 *   3. residual R = W_hat - (diag(lambda) L1s L2)^T against the rounded
 *      factors (float64, then float32), quantised per row and group of 64.
 * W_bf16 [N, K] row-major; bias_bf16 [N] or NULL; group_size must be 64.
 * Returns SVDQ_ERR_NUMERICAL on non-finite W, bias or act_absmax. */
svdq_status_t svdq_prepare_weights(const uint16_t *W_bf16, int N, int K,
                                   const float *act_absmax,
                                   const uint16_t *bias_bf16, int rank,
                                   int group_size, svdq_host_weights_t *out);

/* Size of the device weight blob for (N, K, rank). */
size_t svdq_device_weights_bytes(int N, int K, int rank);

/* Re-tiles prepared host weights into the device blob layout (host memory,
 * caller-allocated, `bytes` >= svdq_device_weights_bytes).  The caller
 * uploads the blob to device memory; the layout is internal to the library
 * and versioned with SVDQ_ABI_VERSION. */
svdq_status_t svdq_pack_device_weights(const svdq_host_weights_t *in,
                                       void *host_blob, size_t bytes);

/* A user LoRA carried by the layer's low-rank branch (host only).  The pages
 * keep LoRA loading working on quantised models ("Bringing Nunchaku 4-bit
 * diffusion inference to Diffusers", Vietnamese edition, section "Tải
 * nguyên bản trong Diffusers"; Russian edition, closing paragraph), and the
 * Hacker News thread "SVDQuant: 4-Bit Quantization Powers 12B Flux on a 16GB
 * 4090 GPU with 3x Speedup" describes the branch itself as a LoRA.  A LoRA
 * with down factor A [r', K] and up factor B [N, r'] (bf16, row-major, the
 * nn.Linear layouts of its two projections) and scale alpha adds
 * alpha (X A^T) B^T to Y.  The merged layer has rank r + r':
 *   l1s' = [l1s | A^T]                  [K, r + r']
 *   l2'  = [l2 ; bf16(fl32(alpha B^T))]  [r + r', N]
 * (one float32 product per element, one rounding to bf16); A acts on the raw
 * activations.  Smoothing factors, residual codes and scales and bias are
 * unchanged, so the 4-bit path is the base layer's bit for bit.
 *   in:  a prepared layer; it is not modified.
 *   out: caller-allocated with svdq_host_weights_sizes(N, K, r + r'); its
 *        l1s and l2 must not overlap in's factors (SVDQ_ERR_INVALID_ARGUMENT).
 *        Its inv_lambda, qweight, wscales and bias may be the very buffers of
 *        `in` (then they are left as they are) or separate ones (copied).
 *        N, K, rank (= r + r') and group_size are set on success.
 * lora_rank = 0 copies the layer.  Errors: SVDQ_ERR_UNSUPPORTED_SHAPE when
 * r + r' exceeds min(N, K, SVDQ_MAX_RANK); SVDQ_ERR_NUMERICAL for a
 * non-finite alpha, down factor or alpha * up factor (nothing is written). */
svdq_status_t svdq_merge_lora(const svdq_host_weights_t *in, const uint16_t *lora_down_bf16,
                              const uint16_t *lora_up_bf16, int lora_rank, float alpha,
                              svdq_host_weights_t *out);

/* A prepared layer resident in device memory. */
typedef struct {
  const void *blob;   /* device pointer to the uploaded blob */
  int32_t N, K, rank;
} svdq_weights_t;

/* =================================================== runtime, device, async */

/* Device scratch needed by svdq_linear_forward for M token rows.  When the
 * GEMM's grid of 128 x 256 output tiles has fewer than 128 tiles (the chip
 * has 256 CUs), the GEMM is split along K into ksplit = min(8, 512 / tiles,
 * (K / 64) / 8) ranges (if that is at least 2) whose fp32 partial tiles a
 * second kernel sums in range order, and the size includes ksplit * Mp * Np
 * * 4 bytes for them (Mp, Np: M and N rounded up to 256).  A workspace
 * without that room is still accepted; the GEMM then runs unsplit (the same
 * result up to the order of fp32 additions). */
size_t svdq_workspace_bytes(int M, int N, int K, int rank);

/* Y = linear(X) [+ epilogue] for X bf16 [M, K] (device, row-major) into
 * Y [M, N] of dtype y_dtype (SVDQ_BF16 or SVDQ_FP32), row-major.
 * Two kernels on `hip_stream`: (1) smoothing + per-group INT4 quantisation of
 * X + low-rank down-projection D = X L1s; (2) INT4 x INT4 group GEMM with
 * fp32 per-group scaling, + D L2 + bias (+ GELU) in the epilogue. */
svdq_status_t svdq_linear_forward(const svdq_weights_t *w, const void *X, int M,
                                  void *Y, svdq_dtype_t y_dtype,
                                  svdq_epilogue_t epilogue, void *workspace,
                                  size_t ws_bytes, void *hip_stream);

/* svdq_linear_forward for callers that cannot allocate device memory at all
 * (code under stream capture, tight serving loops, harnesses that forbid
 * allocation).  The same two kernels, with the workspace in a file-scope
 * device array of the library (SVDQ_STATIC_SCRATCH_BYTES per device,
 * reserved for the life of the process on every device the library runs on)
 * instead of a caller buffer.  Nothing is allocated, by the library or by
 * the call.  Shapes whose svdq_workspace_bytes(M, N, K, rank) without the
 * K-split room exceeds the limit get SVDQ_ERR_WORKSPACE_TOO_SMALL; the
 * K-split runs when its partials fit too.  Every call on one device shares
 * that device's array: calls that overlap in time on one device (two
 * streams, two threads) race, so such callers order them.  The array keeps
 * the last call's contents; the call needs none of it cleared.  Other
 * arguments, validation and errors as for svdq_linear_forward. */
#define SVDQ_STATIC_SCRATCH_BYTES (64ll << 20)
svdq_status_t svdq_linear_forward_static(const svdq_weights_t *w, const void *X, int M,
                                         void *Y, svdq_dtype_t y_dtype,
                                         svdq_epilogue_t epilogue, void *hip_stream);

/* The same forward with the 16-bit branch unfused, for measuring what the
 * fusion saves (the pages credit the original engine with fusing the
 * down-projection into the quantiser and the up-projection into the 4-bit
 * GEMM, Korean edition, section "SVDQuant 및 Nunchaku 엔진").  Four
 * kernels: the quantiser without the down-projection; D = X L1s as its own
 * bf16 GEMM (D to memory); the 4-bit GEMM without the up-projection, its
 * fp32 result (bias included) to memory; Y = epilogue(that + D L2) as a
 * second bf16 GEMM.  Same arguments, results (up to the order of fp32
 * additions) and errors as svdq_linear_forward; the workspace must hold
 * svdq_unfused_workspace_bytes(M, N, K, rank) bytes (the forward's, plus
 * the fp32 result [M, N]). */
size_t svdq_unfused_workspace_bytes(int M, int N, int K, int rank);
svdq_status_t svdq_linear_forward_unfused(const svdq_weights_t *w, const void *X, int M,
                                          void *Y, svdq_dtype_t y_dtype,
                                          svdq_epilogue_t epilogue, void *workspace,
                                          size_t ws_bytes, void *hip_stream);

/* The forward's two kernels as separate calls, for callers that time or
 * schedule them apart.  svdq_linear_quantize runs kernel (1) on X and leaves
 * the activation codes, scales and low-rank partials in `workspace`;
 * svdq_linear_gemm runs kernel (2) from that workspace (same M, same weights,
 * enqueued after the quantize call on the same stream or ordered after it).
 * Calling both is exactly svdq_linear_forward. */
svdq_status_t svdq_linear_quantize(const svdq_weights_t *w, const void *X, int M,
                                   void *workspace, size_t ws_bytes, void *hip_stream);
svdq_status_t svdq_linear_gemm(const svdq_weights_t *w, int M, void *Y, svdq_dtype_t y_dtype,
                               svdq_epilogue_t epilogue, const void *workspace,
                               size_t ws_bytes, void *hip_stream);

/* MLP pair with the GELU/MLP fusion the pages credit to the original engine
 * (VI, section "Giới thiệu Nunchaku Lite"): Y = linear2(bf16(epilogue(
 * linear1(X)))) where linear1's GEMM applies bias (+ GELU), rounds to bf16
 * and quantises the result for linear2 in its epilogue (codes, scales and the
 * low-rank down-projection D, the last as a 64-bit fixed-point sum so the
 * result does not depend on the order of the GEMM's workgroups); the
 * intermediate activations never go to memory.  w2->K must equal w1->N.
 * ws1 / ws2 are the two layers' own workspaces (svdq_workspace_bytes with
 * each layer's shape, same M), distinct and caller-owned.  epilogue applies
 * to linear1 (NONE or GELU_TANH); linear2 adds its bias only.  Y [M, N2] of
 * y_dtype (SVDQ_BF16 or SVDQ_FP32), row-major.  Three kernels on
 * `hip_stream`, also callable apart: svdq_mlp_quantize (linear1's quantiser,
 * which also clears linear2's D), svdq_mlp_gemm1 (linear1's GEMM with the
 * quantising epilogue), svdq_mlp_gemm2 (linear2's GEMM); each must follow
 * the previous on the stream.  Errors as for svdq_linear_forward, plus
 * SVDQ_ERR_UNSUPPORTED_SHAPE when the shapes do not chain and
 * SVDQ_ERR_INVALID_ARGUMENT when ws1 == ws2. */
svdq_status_t svdq_mlp_forward(const svdq_weights_t *w1, const svdq_weights_t *w2,
                               const void *X, int M, void *Y, svdq_dtype_t y_dtype,
                               svdq_epilogue_t epilogue, void *ws1, size_t ws1_bytes,
                               void *ws2, size_t ws2_bytes, void *hip_stream);
svdq_status_t svdq_mlp_quantize(const svdq_weights_t *w1, const svdq_weights_t *w2,
                                const void *X, int M, void *ws1, size_t ws1_bytes,
                                void *ws2, size_t ws2_bytes, void *hip_stream);
svdq_status_t svdq_mlp_gemm1(const svdq_weights_t *w1, const svdq_weights_t *w2, int M,
                             svdq_epilogue_t epilogue, const void *ws1, size_t ws1_bytes,
                             void *ws2, size_t ws2_bytes, void *hip_stream);
svdq_status_t svdq_mlp_gemm2(const svdq_weights_t *w2, int M, void *Y, svdq_dtype_t y_dtype,
                             const void *ws2, size_t ws2_bytes, void *hip_stream);

/* Elementwise bf16 -> bf16 tanh-GELU (the unfused glue between the MLP's
 * projections; same reading as SVDQ_EPILOGUE_GELU_TANH), n elements. */
svdq_status_t svdq_gelu_tanh_bf16(const void *in, void *out, size_t n,
                                  void *hip_stream);

/* ===================================================== FP4 (MXFP4) variant
 * The 4-bit path in the FP4 form the pages name beside INT4 ("Bringing
 * Nunchaku 4-bit diffusion inference to Diffusers", Vietnamese edition,
 * section "Giới thiệu Nunchaku Lite"; Korean edition, section "Diffusers 내
 * Nunchaku Lite 통합": an NVFP4 path for Blackwell, whose numerics the pages
 * do not give).  Everything of the INT4 method is kept (smoothing, low-rank
 * split, residual, 16-bit branch); the residual weights and the smoothed
 * activations are encoded in OCP Microscaling MXFP4 instead, the
 * block-scaled format gfx950's matrix instructions take natively:
 *   - blocks of 32 consecutive values along K share one power-of-two scale
 *     2^e, e = floor(log2(max |v|)) - 2 clamped to [-127, 127] (-127 for an
 *     all-zero block), stored as the E8M0 byte e + 127;
 *   - each value v / 2^e becomes an FP4 E2M1 code (sign bit 3; magnitudes
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7), nearest value, ties to the
 *     even mantissa bit, saturating at 6, zero stored as +0.
 * The matrix instruction applies both scales, so the GEMM needs no
 * per-element scaling work.  K must be a multiple of 64. */

/* Host-side prepared MXFP4 weights; sizes from svdq_mx_host_weights_sizes
 * (order: inv_lambda, l1s, l2, qweight, wscales, bias). */
typedef struct {
  int32_t N, K, rank;
  float *inv_lambda;   /* [K]       as in svdq_host_weights_t */
  uint16_t *l1s;       /* [K, rank] as in svdq_host_weights_t */
  uint16_t *l2;        /* [rank, N] as in svdq_host_weights_t */
  uint8_t *qweight;    /* [N, K/2]  E2M1 codes, byte j = code 2j | code 2j+1 << 4 */
  uint8_t *wscales;    /* [N, K/32] E8M0 block scales (biased exponents) */
  float *bias;         /* [N]       fp32 */
} svdq_mx_host_weights_t;

svdq_status_t svdq_mx_host_weights_sizes(int N, int K, int rank, size_t sizes_out[6]);

/* Steps 1 and 2 of svdq_prepare_weights, then the residual rows in MXFP4.
 * Same arguments and errors (no group size: blocks are 32). */
svdq_status_t svdq_mx_prepare_weights(const uint16_t *W_bf16, int N, int K,
                                      const float *act_absmax,
                                      const uint16_t *bias_bf16, int rank,
                                      svdq_mx_host_weights_t *out);

size_t svdq_mx_device_weights_bytes(int N, int K, int rank);
svdq_status_t svdq_mx_pack_device_weights(const svdq_mx_host_weights_t *in,
                                          void *host_blob, size_t bytes);
size_t svdq_mx_workspace_bytes(int M, int N, int K, int rank);

/* svdq_merge_lora for an MXFP4 layer: the same factor concatenation, the
 * same arguments, ownership and errors; the E8M0 scales are copied like the
 * INT4 group scales. */
svdq_status_t svdq_mx_merge_lora(const svdq_mx_host_weights_t *in, const uint16_t *lora_down_bf16,
                                 const uint16_t *lora_up_bf16, int lora_rank, float alpha,
                                 svdq_mx_host_weights_t *out);

/* Y = linear(X) [+ epilogue] through the MXFP4 path, with the conventions of
 * svdq_linear_forward; `w` describes a blob packed by
 * svdq_mx_pack_device_weights.  Two kernels: (1) smoothing + MXFP4 encoding
 * of X + low-rank down-projection; (2) the block-scaled FP4 GEMM with the
 * low-rank up-projection, bias (+ GELU) in its epilogue.  The quantize and
 * GEMM halves are also callable apart, as for the INT4 path. */
svdq_status_t svdq_mx_linear_forward(const svdq_weights_t *w, const void *X, int M,
                                     void *Y, svdq_dtype_t y_dtype,
                                     svdq_epilogue_t epilogue, void *workspace,
                                     size_t ws_bytes, void *hip_stream);
svdq_status_t svdq_mx_linear_quantize(const svdq_weights_t *w, const void *X, int M,
                                      void *workspace, size_t ws_bytes, void *hip_stream);
svdq_status_t svdq_mx_linear_gemm(const svdq_weights_t *w, int M, void *Y,
                                  svdq_dtype_t y_dtype, svdq_epilogue_t epilogue,
                                  const void *workspace, size_t ws_bytes, void *hip_stream);

/* Canonical export of kernel (1): qact [M, K/2] packed E2M1 codes, ascales
 * [M, K/32] E8M0 bytes, lowrank_down [M, rank] fp32.  Device pointers. */
svdq_status_t svdq_mx_quantize_activations(const svdq_weights_t *w, const void *X, int M,
                                           uint8_t *qact, uint8_t *ascales,
                                           float *lowrank_down, void *workspace,
                                           size_t ws_bytes, void *hip_stream);

/* ------------------------------------------- test / inspection exports
 * Same device kernels as the forward, writing canonical layouts. */

/* qact [M, K/2] canonical packed activation codes, ascales [M, K/64] fp32,
 * lowrank_down [M, rank] fp32 (= X L1s).  All device pointers. */
svdq_status_t svdq_quantize_activations(const svdq_weights_t *w, const void *X,
                                        int M, uint8_t *qact, float *ascales,
                                        float *lowrank_down, void *workspace,
                                        size_t ws_bytes, void *hip_stream);

/* Exact int32 group sums P[i, j, g] = sum_{k in group g} qA[m0+i, k] qW[n0+j, k]
 * for the window [m0, m0+mcount) x [n0, n0+ncount), computed by the GEMM
 * kernel's own matrix-core path from the activation codes a preceding
 * svdq_linear_forward / svdq_quantize_activations left in `workspace`
 * (same M).  P is device [mcount, ncount, K/64] int32.  mcount, ncount in
 * [1, 256]. */
svdq_status_t svdq_debug_group_sums(const svdq_weights_t *w, int M, int m0,
                                    int mcount, int n0, int ncount, int32_t *P,
                                    const void *workspace, size_t ws_bytes,
                                    void *hip_stream);

/* The same group sums for caller-supplied activation codes: qact is device
 * [M, K/2] canonical packed INT4 codes (two's complement nibbles, low nibble
 * = even k), the form svdq_quantize_activations exports.  A first kernel
 * packs them into the fp6 code blocks of `workspace` (overwriting the codes
 * a previous forward left there; the rest of the workspace is untouched),
 * then the GEMM kernel sums them as above.  Codes are -7..7; a nibble 0x8
 * (-8, outside the code set) is entered as 0.  Errors and window limits as
 * svdq_debug_group_sums; M * K <= 2^31. */
svdq_status_t svdq_debug_group_sums_codes(const svdq_weights_t *w, const uint8_t *qact, int M,
                                          int m0, int mcount, int n0, int ncount, int32_t *P,
                                          void *workspace, size_t ws_bytes, void *hip_stream);

/* ============================================================== AWQ W4A16
 * "Bringing Nunchaku 4-bit diffusion inference to Diffusers" (Russian
 * edition, technical-details section; Korean edition, "Diffusers 내
 * Nunchaku Lite 통합"): 4-bit weights with 16-bit activations for
 * memory-bound, precision-sensitive modulation projections. */

/* Host round-to-nearest asymmetric INT4 per group of 64:
 *   s = fp16(fl32(max(wmax - wmin, 1e-5) / 15)), z = clamp(rint(fl32(-wmin/s)), 0, 15),
 *   q = clamp(rint(fl32(w/s)) + z, 0, 15).
 * W_fp16 [N, K]; q [N, K/2] canonical unsigned nibbles (low = even k);
 * scales_fp16, zeros_fp16 [N, K/64]. */
svdq_status_t awq_quantize_weights(const uint16_t *W_fp16, int N, int K,
                                   int group_size, uint8_t *q,
                                   uint16_t *scales_fp16, uint16_t *zeros_fp16);

/* Device blob of AWQ weights (host memory, caller-allocated, `bytes` >=
 * awq_device_weights_bytes).  Zero points must be integers in 0..15 (the
 * kernel forms q - z exactly in fp16 from that range) and scales finite:
 * otherwise SVDQ_ERR_INVALID_ARGUMENT (zero point) or SVDQ_ERR_NUMERICAL
 * (scale), and nothing is written. */
size_t awq_device_weights_bytes(int N, int K);
svdq_status_t awq_pack_device_weights(const uint8_t *q, const uint16_t *scales_fp16,
                                      const uint16_t *zeros_fp16, int N, int K,
                                      void *host_blob, size_t bytes);

/* y [M, N] fp16 = sum_g s (sum_{k in g} x (q - z)) (+ bias) for x fp16 [M, K],
 * M in [1, 16]; bias_fp16 [N] or NULL.  Device pointers; async. */
svdq_status_t awq_w4a16_forward(const void *blob, int N, int K, const void *x_fp16,
                                int M, const void *bias_fp16, void *y_fp16,
                                void *hip_stream);

/* ============================================================ measurement
 * Not part of the layer: the practical HBM rate that the bandwidth-bound
 * kernels (the quantiser, the W4A16 GEMV) are judged against.  Streams
 * `bytes` (a multiple of 16) from device `src` with `grid` workgroups of 256
 * threads: mode 0 reads every 16-byte word once and writes one 32-bit word
 * per workgroup to device `sink` [grid]; mode 1 copies to device `dst`.
 * Asynchronous on `hip_stream`. */
svdq_status_t svdq_measure_stream(const void *src, void *dst, size_t bytes, int grid, int mode,
                                  uint32_t *sink, void *hip_stream);

/* Not part of the layer: the issue rate of the matrix instructions the path
 * uses, operands in registers.  Launches `grid` workgroups of 256 threads;
 * every wavefront runs four independent chains of `iters` instructions of
 * one kind: 0 fp6 32x32x64 block-scaled (K2's group sums), 1 fp4 32x32x64
 * (the MXFP4 form), 2 bf16 32x32x16, 3 bf16 32x32x8 (K2's scale product),
 * 4 int8 32x32x32; or one instruction mix per chain and iteration: 5 an
 * fp6 32x32x64 plus 16 fp32 FMAs on other registers, 6 the 16 FMAs alone,
 * 7 the GEMM's step for one 32 x 32 tile (bf16 32x32x8 scale product, fp6
 * group sum, 16 FMAs).  Each workgroup writes one word to device `sink`
 * [grid] (so no work is optimised away).  The caller times the launch:
 * slots = grid * 4 wavefronts * 4 chains * iters.  Errors:
 * SVDQ_ERR_INVALID_ARGUMENT (kind, NULL sink), SVDQ_ERR_UNSUPPORTED_SHAPE
 * (iters outside 1..2^24, grid outside 1..2^20).  Asynchronous. */
svdq_status_t svdq_measure_mfma(int kind, int iters, int grid, uint32_t *sink, void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* SVDQ_H_ */
