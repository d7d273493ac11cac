// Offline (host) preparation of an SVDQuant layer and of AWQ weights.
#pragma once

#include <cstdint>

#include "svdq.h"

namespace svdq {

// Symmetric INT4 quantiser of one group of 64 float32 values (see the
// definition in svdq_prepare_weights): codes in [-7, 7] and the fp32 scale.
void quantize_group64(const float *v, int8_t *q, float *s);

svdq_status_t prepare_weights(const uint16_t *W_bf16, int N, int K, const float *act_absmax,
                              const uint16_t *bias_bf16, int rank, svdq_host_weights_t *out);

svdq_status_t pack_device_weights(const svdq_host_weights_t *in, void *host_blob, size_t bytes);

// MXFP4: one FP4 E2M1 code (see the definition in svdq_mx_prepare_weights),
// one block of 32 values (codes and the E8M0 scale byte), preparation and
// device packing.
uint8_t e2m1_code(float r);
void quantize_block32_mx(const float *v, uint8_t *codes, uint8_t *e8m0);
svdq_status_t prepare_weights_mx(const uint16_t *W_bf16, int N, int K, const float *act_absmax,
                                 const uint16_t *bias_bf16, int rank, svdq_mx_host_weights_t *out);
svdq_status_t pack_device_weights_mx(const svdq_mx_host_weights_t *in, void *host_blob, size_t bytes);

// User LoRA concatenated onto a low-rank branch (see svdq_merge_lora):
// l1s_out [K, r + r2] = [l1s | A^T], l2_out [r + r2, N] = [l2 ; bf16(fl32(alpha B^T))].
svdq_status_t merge_lora_factors(int N, int K, int rank, const uint16_t *l1s, const uint16_t *l2,
                                 const uint16_t *A_bf16, const uint16_t *B_bf16, int r2,
                                 float alpha, uint16_t *l1s_out, uint16_t *l2_out);

svdq_status_t awq_quantize(const uint16_t *W_fp16, int N, int K, uint8_t *q, uint16_t *s,
                           uint16_t *z);

svdq_status_t awq_pack(const uint8_t *q, const uint16_t *s, const uint16_t *z, int N, int K,
                       void *host_blob, size_t bytes);

}  // namespace svdq
