// Host half of the C ABI: status strings, the thread-local error, offline
// preparation, packing and size queries.  No HIP calls here.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.h"
#include "host_prepare.h"
#include "layout.h"

namespace svdq {

static thread_local char g_last_error[512] = "";

svdq_status_t fail(svdq_status_t s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

static bool shape_ok(int N, int K, int rank, const char *who, svdq_status_t *st) {
  if (N < 1 || K < 1) {
    *st = fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: N=%d K=%d must be >= 1", who, N, K);
    return false;
  }
  if (K % kGroup != 0) {
    *st = fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: K=%d is not a multiple of 64", who, K);
    return false;
  }
  if (rank < 0 || rank > N || rank > K || rank > SVDQ_MAX_RANK) {
    *st = fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: rank=%d outside [0, min(N=%d, K=%d, %d)]", who,
               rank, N, K, SVDQ_MAX_RANK);
    return false;
  }
  if ((int64_t)N * K > (int64_t)1 << 31) {
    *st = fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: N*K=%lld exceeds 2^31", who,
               (long long)N * K);
    return false;
  }
  return true;
}

static bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static void copy_unless_same(void *dst, const void *src, size_t bytes) {
  if (dst != src && bytes) std::memmove(dst, src, bytes);
}

// Shared checks and the factor merge of svdq_merge_lora / svdq_mx_merge_lora.
template <typename HW>
static svdq_status_t merge_lora_checked(const HW *in, const uint16_t *A, const uint16_t *B, int r2,
                                        float alpha, HW *out, const char *who) {
  svdq_status_t st;
  if (!in || !out) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: NULL weights", who);
  if (r2 < 0) return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: lora_rank=%d < 0", who, r2);
  if (r2 > 0 && (!A || !B)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: NULL LoRA factor", who);
  const int N = in->N, K = in->K, r = in->rank;
  if (!shape_ok(N, K, r, who, &st)) return st;
  if (r + r2 > SVDQ_MAX_RANK || r + r2 > N || r + r2 > K)
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: merged rank %d + %d outside [0, min(N=%d, K=%d, %d)]",
                who, r, r2, N, K, SVDQ_MAX_RANK);
  if (!in->inv_lambda || !in->qweight || !in->wscales || !in->bias || (r > 0 && (!in->l1s || !in->l2)))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: NULL input buffer", who);
  const int rt = r + r2;
  if (!out->inv_lambda || !out->qweight || !out->wscales || !out->bias ||
      (rt > 0 && (!out->l1s || !out->l2)))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: NULL output buffer", who);
  const size_t f_in = 2 * (size_t)K * r, u_in = 2 * (size_t)r * N;
  const size_t f_out = 2 * (size_t)K * rt, u_out = 2 * (size_t)rt * N;
  if (overlaps(out->l1s, f_out, in->l1s, f_in) || overlaps(out->l1s, f_out, in->l2, u_in) ||
      overlaps(out->l2, u_out, in->l1s, f_in) || overlaps(out->l2, u_out, in->l2, u_in) ||
      overlaps(out->l1s, f_out, out->l2, u_out))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: output factors overlap the input factors", who);
  st = merge_lora_factors(N, K, r, in->l1s, in->l2, A, B, r2, alpha, out->l1s, out->l2);
  if (st != SVDQ_OK) return st;
  copy_unless_same(out->inv_lambda, in->inv_lambda, sizeof(float) * (size_t)K);
  copy_unless_same(out->bias, in->bias, sizeof(float) * (size_t)N);
  copy_unless_same(out->qweight, in->qweight, (size_t)N * K / 2);
  out->N = N;
  out->K = K;
  out->rank = rt;
  return SVDQ_OK;
}

}  // namespace svdq

using namespace svdq;

extern "C" {

int svdq_abi_version(void) { return SVDQ_ABI_VERSION; }

const char *svdq_status_string(svdq_status_t s) {
  switch (s) {
    case SVDQ_OK: return "ok";
    case SVDQ_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SVDQ_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case SVDQ_ERR_NO_DEVICE: return "no HIP device";
    case SVDQ_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case SVDQ_ERR_WORKSPACE_TOO_SMALL: return "workspace or buffer too small";
    case SVDQ_ERR_NUMERICAL: return "non-finite input";
    case SVDQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *svdq_last_error(void) { return g_last_error; }

svdq_status_t svdq_host_weights_sizes(int N, int K, int rank, size_t sizes_out[6]) {
  svdq_status_t st;
  if (!sizes_out) return fail(SVDQ_ERR_INVALID_ARGUMENT, "sizes_out is NULL");
  if (!shape_ok(N, K, rank, "svdq_host_weights_sizes", &st)) return st;
  sizes_out[0] = sizeof(float) * (size_t)K;
  sizes_out[1] = 2 * (size_t)K * rank;
  sizes_out[2] = 2 * (size_t)rank * N;
  sizes_out[3] = (size_t)N * K / 2;
  sizes_out[4] = sizeof(float) * (size_t)N * (K / kGroup);
  sizes_out[5] = sizeof(float) * (size_t)N;
  return SVDQ_OK;
}

svdq_status_t svdq_calibration_absmax(const uint16_t *X, int rows, int K, float *absmax) {
  if (!X || !absmax) return fail(SVDQ_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (rows < 1 || K < 1) return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "rows=%d K=%d", rows, K);
  for (int k = 0; k < K; ++k) absmax[k] = 0.0f;
  for (int64_t i = 0; i < rows; ++i)
    for (int k = 0; k < K; ++k) {
      const float v = std::fabs(bf16_to_f32(X[i * K + k]));
      if (!std::isfinite(v)) return fail(SVDQ_ERR_NUMERICAL, "non-finite calibration value");
      if (v > absmax[k]) absmax[k] = v;
    }
  return SVDQ_OK;
}

svdq_status_t svdq_prepare_weights(const uint16_t *W, int N, int K, const float *act_absmax,
                                   const uint16_t *bias, int rank, int group_size,
                                   svdq_host_weights_t *out) {
  svdq_status_t st;
  if (!W || !out) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_prepare_weights: NULL pointer");
  if (group_size != kGroup)
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "group_size=%d (only 64 is supported)", group_size);
  if (!shape_ok(N, K, rank, "svdq_prepare_weights", &st)) return st;
  if (!out->inv_lambda || !out->qweight || !out->wscales || !out->bias ||
      (rank > 0 && (!out->l1s || !out->l2)))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_prepare_weights: NULL output buffer");
  return prepare_weights(W, N, K, act_absmax, bias, rank, out);
}

size_t svdq_device_weights_bytes(int N, int K, int rank) {
  svdq_status_t st;
  if (!shape_ok(N, K, rank, "svdq_device_weights_bytes", &st)) return 0;
  return (size_t)WeightLayout(N, K, rank).total;
}

svdq_status_t svdq_pack_device_weights(const svdq_host_weights_t *in, void *blob, size_t bytes) {
  svdq_status_t st;
  if (!in || !blob) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_pack_device_weights: NULL");
  if (!shape_ok(in->N, in->K, in->rank, "svdq_pack_device_weights", &st)) return st;
  if (in->group_size != kGroup) return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "group_size must be 64");
  if (!in->inv_lambda || !in->qweight || !in->wscales || !in->bias ||
      (in->rank > 0 && (!in->l1s || !in->l2)))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_pack_device_weights: NULL input buffer");
  return pack_device_weights(in, blob, bytes);
}

svdq_status_t svdq_merge_lora(const svdq_host_weights_t *in, const uint16_t *lora_down_bf16,
                              const uint16_t *lora_up_bf16, int lora_rank, float alpha,
                              svdq_host_weights_t *out) {
  if (in && in->group_size != kGroup)
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "svdq_merge_lora: group_size=%d (64 only)", in->group_size);
  const svdq_status_t st = merge_lora_checked(in, lora_down_bf16, lora_up_bf16, lora_rank, alpha,
                                              out, "svdq_merge_lora");
  if (st != SVDQ_OK) return st;
  copy_unless_same(out->wscales, in->wscales, sizeof(float) * (size_t)in->N * (in->K / kGroup));
  out->group_size = kGroup;
  return SVDQ_OK;
}

svdq_status_t svdq_mx_host_weights_sizes(int N, int K, int rank, size_t sizes_out[6]) {
  svdq_status_t st;
  if (!sizes_out) return fail(SVDQ_ERR_INVALID_ARGUMENT, "sizes_out is NULL");
  if (!shape_ok(N, K, rank, "svdq_mx_host_weights_sizes", &st)) return st;
  sizes_out[0] = sizeof(float) * (size_t)K;
  sizes_out[1] = 2 * (size_t)K * rank;
  sizes_out[2] = 2 * (size_t)rank * N;
  sizes_out[3] = (size_t)N * K / 2;
  sizes_out[4] = (size_t)N * (K / kMxBlock);
  sizes_out[5] = sizeof(float) * (size_t)N;
  return SVDQ_OK;
}

svdq_status_t svdq_mx_prepare_weights(const uint16_t *W, int N, int K, const float *act_absmax,
                                      const uint16_t *bias, int rank, svdq_mx_host_weights_t *out) {
  svdq_status_t st;
  if (!W || !out) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mx_prepare_weights: NULL pointer");
  if (!shape_ok(N, K, rank, "svdq_mx_prepare_weights", &st)) return st;
  if (!out->inv_lambda || !out->qweight || !out->wscales || !out->bias ||
      (rank > 0 && (!out->l1s || !out->l2)))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mx_prepare_weights: NULL output buffer");
  return prepare_weights_mx(W, N, K, act_absmax, bias, rank, out);
}

size_t svdq_mx_device_weights_bytes(int N, int K, int rank) {
  svdq_status_t st;
  if (!shape_ok(N, K, rank, "svdq_mx_device_weights_bytes", &st)) return 0;
  return (size_t)MxWeightLayout(N, K, rank).total;
}

svdq_status_t svdq_mx_pack_device_weights(const svdq_mx_host_weights_t *in, void *blob, size_t bytes) {
  svdq_status_t st;
  if (!in || !blob) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mx_pack_device_weights: NULL");
  if (!shape_ok(in->N, in->K, in->rank, "svdq_mx_pack_device_weights", &st)) return st;
  if (!in->inv_lambda || !in->qweight || !in->wscales || !in->bias ||
      (in->rank > 0 && (!in->l1s || !in->l2)))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mx_pack_device_weights: NULL input buffer");
  return pack_device_weights_mx(in, blob, bytes);
}

svdq_status_t svdq_mx_merge_lora(const svdq_mx_host_weights_t *in, const uint16_t *lora_down_bf16,
                                 const uint16_t *lora_up_bf16, int lora_rank, float alpha,
                                 svdq_mx_host_weights_t *out) {
  const svdq_status_t st = merge_lora_checked(in, lora_down_bf16, lora_up_bf16, lora_rank, alpha,
                                              out, "svdq_mx_merge_lora");
  if (st != SVDQ_OK) return st;
  copy_unless_same(out->wscales, in->wscales, (size_t)in->N * (in->K / kMxBlock));
  return SVDQ_OK;
}

size_t svdq_mx_workspace_bytes(int M, int N, int K, int rank) {
  svdq_status_t st;
  if (M < 1 || !shape_ok(N, K, rank, "svdq_mx_workspace_bytes", &st)) return 0;
  return (size_t)MxWorkLayout(M, K, rank).total;
}

size_t svdq_workspace_bytes(int M, int N, int K, int rank) {
  svdq_status_t st;
  if (M < 1 || !shape_ok(N, K, rank, "svdq_workspace_bytes", &st)) return 0;
  return (size_t)(WorkLayout(M, K, rank).total + k2_split_bytes(M, N, K));
}

svdq_status_t awq_quantize_weights(const uint16_t *W, int N, int K, int group_size, uint8_t *q,
                                   uint16_t *s, uint16_t *z) {
  svdq_status_t st;
  if (!W || !q || !s || !z) return fail(SVDQ_ERR_INVALID_ARGUMENT, "awq_quantize_weights: NULL");
  if (group_size != kGroup) return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "group_size must be 64");
  if (!shape_ok(N, K, 0, "awq_quantize_weights", &st)) return st;
  return awq_quantize(W, N, K, q, s, z);
}

size_t awq_device_weights_bytes(int N, int K) {
  svdq_status_t st;
  if (!shape_ok(N, K, 0, "awq_device_weights_bytes", &st)) return 0;
  return (size_t)AwqLayout(N, K).total;
}

svdq_status_t awq_pack_device_weights(const uint8_t *q, const uint16_t *s, const uint16_t *z,
                                      int N, int K, void *blob, size_t bytes) {
  svdq_status_t st;
  if (!q || !s || !z || !blob) return fail(SVDQ_ERR_INVALID_ARGUMENT, "awq_pack: NULL");
  if (!shape_ok(N, K, 0, "awq_pack_device_weights", &st)) return st;
  return awq_pack(q, s, z, N, K, blob, bytes);
}

}  // extern "C"
