// Offline preparation (host): smoothing factors, top-r low-rank split,
// residual quantisation, device packing; AWQ round-to-nearest quantiser.
//
// This file is compiled with -ffp-contract=off: every float32 step below is
// one IEEE operation, so the scales and codes are reproducible bit for bit.
#include "host_prepare.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "common.h"
#include "host_linalg.h"
#include "host_threads.h"
#include "layout.h"

namespace svdq {

// ------------------------------------------------------------ conversions
// s = p0 + p1 + p2 exactly, each a bf16: p0 is s with the low 16 bits of
// its encoding cleared, p1 the same of the remainder, p2 the rest (at most
// 8 significant bits).  Every subtraction is exact.
void split_scale_bf16x3(float s, uint16_t p[3]) {
  uint32_t u;
  std::memcpy(&u, &s, 4);
  float a1, r, a2, a3;
  const uint32_t u1 = u & 0xFFFF0000u;
  std::memcpy(&a1, &u1, 4);
  r = s - a1;
  uint32_t ur;
  std::memcpy(&ur, &r, 4);
  const uint32_t u2 = ur & 0xFFFF0000u;
  std::memcpy(&a2, &u2, 4);
  a3 = r - a2;
  uint32_t u3;
  std::memcpy(&u3, &a3, 4);
  p[0] = (uint16_t)(u >> 16);
  p[1] = (uint16_t)(ur >> 16);
  p[2] = (uint16_t)(u3 >> 16);
}

float f16_to_f32(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000) << 16;
  const uint32_t e = (h >> 10) & 0x1F, m = h & 0x3FF;
  if (e == 0) {
    float f = (float)m * (1.0f / 16777216.0f);   // m * 2^-24, exact
    return sign ? -f : f;
  }
  if (e == 31) return f32_from_bits(sign | 0x7F800000u | (m << 13));
  return f32_from_bits(sign | ((e - 15 + 127) << 23) | (m << 13));
}

uint16_t f32_to_f16(float f) {
  const uint32_t x = f32_bits(f);
  const uint16_t sign = (uint16_t)((x >> 16) & 0x8000);
  const uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return sign | 0x7C00 | (ax > 0x7F800000u ? 0x200 : 0);
  if (ax >= 0x477FF000u) return sign | 0x7C00;                 // rounds past 65504
  if (ax < 0x38800000u) {                                      // below 2^-14: subnormal
    const float a = f32_from_bits(ax) * 16777216.0f;           // * 2^24, exact
    return sign | (uint16_t)std::nearbyint(a);                 // 1024 encodes 2^-14
  }
  uint32_t h = (((ax >> 23) - 127 + 15) << 10) | ((ax & 0x7FFFFFu) >> 13);
  const uint32_t rem = ax & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
  return sign | (uint16_t)h;
}

uint16_t f64_to_bf16(double x) {
  if (x == 0.0) return std::signbit(x) ? 0x8000 : 0;
  int e;
  std::frexp(x, &e);                                  // x = m 2^e, 0.5 <= |m| < 1
  const double q = std::ldexp(1.0, std::max(e - 8, -133));
  const double r = std::nearbyint(x / q) * q;         // x / q exact; ties to even
  return (uint16_t)(f32_bits((float)r) >> 16);        // r is a bf16 value
}

// ------------------------------------------------------- user LoRA merge
svdq_status_t merge_lora_factors(int N, int K, int rank, const uint16_t *l1s, const uint16_t *l2,
                                 const uint16_t *A, const uint16_t *B, int r2, float alpha,
                                 uint16_t *l1s_out, uint16_t *l2_out) {
  const int rt = rank + r2;
  if (!std::isfinite(alpha))
    return fail(SVDQ_ERR_NUMERICAL, "svdq_merge_lora: alpha is not finite");
  for (int64_t i = 0; i < (int64_t)r2 * K; ++i)
    if (!std::isfinite(bf16_to_f32(A[i])))
      return fail(SVDQ_ERR_NUMERICAL, "svdq_merge_lora: non-finite LoRA down factor");
  // the scaled up factor first, so that nothing is written on failure
  std::vector<uint16_t> up((size_t)r2 * N);
  for (int n = 0; n < N; ++n)
    for (int j = 0; j < r2; ++j) {
      const float p = alpha * bf16_to_f32(B[(int64_t)n * r2 + j]);   // one fp32 product
      if (!std::isfinite(p))
        return fail(SVDQ_ERR_NUMERICAL, "svdq_merge_lora: alpha * up factor is not finite");
      up[(size_t)j * N + n] = f64_to_bf16((double)p);                // exact widening, one rounding
    }
  for (int k = 0; k < K; ++k) {
    uint16_t *row = l1s_out + (int64_t)k * rt;
    for (int t = 0; t < rank; ++t) row[t] = l1s[(int64_t)k * rank + t];
    for (int j = 0; j < r2; ++j) row[rank + j] = A[(int64_t)j * K + k];
  }
  if (rank > 0) std::memcpy(l2_out, l2, sizeof(uint16_t) * (size_t)rank * N);
  if (r2 > 0) std::memcpy(l2_out + (size_t)rank * N, up.data(), sizeof(uint16_t) * up.size());
  return SVDQ_OK;
}

// --------------------------------------------------------- group quantiser
void quantize_group64(const float *v, int8_t *q, float *s) {
  float a = 0.0f;
  for (int i = 0; i < kGroup; ++i) a = std::max(a, std::fabs(v[i]));
  if (!(a >= 0x1p-100f)) {
    *s = 0.0f;
    std::memset(q, 0, kGroup);
    return;
  }
  *s = a / 7.0f;
  const float inv = 7.0f / a;
  for (int i = 0; i < kGroup; ++i) {
    float t = std::rint(v[i] * inv);
    t = std::min(7.0f, std::max(-7.0f, t));
    q[i] = (int8_t)t;
  }
}

// ------------------------------------------------------ MXFP4 quantiser
// One block of 32 float32 values in OCP MXFP4 (the FP4 form of the 4-bit
// path): the shared scale is 2^e with e = floor(log2(max |v|)) - 2 (2 is the
// largest exponent of FP4 E2M1), clamped to [-127, 127], -127 for an
// all-zero block, stored biased by 127 (E8M0); each value v / 2^e is
// rounded to the nearest E2M1 value (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
// ties to an even mantissa bit; saturating at 6); zero is +0.
uint8_t e2m1_code(float r) {
  const float m = std::fabs(r);
  const int idx = (m > 0.25f) + (m >= 0.75f) + (m > 1.25f) + (m >= 1.75f) + (m > 2.5f) +
                  (m >= 3.5f) + (m > 5.0f);
  return (uint8_t)((r < 0.0f && idx > 0 ? 8 : 0) | idx);
}

void quantize_block32_mx(const float *v, uint8_t *codes, uint8_t *e8m0) {
  float a = 0.0f;
  for (int i = 0; i < kMxBlock; ++i) a = std::max(a, std::fabs(v[i]));
  int e = -127;
  if (a > 0.0f) {
    int f;
    std::frexp(a, &f);                       // a = m 2^f, 0.5 <= m < 1
    e = std::min(127, std::max(-127, f - 1 - 2));
  }
  *e8m0 = (uint8_t)(e + 127);
  for (int i = 0; i < kMxBlock; ++i)
    codes[i] = e2m1_code((float)std::ldexp((double)v[i], -e));   // exact: a power-of-two scaling
}

// ---------------------------------------------------------------- prepare
// The offline steps shared by both 4-bit encodings: smoothing factors, the
// low-rank split of the smoothed weight and the residual against the
// rounded factors, whose rows (float32) go to `emit(n, row)`.
template <class Emit>
static svdq_status_t prepare_common(const uint16_t *W_bf16, int N, int K, const float *act_absmax,
                                    const uint16_t *bias_bf16, int rank, float *inv_lambda,
                                    uint16_t *l1s, uint16_t *l2, float *bias, Emit emit) {
  const int64_t NK = (int64_t)N * K;
  std::vector<float> W((size_t)NK);
  bool finite = true;
  for (int64_t i = 0; i < NK; ++i) {
    W[i] = bf16_to_f32(W_bf16[i]);
    if (!std::isfinite(W[i])) finite = false;
  }
  if (!finite) return fail(SVDQ_ERR_NUMERICAL, "non-finite value in W");
  if (act_absmax)
    for (int k = 0; k < K; ++k)
      if (!std::isfinite(act_absmax[k]) || act_absmax[k] < 0.0f)
        return fail(SVDQ_ERR_NUMERICAL, "act_absmax[%d] is negative or non-finite", k);
  if (bias_bf16)
    for (int n = 0; n < N; ++n)
      if (!std::isfinite(bf16_to_f32(bias_bf16[n])))
        return fail(SVDQ_ERR_NUMERICAL, "non-finite bias[%d]", n);

  // 1. smoothing factors (float32)
  std::vector<float> lam(K, 1.0f), iota(K, 1.0f);
  if (act_absmax) {
    std::vector<float> aw(K, 0.0f);
    for (int64_t n = 0; n < N; ++n)
      for (int k = 0; k < K; ++k) aw[k] = std::max(aw[k], std::fabs(W[n * K + k]));
    const float floor_ = 1e-5f;
    for (int k = 0; k < K; ++k) {
      const float ratio = std::max(act_absmax[k], floor_) / std::max(aw[k], floor_);
      lam[k] = std::sqrt(ratio);
      iota[k] = 1.0f / lam[k];
    }
  }
  std::memcpy(inv_lambda, iota.data(), sizeof(float) * K);

  // 2. smoothed weight (float64, exact) and its top-r SVD
  std::vector<double> What((size_t)NK);
  parallel_for(N, 64, [&](int64_t n0, int64_t n1) {
    for (int64_t n = n0; n < n1; ++n)
      for (int k = 0; k < K; ++k) What[n * K + k] = (double)W[n * K + k] * (double)lam[k];
  });
  std::vector<double> L1s((size_t)K * std::max(rank, 1), 0.0), L2((size_t)rank * N, 0.0);
  if (rank > 0) {
    std::vector<double> U((size_t)N * rank), sig(rank), V((size_t)K * rank);
    if (svd_top(What.data(), N, K, rank, U.data(), sig.data(), V.data()) != 0)
      return fail(SVDQ_ERR_NUMERICAL, "eigensolver produced a non-finite value");
    for (int t = 0; t < rank; ++t) {
      const double root = std::sqrt(sig[t]);
      for (int k = 0; k < K; ++k) {
        const double l1 = V[(int64_t)k * rank + t] * root;
        const uint16_t b = f64_to_bf16((double)iota[k] * l1);
        l1s[(int64_t)k * rank + t] = b;
        L1s[(int64_t)k * rank + t] = (double)bf16_to_f32(b);
      }
      for (int n = 0; n < N; ++n) {
        const uint16_t b = f64_to_bf16(root * U[(int64_t)n * rank + t]);
        l2[(int64_t)t * N + n] = b;
        L2[(int64_t)t * N + n] = (double)bf16_to_f32(b);
      }
    }
  }

  // 3. residual against the rounded factors, float64 -> float32, one row at
  //    a time to the 4-bit encoder
  parallel_for(N, 16, [&](int64_t n0, int64_t n1) {
    std::vector<float> row(K);
    std::vector<double> l2n(std::max(rank, 1));
    for (int64_t n = n0; n < n1; ++n) {
      for (int t = 0; t < rank; ++t) l2n[t] = L2[(int64_t)t * N + n];
      for (int k = 0; k < K; ++k) {
        double s = 0.0;
        const double *l1 = &L1s[(int64_t)k * rank];
        for (int t = 0; t < rank; ++t) s += l1[t] * l2n[t];
        const double branch = s * (double)lam[k];
        row[k] = (float)(What[n * K + k] - branch);
      }
      emit(n, row.data());
    }
  });
  for (int n = 0; n < N; ++n) bias[n] = bias_bf16 ? bf16_to_f32(bias_bf16[n]) : 0.0f;
  return SVDQ_OK;
}

svdq_status_t prepare_weights(const uint16_t *W_bf16, int N, int K, const float *act_absmax,
                              const uint16_t *bias_bf16, int rank, svdq_host_weights_t *out) {
  const int G = K / kGroup;
  svdq_status_t st = prepare_common(
      W_bf16, N, K, act_absmax, bias_bf16, rank, out->inv_lambda, out->l1s, out->l2, out->bias,
      [&](int64_t n, const float *row) {
        int8_t q[kGroup];
        for (int g = 0; g < G; ++g) {
          float sc;
          quantize_group64(&row[g * kGroup], q, &sc);
          out->wscales[n * G + g] = sc;
          uint8_t *dst = out->qweight + n * (K / 2) + g * (kGroup / 2);
          for (int j = 0; j < kGroup / 2; ++j)
            dst[j] = (uint8_t)(((uint8_t)q[2 * j] & 0x0F) | (((uint8_t)q[2 * j + 1] & 0x0F) << 4));
        }
      });
  if (st != SVDQ_OK) return st;
  out->N = N;
  out->K = K;
  out->rank = rank;
  out->group_size = kGroup;
  return SVDQ_OK;
}

svdq_status_t prepare_weights_mx(const uint16_t *W_bf16, int N, int K, const float *act_absmax,
                                 const uint16_t *bias_bf16, int rank, svdq_mx_host_weights_t *out) {
  const int B = K / kMxBlock;
  svdq_status_t st = prepare_common(
      W_bf16, N, K, act_absmax, bias_bf16, rank, out->inv_lambda, out->l1s, out->l2, out->bias,
      [&](int64_t n, const float *row) {
        uint8_t q[kMxBlock];
        for (int b = 0; b < B; ++b) {
          quantize_block32_mx(&row[b * kMxBlock], q, &out->wscales[n * B + b]);
          uint8_t *dst = out->qweight + n * (K / 2) + b * (kMxBlock / 2);
          for (int j = 0; j < kMxBlock / 2; ++j) dst[j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
        }
      });
  if (st != SVDQ_OK) return st;
  out->N = N;
  out->K = K;
  out->rank = rank;
  return SVDQ_OK;
}

// ------------------------------------------------------------ device pack
svdq_status_t pack_device_weights(const svdq_host_weights_t *in, void *host_blob, size_t bytes) {
  const WeightLayout L(in->N, in->K, in->rank);
  if ((int64_t)bytes < L.total)
    return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "blob needs %lld bytes, got %zu",
                (long long)L.total, bytes);
  uint8_t *b = static_cast<uint8_t *>(host_blob);
  std::memset(b, 0, (size_t)L.total);
  const int64_t N = in->N, K = in->K, r = in->rank, T = L.Np / kTile;
  // fp6 codes: for every (group, tile, lane) the lane's 32 codes as 6-bit
  // fields of a 192-bit word string, stored as three 8-byte word pairs
  uint8_t *q = b + L.q;
  const int64_t G = L.G;
  parallel_for(T, 1, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; ++t)
      for (int64_t g = 0; g < G; ++g)
        for (int lane = 0; lane < 64; ++lane) {
          const int64_t n = t * kTile + (lane & 31);
          const int h = lane >> 5;
          uint32_t w[6] = {0, 0, 0, 0, 0, 0};
          if (n < N)
            for (int c = 0; c < 32; ++c) {
              const int64_t k = g * kGroup + lane_code_k(h, c);
              const uint8_t byte = in->qweight[n * (K / 2) + k / 2];
              const int code = (k & 1) ? ((int8_t)byte >> 4) : ((int8_t)(byte << 4) >> 4);
              const uint32_t v = e2m3_of_int(code);
              const int bit = 6 * c;
              w[bit / 32] |= v << (bit % 32);
              if (bit % 32 > 26) w[bit / 32 + 1] |= v >> (32 - bit % 32);
            }
          for (int j = 0; j < 3; ++j)
            std::memcpy(q + pair_offset(g, t, T, lane, j), &w[2 * j], 8);
        }
  });
  // weight scales as the column operand of the GEMM's scale product:
  // b1 b2 b3 b1 b2 b3 b1 b2 (bf16), s = b1 + b2 + b3 exactly (layout.h)
  uint16_t *s = reinterpret_cast<uint16_t *>(b + L.s);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < L.G; ++g) {
      uint16_t p[3];
      split_scale_bf16x3(in->wscales[n * L.G + g], p);
      uint16_t *o = s + (g * L.Np + n) * (kScaleOpBytes / 2);
      const int order[8] = {0, 1, 2, 0, 1, 2, 0, 1};
      for (int e = 0; e < 8; ++e) o[e] = p[order[e]];
    }
  uint16_t *l2t = reinterpret_cast<uint16_t *>(b + L.l2t);
  uint16_t *l1t = reinterpret_cast<uint16_t *>(b + L.l1t);
  for (int64_t t = 0; t < r; ++t) {
    for (int64_t n = 0; n < N; ++n) l2t[n * L.rp + t] = in->l2[t * N + n];
    for (int64_t k = 0; k < K; ++k) l1t[l1_frag_index(k, t, L.rp)] = in->l1s[k * r + t];
  }
  std::memcpy(b + L.iota, in->inv_lambda, sizeof(float) * K);
  std::memcpy(b + L.bias, in->bias, sizeof(float) * N);
  return SVDQ_OK;
}

// --------------------------------------------------------- MXFP4 pack
svdq_status_t pack_device_weights_mx(const svdq_mx_host_weights_t *in, void *host_blob, size_t bytes) {
  const MxWeightLayout L(in->N, in->K, in->rank);
  if ((int64_t)bytes < L.total)
    return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "blob needs %lld bytes, got %zu",
                (long long)L.total, bytes);
  uint8_t *b = static_cast<uint8_t *>(host_blob);
  std::memset(b, 0, (size_t)L.total);
  const int64_t N = in->N, K = in->K, r = in->rank, T = L.Np / kTile, G = L.G;
  // lane l of block (s, t): row 32 t + l % 32, the row's canonical bytes
  // 32 s + 16 (l / 32) + [0, 16) and the scale of MX block 2 s + l / 32;
  // padding rows stay zero (codes +0, scales 2^-127)
  uint8_t *q = b + L.q, *sc = b + L.s;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t g = 0; g < G; ++g)
      for (int lane = 0; lane < 64; ++lane) {
        const int64_t n = t * kTile + (lane & 31);
        if (n >= N) continue;
        const int h = lane >> 5;
        std::memcpy(q + mx_code_offset(g, t, T, lane), in->qweight + n * (K / 2) + 32 * g + 16 * h, 16);
        sc[mx_scale_offset(g, t, T, lane)] = in->wscales[n * (K / kMxBlock) + 2 * g + h];
      }
  uint16_t *l2t = reinterpret_cast<uint16_t *>(b + L.l2t);
  uint16_t *l1t = reinterpret_cast<uint16_t *>(b + L.l1t);
  for (int64_t t = 0; t < r; ++t) {
    for (int64_t n = 0; n < N; ++n) l2t[n * L.rp + t] = in->l2[t * N + n];
    for (int64_t k = 0; k < K; ++k) l1t[l1_frag_index(k, t, L.rp)] = in->l1s[k * r + t];
  }
  std::memcpy(b + L.iota, in->inv_lambda, sizeof(float) * K);
  std::memcpy(b + L.bias, in->bias, sizeof(float) * N);
  return SVDQ_OK;
}

// ------------------------------------------------------------------- AWQ
svdq_status_t awq_quantize(const uint16_t *W_fp16, int N, int K, uint8_t *q, uint16_t *s,
                           uint16_t *z) {
  const int G = K / kGroup;
  for (int64_t i = 0; i < (int64_t)N * K; ++i)
    if (!std::isfinite(f16_to_f32(W_fp16[i])))
      return fail(SVDQ_ERR_NUMERICAL, "non-finite weight at %lld", (long long)i);
  parallel_for(N, 64, [&](int64_t n0, int64_t n1) {
    float w[kGroup];
    for (int64_t n = n0; n < n1; ++n)
      for (int g = 0; g < G; ++g) {
        float wmax = -INFINITY, wmin = INFINITY;
        for (int i = 0; i < kGroup; ++i) {
          w[i] = f16_to_f32(W_fp16[n * K + g * kGroup + i]);
          wmax = std::max(wmax, w[i]);
          wmin = std::min(wmin, w[i]);
        }
        const float range = std::max(wmax - wmin, 1e-5f);
        const uint16_t s16 = f32_to_f16(range / 15.0f);
        const float sc = f16_to_f32(s16);
        const float zf = std::min(15.0f, std::max(0.0f, std::rint(-wmin / sc)));
        s[n * G + g] = s16;
        z[n * G + g] = f32_to_f16(zf);
        uint8_t *dst = q + n * (K / 2) + g * (kGroup / 2);
        for (int j = 0; j < kGroup / 2; ++j) {
          const float a = std::min(15.0f, std::max(0.0f, std::rint(w[2 * j] / sc) + zf));
          const float c = std::min(15.0f, std::max(0.0f, std::rint(w[2 * j + 1] / sc) + zf));
          dst[j] = (uint8_t)((uint8_t)a | ((uint8_t)c << 4));
        }
      }
  });
  return SVDQ_OK;
}

svdq_status_t awq_pack(const uint8_t *q, const uint16_t *s, const uint16_t *z, int N, int K,
                       void *host_blob, size_t bytes) {
  const AwqLayout L(N, K);
  if ((int64_t)bytes < L.total)
    return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "blob needs %lld bytes, got %zu",
                (long long)L.total, bytes);
  // The kernel forms q - z exactly as (1024 + q) - (1024 + z) in fp16, which
  // holds only for integer zero points 0..15; scales must be finite.
  for (int64_t i = 0; i < (int64_t)N * L.G; ++i) {
    const float zf = f16_to_f32(z[i]), sf = f16_to_f32(s[i]);
    if (!(zf >= 0.0f && zf <= 15.0f && zf == std::floor(zf)))
      return fail(SVDQ_ERR_INVALID_ARGUMENT, "awq_pack_device_weights: zero point %g at (%lld, %lld) is not an integer in 0..15",
                  (double)zf, (long long)(i / L.G), (long long)(i % L.G));
    if (!std::isfinite(sf))
      return fail(SVDQ_ERR_NUMERICAL, "awq_pack_device_weights: non-finite scale at (%lld, %lld)",
                  (long long)(i / L.G), (long long)(i % L.G));
  }
  uint8_t *b = static_cast<uint8_t *>(host_blob);
  std::memset(b, 0, (size_t)L.total);
  uint8_t *qd = b + L.q;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const uint8_t byte = q[n * (K / 2) + k / 2];
      const uint8_t code = (k & 1) ? (byte >> 4) : (byte & 0x0F);
      qd[awq_code_byte(n, k, L.G)] |= (uint8_t)(code << awq_code_shift(k));
    }
  uint32_t *sz = reinterpret_cast<uint32_t *>(b + L.sz);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t g = 0; g < L.G; ++g)
      sz[n * awq_g4(L.G) + g] = (uint32_t)s[n * L.G + g] | ((uint32_t)z[n * L.G + g] << 16);
  return SVDQ_OK;
}

}  // namespace svdq
