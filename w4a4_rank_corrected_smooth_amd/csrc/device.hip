// Device half of libsvdq: gfx950 kernels and the asynchronous entry points.
//
//  K1  k1_quantize_lowrank_down  smoothing, per-group INT4 activation codes
//                                and scales, low-rank down-projection D = X L1s
//  K2  k2_w4a4_gemm              INT4 x INT4 group GEMM on int8 MFMA, fp32
//                                per-group scaling, + D L2 + bias (+ GELU)
//  K3  k3_awq_w4a16              AWQ W4A16 GEMV/GEMM on fp16 MFMA
//  +   GELU glue kernel and canonical-layout inspection kernels.
//
// "Bringing Nunchaku 4-bit diffusion inference to Diffusers" (Korean
// edition, section "SVDQuant 및 Nunchaku 엔진") places the low-rank
// down-projection beside activation quantisation and the up-projection
// inside the 4-bit GEMM so the 16-bit branch costs no extra memory pass;
// K1 and K2 follow that split.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "common.h"
#include "layout.h"

using namespace svdq;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ small helpers
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

// tanh-form GELU, 0.5 y (1 + tanh u) with u = sqrt(2/pi) (y + 0.044715 y^3),
// evaluated as y / (1 + exp(-2u)) (the same function) so that large negative
// y keep their relative accuracy instead of cancelling in 1 + tanh(u).  The
// hardware exp2 and reciprocal (about 1 ulp of fp32 each) are far inside the
// half-ulp of the bf16 result; exp overflow gives 1/inf = 0, the right limit.
__device__ __forceinline__ float gelu_tanh_f32(float y) {
  const float k0 = 0.7978845608028654f;   // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float u = k0 * (y + k1 * y * y * y);
  return y * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * u));
}

// ======================================================================= K1
// One workgroup (4 wavefronts) per (tile of 32 token rows, K split).  Lane l
// of a wavefront owns row l % 32 and half h = l / 32 of each group: 32 bf16
// values read as four 16-byte loads.  The four wavefronts interleave groups.
// Per group:  x_hat = fl32(x * iota);  a = max |x_hat| over 64 (two lanes);
// s = a / 7, inv = 7 / a (correctly rounded), q = clamp(rint(x_hat inv), +-7).
// The raw bf16 values also feed a 32x32x16 bf16 MFMA against L1s^T, giving
// the low-rank down-projection; the four wavefronts' partial products are
// summed through LDS and written as this split's partial D.
template <int TB>   // rank_pad / 32
__global__ __launch_bounds__(256) void k1_quantize_lowrank_down(
    const uint16_t *__restrict__ X, int M, int K, int Mp, int S,
    const float *__restrict__ iota, const uint16_t *__restrict__ l1t,
    int8_t *__restrict__ qa, float *__restrict__ sa, float *__restrict__ dpart) {
  const int t = blockIdx.x, s = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = K / kGroup, Gs = G / S, T = Mp / kTile;
  const int row = t * kTile + (lane & 31), h = lane >> 5;
  const bool valid = row < M;
  constexpr int NB = TB > 0 ? TB : 1;
  v16f dacc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dacc[b] = v16f{};

  for (int gi = w; gi < Gs; gi += 4) {
    const int g = s * Gs + gi;
    uint4 xr[4];
    const uint16_t *xp = X + (int64_t)row * K + g * kGroup + 8 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xr[j] = valid ? *reinterpret_cast<const uint4 *>(xp + 16 * j) : make_uint4(0, 0, 0, 0);
    float xh[32];
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 i0 = *reinterpret_cast<const float4 *>(iota + g * kGroup + 16 * j + 8 * h);
      const float4 i1 = *reinterpret_cast<const float4 *>(iota + g * kGroup + 16 * j + 8 * h + 4);
      const uint32_t wv[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
      const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (e & 1) ? bf16_hi(wv[e >> 1]) : bf16_lo(wv[e >> 1]);
        const float v = __fmul_rn(x, iv[e]);
        xh[8 * j + e] = v;
        a = fmaxf(a, fabsf(v));
      }
    }
    a = fmaxf(a, __shfl_xor(a, 32));
    float sc = 0.0f, inv = 0.0f;
    if (a >= 0x1p-100f) {
      sc = a / 7.0f;
      inv = 7.0f / a;
    }
    int8_t *qp = qa + code_offset(g, t, T, lane, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float qf = rintf(__fmul_rn(xh[8 * j + e], inv));
        qf = fminf(7.0f, fmaxf(-7.0f, qf));
        const uint32_t byte = (uint32_t)(int32_t)qf & 0xFFu;
        if (e < 4) lo |= byte << (8 * e);
        else hi |= byte << (8 * (e - 4));
      }
      *reinterpret_cast<uint2 *>(qp + 512 * j) = make_uint2(lo, hi);
    }
    if (h == 0) sa[(int64_t)g * Mp + row] = sc;
    if constexpr (TB > 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8bf av = as_v8bf(xr[j]);
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const uint4 lw = *reinterpret_cast<const uint4 *>(
              l1t + (int64_t)(b * 32 + (lane & 31)) * K + g * kGroup + 16 * j + 8 * h);
          dacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, as_v8bf(lw), dacc[b], 0, 0, 0);
        }
      }
    }
  }
  if constexpr (TB > 0) {
    __shared__ float red[4][16][64];
    constexpr int RP = TB * 32;
    for (int b = 0; b < TB; ++b) {
#pragma unroll
      for (int e = 0; e < 16; ++e) red[w][e][lane] = dacc[b][e];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * w + i;
        const float v = red[0][e][lane] + red[1][e][lane] + red[2][e][lane] + red[3][e][lane];
        const int r = t * kTile + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        dpart[((int64_t)s * Mp + r) * RP + b * 32 + (lane & 31)] = v;
      }
      __syncthreads();
    }
  }
}

// ======================================================================= K2
// Output tile 128 x 128 per workgroup, 64 x 64 per wavefront (2 x 2 MFMA tiles
// of 32 x 32).  For each group g: the int32 group sums P of every 32 x 32 tile
// come from two v_mfma_i32_32x32x32_i8 (K = 32 each) on the int8 codes; then
// acc += (sA[m,g] * sW[n,g]) * float(P) in fp32.  The epilogue adds the
// low-rank up-projection D L2 on bf16 MFMA (D split into a bf16 high part and
// a bf16 remainder, so the product keeps ~16 bits of D), the bias, the
// optional GELU, and stores bf16 or fp32.
// MODE_SUMS stores the raw int32 P of each group for a window instead.
enum { MODE_FWD = 0, MODE_SUMS = 1 };

struct K2Args {
  const int8_t *qa; const float *sa; const float *dpart; int S, M, Mp;
  const int8_t *qw; const float *sw; const uint16_t *l2t; const float *bias;
  int N, Np, K, rp;
  void *Y;
  int32_t *P; int m0, mcount, n0, ncount, tile_m0, tile_n0;
};

__device__ __forceinline__ v4i load_frag(const int8_t *blk, int lane, int half) {
  const uint2 c0 = *reinterpret_cast<const uint2 *>(blk + 1024 * half + lane * 8);
  const uint2 c1 = *reinterpret_cast<const uint2 *>(blk + 1024 * half + 512 + lane * 8);
  return v4i{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y};
}

template <int MODE, int EPI, bool OUT_F32>
__global__ __launch_bounds__(256) void k2_w4a4_gemm(K2Args p) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bm = p.tile_m0 + blockIdx.y * 128, bn = p.tile_n0 + blockIdx.x * 128;
  const int wm = bm + (w >> 1) * 64, wn = bn + (w & 1) * 64;
  const int G = p.K / kGroup, Ta = p.Mp / kTile, Tw = p.Np / kTile;
  const int hl = lane >> 5, ln = lane & 31;
  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  for (int g = 0; g < G; ++g) {
    v4i a[2][2], b[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int8_t *blk = p.qa + ((int64_t)g * Ta + wm / kTile + i) * kBlockBytes;
      a[i][0] = load_frag(blk, lane, 0);
      a[i][1] = load_frag(blk, lane, 1);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int8_t *blk = p.qw + ((int64_t)g * Tw + wn / kTile + j) * kBlockBytes;
      b[j][0] = load_frag(blk, lane, 0);
      b[j][1] = load_frag(blk, lane, 1);
    }
    float sw[2];
    float4 sa[2][4];
    if constexpr (MODE == MODE_FWD) {
#pragma unroll
      for (int j = 0; j < 2; ++j) sw[j] = p.sw[(int64_t)g * p.Np + wn + 32 * j + ln];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          sa[i][q] = *reinterpret_cast<const float4 *>(p.sa + (int64_t)g * p.Mp + wm + 32 * i +
                                                       8 * q + 4 * hl);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        v16i P = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i][0], b[j][0], v16i{}, 0, 0, 0);
        P = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i][1], b[j][1], P, 0, 0, 0);
        if constexpr (MODE == MODE_SUMS) {
          const int n = wn + 32 * j + ln;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = wm + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
            if (m >= p.m0 && m < p.m0 + p.mcount && n >= p.n0 && n < p.n0 + p.ncount)
              p.P[((int64_t)(m - p.m0) * p.ncount + (n - p.n0)) * G + g] = P[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float4 s4 = sa[i][e >> 2];
            const float sae = (e & 3) == 0 ? s4.x : (e & 3) == 1 ? s4.y : (e & 3) == 2 ? s4.z : s4.w;
            acc[i][j][e] = __builtin_fmaf((float)P[e], __fmul_rn(sae, sw[j]), acc[i][j][e]);
          }
        }
      }
  }
  if constexpr (MODE == MODE_FWD) {
    // low-rank up-projection: acc += D L2, D summed over the K1 splits
    for (int c = 0; c < p.rp / 16; ++c) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm + 32 * i + ln;
        float d[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int s = 0; s < p.S; ++s) {
          const float *dp = p.dpart + ((int64_t)s * p.Mp + r) * p.rp + 16 * c + 8 * hl;
          const float4 d0 = *reinterpret_cast<const float4 *>(dp);
          const float4 d1 = *reinterpret_cast<const float4 *>(dp + 4);
          d[0] += d0.x; d[1] += d0.y; d[2] += d0.z; d[3] += d0.w;
          d[4] += d1.x; d[5] += d1.y; d[6] += d1.z; d[7] += d1.w;
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h0 = f32_to_bf16_rne(d[2 * e]), h1 = f32_to_bf16_rne(d[2 * e + 1]);
          const uint32_t l0 = f32_to_bf16_rne(d[2 * e] - __uint_as_float(h0 << 16));
          const uint32_t l1 = f32_to_bf16_rne(d[2 * e + 1] - __uint_as_float(h1 << 16));
          hi[e] = h0 | (h1 << 16);
          lo[e] = l0 | (l1 << 16);
        }
        const v8bf ah = as_v8bf(make_uint4(hi[0], hi[1], hi[2], hi[3]));
        const v8bf al = as_v8bf(make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4 bw = *reinterpret_cast<const uint4 *>(
              p.l2t + (int64_t)(wn + 32 * j + ln) * p.rp + 16 * c + 8 * hl);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, as_v8bf(bw), acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, as_v8bf(bw), acc[i][j], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wn + 32 * j + ln;
      const float bj = p.bias[n];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = wm + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
          float y = acc[i][j][e] + bj;
          if constexpr (EPI == SVDQ_EPILOGUE_GELU_TANH) y = gelu_tanh_f32(y);
          if (m < p.M && n < p.N) {
            if constexpr (OUT_F32)
              reinterpret_cast<float *>(p.Y)[(int64_t)m * p.N + n] = y;
            else
              reinterpret_cast<uint16_t *>(p.Y)[(int64_t)m * p.N + n] = (uint16_t)f32_to_bf16_rne(y);
          }
        }
    }
  }
}

// ======================================================================= K3
// AWQ W4A16: one wavefront per tile of 16 output channels.  For each group of
// 64 input channels, lane l (channel l % 16, quarter q = l / 16) turns its 16
// codes into fp16 (q - z) with the 1024-offset trick (0x6400 | code is the
// fp16 value 1024 + code; subtracting 1024 + z is exact), the activations
// [16, 64] are the A operand, and two v_mfma_f32_16x16x32_f16 give the
// group's inner sums; acc += s * sum in fp32.  Rows m >= M are zero.
__global__ __launch_bounds__(64) void k3_awq_w4a16(const uint8_t *__restrict__ qd,
                                                    const uint32_t *__restrict__ sz,
                                                    const uint16_t *__restrict__ x, int M,
                                                    int N, int Np, int K,
                                                    const uint16_t *__restrict__ bias,
                                                    uint16_t *__restrict__ y) {
  const int lane = threadIdx.x;
  const int tile = blockIdx.x;
  const int G = K / kGroup;
  const int m = lane & 15, qtr = lane >> 4;
  const int n = tile * kAwqTile + (lane & 15);
  v4f acc = v4f{};
  for (int g = 0; g < G; ++g) {
    const uint2 cw = *reinterpret_cast<const uint2 *>(
        qd + ((int64_t)tile * G + g) * kAwqBlockBytes + lane * 8);
    const uint32_t szw = sz[(int64_t)g * Np + n];
    const _Float16 zf = __builtin_bit_cast(_Float16, (uint16_t)(szw >> 16));
    const float sf = (float)__builtin_bit_cast(_Float16, (uint16_t)(szw & 0xFFFF));
    const _Float16 off = -((_Float16)1024.0f + zf);
    const v2h off2 = v2h{off, off};
    v8h bop[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t word = half ? cw.y : cw.x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t pr = ((word >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
        const v2h v = __builtin_bit_cast(v2h, pr) + off2;
        bop[half][2 * j] = v.x;
        bop[half][2 * j + 1] = v.y;
      }
    }
    v8h aop[2];
    if (m < M) {
      const uint16_t *xp = x + (int64_t)m * K + g * kGroup + 16 * qtr;
      aop[0] = __builtin_bit_cast(v8h, *reinterpret_cast<const uint4 *>(xp));
      aop[1] = __builtin_bit_cast(v8h, *reinterpret_cast<const uint4 *>(xp + 8));
    } else {
      aop[0] = v8h{};
      aop[1] = v8h{};
    }
    v4f part = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[0], bop[0], v4f{}, 0, 0, 0);
    part = __builtin_amdgcn_mfma_f32_16x16x32_f16(aop[1], bop[1], part, 0, 0, 0);
    // output layout: lane holds rows 4 * (lane / 16) + i, column lane % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(part[i], sf, acc[i]);
  }
  const int col = tile * kAwqTile + (lane & 15);
  if (col < N) {
    const float b = bias ? (float)__builtin_bit_cast(_Float16, bias[col]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i;
      if (row < M) {
        const _Float16 o = (_Float16)(acc[i] + b);
        y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, o);
      }
    }
  }
}

// ==================================================================== GELU
__global__ __launch_bounds__(256) void gelu_tanh_bf16_kernel(const uint16_t *__restrict__ in,
                                                             uint16_t *__restrict__ out,
                                                             size_t n) {
  const size_t i8 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i8 + 8 <= n) {
    const uint4 v = *reinterpret_cast<const uint4 *>(in + i8);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a = f32_to_bf16_rne(gelu_tanh_f32(bf16_lo(wv[e])));
      const uint32_t b = f32_to_bf16_rne(gelu_tanh_f32(bf16_hi(wv[e])));
      o[e] = a | (b << 16);
    }
    *reinterpret_cast<uint4 *>(out + i8) = make_uint4(o[0], o[1], o[2], o[3]);
  } else {
    for (size_t i = i8; i < n; ++i)
      out[i] = (uint16_t)f32_to_bf16_rne(gelu_tanh_f32(__uint_as_float((uint32_t)in[i] << 16)));
  }
}

// ============================================================ inspection
__global__ void canon_codes_kernel(const int8_t *__restrict__ qa, int M, int K, int T,
                                   uint8_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nb = (int64_t)M * (K / 2);
  if (idx >= nb) return;
  const int64_t m = idx / (K / 2), kb = idx % (K / 2);
  const int8_t c0 = qa[code_offset_rk(m, 2 * kb, T)];
  const int8_t c1 = qa[code_offset_rk(m, 2 * kb + 1, T)];
  out[idx] = (uint8_t)(((uint8_t)c0 & 0x0F) | (((uint8_t)c1 & 0x0F) << 4));
}

__global__ void canon_scales_kernel(const float *__restrict__ sa, int M, int Mp, int G,
                                    float *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * G) return;
  const int64_t m = idx / G, g = idx % G;
  out[idx] = sa[g * Mp + m];
}

__global__ void canon_down_kernel(const float *__restrict__ dpart, int M, int Mp, int S, int rp,
                                  int rank, float *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * rank) return;
  const int64_t m = idx / rank, t = idx % rank;
  float v = 0.0f;
  for (int s = 0; s < S; ++s) v += dpart[((int64_t)s * Mp + m) * rp + t];
  out[idx] = v;
}

// ============================================================ host side
namespace {

std::atomic<int> g_dev_state[64];   // 0 unknown, 1 gfx950, 2 other

svdq_status_t check_device() {
  int dev = -1;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(SVDQ_ERR_NO_DEVICE, "no HIP device is visible");
  }
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(SVDQ_ERR_NO_DEVICE, "hipGetDevice failed");
  if (dev < 64) {
    const int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 1) return SVDQ_OK;
    if (st == 2) return fail(SVDQ_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(SVDQ_ERR_HIP, "hipGetDeviceProperties failed");
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_state[dev].store(ok ? 1 : 2, std::memory_order_release);
  if (!ok)
    return fail(SVDQ_ERR_UNSUPPORTED_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return SVDQ_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

svdq_status_t launch_status(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SVDQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return SVDQ_OK;
}

svdq_status_t validate_weights(const svdq_weights_t *w, const char *who) {
  if (!w || !w->blob) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: NULL weights", who);
  if (!aligned16(w->blob)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: blob not 16-byte aligned", who);
  if (w->N < 1 || w->K < 1 || w->K % kGroup != 0)
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: N=%d K=%d (K must be a multiple of 64)", who,
                w->N, w->K);
  if (w->rank < 0 || w->rank > w->N || w->rank > w->K || w->rank > SVDQ_MAX_RANK)
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: rank=%d out of range", who, w->rank);
  if ((int64_t)w->N * w->K > ((int64_t)1 << 31))
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: N*K too large", who);
  return SVDQ_OK;
}

svdq_status_t launch_k1(const WeightLayout &L, const WorkLayout &Wl, const svdq_weights_t *w,
                        const void *X, int M, uint8_t *ws, hipStream_t st) {
  const uint8_t *blob = static_cast<const uint8_t *>(w->blob);
  const dim3 grid((unsigned)(Wl.Mp / kTile), (unsigned)Wl.S);
  const uint16_t *x = static_cast<const uint16_t *>(X);
  const float *iota = reinterpret_cast<const float *>(blob + L.iota);
  const uint16_t *l1t = reinterpret_cast<const uint16_t *>(blob + L.l1t);
  int8_t *qa = reinterpret_cast<int8_t *>(ws + Wl.qa);
  float *sa = reinterpret_cast<float *>(ws + Wl.sa);
  float *dp = reinterpret_cast<float *>(ws + Wl.d);
  const int K = w->K, Mp = (int)Wl.Mp, S = (int)Wl.S;
  switch (L.rp / 32) {
#define K1_CASE(TB)                                                                       \
  case TB:                                                                                \
    hipLaunchKernelGGL(k1_quantize_lowrank_down<TB>, grid, dim3(256), 0, st, x, M, K, Mp, \
                       S, iota, l1t, qa, sa, dp);                                         \
    break;
    K1_CASE(0) K1_CASE(1) K1_CASE(2) K1_CASE(3) K1_CASE(4) K1_CASE(5) K1_CASE(6) K1_CASE(7)
    K1_CASE(8)
#undef K1_CASE
    default: return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "rank too large");
  }
  return launch_status("quantize kernel launch");
}

K2Args make_k2_args(const WeightLayout &L, const WorkLayout &Wl, const svdq_weights_t *w, int M,
                    const uint8_t *ws) {
  const uint8_t *blob = static_cast<const uint8_t *>(w->blob);
  K2Args a{};
  a.qa = reinterpret_cast<const int8_t *>(ws + Wl.qa);
  a.sa = reinterpret_cast<const float *>(ws + Wl.sa);
  a.dpart = reinterpret_cast<const float *>(ws + Wl.d);
  a.S = (int)Wl.S;
  a.M = M;
  a.Mp = (int)Wl.Mp;
  a.qw = reinterpret_cast<const int8_t *>(blob + L.q);
  a.sw = reinterpret_cast<const float *>(blob + L.s);
  a.l2t = reinterpret_cast<const uint16_t *>(blob + L.l2t);
  a.bias = reinterpret_cast<const float *>(blob + L.bias);
  a.N = w->N;
  a.Np = (int)L.Np;
  a.K = w->K;
  a.rp = (int)L.rp;
  return a;
}

}  // namespace

extern "C" {

svdq_status_t svdq_device_check(void) { return check_device(); }

static svdq_status_t validate_forward(const svdq_weights_t *w, int M, size_t ws_bytes,
                                      const void *workspace, const char *who) {
  svdq_status_t st = validate_weights(w, who);
  if (st != SVDQ_OK) return st;
  if (!workspace) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: NULL workspace", who);
  if (!aligned16(workspace)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: misaligned workspace", who);
  // grid.y of the GEMM counts 128-row tiles and is limited to 65535
  if (M < 1 || M > 65535 * 128 || (int64_t)M * w->K > ((int64_t)1 << 31))
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: M=%d", who, M);
  const WorkLayout Wl(M, w->K, w->rank);
  if ((int64_t)ws_bytes < Wl.total)
    return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %lld bytes, got %zu", who,
                (long long)Wl.total, ws_bytes);
  return SVDQ_OK;
}

static svdq_status_t validate_output(void *Y, svdq_dtype_t y_dtype, svdq_epilogue_t epilogue,
                                     const char *who) {
  if (!Y) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: NULL output", who);
  if (!aligned16(Y)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: misaligned output", who);
  if (y_dtype != SVDQ_BF16 && y_dtype != SVDQ_FP32)
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: y_dtype must be SVDQ_BF16 or SVDQ_FP32", who);
  if (epilogue != SVDQ_EPILOGUE_NONE && epilogue != SVDQ_EPILOGUE_GELU_TANH)
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: unknown epilogue %d", who, (int)epilogue);
  return SVDQ_OK;
}

static svdq_status_t launch_k2(const svdq_weights_t *w, int M, void *Y, svdq_dtype_t y_dtype,
                               svdq_epilogue_t epilogue, const void *workspace, hipStream_t stream) {
  const WeightLayout L(w->N, w->K, w->rank);
  const WorkLayout Wl(M, w->K, w->rank);
  K2Args a = make_k2_args(L, Wl, w, M, static_cast<const uint8_t *>(workspace));
  a.Y = Y;
  const dim3 grid((unsigned)((w->N + 127) / 128), (unsigned)((M + 127) / 128));
  const bool f32 = y_dtype == SVDQ_FP32;
  const bool gelu = epilogue == SVDQ_EPILOGUE_GELU_TANH;
  if (!gelu && f32)
    hipLaunchKernelGGL((k2_w4a4_gemm<MODE_FWD, SVDQ_EPILOGUE_NONE, true>), grid, dim3(256), 0, stream, a);
  else if (!gelu)
    hipLaunchKernelGGL((k2_w4a4_gemm<MODE_FWD, SVDQ_EPILOGUE_NONE, false>), grid, dim3(256), 0, stream, a);
  else if (f32)
    hipLaunchKernelGGL((k2_w4a4_gemm<MODE_FWD, SVDQ_EPILOGUE_GELU_TANH, true>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k2_w4a4_gemm<MODE_FWD, SVDQ_EPILOGUE_GELU_TANH, false>), grid, dim3(256), 0, stream, a);
  return launch_status("GEMM kernel launch");
}

svdq_status_t svdq_linear_quantize(const svdq_weights_t *w, const void *X, int M, void *workspace,
                                   size_t ws_bytes, void *hip_stream) {
  svdq_status_t st = validate_forward(w, M, ws_bytes, workspace, "svdq_linear_quantize");
  if (st != SVDQ_OK) return st;
  if (!X) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_linear_quantize: NULL X");
  if (!aligned16(X)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_linear_quantize: misaligned X");
  if ((st = check_device()) != SVDQ_OK) return st;
  const WeightLayout L(w->N, w->K, w->rank);
  const WorkLayout Wl(M, w->K, w->rank);
  return launch_k1(L, Wl, w, X, M, static_cast<uint8_t *>(workspace),
                   static_cast<hipStream_t>(hip_stream));
}

svdq_status_t svdq_linear_gemm(const svdq_weights_t *w, int M, void *Y, svdq_dtype_t y_dtype,
                               svdq_epilogue_t epilogue, const void *workspace, size_t ws_bytes,
                               void *hip_stream) {
  svdq_status_t st = validate_forward(w, M, ws_bytes, workspace, "svdq_linear_gemm");
  if (st != SVDQ_OK) return st;
  if ((st = validate_output(Y, y_dtype, epilogue, "svdq_linear_gemm")) != SVDQ_OK) return st;
  if ((st = check_device()) != SVDQ_OK) return st;
  return launch_k2(w, M, Y, y_dtype, epilogue, workspace, static_cast<hipStream_t>(hip_stream));
}

svdq_status_t svdq_linear_forward(const svdq_weights_t *w, const void *X, int M, void *Y,
                                  svdq_dtype_t y_dtype, svdq_epilogue_t epilogue,
                                  void *workspace, size_t ws_bytes, void *hip_stream) {
  svdq_status_t st = validate_forward(w, M, ws_bytes, workspace, "svdq_linear_forward");
  if (st != SVDQ_OK) return st;
  if (!X) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_linear_forward: NULL X");
  if (!aligned16(X)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_linear_forward: misaligned X");
  if ((st = validate_output(Y, y_dtype, epilogue, "svdq_linear_forward")) != SVDQ_OK) return st;
  if ((st = check_device()) != SVDQ_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const WeightLayout L(w->N, w->K, w->rank);
  const WorkLayout Wl(M, w->K, w->rank);
  if ((st = launch_k1(L, Wl, w, X, M, static_cast<uint8_t *>(workspace), stream)) != SVDQ_OK)
    return st;
  return launch_k2(w, M, Y, y_dtype, epilogue, workspace, stream);
}

svdq_status_t svdq_gelu_tanh_bf16(const void *in, void *out, size_t n, void *hip_stream) {
  if (!in || !out) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_gelu_tanh_bf16: NULL pointer");
  if (!aligned16(in) || !aligned16(out))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_gelu_tanh_bf16: pointers must be 16-byte aligned");
  if (n == 0) return SVDQ_OK;
  svdq_status_t st = check_device();
  if (st != SVDQ_OK) return st;
  const size_t threads = (n + 7) / 8;
  const dim3 grid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL(gelu_tanh_bf16_kernel, grid, dim3(256), 0, static_cast<hipStream_t>(hip_stream),
                     static_cast<const uint16_t *>(in), static_cast<uint16_t *>(out), n);
  return launch_status("GELU kernel launch");
}

svdq_status_t svdq_quantize_activations(const svdq_weights_t *w, const void *X, int M,
                                        uint8_t *qact, float *ascales, float *lowrank_down,
                                        void *workspace, size_t ws_bytes, void *hip_stream) {
  svdq_status_t st = validate_weights(w, "svdq_quantize_activations");
  if (st != SVDQ_OK) return st;
  if (!X || !qact || !ascales || !workspace || (w->rank > 0 && !lowrank_down))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_quantize_activations: NULL pointer");
  if (!aligned16(X) || !aligned16(workspace))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_quantize_activations: misaligned pointer");
  if (M < 1 || (int64_t)M * w->K > ((int64_t)1 << 31))
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "svdq_quantize_activations: M=%d", M);
  const WeightLayout L(w->N, w->K, w->rank);
  const WorkLayout Wl(M, w->K, w->rank);
  if ((int64_t)ws_bytes < Wl.total)
    return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "workspace needs %lld bytes, got %zu",
                (long long)Wl.total, ws_bytes);
  if ((st = check_device()) != SVDQ_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  if ((st = launch_k1(L, Wl, w, X, M, ws, stream)) != SVDQ_OK) return st;
  const int64_t nb = (int64_t)M * (w->K / 2);
  hipLaunchKernelGGL(canon_codes_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const int8_t *>(ws + Wl.qa), M, w->K, (int)(Wl.Mp / kTile), qact);
  const int64_t ns = (int64_t)M * Wl.G;
  hipLaunchKernelGGL(canon_scales_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream,
                     reinterpret_cast<const float *>(ws + Wl.sa), M, (int)Wl.Mp, (int)Wl.G, ascales);
  if (w->rank > 0) {
    const int64_t nd = (int64_t)M * w->rank;
    hipLaunchKernelGGL(canon_down_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const float *>(ws + Wl.d), M, (int)Wl.Mp, (int)Wl.S,
                       (int)Wl.rp, w->rank, lowrank_down);
  }
  return launch_status("inspection kernels");
}

svdq_status_t svdq_debug_group_sums(const svdq_weights_t *w, int M, int m0, int mcount, int n0,
                                    int ncount, int32_t *P, const void *workspace,
                                    size_t ws_bytes, void *hip_stream) {
  svdq_status_t st = validate_weights(w, "svdq_debug_group_sums");
  if (st != SVDQ_OK) return st;
  if (!P || !workspace) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_debug_group_sums: NULL pointer");
  if (M < 1 || mcount < 1 || ncount < 1 || mcount > 256 || ncount > 256 || m0 < 0 || n0 < 0 ||
      m0 + mcount > M || n0 + ncount > w->N)
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "svdq_debug_group_sums: bad window");
  const WeightLayout L(w->N, w->K, w->rank);
  const WorkLayout Wl(M, w->K, w->rank);
  if ((int64_t)ws_bytes < Wl.total)
    return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "workspace needs %lld bytes", (long long)Wl.total);
  if ((st = check_device()) != SVDQ_OK) return st;
  K2Args a = make_k2_args(L, Wl, w, M, static_cast<const uint8_t *>(workspace));
  a.P = P;
  a.m0 = m0; a.mcount = mcount; a.n0 = n0; a.ncount = ncount;
  a.tile_m0 = m0 / 128 * 128;
  a.tile_n0 = n0 / 128 * 128;
  const int tm1 = (m0 + mcount + 127) / 128 * 128, tn1 = (n0 + ncount + 127) / 128 * 128;
  const dim3 grid((unsigned)((tn1 - a.tile_n0) / 128), (unsigned)((tm1 - a.tile_m0) / 128));
  hipLaunchKernelGGL((k2_w4a4_gemm<MODE_SUMS, SVDQ_EPILOGUE_NONE, true>), grid, dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream), a);
  return launch_status("group-sum kernel launch");
}

svdq_status_t awq_w4a16_forward(const void *blob, int N, int K, const void *x, int M,
                                const void *bias, void *y, void *hip_stream) {
  if (!blob || !x || !y) return fail(SVDQ_ERR_INVALID_ARGUMENT, "awq_w4a16_forward: NULL pointer");
  if (!aligned16(blob) || !aligned16(x) || !aligned16(y) || (bias && ((uintptr_t)bias & 1u)))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "awq_w4a16_forward: misaligned pointer");
  if (N < 1 || K < 1 || K % kGroup != 0 || M < 1 || M > 16 || (int64_t)N * K > ((int64_t)1 << 31))
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "awq_w4a16_forward: N=%d K=%d M=%d (M in 1..16, K %% 64 == 0)", N, K, M);
  svdq_status_t st = check_device();
  if (st != SVDQ_OK) return st;
  const AwqLayout L(N, K);
  const uint8_t *b = static_cast<const uint8_t *>(blob);
  hipLaunchKernelGGL(k3_awq_w4a16, dim3((unsigned)(L.Np / kAwqTile)), dim3(64), 0,
                     static_cast<hipStream_t>(hip_stream), b + L.q,
                     reinterpret_cast<const uint32_t *>(b + L.sz), static_cast<const uint16_t *>(x), M,
                     N, (int)L.Np, K, static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(y));
  return launch_status("AWQ kernel launch");
}

}  // extern "C"
