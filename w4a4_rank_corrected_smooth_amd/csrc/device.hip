// Device half of libsvdq: gfx950 kernels and the asynchronous entry points.
//
//  K1  k1_quantize_lowrank_down  smoothing, per-group INT4 activation codes
//                                and scales, low-rank down-projection D = X L1s
//  K2  k2_w4a4_gemm              INT4 x INT4 group GEMM on the fp6 matrix
//                                instruction (codes -7..7 held exactly), fp32
//                                per-group scaling, + D L2 + bias (+ GELU);
//                                for an MLP pair, the epilogue quantises the
//                                next layer's input instead of storing Y
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

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef unsigned v6u __attribute__((ext_vector_type(6)));
typedef int v8i __attribute__((ext_vector_type(8)));

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
// y keep their relative accuracy instead of cancelling in 1 + tanh(u).  With
// -2u log2(e) = y (c0 + c1 y^2) the exponential is one hardware exp2; exp2
// and the reciprocal (about 1 ulp of fp32 each) are far inside the half-ulp
// of the bf16 result; exp overflow gives 1/inf = 0, the right limit.
__device__ __forceinline__ float gelu_tanh_f32(float y) {
  constexpr float c0 = (float)(-2.0 * 0.7978845608028654 * 1.4426950408889634);
  constexpr float c1 = (float)(-2.0 * 0.7978845608028654 * 1.4426950408889634 * 0.044715);
  const float t = y * __builtin_fmaf(c1, y * y, c0);
  return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}

// Global -> LDS copy of 16 bytes per lane by the load unit
// (global_load_lds_dwordx4): lane i writes LDS address lds_base + 16 i.
// lds_base must be uniform across the wavefront.  Written as inline asm so
// that the copy's completion is tracked by the caller's own vmcnt waits
// (the compiler would otherwise wait for every copy before any LDS read).
// The asm has no register outputs; M0 is set and used inside the block.
__device__ __forceinline__ void lds_dma16(const void *gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gsrc), "s"(lds_base) : "memory");
}
// The same copy with a wave-uniform base address in scalar registers and a
// 32-bit per-lane byte offset.
__device__ __forceinline__ void lds_dma16_s(const void *sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_base) : "memory");
}
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
__device__ __forceinline__ void vmcnt_wait0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// vmcnt(0) through the builtin (expcnt and lgkmcnt left at their maxima), so
// the compiler's own wait bookkeeping knows every load has landed
__device__ __forceinline__ void vmcnt_wait0_known() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until at most n vector-memory operations are outstanding, n a runtime
// value (clamped to the counter's 6-bit maximum, which only waits longer)
template <int N>
__device__ __forceinline__ void vmcnt_wait_le(int n) {
  if constexpr (N == 0) {
    vmcnt_wait0();
  } else {
    if (n >= N) vmcnt_wait<N>(); else vmcnt_wait_le<N - 1>(n);
  }
}
__device__ __forceinline__ void vmcnt_wait_dyn(int n) { vmcnt_wait_le<63>(min(n, 63)); }

// One lane's share of a group's quantisation (the reading of the pages'
// quantiser used throughout): lane l holds half l / 32 of a row's 64 values,
// channels 16 j + 8 h + [0, 8) in xr[j] (bf16 pairs) with their factors
// 1/lambda in io[2 j], io[2 j + 1].
//   x_hat = fl32(x * iota);  a = max |x_hat| over 64 (two lanes);
//   s = a / 7, inv = 7 / a (correctly rounded), q = rint(x_hat inv),
// returned as s and the 32 codes packed as fp6 E2M3 (exact for these
// integers).  The hardware packer interleaves its two 16-value inputs (field
// 2i from the first, 2i+1 from the second), so even and odd elements go in to
// get element order 0..31 at bits 6c.  No clamp to [-7, 7] is needed:
// |x_hat| <= a and inv <= (7/a)(1 + 2^-24) give |fl32(x_hat inv)| <
// 7.0000009, which rounds to at most 7.
__device__ __forceinline__ float quantize_lane(const uint4 (&xr)[4], const float4 (&io)[8],
                                               v6u &packed) {
  float xh[32];
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t wv[4] = {xr[j].x, xr[j].y, xr[j].z, xr[j].w};
    const float iv[8] = {io[2 * j].x, io[2 * j].y, io[2 * j].z, io[2 * j].w,
                         io[2 * j + 1].x, io[2 * j + 1].y, io[2 * j + 1].z, io[2 * j + 1].w};
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
  v16f ev, od;
#pragma unroll
  for (int cc = 0; cc < 16; ++cc) {
    ev[cc] = rintf(__fmul_rn(xh[2 * cc], inv));
    od[cc] = rintf(__fmul_rn(xh[2 * cc + 1], inv));
  }
  // The packer's result must not share registers with its inputs (it writes
  // output dwords while later inputs are still to be read), which the
  // builtin does not guarantee: written as asm with an early-clobber output.
  asm("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, 1.0" : "=&v"(packed) : "v"(ev), "v"(od));
  return sc;
}

// One lane's MXFP4 block (the FP4 form of the 4-bit path, OCP Microscaling
// MXFP4): xm holds 32 consecutive bf16 activations (channels 32 h + [0, 32)
// of a group), io their 1/lambda.  x_hat = fl32(x iota); a = max |x_hat|;
// with E the biased exponent field of a, floor(log2 a) = E - 127 for a
// normal a, so the block exponent e = floor(log2 a) - 2 is E - 129, clamped
// at -127, which also covers a zero or subnormal a (E = 0).  Each
// r = x_hat 2^-e is exact (a power of two, 2^-e a normal float, |r| < 8).
// gfx950's packed FP4 conversion rounds r to the nearest E2M1 value, ties to
// the even mantissa bit, saturating at 6 (checked against that definition
// on every multiple of 1/128 in [-8, 8] and beyond), two values per
// instruction, low nibble first; it keeps the sign of a zero, so -0 codes
// (sign bit alone) are cleared afterwards.  Codes go out in canonical nibble
// order (code i at bits 4 (i % 8) of word i / 8); returns the E8M0 byte
// e + 127.
__device__ __forceinline__ uint32_t quantize_lane_mx(const uint4 (&xm)[4], const float4 (&io)[8],
                                                     uint4 &codes) {
  float v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t wv[4] = {xm[j].x, xm[j].y, xm[j].z, xm[j].w};
    const float4 i0 = io[2 * j], i1 = io[2 * j + 1];
    const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[8 * j + 2 * c] = __fmul_rn(bf16_lo(wv[c]), iv[2 * c]);
      v[8 * j + 2 * c + 1] = __fmul_rn(bf16_hi(wv[c]), iv[2 * c + 1]);
    }
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
  const int E = (int)(__float_as_uint(a) >> 23);
  const int e = E == 0 ? -127 : max(E - 129, -127);
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t d = 0u;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, __fmul_rn(v[8 * j], inv), __fmul_rn(v[8 * j + 1], inv), 1.0f, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, __fmul_rn(v[8 * j + 2], inv), __fmul_rn(v[8 * j + 3], inv), 1.0f, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, __fmul_rn(v[8 * j + 4], inv), __fmul_rn(v[8 * j + 5], inv), 1.0f, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, __fmul_rn(v[8 * j + 6], inv), __fmul_rn(v[8 * j + 7], inv), 1.0f, 3);
    // keep a nibble's sign bit only where its magnitude bits are not all 0
    const uint32_t mag = d & 0x77777777u;
    const uint32_t nz = (mag | (mag >> 1) | (mag >> 2)) & 0x11111111u;
    w[j] = mag | (d & (nz << 3));
  }
  codes = make_uint4(w[0], w[1], w[2], w[3]);
  return (uint32_t)(e + 127);
}

// ======================================================================= K1
// One workgroup (4 wavefronts) per (tile of 32 token rows, K split).  The
// split's groups are taken kK1Chunk = 4 at a time: the workgroup copies the
// chunk's 32 rows x 512 bytes of X, and the chunk's 256 smoothing factors,
// into LDS with the load unit's global->LDS path, each X copy instruction
// moving two whole 512-byte row segments (long contiguous bursts for HBM);
// wavefront w then quantises group w of the chunk.  kK1Bufs chunk buffers are
// in flight.  Inside a row segment the 16-byte pieces are permuted (piece p
// stored at slot p ^ (row % 16)) so that the reads below, one row per lane,
// hit 16 different bank quads.
// Per group, lane l owns row l % 32 and half h = l / 32: its 32 values are
// channels 16 j + 8 h + [0, 8) (j = 0..3), quantised by quantize_lane and
// stored as fp6 E2M3 (exact for these integers).  The raw bf16 values also
// feed a 32x32x16 bf16 MFMA against L1s for the low-rank down-projection;
// the four wavefronts' partial products are summed through LDS and written
// as this split's partial D.
constexpr int kK1Chunk = 4;                        // groups per chunk = wavefronts
constexpr int kK1RowBytes = kK1Chunk * kGroup * 2;  // 512
constexpr int kK1XBytes = kTile * kK1RowBytes;     // 16 KB of X per chunk
constexpr int kK1BufBytes = kK1XBytes + kK1Chunk * kGroup * 4;   // + 1 KB of 1/lambda
constexpr int kK1Bufs = 3;
constexpr int kK1LdsBytes = kK1Bufs * kK1BufBytes;
template <int TB, bool MX = false>   // rank_pad / 32; MXFP4 instead of INT4 codes
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TB <= 1 ? 3 : 1))) void k1_quantize_lowrank_down(
    const uint16_t *__restrict__ X, int M, int K, int Mp, int S,
    const float *__restrict__ iota, const uint16_t *__restrict__ l1t,
    uint8_t *__restrict__ qa, float *__restrict__ sa, float *__restrict__ dpart,
    int64_t *__restrict__ dzero, int rpz) {
  __shared__ __attribute__((aligned(16))) uint8_t k1_lds[kK1LdsBytes];
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)k1_lds;
  const int t = blockIdx.x, s = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int G = K / kGroup, Gs = G / S, T = Mp / kTile;
  const int rr = lane & 31, h = lane >> 5;
  const int row = t * kTile + rr;
  const int nch = (Gs + kK1Chunk - 1) / kK1Chunk;
  constexpr int NB = TB > 0 ? TB : 1;
  constexpr int L1N = 4 * TB;                      // L1s loads per wave and chunk
  const int ncopy = wu == 0 ? 5 : 4;               // copy instructions per wave and chunk
  // Copy of chunk c: wave w issues X instructions i = 4w .. 4w+3; instruction
  // i, lane l moves piece (l % 32) ^ (r % 16) of row r = 2i + l / 32.  Wave 0
  // also copies the chunk's 1/lambda.  Rows past M (padding, never stored by
  // the GEMM nor exported) repeat row M-1; groups past the split repeat its
  // last group.
  auto copy_chunk = [&](int c) {
    const uint32_t dst = lds_u32 + (uint32_t)((c % kK1Bufs) * kK1BufBytes);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * wu + k;
      const int r = 2 * i + (lane >> 5);
      const int piece = (lane & 31) ^ (r & 15);
      const int gq = s * Gs + min(c * kK1Chunk + (piece >> 3), Gs - 1);
      const uint16_t *src = X + (int64_t)min(t * kTile + r, M - 1) * K + gq * kGroup + (piece & 7) * 8;
      lds_dma16(src, dst + (uint32_t)(i * 1024));
    }
    if (wu == 0) {
      const int gq = s * Gs + min(c * kK1Chunk + (lane >> 4), Gs - 1);
      lds_dma16(iota + (int64_t)gq * kGroup + (lane & 15) * 4, dst + (uint32_t)kK1XBytes);
    }
  };
  // L1s operand of this wavefront's group in chunk c, 1 KB contiguous per
  // load (clamped; unused past the split)
  uint4 lring[kK1Bufs][4 * NB];
  auto load_l1 = [&](int c, uint4 (&d)[4 * NB]) {
    if constexpr (TB > 0) {
      // The loads must follow the chunk's copies in issue order (the waits
      // count them); their address takes an offset from an empty asm, which
      // stays after the copy asm, so the compiler cannot hoist them above.
      int zero = 0;
      asm volatile("" : "+s"(zero));
      const int g = s * Gs + min(c * kK1Chunk + wu, Gs - 1) + zero;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < TB; ++b)
          d[j * NB + b] = *reinterpret_cast<const uint4 *>(
              l1t + ((((int64_t)g * TB + b) * 4 + j) * 64 + lane) * 8);
    }
  };
  v16f dacc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dacc[b] = v16f{};

  // Vector-memory operations of one wavefront in issue order: copy(0)
  // l1(0) ... copy(B-1) l1(B-1) (B = kK1Bufs), then per chunk c: stores(c)
  // (kStores of them: INT4 three code pairs and a scale, MXFP4 one 16-byte
  // code store and a scale byte), copy(c+B) l1(c+B).  Before chunk c it
  // waits until copy(c) and l1(c) are done, leaving in flight everything
  // issued after them: the stores of the min(c, B-1) chunks before it and
  // the fetches of chunks c+1 .. c+B-1 that exist; then the workgroup meets.
#pragma unroll
  for (int c = 0; c < kK1Bufs; ++c) {
    if (c < nch) { copy_chunk(c); load_l1(c, lring[c]); }
  }
  for (int c0 = 0; c0 < nch; c0 += kK1Bufs)
#pragma unroll
  for (int u = 0; u < kK1Bufs; ++u) {
    const int c = c0 + u;
    if (c >= nch) break;
    constexpr int kStores = MX ? 2 : 4;
    const int later = kStores * min(c, kK1Bufs - 1) + (ncopy + L1N) * (min(nch - 1, c + kK1Bufs - 1) - c);
    vmcnt_wait_dyn(later);
    __syncthreads();
    const uint8_t *buf = k1_lds + u * kK1BufBytes;
    const float4 *iota_c = reinterpret_cast<const float4 *>(buf + kK1XBytes) + wu * 16;
    const int gi = c * kK1Chunk + wu;              // this wavefront's group in the split
    const bool live = gi < Gs;                     // uniform across the wavefront
    const int g = s * Gs + min(gi, Gs - 1);
    const uint8_t *xb = buf + rr * kK1RowBytes;
    uint4 xr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = wu * 8 + 2 * j + h;
      xr[j] = *reinterpret_cast<const uint4 *>(xb + ((piece ^ (rr & 15)) << 4));
    }
    float4 io[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      io[2 * j] = iota_c[4 * j + 2 * h];
      io[2 * j + 1] = iota_c[4 * j + 2 * h + 1];
    }
    if constexpr (MX) {
      // the lane's MX block: channels 32 h + [0, 32) of its group
      uint4 xm[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int piece = wu * 8 + 4 * h + j;
        xm[j] = *reinterpret_cast<const uint4 *>(xb + ((piece ^ (rr & 15)) << 4));
      }
      float4 iom[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) iom[q] = iota_c[8 * h + q];
      uint4 codes;
      const uint32_t e8 = quantize_lane_mx(xm, iom, codes);
      *reinterpret_cast<uint4 *>(qa + mx_code_offset(g, t, T, lane)) = codes;
      reinterpret_cast<uint8_t *>(sa)[mx_scale_offset(g, t, T, lane)] = (uint8_t)e8;
    } else {
      v6u packed;
      const float sc = quantize_lane(xr, io, packed);
      uint8_t *qp = qa + pair_offset(g, t, T, lane, 0);
#pragma unroll
      for (int j = 0; j < 3; ++j)
        *reinterpret_cast<uint2 *>(qp + 512 * j) = make_uint2(packed[2 * j], packed[2 * j + 1]);
      sa[(int64_t)g * Mp + row] = sc;            // both halves hold the same scale
    }
    if (TB > 0 && live) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v8bf av = as_v8bf(xr[j]);
#pragma unroll
        for (int b = 0; b < TB; ++b)
          dacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, as_v8bf(lring[u][j * NB + b]), dacc[b], 0, 0, 0);
      }
    }
    __syncthreads();                               // buffer u is free again
    if (c + kK1Bufs < nch) { copy_chunk(c + kK1Bufs); load_l1(c + kK1Bufs, lring[u]); }
  }
  if constexpr (TB > 0) {
    // the copy buffers are free now: the four wavefronts' partial products
    // meet there (4 x 16 x 64 floats = 16 KB)
    float (*red)[16][64] = reinterpret_cast<float (*)[16][64]>(k1_lds);
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
  // For a fused MLP pair: clear this row tile's rows of the next layer's
  // fixed-point D, which the GEMM that follows accumulates into.
  if (dzero != nullptr && s == 0) {
    int64_t *dz = dzero + (int64_t)t * kTile * rpz;
    for (int i = threadIdx.x; i < kTile * rpz / 2; i += 256)
      reinterpret_cast<int4 *>(dz)[i] = make_int4(0, 0, 0, 0);
  }
}

// ======================================================================= K2
// INT4 x INT4 group GEMM with per-group fp32 scaling.
//
// Workgroup: 4 wavefronts (2 x 2), output tile 128 x 256; wavefront tile
// 64 x 128 (2 x 4 MFMA tiles of 32 x 32).  Two workgroups share a CU, so
// each SIMD runs wavefronts of two independent workgroups.  One pipeline
// stage holds one group of 64 input channels in LDS (A codes, B codes, their
// fp32 scales), copied global -> LDS by the load unit; four stages rotate.
// Per group a workgroup copies 20 KB for 32768 outputs.
//
// Per 32 x 32 tile and group:
//   P  = v_mfma_scale_f32_32x32x64_f8f6f4 on fp6 codes (unit block scales):
//        the exact int32 group sums, delivered as fp32 (|P| <= 3136)
//   acc = fma(P, fl32(sA[m] sW[n]), acc)        (two VALU ops per element)
// The accumulators start from the low-rank up-projection D L2 (bf16 MFMA,
// D split into a bf16 high part and a bf16 remainder), computed while the
// first stages are copied; the epilogue adds the bias, the optional GELU,
// and stores bf16 or fp32.  MODE_SUMS stores P for a window instead.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so block id b
// runs on XCD b % 8; each XCD is given a contiguous range of tiles, walked
// GM tile-rows at a time, so the A and B panels its CUs share stay in its
// L2.
enum { MODE_FWD = 0, MODE_SUMS = 1, MODE_MX = 2 };

struct K2Args {
  const uint8_t *qa; const float *sa; const float *dpart; int S, M, Mp;
  const uint8_t *qw; const float *sw; const uint16_t *l2t; const float *bias;
  int N, Np, K, rp;
  void *Y;
  int32_t *P; int m0, mcount, n0, ncount;
  int tile_m0, tile_n0, TM, TN;     // tile grid (units of the workgroup tile)
  // D as one int64 fixed-point sum [Mp][rp] (input quantised by the previous
  // layer's GEMM) instead of fp32 partials
  const int64_t *dfix;
  // quantisation of the next layer's input in the epilogue (MLP pair): its
  // 1/lambda [N], L1s in fragment order, codes, scales and fixed-point D
  const float *iota2; const uint16_t *l1f2; uint8_t *qa2; float *sa2; int64_t *d2;
  int G2, rp2;
  // MXFP4 (MODE_MX): qa / qw hold E2M1 codes, these the E8M0 block scales
  const uint8_t *sqa; const uint8_t *sqw;
  // K-split (SPLIT): ksplit ranges of groups, fp32 partial tiles [ksplit][Mp][Np]
  int ksplit; float *part;
};

namespace k2c {
constexpr int WTM = 2, WTN = 4;                   // MFMA tiles per wavefront (rows, columns)
constexpr int WROWS = 32 * WTM, WCOLS = 32 * WTN; // 64 x 128
constexpr int BM = 2 * WROWS, BN = 2 * WCOLS, THREADS = 256, NWAVES = THREADS / 64;
static_assert(BM == kK2TileM && BN == kK2TileN, "the K-split sizing uses the workgroup tile");
constexpr int A_BLK = BM / kTile, B_BLK = BN / kTile;
constexpr int A_BYTES = A_BLK * kBlockBytes;     // one group per stage
constexpr int B_BYTES = B_BLK * kBlockBytes;
constexpr int SA_BYTES = BM * 4, SW_BYTES = BN * 4;
constexpr int STAGE_USED = A_BYTES + B_BYTES + SA_BYTES + SW_BYTES;   // 19968
constexpr int UNITS = STAGE_USED / 16;                                 // 1248
constexpr int WAVE_LOADS = (UNITS + 63) / 64;                          // 20
constexpr int STAGE = WAVE_LOADS * 64 * 16;                            // 20480, padded
constexpr int MAX_LOADS = WAVE_LOADS / NWAVES;                         // 5 per wave
constexpr int NBUF = 4;                                                // stages in LDS
constexpr int GM = 8;             // tile-rows walked together on one XCD
constexpr int EPI_WAVE_BYTES = 32 * WCOLS * 4;   // one 32-row half of a wavefront tile, fp32
static_assert(STAGE_USED % 16 == 0, "stage must be whole 16-byte units");
static_assert(WAVE_LOADS % NWAVES == 0, "every wavefront issues the same number of copies per stage");
static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0 && SW_BYTES % 1024 == 0 && SA_BYTES == 512 &&
              WAVE_LOADS * 1024 == A_BYTES + B_BYTES + SW_BYTES + 1024,
              "each copy reads one array; sA is the upper half of the last");
static_assert(2 * NBUF * STAGE <= 160 * 1024, "two workgroups must fit in one CU's LDS");
static_assert(NWAVES * EPI_WAVE_BYTES <= NBUF * STAGE, "epilogue staging reuses the stages");
}  // namespace k2c

// The fp6 operand occupies six registers; the instruction's 8-register
// operand slot leaves the last two unread, so they are left undefined
// rather than cleared on every load.
__device__ __forceinline__ v8i k2_frag(const uint8_t *blk, int lane) {
  const uint2 w0 = *reinterpret_cast<const uint2 *>(blk + lane * 8);
  const uint2 w1 = *reinterpret_cast<const uint2 *>(blk + 512 + lane * 8);
  const uint2 w2 = *reinterpret_cast<const uint2 *>(blk + 1024 + lane * 8);
  v8i r = __builtin_nondeterministic_value(r);
  r[0] = (int)w0.x; r[1] = (int)w0.y; r[2] = (int)w1.x;
  r[3] = (int)w1.y; r[4] = (int)w2.x; r[5] = (int)w2.y;
  return r;
}

// The FP4 operand occupies four registers (16 bytes: the lane's 32 codes);
// the rest of the 8-register slot is left undefined.
__device__ __forceinline__ v8i mx_frag(const uint8_t *blk, int lane) {
  const uint4 w = *reinterpret_cast<const uint4 *>(blk + lane * 16);
  v8i r = __builtin_nondeterministic_value(r);
  r[0] = (int)w.x; r[1] = (int)w.y; r[2] = (int)w.z; r[3] = (int)w.w;
  return r;
}

// Instruction order inside one step of K2's pipeline: the step's matrix
// instruction first, then D1 LDS reads (operands it no longer needs), the
// vector work, then D2 more LDS reads (scales the vector work has just used
// for the last time), and a fence so nothing crosses into the next step.
// This keeps the matrix core busy under the FMAs.
template <int D1, int D2>
__device__ __forceinline__ void k2_order() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  if constexpr (D1 > 0) __builtin_amdgcn_sched_group_barrier(0x100, D1, 0);
  __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
  if constexpr (D2 > 0) __builtin_amdgcn_sched_group_barrier(0x100, D2, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// As k2_order, for a step whose vector work swaps the activation scales for
// the next row tile: each of the four float4 reads goes right after the FMAs
// that last read the register it overwrites.
template <int D1, int D2 = 0>
__device__ __forceinline__ void k2_order_r() {
  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  if constexpr (D1 > 0) __builtin_amdgcn_sched_group_barrier(0x100, D1, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  if constexpr (D2 > 0) __builtin_amdgcn_sched_group_barrier(0x100, D2, 0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int MODE, int EPI, bool OUT_F32, bool DFIX = false, bool QNEXT = false, bool SPLIT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k2_w4a4_gemm(K2Args p) {
  using namespace k2c;
  static_assert(!SPLIT || (MODE == MODE_FWD && !QNEXT), "K-split: plain INT4 forward only");
  // ---- tile of this workgroup (XCD-aware, grouped); with a K-split,
  // consecutive workgroups on one XCD take different tiles of one K range
  const int T = p.TM * p.TN;
  const int TS = SPLIT ? T * p.ksplit : T;
  const int per_xcd = (TS + 7) / 8;
  const int L0 = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (L0 >= TS) return;
  const int split = SPLIT ? L0 / T : 0;
  const int L = SPLIT ? L0 - split * T : L0;
  const int band = L / (GM * p.TN);
  const int first_m = band * GM;
  const int gm = min(GM, p.TM - first_m);
  const int within = L - band * GM * p.TN;
  const int tm = first_m + within % gm, tn = within / gm;
  const int bm = p.tile_m0 + tm * BM, bn = p.tile_n0 + tn * BN;

  __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * STAGE];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int wu = __builtin_amdgcn_readfirstlane(w);      // wavefront index, scalar
  const int wmi = wu >> 1, wni = wu & 1;
  const int wm = bm + WROWS * wmi, wn = bn + WCOLS * wni;
  // groups [g0, g0 + G) of the K range (all of K without a split)
  const int Gall = p.K / kGroup;
  const int g0 = SPLIT ? split * Gall / p.ksplit : 0;
  const int G = SPLIT ? (split + 1) * Gall / p.ksplit - g0 : Gall;
  const int Ta = p.Mp / kTile, Tw = p.Np / kTile;
  const int hl = lane >> 5, ln = lane & 31;

  v16f acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = v16f{};

  // Copy schedule: a stage is WAVE_LOADS wavefront-loads of 64 x 16 bytes,
  // A codes | B codes | sW | sA, each load from one array: wave w issues
  // loads w, w + 4, w + 8, ... with every lane active; the last load's upper
  // half repeats sA into the padding.  A load's source is a wave-uniform
  // base (scalar registers) plus the lane's byte offset, and advances by one
  // row of blocks (codes) or one row of the [G][Mp] / [G][Np] scale arrays
  // from one group to the next.
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
  const uint8_t *sbase[MAX_LOADS];
  int64_t sstride[MAX_LOADS];
#pragma unroll
  for (int r = 0; r < MAX_LOADS; ++r) {
    const int L = wu + NWAVES * r;               // load index within the stage
    if (L < A_BYTES / 1024) {
      sbase[r] = p.qa + (int64_t)(bm / kTile) * kBlockBytes + 1024 * L;
      sstride[r] = (int64_t)Ta * kBlockBytes;
    } else if (L < (A_BYTES + B_BYTES) / 1024) {
      sbase[r] = p.qw + (int64_t)(bn / kTile) * kBlockBytes + 1024 * (L - A_BYTES / 1024);
      sstride[r] = (int64_t)Tw * kBlockBytes;
    } else if (L < (A_BYTES + B_BYTES + SW_BYTES) / 1024) {
      sbase[r] = reinterpret_cast<const uint8_t *>(p.sw + bn) + 1024 * (L - (A_BYTES + B_BYTES) / 1024);
      sstride[r] = (int64_t)p.Np * 4;
    } else {
      sbase[r] = reinterpret_cast<const uint8_t *>(p.sa + bm);
      sstride[r] = (int64_t)p.Mp * 4;
    }
    if constexpr (SPLIT) sbase[r] += g0 * sstride[r];   // loop indices count from g0
  }
  const uint32_t voff = 16u * lane;
  const uint32_t voff_sa = 16u * (lane & 31);     // sA is half a load
  auto fetch = [&](int g) {
    const uint32_t buf = smem_lds + (uint32_t)((g % NBUF) * STAGE) + (uint32_t)(wu * 64 * 16);
#pragma unroll
    for (int r = 0; r < MAX_LOADS; ++r) {
      const int L = wu + NWAVES * r;
      lds_dma16_s(sbase[r] + g * sstride[r], (r == MAX_LOADS - 1 && L == WAVE_LOADS - 1) ? voff_sa : voff,
                  buf + (uint32_t)(r * NWAVES * 64 * 16));
    }
  };

  // MXFP4 stage of K-step g: A codes (4 tile blocks of 1 KB), B codes (8),
  // and one copy of the step's E8M0 scales (lanes 0-15: A's 256 bytes,
  // 16-47: B's 512, 48-63 repeat A's); 13 wavefront-loads.  Wavefront w
  // copies A block w and B blocks w and w + 4; wavefront 0 also the scales.
  // Every source is a base fixed per wavefront (per lane for the scales)
  // plus g times a fixed step, so the copies take no branches.  LDS: [A 4 KB]
  // [B 8 KB][A scales 256 B][B scales 512 B].
  const uint8_t *mx_a = p.qa + (int64_t)(bm / kTile + wu) * 1024;
  const uint8_t *mx_b = p.qw + (int64_t)(bn / kTile + wu) * 1024;
  const int64_t mx_astep = (int64_t)Ta * 1024, mx_bstep = (int64_t)Tw * 1024;
  const bool sc_b = lane >= 16 && lane < 48;
  const uint8_t *mx_sc = sc_b ? p.sqw + (int64_t)(bn / kTile) * 64 + (lane - 16) * 16
                              : p.sqa + (int64_t)(bm / kTile) * 64 + (lane & 15) * 16;
  const int64_t mx_scstep = sc_b ? (int64_t)Tw * 64 : (int64_t)Ta * 64;
  auto fetch_mx = [&](int g) {
    const uint32_t buf = smem_lds + (uint32_t)((g % NBUF) * STAGE);
    lds_dma16_s(mx_a + g * mx_astep, voff, buf + (uint32_t)(wu * 1024));
    lds_dma16_s(mx_b + g * mx_bstep, voff, buf + (uint32_t)((4 + wu) * 1024));
    lds_dma16_s(mx_b + g * mx_bstep + 4 * 1024, voff, buf + (uint32_t)((8 + wu) * 1024));
    if (wu == 0) lds_dma16(mx_sc + g * mx_scstep, buf + (uint32_t)(12 * 1024));
  };

  // Operands of one group as a wavefront holds them in registers: the fp6
  // codes of its row tiles and column tiles, the activation scales of the
  // 16 rows each lane's accumulator elements belong to (per row tile: rows
  // 8 q + 4 (lane / 32) + [0, 4), q = 0..3, four float4 reads), and the
  // weight scale of the lane's column in each column tile.
  struct Frags { v8i a[WTM], b[WTN]; float4 sa[4]; float sw[WTN]; };
  Frags F;
  auto stage_of = [&](int g) { return smem + (g % NBUF) * STAGE; };
  auto load_a = [&](int g, int i) {
    F.a[i] = k2_frag(stage_of(g) + (WTM * wmi + i) * kBlockBytes, lane);
  };
  auto load_b = [&](int g, int j) {
    F.b[j] = k2_frag(stage_of(g) + A_BYTES + (WTN * wni + j) * kBlockBytes, lane);
  };
  auto sa_src = [&](int g, int i) {
    return reinterpret_cast<const float4 *>(stage_of(g) + A_BYTES + B_BYTES + SW_BYTES) +
           (WROWS * wmi + 32 * i + 4 * hl) / 4;
  };
  auto load_sw = [&](int g, int j) {
    F.sw[j] = reinterpret_cast<const float *>(stage_of(g) + A_BYTES + B_BYTES)
        [WCOLS * wni + 32 * j + ln];
  };
  // Per group each of the wavefront's 32 x 32 tiles t = (i, j) =
  // (t / WTN, t % WTN) takes one fp6 product; its elements are then scaled
  // by the fp32 product sA[m] sW[n] (one rounding) and accumulated with one
  // FMA.
  auto mm = [&](int t, v16f &P) {
    const int i = t / WTN, j = t % WTN;
    P = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], v16f{}, 2, 2, 0, 127, 0, 127);
  };
  auto consume_impl = [&](int t, int g, const v16f &P, const float4 *next, auto swap) {
    const int i = t / WTN, j = t % WTN;
    if constexpr (MODE == MODE_SUMS) {
      const int n = wn + 32 * j + ln;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = wm + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3);
        if (m >= p.m0 && m < p.m0 + p.mcount && n >= p.n0 && n < p.n0 + p.ncount)
          p.P[((int64_t)(m - p.m0) * p.ncount + (n - p.n0)) * G + g] = (int32_t)P[e];
      }
      if constexpr (decltype(swap)::value) {
#pragma unroll
        for (int q = 0; q < 4; ++q) F.sa[q] = next[2 * q];
      }
    } else {
      const float swj = F.sw[j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 sa4 = F.sa[q];
        const float sv[4] = {sa4.x, sa4.y, sa4.z, sa4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int e = 4 * q + k;
          acc[i][j][e] = __builtin_fmaf(P[e], __fmul_rn(sv[k], swj), acc[i][j][e]);
        }
        if constexpr (decltype(swap)::value) F.sa[q] = next[2 * q];
      }
    }
  };
  // consume(t): scale and accumulate tile t.  consume_swap(t, next): the
  // same, and each float4 of activation scales is replaced by the one at
  // `next` (the next row tile's) as soon as its last FMA has read it.
  auto consume = [&](int t, int g, const v16f &P) {
    consume_impl(t, g, P, nullptr, std::false_type{});
  };
  auto consume_swap = [&](int t, int g, const v16f &P, const float4 *next) {
    consume_impl(t, g, P, next, std::true_type{});
  };
  auto mm_hi = [&](int t, v16f &P) {
    __builtin_amdgcn_s_setprio(1);
    mm(t, P);
    __builtin_amdgcn_s_setprio(0);
  };

  // Software pipeline over (group, tile): while the FMAs of tile t run on
  // the vector ALU, the matrix core works on tile t + 1 (the next group's
  // first tile after the last).  Each operand of group g + 1 is read from
  // LDS into its registers right after the last instruction of group g that
  // uses it; the activation scales are held for one row tile at a time and
  // swapped float4 by float4 inside the last tile that reads them.  The
  // matrix instructions are issued at raised wave priority so the SIMD's
  // other wavefront does not delay them.  One barrier per group; three of
  // the four buffers hold stages g, g + 1, g + 2 while stage g + 3 is being
  // requested.  The scheduling fences keep each step's products from being
  // hoisted above the FMAs that still read the registers they overwrite.
  // After the last group the loads and the first product still run, on a
  // stale but in-bounds LDS buffer, and their results are never used:
  // branch-free code keeps the operands and products in fixed registers.
  v16f Pa, Pb;
  for (int g = 0; g < 3 && g < G; ++g) {
    if constexpr (MODE == MODE_MX) fetch_mx(g); else fetch(g);
  }
  if constexpr (MODE == MODE_FWD || MODE == MODE_MX) {
    // Low-rank up-projection first, while the first stages are in flight
    // (with a K-split, the 32-rank chunks are dealt round the ranges, so
    // each range's partial carries some of them and no range waits on all):
    // acc = D L2 on bf16 matrix cores, D entered as a bf16 high part plus a
    // bf16 remainder.  D of the workgroup's 128 rows is assembled once, in
    // the fourth stage buffer (free until the main loop starts), 32 ranks at
    // a time: wavefront w sums the K1 splits' partials of rows 32 w .. 32 w
    // + 31 in split order (lane l: row l / 2, ranks 16 (l % 2) + [0, 16);
    // loads issued four splits at a time, indices clamped, surplus ones not
    // added) and stores the two bf16 parts; every wavefront then reads its
    // operands from there.
    uint16_t *dhi = reinterpret_cast<uint16_t *>(smem + 3 * STAGE);   // [BM][32]
    uint16_t *dlo = dhi + BM * 32;                                     // [BM][32]
    static_assert(BM * 32 * 2 * 2 <= STAGE, "low-rank staging fits one stage buffer");
    const int rloc = 32 * wu + (lane >> 1), k0 = 16 * (lane & 1);
    for (int c2 = split; c2 < p.rp / 32; c2 += SPLIT ? p.ksplit : 1) {
      float d[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) d[e] = 0.f;
      if constexpr (DFIX) {
        // one fixed-point sum: 16 int64 per lane, converted with one rounding
        const int4 *q = reinterpret_cast<const int4 *>(p.dfix + (int64_t)(bm + rloc) * p.rp + 32 * c2 + k0);
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int4 v = q[x];
          const int64_t a0 = (int64_t)(((uint64_t)(uint32_t)v.y << 32) | (uint32_t)v.x);
          const int64_t a1 = (int64_t)(((uint64_t)(uint32_t)v.w << 32) | (uint32_t)v.z);
          d[2 * x] = (float)((double)a0 * (1.0 / kDFixScale));
          d[2 * x + 1] = (float)((double)a1 * (1.0 / kDFixScale));
        }
      }
      const float *dp0 = p.dpart + (int64_t)(bm + rloc) * p.rp + 32 * c2 + k0;
      for (int s0 = 0; s0 < (DFIX ? 0 : p.S); s0 += 4) {
        float4 v[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 *q = reinterpret_cast<const float4 *>(dp0 + (int64_t)min(s0 + u, p.S - 1) * p.Mp * p.rp);
#pragma unroll
          for (int x = 0; x < 4; ++x) v[u][x] = q[x];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (s0 + u < p.S) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              d[4 * x + 0] += v[u][x].x; d[4 * x + 1] += v[u][x].y;
              d[4 * x + 2] += v[u][x].z; d[4 * x + 3] += v[u][x].w;
            }
          }
        }
      }
      uint32_t hw[8], lw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t h0 = f32_to_bf16_rne(d[2 * e]), h1 = f32_to_bf16_rne(d[2 * e + 1]);
        const uint32_t l0 = f32_to_bf16_rne(d[2 * e] - __uint_as_float(h0 << 16));
        const uint32_t l1 = f32_to_bf16_rne(d[2 * e + 1] - __uint_as_float(h1 << 16));
        hw[e] = h0 | (h1 << 16);
        lw[e] = l0 | (l1 << 16);
      }
      uint4 *hp = reinterpret_cast<uint4 *>(dhi + rloc * 32 + k0);
      uint4 *lp = reinterpret_cast<uint4 *>(dlo + rloc * 32 + k0);
      hp[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]); hp[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
      lp[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]); lp[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
      uint4 bw[2][WTN];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
          bw[cc][j] = *reinterpret_cast<const uint4 *>(p.l2t + (int64_t)(wn + 32 * j + ln) * p.rp + 32 * c2 + 16 * cc + 8 * hl);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        const int r = WROWS * wmi + 32 * i + ln;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const v8bf ah = as_v8bf(*reinterpret_cast<const uint4 *>(dhi + r * 32 + 16 * cc + 8 * hl));
          const v8bf al = as_v8bf(*reinterpret_cast<const uint4 *>(dlo + r * 32 + 16 * cc + 8 * hl));
#pragma unroll
          for (int j = 0; j < WTN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, as_v8bf(bw[cc][j]), acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, as_v8bf(bw[cc][j]), acc[i][j], 0, 0, 0);
          }
        }
      }
      __syncthreads();                   // staging free for the next 32 ranks
    }
  }
  if constexpr (MODE == MODE_MX) {
    // Block-scaled FP4 main loop.  Per K-step each wavefront issues its 8
    // matrix instructions (2 x 4 tiles of 32 x 32), each taking the step's
    // codes and the lanes' E8M0 block scales and accumulating into its tile:
    // the instruction applies both scales, so no vector work is left per
    // element.  Operands of step g + 1 are read from LDS behind the step's
    // matrix instructions; waits and barriers as in the INT4 loop below,
    // with this wavefront's own copy count per stage (4 for wavefront 0, 3
    // for the others).
    auto mx_wait = [&](bool all) {
      if (all) vmcnt_wait0();
      else if (wu == 0) vmcnt_wait<4>();
      else vmcnt_wait<3>();
    };
    // Scales: one word per lane for the workgroup's 4 A tiles (this
    // wavefront's two moved to bytes 0 and 1) and one for its own 4 B tiles;
    // the matrix instruction selects the tile's byte.
    v8i xa[WTM], xb[WTN];
    int xsa, xsb;
    auto mx_load = [&](int g) {
      const uint8_t *st = stage_of(g);
#pragma unroll
      for (int i = 0; i < WTM; ++i) xa[i] = mx_frag(st + (WTM * wmi + i) * 1024, lane);
#pragma unroll
      for (int j = 0; j < WTN; ++j) xb[j] = mx_frag(st + 4096 + (WTN * wni + j) * 1024, lane);
      xsa = (int)(reinterpret_cast<const uint32_t *>(st + 12288)[lane] >> (16 * wmi));
      xsb = (int)reinterpret_cast<const uint32_t *>(st + 12288 + 256 + 256 * wni)[lane];
    };
    mx_wait(G <= 2);
    __syncthreads();
    mx_load(0);
    for (int g = 0; g < G; ++g) {
      if (g + 1 < G) {
        mx_wait(g + 2 >= G);
        __syncthreads();
        if (g + 3 < G) fetch_mx(g + 3);
      }
      static_assert(WTM == 2 && WTN == 4, "scale bytes: two A tiles and four B tiles per wavefront");
#define MX_MM(i, j)                                                                                    \
  acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa[i], xb[j], acc[i][j], 4, 4, i, xsa, j, xsb)
      MX_MM(0, 0); MX_MM(0, 1); MX_MM(0, 2); MX_MM(0, 3);
      MX_MM(1, 0); MX_MM(1, 1); MX_MM(1, 2); MX_MM(1, 3);
#undef MX_MM
      mx_load(g + 1);
    }
  } else {
  if (G > 2) vmcnt_wait<MAX_LOADS>(); else vmcnt_wait0();
  __syncthreads();
  load_a(0, 0); load_a(0, 1);
#pragma unroll
  for (int j = 0; j < WTN; ++j) { load_b(0, j); load_sw(0, j); }
  {
    const float4 *s0 = sa_src(0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) F.sa[q] = s0[2 * q];
  }
  mm(0, Pa);
  for (int g = 0; g < G; ++g) {
    // Every wavefront waits for its copies of stage g + 1 (stage g + 2 may
    // still be in flight) and meets the others; stage g - 1 has then been
    // read by all of them, so its buffer takes stage g + 3.
    if (g + 1 < G) {
      if (MODE == MODE_FWD && g + 2 < G) vmcnt_wait<MAX_LOADS>(); else vmcnt_wait0();
      __syncthreads();
      if (g + 3 < G) fetch(g + 3);
    }
    mm_hi(1, Pb);                         // tile (0,1)
    consume(0, g, Pa);
    k2_order<0, 0>();
    mm_hi(2, Pa);                         // tile (0,2)
    consume(1, g, Pb);
    k2_order<0, 0>();
    mm_hi(3, Pb);                         // tile (0,3): last use of a0
    load_a(g + 1, 0);
    consume(2, g, Pa);
    k2_order<3, 0>();
    mm_hi(4, Pa);                         // tile (1,0): last use of b0
    load_b(g + 1, 0);
    consume_swap(3, g, Pb, sa_src(g, 1));      // row-0 scales give way to row 1
    k2_order_r<3>();
    mm_hi(5, Pb);                         // tile (1,1): last use of b1
    load_b(g + 1, 1);
    consume(4, g, Pa);           // last use of sw0
    load_sw(g + 1, 0);
    k2_order<3, 1>();
    mm_hi(6, Pa);                         // tile (1,2): last use of b2
    load_b(g + 1, 2);
    consume(5, g, Pb);           // last use of sw1
    load_sw(g + 1, 1);
    k2_order<3, 1>();
    mm_hi(7, Pb);                         // tile (1,3): last use of a1, b3
    load_a(g + 1, 1); load_b(g + 1, 3);
    consume(6, g, Pa);           // last use of sw2
    load_sw(g + 1, 2);
    k2_order<6, 1>();
    mm_hi(0, Pa);                         // next group's tile (0,0)
    consume_swap(7, g, Pb, sa_src(g + 1, 0));  // row-1 scales give way to the next group's row 0
    load_sw(g + 1, 3);
    k2_order_r<0, 1>();
  }
  }  // INT4 main loop

  if constexpr (SPLIT) {
    // K-split: the fp32 partial tile, padded rows and columns included (the
    // partial buffer is [Mp][Np]); bias and the epilogue come in the sum.
    float *pp = p.part + (int64_t)split * p.Mp * p.Np;
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = wm + 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3), n = wn + 32 * j + ln;
          pp[(int64_t)m * p.Np + n] = acc[i][j][e];
        }
  } else if constexpr (MODE == MODE_FWD && QNEXT) {
    // MLP pair: this layer's output never goes to memory.  Bias (+ GELU),
    // rounded to bf16 (exactly the values the unfused path stores), then the
    // next layer's quantiser runs on the tile: every (32-row tile, group of 64
    // columns) block of the wavefront's 64 x 128 tile lies wholly inside it.
    // The tile is staged row-major in the wavefront's own LDS, 16-byte chunks
    // XOR-permuted by row so the one-row-per-lane reads spread over the banks.
    __syncthreads();                    // every wavefront is done with the stages
    uint8_t *xs = smem + w * EPI_WAVE_BYTES;   // 64 rows x 256 bytes
    static_assert(WROWS * WCOLS * 2 <= EPI_WAVE_BYTES, "bf16 tile fits the wavefront's staging");
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
        const float bj = p.bias[wn + 32 * j + ln];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 32 * i + 8 * (e >> 2) + 4 * hl + (e & 3), c = 32 * j + ln;
          float y = acc[i][j][e] + bj;
          if constexpr (EPI == SVDQ_EPILOGUE_GELU_TANH) y = gelu_tanh_f32(y);
          *reinterpret_cast<__bf16 *>(xs + r * (WCOLS * 2) + ((((c >> 3) ^ (r & 15))) << 4) + (c & 7) * 2) =
              (__bf16)y;
        }
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int rr = lane & 31, h = lane >> 5;
    const int T2 = p.Mp / kTile;
    // block (i, gl): lane's 32 values, row 32 i + rr, channels 16 j + 8 h + [0, 8)
    auto load_block = [&](int i, int gl, uint4 (&xr)[4]) {
      const int r = 32 * i + rr;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xr[j] = *reinterpret_cast<const uint4 *>(xs + r * (WCOLS * 2) + (((8 * gl + 2 * j + h) ^ (r & 15)) << 4));
    };
    // The next layer's low-rank down-projection over this tile's channels,
    // 32 ranks at a time: bf16 MFMA of the tile's raw bf16 values against
    // L1s (the first 32 ranks in the same pass as the quantisation); the two
    // wavefronts sharing rows add their halves through LDS in a fixed order,
    // and the sum goes into the next layer's D as 64-bit fixed point (units
    // of 2^-32; integer addition, so the result does not depend on the order
    // in which workgroups arrive).  Partial sums are clamped to +-2^56 so no
    // sum of the column tiles can overflow.
    const int TB2 = p.rp2 / 32;
    auto load_l1f = [&](int g2, int b, uint4 (&lf)[4]) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        lf[j] = *reinterpret_cast<const uint4 *>(p.l1f2 + ((((int64_t)g2 * TB2 + b) * 4 + j) * 64 + lane) * 8);
    };
    float *exch = reinterpret_cast<float *>(smem + NWAVES * EPI_WAVE_BYTES);   // [4][16][64]
    static_assert(NWAVES * EPI_WAVE_BYTES + NWAVES * 16 * 64 * 4 <= NBUF * STAGE, "exchange fits");
    auto finish = [&](int b, const v16f (&dacc)[WTM]) {
      // wavefront (wmi, wni) finishes row tile wni of its pair's rows
#pragma unroll
      for (int e = 0; e < 16; ++e) exch[(w * 16 + e) * 64 + lane] = wni == 0 ? dacc[1][e] : dacc[0][e];
      __syncthreads();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float other = exch[((w ^ 1) * 16 + e) * 64 + lane];
        const float v = wni == 0 ? dacc[0][e] + other : other + dacc[1][e];
        const double q = fmin(fmax(rint((double)v * kDFixScale), -0x1p56), 0x1p56);
        const int m = wm + 32 * wni + 8 * (e >> 2) + 4 * hl + (e & 3);
        atomicAdd(reinterpret_cast<unsigned long long *>(p.d2 + (int64_t)m * p.rp2 + 32 * b + ln),
                  (unsigned long long)(long long)q);
      }
      __syncthreads();                   // the exchange buffer is reused
    };
    v16f dacc[WTM];
#pragma unroll
    for (int i = 0; i < WTM; ++i) dacc[i] = v16f{};
#pragma unroll
    for (int gl = 0; gl < WCOLS / kGroup; ++gl) {
      const int g2 = (wn + kGroup * gl) / kGroup;
      if (g2 >= p.G2) continue;                  // padding columns past the layer's N
      float4 io[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 *ip = reinterpret_cast<const float4 *>(p.iota2 + (int64_t)g2 * kGroup + 16 * j + 8 * h);
        io[2 * j] = ip[0];
        io[2 * j + 1] = ip[1];
      }
      uint4 lf[4];
      if (TB2 > 0) load_l1f(g2, 0, lf);
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        uint4 xr[4];
        load_block(i, gl, xr);
        v6u packed;
        const float sc = quantize_lane(xr, io, packed);
        uint8_t *qp = p.qa2 + pair_offset(g2, (wm + 32 * i) / kTile, T2, lane, 0);
#pragma unroll
        for (int j = 0; j < 3; ++j)
          *reinterpret_cast<uint2 *>(qp + 512 * j) = make_uint2(packed[2 * j], packed[2 * j + 1]);
        p.sa2[(int64_t)g2 * p.Mp + wm + 32 * i + rr] = sc;   // both halves hold the same scale
        if (TB2 > 0) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(xr[j]), as_v8bf(lf[j]), dacc[i], 0, 0, 0);
        }
      }
    }
    if (TB2 > 0) finish(0, dacc);
    for (int b = 1; b < TB2; ++b) {
#pragma unroll
      for (int i = 0; i < WTM; ++i) dacc[i] = v16f{};
#pragma unroll
      for (int gl = 0; gl < WCOLS / kGroup; ++gl) {
        const int g2 = (wn + kGroup * gl) / kGroup;
        if (g2 >= p.G2) continue;
        uint4 lf[4];
        load_l1f(g2, b, lf);
#pragma unroll
        for (int i = 0; i < WTM; ++i) {
          uint4 xr[4];
          load_block(i, gl, xr);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            dacc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_v8bf(xr[j]), as_v8bf(lf[j]), dacc[i], 0, 0, 0);
        }
      }
      finish(b, dacc);
    }
  } else if constexpr (MODE == MODE_FWD || MODE == MODE_MX) {
    // Bias (+ GELU), then the wavefront's tile goes out through its own LDS
    // one 32-row half at a time, so global stores are whole 16-byte vectors
    // along a row instead of 2- or 4-byte scattered stores.
    __syncthreads();                    // every wavefront is done with the stages
    uint8_t *wbuf = smem + w * EPI_WAVE_BYTES;
    constexpr int ES = OUT_F32 ? 4 : 2;          // bytes per output element
    constexpr int VE = 16 / ES;                  // elements per 16-byte vector
    constexpr int LPR = WCOLS / VE;              // lanes per row of the wavefront tile
    const bool vec_ok = (p.N % VE) == 0;
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
        const float bj = p.bias[wn + 32 * j + ln];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 8 * (e >> 2) + 4 * hl + (e & 3);
          float y = acc[i][j][e] + bj;
          if constexpr (EPI == SVDQ_EPILOGUE_GELU_TANH) y = gelu_tanh_f32(y);
          if constexpr (OUT_F32)
            reinterpret_cast<float *>(wbuf)[r * WCOLS + 32 * j + ln] = y;
          else
            reinterpret_cast<__bf16 *>(wbuf)[r * WCOLS + 32 * j + ln] = (__bf16)y;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int q = 0; q < 32 * LPR / 64; ++q) {
        const int r = q * (64 / LPR) + lane / LPR;
        const int c = (lane % LPR) * VE;
        const int m = wm + 32 * i + r, n = wn + c;
        const uint4 v = *reinterpret_cast<const uint4 *>(wbuf + (r * WCOLS + c) * ES);
        if (m < p.M) {
          uint8_t *dst = reinterpret_cast<uint8_t *>(p.Y) + ((int64_t)m * p.N + n) * ES;
          if (vec_ok && n + VE <= p.N) {
            *reinterpret_cast<uint4 *>(dst) = v;
          } else {
            const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int t = 0; t < VE; ++t)
              if (n + t < p.N) {
                if constexpr (OUT_F32)
                  reinterpret_cast<float *>(dst)[t] = __uint_as_float(wv[t]);
                else
                  reinterpret_cast<uint16_t *>(dst)[t] = (uint16_t)(wv[t >> 1] >> (16 * (t & 1)));
              }
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// Sum of a K-split GEMM's partial tiles, in range order, + bias (+ GELU),
// stored as Y.  Thread: 4 consecutive columns of one row.
template <int EPI, bool OUT_F32>
__global__ __launch_bounds__(256) void k2_split_sum(const float *__restrict__ part, int ksplit, int M,
                                                    int N, int Mp, int Np, const float *__restrict__ bias,
                                                    void *__restrict__ Y) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nq = Np / 4;
  const int64_t m = idx / nq;
  const int n0 = (int)(idx - m * nq) * 4;
  if (m >= M || n0 >= N) return;
  const float *src = part + m * Np + n0;
  float4 acc = *reinterpret_cast<const float4 *>(src);
  for (int k = 1; k < ksplit; ++k) {
    const float4 v = *reinterpret_cast<const float4 *>(src + (int64_t)k * Mp * Np);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  const float a4[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int n = n0 + t;
    if (n >= N) break;
    float y = a4[t] + bias[n];
    if constexpr (EPI == SVDQ_EPILOGUE_GELU_TANH) y = gelu_tanh_f32(y);
    if constexpr (OUT_F32)
      reinterpret_cast<float *>(Y)[m * N + n] = y;
    else
      reinterpret_cast<__bf16 *>(Y)[m * N + n] = (__bf16)y;
  }
}

// ======================================================================= K3
// AWQ W4A16.  A workgroup of 4 wavefronts owns a tile of 16 output channels;
// wavefront w takes a contiguous quarter of the groups of 64 input channels
// (rounded up to a multiple of 4, so its range starts on a pair of code
// blocks and on a 16-byte quad of scale words), kAwqChunk groups at a time.
// Per chunk it first copies the chunk's activations (M rows, a few kilobytes
// shared by every workgroup, so cache hits) into its own LDS with the
// global->LDS path, then issues its code loads (16 bytes per lane: two
// groups) and scale loads (16 bytes: four groups), the HBM stream, and waits
// only for the copies; each group's compute then waits for its own loads
// alone, in issue order.  Every load is unconditional (indices clamped;
// groups past the range weigh 0, and every value they touch is finite: the
// copies fill whole rows of kAwqChunk groups, repeating the last group of
// the range, and the blob's padding words are zero), so the completion
// counts are exact.  For each group, lane l (channel l % 16, quarter
// q = l / 16) turns its 16 codes into fp16 (q - z) with the 1024-offset
// trick (0x6400 | code is the fp16 value 1024 + code; subtracting 1024 + z
// is exact), the activations [16, 64] read from LDS are the A operand, and
// two v_mfma_f32_16x16x32_f16 give the group's inner sums; acc += s * sum in
// fp32.  Rows m >= M repeat row M - 1 and are never stored.  The four
// partial sums meet in LDS, in a fixed order.
constexpr int kAwqChunk = 12;                          // a multiple of 4

// One group of 64 input channels for a wavefront's 16 x 16 output block:
// xg points at the lane's activations in LDS (row lane % 16, channels
// 16 (lane / 16) + [0, 16)), w0 / w1 hold its 16 codes (column lane % 16,
// the same channels; even channels in the low half-words), szv the column's
// fp16 scale | zero << 16.  acc += s * sum over the group (weight 0 when the
// group is not valid; every input is finite either way).
__device__ __forceinline__ void awq_group(const uint16_t *xg, uint32_t w0, uint32_t w1, uint32_t szv,
                                          bool valid, v4f &acc) {
  const uint4 xa0 = *reinterpret_cast<const uint4 *>(xg);
  const uint4 xa1 = *reinterpret_cast<const uint4 *>(xg + 8);
  const _Float16 zf = __builtin_bit_cast(_Float16, (uint16_t)(szv >> 16));
  const float sf = valid ? (float)__builtin_bit_cast(_Float16, (uint16_t)(szv & 0xFFFF)) : 0.0f;
  const _Float16 off = -((_Float16)1024.0f + zf);
  const v2h off2 = v2h{off, off};
  v8h bop[2];
  const uint32_t magic = 0x64006400u;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t word = half ? w1 : w0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // (word >> 4j) & 0x000F000F | 0x64006400 in one vector instruction
      uint32_t pr;
      asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(pr) : "v"(word >> (4 * j)), "s"(0x000F000Fu), "v"(magic));
      const v2h v = __builtin_bit_cast(v2h, pr) + off2;
      bop[half][2 * j] = v.x;
      bop[half][2 * j + 1] = v.y;
    }
  }
  v4f part = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, xa0), bop[0], v4f{}, 0, 0, 0);
  part = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, xa1), bop[1], part, 0, 0, 0);
  // output layout: lane holds rows 4 * (lane / 16) + e, column lane % 16
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(part[e], sf, acc[e]);
}
__global__ __launch_bounds__(256) void k3_awq_w4a16(const uint8_t *__restrict__ qd,
                                                     const uint32_t *__restrict__ sz,
                                                     const uint16_t *__restrict__ x, int M,
                                                     int N, int K,
                                                     const uint16_t *__restrict__ bias,
                                                     uint16_t *__restrict__ y) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  const int G = K / kGroup;
  const int G4 = (G + 3) & ~3;
  const int Gq = ((G + 3) / 4 + 3) & ~3;
  const int g0 = min(G, w * Gq), g1 = min(G, g0 + Gq);
  const int m = lane & 15, qtr = lane >> 4;
  const int n = tile * kAwqTile + (lane & 15);
  const uint8_t *qbase = qd + (int64_t)tile * ((G + 1) / 2) * kAwqBlockBytes + lane * 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t awq_lds[];
  v4f acc = v4f{};
  // this wavefront's copy of the chunk's activations: rows 0..M-1 of
  // kAwqChunk groups each, one 16-byte piece per lane and copy
  constexpr int npr = kAwqChunk * (kGroup / 8);         // pieces per row
  const int npc = M * npr;
  const int xw_bytes = (npc + 63) / 64 * 1024;
  const uint32_t xl_u32 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)awq_lds +
                          (uint32_t)(__builtin_amdgcn_readfirstlane(w) * xw_bytes);
  const uint16_t *xl = reinterpret_cast<const uint16_t *>(awq_lds + w * xw_bytes);
  const uint16_t *xm = xl + min(m, M - 1) * (npr * 8) + 16 * qtr;
  for (int gc = g0; gc < g1; gc += kAwqChunk) {
    // activations first (cache hits), then the code and scale stream; every
    // load after the copies is unconditional, so the copies are complete
    // once at most kAwqChunk / 2 + kAwqChunk / 4 loads remain
    for (int c0 = 0; c0 < npc; c0 += 64) {
      const int pc = min(c0 + lane, npc - 1);
      const int mr = pc / npr, o = pc - mr * npr;
      const int gi = min(gc + o / 8, g1 - 1);
      lds_dma16(x + (int64_t)mr * K + gi * kGroup + (o % 8) * 8, xl_u32 + (uint32_t)(c0 * 16));
    }
    // The code and scale loads must follow the copies in issue order (the
    // wait below counts them); their addresses take an offset from an empty
    // asm placed after the copies, so the compiler cannot hoist them above.
    int zero = 0;
    asm volatile("" : "+s"(zero));
    const uint8_t *qb = qbase + zero;
    const uint32_t *szb = sz + (int64_t)n * G4 + zero;
    uint4 cw[kAwqChunk / 2];
    uint4 szw[kAwqChunk / 4];
#pragma unroll
    for (int j = 0; j < kAwqChunk / 2; ++j) {
      const int pr = min(gc / 2 + j, (g1 - 1) / 2);
      cw[j] = *reinterpret_cast<const uint4 *>(qb + (int64_t)pr * kAwqBlockBytes);
    }
#pragma unroll
    for (int j = 0; j < kAwqChunk / 4; ++j) {
      const int qd4 = min(gc / 4 + j, (g1 - 1) / 4);
      szw[j] = *reinterpret_cast<const uint4 *>(szb + 4 * qd4);
    }
    vmcnt_wait<kAwqChunk / 2 + kAwqChunk / 4>();
#pragma unroll
    for (int i = 0; i < kAwqChunk; ++i) {
      const uint4 q4 = szw[i / 4];
      const uint32_t szv = (i % 4 == 0) ? q4.x : (i % 4 == 1) ? q4.y : (i % 4 == 2) ? q4.z : q4.w;
      const uint4 c = cw[i / 2];
      // groups past the wavefront's range weigh 0, so every load above is
      // used and none is moved below the wait
      awq_group(xm + i * kGroup, i % 2 == 0 ? c.x : c.z, i % 2 == 0 ? c.y : c.w, szv, gc + i < g1, acc);
    }
  }
  __shared__ v4f red[4][64];
  red[w][lane] = acc;
  __syncthreads();
  if (w != 0) return;
  const v4f r0 = red[0][lane], r1 = red[1][lane], r2 = red[2][lane], r3 = red[3][lane];
  const int col = tile * kAwqTile + (lane & 15);
  if (col < N) {
    const float b = bias ? (float)__builtin_bit_cast(_Float16, bias[col]) : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * (lane >> 4) + e;
      if (row < M) {
        const float v = ((r0[e] + r1[e]) + (r2[e] + r3[e])) + b;
        y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
  }
}

// AWQ W4A16 for more rows (M = 5..16).  With 16 rows, a private copy of a
// 12-group chunk's activations per wavefront (24 KB) would leave one
// workgroup per CU.  Here a workgroup covers two column tiles (32 output
// channels) and splits the groups in two halves: wavefront w takes tile
// w % 2 and half w / 2, so the two wavefronts of a half share one copy of
// its activations.  Chunks are kAwqWideChunk groups, double-buffered in LDS
// per half; each wavefront issues the code and scale loads of up to
// kAwqWideChunks chunks at once (the HBM stream, all in flight together),
// then the copy of its half's first chunk.  Chunk k then runs as: a barrier
// (chunk k - 1 is done with the buffer the next copy overwrites), the copy
// of chunk k + 1, a wait for everything older (chunk k's copy and, at
// k = 0, every code load), a barrier (both wavefronts' copies of chunk k
// are in), and chunk k's groups.  Both halves run the same number of chunks
// (surplus ones load clamped data and weigh 0), so every barrier is met by
// all four wavefronts; the halves' sums meet in LDS in a fixed order.
constexpr int kAwqWideChunk = 4;                       // groups per chunk (one scale quad)
constexpr int kAwqWideChunks = 8;                      // chunks whose codes are in flight together
// M from which this kernel runs: measured on MI355X at N = 18432, K = 3072
// against the one above, 16.0 vs 12.4 us at M = 8 and 18.7 vs 24.4 us at
// M = 16 (the one above then holds 24 KB of activations per wavefront, one
// workgroup per CU).  Here each chunk waits on a copy issued one chunk
// earlier, which bounds it at smaller M.
constexpr int kAwqWideMinRows = 10;
__global__ __launch_bounds__(256) void k3_awq_w4a16_wide(const uint8_t *__restrict__ qd,
                                                          const uint32_t *__restrict__ sz,
                                                          const uint16_t *__restrict__ x, int M,
                                                          int N, int K,
                                                          const uint16_t *__restrict__ bias,
                                                          uint16_t *__restrict__ y) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int tl = wu & 1, h = wu >> 1;                  // tile within the workgroup, group half
  const int G = K / kGroup, G4 = (G + 3) & ~3, P = (G + 1) / 2;
  const int Gh = (((G + 1) / 2) + kAwqWideChunk - 1) / kAwqWideChunk * kAwqWideChunk;
  const int g0 = h * Gh;                               // this half: groups [g0, g0 + Gh) within [0, G)
  const int nch = Gh / kAwqWideChunk;
  const int ntiles = (N + kAwqTile - 1) / kAwqTile;
  const int tile_raw = blockIdx.x * 2 + tl;
  const int tile = min(tile_raw, ntiles - 1);
  const int m = lane & 15, qtr = lane >> 4;
  const int n = tile * kAwqTile + (lane & 15);
  const uint8_t *qbase = qd + (int64_t)tile * P * kAwqBlockBytes + lane * 16;
  const uint32_t *szrow = sz + (int64_t)n * G4;
  extern __shared__ __attribute__((aligned(16))) uint8_t awq_lds[];
  constexpr int npr = kAwqWideChunk * (kGroup / 8);    // 16-byte pieces per row of a chunk
  const int npc = M * npr;
  const int rounds = (npc + 127) / 128;                // copies per thread per chunk (two wavefronts)
  const int buf_bytes = rounds * 2048;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)awq_lds;
  v4f acc = v4f{};
  // chunk c of this half (groups g0 + 4c + [0, 4), the layer's last group
  // repeated past G) into the half's buffer `buf`
  auto copy_x = [&](int c, int buf) {
    const int gc = g0 + c * kAwqWideChunk;
    const uint32_t base = lds0 + (uint32_t)((2 * h + buf) * buf_bytes);
    for (int r = 0; r < rounds; ++r) {
      const int p0 = 128 * r + 64 * tl;                // this wavefront's 64 pieces
      const int pc = min(p0 + lane, npc - 1);
      const int mr = pc / npr, o = pc - mr * npr;
      const int gi = min(gc + o / 8, G - 1);
      lds_dma16(x + (int64_t)mr * K + gi * kGroup + (o % 8) * 8, base + (uint32_t)(p0 * 16));
    }
  };
  for (int sc = 0; sc < nch; sc += kAwqWideChunks) {
    const int nc = min(kAwqWideChunks, nch - sc);
    __syncthreads();                                   // the previous super-chunk is done with the LDS
    uint4 cw[kAwqWideChunks][kAwqWideChunk / 2], szw[kAwqWideChunks];
#pragma unroll
    for (int k = 0; k < kAwqWideChunks; ++k) {
      const int gc = min(g0 + min(sc + k, nch - 1) * kAwqWideChunk, G - 1) & ~3;
#pragma unroll
      for (int j = 0; j < kAwqWideChunk / 2; ++j)
        cw[k][j] = *reinterpret_cast<const uint4 *>(qbase + (int64_t)min(gc / 2 + j, P - 1) * kAwqBlockBytes);
      szw[k] = *reinterpret_cast<const uint4 *>(szrow + gc);
    }
    // the copies follow the code loads in issue order (the waits below
    // count on it): their LDS buffer index takes an offset from an empty
    // asm placed after the loads
    int zero = 0;
    asm volatile("" : "+s"(zero) :: "memory");
    copy_x(sc, zero);
#pragma unroll
    for (int k = 0; k < kAwqWideChunks; ++k) {
      if (k >= nc) break;
      if (k > 0) __syncthreads();                      // chunk k - 1 is done with buffer (k + 1) % 2
      if (k + 1 < nc) {
        copy_x(sc + k + 1, (k + 1) & 1);
        vmcnt_wait_dyn(rounds);
      } else {
        vmcnt_wait0_known();
      }
      __syncthreads();                                 // both wavefronts' copies of chunk k are in
      const int gc = g0 + (sc + k) * kAwqWideChunk;
      const uint16_t *xm = reinterpret_cast<const uint16_t *>(awq_lds + (2 * h + (k & 1)) * buf_bytes) +
                           min(m, M - 1) * (npr * 8) + 16 * qtr;
#pragma unroll
      for (int i = 0; i < kAwqWideChunk; ++i) {
        const uint4 q4 = szw[k];
        const uint32_t szv = (i == 0) ? q4.x : (i == 1) ? q4.y : (i == 2) ? q4.z : q4.w;
        const uint4 cc = cw[k][i / 2];
        awq_group(xm + i * kGroup, i % 2 == 0 ? cc.x : cc.z, i % 2 == 0 ? cc.y : cc.w, szv,
                  gc + i < G && gc + i < g0 + Gh, acc);
      }
    }
  }
  __syncthreads();                                     // the buffers are free for the reduction
  v4f *red = reinterpret_cast<v4f *>(awq_lds);
  if (h == 1) red[tl * 64 + lane] = acc;
  __syncthreads();
  if (h == 1) return;
  const v4f other = red[tl * 64 + lane];
  const int col = tile_raw * kAwqTile + (lane & 15);
  if (tile_raw < ntiles && col < N) {
    const float b = bias ? (float)__builtin_bit_cast(_Float16, bias[col]) : 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * (lane >> 4) + e;
      if (row < M) y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)((acc[e] + other[e]) + b));
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
__global__ void canon_codes_kernel(const uint8_t *__restrict__ qa, int M, int K, int T,
                                   uint8_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nb = (int64_t)M * (K / 2);
  if (idx >= nb) return;
  const int64_t m = idx / (K / 2), kb = idx % (K / 2);
  int code[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const CodePos cp = code_pos(m, 2 * kb + u);
    const uint32_t *wp = reinterpret_cast<const uint32_t *>(qa + pair_offset(cp.g, cp.t, T, cp.lane, 0));
    // the lane's words 0..5 live as pairs 512 bytes apart
    const int bit = 6 * cp.c, wi = bit / 32, sh = bit % 32;
    const uint32_t w0 = wp[(wi / 2) * 128 + (wi & 1)];
    uint32_t v = w0 >> sh;
    if (sh > 26) {
      const int wj = wi + 1;
      v |= wp[(wj / 2) * 128 + (wj & 1)] << (32 - sh);
    }
    code[u] = int_of_e2m3(v & 63u);
  }
  out[idx] = (uint8_t)(((uint32_t)code[0] & 0x0Fu) | (((uint32_t)code[1] & 0x0Fu) << 4));
}

__global__ void canon_scales_kernel(const float *__restrict__ sa, int M, int Mp, int G,
                                    float *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * G) return;
  const int64_t m = idx / G, g = idx % G;
  out[idx] = sa[g * Mp + m];
}

// MXFP4 codes and scales of the workspace -> canonical [M, K/2] bytes and
// [M, K/32] E8M0 bytes.  Byte j of row m sits in lane (m % 32) + 32 h of
// block (j / 32, m / 32), h = (j % 32) / 16, at byte j % 16.
__global__ void canon_mx_codes_kernel(const uint8_t *__restrict__ qa, int M, int K, int T,
                                      uint8_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * (K / 2)) return;
  const int64_t m = idx / (K / 2), j = idx % (K / 2);
  const int lane = (int)(m % 32) + 32 * (int)((j % 32) / 16);
  out[idx] = qa[mx_code_offset(j / 32, m / 32, T, lane) + j % 16];
}

__global__ void canon_mx_scales_kernel(const uint8_t *__restrict__ sa, int M, int K, int T,
                                       uint8_t *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int B = K / kMxBlock;
  if (idx >= (int64_t)M * B) return;
  const int64_t m = idx / B, b = idx % B;
  out[idx] = sa[mx_scale_offset(b / 2, m / 32, T, (int)(m % 32) + 32 * (int)(b % 2))];
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

template <bool MX = false, class WL, class KL>
svdq_status_t launch_k1(const WL &L, const KL &Wl, const svdq_weights_t *w,
                        const void *X, int M, uint8_t *ws, hipStream_t st,
                        int64_t *dzero = nullptr, int rpz = 0) {
  const uint8_t *blob = static_cast<const uint8_t *>(w->blob);
  const dim3 grid((unsigned)(Wl.Mp / kTile), (unsigned)Wl.S);
  const uint16_t *x = static_cast<const uint16_t *>(X);
  const float *iota = reinterpret_cast<const float *>(blob + L.iota);
  const uint16_t *l1t = reinterpret_cast<const uint16_t *>(blob + L.l1t);
  uint8_t *qa = ws + Wl.qa;
  float *sa = reinterpret_cast<float *>(ws + Wl.sa);
  float *dp = reinterpret_cast<float *>(ws + Wl.d);
  const int K = w->K, Mp = (int)Wl.Mp, S = (int)Wl.S;
  const size_t lds = 0;
  switch (L.rp / 32) {
#define K1_CASE(TB)                                                                       \
  case TB:                                                                                \
    hipLaunchKernelGGL((k1_quantize_lowrank_down<TB, MX>), grid, dim3(256), lds, st, x, M, K, Mp, \
                       S, iota, l1t, qa, sa, dp, dzero, rpz);                             \
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
  a.qa = ws + Wl.qa;
  a.sa = reinterpret_cast<const float *>(ws + Wl.sa);
  a.dpart = reinterpret_cast<const float *>(ws + Wl.d);
  a.S = (int)Wl.S;
  a.M = M;
  a.Mp = (int)Wl.Mp;
  a.qw = blob + L.q;
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
  if (M < 1 || (int64_t)M * w->K > ((int64_t)1 << 31))
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

// Input D of the GEMM: fp32 partials from the quantiser, or one fixed-point
// sum written by the previous layer's fused epilogue.  Output: Y, or (w2 set)
// the next layer's codes, scales and D in ws2.
enum K2In { K2_D_PARTIALS = 0, K2_D_FIXED = 1 };
static svdq_status_t launch_k2(const svdq_weights_t *w, int M, void *Y, svdq_dtype_t y_dtype,
                               svdq_epilogue_t epilogue, const void *workspace, hipStream_t stream,
                               K2In din = K2_D_PARTIALS, const svdq_weights_t *w2 = nullptr,
                               void *ws2 = nullptr, size_t ws_bytes = 0) {
  const WeightLayout L(w->N, w->K, w->rank);
  const WorkLayout Wl(M, w->K, w->rank);
  K2Args a = make_k2_args(L, Wl, w, M, static_cast<const uint8_t *>(workspace));
  a.Y = Y;
  a.TM = (M + k2c::BM - 1) / k2c::BM;
  a.TN = (w->N + k2c::BN - 1) / k2c::BN;
  a.dfix = reinterpret_cast<const int64_t *>(static_cast<const uint8_t *>(workspace) + Wl.d);
  if (w2) {
    const WeightLayout L2(w2->N, w2->K, w2->rank);
    const WorkLayout W2(M, w2->K, w2->rank);
    const uint8_t *b2 = static_cast<const uint8_t *>(w2->blob);
    uint8_t *s2 = static_cast<uint8_t *>(ws2);
    a.iota2 = reinterpret_cast<const float *>(b2 + L2.iota);
    a.l1f2 = reinterpret_cast<const uint16_t *>(b2 + L2.l1t);
    a.qa2 = s2 + W2.qa;
    a.sa2 = reinterpret_cast<float *>(s2 + W2.sa);
    a.d2 = reinterpret_cast<int64_t *>(s2 + W2.d);
    a.G2 = (int)W2.G;
    a.rp2 = (int)W2.rp;
  }
  const dim3 block(k2c::THREADS);
  const bool f32 = y_dtype == SVDQ_FP32;
  const bool gelu = epilogue == SVDQ_EPILOGUE_GELU_TANH;
  constexpr int NONE = SVDQ_EPILOGUE_NONE, GELU = SVDQ_EPILOGUE_GELU_TANH;
  // K-split when the tile grid leaves the chip idle and the workspace has
  // room for the partials (svdq_workspace_bytes includes it)
  const int ks = (int)k2_ksplit(M, w->N, w->K);
  if (!w2 && ks > 1 && (int64_t)ws_bytes >= Wl.total + k2_split_bytes(M, w->N, w->K)) {
    a.ksplit = ks;
    a.part = reinterpret_cast<float *>(static_cast<uint8_t *>(const_cast<void *>(workspace)) + Wl.total);
    const dim3 sgrid((unsigned)round_up((int64_t)a.TM * a.TN * ks, 8));
    if (din == K2_D_FIXED)
      hipLaunchKernelGGL((k2_w4a4_gemm<MODE_FWD, NONE, true, true, false, true>), sgrid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((k2_w4a4_gemm<MODE_FWD, NONE, true, false, false, true>), sgrid, block, 0, stream, a);
    svdq_status_t st = launch_status("GEMM kernel launch");
    if (st != SVDQ_OK) return st;
    const int64_t threads = (int64_t)M * (L.Np / 4);
    const dim3 rgrid((unsigned)((threads + 255) / 256));
#define K2_SUM(E, F) hipLaunchKernelGGL((k2_split_sum<E, F>), rgrid, dim3(256), 0, stream, a.part, ks, M, \
                                        w->N, (int)Wl.Mp, (int)L.Np, a.bias, Y)
    if (!gelu && f32) K2_SUM(NONE, true);
    else if (!gelu) K2_SUM(NONE, false);
    else if (f32) K2_SUM(GELU, true);
    else K2_SUM(GELU, false);
#undef K2_SUM
    return launch_status("K-split sum launch");
  }
  const dim3 grid((unsigned)round_up((int64_t)a.TM * a.TN, 8));
#define K2_GO(E, F, DF, QN) hipLaunchKernelGGL((k2_w4a4_gemm<MODE_FWD, E, F, DF, QN>), grid, block, 0, stream, a)
  if (w2) {
    if (din == K2_D_FIXED) return fail(SVDQ_ERR_INVALID_ARGUMENT, "chained fused epilogues are not supported");
    if (gelu) K2_GO(GELU, false, false, true); else K2_GO(NONE, false, false, true);
  } else if (din == K2_D_FIXED) {
    if (!gelu && f32) K2_GO(NONE, true, true, false);
    else if (!gelu) K2_GO(NONE, false, true, false);
    else if (f32) K2_GO(GELU, true, true, false);
    else K2_GO(GELU, false, true, false);
  } else {
    if (!gelu && f32) K2_GO(NONE, true, false, false);
    else if (!gelu) K2_GO(NONE, false, false, false);
    else if (f32) K2_GO(GELU, true, false, false);
    else K2_GO(GELU, false, false, false);
  }
#undef K2_GO
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
  return launch_k2(w, M, Y, y_dtype, epilogue, workspace, static_cast<hipStream_t>(hip_stream),
                   K2_D_PARTIALS, nullptr, nullptr, ws_bytes);
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
  return launch_k2(w, M, Y, y_dtype, epilogue, workspace, stream, K2_D_PARTIALS, nullptr, nullptr,
                   ws_bytes);
}

static svdq_status_t validate_pair(const svdq_weights_t *w1, const svdq_weights_t *w2, int M,
                                   size_t ws1_bytes, const void *ws1, size_t ws2_bytes,
                                   const void *ws2, const char *who) {
  svdq_status_t st = validate_forward(w1, M, ws1_bytes, ws1, who);
  if (st != SVDQ_OK) return st;
  if ((st = validate_forward(w2, M, ws2_bytes, ws2, who)) != SVDQ_OK) return st;
  if (w2->K != w1->N)
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: second layer's K=%d != first layer's N=%d", who,
                w2->K, w1->N);
  if (ws1 == ws2) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: the two workspaces must differ", who);
  return check_device();
}

svdq_status_t svdq_mlp_quantize(const svdq_weights_t *w1, const svdq_weights_t *w2, const void *X,
                                int M, void *ws1, size_t ws1_bytes, void *ws2, size_t ws2_bytes,
                                void *hip_stream) {
  svdq_status_t st = validate_pair(w1, w2, M, ws1_bytes, ws1, ws2_bytes, ws2, "svdq_mlp_quantize");
  if (st != SVDQ_OK) return st;
  if (!X) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mlp_quantize: NULL X");
  if (!aligned16(X)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mlp_quantize: misaligned X");
  const WeightLayout L(w1->N, w1->K, w1->rank);
  const WorkLayout Wl(M, w1->K, w1->rank);
  const WorkLayout W2(M, w2->K, w2->rank);
  int64_t *dz = W2.rp > 0 ? reinterpret_cast<int64_t *>(static_cast<uint8_t *>(ws2) + W2.d) : nullptr;
  return launch_k1(L, Wl, w1, X, M, static_cast<uint8_t *>(ws1), static_cast<hipStream_t>(hip_stream),
                   dz, (int)W2.rp);
}

svdq_status_t svdq_mlp_gemm1(const svdq_weights_t *w1, const svdq_weights_t *w2, int M,
                             svdq_epilogue_t epilogue, const void *ws1, size_t ws1_bytes,
                             void *ws2, size_t ws2_bytes, void *hip_stream) {
  svdq_status_t st = validate_pair(w1, w2, M, ws1_bytes, ws1, ws2_bytes, ws2, "svdq_mlp_gemm1");
  if (st != SVDQ_OK) return st;
  if (epilogue != SVDQ_EPILOGUE_NONE && epilogue != SVDQ_EPILOGUE_GELU_TANH)
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mlp_gemm1: unknown epilogue %d", (int)epilogue);
  return launch_k2(w1, M, nullptr, SVDQ_BF16, epilogue, ws1, static_cast<hipStream_t>(hip_stream),
                   K2_D_PARTIALS, w2, ws2);
}

svdq_status_t svdq_mlp_gemm2(const svdq_weights_t *w2, int M, void *Y, svdq_dtype_t y_dtype,
                             const void *ws2, size_t ws2_bytes, void *hip_stream) {
  svdq_status_t st = validate_forward(w2, M, ws2_bytes, ws2, "svdq_mlp_gemm2");
  if (st != SVDQ_OK) return st;
  if ((st = validate_output(Y, y_dtype, SVDQ_EPILOGUE_NONE, "svdq_mlp_gemm2")) != SVDQ_OK) return st;
  if ((st = check_device()) != SVDQ_OK) return st;
  return launch_k2(w2, M, Y, y_dtype, SVDQ_EPILOGUE_NONE, ws2, static_cast<hipStream_t>(hip_stream),
                   K2_D_FIXED, nullptr, nullptr, ws2_bytes);
}

svdq_status_t svdq_mlp_forward(const svdq_weights_t *w1, const svdq_weights_t *w2, const void *X,
                               int M, void *Y, svdq_dtype_t y_dtype, svdq_epilogue_t epilogue,
                               void *ws1, size_t ws1_bytes, void *ws2, size_t ws2_bytes,
                               void *hip_stream) {
  svdq_status_t st = validate_output(Y, y_dtype, epilogue, "svdq_mlp_forward");
  if (st != SVDQ_OK) return st;
  if ((st = svdq_mlp_quantize(w1, w2, X, M, ws1, ws1_bytes, ws2, ws2_bytes, hip_stream)) != SVDQ_OK)
    return st;
  if ((st = svdq_mlp_gemm1(w1, w2, M, epilogue, ws1, ws1_bytes, ws2, ws2_bytes, hip_stream)) != SVDQ_OK)
    return st;
  return svdq_mlp_gemm2(w2, M, Y, y_dtype, ws2, ws2_bytes, hip_stream);
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
                     ws + Wl.qa, M, w->K, (int)(Wl.Mp / kTile), qact);
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
  a.tile_m0 = m0 / k2c::BM * k2c::BM;
  a.tile_n0 = n0 / k2c::BN * k2c::BN;
  a.TM = (m0 + mcount - a.tile_m0 + k2c::BM - 1) / k2c::BM;
  a.TN = (n0 + ncount - a.tile_n0 + k2c::BN - 1) / k2c::BN;
  const dim3 grid((unsigned)round_up((int64_t)a.TM * a.TN, 8));
  hipLaunchKernelGGL((k2_w4a4_gemm<MODE_SUMS, SVDQ_EPILOGUE_NONE, true>), grid, dim3(k2c::THREADS), 0,
                     static_cast<hipStream_t>(hip_stream), a);
  return launch_status("group-sum kernel launch");
}

// ------------------------------------------------------------- MXFP4
static svdq_status_t validate_forward_mx(const svdq_weights_t *w, int M, size_t ws_bytes,
                                         const void *workspace, const char *who) {
  svdq_status_t st = validate_weights(w, who);
  if (st != SVDQ_OK) return st;
  if (!workspace) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: NULL workspace", who);
  if (!aligned16(workspace)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "%s: misaligned workspace", who);
  if (M < 1 || (int64_t)M * w->K > ((int64_t)1 << 31))
    return fail(SVDQ_ERR_UNSUPPORTED_SHAPE, "%s: M=%d", who, M);
  const MxWorkLayout Wl(M, w->K, w->rank);
  if ((int64_t)ws_bytes < Wl.total)
    return fail(SVDQ_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %lld bytes, got %zu", who,
                (long long)Wl.total, ws_bytes);
  return SVDQ_OK;
}

static svdq_status_t launch_k2_mx(const svdq_weights_t *w, int M, void *Y, svdq_dtype_t y_dtype,
                                  svdq_epilogue_t epilogue, const void *workspace, hipStream_t stream) {
  const MxWeightLayout L(w->N, w->K, w->rank);
  const MxWorkLayout Wl(M, w->K, w->rank);
  const uint8_t *blob = static_cast<const uint8_t *>(w->blob);
  const uint8_t *ws = static_cast<const uint8_t *>(workspace);
  K2Args a{};
  a.qa = ws + Wl.qa;
  a.sqa = ws + Wl.sa;
  a.dpart = reinterpret_cast<const float *>(ws + Wl.d);
  a.S = (int)Wl.S;
  a.M = M;
  a.Mp = (int)Wl.Mp;
  a.qw = blob + L.q;
  a.sqw = blob + L.s;
  a.l2t = reinterpret_cast<const uint16_t *>(blob + L.l2t);
  a.bias = reinterpret_cast<const float *>(blob + L.bias);
  a.N = w->N;
  a.Np = (int)L.Np;
  a.K = w->K;
  a.rp = (int)L.rp;
  a.Y = Y;
  a.TM = (M + k2c::BM - 1) / k2c::BM;
  a.TN = (w->N + k2c::BN - 1) / k2c::BN;
  const dim3 grid((unsigned)round_up((int64_t)a.TM * a.TN, 8));
  const dim3 block(k2c::THREADS);
  const bool f32 = y_dtype == SVDQ_FP32;
  const bool gelu = epilogue == SVDQ_EPILOGUE_GELU_TANH;
  constexpr int NONE = SVDQ_EPILOGUE_NONE, GELU = SVDQ_EPILOGUE_GELU_TANH;
  if (!gelu && f32) hipLaunchKernelGGL((k2_w4a4_gemm<MODE_MX, NONE, true>), grid, block, 0, stream, a);
  else if (!gelu) hipLaunchKernelGGL((k2_w4a4_gemm<MODE_MX, NONE, false>), grid, block, 0, stream, a);
  else if (f32) hipLaunchKernelGGL((k2_w4a4_gemm<MODE_MX, GELU, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((k2_w4a4_gemm<MODE_MX, GELU, false>), grid, block, 0, stream, a);
  return launch_status("FP4 GEMM kernel launch");
}

svdq_status_t svdq_mx_linear_quantize(const svdq_weights_t *w, const void *X, int M, void *workspace,
                                      size_t ws_bytes, void *hip_stream) {
  svdq_status_t st = validate_forward_mx(w, M, ws_bytes, workspace, "svdq_mx_linear_quantize");
  if (st != SVDQ_OK) return st;
  if (!X) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mx_linear_quantize: NULL X");
  if (!aligned16(X)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mx_linear_quantize: misaligned X");
  if ((st = check_device()) != SVDQ_OK) return st;
  return launch_k1<true>(MxWeightLayout(w->N, w->K, w->rank), MxWorkLayout(M, w->K, w->rank), w, X, M,
                         static_cast<uint8_t *>(workspace), static_cast<hipStream_t>(hip_stream));
}

svdq_status_t svdq_mx_linear_gemm(const svdq_weights_t *w, int M, void *Y, svdq_dtype_t y_dtype,
                                  svdq_epilogue_t epilogue, const void *workspace, size_t ws_bytes,
                                  void *hip_stream) {
  svdq_status_t st = validate_forward_mx(w, M, ws_bytes, workspace, "svdq_mx_linear_gemm");
  if (st != SVDQ_OK) return st;
  if ((st = validate_output(Y, y_dtype, epilogue, "svdq_mx_linear_gemm")) != SVDQ_OK) return st;
  if ((st = check_device()) != SVDQ_OK) return st;
  return launch_k2_mx(w, M, Y, y_dtype, epilogue, workspace, static_cast<hipStream_t>(hip_stream));
}

svdq_status_t svdq_mx_linear_forward(const svdq_weights_t *w, const void *X, int M, void *Y,
                                     svdq_dtype_t y_dtype, svdq_epilogue_t epilogue, void *workspace,
                                     size_t ws_bytes, void *hip_stream) {
  svdq_status_t st = validate_output(Y, y_dtype, epilogue, "svdq_mx_linear_forward");
  if (st != SVDQ_OK) return st;
  if ((st = svdq_mx_linear_quantize(w, X, M, workspace, ws_bytes, hip_stream)) != SVDQ_OK) return st;
  return launch_k2_mx(w, M, Y, y_dtype, epilogue, workspace, static_cast<hipStream_t>(hip_stream));
}

svdq_status_t svdq_mx_quantize_activations(const svdq_weights_t *w, const void *X, int M,
                                           uint8_t *qact, uint8_t *ascales, float *lowrank_down,
                                           void *workspace, size_t ws_bytes, void *hip_stream) {
  svdq_status_t st = validate_forward_mx(w, M, ws_bytes, workspace, "svdq_mx_quantize_activations");
  if (st != SVDQ_OK) return st;
  if (!X || !qact || !ascales || (w->rank > 0 && !lowrank_down))
    return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mx_quantize_activations: NULL pointer");
  if (!aligned16(X)) return fail(SVDQ_ERR_INVALID_ARGUMENT, "svdq_mx_quantize_activations: misaligned X");
  if ((st = check_device()) != SVDQ_OK) return st;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const MxWorkLayout Wl(M, w->K, w->rank);
  uint8_t *ws = static_cast<uint8_t *>(workspace);
  if ((st = launch_k1<true>(MxWeightLayout(w->N, w->K, w->rank), Wl, w, X, M, ws, stream)) != SVDQ_OK)
    return st;
  const int T = (int)(Wl.Mp / kTile);
  const int64_t nb = (int64_t)M * (w->K / 2);
  hipLaunchKernelGGL(canon_mx_codes_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, stream,
                     ws + Wl.qa, M, w->K, T, qact);
  const int64_t ns = (int64_t)M * (w->K / kMxBlock);
  hipLaunchKernelGGL(canon_mx_scales_kernel, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, stream,
                     ws + Wl.sa, M, w->K, T, ascales);
  if (w->rank > 0) {
    const int64_t nd = (int64_t)M * w->rank;
    hipLaunchKernelGGL(canon_down_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<const float *>(ws + Wl.d), M, (int)Wl.Mp, (int)Wl.S,
                       (int)Wl.rp, w->rank, lowrank_down);
  }
  return launch_status("inspection kernels");
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
  const int pieces = M * kAwqChunk * (kGroup / 8);     // 16-byte copies of a chunk's activations
  if (M <= kAwqWideMinRows - 1) {
    // per wavefront: M rows of a chunk, in whole 1 KB copies
    const size_t lds = (size_t)4 * ((pieces + 63) / 64 * 1024);
    hipLaunchKernelGGL(k3_awq_w4a16, dim3((unsigned)(L.Np / kAwqTile)), dim3(256), lds,
                       static_cast<hipStream_t>(hip_stream), b + L.q,
                       reinterpret_cast<const uint32_t *>(b + L.sz), static_cast<const uint16_t *>(x), M,
                       N, K, static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(y));
  } else {
    // per workgroup: two halves x two buffers of a 4-group chunk's
    // activations, in whole 2 KB rounds (also holds the reduction's 2 KB)
    const int wpieces = M * kAwqWideChunk * (kGroup / 8);
    const size_t lds = (size_t)4 * ((wpieces + 127) / 128 * 2048);
    const int64_t tiles = L.Np / kAwqTile;
    hipLaunchKernelGGL(k3_awq_w4a16_wide, dim3((unsigned)((tiles + 1) / 2)),
                       dim3(256), lds, static_cast<hipStream_t>(hip_stream), b + L.q,
                       reinterpret_cast<const uint32_t *>(b + L.sz), static_cast<const uint16_t *>(x), M,
                       N, K, static_cast<const uint16_t *>(bias), static_cast<uint16_t *>(y));
  }
  return launch_status("AWQ kernel launch");
}

}  // extern "C"
