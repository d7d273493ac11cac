// Device data layouts shared by the host packer and the device kernels.
// Everything here is constexpr so the same definitions serve both sides.
//
// INT4 codes live on the device as 6-bit floating-point values (OCP FP6
// E2M3: sign, 2 exponent bits with bias 1, 3 mantissa bits), which hold the
// integers -7..7 exactly and are the native operand of gfx950's fp6 matrix
// instructions.  Rows (tokens for activations, output channels for weights)
// are cut into tiles of 32; for every (group g of 64 input channels, tile t)
// one 1536-byte block holds 32 codes for each of the 64 lanes of a
// wavefront.  Lane l covers row l % 32 of the tile and half h = l / 32 of the
// group; its code c (0..31) is input channel
//     k = 64 g + 16 (c / 8) + 8 h + (c % 8)
// and sits at bits 6c..6c+5 of the lane's 192-bit little-endian word string.
// Inside the block, 8-byte word pair j (j = 0..2) of lane l is at byte
// 512 j + 8 l, so every pair is one coalesced 512-byte line per wavefront.
// Activations and weights use the identical assignment, which is all the
// integer dot products need: a group's sum does not depend on how its 64
// channels are ordered as long as both operands agree.
#pragma once

#include <stdint.h>

namespace svdq {

constexpr int kGroup = 64;
constexpr int kTile = 32;
constexpr int kPad = 256;                // M and N are padded to multiples of this
constexpr int kLaneBytes = 24;           // 32 fp6 codes per lane
constexpr int kBlockBytes = 64 * kLaneBytes;
constexpr int64_t kAlign = 256;
constexpr double kDFixScale = 4294967296.0;   // 2^32: fixed-point unit of a fused D sum

constexpr int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
constexpr int rank_pad(int rank) { return rank <= 0 ? 0 : (int)round_up(rank, 32); }

// input channel (within the group) of code c held by half h
constexpr int lane_code_k(int h, int c) { return 16 * (c >> 3) + 8 * h + (c & 7); }

// where the code for (row, k) lives: block (g, t), lane, code index c
struct CodePos { int64_t g, t; int lane, c; };
constexpr CodePos code_pos(int64_t row, int64_t k) {
  return CodePos{k / kGroup, row / kTile, (int)(row % kTile) + 32 * (int)((k % 16) / 8),
                 8 * (int)((k % kGroup) / 16) + (int)(k % 8)};
}

// byte offset of 8-byte word pair j of `lane` in block (g, t), T tiles
constexpr int64_t pair_offset(int64_t g, int64_t t, int64_t T, int lane, int j) {
  return (g * T + t) * kBlockBytes + (int64_t)j * 512 + (int64_t)lane * 8;
}

// FP6 E2M3 encoding of an integer code in [-7, 7]
constexpr uint32_t e2m3_of_int(int q) {
  const int a = q < 0 ? -q : q;
  const uint32_t mag = a == 0 ? 0u : a == 1 ? 8u : a < 4 ? (uint32_t)(8 + 4 * a) : (uint32_t)(16 + 2 * a);
  return (q < 0 ? 0x20u : 0u) | mag;
}

// integer value of an FP6 E2M3 code that holds an integer
constexpr int int_of_e2m3(uint32_t v) {
  const int e = (int)((v >> 3) & 3u), m = (int)(v & 7u);
  const int mag = e == 0 ? 0 : ((8 + m) << (e - 1)) / 8;
  return (v & 0x20u) ? -mag : mag;
}

// Group scales are stored as matrix-core operands.  A float32 scale s splits
// exactly into three bf16 pieces, s = s1 + s2 + s3: s1 = s with the low 16
// bits of its encoding cleared, s2 the same of s - s1, s3 = s - s1 - s2
// (each subtraction exact; s3 has at most 8 significant bits).  The GEMM
// forms sA sW for a 32 x 32 tile with one 32x32x8 bf16 matrix instruction
// whose eight K slots hold
//     activation row m:   a1 a1 a1 a2 | a2 a2 a3 a3
//     weight column n:    b1 b2 b3 b1 | b2 b3 b1 b2
// (slots 0..3 in lanes 0..31, slots 4..7 in lanes 32..63), so the sum of
// the eight exact products is sA sW - a3 b3 (a3 b3 < 2^-32 sA sW).  Each row
// or column takes 16 bytes, the bf16 values in that order: a lane reads the
// 8-byte half of its lane half.
constexpr int kScaleOpBytes = 16;

// The down-projection factor L1s [K][rp] is stored in the order in which the
// quantiser's matrix instruction consumes it (B operand of a 32x32x16 bf16
// product, one 32-rank block b at a time): for group g, block b and 16-channel
// step j, 64 lanes x 8 bf16 form one contiguous 1 KB piece; lane l holds rank
// 32 b + l % 32 at channels 64 g + 16 j + 8 (l / 32) + [0, 8).  Element index
// (in bf16 units) of (channel k, rank t):
constexpr int64_t l1_frag_index(int64_t k, int64_t t, int64_t rp) {
  return ((((k / kGroup) * (rp / 32) + t / 32) * 4 + (k % kGroup) / 16) * 64 + t % 32 +
          32 * ((k % 16) / 8)) * 8 + k % 8;
}

// Device weight blob of one prepared layer.
struct WeightLayout {
  int64_t N = 0, K = 0, rank = 0, Np = 0, rp = 0, G = 0;
  int64_t q = 0, s = 0, l2t = 0, l1t = 0, iota = 0, bias = 0, total = 0;
  constexpr WeightLayout(int64_t N_, int64_t K_, int64_t rank_)
      : N(N_), K(K_), rank(rank_), Np(round_up(N_, kPad)), rp(rank_pad((int)rank_)),
        G(K_ / kGroup) {
    int64_t o = 0;
    q = o;    o = round_up(o + Np * K * 3 / 4, kAlign);  // fp6 codes, tiled
    s = o;    o = round_up(o + G * Np * kScaleOpBytes, kAlign);   // scale operands [G][Np]
    l2t = o;  o = round_up(o + Np * rp * 2, kAlign);     // bf16 L2^T [Np][rp]
    l1t = o;  o = round_up(o + rp * K * 2, kAlign);      // bf16 L1s, MFMA fragment order (l1_frag_index)
    iota = o; o = round_up(o + K * 4, kAlign);           // fp32 1/lambda [K]
    bias = o; o = round_up(o + Np * 4, kAlign);          // fp32 [Np]
    total = o;
  }
};

// Groups of 64 handled by one quantiser workgroup: the K range is split S
// ways so that enough workgroups exist to keep every CU streaming (about 384:
// more, shorter splits lose more to each workgroup's start-up than they gain),
// with at least 4 groups per split (one per wavefront).  With a low-rank
// branch, splits hold at least 12 groups where K has them (three chunks of
// four, the depth of the quantiser's copy pipeline): every split adds a
// partial low-rank product that each GEMM workgroup holding a rank chunk has
// to sum.  At 1024 x 3072, r = 128, twelve splits of 4 groups took 10.4 +
// 48.0 us (quantiser + GEMM, back to back) against 9.6 + 40.5 us for four
// splits of 12 (6 splits: 8.5 + 45.2 us; 3 splits: 11.0 + 40.3 us); at
// rank 0 the twelve splits are faster (4.2 against 5.6 us for the quantiser
// alone).  The 4608-token shapes get 3 splits either way.
constexpr int64_t k1_splits(int64_t Mp, int64_t G, int64_t rank) {
  const int64_t T = Mp / kTile;
  const int64_t gmin = rank > 0 && G >= 12 ? 12 : 4;
  int64_t best = 1;
  for (int64_t s = 1; s <= G; ++s) {
    if (G % s != 0) continue;
    if (s == 1 || G / s >= gmin) best = s;
    if (G / s >= gmin && T * s >= 384) return s;
  }
  return best;
}

// Device workspace of one forward call.
struct WorkLayout {
  int64_t M = 0, Mp = 0, K = 0, G = 0, rp = 0, S = 0;
  int64_t qa = 0, sa = 0, d = 0, total = 0;
  constexpr WorkLayout(int64_t M_, int64_t K_, int64_t rank_)
      : M(M_), Mp(round_up(M_, kPad)), K(K_), G(K_ / kGroup), rp(rank_pad((int)rank_)),
        S(k1_splits(round_up(M_, kPad), K_ / kGroup, rank_)) {
    int64_t o = 0;
    qa = o; o = round_up(o + Mp * K * 3 / 4, kAlign);    // fp6 codes, tiled
    sa = o; o = round_up(o + G * Mp * kScaleOpBytes, kAlign);   // scale operands [G][Mp]
    // D = X L1s: either fp32 partials [S][Mp][rp] from the quantiser, or,
    // when the previous layer's GEMM quantised this layer's input in its
    // epilogue, one int64 fixed-point sum [Mp][rp] (units of 2^-32)
    d = o;  o = round_up(o + (S > 2 ? S : 2) * Mp * rp * 4, kAlign);
    total = o;
  }
};

// K-split of the INT4 GEMM.  A grid of fewer than 128 workgroup tiles
// (128 x 256) leaves most of the chip idle; such a GEMM is split along K
// into up to 8 ranges of at least 8 groups each, aiming at about 512
// workgroups.  (From 128 tiles on, the partials' traffic costs more than
// the idle CUs: measured at 144 tiles, 52.6 us split against 49.1.)
// Each range's fp32 partial tile goes to the workspace ([ksplit][Mp][Np]
// after the quantiser's part), and a second kernel sums the ranges in order
// and adds the bias (+ GELU).
constexpr int kK2TileM = 128, kK2TileN = 256;
constexpr int64_t k2_ksplit(int64_t M, int64_t N, int64_t K) {
  const int64_t T = ((M + kK2TileM - 1) / kK2TileM) * ((N + kK2TileN - 1) / kK2TileN);
  if (T >= 128) return 1;
  int64_t s = 512 / T;
  if (s > 8) s = 8;
  if (s > K / kGroup / 8) s = K / kGroup / 8;
  return s >= 2 ? s : 1;
}
// Narrow tiles (64 x 128 instead of 128 x 256) for grids of fewer than 128
// wide tiles whose narrow grid holds at least 256 tiles: no K-split, no
// partials.
#ifndef K2_NARROW
#define K2_NARROW 1
#endif
constexpr bool k2_narrow(int64_t M, int64_t N) {
  const int64_t wide = ((M + kK2TileM - 1) / kK2TileM) * ((N + kK2TileN - 1) / kK2TileN);
  const int64_t narrow = ((M + 63) / 64) * ((N + 127) / 128);
  return K2_NARROW && wide < 128 && narrow >= 256;
}
// bytes of the K-split partials after the quantiser's part of the workspace
constexpr int64_t k2_split_bytes(int64_t M, int64_t N, int64_t K) {
  const int64_t s = k2_ksplit(M, N, K);
  return s > 1 ? s * round_up(M, kPad) * round_up(N, kPad) * 4 : 0;
}

// MXFP4 device layouts (the FP4 form of the 4-bit path).  A K-step of 64
// input channels is one block-scaled FP4 matrix instruction: for every
// (K-step s, tile t of 32 rows) a 1 KB code block holds 16 bytes per lane;
// lane l covers row l % 32 and the MX block h = l / 32 of the step, its 32
// codes being channels 64 s + 32 h + [0, 32) in the canonical nibble order
// (byte i = code 2i | code 2i+1 << 4), i.e. the row's canonical bytes
// 32 s + 16 h + [0, 16).  The E8M0 scales sit in a separate array, 64
// bytes per (s, t), interleaved over 4 tiles: for the tiles 4q .. 4q + 3 of
// step s, a 256-byte block holds one 32-bit word per lane whose byte i is
// the lane's scale in tile 4q + i, so one word read gives a lane the scales
// of four tiles and the matrix instruction picks the byte.  T (a multiple of
// 8 after padding) keeps the blocks whole.
constexpr int kMxBlock = 32;
constexpr int64_t mx_code_offset(int64_t s, int64_t t, int64_t T, int lane) {
  return ((s * T + t) * 64 + lane) * 16;
}
constexpr int64_t mx_scale_offset(int64_t s, int64_t t, int64_t T, int lane) {
  return (s * T + (t & ~int64_t(3))) * 64 + lane * 4 + (t & 3);
}

struct MxWeightLayout {
  int64_t N = 0, K = 0, rank = 0, Np = 0, rp = 0, G = 0;
  int64_t q = 0, s = 0, l2t = 0, l1t = 0, iota = 0, bias = 0, total = 0;
  constexpr MxWeightLayout(int64_t N_, int64_t K_, int64_t rank_)
      : N(N_), K(K_), rank(rank_), Np(round_up(N_, kPad)), rp(rank_pad((int)rank_)),
        G(K_ / kGroup) {
    int64_t o = 0;
    q = o;    o = round_up(o + Np * K / 2, kAlign);        // E2M1 codes, tiled
    s = o;    o = round_up(o + Np * (K / kMxBlock), kAlign);  // E8M0 scales, tiled
    l2t = o;  o = round_up(o + Np * rp * 2, kAlign);       // as WeightLayout
    l1t = o;  o = round_up(o + rp * K * 2, kAlign);
    iota = o; o = round_up(o + K * 4, kAlign);
    bias = o; o = round_up(o + Np * 4, kAlign);
    total = o;
  }
};

struct MxWorkLayout {
  int64_t M = 0, Mp = 0, K = 0, G = 0, rp = 0, S = 0;
  int64_t qa = 0, sa = 0, d = 0, total = 0;
  constexpr MxWorkLayout(int64_t M_, int64_t K_, int64_t rank_)
      : M(M_), Mp(round_up(M_, kPad)), K(K_), G(K_ / kGroup), rp(rank_pad((int)rank_)),
        S(k1_splits(round_up(M_, kPad), K_ / kGroup, rank_)) {
    int64_t o = 0;
    qa = o; o = round_up(o + Mp * K / 2, kAlign);          // E2M1 codes, tiled
    sa = o; o = round_up(o + Mp * (K / kMxBlock), kAlign); // E8M0 scales, tiled
    d = o;  o = round_up(o + (S > 2 ? S : 2) * Mp * rp * 4, kAlign);   // fp32 partials of D
    total = o;
  }
};

// AWQ W4A16 device blob.  Output channels are cut into tiles of 16; for each
// (tile, pair of groups of 64) there is a 1024-byte block: lane l (column
// l % 16 of the tile, quarter q = l / 16 of a group) holds, in 16 bytes, the
// 16 codes of input channels 64 g + 16 q + [0, 16) of the pair's first group
// and then those of its second (zero past the last group), so one 16-byte
// load brings two groups.  Within each 4-byte word the low 16 bits hold the
// codes of the even channels (nibble j = channel 2j) and the high 16 bits
// those of the odd channels, so one shift and one mask turn a word into pairs
// of fp16 operands.  Scales and zero points follow as one 32-bit word per
// (column, group): fp16 scale | fp16 zero << 16, [Np][G4] with G4 = G rounded
// up to 4, so one 16-byte load brings a column's words for four groups.
constexpr int kAwqTile = 16;
constexpr int kAwqBlockBytes = 1024;   // a pair of groups

constexpr int64_t awq_pairs(int64_t G) { return (G + 1) / 2; }
constexpr int64_t awq_g4(int64_t G) { return round_up(G, 4); }

// byte offset and nibble shift of the code for (n, k)
constexpr int64_t awq_code_byte(int64_t n, int64_t k, int64_t G) {
  return ((n / kAwqTile) * awq_pairs(G) + k / kGroup / 2) * kAwqBlockBytes +
         ((n % kAwqTile) + 16 * ((k % kGroup) / 16)) * 16 + 8 * ((k / kGroup) % 2) +
         4 * ((k % 16) / 8) + (((k % 8) / 2) / 2) + 2 * (k % 2);
}
constexpr int awq_code_shift(int64_t k) { return 4 * (((k % 8) / 2) % 2); }

struct AwqLayout {
  int64_t N = 0, K = 0, G = 0, Np = 0;
  int64_t q = 0, sz = 0, total = 0;
  constexpr AwqLayout(int64_t N_, int64_t K_)
      : N(N_), K(K_), G(K_ / kGroup), Np(round_up(N_, kAwqTile)) {
    int64_t o = 0;
    q = o;  o = round_up(o + Np / kAwqTile * awq_pairs(G) * kAwqBlockBytes, kAlign);
    sz = o; o = round_up(o + Np * awq_g4(G) * 4, kAlign);
    total = o;
  }
};

}  // namespace svdq
