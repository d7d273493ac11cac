// Internal helpers shared by the host and device translation units.
#pragma once

#include <cstdint>
#include <cstring>

#include "svdq.h"

namespace svdq {

// Records a formatted message as this thread's last error and returns `s`.
svdq_status_t fail(svdq_status_t s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

inline float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

inline uint32_t f32_bits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

inline float f32_from_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// float16 <-> float32 (round to nearest even), finite inputs.
float f16_to_f32(uint16_t h);
uint16_t f32_to_f16(float f);
// float64 -> nearest bfloat16, ties to even, one rounding.
uint16_t f64_to_bf16(double x);

}  // namespace svdq
