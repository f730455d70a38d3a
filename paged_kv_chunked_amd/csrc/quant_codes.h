// INT8 / INT4 codes to fp16, exactly (every code is a small integer).
#pragma once

#include "fp16_shape.h"

namespace pkv {
namespace {

// 8 int8 codes (two words, lowest byte first) to fp16: byte b becomes the fp16
// with bits 0x6400 | (b ^ 0x80), i.e. 1024 + 128 + code, minus 1152.
__device__ inline half8_t codes_to_half(uint32_t lo, uint32_t hi) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  const uint32_t c = 0x64646464u;
  // byte selectors: result bytes [a0, 0x64, a1, 0x64] etc. (perm indexes the
  // 8 bytes {src1 (0..3), src0 (4..7)})
  const uint32_t w0 = __builtin_amdgcn_perm(c, a, 0x05010400u);
  const uint32_t w1 = __builtin_amdgcn_perm(c, a, 0x05030402u);
  const uint32_t w2 = __builtin_amdgcn_perm(c, b, 0x05010400u);
  const uint32_t w3 = __builtin_amdgcn_perm(c, b, 0x05030402u);
  half8_t h = __builtin_bit_cast(half8_t, u32x4{w0, w1, w2, w3});
  return h - (half8_t)(_Float16)1152.f;
}

// The low nibbles of the 8 bytes of (lo, hi), two's-complement 4-bit codes,
// to fp16: nibble n becomes 1024 + (n ^ 8), minus 1032.
__device__ inline half8_t nibbles_to_half(uint32_t lo, uint32_t hi) {
  const uint32_t a = (lo & 0x0F0F0F0Fu) ^ 0x08080808u, b = (hi & 0x0F0F0F0Fu) ^ 0x08080808u;
  const uint32_t c = 0x64646464u;
  const uint32_t w0 = __builtin_amdgcn_perm(c, a, 0x05010400u);
  const uint32_t w1 = __builtin_amdgcn_perm(c, a, 0x05030402u);
  const uint32_t w2 = __builtin_amdgcn_perm(c, b, 0x05010400u);
  const uint32_t w3 = __builtin_amdgcn_perm(c, b, 0x05030402u);
  half8_t h = __builtin_bit_cast(half8_t, u32x4{w0, w1, w2, w3});
  return h - (half8_t)(_Float16)1032.f;
}

}  // namespace
}  // namespace pkv
