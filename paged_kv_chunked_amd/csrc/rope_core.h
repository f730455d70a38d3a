// RoPE rotation of one pair and its rounding to the storage dtype, shared by
// the append kernels and the decode kernel that fuses the step's append
// (Kshipra part 3, section 4: RoPE at absolute positions).
#pragma once

#include "fp16_shape.h"

namespace pkv {
namespace {

template <typename T> __device__ inline T store_f64(double x);
// fp64 -> fp16 with one rounding (to nearest, ties to even): the value is
// rounded to fp32 with round-to-odd (toward zero, then the last bit set if the
// conversion was inexact) and that to fp16 to nearest-even.  Rounding to odd
// in a format of at least 2p + 2 bits (24 >= 2 * 11 + 2) and then to nearest
// gives the correctly rounded result (Boldo and Melquiond, "Emulation of FMA
// and correctly rounded sums: proved algorithms using rounding to odd").
// Matches f64_to_f16_bits, the definition-based conversion the host side uses.
template <> __device__ inline _Float16 store_f64<_Float16>(double x) {
  float f = __double2float_rz(x);
  if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
  return (_Float16)f;
}
template <> __device__ inline float store_f64<float>(double x) { return (float)x; }

__device__ inline void rope_pair(double x0, double x1, double c, double s, double& o0,
                                 double& o1) {
#pragma clang fp contract(off)
  o0 = x0 * c - x1 * s;
  o1 = x1 * c + x0 * s;
}

}  // namespace
}  // namespace pkv
