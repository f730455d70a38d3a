// Quantizing append of one (token, KV head) vector into an INT8 or INT4
// arena tile, one wave: the codec of Kshipra part 3 section 2 applied to
// cached K and V (one fp16 scale per vector, used to encode and to decode).
// Shared by kv_append_rope's quantized kernels and the fused decode-step
// kernels, so both write the same bytes.
#pragma once

#include <cstdint>

#include "fp16_shape.h"
#include "pkv_internal.h"
#include "rope_core.h"

namespace pkv {
namespace {

// Group quantization: scale s = fp16(fp32(amax) / qmax) (floored at the
// smallest positive fp16), codes round-half-even(fp32(x) / fp32(s)) clamped
// to [-qmax, qmax].  Lane l holds elements l, l + 64, l + 128, l + 192 of the
// vector (those below D).
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ inline _Float16 group_scale(float amax) {
  const _Float16 s = (_Float16)(amax / 127.f);
  const _Float16 smin = __builtin_bit_cast(_Float16, (uint16_t)1);  // 2^-24
  return s < smin ? smin : s;
}

__device__ inline int8_t encode8(float x, float s) {
  const float r = __builtin_rintf(x / s);
  return (int8_t)fminf(fmaxf(r, -127.f), 127.f);
}

// 4 bits: s = fp16(fp32(amax) / 7), codes in [-7, 7] stored as
// two's-complement nibbles.
__device__ inline _Float16 group_scale4(float amax) {
  const _Float16 s = (_Float16)(amax / 7.f);
  const _Float16 smin = __builtin_bit_cast(_Float16, (uint16_t)1);  // 2^-24
  return s < smin ? smin : s;
}

__device__ inline int encode4(float x, float s) {
  const float r = __builtin_rintf(x / s);
  return (int)fminf(fmaxf(r, -7.f), 7.f);
}

// The key of one (token, head), kp[0 .. D), rotated at the position whose
// cos/sin row is `row` and rounded to fp16 exactly as for an fp16 arena, as
// fp32: lane l takes the pairs (l, l + D/2) and (l + 64, l + 64 + D/2) that
// exist (x[2u], x[2u + 1] for u = 0, 1); returns the wave's largest magnitude.
__device__ inline float rotate_key(const _Float16* kp, const double2* row, int D, int lane,
                                   float (&x)[4]) {
  const int half = D >> 1;
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = lane + 64 * u;
    x[2 * u] = x[2 * u + 1] = 0.f;
    if (i < half) {
      const double2 c = row[i];
      double o0, o1;
      rope_pair((double)kp[i], (double)kp[i + half], c.x, c.y, o0, o1);
      x[2 * u] = (float)store_f64<_Float16>(o0);
      x[2 * u + 1] = (float)store_f64<_Float16>(o1);
      amax = fmaxf(amax, fmaxf(fabsf(x[2 * u]), fabsf(x[2 * u + 1])));
    }
  }
  return wave_max(amax);
}

// The value of one (token, head) as fp32, lane l: elements l + 64u.
__device__ inline float load_value(const _Float16* vp, int D, int lane, float (&x)[4]) {
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    x[u] = d < D ? (float)vp[d] : 0.f;
    amax = fmaxf(amax, fabsf(x[u]));
  }
  return wave_max(amax);
}

// INT8 tile of one (block, head): K codes [D/16][16][16] (the key of slot s
// at position i8_kpos(s) of each 16-dim piece) then 16 fp16 scales; V codes
// [D][16] then 16 fp16 scales.
__device__ inline void append_k_i8(const _Float16* kp, const double2* row, uint8_t* tile, int slot,
                                   int D, int lane) {
  float x[4];
  const _Float16 sh = group_scale(rotate_key(kp, row, D, lane, x));
  const float s = (float)sh;
  const int half = D >> 1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = lane + 64 * u;
    if (i < half) {
      const int d0 = i, d1 = i + half;
      tile[(d0 >> 4) * 256 + i8_kpos(slot) * 16 + (d0 & 15)] = (uint8_t)encode8(x[2 * u], s);
      tile[(d1 >> 4) * 256 + i8_kpos(slot) * 16 + (d1 & 15)] = (uint8_t)encode8(x[2 * u + 1], s);
    }
  }
  if (lane == 0) *(_Float16*)(tile + (size_t)kBlock * D + 2 * slot) = sh;
}

__device__ inline void append_v_i8(const _Float16* vp, uint8_t* tile, int slot, int D, int lane) {
  float x[4];
  const _Float16 sh = group_scale(load_value(vp, D, lane, x));
  const float s = (float)sh;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    if (d < D) tile[d * kBlock + slot] = (uint8_t)encode8(x[u], s);
  }
  if (lane == 0) *(_Float16*)(tile + (size_t)kBlock * D + 2 * slot) = sh;
}

// INT4 tile: K, per 16-dim piece 16 records of 8 bytes (slot s at record
// i4_krec(s)), byte i holding dims i (low nibble) and i + 8 -- lanes i and
// i + 8, joined with one shuffle; then 16 fp16 scales.  V: the byte of head
// dim d that holds slot s (i4_vbyte) also holds slot s ^ 4 (high nibble when
// i4_vhigh(s)); then 16 fp16 scales.
__device__ inline void append_k_i4(const _Float16* kp, const double2* row, uint8_t* tile, int slot,
                                   int D, int lane) {
  float x[4];
  const _Float16 sh = group_scale4(rotate_key(kp, row, D, lane, x));
  const float s = (float)sh;
  const int half = D >> 1, krec = i4_krec(slot);
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = lane + 64 * u;
    const int c0 = i < half ? encode4(x[2 * u], s) : 0;
    const int c1 = i < half ? encode4(x[2 * u + 1], s) : 0;
    const int p0 = __shfl_down(c0, 8), p1 = __shfl_down(c1, 8);  // dims i + 8, i + 8 + half
    if (i < half && (i & 8) == 0) {  // half is a multiple of 16: i + half has bit 3 clear too
      const int d0 = i, d1 = i + half;
      tile[(d0 >> 4) * 128 + krec * 8 + (d0 & 7)] = (uint8_t)((c0 & 15) | ((p0 & 15) << 4));
      tile[(d1 >> 4) * 128 + krec * 8 + (d1 & 7)] = (uint8_t)((c1 & 15) | ((p1 & 15) << 4));
    }
  }
  if (lane == 0) *(_Float16*)(tile + (size_t)kBlock * D / 2 + 2 * slot) = sh;
}

// The value's scale always; its nibbles when `leader` (the token whose byte
// partner, slot ^ 4, is not appended by another wave of the call): merged
// with the partner's code when the partner's value pp is given, else with the
// nibble the byte holds.
__device__ inline void append_v_i4(const _Float16* vp, const _Float16* pp, bool leader,
                                   uint8_t* tile, int slot, int D, int lane) {
  float x[4];
  const _Float16 sh = group_scale4(load_value(vp, D, lane, x));
  const float s = (float)sh;
  if (lane == 0) *(_Float16*)(tile + (size_t)kBlock * D / 2 + 2 * slot) = sh;
  if (!leader) return;
  float y[4] = {0.f, 0.f, 0.f, 0.f};
  float sp = 1.f;
  if (pp != nullptr) sp = (float)group_scale4(load_value(pp, D, lane, y));
  const int vhigh = i4_vhigh(slot);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = lane + 64 * u;
    if (d >= D) continue;
    uint8_t* at = tile + i4_vbyte(d, slot, D);
    const int own = encode4(x[u], s) & 15;
    // the other nibble: the partner's code, or what the byte holds already
    // (read at device scope, so that it leaves no copy of the line in the
    // CU's cache that a later read could see instead of this store)
    int other;
    if (pp != nullptr) {
      other = encode4(y[u], sp) & 15;
    } else {
      const int held = __hip_atomic_load(at, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      other = vhigh ? (held & 15) : (held >> 4);
    }
    *at = (uint8_t)(vhigh ? (other | (own << 4)) : (own | (other << 4)));
  }
}

}  // namespace
}  // namespace pkv
