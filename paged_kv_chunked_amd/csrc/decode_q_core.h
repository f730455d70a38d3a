// Quantized (INT8 / INT4) decode split: one wave per (split, KV head), used by
// the quantized decode kernels and by the mixed-batch kernel (the design is
// described with the quantized decode kernels in decode.hip).
#pragma once

#include <type_traits>

#include "decode_core.h"
#include "quant_append_core.h"
#include "quant_codes.h"

namespace pkv {
namespace {

#ifndef PKV_DECODE_I8_AHEAD
#define PKV_DECODE_I8_AHEAD 1
#endif
#ifndef PKV_DECODE_I4_AHEAD
#define PKV_DECODE_I4_AHEAD 1
#endif

// v_mul_legacy_f32: x * y, except that 0 times anything (NaN, infinity) is 0.
__device__ float pkv_fmul_legacy(float, float) __asm("llvm.amdgcn.fmul.legacy");

struct PairI8 {
  u32x4 k[2][2];  // [u][j]: 16 codes (dims 16(4j + lq) .. +16) of the lane's key row
  u32x2 v[8];     // [db]: 8 codes of dim 16db + ln, the lane's 8 keys
  u32x4 ks, vs;   // fp16 scales of the lane's 8 keys (K, V)
};

__device__ inline PairI8 load_pair_i8(const uint8_t* __restrict__ k_arena,
                                      const uint8_t* __restrict__ v_arena, int blk_a, int blk_b,
                                      int Hkv, int g, int ln, int lq) {
  constexpr size_t kTile = i8_tile_bytes(kD);
  PairI8 pr;
  // K row of this lane (MFMA row ln) for MFMA u: block A or B by ln >> 3
  const uint8_t* kt = k_arena + ((size_t)((ln >> 3) ? blk_b : blk_a) * Hkv + g) * kTile;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    // the lane's token 8((ln >> 2) & 1) + 4u + (ln & 3) is stored at position
    // 8u + (ln & 7): MFMA u reads one 128-byte run per (block, piece)
    const int slot = 8 * u + (ln & 7);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      pr.k[u][j] = __builtin_nontemporal_load((const u32x4*)(kt + (4 * j + lq) * 256 + slot * 16));
  }
  // the lane's keys (as head ln of the scores): block lq >> 1, tokens 8(lq & 1) .. +8
  const size_t tv = ((size_t)((lq >> 1) ? blk_b : blk_a) * Hkv + g) * kTile;
  const uint8_t* vt = v_arena + tv;
#pragma unroll
  for (int db = 0; db < 8; ++db)
    pr.v[db] = __builtin_nontemporal_load((const u32x2*)(vt + (16 * db + ln) * kBlock + 8 * (lq & 1)));
  pr.ks = __builtin_nontemporal_load((const u32x4*)(k_arena + tv + kBlock * kD + 16 * (lq & 1)));
  pr.vs = __builtin_nontemporal_load((const u32x4*)(vt + kBlock * kD + 16 * (lq & 1)));
  return pr;
}

// INT4 arenas (PKV_I4KV): the same kernel over 4-bit codes.  A lane's 16-byte
// K load holds its two keys' records (MFMA u = 0, 1) of one 16-dim piece: low
// nibbles are dims 0-7, high nibbles dims 8-15 of the piece, so each MFMA
// operand is one mask per word.  Each 4-byte word of V holds the lane's 8
// keys of one head dim (low nibbles keys 0-3, high nibbles keys 4-7), and one
// 16-byte V load brings the words of four dim blocks.  Nibbles become fp16
// exactly: (n ^ 8) + 1024 - 1032.
struct PairI4 {
  u32x4 k[2];     // [j]: records (u = 0: x, y; u = 1: z, w) of piece 4j + lq
  uint32_t v[8];  // [db]: 8 codes of dim 16db + ln, the lane's 8 keys
  u32x4 ks, vs;   // fp16 scales of the lane's 8 keys (K, V)
};

__device__ inline PairI4 load_pair_i4(const uint8_t* __restrict__ k_arena,
                                      const uint8_t* __restrict__ v_arena, int blk_a, int blk_b,
                                      int Hkv, int g, int ln, int lq) {
  constexpr size_t kTile = i4_tile_bytes(kD);
  PairI4 pr;
  // the lane's key row (MFMA row ln) lives in block A or B by ln >> 3; its
  // records for u = 0, 1 are 16 bytes at record 2 (ln & 7)
  const uint8_t* kt = k_arena + ((size_t)((ln >> 3) ? blk_b : blk_a) * Hkv + g) * kTile;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    pr.k[j] = __builtin_nontemporal_load((const u32x4*)(kt + (4 * j + lq) * 128 + (ln & 7) * 16));
  const size_t tv = ((size_t)((lq >> 1) ? blk_b : blk_a) * Hkv + g) * kTile;
  const uint8_t* vt = v_arena + tv;
  // V: the lane's 8 keys (half lq & 1 of its block) for dims 16db + ln, four
  // dim blocks per 16-byte load (i4_vbyte with D = 128)
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x4 w =
        __builtin_nontemporal_load((const u32x4*)(vt + ((2 * j + (lq & 1)) * 16 + ln) * 16));
    pr.v[4 * j] = w.x;
    pr.v[4 * j + 1] = w.y;
    pr.v[4 * j + 2] = w.z;
    pr.v[4 * j + 3] = w.w;
  }
  pr.ks = __builtin_nontemporal_load((const u32x4*)(k_arena + tv + kBlock * kD / 2 + 16 * (lq & 1)));
  pr.vs = __builtin_nontemporal_load((const u32x4*)(vt + kBlock * kD / 2 + 16 * (lq & 1)));
  return pr;
}

// The two code widths as traits of one split kernel: the pair type, its load,
// and the MFMA operands (K operand of MFMA u, contraction step kd; V operand
// of dims block db).
struct CodesI8 {
  using Pair = PairI8;
  static constexpr size_t kTile = i8_tile_bytes(kD);
  // the fused append: the new key and value of one (token, head) into the tiles
  __device__ static void append(const _Float16* kp, const _Float16* vp, const double2* row,
                                uint8_t* kt, uint8_t* vt, int slot, int lane) {
    append_k_i8(kp, row, kt, slot, kD, lane);
    append_v_i8(vp, vt, slot, kD, lane);
  }
  static constexpr int kAhead = PKV_DECODE_I8_AHEAD;  // pairs in flight behind the computed one
  // the pair loop runs its whole length (the early exit's extra paths spill
  // at this unit's 168 registers, three waves per SIMD)
  static constexpr bool kEarlyExit = false;
  static constexpr float kPvBoost = 64.f;
  static constexpr int kDimOrder[8] = {0, 1, 2, 3, 4, 5, 6, 7};
  static constexpr int kKeyOrder[8] = {0, 1, 2, 3, 4, 5, 6, 7};
  __device__ static Pair load(const uint8_t* k, const uint8_t* v, int a, int b, int Hkv, int g,
                              int ln, int lq) {
    return load_pair_i8(k, v, a, b, Hkv, g, ln, lq);
  }
  __device__ static half8_t kop(const Pair& pr, int u, int kd) {
    const u32x4 c = pr.k[u][kd >> 1];
    return (kd & 1) ? codes_to_half(c.z, c.w) : codes_to_half(c.x, c.y);
  }
  __device__ static half8_t vop(const Pair& pr, int db) {
    return codes_to_half(pr.v[db].x, pr.v[db].y);
  }
};
// Two nibbles of a word (bits 0-3 and 16-19, or 4-7 and 20-23) as an fp16
// pair, two instructions: one AND-XOR puts 0x6400 | (n ^ 8) (resp.
// 0x6400 | (n ^ 8) << 4) in each half -- 1024 + (n + 8), resp. 1024 +
// 16 (n + 8), n the signed code -- and one packed subtract of 1032 (resp. one
// exact packed fma: times 1/16, minus 72) leaves n.  Nibbles at bits 8-15 of
// each half take the word shifted right by 8.
__device__ inline uint32_t nib_lo(uint32_t w) {
  const half2_t h = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) ^ 0x64086408u);
  return __builtin_bit_cast(uint32_t, h - (half2_t)(_Float16)1032.f);
}
__device__ inline uint32_t nib_hi(uint32_t w) {
  const half2_t h = __builtin_bit_cast(half2_t, (w & 0x00F000F0u) ^ 0x64806480u);
  return __builtin_bit_cast(
      uint32_t, __builtin_elementwise_fma(h, (half2_t)(_Float16)0.0625f, (half2_t)(_Float16)-72.f));
}

struct CodesI4 {
  static constexpr int kAhead = PKV_DECODE_I4_AHEAD;
  static constexpr bool kEarlyExit = true;  // the pair loop stops at the split's end
  static constexpr size_t kTile = i4_tile_bytes(kD);
  // (one token per sequence: the byte partner slot ^ 4 is never appended by
  // the same call, so the new nibble merges with the stored one)
  __device__ static void append(const _Float16* kp, const _Float16* vp, const double2* row,
                                uint8_t* kt, uint8_t* vt, int slot, int lane) {
    append_k_i4(kp, row, kt, slot, kD, lane);
    append_v_i4(vp, nullptr, true, vt, slot, kD, lane);
  }
  static constexpr float kPvBoost = 4.f;
  using Pair = PairI4;
  // Order of the 8 elements in an MFMA operand register: K operands hold dims
  // [0, 2, 1, 3, 4, 6, 5, 7] of their 8 (the query operand is loaded in the
  // same order), V operands keys [0, 2, 4, 6, 1, 3, 5, 7] of the lane's 8
  // (the weights are placed in the same order): the order in which the
  // two-instruction conversion above produces them.
  static constexpr int kDimOrder[8] = {0, 2, 1, 3, 4, 6, 5, 7};
  static constexpr int kKeyOrder[8] = {0, 2, 4, 6, 1, 3, 5, 7};
  __device__ static Pair load(const uint8_t* k, const uint8_t* v, int a, int b, int Hkv, int g,
                              int ln, int lq) {
    return load_pair_i4(k, v, a, b, Hkv, g, ln, lq);
  }
  // word w0 (w1): low nibbles dims 0-3 (4-7) of the 16-dim piece, high
  // nibbles dims 8-11 (12-15); kd odd takes the high nibbles
  __device__ static half8_t kop(const Pair& pr, int u, int kd) {
    const u32x4 c = pr.k[kd >> 1];
    const uint32_t x0 = u ? c.z : c.x, x1 = u ? c.w : c.y;
    const uint32_t y0 = x0 >> 8, y1 = x1 >> 8;
    const u32x4 r = (kd & 1) ? u32x4{nib_hi(x0), nib_hi(y0), nib_hi(x1), nib_hi(y1)}
                             : u32x4{nib_lo(x0), nib_lo(y0), nib_lo(x1), nib_lo(y1)};
    return __builtin_bit_cast(half8_t, r);
  }
  // low nibbles keys 0-3, high nibbles keys 4-7
  __device__ static half8_t vop(const Pair& pr, int db) {
    const uint32_t x = pr.v[db], y = x >> 8;
    return __builtin_bit_cast(half8_t, u32x4{nib_lo(x), nib_hi(x), nib_lo(y), nib_hi(y)});
  }
};

// Waves per workgroup and minimum resident waves per SIMD of the quantized
// split kernels (their register budget differs from the fp16 kernel's):
// three waves per SIMD keep the INT8 unit at 168 VGPRs, no spills.
#ifndef PKV_DECODE_I8_WAVES_PER_WG
#define PKV_DECODE_I8_WAVES_PER_WG 8
#endif
#ifndef PKV_DECODE_I8_WAVES_PER_SIMD
#define PKV_DECODE_I8_WAVES_PER_SIMD 3
#endif
#ifndef PKV_DECODE_I4_WAVES_PER_SIMD
#define PKV_DECODE_I4_WAVES_PER_SIMD 3
#endif
constexpr int kI8WavesPerWG = PKV_DECODE_I8_WAVES_PER_WG;

// Split `split` of sequence b (its block-table row and its partials in the
// workspace) for KV head g, one wave; the query and output live at packed row
// `row` and the context length is lens[b] + len_add.  kAppend (the fused
// decode step): the query is app.q rotated here at pos = L - 1 (split 0
// writes it to app.q_out), and the wave of the sequence's last split first
// quantizes the new key and value into the arena with kv_append_rope's code
// and waits for those stores before it requests any pair, so its loads read
// them back; the outputs, the rotated queries and the arena bytes are those
// of kv_append_rope followed by the plain decode.
template <class Codes, bool kAppend = false>
__device__ __forceinline__ void decode_split_q_unit(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q,
    const uint8_t* __restrict__ k_arena, const uint8_t* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks, int b, int row,
    const int32_t* __restrict__ lens, int len_add, float scale_log2, int Hkv, int nsplit_max,
    int num_blocks, int split, int g, DecodeAppend app = DecodeAppend{}) {
  // No contraction of a multiply and an add into one fma at the compiler's
  // choice: the decode kernel and the mixed kernel inline this unit into
  // different code and must round every step alike (the one fma wanted is
  // written out).
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, lq = lane >> 4;
  const int Hq = Hkv * kG;
  const int blk0 = split * kSB;
  int my_blk = 0;
  if (lane < kSB && blk0 + lane < max_blocks)
    my_blk = block_table[(size_t)b * max_blocks + blk0 + lane];
  // Q^T (B operand) in the permuted dim order: MFMA kd, lane group lq holds
  // dims 16(4(kd >> 1) + lq) + 8(kd & 1) .. +8 of head g*4+ln
  half8_t qb[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) {
    const half8_t x = !kAppend && ln < kG
                          ? *(const half8_t*)(q + ((size_t)row * Hq + g * kG + ln) * kD +
                                              16 * (4 * (kd >> 1) + lq) + 8 * (kd & 1))
                          : (half8_t)(_Float16)0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) qb[kd][j] = x[Codes::kDimOrder[j]];
  }
  const int L = min(min(lens[b] + len_add, max_blocks * kBlock), nsplit_max * kDecodeSplit);
  if (L <= 0) {
    if (split == 0 && ln < kG) {
      float* o = out + ((size_t)row * Hq + g * kG + ln) * kD + 4 * lq;
#pragma unroll
      for (int db = 0; db < 8; ++db) *(f32x4*)(o + 16 * db) = (f32x4)0.f;
    }
    return;
  }
  const int nb_seq = (L + kBlock - 1) / kBlock;
  if (blk0 >= nb_seq) return;
  const int nb = min(kSB, nb_seq - blk0);
  const int nsplit = (nb_seq + kSB - 1) / kSB;
  const int npairs = (nb + 1) >> 1;
  [[maybe_unused]] const int raw_blk = my_blk;  // (unclamped, for the fused append's write)
  if (lane >= nb || my_blk < 0 || my_blk >= num_blocks) my_blk = 0;

  if constexpr (kAppend) {
    // The query: lane l rotates pairs 4 (l & 15) .. +3 of head l >> 4 of the
    // wave's group (fp64, one rounding: kv_append_rope's arithmetic) into the
    // wave's LDS, and the operand lanes read their pieces in the order above.
    // A position outside the table leaves the query as given and skips the
    // append, as kv_append_rope does.
    const int pos = L - 1;
    const bool app_ok = pos < app.rope_max_pos;
    const double2* rrow = app.rope + (size_t)min(pos, app.rope_max_pos - 1) * (kD / 2);
    __shared__ _Float16 qapp_lds[kI8WavesPerWG][kG * kD];
    _Float16* wl = qapp_lds[threadIdx.x >> 6];
    {
      const int h = lane >> 4, i0 = 4 * (lane & 15);
      const _Float16* qs = app.q + ((size_t)row * Hq + g * kG + h) * kD;
      const half4_t lo = *(const half4_t*)(qs + i0), hi = *(const half4_t*)(qs + i0 + kD / 2);
      half4_t olo = lo, ohi = hi;
      if (app_ok) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double2 c = rrow[i0 + r];
          double o0, o1;
          rope_pair((double)lo[r], (double)hi[r], c.x, c.y, o0, o1);
          olo[r] = store_f64<_Float16>(o0);
          ohi[r] = store_f64<_Float16>(o1);
        }
      }
      const u32x2 wlo = __builtin_bit_cast(u32x2, olo), whi = __builtin_bit_cast(u32x2, ohi);
      *(u32x2*)(wl + h * kD + i0) = wlo;
      *(u32x2*)(wl + h * kD + i0 + kD / 2) = whi;
      if (app_ok && split == 0) {
        _Float16* qo = app.q_out + ((size_t)row * Hq + g * kG + h) * kD;
        *(u32x2*)(qo + i0) = wlo;
        *(u32x2*)(qo + i0 + kD / 2) = whi;
      }
    }
    // one wave writes and reads its LDS, in order
    if (ln < kG) {
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) {
        const half8_t x = *(const half8_t*)(wl + ln * kD + 16 * (4 * (kd >> 1) + lq) + 8 * (kd & 1));
#pragma unroll
        for (int j = 0; j < 8; ++j) qb[kd][j] = x[Codes::kDimOrder[j]];
      }
    }
    // The new key and value (the last split holds their block).  The tiles
    // are addressed from the arena pointers the pairs are read through, and
    // every store has completed before the first pair is requested.
    if (app_ok && split == nsplit - 1) {
      const int nblk = __builtin_amdgcn_readlane(raw_blk, (pos >> 4) - blk0);
      if (nblk >= 0 && nblk < num_blocks) {
        const size_t tile = ((size_t)nblk * Hkv + g) * Codes::kTile;
        Codes::append(app.k + ((size_t)b * Hkv + g) * kD, app.v + ((size_t)b * Hkv + g) * kD,
                      rrow, const_cast<uint8_t*>(k_arena) + tile,
                      const_cast<uint8_t*>(v_arena) + tile, pos & 15, lane);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
  }

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = (f32x4)0.f;
  float m_run = -INFINITY, l_run = 0.f;

  auto pair_ids = [&](int p, int& a, int& c) {
    a = __builtin_amdgcn_readlane(my_blk, 2 * p);
    c = 2 * p + 1 < nb ? __builtin_amdgcn_readlane(my_blk, 2 * p + 1) : a;
  };
  using Pair = typename Codes::Pair;
  // The probabilities carry the factor kPvBoost from the start: the
  // exponent gets log2(kPvBoost) added, so p * boost comes out of the
  // exponential and one mixed multiply by the fp16 V scale gives the weight
  // (the denominator sums the same boosted p, so the factor cancels in o / l
  // and in the merge of the splits).  Keys past the context exist only in a
  // sequence's last pair, which is computed after the loop with the masks
  // (tail); the loop's pairs need none.
  const float pv_bias = __builtin_log2f(Codes::kPvBoost);  // exact: a power of two
  auto compute = [&](const Pair& pr, int p, auto tail) {
    f32x4 s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] = (f32x4)0.f;
#pragma unroll
      for (int kd = 0; kd < 4; ++kd)
        s[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Codes::kop(pr, u, kd), qb[kd], s[u], 0, 0, 0);
    }
    // element e = 4u + i of this lane: token 8(lq & 1) + e of block lq >> 1
    const half8_t ksc = __builtin_bit_cast(half8_t, pr.ks);
    const half8_t vsc = __builtin_bit_cast(half8_t, pr.vs);
    const int tok0 = (blk0 + 2 * p + (lq >> 1)) * kBlock + 8 * (lq & 1);
    const int nvalid = L - tok0;  // keys e < nvalid exist
    // raw score of the decoded key: (q . codes) * scale, one rounding
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = s[e >> 2][e & 3] * (float)ksc[e];
    if constexpr (decltype(tail)::value) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = e < nvalid ? sv[e] : -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // running max in log2 units, the raw maximum scaled once (monotone);
    // finite: the first key of a split is real
    const float m_new = fmaxf(m_run, mx * scale_log2);
    if (__any(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] *= alpha;
    }
    m_run = m_new;
    const float bias = pv_bias - m_new;
    float pe[8];
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], scale_log2, bias));  // p * boost
      lsum += pe[e];
    }
    l_run += lsum;
    // The legacy multiply gives 0 for p = 0 whatever the V scale (past the end
    // it may be NaN: an unwritten slot), and, unlike a plain multiply, is
    // never fused with the fp16 conversion: the weight is the fp32 product
    // rounded to fp16 in every kernel that inlines this unit.  Element j of
    // the operand is key kKeyOrder[j], as in the V operand.
    half8_t pb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = Codes::kKeyOrder[j];
      pb[j] = (_Float16)pkv_fmul_legacy(pe[e], (float)vsc[e]);
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Codes::vop(pr, db), pb, o[db], 0, 0, 0);
  };

  // kAhead pairs are kept in flight behind the one being computed (same
  // unconditional-prefetch scheme as the fp16 kernel).  One measured best:
  // two or three cost registers (INT8: occupancy 3 -> 2) and ran 4-12%
  // slower.
  constexpr int kAhead = Codes::kAhead;
  // pairs whose keys all exist; a partial last pair is left for after the loop
  const bool has_tail = (blk0 + 2 * npairs) * kBlock > L;
  const int n_full = npairs - (has_tail ? 1 : 0);
  Pair buf[kAhead + 1];
#pragma unroll
  for (int p = 0; p < kAhead; ++p) {
    int ba, bb;
    pair_ids(min(p, npairs - 1), ba, bb);
    buf[p] = Codes::load(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
  }
  if constexpr (Codes::kEarlyExit) {
    // The loop is left (a wave-uniform branch) once the full pairs are done,
    // so a short split issues no loads past its end; pair p is in buffer
    // p % (kAhead + 1), and the tail pair, requested kAhead iterations
    // earlier or before the loop, is taken from its buffer after it.
    run_steps([&](auto P) {
      constexpr int p = decltype(P)::value;
      if (p >= n_full) return false;
      if (p + kAhead < kSB / 2) {
        int ba, bb;
        pair_ids(min(p + kAhead, npairs - 1), ba, bb);
        buf[(p + kAhead) % (kAhead + 1)] = Codes::load(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
        __builtin_amdgcn_sched_barrier(0);
      }
      compute(buf[p % (kAhead + 1)], p, std::false_type{});
      return true;
    }, std::make_integer_sequence<int, kSB / 2>{});
    if (has_tail) {
      // (one branch per buffer: a copy of the selected buffer would cost a
      // pair's registers)
      const int tb = (npairs - 1) % (kAhead + 1);
      run_steps([&](auto I) {
        constexpr int i = decltype(I)::value;
        if (tb != i) return true;
        compute(buf[i], npairs - 1, std::true_type{});
        return false;
      }, std::make_integer_sequence<int, kAhead + 1>{});
    }
  } else {
    // The whole loop: past the split's pairs the prefetch re-requests the
    // last pair (cache hits), so the last prefetch (at
    // p = kSB / 2 - 1 - kAhead, clamped to the last pair) leaves pair
    // npairs - 1 in buffer (kSB / 2 - 1) % (kAhead + 1), whatever npairs is.
#pragma unroll
    for (int p = 0; p < kSB / 2; ++p) {
      if (p + kAhead < kSB / 2) {
        int ba, bb;
        pair_ids(min(p + kAhead, npairs - 1), ba, bb);
        buf[(p + kAhead) % (kAhead + 1)] = Codes::load(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (p < n_full) compute(buf[p % (kAhead + 1)], p, std::false_type{});
    }
    if (has_tail) compute(buf[(kSB / 2 - 1) % (kAhead + 1)], npairs - 1, std::true_type{});
  }

  float l_row = l_run;
  l_row += __shfl_xor(l_row, 16);
  l_row += __shfl_xor(l_row, 32);
  const int hq = g * kG + ln;
  if (nsplit == 1) {
    if (ln < kG) {
      const float inv = 1.f / l_row;
      float* dst = out + ((size_t)row * Hq + hq) * kD + 4 * lq;
#pragma unroll
      for (int db = 0; db < 8; ++db) *(f32x4*)(dst + 16 * db) = o[db] * inv;
    }
    return;
  }
  if (ln < kG) {
    const size_t part = ((size_t)b * nsplit_max + split) * Hq + hq;
    float* dst = ws_o + part * kD + 4 * lq;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(f32x4*)(dst + 16 * db) = o[db];
    if (lq == 0) {
      ws_ml[2 * part] = m_run;
      ws_ml[2 * part + 1] = l_row;
    }
  }
}


}  // namespace
}  // namespace pkv
