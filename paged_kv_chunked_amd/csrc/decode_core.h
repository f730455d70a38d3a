// Core of the tuned decode: one (sequence, KV head, 384-token split) unit of
// split-KV attention, used by paged_attention_decode and by the mixed-batch
// kernel (the design is described at the top of decode.hip).
#pragma once

#include "fp16_shape.h"

namespace pkv {
namespace {

// Minimum resident waves per SIMD the split kernel is compiled for (register
// budget 512 / this).
#ifndef PKV_DECODE_WAVES_PER_SIMD
#define PKV_DECODE_WAVES_PER_SIMD 2
#endif

// Blocks per split: kDecodeSplit tokens (at most 64: one table entry per lane).
constexpr int kSB = kDecodeSplit / kBlock;
static_assert(kSB <= 64, "one block-table entry per lane");
static_assert(kSB % 2 == 0, "splits are walked in pairs of blocks");

// fp16 elements per 16-byte piece of the K layout [block][head][D/8][16][8].
constexpr int kX = 8;

// K/V loads.  Streaming (non-temporal) where every byte is read once per
// call; cached (kNT false) where several workgroups read the same blocks
// close in time, as the shared-prefix units do: non-temporal lines are not
// kept for them (measured: the shared units' 16 quads per split then each
// fetch the split from memory).
template <bool kNT>
__device__ inline half8_t ld16(const _Float16* p) {
  if constexpr (kNT) return __builtin_bit_cast(half8_t, __builtin_nontemporal_load((const u32x4*)p));
  else return __builtin_bit_cast(half8_t, *(const u32x4*)p);
}
template <bool kNT>
__device__ inline u32x2 ld8(const _Float16* p) {
  if constexpr (kNT) return __builtin_nontemporal_load((const u32x2*)p);
  else return *(const u32x2*)p;
}

// The K and V tiles of a pair of arena blocks A, B (32 tokens), already in the
// MFMA operand layouts.
struct Pair {
  half8_t k[2][4];  // [block][kd]: A operand of S^T = K . Q^T
  half8_t v[8];     // [db]:        A operand of O^T += V^T . P^T
};

template <bool kNT = true>
__device__ inline Pair load_pair(const _Float16* __restrict__ k_arena,
                                 const _Float16* __restrict__ v_arena, int blk_a, int blk_b,
                                 int Hkv, int g, int ln, int lq) {
  Pair pr;
  const size_t tile = (size_t)kBlock * kD;
  const _Float16* ka = k_arena + ((size_t)blk_a * Hkv + g) * tile;
  const _Float16* kb = k_arena + ((size_t)blk_b * Hkv + g) * tile;
  // K: MFMA row ln = token ln of the block; the lane supplies head dims
  // 8 * (4kd + lq) .. +8, i.e. piece 4kd + lq.  Per instruction the wave reads
  // pieces 4kd .. 4kd+3 of all 16 tokens: 1 KiB contiguous.
#pragma unroll
  for (int kd = 0; kd < 4; ++kd) {
    pr.k[0][kd] = ld16<kNT>(ka + ((4 * kd + lq) * kBlock + ln) * kX);
    pr.k[1][kd] = ld16<kNT>(kb + ((4 * kd + lq) * kBlock + ln) * kX);
  }
  // V^T: MFMA row ln = head dim 16db + ln; the lane supplies keys 4lq .. 4lq+3
  // of block A then of block B (the order the probabilities come out of the
  // first product in).  Per instruction: 512 contiguous bytes of a V tile.
  const _Float16* va = v_arena + ((size_t)blk_a * Hkv + g) * tile;
  const _Float16* vb = v_arena + ((size_t)blk_b * Hkv + g) * tile;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const u32x2 lo = ld8<kNT>(va + (16 * db + ln) * kBlock + 4 * lq);
    const u32x2 hi = ld8<kNT>(vb + (16 * db + ln) * kBlock + 4 * lq);
    pr.v[db] = __builtin_bit_cast(half8_t, u32x4{lo.x, lo.y, hi.x, hi.y});
  }
  return pr;
}

// One 64-lane wavefront per (sequence b, KV head g, split of kSB blocks).
// Per pair of blocks A, B (32 tokens):
//   S^T[token][head] = K . Q^T on 2 x 4 MFMAs 16x16x32 (only columns 0..3 are
//     real heads; the query group is 4); lane (ln, lq) then holds tokens
//     4lq .. 4lq+3 of A and of B for head ln;
//   online softmax on those values (row max: 2 cross-lane steps);
//   O^T[dim][head] += V^T . P^T on 8 MFMAs, P rounded to fp16 and the
//     denominator summed from the rounded values.
// K/V go from HBM straight into operand registers; the next pair is loaded
// while the current one is computed.
// Waves per workgroup: the KV heads of one (sequence, split) run side by side,
// so a block's heads (contiguous in the arena) are fetched together and the
// block-table entries are shared through the cache.
#ifndef PKV_DECODE_WAVES_PER_WG
#define PKV_DECODE_WAVES_PER_WG 8
#endif
constexpr int kDecodeWavesPerWG = PKV_DECODE_WAVES_PER_WG;

// Sequence b (its block-table row and its partials in the workspace), whose
// query and output live at packed row `row`; its context length is
// lens[b] + len_add.  Wave (threadIdx.x >> 6) serves KV head g of split
// `split`.  kNT: streaming loads (false: cached, for blocks other
// workgroups of the call read too).
template <bool kNT = true>
__device__ __forceinline__ void decode_split_unit(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const _Float16* __restrict__ k_arena,
    const _Float16* __restrict__ v_arena, const int32_t* __restrict__ block_table,
    int max_blocks, int b, int row, const int32_t* __restrict__ lens, int len_add,
    float scale_log2, int Hkv, int nsplit_max, int num_blocks, int split, int g) {
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, lq = lane >> 4;
  const int Hq = Hkv * kG;
  const int blk0 = split * kSB;
  // Everything that does not depend on the context length is requested first,
  // so the three loads below overlap instead of forming a dependent chain:
  // this split's block-table entries (lane i: entry i; entries past the
  // sequence are never used), the group's queries, and the length itself.
  int my_blk = 0;
  if (lane < kSB && blk0 + lane < max_blocks)
    my_blk = block_table[(size_t)b * max_blocks + blk0 + lane];
  // Q^T (B operand): column ln = head g*4+ln, dims 32kd + 8lq .. +8
  half8_t qb[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd)
    qb[kd] = ln < kG ? *(const half8_t*)(q + ((size_t)row * Hq + g * kG + ln) * kD + 32 * kd + 8 * lq)
                     : (half8_t)(_Float16)0.f;
  // clamp to what the grid and workspace cover (a caller contract violation
  // then gives unspecified values, never an out-of-bounds access)
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
  if (lane >= nb || my_blk < 0 || my_blk >= num_blocks) my_blk = 0;

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = (f32x4)0.f;
  float m_run = -INFINITY, l_run = 0.f;

  auto pair_ids = [&](int p, int& a, int& c) {
    a = __builtin_amdgcn_readlane(my_blk, 2 * p);
    c = 2 * p + 1 < nb ? __builtin_amdgcn_readlane(my_blk, 2 * p + 1) : a;
  };
  auto compute = [&](const Pair& pr, int p) {
    f32x4 s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] = (f32x4)0.f;
#pragma unroll
      for (int kd = 0; kd < 4; ++kd)
        s[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pr.k[u][kd], qb[kd], s[u], 0, 0, 0);
    }
    // element e of this lane: token 4lq + (e & 3) of block A (e < 4) or B
    const int tok_a = (blk0 + 2 * p) * kBlock + 4 * lq;
    const int nva = L - tok_a, nvb = nva - kBlock;  // valid elements of A / B
    // The base-2 exponent of key e is fma(score_e, scale_log2, -m): one
    // rounding, written out so that no kernel leaves it to the compiler's
    // contraction choices (decode_shared_kernel must round it identically).
    // The running max is taken over raw scores and scaled once (scale_log2 >
    // 0 and rounding is monotone, so this is the max of the scaled scores).
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = e < 4 ? e < nva : e - 4 < nvb;
      mx = fmaxf(mx, ok ? s[e >> 2][e & 3] : -INFINITY);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);  // finite: the first key of a split is real
    if (__any(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db) o[db] *= alpha;
    }
    m_run = m_new;
    half8_t pb;
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = e < 4 ? e < nva : e - 4 < nvb;
      const float arg = ok ? __builtin_fmaf(s[e >> 2][e & 3], scale_log2, -m_new) : -INFINITY;
      const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(arg);
      pb[e] = ph;
      lsum += (float)ph;
    }
    l_run += lsum;
    // keys past the context (only in the sequence's last pair): zero V, since
    // their p is 0 but 0 * NaN is not
    const bool tail_pair = (blk0 + 2 * p + 2) * kBlock > L;  // wave-uniform
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      half8_t va = pr.v[db];
      if (tail_pair) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          va[e] = (e < 4 ? e < nva : e - 4 < nvb) ? va[e] : (_Float16)0.f;
      }
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o[db], 0, 0, 0);
    }
  };

  // Two pair buffers in flight, loop fully unrolled (a split is at most
  // kSB / 2 pairs).  The prefetch is issued unconditionally (past the last
  // pair it re-requests the last pair, a cache hit), so the loads outstanding
  // at each wait are the same on every path and the wait before a pair's MFMAs
  // covers that pair only, never the prefetch behind it.
  Pair buf[2];
  {
    int ba, bb;
    pair_ids(0, ba, bb);
    buf[0] = load_pair<kNT>(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
  }
#pragma unroll
  for (int p = 0; p < kSB / 2; ++p) {
    if (p + 1 < kSB / 2) {
      int ba, bb;
      pair_ids(min(p + 1, npairs - 1), ba, bb);
      buf[(p + 1) & 1] = load_pair<kNT>(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
      __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the compute
    }
    if (p < npairs) compute(buf[p & 1], p);
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
