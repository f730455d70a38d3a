// Core of the tuned decode: one (sequence, KV head, 384-token split) unit of
// split-KV attention, used by paged_attention_decode and by the mixed-batch
// kernel (the design is described at the top of decode.hip).
#pragma once

#include <type_traits>
#include <utility>

#include "fp16_shape.h"
#include "rope_core.h"

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

// Steps f(0), f(1), ... f(N - 1) as straight-line code, stopping after the
// first that returns false: an unrolled loop with an early exit, which the
// compiler does not unroll when written as a loop with a break (it then
// indexes the pair buffers at run time, from scratch memory).
template <typename F, int... Is>
__device__ __forceinline__ void run_steps(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}) && ...);
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

// The step's append fused into the decode (paged_attention_decode_append):
// each sequence's new token, at position context length - 1, with its query,
// key and value as the caller passes them to kv_append_rope.
struct DecodeAppend {
  const _Float16* q;      // [num_seqs][Hq][D] queries, not yet rotated
  _Float16* q_out;        // [num_seqs][Hq][D] rotated queries (written by split 0)
  const _Float16* k;      // [num_seqs][Hkv][D] keys, not yet rotated
  const _Float16* v;      // [num_seqs][Hkv][D] values
  _Float16* k_arena;      // the arenas, written at the new token's slot
  _Float16* v_arena;
  const double2* rope;    // [rope_max_pos][D/2] (cos, sin)
  int rope_max_pos;
};

// Sequence b (its block-table row and its partials in the workspace), whose
// query and output live at packed row `row`; its context length is
// lens[b] + len_add.  Wave (threadIdx.x >> 6) serves KV head g of split
// `split`.  kNT: streaming loads (false: cached, for blocks other
// workgroups of the call read too).  kAppend: the query is app.q rotated
// here, and the new token's rotated key and value enter the last pair from
// registers (and are written to the arena by the wave of the last split),
// with the values, roundings and order of kv_append_rope followed by the
// plain decode, so the outputs, the rotated queries and the arena bytes are
// bit for bit those of the two calls.
template <bool kNT = true, bool kAppend = false>
__device__ __forceinline__ void decode_split_unit(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const _Float16* __restrict__ k_arena,
    const _Float16* __restrict__ v_arena, const int32_t* __restrict__ block_table,
    int max_blocks, int b, int row, const int32_t* __restrict__ lens, int len_add,
    float scale_log2, int Hkv, int nsplit_max, int num_blocks, int split, int g,
    DecodeAppend app = DecodeAppend{}) {
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
  // Q^T (B operand): column ln = head g*4+ln, dims 32kd + 8lq .. +8 (the
  // fused append fills it from its rotation below)
  half8_t qb[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd)
    qb[kd] = !kAppend && ln < kG
                 ? *(const half8_t*)(q + ((size_t)row * Hq + g * kG + ln) * kD + 32 * kd + 8 * lq)
                 : (half8_t)(_Float16)0.f;
  // The fused append's inputs that do not depend on the length (the rotation
  // table's row does): lane l takes pairs 4 (l & 15) .. +3 of the wave's
  // query head l >> 4, key pair (l, l + 64) and value dims l, l + 64.
  [[maybe_unused]] const int ah = lane >> 4, ai0 = 4 * (lane & 15);
  [[maybe_unused]] half4_t qlo, qhi;
  [[maybe_unused]] _Float16 kr0, kr1, vr0, vr1;
  if constexpr (kAppend) {
    const _Float16* qs = app.q + ((size_t)row * Hq + g * kG + ah) * kD;
    qlo = *(const half4_t*)(qs + ai0);
    qhi = *(const half4_t*)(qs + ai0 + kD / 2);
    const _Float16* kp = app.k + ((size_t)b * Hkv + g) * kD;
    const _Float16* vp = app.v + ((size_t)b * Hkv + g) * kD;
    kr0 = kp[lane];
    kr1 = kp[lane + kD / 2];
    vr0 = vp[lane];
    vr1 = vp[lane + kD / 2];
  }
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

  // Fused append: rotate the query (and, in the sequence's last split, the new
  // key) at pos = L - 1, spread over the wave's 64 lanes and handed to the
  // MFMA operand layout through the wave's LDS; positions outside the table
  // skip the append (the query stays as given), as kv_append_rope does.  The
  // last split keeps the new key and value in LDS until its last pair, rather
  // than in registers across the loop.  Its inputs are requested before the
  // first two pairs, by every wave and on every path (the same number of
  // loads outstanding everywhere, so the waits stay exact): a wait for them
  // then leaves both pairs in flight.
  [[maybe_unused]] const int pos = L - 1;
  [[maybe_unused]] bool app_ok = false, app_kv = false;
  [[maybe_unused]] double2 qc[4], kc;
  if constexpr (kAppend) {
    app_ok = pos < app.rope_max_pos;
    app_kv = app_ok && split == nsplit - 1;
    // (a position outside the table reads the table's last row, unused)
    const double2* rrow = app.rope + (size_t)min(pos, app.rope_max_pos - 1) * (kD / 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) qc[r] = rrow[ai0 + r];
    kc = rrow[lane];
  }
  // (the unclamped id of this split's blocks, for the fused append's write)
  [[maybe_unused]] const int raw_blk = my_blk;
  if (lane >= nb || my_blk < 0 || my_blk >= num_blocks) my_blk = 0;
  auto pair_ids = [&](int p, int& a, int& c) {
    a = __builtin_amdgcn_readlane(my_blk, 2 * p);
    c = 2 * p + 1 < nb ? __builtin_amdgcn_readlane(my_blk, 2 * p + 1) : a;
  };
  // The first pair (with the fused append, the first two) is requested before
  // anything else waits.
  Pair buf[2];
  {
    int ba, bb;
    pair_ids(0, ba, bb);
    buf[0] = load_pair<kNT>(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
    if constexpr (kAppend) {
      pair_ids(min(1, npairs - 1), ba, bb);
      buf[1] = load_pair<kNT>(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
    }
  }

  [[maybe_unused]] _Float16* kv_lds = nullptr;
  if constexpr (kAppend) {
    // per wave: rotated queries of its 4 heads, then the new key and value
    __shared__ _Float16 app_lds[kDecodeWavesPerWG][(kG + 2) * kD];
    _Float16* wl = app_lds[threadIdx.x >> 6];
    kv_lds = wl + kG * kD;
    half4_t olo = qlo, ohi = qhi;
    if (app_ok) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        double o0, o1;
        rope_pair((double)qlo[r], (double)qhi[r], qc[r].x, qc[r].y, o0, o1);
        olo[r] = store_f64<_Float16>(o0);
        ohi[r] = store_f64<_Float16>(o1);
      }
    }
    const u32x2 wlo = __builtin_bit_cast(u32x2, olo), whi = __builtin_bit_cast(u32x2, ohi);
    *(u32x2*)(wl + ah * kD + ai0) = wlo;
    *(u32x2*)(wl + ah * kD + ai0 + kD / 2) = whi;
    if (app_ok && split == 0) {
      _Float16* qo = app.q_out + ((size_t)row * Hq + g * kG + ah) * kD;
      *(u32x2*)(qo + ai0) = wlo;
      *(u32x2*)(qo + ai0 + kD / 2) = whi;
    }
    // one wave writes and reads its LDS, in order
    if (ln < kG) {
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) qb[kd] = *(const half8_t*)(wl + ln * kD + 32 * kd + 8 * lq);
    }
    if (app_kv) {
      // (keeps the key's conversion, and so the wait for its load, after the
      // pair requests above)
      asm volatile("" : "+v"(kr0), "+v"(kr1));
      double o0, o1;
      rope_pair((double)kr0, (double)kr1, kc.x, kc.y, o0, o1);
      kv_lds[lane] = store_f64<_Float16>(o0);
      kv_lds[lane + kD / 2] = store_f64<_Float16>(o1);
      kv_lds[kD + lane] = vr0;
      kv_lds[kD + lane + kD / 2] = vr1;
    }
  }
  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = (f32x4)0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // The fused append's arena write, after everything else the wave does (a
  // store counts in the same in-order counter as the pair loads, so one issued
  // before the loop would hold up the later pairs' waits).  Nothing in this
  // call reads the slot back from memory: the last pair took the new key and
  // value from LDS.
  auto store_new_kv = [&]() {
    if constexpr (kAppend) {
      if (!app_kv) return;
      const int nblk = __builtin_amdgcn_readlane(raw_blk, (pos >> 4) - blk0);
      const int slot = pos & 15;
      if (nblk >= 0 && nblk < num_blocks) {
        _Float16* kt = app.k_arena + ((size_t)nblk * Hkv + g) * kBlock * kD;
        kt[((lane / kX) * kBlock + slot) * kX + lane % kX] = kv_lds[lane];
        kt[(((lane + kD / 2) / kX) * kBlock + slot) * kX + lane % kX] = kv_lds[lane + kD / 2];
        _Float16* vt = app.v_arena + ((size_t)nblk * Hkv + g) * kD * kBlock;
        vt[lane * kBlock + slot] = kv_lds[kD + lane];
        vt[(lane + kD / 2) * kBlock + slot] = kv_lds[kD + lane + kD / 2];
      }
    }
  };

  // Keys past the context exist only in a sequence's last pair.  kMask: 0
  // masks by the position test on every pair (the plain kernel's loop, one
  // body for all pairs), 1 none (a full pair), 2 always (the last pair).
  auto compute = [&](const Pair& pr, int p, auto mode) {
    constexpr int kMask = decltype(mode)::value;
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
    auto valid = [&](int e) { return kMask == 1 || (e < 4 ? e < nva : e - 4 < nvb); };
    // The base-2 exponent of key e is fma(score_e, scale_log2, -m): one
    // rounding, written out so that no kernel leaves it to the compiler's
    // contraction choices (decode_shared_kernel must round it identically).
    // The running max is taken over raw scores and scaled once (scale_log2 >
    // 0 and rounding is monotone, so this is the max of the scaled scores).
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, valid(e) ? s[e >> 2][e & 3] : -INFINITY);
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
      const float arg = valid(e) ? __builtin_fmaf(s[e >> 2][e & 3], scale_log2, -m_new) : -INFINITY;
      const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(arg);
      pb[e] = ph;
      lsum += (float)ph;
    }
    l_run += lsum;
    // keys past the context: zero V, since their p is 0 but 0 * NaN is not
    const bool tail_pair = kMask == 2 || (kMask == 0 && (blk0 + 2 * p + 2) * kBlock > L);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      half8_t va = pr.v[db];
      if (kMask != 1 && tail_pair) {
#pragma unroll
        for (int e = 0; e < 8; ++e) va[e] = valid(e) ? va[e] : (_Float16)0.f;
      }
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o[db], 0, 0, 0);
    }
  };

  // Two pair buffers in flight, loop fully unrolled (a split is at most
  // kSB / 2 pairs).  Within the split's pairs the prefetch is issued
  // unconditionally (for the last pair it re-requests that pair, a cache
  // hit), so the loads outstanding at each wait are the same on every path
  // and the wait before a pair's MFMAs covers that pair only, never the
  // prefetch behind it; the loop is left (a wave-uniform branch) as soon as
  // the split's pairs are done (the fused append: all but the last, which is
  // computed after the loop), so a short split issues no loads past its end.
  // (A loop that ran all kSB / 2 iterations and re-requested the last pair in
  // each measured ~17 us for a one-pair split under load, against ~24 us for
  // a whole one: the re-requests occupy the compute unit's vector-memory
  // path.)  Pair p is in buffer p & 1.  (The fused append has requested the
  // second pair already.)
  run_steps([&](auto P) {
    constexpr int p = decltype(P)::value;
    if (kAppend ? p + 1 >= npairs : p >= npairs) return false;
    if (p + 1 < kSB / 2 && !(kAppend && p == 0)) {
      int ba, bb;
      pair_ids(min(p + 1, npairs - 1), ba, bb);
      buf[(p + 1) & 1] = load_pair<kNT>(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
      __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before the compute
    }
    if constexpr (kAppend) compute(buf[p & 1], p, std::integral_constant<int, 1>{});
    else compute(buf[p & 1], p, std::integral_constant<int, 0>{});
    return true;
  }, std::make_integer_sequence<int, kSB / 2>{});
  if constexpr (kAppend) {
    // The last pair, after the loop, from buffer (npairs - 1) & 1.  The new
    // token (the context's last key) enters from registers: key row `slot`
    // of its block, and the value element of key slot in lane group
    // slot >> 2.
    Pair last = ((npairs - 1) & 1) ? buf[1] : buf[0];
    if (app_kv) {
      const int slot = pos & 15, ab = ((pos >> 4) - blk0) & 1;
      // (ab and slot are wave-uniform; constant indices keep the pair in registers)
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) {
        const half8_t x = *(const half8_t*)(kv_lds + 32 * kd + 8 * lq);
        if (ln == slot) {
          if (ab == 0) last.k[0][kd] = x;
          else last.k[1][kd] = x;
        }
      }
      const int ev = 4 * ab + (slot & 3);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const _Float16 x = kv_lds[kD + 16 * db + ln];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (lq == (slot >> 2) && e == ev) last.v[db][e] = x;
      }
    }
    compute(last, npairs - 1, std::integral_constant<int, 2>{});
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
    store_new_kv();
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
  store_new_kv();
}

}  // namespace
}  // namespace pkv
