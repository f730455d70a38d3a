// kv_append_rope: rotate new q/k at their absolute positions and scatter k/v
// into the block arena (Kshipra part 3, section 1 "Block-Arena KV Cache" and
// section 4 "Chunked Prefill": RoPE at absolute positions P onward).
//
// Arena layouts: K [block][head][D/x][16][x] with x = 16 bytes of elements,
// V [block][head][D][16].  One or (small batches) four 256-thread workgroups
// per new token, each with an even share of its work; each thread owns whole rotation pairs
// (i, i + D/2), so an in-place q rotation is race-free.  The rotation runs in fp64 with fused multiply-add disabled and is
// rounded once to the storage dtype (fp16: round-to-odd to fp32, then to
// nearest-even; fp32: the hardware's round-to-nearest-even convert), so the
// stored values are exactly determined by the inputs.
#include "fp16_shape.h"
#include "pkv_internal.h"
#include "quant_append_core.h"
#include "rope_core.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// The query pairs (i, i + D/2) of one token that this thread rotates: the
// first kQBatch are loaded into registers before the token's position is
// looked up (their addresses depend on the token index only), so those loads
// overlap the lookup chain instead of following it.  q may alias q_out: every
// pair is read and written by one thread, and a thread reads its pairs before
// writing any of them.
constexpr int kQBatch = 8;
template <typename T>
struct QRotation {
  T lo[kQBatch], hi[kQBatch];
  int n0, n, half;  // pairs [n0, n) of the token are this workgroup's
  size_t tok;       // element offset of the token's first query head
  // k_tok: the token's k, read instead when there is no q to rotate, so the
  // loads need no branch (values past the end are never used)
  __device__ void load(const T* q, const T* k_tok, int t, int Hq, int D, int slice,
                       int slices) {
    half = D >> 1;
    const int total = q != nullptr ? Hq * half : 0;
    n0 = (int)((long)total * slice / slices);
    n = (int)((long)total * (slice + 1) / slices);
    tok = (size_t)t * Hq * D;
    const T* src = q != nullptr ? q + tok : k_tok;
    // unconditional loads (indices past the end read the last pair, unused),
    // so that they are all in flight together
#pragma unroll
    for (int j = 0; j < kQBatch; ++j) {
      const int idx = min(n0 + (int)threadIdx.x + j * kThreads, max(n - 1, 0));
      const int h = idx / half, i = idx - h * half;
      lo[j] = src[(size_t)h * D + i];
      hi[j] = src[(size_t)h * D + i + half];
    }
  }
  __device__ void finish(const T* q, T* q_out, const double2* __restrict__ row, int D) {
#pragma unroll
    for (int j = 0; j < kQBatch; ++j) {
      const int idx = n0 + threadIdx.x + j * kThreads;
      if (idx < n) {
        const int h = idx / half, i = idx - h * half;
        const size_t base = tok + (size_t)h * D;
        const double2 c = row[i];
        double o0, o1;
        rope_pair((double)lo[j], (double)hi[j], c.x, c.y, o0, o1);
        q_out[base + i] = store_f64<T>(o0);
        q_out[base + i + half] = store_f64<T>(o1);
      }
    }
    // heads beyond the register batch (more than kQBatch * kThreads pairs)
    for (int idx = n0 + threadIdx.x + kQBatch * kThreads; idx < n; idx += kThreads) {
      const int h = idx / half, i = idx - h * half;
      const size_t base = tok + (size_t)h * D;
      const double2 c = row[i];
      double o0, o1;
      rope_pair((double)q[base + i], (double)q[base + i + half], c.x, c.y, o0, o1);
      q_out[base + i] = store_f64<T>(o0);
      q_out[base + i + half] = store_f64<T>(o1);
    }
  }
};

// The same rotation in 16-byte pieces of 8 pairs (head dims that are a
// multiple of 16): thread i takes pieces n0 + i, n0 + i + kThreads, ... of the
// workgroup's share, each read whole and written whole (in place allowed: a
// piece is read before it is written, by the same thread).
struct QRotationVec {
  half8_t lo, hi;   // the thread's first piece, loaded before the position lookup
  int n0, n, cph, iq;
  size_t tok;
  __device__ void load(const _Float16* q, const _Float16* k_tok, int t, int Hq, int D, int slice,
                       int slices) {
    cph = (D >> 1) / 8;  // pieces per half head
    const int total = q != nullptr ? Hq * cph : 0;
    n0 = (int)((long)total * slice / slices);
    n = (int)((long)total * (slice + 1) / slices);
    tok = (size_t)t * Hq * D;
    const _Float16* src = q != nullptr ? q + tok : k_tok;
    iq = min(n0 + (int)threadIdx.x, max(n - 1, 0));
    const _Float16* at = src + (size_t)(iq / cph) * D + (iq % cph) * 8;
    lo = *(const half8_t*)at;
    hi = *(const half8_t*)(at + (D >> 1));
  }
  __device__ void finish(const _Float16* q, _Float16* q_out, const double2* __restrict__ row,
                         int D) {
    const int half = D >> 1;
    for (int idx = n0 + (int)threadIdx.x; idx < n; idx += kThreads) {
      const size_t off = tok + (size_t)(idx / cph) * D + (idx % cph) * 8;
      const half8_t a = idx == iq ? lo : *(const half8_t*)(q + off);
      const half8_t c = idx == iq ? hi : *(const half8_t*)(q + off + half);
      half8_t oa, oc;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double2 r = row[(idx % cph) * 8 + e];
        double o0, o1;
        rope_pair((double)a[e], (double)c[e], r.x, r.y, o0, o1);
        oa[e] = store_f64<_Float16>(o0);
        oc[e] = store_f64<_Float16>(o1);
      }
      *(half8_t*)(q_out + off) = oa;
      *(half8_t*)(q_out + off + half) = oc;
    }
  }
};

// Token of workgroup column x of n.  Workgroups are dealt to the 8 XCDs
// round-robin by linear id; this permutation gives XCD c the tokens
// [c q + min(c, r), ...) in order (n = 8 q + r), so the 16 tokens of an arena
// block, whose V elements interleave within each 32-byte row of the tile, are
// written through one L2 and merge there into whole lines.
__device__ inline int xcd_token(int x, int n) {
  const int q = n >> 3, r = n & 7, c = x & 7;
  return c * q + min(c, r) + (x >> 3);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void append_rope_kernel(
    const T* q, T* q_out, const T* __restrict__ k,
    const T* __restrict__ v, T* __restrict__ k_arena, T* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    int num_seqs, const double2* __restrict__ cs, int rope_max_pos, int num_blocks, int Hq,
    int Hkv, int D) {
  const int t = xcd_token(blockIdx.x, gridDim.x);
  const int half = D >> 1;
  // workgroup blockIdx.y of gridDim.y takes an even share of the token's q
  // pairs, k pairs and v elements
  const int sl = blockIdx.y, S = gridDim.y;
  // the token's q, k and v are requested before its position is looked up
  QRotation<T> qr;
  qr.load(q, k + (size_t)t * Hkv * D, t, Hq, D, sl, S);
  constexpr int kKB = 2, kVB = 4;
  const int nk0 = (int)((long)Hkv * half * sl / S), nk = (int)((long)Hkv * half * (sl + 1) / S);
  const int nv0 = (int)((long)Hkv * D * sl / S), nv = (int)((long)Hkv * D * (sl + 1) / S);
  T klo[kKB], khi[kKB], vv[kVB];
#pragma unroll
  for (int j = 0; j < kKB; ++j) {  // unconditional, as for q
    const int idx = max(min(nk0 + (int)threadIdx.x + j * kThreads, nk - 1), 0);
    const int h = idx / half, i = idx - h * half;
    const T* kp = k + ((size_t)t * Hkv + h) * D;
    klo[j] = kp[i];
    khi[j] = kp[i + half];
  }
#pragma unroll
  for (int j = 0; j < kVB; ++j)
    vv[j] = v[(size_t)t * Hkv * D + max(min(nv0 + (int)threadIdx.x + j * kThreads, nv - 1), 0)];
  int row0, P;
  const int b = find_seq_start(cu_q_lens, chunk_start, num_seqs, t, row0, P);
  const int pos = P + (t - row0);
  if (pos < 0 || pos >= rope_max_pos || (pos >> 4) >= max_blocks) return;
  const int blk = block_table[(size_t)b * max_blocks + (pos >> 4)];
  const int slot = pos & 15;
  const double2* row = cs + (size_t)pos * half;

  qr.finish(q, q_out, row, D);
  if (blk < 0 || blk >= num_blocks) return;
  constexpr int x = 16 / sizeof(T);  // K tile layout [D/x][16][x]
  auto put_k = [&](int idx, T a, T c_hi) {
    const int h = idx / half, i = idx - h * half;
    const double2 c = row[i];
    double o0, o1;
    rope_pair((double)a, (double)c_hi, c.x, c.y, o0, o1);
    T* tile = k_arena + ((size_t)blk * Hkv + h) * kBlock * D;
    tile[((i / x) * kBlock + slot) * x + i % x] = store_f64<T>(o0);
    tile[(((i + half) / x) * kBlock + slot) * x + (i + half) % x] = store_f64<T>(o1);
  };
#pragma unroll
  for (int j = 0; j < kKB; ++j) {
    const int idx = nk0 + threadIdx.x + j * kThreads;
    if (idx < nk) put_k(idx, klo[j], khi[j]);
  }
  for (int idx = nk0 + threadIdx.x + kKB * kThreads; idx < nk; idx += kThreads) {
    const int h = idx / half, i = idx - h * half;
    const T* kp = k + ((size_t)t * Hkv + h) * D;
    put_k(idx, kp[i], kp[i + half]);
  }
  auto put_v = [&](int idx, T val) {
    const int h = idx / D, d = idx - h * D;
    v_arena[(((size_t)blk * Hkv + h) * D + d) * kBlock + slot] = val;
  };
#pragma unroll
  for (int j = 0; j < kVB; ++j) {
    const int idx = nv0 + threadIdx.x + j * kThreads;
    if (idx < nv) put_v(idx, vv[j]);
  }
  for (int idx = nv0 + threadIdx.x + kVB * kThreads; idx < nv; idx += kThreads)
    put_v(idx, v[(size_t)t * Hkv * D + idx]);
}

// Vector form for head dims whose halves are whole 16-byte pieces (the
// tuned shapes): a thread rotates one piece of x = 16 / sizeof(T) pairs --
// dims i0 .. i0+x-1 with their partners i0+D/2 .. -- with two 16-byte loads
// and two 16-byte stores, for q and for k; a k piece is exactly one 16-byte
// slot of the K tile.  V keeps element stores (its tile is head-dim-major).
// The first piece of each kind and the first v elements are loaded before the
// position lookup, as in the scalar form.
template <typename T>
__global__ __launch_bounds__(kThreads) void append_rope_vec_kernel(
    const T* q, T* q_out, const T* __restrict__ k, const T* __restrict__ v,
    T* __restrict__ k_arena, T* __restrict__ v_arena, const int32_t* __restrict__ block_table,
    int max_blocks, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ chunk_start, int num_seqs, const double2* __restrict__ cs,
    int rope_max_pos, int num_blocks, int Hq, int Hkv, int D) {
  constexpr int x = 16 / sizeof(T);
  typedef T vecT __attribute__((ext_vector_type(x)));
  const int t = xcd_token(blockIdx.x, gridDim.x), sl = blockIdx.y, S = gridDim.y;
  const int half = D >> 1, cph = half / x;  // pieces per half head
  auto share = [&](int n, int& lo, int& hi) {
    lo = (int)((long)n * sl / S);
    hi = (int)((long)n * (sl + 1) / S);
  };
  int nq0, nq, nk0, nk, nv0, nv;
  share(q != nullptr ? Hq * cph : 0, nq0, nq);
  share(Hkv * cph, nk0, nk);
  share(Hkv * D, nv0, nv);
  const size_t qtok = (size_t)t * Hq * D, ktok = (size_t)t * Hkv * D;
  // first pieces, unconditionally (a clamped index past the end is unused)
  const T* qsrc = q != nullptr ? q + qtok : k + ktok;
  auto piece_ptr = [&](const T* base, int idx) { return base + (idx / cph) * D + (idx % cph) * x; };
  const int iq = min(nq0 + (int)threadIdx.x, max(nq - 1, 0));
  const int ik = max(min(nk0 + (int)threadIdx.x, nk - 1), 0);  // a share may be empty
  const vecT qlo = *(const vecT*)piece_ptr(qsrc, iq), qhi = *(const vecT*)(piece_ptr(qsrc, iq) + half);
  const vecT klo = *(const vecT*)piece_ptr(k + ktok, ik), khi = *(const vecT*)(piece_ptr(k + ktok, ik) + half);
  constexpr int kVB = 4;
  T vv[kVB];
#pragma unroll
  for (int j = 0; j < kVB; ++j)
    vv[j] = v[ktok + max(min(nv0 + (int)threadIdx.x + j * kThreads, nv - 1), 0)];

  int row0, P;
  const int b = find_seq_start(cu_q_lens, chunk_start, num_seqs, t, row0, P);
  const int pos = P + (t - row0);
  if (pos < 0 || pos >= rope_max_pos || (pos >> 4) >= max_blocks) return;
  const int blk = block_table[(size_t)b * max_blocks + (pos >> 4)];
  const int slot = pos & 15;
  const double2* row = cs + (size_t)pos * half;

  auto rotate = [&](vecT lo, vecT hi, int c, vecT& olo, vecT& ohi) {
#pragma unroll
    for (int e = 0; e < x; ++e) {
      const double2 r = row[c * x + e];
      double o0, o1;
      rope_pair((double)lo[e], (double)hi[e], r.x, r.y, o0, o1);
      olo[e] = store_f64<T>(o0);
      ohi[e] = store_f64<T>(o1);
    }
  };
  // q: in place allowed (each piece is read and written by one thread, which
  // reads it before writing)
  for (int idx = nq0 + threadIdx.x; idx < nq; idx += kThreads) {
    const vecT lo = idx == iq ? qlo : *(const vecT*)piece_ptr(q + qtok, idx);
    const vecT hi = idx == iq ? qhi : *(const vecT*)(piece_ptr(q + qtok, idx) + half);
    vecT olo, ohi;
    rotate(lo, hi, idx % cph, olo, ohi);
    T* dst = q_out + qtok + (idx / cph) * D + (idx % cph) * x;
    *(vecT*)dst = olo;
    *(vecT*)(dst + half) = ohi;
  }
  if (blk < 0 || blk >= num_blocks) return;
  for (int idx = nk0 + threadIdx.x; idx < nk; idx += kThreads) {
    const vecT lo = idx == ik ? klo : *(const vecT*)piece_ptr(k + ktok, idx);
    const vecT hi = idx == ik ? khi : *(const vecT*)(piece_ptr(k + ktok, idx) + half);
    const int h = idx / cph, c = idx % cph;
    vecT olo, ohi;
    rotate(lo, hi, c, olo, ohi);
    T* tile = k_arena + ((size_t)blk * Hkv + h) * kBlock * D;  // [D/x][16][x]
    *(vecT*)(tile + (c * kBlock + slot) * x) = olo;
    *(vecT*)(tile + ((c + cph) * kBlock + slot) * x) = ohi;
  }
  auto put_v = [&](int idx, T val) {
    const int h = idx / D, d = idx - h * D;
    v_arena[(((size_t)blk * Hkv + h) * D + d) * kBlock + slot] = val;
  };
#pragma unroll
  for (int j = 0; j < kVB; ++j) {
    const int idx = nv0 + threadIdx.x + j * kThreads;
    if (idx < nv) put_v(idx, vv[j]);
  }
  for (int idx = nv0 + threadIdx.x + kVB * kThreads; idx < nv; idx += kThreads)
    put_v(idx, v[ktok + idx]);
}

// kv_append_rope for batches of long chunks (fp16, head dims whose halves are
// whole 16-byte pieces, at most kBlockSeqs sequences): one workgroup per
// (sequence, arena block) the call writes, so that a block filled whole by the
// call is written as whole lines -- each K piece's 16 slots (256 bytes) and
// each value row's 16 slots (32 bytes, eight rows per thread) together --
// instead of each token writing 2-byte pieces of 48 lines per head.  Blocks
// the call fills in part (a sequence's first and last) write the slots they
// hold, as the per-token kernel does.  The same arithmetic as
// append_rope_vec_kernel, so the same bytes.
constexpr int kBlockSeqs = 64;
#ifndef PKV_APPEND_BLOCK_SLICES
#define PKV_APPEND_BLOCK_SLICES 4
#endif
constexpr int kBlockSlices = PKV_APPEND_BLOCK_SLICES;  // workgroups per block
__global__ __launch_bounds__(kThreads) void append_rope_block_kernel(
    const _Float16* q, _Float16* q_out, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, _Float16* __restrict__ k_arena, _Float16* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    int num_seqs, int num_tokens, const double2* __restrict__ cs, int rope_max_pos,
    int num_blocks, int Hq, int Hkv, int D) {
  constexpr int x = 8;  // fp16 elements per 16-byte piece
  typedef _Float16 vecT __attribute__((ext_vector_type(x)));
  const int lane = threadIdx.x & 63, w = blockIdx.x;
  // workgroup slice sl of S takes items sl * kThreads + i, + S * kThreads, ...
  const int first = blockIdx.y * kThreads + threadIdx.x, stride = gridDim.y * kThreads;
  // the sequences' block ranges, one sequence per lane (every wave alike)
  int row0 = 0, C = 0, P = 0, nblk = 0;
  if (lane < num_seqs) {
    row0 = cu_q_lens[lane];
    C = min(cu_q_lens[lane + 1], num_tokens) - row0;
    P = chunk_start[lane];
    if (C > 0) nblk = ((P + C - 1) >> 4) - (P >> 4) + 1;
  }
  int incl = nblk;  // inclusive prefix sum over the lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  const int excl = incl - nblk;
  const unsigned long long m = __ballot(lane < num_seqs && nblk > 0 && excl <= w && w < incl);
  if (m == 0) return;  // past the call's blocks
  const int sb = __ffsll((long long)m) - 1;
  const int b_row0 = __builtin_amdgcn_readlane(row0, sb);
  const int b_C = __builtin_amdgcn_readlane(C, sb), b_P = __builtin_amdgcn_readlane(P, sb);
  const int j = (b_P >> 4) + (w - __builtin_amdgcn_readlane(excl, sb));
  // positions of this block the call holds, as the per-token kernel accepts them
  const int pos_lo = max(max(b_P, 16 * j), 0);
  const int pos_hi = min(min(b_P + b_C, 16 * j + 16), rope_max_pos);
  if (j < 0 || j >= max_blocks || pos_lo >= pos_hi) return;
  const int s_lo = pos_lo - 16 * j, s_hi = pos_hi - 16 * j, ns = s_hi - s_lo;
  const int t_lo = b_row0 + (pos_lo - b_P);  // token of slot s_lo
  const int half = D >> 1, cph = half / x;
  const int blk = block_table[(size_t)__builtin_amdgcn_readfirstlane(sb) * max_blocks + j];
  auto rotate = [&](vecT lo, vecT hi, const double2* row, int c, vecT& olo, vecT& ohi) {
#pragma unroll
    for (int e = 0; e < x; ++e) {
      const double2 r = row[c * x + e];
      double o0, o1;
      rope_pair((double)lo[e], (double)hi[e], r.x, r.y, o0, o1);
      olo[e] = store_f64<_Float16>(o0);
      ohi[e] = store_f64<_Float16>(o1);
    }
  };
  // q (in place allowed: each piece is read and written by one thread)
  if (q != nullptr) {
    const int nq = ns * Hq * cph;
    for (int idx = first; idx < nq; idx += stride) {
      const int st = idx / (Hq * cph), r = idx - st * (Hq * cph);
      const int h = r / cph, c = r - h * cph;
      const size_t off = ((size_t)(t_lo + st) * Hq + h) * D + c * x;
      const vecT lo = *(const vecT*)(q + off), hi = *(const vecT*)(q + off + half);
      vecT olo, ohi;
      rotate(lo, hi, cs + (size_t)(pos_lo + st) * half, c, olo, ohi);
      *(vecT*)(q_out + off) = olo;
      *(vecT*)(q_out + off + half) = ohi;
    }
  }
  if (blk < 0 || blk >= num_blocks) return;
  // K: item (head h, piece c, slot s), slot fastest, so a wave writes whole
  // 256-byte runs [c][0..16][x] of a tile
  for (int idx = first; idx < Hkv * cph * 16; idx += stride) {
    const int s = idx & 15, hc = idx >> 4, h = hc / cph, c = hc - h * cph;
    if (s < s_lo || s >= s_hi) continue;
    const size_t off = ((size_t)(t_lo + s - s_lo) * Hkv + h) * D + c * x;
    const vecT lo = *(const vecT*)(k + off), hi = *(const vecT*)(k + off + half);
    vecT olo, ohi;
    rotate(lo, hi, cs + (size_t)(16 * j + s) * half, c, olo, ohi);
    _Float16* tile = k_arena + ((size_t)blk * Hkv + h) * kBlock * D;  // [D/x][16][x]
    *(vecT*)(tile + (c * kBlock + s) * x) = olo;
    *(vecT*)(tile + ((c + cph) * kBlock + s) * x) = ohi;
  }
  // V tile [D][16]
  if (ns == kBlock) {
    // whole block: item (head h, 8 dims from 8 g); the thread reads the 16
    // tokens' 8 values and writes the 8 rows of 16 slots
    for (int idx = first; idx < Hkv * (D / x); idx += stride) {
      const int h = idx / (D / x), g8 = idx - h * (D / x);
      vecT col[kBlock];
#pragma unroll
      for (int s = 0; s < kBlock; ++s)
        col[s] = *(const vecT*)(v + ((size_t)(t_lo + s) * Hkv + h) * D + g8 * x);
      _Float16* vt = v_arena + (((size_t)blk * Hkv + h) * D + g8 * x) * kBlock;
#pragma unroll
      for (int e = 0; e < x; ++e) {
        vecT r0, r1;
#pragma unroll
        for (int s = 0; s < x; ++s) {
          r0[s] = col[s][e];
          r1[s] = col[s + x][e];
        }
        *(vecT*)(vt + e * kBlock) = r0;
        *(vecT*)(vt + e * kBlock + x) = r1;
      }
    }
  } else {
    // the slots this call holds: item (head h, dim d, slot s), slot fastest
    for (int idx = first; idx < Hkv * D * ns; idx += stride) {
      const int st = idx % ns, hd = idx / ns, h = hd / D, d = hd - h * D;
      v_arena[(((size_t)blk * Hkv + h) * D + d) * kBlock + s_lo + st] =
          v[((size_t)(t_lo + st) * Hkv + h) * D + d];
    }
  }
}

// kv_append_rope for INT8 arenas (q, k, v fp16).  Tile of one (block, head):
// K codes [D/16][16][16] then 16 fp16 scales; V codes [D][16] then 16 fp16
// scales.  k is rotated and rounded to fp16 exactly as for an fp16 arena, then
// quantized.
__global__ __launch_bounds__(kThreads) void append_rope_i8_kernel(
    const _Float16* q, _Float16* q_out, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, uint8_t* __restrict__ k_arena, uint8_t* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    int num_seqs, const double2* __restrict__ cs, int rope_max_pos, int num_blocks, int Hq,
    int Hkv, int D) {
  const int t = xcd_token(blockIdx.x, gridDim.x);
  // workgroup blockIdx.y of gridDim.y takes an even share of the q pairs and
  // the KV heads blockIdx.y * kWaves + wave, + gridDim.y * kWaves, ...
  const int sl = blockIdx.y, S = gridDim.y;
  QRotationVec qr;
  qr.load(q, k + (size_t)t * Hkv * D, t, Hq, D, sl, S);  // before the position lookup
  int row0, P;
  const int b = find_seq_start(cu_q_lens, chunk_start, num_seqs, t, row0, P);
  const int pos = P + (t - row0);
  if (pos < 0 || pos >= rope_max_pos || (pos >> 4) >= max_blocks) return;
  const int blk = block_table[(size_t)b * max_blocks + (pos >> 4)];
  const int slot = pos & 15;
  const int half = D >> 1;
  const double2* row = cs + (size_t)pos * half;

  qr.finish(q, q_out, row, D);
  if (blk < 0 || blk >= num_blocks) return;
  const size_t tile_bytes = i8_tile_bytes(D);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int kWaves = kThreads / 64;
  // K: wave w quantizes heads w, w + kWaves, ...; lane l rotates the pairs
  // (l, l + half) and (l + 64, l + 64 + half) that exist
  for (int h = sl * kWaves + wave; h < Hkv; h += S * kWaves)
    append_k_i8(k + ((size_t)t * Hkv + h) * D, row, k_arena + ((size_t)blk * Hkv + h) * tile_bytes,
                slot, D, lane);
  // V: lane l holds elements l, l + 64, l + 128, l + 192
  for (int h = sl * kWaves + wave; h < Hkv; h += S * kWaves)
    append_v_i8(v + ((size_t)t * Hkv + h) * D, v_arena + ((size_t)blk * Hkv + h) * tile_bytes,
                slot, D, lane);
}

// kv_append_rope for INT4 arenas.  K: byte i of a key's 8-byte record in a
// 16-dim piece holds dims i and i + 8 -- lanes i and i + 8 of the wave, joined
// with one shuffle.  V: the byte of a head dim that holds slot s also holds
// slot s ^ 4; when both tokens are in this call the one with bit 2 clear
// writes the byte, otherwise the token present merges its nibble into the
// stored byte.  No byte is written by two workgroups of one call.
__global__ __launch_bounds__(kThreads) void append_rope_i4_kernel(
    const _Float16* q, _Float16* q_out, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, uint8_t* __restrict__ k_arena, uint8_t* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    int num_seqs, int num_tokens, const double2* __restrict__ cs, int rope_max_pos,
    int num_blocks, int Hq, int Hkv, int D) {
  const int t = xcd_token(blockIdx.x, gridDim.x);
  // workgroup blockIdx.y of gridDim.y takes an even share of the q pairs and
  // the KV heads blockIdx.y * kWaves + wave, + gridDim.y * kWaves, ...
  const int sl = blockIdx.y, S = gridDim.y;
  QRotationVec qr;
  qr.load(q, k + (size_t)t * Hkv * D, t, Hq, D, sl, S);  // before the position lookup
  int row0, P;
  const int b = find_seq_start(cu_q_lens, chunk_start, num_seqs, t, row0, P);
  const int pos = P + (t - row0);
  if (pos < 0 || pos >= rope_max_pos || (pos >> 4) >= max_blocks) return;
  const int blk = block_table[(size_t)b * max_blocks + (pos >> 4)];
  const int slot = pos & 15;
  const int half = D >> 1;
  const double2* row = cs + (size_t)pos * half;

  qr.finish(q, q_out, row, D);
  if (blk < 0 || blk >= num_blocks) return;
  const size_t tile_bytes = i4_tile_bytes(D);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int kWaves = kThreads / 64;
  for (int h = sl * kWaves + wave; h < Hkv; h += S * kWaves)
    append_k_i4(k + ((size_t)t * Hkv + h) * D, row, k_arena + ((size_t)blk * Hkv + h) * tile_bytes,
                slot, D, lane);
  // V: the token sharing this token's bytes, and which of the two writes them
  const int C = min(cu_q_lens[b + 1], num_tokens) - row0;
  const int ppos = pos ^ 4;
  const bool partner_in = ppos >= P && ppos < P + C;
  const bool leader = (pos & 4) == 0 || !partner_in;
  const int tp = t + (ppos - pos);
  for (int h = sl * kWaves + wave; h < Hkv; h += S * kWaves)
    append_v_i4(v + ((size_t)t * Hkv + h) * D,
                partner_in ? v + ((size_t)tp * Hkv + h) * D : nullptr, leader,
                v_arena + ((size_t)blk * Hkv + h) * tile_bytes, slot, D, lane);
}

}  // namespace

hipError_t launch_append_rope(const pkv_geom& g, const void* q, void* q_out, const void* k,
                              const void* v, void* k_arena, void* v_arena,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* cu_q_lens, const int32_t* chunk_start,
                              int num_seqs, int num_tokens, const void* rope_table,
                              int rope_max_pos, hipStream_t stream) {
  // Small batches (decode steps) spread each token over 4 workgroups: their
  // append is latency-bound, and shorter per-workgroup chains help (10.8 ->
  // 6.0 us for 64 tokens).  Large batches already fill the chip with one
  // workgroup per token, and slicing them only adds lookups (58 -> 75 us for
  // 4096 tokens).
  const int slices = num_tokens < 512 ? 4 : 1;
  const dim3 grid(num_tokens, slices), block(kThreads);
  if (g.dtype == PKV_I4KV) {
    hipLaunchKernelGGL(append_rope_i4_kernel, grid, block, 0, stream, (const _Float16*)q,
                       (_Float16*)q_out, (const _Float16*)k, (const _Float16*)v,
                       (uint8_t*)k_arena, (uint8_t*)v_arena, block_table, max_blocks, cu_q_lens,
                       chunk_start, num_seqs, num_tokens, (const double2*)rope_table,
                       rope_max_pos, g.num_blocks, g.num_q_heads, g.num_kv_heads, g.head_dim);
    return hipGetLastError();
  }
  if (g.dtype == PKV_I8KV) {
    hipLaunchKernelGGL(append_rope_i8_kernel, grid, block, 0, stream, (const _Float16*)q,
                       (_Float16*)q_out, (const _Float16*)k, (const _Float16*)v,
                       (uint8_t*)k_arena, (uint8_t*)v_arena, block_table, max_blocks, cu_q_lens,
                       chunk_start, num_seqs, (const double2*)rope_table, rope_max_pos,
                       g.num_blocks, g.num_q_heads, g.num_kv_heads, g.head_dim);
    return hipGetLastError();
  }
  const bool vec = (g.head_dim / 2) % (g.dtype == PKV_F16 ? 8 : 4) == 0;
  // batches of long chunks: one workgroup per (sequence, arena block)
  if (g.dtype == PKV_F16 && vec && num_seqs <= kBlockSeqs && num_tokens >= 512 &&
      num_tokens >= 32 * num_seqs) {
    const int nwg = num_tokens / kBlock + 2 * num_seqs;
    hipLaunchKernelGGL(append_rope_block_kernel, dim3(nwg, kBlockSlices), block, 0, stream,
                       (const _Float16*)q, (_Float16*)q_out, (const _Float16*)k,
                       (const _Float16*)v, (_Float16*)k_arena, (_Float16*)v_arena, block_table,
                       max_blocks, cu_q_lens, chunk_start, num_seqs, num_tokens,
                       (const double2*)rope_table, rope_max_pos, g.num_blocks, g.num_q_heads,
                       g.num_kv_heads, g.head_dim);
    return hipGetLastError();
  }
  if (g.dtype == PKV_F16 && vec) {
    hipLaunchKernelGGL(append_rope_vec_kernel<_Float16>, grid, block, 0, stream,
                       (const _Float16*)q, (_Float16*)q_out, (const _Float16*)k,
                       (const _Float16*)v, (_Float16*)k_arena, (_Float16*)v_arena, block_table,
                       max_blocks, cu_q_lens, chunk_start, num_seqs, (const double2*)rope_table,
                       rope_max_pos, g.num_blocks, g.num_q_heads, g.num_kv_heads, g.head_dim);
  } else if (g.dtype == PKV_F32 && vec) {
    hipLaunchKernelGGL(append_rope_vec_kernel<float>, grid, block, 0, stream, (const float*)q,
                       (float*)q_out, (const float*)k, (const float*)v, (float*)k_arena,
                       (float*)v_arena, block_table, max_blocks, cu_q_lens, chunk_start,
                       num_seqs, (const double2*)rope_table, rope_max_pos, g.num_blocks,
                       g.num_q_heads, g.num_kv_heads, g.head_dim);
  } else if (g.dtype == PKV_F16) {
    hipLaunchKernelGGL(append_rope_kernel<_Float16>, grid, block, 0, stream,
                       (const _Float16*)q, (_Float16*)q_out, (const _Float16*)k,
                       (const _Float16*)v, (_Float16*)k_arena, (_Float16*)v_arena, block_table,
                       max_blocks, cu_q_lens, chunk_start, num_seqs, (const double2*)rope_table,
                       rope_max_pos, g.num_blocks, g.num_q_heads, g.num_kv_heads, g.head_dim);
  } else {
    hipLaunchKernelGGL(append_rope_kernel<float>, grid, block, 0, stream, (const float*)q,
                       (float*)q_out, (const float*)k, (const float*)v, (float*)k_arena,
                       (float*)v_arena, block_table, max_blocks, cu_q_lens, chunk_start,
                       num_seqs, (const double2*)rope_table, rope_max_pos, g.num_blocks,
                       g.num_q_heads, g.num_kv_heads, g.head_dim);
  }
  return hipGetLastError();
}

}  // namespace pkv
