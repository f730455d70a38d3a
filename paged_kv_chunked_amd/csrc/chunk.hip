// paged_attention_chunk: chunked prefill over the block arena (Kshipra part 3,
// section 4 "Chunked Prefill": an online softmax across KV blocks read in place,
// RoPE already applied at absolute positions P onward, a causal mask over the
// chunk so that row i sees the cached prefix and the chunk up to itself).
//
// Tuned path (fp16 storage, head_dim 128, 4 query heads per KV head): a dense
// contraction, so both products run on gfx950 fp16 matrix cores
// (v_mfma_f32_16x16x32_f16, fp32 accumulation).
//   * one workgroup = (sequence, KV head, tile of 32 chunk rows); its 4 waves
//     are the 4 query heads of the group, so every K/V tile is fetched from
//     memory once for all of them;
//   * keys are walked in tiles of 64 = 4 arena blocks looked up in the block
//     table; a tile is loaded into registers one step ahead and staged in LDS
//     in the arena's own tile layouts (K in 16-byte pieces grouped by piece,
//     V head-dim-major, the latter XOR-swizzled), so every MFMA operand read
//     is bank-conflict free;
//   * S^T = K Q^T is computed with keys along the MFMA M dimension, so each
//     lane ends up holding 16 keys of one query row: the row max and sum are
//     lane-local plus two cross-lane steps, and the probabilities are already
//     in the B-operand layout of O^T += V^T P^T (the V^T operand takes the
//     same keys, 4 from each of two blocks, in the same order);
//   * online softmax in fp32 (scores in log2 units), P rounded to fp16 for the
//     second product, and the denominator summed from those rounded values so
//     the weights still add up to one;
//   * the causal mask is applied only on tiles that reach past the tile's
//     first row position; V slots past the sequence's length are zeroed in LDS
//     (p = 0 there, but 0 * NaN would not be 0).
// Other shapes run the generic kernel.
#include <cmath>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kG = 4;
constexpr int kBM = 32;  // chunk rows per workgroup (per wave: 32 rows of one head)
constexpr int kBN = 64;  // keys per tile (4 arena blocks)

// fp16 elements per 16-byte piece of the K layout [block][head][D/8][16][8].
constexpr int kX = 8;

__device__ inline uint32_t mask_pair(uint32_t x, int key0, int limit) {
  if (key0 >= limit) return 0u;
  if (key0 + 1 >= limit) return x & 0xFFFFu;
  return x;
}

// Reductions over the four lanes {l, l^16, l^32, l^48} that hold one row,
// through the gfx950 cross-row lane swaps (no LDS round trip).
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// How far (log2 units) a row's running maximum may lag the true maximum before
// the accumulator is rescaled: probabilities stay <= 2^8, well inside fp16.
constexpr float kSlack = 8.f;

__global__ __launch_bounds__(256, 2) void chunk_mfma_kernel(
    float* __restrict__ out, const _Float16* __restrict__ q,
    const _Float16* __restrict__ k_arena, const _Float16* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    float scale_log2, int Hkv, int num_seqs, int n_qtiles, int num_blocks, int num_tokens) {
  // XCD-aware order.  Linear workgroup id i runs on XCD i % 8.  The pairs
  // p = b * Hkv + g are dealt to XCDs round-robin (p % 8) and all row tiles of
  // a pair stay on its XCD, so the pair's K/V tiles are fetched into one L2
  // and reused by its row tiles; within an XCD, later (longer) row tiles of a
  // pair are issued first.
  const int npairs = num_seqs * Hkv;
  const int i = blockIdx.x;
  const int xcd = i & 7, j = i >> 3;
  const int lp = j / n_qtiles;                  // pair index among this XCD's pairs
  const int qt = n_qtiles - 1 - (j - lp * n_qtiles);
  const int p = lp * 8 + xcd;
  if (p >= npairs) return;
  const int b = p / Hkv, g = p - b * Hkv;
  const int row0 = cu_q_lens[b];
  const int C = min(cu_q_lens[b + 1], num_tokens) - row0;
  if (qt * kBM >= C) return;
  const int P = chunk_start[b];
  const int Lc = min(P + C, max_blocks * kBlock);  // keys that exist
  if (Lc <= 0) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int Hq = Hkv * kG;
  const int h = g * kG + wave;

  // Q^T as the B operand: qf[rb][kd] = Q[row 16rb + lr][dims 32kd + 8lq .. +8]
  half8_t qf[2][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = qt * kBM + 16 * rb + lr;
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) {
      if (r < C) {
        qf[rb][kd] = __builtin_bit_cast(
            half8_t, *(const u32x4*)(q + ((size_t)(row0 + r) * Hq + h) * kD + 32 * kd + 8 * lq));
      } else {
        qf[rb][kd] = (half8_t)(_Float16)0.f;
      }
    }
  }
  // absolute positions of this lane's two rows (rows past the chunk borrow the
  // last valid position so they stay finite; they are never stored)
  int prow[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) prow[rb] = min(P + qt * kBM + 16 * rb + lr, Lc - 1);

  const int row_hi = min(C, qt * kBM + kBM);
  const int kend = min(Lc, P + row_hi);  // keys [0, kend) are visible to some row
  const int ntiles = (kend + kBN - 1) / kBN;
  const int first_pos = P + qt * kBM;    // smallest row position in the tile
  const int nblk_seq = (Lc + kBlock - 1) / kBlock;
  const int32_t* bt = block_table + (size_t)b * max_blocks;

  // Two LDS buffers (tile t in buffer t & 1), so one barrier per tile suffices.
  // K: 4 blocks in the arena's own tile layout [block][piece][key][16 B], so
  //    the operand reads (16 keys x one piece per 16 lanes) are contiguous.
  // V: [block pair u][dim][4 units of 16 B]; unit j of (u, d) holds keys
  //    4j..4j+3 of block 2u followed by the same keys of block 2u+1, exactly
  //    the A operand of one PV MFMA.  Unit j sits in slot j ^ ((d >> 1) & 3),
  //    so any 8 consecutive dims of one unit index fill a 128-byte bank line.
  __shared__ u32x4 k_lds[2][4 * 256];       // 2 x 16 KiB
  __shared__ u32x4 v_lds[2][2 * kD * 4];    // 2 x 16 KiB

  u32x4 kst[4], vst[4];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int lb = t * 4 + a;
      if (lb < nblk_seq) {
        int blk = bt[lb];
        if (blk < 0 || blk >= num_blocks) blk = 0;
        const size_t tile = ((size_t)blk * Hkv + g) * (kBlock * kD / 8);
        kst[a] = ((const u32x4*)k_arena)[tile + tid];
        vst[a] = ((const u32x4*)v_arena)[tile + tid];
      } else {
        kst[a] = (u32x4)0u;
        vst[a] = (u32x4)0u;
      }
    }
  };
  auto store_tile = [&](int t) {
    u32x4* kl = k_lds[t & 1];
    u32x4* vl = v_lds[t & 1];
    const int d = tid >> 1, hh = tid & 1;  // V tile 16-byte unit tid: dim d, keys 8hh..
    const int sw = (d >> 1) & 3;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      kl[a * 256 + tid] = kst[a];
      const int k0 = t * kBN + 16 * a + 8 * hh;  // absolute key of its first half
      if (k0 + 8 > Lc) {  // zero V past the sequence: p = 0 there, but 0 * NaN is not 0
        vst[a].x = mask_pair(vst[a].x, k0, Lc);
        vst[a].y = mask_pair(vst[a].y, k0 + 2, Lc);
        vst[a].z = mask_pair(vst[a].z, k0 + 4, Lc);
        vst[a].w = mask_pair(vst[a].w, k0 + 6, Lc);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 e = vst[2 * u], o = vst[2 * u + 1];
      vl[(u * kD + d) * 4 + ((2 * hh) ^ sw)] = u32x4{e.x, e.y, o.x, o.y};
      vl[(u * kD + d) * 4 + ((2 * hh + 1) ^ sw)] = u32x4{e.z, e.w, o.z, o.w};
    }
  };

  f32x4 oacc[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) oacc[db][rb] = (f32x4)0.f;
  // Per row: running maximum of the raw scores, the raw score above which
  // the accumulator must be rescaled, -max * scale_log2, and the denominator.
  float m_raw[2] = {-INFINITY, -INFINITY}, m_lim[2] = {-INFINITY, -INFINITY};
  float m_off[2] = {0.f, 0.f}, l_run[2] = {0.f, 0.f};
  const float slack_raw = kSlack / scale_log2;
  const half2_t ones = {(_Float16)1.f, (_Float16)1.f};

  load_tile(0);
  store_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // tile t is in LDS; every wave is done with tile t - 1
    if (t + 1 < ntiles) load_tile(t + 1);
    const u32x4* kl = k_lds[t & 1];
    const u32x4* vl = v_lds[t & 1];

    // S^T[key][row] = K . Q^T (raw scores); block kb of the tile = MFMA rows 0..15
    f32x4 sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb][0] = (f32x4)0.f;
      sacc[kb][1] = (f32x4)0.f;
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) {
        const half8_t ka = __builtin_bit_cast(half8_t, kl[kb * 256 + (4 * kd + lq) * 16 + lr]);
        sacc[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[0][kd], sacc[kb][0], 0, 0, 0);
        sacc[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[1][kd], sacc[kb][1], 0, 0, 0);
      }
    }

    // causal mask (and keys past the sequence) only where the tile reaches
    // past the smallest row position
    if (t * kBN + kBN - 1 > first_pos || t * kBN + kBN > Lc) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t * kBN + 16 * kb + 4 * lq + i > prow[rb]) sacc[kb][rb][i] = -INFINITY;
    }

    // online softmax per row (this lane: rows 16rb + lr, keys 16kb + 4lq + i).
    // The running maximum is only raised when some score exceeds it by more
    // than kSlack; both the numerator and the denominator use the same
    // (possibly stale) maximum, so the quotient is unchanged.
    float mloc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float a0 = fmaxf(sacc[0][rb][0], sacc[0][rb][1]), a1 = fmaxf(sacc[0][rb][2], sacc[0][rb][3]);
#pragma unroll
      for (int kb = 1; kb < 4; ++kb) {
        a0 = fmaxf(a0, fmaxf(sacc[kb][rb][0], sacc[kb][rb][1]));
        a1 = fmaxf(a1, fmaxf(sacc[kb][rb][2], sacc[kb][rb][3]));
      }
      mloc[rb] = fmaxf(a0, a1);
    }
    if (__any(mloc[0] > m_lim[0] || mloc[1] > m_lim[1])) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float mx = max_xor16(max_xor32(mloc[rb]));
        const float m_new = fmaxf(m_raw[rb], mx);  // finite: key 0 is in tile 0 for every row
        const float alpha = __builtin_amdgcn_exp2f((m_raw[rb] - m_new) * scale_log2);
        m_raw[rb] = m_new;
        m_lim[rb] = m_new + slack_raw;
        m_off[rb] = -m_new * scale_log2;
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[db][rb] *= alpha;
      }
    }

    half8_t pb[2][2];  // [u][rb]: B operand of the second product
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const half2_t ph = {
              (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][rb][i], scale_log2, m_off[rb])),
              (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][rb][i + 1], scale_log2, m_off[rb]))};
          lsum = __builtin_amdgcn_fdot2(ph, ones, lsum, false);
          pb[kb >> 1][rb][4 * (kb & 1) + i] = ph[0];
          pb[kb >> 1][rb][4 * (kb & 1) + i + 1] = ph[1];
        }
      l_run[rb] += lsum;
    }

    // O^T[dim][row] += V^T[dim][key] . P^T[key][row]; MFMA u contracts keys
    // 4lq..4lq+3 of blocks 2u and 2u+1 in this lane (the order of pb)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 16 * db + lr;
        const half8_t va = __builtin_bit_cast(half8_t, vl[(u * kD + d) * 4 + (lq ^ ((d >> 1) & 3))]);
        oacc[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[u][0], oacc[db][0], 0, 0, 0);
        oacc[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[u][1], oacc[db][1], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) store_tile(t + 1);  // other buffer: its readers passed the barrier
  }

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float l = sum_xor16(sum_xor32(l_run[rb]));
    const float inv = 1.f / l;
    const int r = qt * kBM + 16 * rb + lr;
    if (r < C) {
      float* dst = out + ((size_t)(row0 + r) * Hq + h) * kD + 4 * lq;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f32x4 v = oacc[db][rb] * inv;
        *(f32x4*)(dst + 16 * db) = v;
      }
    }
  }
}

}  // namespace

bool chunk_fast_path(const pkv_geom& g) {
  return g.dtype == PKV_F16 && g.head_dim == kD && g.num_q_heads == kG * g.num_kv_heads;
}

hipError_t launch_chunk(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                        const void* v_arena, const int32_t* block_table, int max_blocks,
                        const int32_t* cu_q_lens, const int32_t* chunk_start, int num_seqs,
                        int num_tokens, int max_q_len, int max_context_len, float scale,
                        hipStream_t stream) {
  (void)max_context_len;
  // the fast path tracks maxima of raw scores, which needs scale > 0
  if (!chunk_fast_path(g) || !(scale > 0.f) || !std::isfinite(scale))
    return launch_attend_generic(g, out, q, k_arena, v_arena, block_table, max_blocks, nullptr,
                                 cu_q_lens, chunk_start, num_seqs, num_tokens, scale, stream);
  const int n_qtiles = (max_q_len + kBM - 1) / kBM;
  const float scale_log2 = scale * 1.4426950408889634f;
  const long npairs = (long)num_seqs * g.num_kv_heads;
  const long nwg = 8 * ((npairs + 7) / 8) * n_qtiles;
  hipLaunchKernelGGL(chunk_mfma_kernel, dim3((unsigned)nwg), dim3(256), 0, stream, out,
                     (const _Float16*)q, (const _Float16*)k_arena, (const _Float16*)v_arena,
                     block_table, max_blocks, cu_q_lens, chunk_start, scale_log2,
                     g.num_kv_heads, num_seqs, n_qtiles, g.num_blocks, num_tokens);
  return hipGetLastError();
}

}  // namespace pkv
