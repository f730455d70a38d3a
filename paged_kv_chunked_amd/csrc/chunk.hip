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
//     table; a tile is loaded into registers one step ahead and staged in LDS:
//     K token-major, V head-dim-major (the arena's own layouts), XOR-swizzled
//     so the MFMA operand reads are bank-conflict free;
//   * S^T = K Q^T is computed with keys along the MFMA M dimension, so each
//     lane ends up holding 16 keys of one query row: the row max and sum are
//     lane-local plus two cross-lane steps, and the probabilities are already
//     in the B-operand layout of O^T += V^T P^T (keys are permuted
//     consistently in both products, which a contraction allows);
//   * online softmax in fp32 (scores in log2 units), P rounded to fp16 for the
//     second product, and the denominator summed from those rounded values so
//     the weights still add up to one;
//   * the causal mask is applied only on tiles that reach past the tile's
//     first row position; V slots past the sequence's length are zeroed in LDS
//     (p = 0 there, but 0 * NaN would not be 0).
// Other shapes run the generic kernel.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kG = 4;
constexpr int kBM = 32;  // chunk rows per workgroup (per wave: 32 rows of one head)
constexpr int kBN = 64;  // keys per tile (4 arena blocks)

// K LDS swizzle: the 16 keys one MFMA reads together differ in key bits
// {0,1,3,4}; mapping them to 4 distinct bits spreads the 16 lanes over 16
// different 16-byte chunks.
__device__ inline int k_swz(int key) { return (key & 3) | ((key >> 1) & 12); }

// Physical key (0..63 in the tile) behind row m of the 16-key S^T block kb.
// Chosen so that, after the first product, lane group q holds keys
// 32u + 8q .. 32u + 8q + 7 (u = kb / 2): 8 consecutive keys of one arena
// block — exactly one 16-byte V^T read in the second product.
__device__ inline int key_of(int kb, int m) {
  return 32 * (kb >> 1) + 8 * (m >> 2) + 4 * (kb & 1) + (m & 3);
}

__device__ inline uint32_t mask_pair(uint32_t x, int key0, int limit) {
  if (key0 >= limit) return 0u;
  if (key0 + 1 >= limit) return x & 0xFFFFu;
  return x;
}

__global__ __launch_bounds__(256, 2) void chunk_mfma_kernel(
    float* __restrict__ out, const _Float16* __restrict__ q,
    const _Float16* __restrict__ k_arena, const _Float16* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    float scale_log2, int Hkv, int n_qtiles, int num_blocks, int num_tokens) {
  const int qt = n_qtiles - 1 - (int)blockIdx.x;  // later (longer) row tiles first
  const int g = blockIdx.y, b = blockIdx.z;
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

  __shared__ u32x4 k_lds[kBN * 16];      // [key][16 B chunk ^ k_swz(key)]   16 KiB
  __shared__ u32x4 v_lds[4 * kD * 2];    // [block][dim][half ^ sw(dim)]      16 KiB

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
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int key = 16 * a + (tid >> 4), c = tid & 15;
      k_lds[key * 16 + (c ^ k_swz(key))] = kst[a];
      const int d = tid >> 1, hh = tid & 1;
      u32x4 x = vst[a];
      const int k0 = t * kBN + 16 * a + 8 * hh;  // absolute key of the first half
      if (k0 + 8 > Lc) {
        x.x = mask_pair(x.x, k0, Lc);
        x.y = mask_pair(x.y, k0 + 2, Lc);
        x.z = mask_pair(x.z, k0 + 4, Lc);
        x.w = mask_pair(x.w, k0 + 6, Lc);
      }
      v_lds[(a * kD + d) * 2 + (hh ^ ((d >> 3) & 1))] = x;
    }
  };

  f32x4 oacc[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) oacc[db][rb] = (f32x4)0.f;
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

  load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile(t);
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    // S^T[key][row] = K . Q^T
    f32x4 sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb][0] = (f32x4)0.f;
      sacc[kb][1] = (f32x4)0.f;
      const int key = key_of(kb, lr);
      const int sw = k_swz(key);
#pragma unroll
      for (int kd = 0; kd < 4; ++kd) {
        const half8_t ka = __builtin_bit_cast(half8_t, k_lds[key * 16 + ((4 * kd + lq) ^ sw)]);
        sacc[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[0][kd], sacc[kb][0], 0, 0, 0);
        sacc[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qf[1][kd], sacc[kb][1], 0, 0, 0);
      }
    }

    // online softmax per row (this lane: rows 16rb + lr, keys key_of(kb, 4lq + i))
    const bool need_mask = t * kBN + kBN - 1 > first_pos;
    half8_t pb[2][2];  // [u][rb]: B operand of the second product
    float alpha[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float s = sacc[kb][rb][i] * scale_log2;
          if (need_mask && t * kBN + key_of(kb, 4 * lq + i) > prow[rb]) s = -INFINITY;
          sacc[kb][rb][i] = s;
          mx = fmaxf(mx, s);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[rb], mx);  // finite: key 0 is in tile 0 for every row
      alpha[rb] = exp2f(m_run[rb] - m_new);
      m_run[rb] = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const _Float16 ph = (_Float16)exp2f(sacc[kb][rb][i] - m_new);
          lsum += (float)ph;
          pb[kb >> 1][rb][4 * (kb & 1) + i] = ph;
        }
      l_run[rb] = l_run[rb] * alpha[rb] + lsum;
    }
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) oacc[db][rb] *= alpha[rb];

    // O^T[dim][row] += V^T[dim][key] . P^T[key][row]
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int a = 2 * u + (lq >> 1), hh = lq & 1;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int d = 16 * db + lr;
        const half8_t va =
            __builtin_bit_cast(half8_t, v_lds[(a * kD + d) * 2 + (hh ^ ((d >> 3) & 1))]);
        oacc[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[u][0], oacc[db][0], 0, 0, 0);
        oacc[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[u][1], oacc[db][1], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float l = l_run[rb];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
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
  if (!chunk_fast_path(g))
    return launch_attend_generic(g, out, q, k_arena, v_arena, block_table, max_blocks, nullptr,
                                 cu_q_lens, chunk_start, num_seqs, num_tokens, scale, stream);
  const int n_qtiles = (max_q_len + kBM - 1) / kBM;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(chunk_mfma_kernel, dim3(n_qtiles, g.num_kv_heads, num_seqs), dim3(256), 0,
                     stream, out, (const _Float16*)q, (const _Float16*)k_arena,
                     (const _Float16*)v_arena, block_table, max_blocks, cu_q_lens, chunk_start,
                     scale_log2, g.num_kv_heads, n_qtiles, g.num_blocks, num_tokens);
  return hipGetLastError();
}

}  // namespace pkv
