// paged_attention_decode: one query token per sequence over its block-arena
// KV cache (Kshipra part 2, section 1: decode attends over the cache holding
// the new token too; part 3, section 4: online-softmax merge over KV blocks read
// in place through the block table, out = o / l).
//
// Tuned path (fp16 storage, head_dim 128, 4 query heads per KV head — the
// Llama-3-8B layer shape):
//   * split-KV: the keys of each sequence are cut into fixed 256-token splits
//     (16 arena blocks); one 64-lane wavefront per (sequence, KV head, split)
//     serves all 4 query heads of the group, so each K/V byte is read once;
//   * each 16-token block is one 4 KiB K tile and one 4 KiB V tile, fetched
//     with 16-byte fully coalesced loads into registers one block ahead, then
//     staged in LDS (XOR-swizzled: conflict-free 16-byte reads);
//   * QK: lane (h, j) = (query head, token) dots q_h with k_j using packed
//     fp16 dot products accumulating in fp32; the per-head block max is a
//     16-lane reduction; p = 2^(s - m) in fp32 (scores carry log2(e));
//   * PV: lane (h, c) accumulates 8 head dims (c, c+16, ...) over the block's
//     16 tokens with mixed fp16 x fp32 fused multiply-adds, rescaled by
//     2^(m_old - m_new) when the running max moves;
//   * a split writes its unnormalised (o, m, l); a second kernel merges the
//     splits of each (sequence, head) by their log-sum-exp.  A sequence that
//     fits one split is normalised and written by the split kernel directly.
// Other shapes run the generic kernel.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kG = 4;

__device__ inline half2_t as_h2(uint32_t x) { return __builtin_bit_cast(half2_t, x); }

__device__ inline float lo_f(uint32_t x) { return (float)__builtin_bit_cast(half2_t, x).x; }
__device__ inline float hi_f(uint32_t x) { return (float)__builtin_bit_cast(half2_t, x).y; }

__device__ inline uint32_t mask_pair(uint32_t x, int key0, int valid) {
  // zero the fp16 halves whose key index (key0, key0 + 1) is >= valid
  if (key0 >= valid) return 0u;
  if (key0 + 1 >= valid) return x & 0xFFFFu;
  return x;
}

// One block's K tile and V tile of one KV head: 4 x 16 B per lane, each
// 64-lane load covering 1 KiB contiguously.
struct Tile {
  u32x4 k[4], v[4];
};

__device__ inline Tile load_tile(const _Float16* __restrict__ k_arena,
                                 const _Float16* __restrict__ v_arena, int blk, int num_blocks,
                                 int Hkv, int g, int lane) {
  if (blk < 0 || blk >= num_blocks) blk = 0;
  const size_t tile = ((size_t)blk * Hkv + g) * (kBlock * kD / 8);  // in u32x4
  const u32x4* kb = (const u32x4*)k_arena + tile;
  const u32x4* vb = (const u32x4*)v_arena + tile;
  Tile t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.k[i] = kb[i * 64 + lane];
    t.v[i] = vb[i * 64 + lane];
  }
  return t;
}

__global__ __launch_bounds__(64) void decode_split_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const _Float16* __restrict__ k_arena,
    const _Float16* __restrict__ v_arena, const int32_t* __restrict__ block_table,
    int max_blocks, const int32_t* __restrict__ context_lens, float scale_log2, int Hkv,
    int nsplit_max, int num_blocks) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int Hq = Hkv * kG;
  const int h = lane >> 4;  // query head within the group
  const int j = lane & 15;  // token (QK) / head-dim lane (PV)
  // clamp to what the grid and workspace cover (a caller contract violation
  // then gives unspecified values, never an out-of-bounds access)
  const int L = min(min(context_lens[b], max_blocks * kBlock), nsplit_max * kDecodeSplit);
  const int tok0 = split * kDecodeSplit;
  if (L <= 0) {
    if (split == 0) {
      float* o = out + ((size_t)b * Hq + g * kG + h) * kD;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) o[j + 16 * dd] = 0.f;
    }
    return;
  }
  if (tok0 >= L) return;
  const int tok1 = min(L, tok0 + kDecodeSplit);
  const int nblk = (tok1 - tok0 + kBlock - 1) / kBlock;
  const int nsplit = (L + kDecodeSplit - 1) / kDecodeSplit;

  // q of head g*4+h, all 128 dims, as 64 packed fp16 pairs
  uint32_t qv[64];
  {
    const u32x4* qp = (const u32x4*)(q + ((size_t)b * Hq + g * kG + h) * kD);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const u32x4 x = qp[c];
      qv[4 * c] = x.x; qv[4 * c + 1] = x.y; qv[4 * c + 2] = x.z; qv[4 * c + 3] = x.w;
    }
  }

  __shared__ u32x4 k_lds[16 * 16];   // [token][16 B chunk ^ token]
  __shared__ u32x4 v_lds[kD * 2];    // [dim][8-key half ^ ((dim >> 3) & 1)]
  __shared__ float p_lds[64];        // [head][token]

  const int32_t* bt = block_table + (size_t)b * max_blocks + (tok0 >> 4);
  float m_run = -INFINITY, l_run = 0.f;
  float o[8];
#pragma unroll
  for (int dd = 0; dd < 8; ++dd) o[dd] = 0.f;
  const int vsw = (j >> 3) & 1;

  Tile nxt = load_tile(k_arena, v_arena, bt[0], num_blocks, Hkv, g, lane);
  for (int n = 0; n < nblk; ++n) {
    const Tile cur = nxt;
    const int valid = min(kBlock, tok1 - (tok0 + n * kBlock));
    __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 4 + (lane >> 4), c = lane & 15;
      k_lds[row * 16 + (c ^ row)] = cur.k[i];
      const int d = i * 32 + (lane >> 1), hh = lane & 1;
      u32x4 x = cur.v[i];
      if (valid < kBlock) {  // keys past the context: zero V (their p is 0, 0*NaN is not)
        const int k0 = hh * 8;
        x.x = mask_pair(x.x, k0, valid);
        x.y = mask_pair(x.y, k0 + 2, valid);
        x.z = mask_pair(x.z, k0 + 4, valid);
        x.w = mask_pair(x.w, k0 + 6, valid);
      }
      v_lds[d * 2 + (hh ^ ((d >> 3) & 1))] = x;
    }
    __syncthreads();
    if (n + 1 < nblk) nxt = load_tile(k_arena, v_arena, bt[n + 1], num_blocks, Hkv, g, lane);

    // scores of the block: lane (h, j)
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const u32x4 kk = k_lds[j * 16 + (c ^ j)];
      a0 = __builtin_amdgcn_fdot2(as_h2(qv[4 * c]), as_h2(kk.x), a0, false);
      a1 = __builtin_amdgcn_fdot2(as_h2(qv[4 * c + 1]), as_h2(kk.y), a1, false);
      a0 = __builtin_amdgcn_fdot2(as_h2(qv[4 * c + 2]), as_h2(kk.z), a0, false);
      a1 = __builtin_amdgcn_fdot2(as_h2(qv[4 * c + 3]), as_h2(kk.w), a1, false);
    }
    const float s = j < valid ? (a0 + a1) * scale_log2 : -INFINITY;
    float mb = s;
    mb = fmaxf(mb, __shfl_xor(mb, 1, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 2, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 4, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 8, 16));
    const float m_new = fmaxf(m_run, mb);  // finite: every block has a valid token
    const float alpha = exp2f(m_run - m_new);
    const float p = exp2f(s - m_new);
    l_run = l_run * alpha + p;
    m_run = m_new;
    p_lds[lane] = p;
    __syncthreads();

    float pj[16];
    {
      const f32x4* pp = (const f32x4*)(p_lds + h * 16);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 x = pp[c];
        pj[4 * c] = x.x; pj[4 * c + 1] = x.y; pj[4 * c + 2] = x.z; pj[4 * c + 3] = x.w;
      }
    }
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int d = j + 16 * dd;
      const u32x4 v0 = v_lds[d * 2 + vsw];        // keys 0..7
      const u32x4 v1 = v_lds[d * 2 + (vsw ^ 1)];  // keys 8..15
      float acc = o[dd] * alpha;
      acc = __builtin_fmaf(pj[0], lo_f(v0.x), acc);
      acc = __builtin_fmaf(pj[1], hi_f(v0.x), acc);
      acc = __builtin_fmaf(pj[2], lo_f(v0.y), acc);
      acc = __builtin_fmaf(pj[3], hi_f(v0.y), acc);
      acc = __builtin_fmaf(pj[4], lo_f(v0.z), acc);
      acc = __builtin_fmaf(pj[5], hi_f(v0.z), acc);
      acc = __builtin_fmaf(pj[6], lo_f(v0.w), acc);
      acc = __builtin_fmaf(pj[7], hi_f(v0.w), acc);
      acc = __builtin_fmaf(pj[8], lo_f(v1.x), acc);
      acc = __builtin_fmaf(pj[9], hi_f(v1.x), acc);
      acc = __builtin_fmaf(pj[10], lo_f(v1.y), acc);
      acc = __builtin_fmaf(pj[11], hi_f(v1.y), acc);
      acc = __builtin_fmaf(pj[12], lo_f(v1.z), acc);
      acc = __builtin_fmaf(pj[13], hi_f(v1.z), acc);
      acc = __builtin_fmaf(pj[14], lo_f(v1.w), acc);
      acc = __builtin_fmaf(pj[15], hi_f(v1.w), acc);
      o[dd] = acc;
    }
  }

  float l_row = l_run;
  l_row += __shfl_xor(l_row, 1, 16);
  l_row += __shfl_xor(l_row, 2, 16);
  l_row += __shfl_xor(l_row, 4, 16);
  l_row += __shfl_xor(l_row, 8, 16);
  const int hq = g * kG + h;
  if (nsplit == 1) {
    const float inv = 1.f / l_row;
    float* dst = out + ((size_t)b * Hq + hq) * kD;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) dst[j + 16 * dd] = o[dd] * inv;
  } else {
    const size_t part = ((size_t)b * Hq + hq) * nsplit_max + split;
    float* dst = ws_o + part * kD;
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) dst[j + 16 * dd] = o[dd];
    if (j == 0) {
      ws_ml[2 * part] = m_run;
      ws_ml[2 * part + 1] = l_row;
    }
  }
}

// Merge the splits of one (sequence, query head): weights 2^(m_s - M).
__global__ __launch_bounds__(128) void decode_combine_kernel(
    float* __restrict__ out, const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ context_lens, int max_blocks, int Hq, int nsplit_max) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = min(min(context_lens[b], max_blocks * kBlock), nsplit_max * kDecodeSplit);
  const int nsplit = (L + kDecodeSplit - 1) / kDecodeSplit;
  if (nsplit <= 1) return;
  const size_t part0 = ((size_t)b * Hq + h) * nsplit_max;
  const float* ml = ws_ml + 2 * part0;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  float den = 0.f, acc = 0.f;
  const float* po = ws_o + part0 * kD + threadIdx.x;
  for (int s = 0; s < nsplit; ++s) {
    const float w = exp2f(ml[2 * s] - M);
    den += w * ml[2 * s + 1];
    acc += w * po[(size_t)s * kD];
  }
  out[((size_t)b * Hq + h) * kD + threadIdx.x] = acc / den;
}

}  // namespace

bool decode_fast_path(const pkv_geom& g) {
  return g.dtype == PKV_F16 && g.head_dim == kD && g.num_q_heads == kG * g.num_kv_heads;
}

size_t decode_workspace_bytes(const pkv_geom& g, int num_seqs, int max_context_len) {
  if (!decode_fast_path(g)) return 0;
  const size_t nsplit = (size_t)(max_context_len + kDecodeSplit - 1) / kDecodeSplit;
  if (nsplit <= 1) return 0;
  return (size_t)num_seqs * g.num_q_heads * nsplit * (kD + 2) * sizeof(float);
}

hipError_t launch_decode(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                         const void* v_arena, const int32_t* block_table, int max_blocks,
                         const int32_t* context_lens, int num_seqs, int max_context_len,
                         float scale, void* workspace, hipStream_t stream) {
  if (!decode_fast_path(g))
    return launch_attend_generic(g, out, q, k_arena, v_arena, block_table, max_blocks,
                                 context_lens, nullptr, nullptr, num_seqs, num_seqs, scale,
                                 stream);
  const int nsplit = (max_context_len + kDecodeSplit - 1) / kDecodeSplit;
  float* ws_o = (float*)workspace;
  float* ws_ml = ws_o ? ws_o + (size_t)num_seqs * g.num_q_heads * nsplit * kD : nullptr;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(decode_split_kernel, dim3(nsplit, g.num_kv_heads, num_seqs), dim3(64), 0,
                     stream, out, ws_o, ws_ml, (const _Float16*)q, (const _Float16*)k_arena,
                     (const _Float16*)v_arena, block_table, max_blocks, context_lens,
                     scale_log2, g.num_kv_heads, nsplit, g.num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit <= 1) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(g.num_q_heads, num_seqs), dim3(kD), 0, stream,
                     out, ws_o, ws_ml, context_lens, max_blocks, g.num_q_heads, nsplit);
  return hipGetLastError();
}

}  // namespace pkv
