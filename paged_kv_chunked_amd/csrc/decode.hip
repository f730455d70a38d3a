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
//   * per pair of blocks (32 tokens) the two small contractions, S = q . K^T
//     ([4 heads x 128] . [128 x 32]) and o += P . V, run on the fp16 matrix
//     cores (v_mfma_f32_16x16x32_f16, fp32 accumulation).  This is not to
//     reach matrix-core throughput (4 of the 16 MFMA columns carry heads): it
//     takes the multiply-adds, fp16 conversions and cross-lane traffic off the
//     vector ALUs and LDS, which otherwise sit at ~50% busy at full HBM rate;
//   * K and V tiles go from HBM straight into operand registers: each lane
//     issues 16-byte loads (64 B contiguous per token row for K; 512 B
//     contiguous per block for the head-dim-major V tile), the next pair is in
//     flight while the current one is computed, and the split's block-table
//     entries are fetched once into a register up front;
//   * online softmax in fp32 on scores in log2 units; accumulators are
//     rescaled only when some head's running max moved; P is rounded to fp16
//     for the second product and the denominator sums those rounded values;
//   * a split writes its unnormalised (o, m, l); a second kernel merges the
//     splits of each (sequence, head) by their log-sum-exp.  A sequence that
//     fits one split is normalised and written by the split kernel directly.
// Other shapes run the generic kernel.
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kG = 4;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// Blocks per split: kDecodeSplit tokens.
constexpr int kSB = kDecodeSplit / kBlock;
static_assert(kSB % 2 == 0, "splits are walked in pairs of blocks");

// The K and V tiles of a pair of arena blocks (32 tokens), already in the MFMA
// operand layouts (see decode_split_kernel).
struct Pair {
  half8_t k[2][4];  // [u][kd]: A operand of S^T = K . Q^T
  half8_t v[8];     // [db]:    A operand of O^T += V^T . P^T
};

__device__ inline Pair load_pair(const _Float16* __restrict__ k_arena,
                                 const _Float16* __restrict__ v_arena, int blk_a, int blk_b,
                                 int Hkv, int g, int ln, int lq) {
  Pair pr;
  const size_t tile_elems = (size_t)kBlock * kD;
  // K: this lane is MFMA row ln -> block ln/8, token 8*((ln>>2)&1) + 4u + (ln&3);
  // it supplies head dims 32kd + 8lq .. +8 of that token.
  {
    const int blk = (ln >> 3) ? blk_b : blk_a;
    const _Float16* kt = k_arena + ((size_t)blk * Hkv + g) * tile_elems;
    const int tok = 8 * ((ln >> 2) & 1) + (ln & 3);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kd = 0; kd < 4; ++kd)
        pr.k[u][kd] = *(const half8_t*)(kt + (tok + 4 * u) * kD + 32 * kd + 8 * lq);
  }
  // V^T: this lane is MFMA row ln -> head dim 16db + ln; it supplies the 8
  // tokens 8*(lq&1) .. +8 of block lq/2 (16 contiguous bytes of the V tile).
  {
    const int blk = (lq >> 1) ? blk_b : blk_a;
    const _Float16* vt = v_arena + ((size_t)blk * Hkv + g) * tile_elems;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      pr.v[db] = *(const half8_t*)(vt + (16 * db + ln) * kBlock + 8 * (lq & 1));
  }
  return pr;
}

// One 64-lane wavefront per (sequence b, KV head g, split of kSB blocks).
// Per pair of blocks (32 tokens):
//   S^T[token][head] = K . Q^T on 2 x 4 MFMAs 16x16x32 (only columns 0..3 are
//     real heads; the query group is 4), keys permuted so that afterwards
//     lane (ln, lq) holds 8 consecutive tokens 8*(lq&1).. of block lq/2 for
//     head ln;
//   online softmax on those values (row max: 2 cross-lane steps);
//   O^T[dim][head] += V^T . P^T on 8 MFMAs, P rounded to fp16 and the
//     denominator summed from the rounded values.
// K/V go from HBM straight into operand registers; the next pair is loaded
// while the current one is computed.
__global__ __launch_bounds__(64) void decode_split_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const _Float16* __restrict__ k_arena,
    const _Float16* __restrict__ v_arena, const int32_t* __restrict__ block_table,
    int max_blocks, const int32_t* __restrict__ context_lens, float scale_log2, int Hkv,
    int nsplit_max, int num_blocks) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int ln = lane & 15, lq = lane >> 4;
  const int Hq = Hkv * kG;
  // clamp to what the grid and workspace cover (a caller contract violation
  // then gives unspecified values, never an out-of-bounds access)
  const int L = min(min(context_lens[b], max_blocks * kBlock), nsplit_max * kDecodeSplit);
  if (L <= 0) {
    if (split == 0 && ln < kG) {
      float* o = out + ((size_t)b * Hq + g * kG + ln) * kD + 4 * lq;
#pragma unroll
      for (int db = 0; db < 8; ++db) *(f32x4*)(o + 16 * db) = (f32x4)0.f;
    }
    return;
  }
  const int nb_seq = (L + kBlock - 1) / kBlock;
  const int blk0 = split * kSB;
  if (blk0 >= nb_seq) return;
  const int nb = min(kSB, nb_seq - blk0);
  const int nsplit = (nb_seq + kSB - 1) / kSB;
  const int npairs = (nb + 1) >> 1;

  // physical ids of this split's blocks: lane i holds entry i
  int my_blk = 0;
  if (lane < nb) {
    my_blk = block_table[(size_t)b * max_blocks + blk0 + lane];
    if (my_blk < 0 || my_blk >= num_blocks) my_blk = 0;
  }
  // Q^T (B operand): column ln = head g*4+ln, dims 32kd + 8lq .. +8
  half8_t qb[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd)
    qb[kd] = ln < kG ? *(const half8_t*)(q + ((size_t)b * Hq + g * kG + ln) * kD + 32 * kd + 8 * lq)
                     : (half8_t)(_Float16)0.f;

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
    // absolute token of element e = 4u + i of this lane
    const int tok0 = (blk0 + 2 * p + (lq >> 1)) * kBlock + 8 * (lq & 1);
    const int nvalid = L - tok0;  // elements e < nvalid are real keys
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = s[e >> 2][e & 3] * scale_log2;
      if (e >= nvalid) x = -INFINITY;
      sv[e] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);  // finite: the first key of a split is real
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
      const _Float16 ph = (_Float16)__builtin_amdgcn_exp2f(sv[e] - m_new);
      pb[e] = ph;
      lsum += (float)ph;
    }
    l_run += lsum;
    const bool tail = nvalid < 8;  // keys past the context: zero V (0 * NaN is NaN)
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      half8_t va = pr.v[db];
      if (tail) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= nvalid) va[e] = (_Float16)0.f;
      }
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o[db], 0, 0, 0);
    }
  };

  int ba, bb;
  pair_ids(0, ba, bb);
  Pair cur = load_pair(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
  for (int p = 0; p < npairs; p += 2) {
    Pair nxt;
    if (p + 1 < npairs) {
      pair_ids(p + 1, ba, bb);
      nxt = load_pair(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
    }
    compute(cur, p);
    if (p + 1 >= npairs) break;
    if (p + 2 < npairs) {
      pair_ids(p + 2, ba, bb);
      cur = load_pair(k_arena, v_arena, ba, bb, Hkv, g, ln, lq);
    }
    compute(nxt, p + 1);
  }

  float l_row = l_run;
  l_row += __shfl_xor(l_row, 16);
  l_row += __shfl_xor(l_row, 32);
  if (ln >= kG) return;
  const int hq = g * kG + ln;
  if (nsplit == 1) {
    const float inv = 1.f / l_row;
    float* dst = out + ((size_t)b * Hq + hq) * kD + 4 * lq;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(f32x4*)(dst + 16 * db) = o[db] * inv;
  } else {
    const size_t part = ((size_t)b * Hq + hq) * nsplit_max + split;
    float* dst = ws_o + part * kD + 4 * lq;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(f32x4*)(dst + 16 * db) = o[db];
    if (lq == 0) {
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
