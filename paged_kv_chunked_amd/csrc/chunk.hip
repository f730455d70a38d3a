// paged_attention_chunk: chunked prefill over the block arena (Kshipra part 3,
// section 4 "Chunked Prefill": an online softmax across KV blocks read in place,
// RoPE already applied at absolute positions P onward, a causal mask over the
// chunk so that row i sees the cached prefix and the chunk up to itself).
//
// Tuned path (fp16, INT8 or INT4 storage, head_dim 128, 4 query heads per KV
// head): a dense contraction, so both products run on gfx950 fp16 matrix cores
// (v_mfma_f32_16x16x32_f16, fp32 accumulation).  Quantized tiles are staged
// as codes and dequantized to fp16 in LDS once per workgroup (chunk_core.h).
//   * one workgroup = (sequence, KV head, tile of 64 chunk rows), 8 waves: wave
//     w serves query head 4g + (w & 3) for rows 32 (w >> 2) .. +31 of the tile,
//     so every K/V tile is fetched once for 4 heads x 64 rows;
//   * keys are walked in tiles of 64 = 4 arena blocks looked up in the block
//     table.  Tiles travel from memory straight into a 4-stage LDS ring
//     (direct-to-LDS 16-byte loads, up to three tiles in flight) in the
//     arena's own layouts: K [block][16-byte dim piece][key] and V
//     [block][dim][two 8-key halves], with 16-byte units permuted on the way
//     in so the operand reads below are bank-conflict free;
//   * S^T = K Q^T puts keys on the MFMA M dimension, so each lane ends up
//     holding 16 keys of one query row: the row max and sum are lane-local
//     plus two cross-lane steps.  The keys are assigned to MFMA rows so that
//     a lane's 8 probabilities for the second product are 8 consecutive keys
//     of one block: the B operand of O^T += V^T P^T is then built in
//     registers, and the matching V^T operand is one 16-byte piece of the
//     arena's V row;
//   * online softmax in fp32 (scores in log2 units), P rounded to fp16 for the
//     second product, and the denominator summed from those rounded values so
//     the weights still add up to one; a row's running maximum is only moved
//     when one of its scores exceeds it by a margin (quotient unchanged, see
//     kSlack);
//   * the causal mask is applied only on tiles that reach past a wave's first
//     row position; V slots past the sequence's length are zeroed in LDS in
//     the last tile (p = 0 there, but 0 * NaN would not be 0).
// Work items are dispatched longest first (chunk_order_kernel).  Other shapes
// run the generic kernel.
#include <algorithm>
#include <cmath>

#include "chunk_core.h"

namespace pkv {
namespace {

constexpr int kOrderBuckets = 4096;  // costs at or above the last bucket share it
constexpr int kRankSortMax = 256;    // item counts ranked directly instead
// Key-range parts: a call with fewer than kChunkTargetUnits (row tile, KV
// head) units (two per compute unit of the chip) splits each item's keys into
// up to kChunkMaxParts parts of at least kChunkMinPartTiles key tiles (of the
// longest context), merged by chunk_combine_kernel.  Measured on one GPU's
// share of a head-split layer (64 units, contexts up to 3632): 7 parts
// 58.8-59.5 us, 4 parts 52.9-53.1 us, 3 parts 56.8-57.2 us, 2 parts
// 68.6-69.4 us; on the mixed step's chunk call (128 units) 4 parts 75-77 us
// against 104-107 us for 2 or 8.
#ifndef PKV_CHUNK_TARGET_UNITS
#define PKV_CHUNK_TARGET_UNITS 512
#endif
constexpr long kChunkTargetUnits = PKV_CHUNK_TARGET_UNITS;
constexpr int kChunkMaxParts = 8;
#ifndef PKV_CHUNK_MIN_PART_TILES
#define PKV_CHUNK_MIN_PART_TILES 12
#endif
constexpr int kChunkMinPartTiles = PKV_CHUNK_MIN_PART_TILES;

// Schedule of the attention kernel: the (sequence, row tile) items sorted by
// decreasing work (counting sort on the tile count, or for at most
// kRankSortMax items a direct ranking; equal costs in any order),
// so the longest items are dispatched first and the short ones fill the gaps
// at the end.  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void chunk_order_kernel(
    int32_t* __restrict__ order, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ chunk_start, int num_seqs, int n_rtiles, int max_blocks,
    int num_tokens) {
  __shared__ int hist[kOrderBuckets];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int n = num_seqs * n_rtiles;
  if (n <= kRankSortMax) {
    // few items: each thread ranks its own item against all of them (rank =
    // items of higher cost, ties broken by index), one LDS pass
    const int c = tid < n ? chunk_item_cost(cu_q_lens, chunk_start, tid / n_rtiles,
                                            tid - tid / n_rtiles * n_rtiles, max_blocks, num_tokens)
                          : 0;
    part[tid] = c;
    __syncthreads();
    if (tid < n) {
      int rank = 0;
      for (int j = 0; j < n; ++j) {
        const int cj = part[j];
        rank += cj > c || (cj == c && j < tid);
      }
      order[rank] = tid;
    }
    return;
  }
  for (int c = tid; c < kOrderBuckets; c += 1024) hist[c] = 0;
  __syncthreads();
  for (int k = tid; k < n; k += 1024) {
    const int b = k / n_rtiles, rt = k - b * n_rtiles;
    const int c = min(chunk_item_cost(cu_q_lens, chunk_start, b, rt, max_blocks, num_tokens),
                      kOrderBuckets - 1);
    atomicAdd(&hist[c], 1);
  }
  __syncthreads();
  // exclusive scan in decreasing cost order: thread t owns the 4 buckets
  // kOrderBuckets - 1 - 4t - {0..3}
  int own[4], sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    own[u] = hist[kOrderBuckets - 1 - 4 * tid - u];
    sum += own[u];
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int x = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += x;
    __syncthreads();
  }
  int start = part[tid] - sum;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    hist[kOrderBuckets - 1 - 4 * tid - u] = start;
    start += own[u];
  }
  __syncthreads();
  for (int k = tid; k < n; k += 1024) {
    const int b = k / n_rtiles, rt = k - b * n_rtiles;
    const int c = min(chunk_item_cost(cu_q_lens, chunk_start, b, rt, max_blocks, num_tokens),
                      kOrderBuckets - 1);
    order[atomicAdd(&hist[c], 1)] = k;
  }
}

template <int kQ>
__global__ __launch_bounds__(kThreads, 1) void chunk_mfma_kernel(
    float* __restrict__ out, const _Float16* __restrict__ q,
    const void* __restrict__ k_arena, const void* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    const int32_t* __restrict__ order, float scale_log2, int Hkv, int num_seqs, int n_rtiles,
    int num_blocks, int num_tokens, int parts, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  // Workgroup i takes part (i / Hkv) % parts of item order[i / (Hkv * parts)]
  // for KV head i % Hkv.  Linear workgroup ids are dealt to the 8 XCDs
  // round-robin, so with Hkv a multiple of 8 every row tile (and part) of a
  // (sequence, KV head) pair runs on one XCD and the pair's K/V tiles are
  // fetched into that XCD's L2 once; the longest items are issued first.
  const int i = blockIdx.x;
  const int k = i / (Hkv * parts), rem = i - k * (Hkv * parts);
  const int part = rem / Hkv, g = rem - part * Hkv;
  if (k >= num_seqs * n_rtiles) return;
  // (a schedule left by another batch description may hold any value: an
  // entry outside the item range is skipped, never followed)
  const int item = order[k];
  if ((unsigned)item >= (unsigned)(num_seqs * n_rtiles)) return;
  const int b = item / n_rtiles, rt = item - b * n_rtiles;
  __shared__ u32x4 lds[ChunkLds<kQ>::kUnits];
  chunk_tile_unit<kQ>(lds, out, q, k_arena, v_arena, block_table, max_blocks, cu_q_lens, chunk_start,
                      scale_log2, Hkv, num_blocks, num_tokens, b, rt, g, part, parts, part_o,
                      part_ml);
}

// Merge of the key-range parts of every chunk row (only when the call is split):
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p, M = max_p m_p.  One wave
// per (row, query head), each lane 2 head dims.  Rows the attention kernel
// skips (a sequence with no keys) are skipped here too.
__global__ __launch_bounds__(256) void chunk_combine_kernel(
    float* __restrict__ out, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    int num_seqs, int num_tokens, int max_blocks, int Hq, int parts) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int b = find_seq(cu_q_lens, num_seqs, t);
  const int C = min(cu_q_lens[b + 1], num_tokens) - cu_q_lens[b];
  const int Lc = min(chunk_start[b] + C, max_blocks * kBlock);
  if (h >= Hq || Lc <= 0) return;
  float2 ml[kChunkMaxParts], o[kChunkMaxParts];
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < kChunkMaxParts; ++p) {
    if (p < parts) {
      const size_t pr = ((size_t)p * num_tokens + t) * Hq + h;
      ml[p] = *(const float2*)(part_ml + 2 * pr);
      o[p] = *(const float2*)(part_o + pr * kD + 2 * lane);
      M = fmaxf(M, ml[p].x);
    }
  }
  float den = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int p = 0; p < kChunkMaxParts; ++p) {
    if (p < parts && ml[p].x != -INFINITY) {  // a part that saw no key of this row
      const float w = exp2f(ml[p].x - M);
      den += w * ml[p].y;
      a0 += w * o[p].x;
      a1 += w * o[p].y;
    }
  }
  const float inv = 1.f / den;
  *(float2*)(out + ((size_t)t * Hq + h) * kD + 2 * lane) = make_float2(a0 * inv, a1 * inv);
}

}  // namespace

bool chunk_fast_path(const pkv_geom& g) {
  return (g.dtype == PKV_F16 || g.dtype == PKV_I8KV || g.dtype == PKV_I4KV) &&
         g.head_dim == kD && g.num_q_heads == kG * g.num_kv_heads;
}

int chunk_parts(const pkv_geom& g, int num_tokens, int max_context_len) {
  if (!chunk_fast_path(g) || num_tokens <= 0) return 1;
  // fewest (row tile, KV head) units the call can have: its rows packed in
  // whole 64-row tiles
  const long units = (long)((num_tokens + kRows - 1) / kRows) * g.num_kv_heads;
  if (units >= kChunkTargetUnits) return 1;
  long parts = (kChunkTargetUnits + units - 1) / units;
  parts = std::min(parts, (long)kChunkMaxParts);
  parts = std::min(parts, (long)(max_context_len / (kChunkMinPartTiles * kBN)));
  return (int)std::max(parts, 1L);
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t chunk_workspace_bytes(const pkv_geom& g, int num_seqs, int num_tokens,
                             int max_context_len) {
  if (!chunk_fast_path(g) || num_seqs <= 0 || num_tokens <= 0) return 0;
  // the schedule: one int32 per (sequence, row tile)
  const size_t sched = (size_t)num_seqs * (size_t)((num_tokens + kRows - 1) / kRows) * sizeof(int32_t);
  const int parts = chunk_parts(g, num_tokens, max_context_len);
  if (parts == 1) return sched;
  // the parts' partials: o [parts][num_tokens][Hq][D] and (m, l) [parts][num_tokens][Hq][2]
  const size_t rows = (size_t)parts * num_tokens * g.num_q_heads;
  return align256(sched) + align256(rows * kD * sizeof(float)) + rows * 2 * sizeof(float);
}

// The tuned kernel's schedule for one batch description: the longest-first
// order of the (sequence, 64-row tile) items, one int32 each at the head of the
// workspace.  It depends only on cu_q_lens, chunk_start, num_seqs, num_tokens,
// max_q_len and max_blocks, so a step computes it once for all its layers.
hipError_t launch_chunk_plan(const pkv_geom& g, const int32_t* cu_q_lens,
                             const int32_t* chunk_start, int max_blocks, int num_seqs,
                             int num_tokens, int max_q_len, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!chunk_fast_path(g)) return hipSuccess;  // the generic kernel needs no schedule
  // no sequence has more rows than the batch
  const int n_rtiles = (min(max_q_len, num_tokens) + kRows - 1) / kRows;
  const long n_items = (long)num_seqs * n_rtiles;
  if (!workspace || workspace_bytes < (size_t)n_items * sizeof(int32_t))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(chunk_order_kernel, dim3(1), dim3(1024), 0, stream, (int32_t*)workspace,
                     cu_q_lens, chunk_start, num_seqs, n_rtiles, max_blocks, num_tokens);
  return hipGetLastError();
}

static bool chunk_tuned(const pkv_geom& g, float scale) {
  // the fast path tracks maxima of raw scores, which needs scale > 0
  return chunk_fast_path(g) && scale > 0.f && std::isfinite(scale);
}

// The attention (and, for a split call, the merge of its parts) over the
// schedule that launch_chunk_plan left in the workspace.
hipError_t launch_chunk_run(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                            const void* v_arena, const int32_t* block_table, int max_blocks,
                            const int32_t* cu_q_lens, const int32_t* chunk_start, int num_seqs,
                            int num_tokens, int max_q_len, int max_context_len, float scale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!chunk_tuned(g, scale))
    return launch_attend_generic(g, out, q, k_arena, v_arena, block_table, max_blocks, nullptr,
                                 cu_q_lens, chunk_start, num_seqs, num_tokens, scale, stream);
  const int n_rtiles = (min(max_q_len, num_tokens) + kRows - 1) / kRows;
  const long n_items = (long)num_seqs * n_rtiles;
  if (!workspace || workspace_bytes < (size_t)n_items * sizeof(int32_t))
    return hipErrorInvalidValue;
  const int32_t* order = (const int32_t*)workspace;
  const float scale_log2 = scale * 1.4426950408889634f;
  const int parts = chunk_parts(g, num_tokens, max_context_len);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (parts > 1) {
    const size_t rows = (size_t)parts * num_tokens * g.num_q_heads;
    const size_t sched = align256((size_t)n_items * sizeof(int32_t));
    if (workspace_bytes < sched + align256(rows * kD * sizeof(float)) + rows * 2 * sizeof(float))
      return hipErrorInvalidValue;
    part_o = (float*)((char*)workspace + sched);
    part_ml = part_o + align256(rows * kD * sizeof(float)) / sizeof(float);
  }
  const long nwg = n_items * g.num_kv_heads * parts;
  if (nwg > 0x7fffffffL) return hipErrorInvalidValue;
  auto kernel = g.dtype == PKV_I8KV ? chunk_mfma_kernel<1>
                : g.dtype == PKV_I4KV ? chunk_mfma_kernel<2> : chunk_mfma_kernel<0>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)nwg), dim3(kThreads), 0, stream, out,
                     (const _Float16*)q, k_arena, v_arena, block_table, max_blocks, cu_q_lens,
                     chunk_start, order, scale_log2, g.num_kv_heads, num_seqs, n_rtiles,
                     g.num_blocks, num_tokens, parts, part_o, part_ml);
  if (parts == 1) return hipGetLastError();
  hipLaunchKernelGGL(chunk_combine_kernel, dim3((unsigned)num_tokens, (g.num_q_heads + 3) / 4),
                     dim3(256), 0, stream, out, part_o, part_ml, cu_q_lens, chunk_start,
                     num_seqs, num_tokens, max_blocks, g.num_q_heads, parts);
  return hipGetLastError();
}

hipError_t launch_chunk(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                        const void* v_arena, const int32_t* block_table, int max_blocks,
                        const int32_t* cu_q_lens, const int32_t* chunk_start, int num_seqs,
                        int num_tokens, int max_q_len, int max_context_len, float scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (chunk_tuned(g, scale)) {
    const hipError_t e = launch_chunk_plan(g, cu_q_lens, chunk_start, max_blocks, num_seqs,
                                           num_tokens, max_q_len, workspace, workspace_bytes,
                                           stream);
    if (e != hipSuccess) return e;
  }
  return launch_chunk_run(g, out, q, k_arena, v_arena, block_table, max_blocks, cu_q_lens,
                          chunk_start, num_seqs, num_tokens, max_q_len, max_context_len, scale,
                          workspace, workspace_bytes, stream);
}

}  // namespace pkv
