// paged_attention_mixed: one continuous-batching step in one attention launch
// (Kshipra part 3, section 5 "Continuous Batching and Admission Control": each
// step mixes prefill chunks and decode tokens under a token budget).
//
// The batch is the varlen description of paged_attention_chunk.  A sequence
// with one new row is a decode: its keys are cut into the 384-token splits of
// paged_attention_decode and each (split, KV-head group) is one work unit.  A
// sequence with two or more rows is a prefill chunk: each (64-row tile, KV
// head) is one work unit of the chunk kernel.  Both kinds of unit run in one
// persistent launch, so the matrix-core-bound chunk tiles and the HBM-bound
// decode splits share the chip instead of running one after the other (the
// chunk kernel alone fills only a few hundred workgroups for a 1024-token
// budget, leaving most CUs idle for its duration).
//   * mixed_order_kernel (one workgroup) lists the units longest first: chunk
//     tiles by their number of 64-key tiles, then decode splits by their number
//     of blocks (counting sorts), and resets the queue counter;
//   * mixed_kernel: 256 workgroups (one per CU: each holds the chunk unit's
//     128 KiB LDS ring) take units from that list through an atomic counter
//     until it runs past the last unit; every workgroup reaches that exit.
//     A unit runs exactly the code of the stand-alone kernels (chunk_core.h,
//     decode_core.h), so its results are bit for bit theirs;
//   * decode_combine_kernel then merges the splits of the decode rows.
#include <type_traits>

#include "chunk_core.h"
#include "decode_core.h"
#include "decode_q_core.h"

namespace pkv {
namespace {

static_assert(kThreads == 64 * kDecodeWavesPerWG, "one workgroup shape for both unit kinds");

constexpr int kChunkBuckets = 4096;  // chunk costs at or above the last bucket share it
constexpr int kDecBuckets = kSB + 1;  // blocks in a split: 0 .. kSB
// Schedule header in the workspace (int32): unit counts and the queue counter.
constexpr int kHdrChunk = 0, kHdrDec = 1, kHdrNext = 2, kHdrInts = 4;

// Rows of sequence b in the packed batch (clamped to the batch).
__device__ inline int rows_of(const int32_t* __restrict__ cu_q_lens, int b, int num_tokens) {
  return min(cu_q_lens[b + 1], num_tokens) - cu_q_lens[b];
}

// Work lists: chunk items (b * n_rtiles + rt) of sequences with >= 2 rows, by
// decreasing tile count; then decode units (b * nsplit_max + s) of sequences
// with one row, by decreasing block count.  Equal costs in any order (no
// result depends on the order).  One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void mixed_order_kernel(
    int32_t* __restrict__ sched, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ chunk_start, int num_seqs, int n_rtiles, int nsplit_max,
    int max_blocks, int num_tokens) {
  __shared__ int hist[kChunkBuckets];
  __shared__ int dhist[kDecBuckets];
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  int32_t* chunk_list = sched + kHdrInts;
  int32_t* dec_list = chunk_list + (size_t)num_seqs * n_rtiles;
  for (int c = tid; c < kChunkBuckets; c += 1024) hist[c] = 0;
  if (tid < kDecBuckets) dhist[tid] = 0;
  __syncthreads();
  // One thread per sequence.  A decode's splits are all full (kSB blocks)
  // but the last, so it adds its full splits to that bucket with one atomic
  // and its last split to the bucket of its size; a chunk adds each of its row
  // tiles.  The scatter pass reserves the same ranges and fills them.
  auto each_seq = [&](auto&& chunk_fn, auto&& dec_fn) {
    for (int b = tid; b < num_seqs; b += 1024) {
      const int C = rows_of(cu_q_lens, b, num_tokens);
      if (C >= 2) {
        for (int rt = 0; rt * kRows < C; ++rt) {
          const int c = chunk_item_cost(cu_q_lens, chunk_start, b, rt, max_blocks, num_tokens);
          if (c > 0) chunk_fn(b * n_rtiles + rt, min(c, kChunkBuckets - 1));
        }
      } else if (C == 1) {
        const int L = min(min(chunk_start[b] + 1, max_blocks * kBlock), nsplit_max * kDecodeSplit);
        const int nb = (max(L, 0) + kBlock - 1) / kBlock;
        const int ns = max(1, (nb + kSB - 1) / kSB);  // >= 1: an empty context writes zeros
        const int last = nb - (ns - 1) * kSB;         // blocks of the last split (0 .. kSB)
        dec_fn(b * nsplit_max, ns - 1, last);
      }
    }
  };
  each_seq([&](int, int c) { atomicAdd(&hist[c], 1); },
           [&](int, int nfull, int last) {
             if (nfull > 0) atomicAdd(&dhist[kSB], nfull);
             atomicAdd(&dhist[max(last, 0)], 1);
           });
  __syncthreads();
  // chunk buckets: exclusive scan in decreasing cost order (thread t owns the
  // 4 buckets kChunkBuckets - 1 - 4t - {0..3})
  int own[4], sum = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    own[u] = hist[kChunkBuckets - 1 - 4 * tid - u];
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
    hist[kChunkBuckets - 1 - 4 * tid - u] = start;
    start += own[u];
  }
  if (tid == 0) {
    int acc = 0;
    for (int c = kDecBuckets - 1; c >= 0; --c) {
      const int n = dhist[c];
      dhist[c] = acc;
      acc += n;
    }
    sched[kHdrChunk] = part[1023];
    sched[kHdrDec] = acc;
    sched[kHdrNext] = 0;
  }
  __syncthreads();
  each_seq([&](int k, int c) { chunk_list[atomicAdd(&hist[c], 1)] = k; },
           [&](int k0, int nfull, int last) {
             if (nfull > 0) {
               const int at = atomicAdd(&dhist[kSB], nfull);
               for (int s = 0; s < nfull; ++s) dec_list[at + s] = k0 + s;
             }
             dec_list[atomicAdd(&dhist[max(last, 0)], 1)] = k0 + nfull;
           });
}

// Persistent: each workgroup takes the next unit until the list is exhausted.
// Units [0, n_chunk * Hkv) are chunk tiles (item k / Hkv for KV head k % Hkv);
// the rest are decode units (list entry j / zg for KV heads 8 (j % zg) ..).
// kQ: arena storage, 0 fp16, 1 INT8, 2 INT4.
template <int kQ>
__global__ __launch_bounds__(kThreads, 1) void mixed_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const void* __restrict__ k_arena,
    const void* __restrict__ v_arena, const int32_t* __restrict__ block_table,
    int max_blocks, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ sched,
    int32_t* __restrict__ counter, float scale_log2, int Hkv, int zg, int num_seqs,
    int n_rtiles, int nsplit_max, int num_blocks, int num_tokens) {
  // sched (counts and lists, read-only here: scalar loads) and counter (the
  // queue) are disjoint parts of the schedule
  // While more than two grids' worth of units remain, the next unit's index
  // is fetched while the current one runs; near the end of the list a unit is
  // only claimed once the previous one is done, so the longest-first order
  // balances the tail.  The index goes through a double-buffered LDS slot
  // (one barrier per unit), at the end of the chunk unit's LDS layout.
  __shared__ u32x4 lds[ChunkLds<kQ>::kUnits];
  int* const unit_slot = (int*)(lds + ChunkLds<kQ>::kSlot / 16);
  const int32_t* chunk_list = sched + kHdrInts;
  const int32_t* dec_list = chunk_list + (size_t)num_seqs * n_rtiles;
  const int n_chunk_units = sched[kHdrChunk] * Hkv;
  const int n_units = n_chunk_units + sched[kHdrDec] * zg;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x == 0) unit_slot[0] = atomicAdd(counter, 1);
  __syncthreads();
  int u = unit_slot[0];
  const int ahead = 2 * (int)gridDim.x;
  for (int it = 1; u < n_units; ++it) {
    // in flight during the unit (this file is built without the compiler's
    // wave aggregation of atomics, which would wait for the result at once):
    // the chunk unit drains it with its first wait, before any tile load
    const bool early = u + ahead < n_units;
    int next = 0;
    if (early && threadIdx.x == 0) next = atomicAdd(counter, 1);
    if (u < n_chunk_units) {
      const int k = u / Hkv, g = u - k * Hkv;
      const int item = chunk_list[k];
      const int b = item / n_rtiles, rt = item - b * n_rtiles;
      chunk_tile_unit<kQ>(lds, out, q, k_arena, v_arena, block_table, max_blocks, cu_q_lens,
                          chunk_start, scale_log2, Hkv, num_blocks, num_tokens, b, rt, g);
    } else {
      const int j = u - n_chunk_units;
      const int e = j / zg, z = j - e * zg;
      const int unit = dec_list[e];
      const int b = unit / nsplit_max, split = unit - b * nsplit_max;
      const int g = z * kDecodeWavesPerWG + wave;
      if (g < Hkv) {
        if constexpr (kQ == 0)
          decode_split_unit(out, ws_o, ws_ml, q, (const _Float16*)k_arena,
                            (const _Float16*)v_arena, block_table, max_blocks, b, cu_q_lens[b],
                            chunk_start, 1, scale_log2, Hkv, nsplit_max, num_blocks, split, g);
        else
          decode_split_q_unit<std::conditional_t<kQ == 1, CodesI8, CodesI4>>(
              out, ws_o, ws_ml, q, (const uint8_t*)k_arena, (const uint8_t*)v_arena,
              block_table, max_blocks, b, cu_q_lens[b], chunk_start, 1, scale_log2, Hkv,
              nsplit_max, num_blocks, split, g);
      }
    }
    if (threadIdx.x == 0) unit_slot[it & 1] = early ? next : atomicAdd(counter, 1);
    __syncthreads();  // every wave has left the unit (and its LDS) and may read the slot
    u = unit_slot[it & 1];
  }
}

}  // namespace

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool mixed_fast_path(const pkv_geom& g) { return chunk_fast_path(g) && decode_fast_path(g); }

// Workspace: [schedule: header + chunk list + decode list, 256-aligned]
// [decode partials as paged_attention_decode lays them out].
size_t mixed_workspace_bytes(const pkv_geom& g, int num_seqs, int num_tokens,
                             int max_context_len) {
  if (!mixed_fast_path(g) || num_seqs <= 0 || num_tokens <= 0) return 0;
  const size_t n_rtiles = (size_t)(num_tokens + kRows - 1) / kRows;
  const size_t nsplit = (size_t)(max(max_context_len, 1) + kDecodeSplit - 1) / kDecodeSplit;
  const size_t sched = align256((kHdrInts + (size_t)num_seqs * (n_rtiles + nsplit)) * 4);
  return sched + decode_workspace_bytes(g, num_seqs, max_context_len);
}

hipError_t launch_mixed(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                        const void* v_arena, const int32_t* block_table, int max_blocks,
                        const int32_t* cu_q_lens, const int32_t* chunk_start, int num_seqs,
                        int num_tokens, int max_q_len, int max_context_len, float scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // the chunk units track maxima of raw scores, which needs scale > 0
  if (!mixed_fast_path(g) || !(scale > 0.f) || !(scale < INFINITY))
    return launch_attend_generic(g, out, q, k_arena, v_arena, block_table, max_blocks, nullptr,
                                 cu_q_lens, chunk_start, num_seqs, num_tokens, scale, stream);
  // the schedule is laid out for the bounds mixed_workspace_bytes assumed
  const int n_rtiles = (num_tokens + kRows - 1) / kRows;
  const int nsplit_max = (max(max_context_len, 1) + kDecodeSplit - 1) / kDecodeSplit;
  (void)max_q_len;
  if (!workspace ||
      workspace_bytes < mixed_workspace_bytes(g, num_seqs, num_tokens, max_context_len))
    return hipErrorInvalidValue;
  int32_t* sched = (int32_t*)workspace;
  const size_t sched_bytes =
      align256((kHdrInts + (size_t)num_seqs * (n_rtiles + nsplit_max)) * 4);
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (nsplit_max > 1) {
    const size_t parts = (size_t)num_seqs * g.num_q_heads * nsplit_max;
    ws_o = (float*)((char*)workspace + sched_bytes);
    ws_ml = (float*)((char*)ws_o + align256(parts * kD * sizeof(float)));
  }
  hipLaunchKernelGGL(mixed_order_kernel, dim3(1), dim3(1024), 0, stream, sched, cu_q_lens,
                     chunk_start, num_seqs, n_rtiles, nsplit_max, max_blocks, num_tokens);
  const float scale_log2 = scale * 1.4426950408889634f;
  const int zg = (g.num_kv_heads + kDecodeWavesPerWG - 1) / kDecodeWavesPerWG;
  int dev = 0, num_cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  auto kernel = g.dtype == PKV_I8KV ? mixed_kernel<1>
                : g.dtype == PKV_I4KV ? mixed_kernel<2> : mixed_kernel<0>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)max(num_cus, 1)), dim3(kThreads), 0, stream,
                     out, ws_o, ws_ml, (const _Float16*)q, k_arena, v_arena, block_table,
                     max_blocks, cu_q_lens, chunk_start, sched, sched + kHdrNext, scale_log2,
                     g.num_kv_heads, zg, num_seqs, n_rtiles, nsplit_max, g.num_blocks,
                     num_tokens);
  e = hipGetLastError();
  if (e != hipSuccess || nsplit_max <= 1) return e;
  return launch_decode_combine(g, out, ws_o, ws_ml, chunk_start, cu_q_lens, num_tokens,
                               max_blocks, num_seqs, nsplit_max, stream);
}

}  // namespace pkv
