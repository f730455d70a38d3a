// Internal declarations shared by the libpkv translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkv.h"

namespace pkv {

// Decode split size in tokens (a multiple of 32).  Fixed at build time, never
// derived from the batch, so a sequence's decode result is independent of the
// other sequences.
#ifndef PKV_DECODE_SPLIT
#define PKV_DECODE_SPLIT 384
#endif
constexpr int kDecodeSplit = PKV_DECODE_SPLIT;
constexpr int kBlock = PKV_BLOCK_SIZE;

// fp64 -> IEEE binary16 bits, round to nearest, ties to even, written from the
// IEEE 754 definition: the exact value sig * 2^(e-52) is expressed in units of
// the destination ulp 2^(max(e,-14)-10); the dropped bits decide the rounding.
// Handles fp16 subnormals, overflow to infinity, infinities and NaN.
__host__ __device__ inline uint16_t f64_to_f16_bits(double x) {
  uint64_t u;
  __builtin_memcpy(&u, &x, 8);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const int bexp = (int)((u >> 52) & 0x7FF);
  const uint64_t man = u & ((1ull << 52) - 1);
  if (bexp == 0x7FF) return (uint16_t)(sign | 0x7C00u | (man ? 0x0200u : 0u));
  if (bexp == 0) return sign;                     // |x| < 2^-1022: rounds to zero
  const int e = bexp - 1023;
  if (e > 15) return (uint16_t)(sign | 0x7C00u);  // >= 2^16: infinity
  const uint64_t sig = (1ull << 52) | man;
  const int te = e < -14 ? -14 : e;
  const int shift = 42 + (te - e);               // 52 - 10 + (te - e)
  if (shift >= 54) return sign;                   // below half the smallest subnormal
  uint64_t qv = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (qv & 1))) ++qv;
  if (te == -14 && qv < 1024) return (uint16_t)(sign | qv);          // subnormal
  const uint32_t bits = ((uint32_t)(te + 15) << 10) + (uint32_t)(qv - 1024);  // carry ok
  if (bits >= 0x7C00u) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | bits);
}

// Sequence of packed row t: the last b in [0, num_seqs) with cu[b] <= t
// (cu nondecreasing, cu[0] = 0).  Wave-parallel search: each round the 64
// lanes test 64 evenly spaced candidates and the range shrinks 64-fold, so up
// to 4096 sequences cost two dependent loads.  Every lane of the wave must
// call it with the same t.
__device__ inline int find_seq(const int32_t* __restrict__ cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs;  // the answer lies in [lo, hi); cu[lo] <= t
  const int lane = threadIdx.x & 63;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const unsigned long long m = __ballot(idx < hi && cu[idx] <= t);
    if (m == 0) break;  // only if cu[0] > t (caller contract violation)
    lo += (63 - __clzll(m)) * step;  // true lanes form a prefix: cu is sorted
    hi = min(hi, lo + step);
  }
  return lo;
}

// find_seq for the append kernels, which also need the row's sequence start
// row0 = cu[b] and chunk start P = start[b]: the final round (at most 64
// candidates, one per lane) loads each candidate's start beside its cu, so the
// lookup of a batch of up to 64 sequences is one dependent load, not two.
__device__ inline int find_seq_start(const int32_t* __restrict__ cu,
                                     const int32_t* __restrict__ start, int num_seqs, int t,
                                     int& row0, int& P) {
  int lo = 0, hi = num_seqs;  // the answer lies in [lo, hi); cu[lo] <= t
  const int lane = threadIdx.x & 63;
  while (hi - lo > 64) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const unsigned long long m = __ballot(idx < hi && cu[idx] <= t);
    if (m == 0) break;  // only if cu[0] > t (caller contract violation)
    lo += (63 - __clzll(m)) * step;
    hi = min(hi, lo + step);
  }
  const int idx = lo + lane;
  const bool in = idx < hi;
  const int c = in ? cu[idx] : 0, p = in ? start[idx] : 0;
  const unsigned long long m = __ballot(in && c <= t);
  const int l = m ? 63 - __clzll(m) : 0;  // lane 0 (= lo) on a contract violation
  row0 = __builtin_amdgcn_readlane(c, l);
  P = __builtin_amdgcn_readlane(p, l);
  return lo + l;
}

// INT8 tiles: codes then 16 fp16 scales, padded to whole 128-byte lines.
__host__ __device__ constexpr size_t i8_tile_bytes(int head_dim) {
  return ((size_t)kBlock * head_dim + 2 * kBlock + 127) / 128 * 128;
}
// Stored position of slot s among the 16 keys of an INT8 K piece: bits 2 and 3
// exchanged, so that the slots {0-3, 8-11} and {4-7, 12-15} the decode kernel
// reads together are each one contiguous 128-byte run.
__host__ __device__ constexpr int i8_kpos(int s) {
  return (s & 3) | ((s >> 1) & 4) | ((s << 1) & 8);
}

// INT4 tiles: 4-bit codes (two per byte) then 16 fp16 scales, padded to
// whole 128-byte lines.
__host__ __device__ constexpr size_t i4_tile_bytes(int head_dim) {
  return ((size_t)kBlock * head_dim / 2 + 2 * kBlock + 127) / 128 * 128;
}
// INT4 K: 8-byte record of slot s within a 16-dim piece, so that the two keys
// one decode lane reads (s and s + 4 within a group of 8) are adjacent.
__host__ __device__ constexpr int i4_krec(int s) {
  return 2 * (4 * ((s >> 3) & 1) + (s & 3)) + ((s >> 2) & 1);
}
// INT4 V: byte holding the code of slot s for head dim d (head_dim D, a
// multiple of 32), and its nibble.  Head dims go in groups of 64 (the last
// may hold 32); a group of G 16-dim blocks is [key half s >> 3][d & 15][block
// (d >> 4) & 3] words of 4 bytes, byte i of a word holding slots 8h + i (low
// nibble) and 8h + 4 + i (high).  One 16-byte load then gives a decode lane
// the 8 keys of one half for 4 dim blocks.
__host__ __device__ constexpr int i4_vbyte(int d, int s, int D) {
  return 512 * (d >> 6) +
         4 * (((s >> 3) * 16 + (d & 15)) * (D - 64 * (d >> 6) >= 64 ? 4 : 2) + ((d >> 4) & 3)) +
         (s & 3);
}
__host__ __device__ constexpr int i4_vhigh(int s) { return (s >> 2) & 1; }

// Bytes of one (block, KV head) tile of either arena.
inline size_t kv_tile_bytes(const pkv_geom& g) {
  if (g.dtype == PKV_I8KV) return i8_tile_bytes(g.head_dim);
  if (g.dtype == PKV_I4KV) return i4_tile_bytes(g.head_dim);
  return (size_t)kBlock * g.head_dim * (g.dtype == PKV_F16 ? 2 : 4);
}

// ---- launchers (defined in the kernel translation units) -------------------
hipError_t launch_append_rope(const pkv_geom& g, const void* q, void* q_out, const void* k,
                              const void* v, void* k_arena, void* v_arena,
                              const int32_t* block_table, int max_blocks,
                              const int32_t* cu_q_lens, const int32_t* chunk_start,
                              int num_seqs, int num_tokens, const void* rope_table,
                              int rope_max_pos, hipStream_t stream);

bool decode_fast_path(const pkv_geom& g);
size_t decode_workspace_bytes(const pkv_geom& g, int num_seqs, int max_context_len);
// Rows sharing their leading splits (decode_shared_kernel).  Device arrays:
// group_start [num_groups + 1] (group i = rows group_start[i] .. [i+1]),
// row_skip [num_seqs] (leading splits of the row computed with its group).
struct DecodeGroups {
  const int32_t* group_start;
  const int32_t* row_skip;
  int num_groups;
  int max_skip;        // host bound of row_skip
  int max_group_size;  // host bound of a group's row count
};
hipError_t launch_decode(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                         const void* v_arena, const int32_t* block_table, int max_blocks,
                         const int32_t* context_lens, int num_seqs, int max_context_len,
                         float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, const DecodeGroups* groups = nullptr);

// paged_attention_decode with the step's append fused in (fp16 arenas on the
// decode fast path; the caller checks).
hipError_t launch_decode_append(const pkv_geom& g, float* out, const void* q, void* q_out,
                                const void* k, const void* v, void* k_arena, void* v_arena,
                                const int32_t* block_table, int max_blocks,
                                const int32_t* context_lens, int num_seqs, int max_context_len,
                                float scale, const void* rope_table, int rope_max_pos,
                                void* workspace, hipStream_t stream);

// The device address and size of the calling device's decode scratch array
// (the split partials of paged_attention_decode_noalloc); looked up once per
// device.
hipError_t decode_scratch(void** ptr, size_t* bytes);

// Merge of decode split partials (decode_combine_kernel): decode rows, or the
// one-row sequences of a varlen batch when cu_q_lens != nullptr (lens then
// holds chunk starts).
hipError_t launch_decode_combine(const pkv_geom& g, float* out, const float* ws_o,
                                 const float* ws_ml, const int32_t* lens,
                                 const int32_t* cu_q_lens, int num_tokens, int max_blocks,
                                 int num_seqs, int nsplit_max, hipStream_t stream);

bool chunk_fast_path(const pkv_geom& g);
size_t chunk_workspace_bytes(const pkv_geom& g, int num_seqs, int num_tokens,
                             int max_context_len);
// key-range parts paged_attention_chunk splits a call's items into (1: none)
int chunk_parts(const pkv_geom& g, int num_tokens, int max_context_len);
// paged_attention_chunk = launch_chunk_plan (the schedule into the workspace)
// then launch_chunk_run (the attention over it)
hipError_t launch_chunk(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                        const void* v_arena, const int32_t* block_table, int max_blocks,
                        const int32_t* cu_q_lens, const int32_t* chunk_start, int num_seqs,
                        int num_tokens, int max_q_len, int max_context_len, float scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);
hipError_t launch_chunk_plan(const pkv_geom& g, const int32_t* cu_q_lens,
                             const int32_t* chunk_start, int max_blocks, int num_seqs,
                             int num_tokens, int max_q_len, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
hipError_t launch_chunk_run(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                            const void* v_arena, const int32_t* block_table, int max_blocks,
                            const int32_t* cu_q_lens, const int32_t* chunk_start, int num_seqs,
                            int num_tokens, int max_q_len, int max_context_len, float scale,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

// One attention launch for a varlen batch of prefill chunks and decodes
// (sequences of one row), with a schedule and decode partials in the workspace.
bool mixed_fast_path(const pkv_geom& g);
size_t mixed_workspace_bytes(const pkv_geom& g, int num_seqs, int num_tokens,
                             int max_context_len);
hipError_t launch_mixed(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                        const void* v_arena, const int32_t* block_table, int max_blocks,
                        const int32_t* cu_q_lens, const int32_t* chunk_start, int num_seqs,
                        int num_tokens, int max_q_len, int max_context_len, float scale,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

// Generic (any dtype / head_dim / group) attention, one workgroup per
// (row, query head).  Decode rows when cu_q_lens == nullptr.
hipError_t launch_attend_generic(const pkv_geom& g, float* out, const void* q,
                                 const void* k_arena, const void* v_arena,
                                 const int32_t* block_table, int max_blocks,
                                 const int32_t* context_lens, const int32_t* cu_q_lens,
                                 const int32_t* chunk_start, int num_seqs, int num_rows,
                                 float scale, hipStream_t stream);

hipError_t launch_copy_blocks(const pkv_geom& g, void* k_arena, void* v_arena,
                              const int32_t* src_dst, int n, hipStream_t stream);
size_t swap_tile_bytes(const pkv_geom& g);
hipError_t launch_swap_blocks(const pkv_geom& g, void* k_arena, void* v_arena,
                              const int32_t* ids, int n, void* buf, bool swap_in,
                              hipStream_t stream);

}  // namespace pkv
