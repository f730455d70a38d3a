// Generic paged attention: any storage dtype (INT8 arenas dequantized element
// by element, x_hat = code * scale, exact in fp32), head_dim <= 256, any
// query/KV head ratio.  One workgroup per (row, query head) walks the row's blocks in
// place through the block table with the online-softmax merge of Kshipra
// part 3, section 4 (running max, rescaled denominator and accumulator, then
// out = o / l).  It serves the shapes the tuned kernels do not cover (fp32
// storage, other head dims and group sizes); fp32 arithmetic throughout.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 128;

// Element (d, slot) of a K / V tile of the arena, as a float.
template <typename T>
struct TileReader {
  const T* kt;
  const T* vt;
  __device__ TileReader(const void* k_arena, const void* v_arena, int blk, int Hkv, int g, int D)
      : kt((const T*)k_arena + ((size_t)blk * Hkv + g) * kBlock * D),
        vt((const T*)v_arena + ((size_t)blk * Hkv + g) * D * kBlock) {}
  __device__ float k(int d, int slot, int D) const {
    constexpr int x = 16 / sizeof(T);  // K tile layout [D/x][16][x]
    (void)D;
    return (float)kt[((d / x) * kBlock + slot) * x + d % x];
  }
  __device__ float v(int d, int slot) const { return (float)vt[d * kBlock + slot]; }
};
// INT8 tiles: codes then 16 fp16 scales, padded to 128-byte lines; K keys at
// their stored positions i8_kpos(slot)
struct TileReaderI8 {
  const uint8_t* kt;
  const uint8_t* vt;
  int D;
  __device__ TileReaderI8(const void* k_arena, const void* v_arena, int blk, int Hkv, int g, int D_)
      : D(D_) {
    const size_t tb = i8_tile_bytes(D_);
    kt = (const uint8_t*)k_arena + ((size_t)blk * Hkv + g) * tb;
    vt = (const uint8_t*)v_arena + ((size_t)blk * Hkv + g) * tb;
  }
  __device__ float k(int d, int slot, int) const {
    const float code = (float)(int8_t)kt[(d >> 4) * 256 + i8_kpos(slot) * 16 + (d & 15)];
    return code * (float)((const _Float16*)(kt + (size_t)kBlock * D))[slot];
  }
  __device__ float v(int d, int slot) const {
    const float code = (float)(int8_t)vt[d * kBlock + slot];
    return code * (float)((const _Float16*)(vt + (size_t)kBlock * D))[slot];
  }
};

// INT4 tiles: two codes per byte (two's-complement nibbles), then 16 fp16
// scales, padded to 128-byte lines; K records i4_krec(slot) of 8 bytes per
// 16-dim piece (byte i: dims i, i + 8), V byte i4_vbyte(d, slot, D).
struct TileReaderI4 {
  const uint8_t* kt;
  const uint8_t* vt;
  int D;
  __device__ TileReaderI4(const void* k_arena, const void* v_arena, int blk, int Hkv, int g, int D_)
      : D(D_) {
    const size_t tb = i4_tile_bytes(D_);
    kt = (const uint8_t*)k_arena + ((size_t)blk * Hkv + g) * tb;
    vt = (const uint8_t*)v_arena + ((size_t)blk * Hkv + g) * tb;
  }
  __device__ static float nibble(uint8_t byte, int high) {
    const int n = high ? byte >> 4 : byte & 15;
    return (float)((n ^ 8) - 8);
  }
  __device__ float k(int d, int slot, int) const {
    const uint8_t byte = kt[(d >> 4) * 128 + i4_krec(slot) * 8 + (d & 7)];
    return nibble(byte, (d >> 3) & 1) * (float)((const _Float16*)(kt + (size_t)kBlock * D / 2))[slot];
  }
  __device__ float v(int d, int slot) const {
    const uint8_t byte = vt[i4_vbyte(d, slot, D)];
    return nibble(byte, i4_vhigh(slot)) * (float)((const _Float16*)(vt + (size_t)kBlock * D / 2))[slot];
  }
};

template <typename T, typename Reader>
__global__ __launch_bounds__(kThreads) void attend_generic_kernel(
    float* __restrict__ out, const T* __restrict__ q, const void* __restrict__ k_arena,
    const void* __restrict__ v_arena, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ chunk_start, int num_seqs, float scale, int num_blocks, int Hq,
    int Hkv, int D) {
  const int row = blockIdx.x;  // decode: sequence index; chunk: packed token index
  const int h = blockIdx.y;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x;
  int b, L;
  if (cu_q_lens == nullptr) {
    b = row;
    L = context_lens[b];
  } else {
    b = find_seq(cu_q_lens, num_seqs, row);
    L = chunk_start[b] + (row - cu_q_lens[b]) + 1;  // keys j <= own position
  }
  L = min(L, max_blocks * kBlock);
  float* o_out = out + ((size_t)row * Hq + h) * D;
  if (L <= 0) {
    for (int d = tid; d < D; d += kThreads) o_out[d] = 0.f;
    return;
  }

  __shared__ float qs[256];
  __shared__ float sc[kBlock];
  const T* qp = q + ((size_t)row * Hq + h) * D;
  for (int d = tid; d < D; d += kThreads) qs[d] = (float)qp[d];
  __syncthreads();

  const int jl = tid >> 3, sub = tid & 7;  // 16 tokens x 8 partial-dot lanes
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  const int nblk = (L + kBlock - 1) / kBlock;
  const int32_t* bt = block_table + (size_t)b * max_blocks;
  for (int n = 0; n < nblk; ++n) {
    int blk = bt[n];
    if (blk < 0 || blk >= num_blocks) blk = 0;
    const Reader tr(k_arena, v_arena, blk, Hkv, g, D);
    const int tok = n * kBlock + jl;
    float part = 0.f;
    if (tok < L)
      for (int d = sub; d < D; d += 8) part += qs[d] * tr.k(d, jl, D);
    part += __shfl_xor(part, 1, 8);
    part += __shfl_xor(part, 2, 8);
    part += __shfl_xor(part, 4, 8);
    if (sub == 0) sc[jl] = tok < L ? part * scale : -INFINITY;
    __syncthreads();
    float mb = -INFINITY;
    for (int j = 0; j < kBlock; ++j) mb = fmaxf(mb, sc[j]);
    const float m_new = fmaxf(m, mb);
    const float alpha = expf(m - m_new);
    const int nvalid = min(kBlock, L - n * kBlock);
    float psum = 0.f, a0 = acc0 * alpha, a1 = acc1 * alpha;
    for (int j = 0; j < nvalid; ++j) {
      const float p = expf(sc[j] - m_new);
      psum += p;
      if (tid < D) a0 += p * tr.v(tid, j);
      if (tid + kThreads < D) a1 += p * tr.v(tid + kThreads, j);
    }
    l = l * alpha + psum;
    acc0 = a0;
    acc1 = a1;
    m = m_new;
    __syncthreads();
  }
  const float inv = 1.f / l;
  if (tid < D) o_out[tid] = acc0 * inv;
  if (tid + kThreads < D) o_out[tid + kThreads] = acc1 * inv;
}

}  // namespace

hipError_t launch_attend_generic(const pkv_geom& g, float* out, const void* q,
                                 const void* k_arena, const void* v_arena,
                                 const int32_t* block_table, int max_blocks,
                                 const int32_t* context_lens, const int32_t* cu_q_lens,
                                 const int32_t* chunk_start, int num_seqs, int num_rows,
                                 float scale, hipStream_t stream) {
  const dim3 grid(num_rows, g.num_q_heads), block(kThreads);
  if (g.dtype == PKV_I4KV) {
    hipLaunchKernelGGL((attend_generic_kernel<_Float16, TileReaderI4>), grid, block, 0, stream,
                       out, (const _Float16*)q, k_arena, v_arena, block_table, max_blocks,
                       context_lens, cu_q_lens, chunk_start, num_seqs, scale, g.num_blocks,
                       g.num_q_heads, g.num_kv_heads, g.head_dim);
  } else if (g.dtype == PKV_I8KV) {
    hipLaunchKernelGGL((attend_generic_kernel<_Float16, TileReaderI8>), grid, block, 0, stream,
                       out, (const _Float16*)q, k_arena, v_arena, block_table, max_blocks,
                       context_lens, cu_q_lens, chunk_start, num_seqs, scale, g.num_blocks,
                       g.num_q_heads, g.num_kv_heads, g.head_dim);
  } else if (g.dtype == PKV_F16) {
    hipLaunchKernelGGL((attend_generic_kernel<_Float16, TileReader<_Float16>>), grid, block, 0,
                       stream, out, (const _Float16*)q, k_arena, v_arena,
                       block_table, max_blocks, context_lens, cu_q_lens, chunk_start, num_seqs,
                       scale, g.num_blocks, g.num_q_heads, g.num_kv_heads, g.head_dim);
  } else {
    hipLaunchKernelGGL((attend_generic_kernel<float, TileReader<float>>), grid, block, 0,
                       stream, out, (const float*)q, k_arena, v_arena,
                       block_table, max_blocks, context_lens, cu_q_lens, chunk_start, num_seqs,
                       scale, g.num_blocks, g.num_q_heads, g.num_kv_heads, g.head_dim);
  }
  return hipGetLastError();
}

}  // namespace pkv
