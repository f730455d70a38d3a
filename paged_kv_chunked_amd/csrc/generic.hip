// Generic paged attention: any storage dtype, head_dim <= 256, any query/KV
// head ratio.  One workgroup per (row, query head) walks the row's blocks in
// place through the block table with the online-softmax merge of Kshipra
// part 3, section 4 (running max, rescaled denominator and accumulator, then
// out = o / l).  It serves the shapes the tuned kernels do not cover (fp32
// storage, other head dims and group sizes); fp32 arithmetic throughout.
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 128;

template <typename T>
__global__ __launch_bounds__(kThreads) void attend_generic_kernel(
    float* __restrict__ out, const T* __restrict__ q, const T* __restrict__ k_arena,
    const T* __restrict__ v_arena, const int32_t* __restrict__ block_table, int max_blocks,
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
    const T* kt = k_arena + ((size_t)blk * Hkv + g) * kBlock * D;
    const T* vt = v_arena + ((size_t)blk * Hkv + g) * D * kBlock;
    const int tok = n * kBlock + jl;
    float part = 0.f;
    constexpr int x = 16 / sizeof(T);  // K tile layout [D/x][16][x]
    if (tok < L)
      for (int d = sub; d < D; d += 8) part += qs[d] * (float)kt[((d / x) * kBlock + jl) * x + d % x];
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
      if (tid < D) a0 += p * (float)vt[tid * kBlock + j];
      if (tid + kThreads < D) a1 += p * (float)vt[(tid + kThreads) * kBlock + j];
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
  if (g.dtype == PKV_F16) {
    hipLaunchKernelGGL(attend_generic_kernel<_Float16>, grid, block, 0, stream, out,
                       (const _Float16*)q, (const _Float16*)k_arena, (const _Float16*)v_arena,
                       block_table, max_blocks, context_lens, cu_q_lens, chunk_start, num_seqs,
                       scale, g.num_blocks, g.num_q_heads, g.num_kv_heads, g.head_dim);
  } else {
    hipLaunchKernelGGL(attend_generic_kernel<float>, grid, block, 0, stream, out,
                       (const float*)q, (const float*)k_arena, (const float*)v_arena,
                       block_table, max_blocks, context_lens, cu_q_lens, chunk_start, num_seqs,
                       scale, g.num_blocks, g.num_q_heads, g.num_kv_heads, g.head_dim);
  }
  return hipGetLastError();
}

}  // namespace pkv
