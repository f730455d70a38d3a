// Whole-block copies of the arena.
//   pkv_copy_blocks: the copy of copy-on-write (Kshipra part 3, section 3: a
//   shared block a request diverges inside is copied before it is written).
//   One workgroup per (src, dst) pair copies the whole block — every KV head
//   and all 16 slots — of both arenas with 16-byte loads and stores.
//   pkv_swap_out / pkv_swap_in: preemption by swapping (part 3, section 5: a
//   running sequence's blocks are swapped out of the arena and restored later
//   instead of being recomputed).  One workgroup per (block, K or V) moves the
//   block's tile between the arena and a packed buffer, normally pinned host
//   memory read and written directly over the host link.
#include "pkv_internal.h"

namespace pkv {
namespace {

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_arena,
                                                         uint4* __restrict__ v_arena,
                                                         const int32_t* __restrict__ src_dst,
                                                         size_t vecs_per_block, int num_blocks) {
  const int src = src_dst[2 * blockIdx.x], dst = src_dst[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const uint4* ks = k_arena + (size_t)src * vecs_per_block;
  const uint4* vs = v_arena + (size_t)src * vecs_per_block;
  uint4* kd = k_arena + (size_t)dst * vecs_per_block;
  uint4* vd = v_arena + (size_t)dst * vecs_per_block;
  for (size_t i = threadIdx.x; i < vecs_per_block; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

// dir 0: arena -> buf (swap out); dir 1: buf -> arena (swap in).  Buffer
// layout: [n][K tile, V tile], each tile vecs_per_block 16-byte units.
template <int DIR>
__global__ __launch_bounds__(256) void swap_blocks_kernel(uint4* __restrict__ k_arena,
                                                         uint4* __restrict__ v_arena,
                                                         const int32_t* __restrict__ ids,
                                                         uint4* __restrict__ buf,
                                                         size_t vecs_per_block, int num_blocks) {
  const int i = blockIdx.x, which = blockIdx.y;
  const int blk = ids[i];
  if (blk < 0 || blk >= num_blocks) return;
  uint4* tile = (which == 0 ? k_arena : v_arena) + (size_t)blk * vecs_per_block;
  uint4* packed = buf + ((size_t)2 * i + which) * vecs_per_block;
  constexpr int kUnroll = 4;
  for (size_t j0 = 0; j0 < vecs_per_block; j0 += kUnroll * blockDim.x) {
    uint4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = j0 + u * blockDim.x + threadIdx.x;
      if (j < vecs_per_block) r[u] = DIR == 0 ? tile[j] : packed[j];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t j = j0 + u * blockDim.x + threadIdx.x;
      if (j < vecs_per_block) {
        if (DIR == 0) packed[j] = r[u];
        else tile[j] = r[u];
      }
    }
  }
}

}  // namespace

size_t swap_tile_bytes(const pkv_geom& g) { return (size_t)g.num_kv_heads * kv_tile_bytes(g); }

hipError_t launch_swap_blocks(const pkv_geom& g, void* k_arena, void* v_arena,
                              const int32_t* ids, int n, void* buf, bool swap_in,
                              hipStream_t stream) {
  const size_t vecs = swap_tile_bytes(g) / 16;
  const dim3 grid(n, 2);
  if (swap_in)
    hipLaunchKernelGGL(swap_blocks_kernel<1>, grid, dim3(256), 0, stream, (uint4*)k_arena,
                       (uint4*)v_arena, ids, (uint4*)buf, vecs, g.num_blocks);
  else
    hipLaunchKernelGGL(swap_blocks_kernel<0>, grid, dim3(256), 0, stream, (uint4*)k_arena,
                       (uint4*)v_arena, ids, (uint4*)buf, vecs, g.num_blocks);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const pkv_geom& g, void* k_arena, void* v_arena,
                              const int32_t* src_dst, int n, hipStream_t stream) {
  const size_t vecs = (size_t)g.num_kv_heads * kv_tile_bytes(g) / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n), dim3(256), 0, stream, (uint4*)k_arena,
                     (uint4*)v_arena, src_dst, vecs, g.num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
