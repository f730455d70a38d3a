// pkv_copy_blocks: the copy of copy-on-write (Kshipra part 3, section 3: a
// shared block a request diverges inside is copied before it is written).
// One workgroup per (src, dst) pair copies the whole block — every KV head and
// all 16 slots — of both arenas with 16-byte loads and stores.
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

}  // namespace

hipError_t launch_copy_blocks(const pkv_geom& g, void* k_arena, void* v_arena,
                              const int32_t* src_dst, int n, hipStream_t stream) {
  const size_t elt = g.dtype == PKV_F16 ? 2 : 4;
  const size_t vecs = (size_t)g.num_kv_heads * kBlock * g.head_dim * elt / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n), dim3(256), 0, stream, (uint4*)k_arena,
                     (uint4*)v_arena, src_dst, vecs, g.num_blocks);
  return hipGetLastError();
}

}  // namespace pkv
