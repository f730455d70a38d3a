// C ABI entry points of libpkv: host-side validation, then kernel launches on
// the caller's stream.  See include/pkv.h for the contracts.
#include "pkv_internal.h"

namespace {

pkv_status check_geom(const pkv_geom* g) {
  if (!g) return PKV_ERR_NULL;
  if (g->block_size != PKV_BLOCK_SIZE) return PKV_ERR_SHAPE;
  if (g->num_blocks < 1 || g->num_kv_heads < 1 || g->num_q_heads < 1) return PKV_ERR_SHAPE;
  if (g->num_q_heads % g->num_kv_heads) return PKV_ERR_SHAPE;
  if (g->dtype != PKV_F16 && g->dtype != PKV_F32 && g->dtype != PKV_I8KV &&
      g->dtype != PKV_I4KV)
    return PKV_ERR_DTYPE;
  // head_dim: a whole number of 16-byte pieces (the K tile layout), <= 256;
  // INT4 pairs dims i and i + 8 of 16-dim pieces in both halves of a head
  const int piece = g->dtype == PKV_F16 ? 8 : g->dtype == PKV_F32 ? 4
                    : g->dtype == PKV_I8KV ? 16 : 32;
  if (g->head_dim < piece || g->head_dim % piece || g->head_dim > 256) return PKV_ERR_SHAPE;
  return PKV_OK;
}

pkv_status hip_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_HIP; }

}  // namespace

namespace pkv {
// measurement helper (stream.hip)
hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t stream);
}  // namespace pkv

extern "C" {

pkv_status kv_append_rope(const pkv_geom* geom, void* q, void* q_out, const void* k,
                          const void* v,
                          void* k_arena, void* v_arena, const int32_t* block_table,
                          int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                          const int32_t* chunk_start, int32_t num_seqs, int32_t num_tokens,
                          const void* rope_table, int32_t rope_max_pos, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_tokens < 0) return PKV_ERR_RANGE;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_arena || !v_arena || !block_table || !cu_q_lens || !chunk_start ||
      !rope_table)
    return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || rope_max_pos < 1) return PKV_ERR_RANGE;
  return hip_status(pkv::launch_append_rope(*geom, q, q_out ? q_out : q, k, v, k_arena,
                                            v_arena, block_table, max_blocks_per_seq,
                                            cu_q_lens, chunk_start, num_seqs, num_tokens,
                                            rope_table, rope_max_pos, (hipStream_t)stream));
}

pkv_status paged_attention_decode_workspace_bytes(const pkv_geom* geom, int32_t num_seqs,
                                                  int32_t max_context_len, size_t* bytes) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (!bytes) return PKV_ERR_NULL;
  if (num_seqs < 0 || max_context_len < 0) return PKV_ERR_RANGE;
  *bytes = pkv::decode_workspace_bytes(*geom, num_seqs, max_context_len);
  return PKV_OK;
}

pkv_status paged_attention_decode(const pkv_geom* geom, void* out, int32_t out_dtype,
                                  const void* q, const void* k_arena, const void* v_arena,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, float scale, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (out_dtype != PKV_F32) return PKV_ERR_DTYPE;
  if (num_seqs < 0) return PKV_ERR_RANGE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_arena || !v_arena || !block_table || !context_lens) return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || max_context_len < 1 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return PKV_ERR_RANGE;
  const size_t need = pkv::decode_workspace_bytes(*geom, num_seqs, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  return hip_status(pkv::launch_decode(*geom, (float*)out, q, k_arena, v_arena, block_table,
                                       max_blocks_per_seq, context_lens, num_seqs,
                                       max_context_len, scale, workspace, workspace_bytes,
                                       (hipStream_t)stream));
}

pkv_status paged_attention_decode_append(const pkv_geom* geom, void* out, int32_t out_dtype,
                                         const void* q, void* q_out, const void* k, const void* v,
                                         void* k_arena, void* v_arena, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t max_context_len, float scale,
                                         const void* rope_table, int32_t rope_max_pos,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (out_dtype != PKV_F32) return PKV_ERR_DTYPE;
  if (geom->dtype == PKV_F32) return PKV_ERR_DTYPE;
  if (!pkv::decode_fast_path(*geom)) return PKV_ERR_SHAPE;
  if (num_seqs < 0) return PKV_ERR_RANGE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !q_out || !k || !v || !k_arena || !v_arena || !block_table ||
      !context_lens || !rope_table)
    return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || max_context_len < 1 || rope_max_pos < 1 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return PKV_ERR_RANGE;
  // every workgroup of a sequence reads q while its first split writes q_out
  const size_t qbytes = (size_t)num_seqs * geom->num_q_heads * geom->head_dim * 2;
  const char* q0 = (const char*)q;
  const char* o0 = (const char*)q_out;
  if (o0 < q0 + qbytes && q0 < o0 + qbytes) return PKV_ERR_RANGE;
  const size_t need = pkv::decode_workspace_bytes(*geom, num_seqs, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  return hip_status(pkv::launch_decode_append(*geom, (float*)out, q, q_out, k, v, k_arena, v_arena,
                                              block_table, max_blocks_per_seq, context_lens,
                                              num_seqs, max_context_len, scale, rope_table,
                                              rope_max_pos, workspace, (hipStream_t)stream));
}

pkv_status paged_attention_decode_noalloc(const pkv_geom* geom, void* out, int32_t out_dtype,
                                          const void* q, const void* k_arena,
                                          const void* v_arena, const int32_t* block_table,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t max_context_len, float scale, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (out_dtype != PKV_F32) return PKV_ERR_DTYPE;
  if (num_seqs < 0) return PKV_ERR_RANGE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_arena || !v_arena || !block_table || !context_lens) return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || max_context_len < 1 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return PKV_ERR_RANGE;
  const size_t need = pkv::decode_workspace_bytes(*geom, num_seqs, max_context_len);
  if (need > PKV_DECODE_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (need > 0) {
    const hipError_t e = pkv::decode_scratch(&ws, &ws_bytes);
    if (e != hipSuccess) return PKV_ERR_HIP;
    if (ws_bytes < need) return PKV_ERR_WORKSPACE;
  }
  return hip_status(pkv::launch_decode(*geom, (float*)out, q, k_arena, v_arena, block_table,
                                       max_blocks_per_seq, context_lens, num_seqs,
                                       max_context_len, scale, ws, ws_bytes,
                                       (hipStream_t)stream));
}

pkv_status paged_attention_decode_shared(
    const pkv_geom* geom, void* out, int32_t out_dtype, const void* q, const void* k_arena,
    const void* v_arena, const int32_t* block_table, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len, float scale,
    const int32_t* group_start, const int32_t* row_skip, int32_t num_groups, int32_t max_skip,
    int32_t max_group_size, void* workspace, size_t workspace_bytes, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (out_dtype != PKV_F32) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_groups < 0 || max_skip < 0 || max_group_size < 0) return PKV_ERR_RANGE;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_arena || !v_arena || !block_table || !context_lens) return PKV_ERR_NULL;
  if (num_groups > 0 && (!group_start || !row_skip)) return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || max_context_len < 1 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return PKV_ERR_RANGE;
  const size_t need = pkv::decode_workspace_bytes(*geom, num_seqs, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  const pkv::DecodeGroups groups{group_start, row_skip, num_groups, max_skip, max_group_size};
  return hip_status(pkv::launch_decode(*geom, (float*)out, q, k_arena, v_arena, block_table,
                                       max_blocks_per_seq, context_lens, num_seqs,
                                       max_context_len, scale, workspace, workspace_bytes,
                                       (hipStream_t)stream, num_groups > 0 ? &groups : nullptr));
}

pkv_status paged_attention_chunk_workspace_bytes(const pkv_geom* geom, int32_t num_seqs,
                                                 int32_t num_tokens, int32_t max_context_len,
                                                 size_t* bytes) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (!bytes) return PKV_ERR_NULL;
  if (num_seqs < 0 || num_tokens < 0 || max_context_len < 0) return PKV_ERR_RANGE;
  *bytes = pkv::chunk_workspace_bytes(*geom, num_seqs, num_tokens, max_context_len);
  return PKV_OK;
}

pkv_status paged_attention_chunk_parts(const pkv_geom* geom, int32_t num_seqs,
                                      int32_t num_tokens, int32_t max_context_len,
                                      int32_t* parts) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (!parts) return PKV_ERR_NULL;
  if (num_seqs < 0 || num_tokens < 0 || max_context_len < 0) return PKV_ERR_RANGE;
  *parts = pkv::chunk_parts(*geom, num_tokens, max_context_len);
  return PKV_OK;
}

// Checks shared by paged_attention_chunk and its two halves (plan, run).
static pkv_status check_chunk_batch(const pkv_geom* geom, int32_t max_blocks_per_seq,
                                    const int32_t* cu_q_lens,
                                    const int32_t* chunk_start, int32_t num_seqs,
                                    int32_t num_tokens, int32_t max_q_len,
                                    int32_t max_context_len, void* workspace,
                                    size_t workspace_bytes) {
  if (!cu_q_lens || !chunk_start) return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || max_q_len < 1 || max_context_len < max_q_len ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return PKV_ERR_RANGE;
  const size_t need = pkv::chunk_workspace_bytes(*geom, num_seqs, num_tokens, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  return PKV_OK;
}

static pkv_status chunk_call(bool plan, bool run, const pkv_geom* geom, void* out,
                             int32_t out_dtype, const void* q, const void* k_arena,
                             const void* v_arena, const int32_t* block_table,
                             int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                             const int32_t* chunk_start, int32_t num_seqs, int32_t num_tokens,
                             int32_t max_q_len, int32_t max_context_len, float scale,
                             void* workspace, size_t workspace_bytes, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (run && out_dtype != PKV_F32) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_tokens < 0) return PKV_ERR_RANGE;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (run && (!out || !q || !k_arena || !v_arena || !block_table)) return PKV_ERR_NULL;
  st = check_chunk_batch(geom, max_blocks_per_seq, cu_q_lens, chunk_start, num_seqs,
                         num_tokens, max_q_len, max_context_len, workspace, workspace_bytes);
  if (st != PKV_OK) return st;
  if (!run)
    return hip_status(pkv::launch_chunk_plan(*geom, cu_q_lens, chunk_start, max_blocks_per_seq,
                                             num_seqs, num_tokens, max_q_len, workspace,
                                             workspace_bytes, (hipStream_t)stream));
  auto launch = plan ? pkv::launch_chunk : pkv::launch_chunk_run;
  return hip_status(launch(*geom, (float*)out, q, k_arena, v_arena, block_table,
                           max_blocks_per_seq, cu_q_lens, chunk_start, num_seqs, num_tokens,
                           max_q_len, max_context_len, scale, workspace, workspace_bytes,
                           (hipStream_t)stream));
}

pkv_status paged_attention_chunk(const pkv_geom* geom, void* out, int32_t out_dtype,
                                 const void* q, const void* k_arena, const void* v_arena,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* cu_q_lens, const int32_t* chunk_start,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                                 int32_t max_context_len, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return chunk_call(true, true, geom, out, out_dtype, q, k_arena, v_arena, block_table,
                    max_blocks_per_seq, cu_q_lens, chunk_start, num_seqs, num_tokens, max_q_len,
                    max_context_len, scale, workspace, workspace_bytes, stream);
}

pkv_status paged_attention_chunk_plan(const pkv_geom* geom, int32_t max_blocks_per_seq,
                                      const int32_t* cu_q_lens, const int32_t* chunk_start,
                                      int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                                      int32_t max_context_len, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return chunk_call(true, false, geom, nullptr, PKV_F32, nullptr, nullptr, nullptr, nullptr,
                    max_blocks_per_seq, cu_q_lens, chunk_start, num_seqs, num_tokens, max_q_len,
                    max_context_len, 1.f, workspace, workspace_bytes, stream);
}

pkv_status paged_attention_chunk_run(const pkv_geom* geom, void* out, int32_t out_dtype,
                                     const void* q, const void* k_arena, const void* v_arena,
                                     const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* cu_q_lens, const int32_t* chunk_start,
                                     int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                                     int32_t max_context_len, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return chunk_call(false, true, geom, out, out_dtype, q, k_arena, v_arena, block_table,
                    max_blocks_per_seq, cu_q_lens, chunk_start, num_seqs, num_tokens, max_q_len,
                    max_context_len, scale, workspace, workspace_bytes, stream);
}

pkv_status paged_attention_mixed_workspace_bytes(const pkv_geom* geom, int32_t num_seqs,
                                                 int32_t num_tokens, int32_t max_context_len,
                                                 size_t* bytes) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (!bytes) return PKV_ERR_NULL;
  if (num_seqs < 0 || num_tokens < 0 || max_context_len < 0) return PKV_ERR_RANGE;
  *bytes = pkv::mixed_workspace_bytes(*geom, num_seqs, num_tokens, max_context_len);
  return PKV_OK;
}

pkv_status paged_attention_mixed(const pkv_geom* geom, void* out, int32_t out_dtype,
                                 const void* q, const void* k_arena, const void* v_arena,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* cu_q_lens, const int32_t* chunk_start,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                                 int32_t max_context_len, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (out_dtype != PKV_F32) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_tokens < 0) return PKV_ERR_RANGE;
  if (num_seqs == 0 || num_tokens == 0) return PKV_OK;
  if (!out || !q || !k_arena || !v_arena || !block_table || !cu_q_lens || !chunk_start)
    return PKV_ERR_NULL;
  if (max_blocks_per_seq < 1 || max_q_len < 1 || max_context_len < max_q_len ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * PKV_BLOCK_SIZE)
    return PKV_ERR_RANGE;
  const size_t need = pkv::mixed_workspace_bytes(*geom, num_seqs, num_tokens, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  return hip_status(pkv::launch_mixed(*geom, (float*)out, q, k_arena, v_arena, block_table,
                                      max_blocks_per_seq, cu_q_lens, chunk_start, num_seqs,
                                      num_tokens, max_q_len, max_context_len, scale, workspace,
                                      workspace_bytes, (hipStream_t)stream));
}

pkv_status pkv_copy_blocks(const pkv_geom* geom, void* k_arena, void* v_arena,
                           const int32_t* src_dst, int32_t n, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (n < 0) return PKV_ERR_RANGE;
  if (n == 0) return PKV_OK;
  if (!k_arena || !v_arena || !src_dst) return PKV_ERR_NULL;
  return hip_status(pkv::launch_copy_blocks(*geom, k_arena, v_arena, src_dst, n,
                                            (hipStream_t)stream));
}

pkv_status pkv_swap_bytes(const pkv_geom* geom, int32_t n, size_t* bytes) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (!bytes) return PKV_ERR_NULL;
  if (n < 0) return PKV_ERR_RANGE;
  *bytes = (size_t)n * 2 * pkv::swap_tile_bytes(*geom);
  return PKV_OK;
}

static pkv_status swap_common(const pkv_geom* geom, void* k_arena, void* v_arena,
                              const int32_t* ids, int32_t n, void* buf, size_t buf_bytes,
                              bool swap_in, void* stream) {
  pkv_status st = check_geom(geom);
  if (st != PKV_OK) return st;
  if (n < 0) return PKV_ERR_RANGE;
  if (n == 0) return PKV_OK;
  if (!k_arena || !v_arena || !ids || !buf) return PKV_ERR_NULL;
  if (((uintptr_t)buf & 15) != 0) return PKV_ERR_RANGE;  // 16-byte units
  if (buf_bytes < (size_t)n * 2 * pkv::swap_tile_bytes(*geom)) return PKV_ERR_WORKSPACE;
  return hip_status(pkv::launch_swap_blocks(*geom, k_arena, v_arena, ids, n, buf, swap_in,
                                            (hipStream_t)stream));
}

pkv_status pkv_swap_out(const pkv_geom* geom, const void* k_arena, const void* v_arena,
                        const int32_t* ids, int32_t n, void* buf, size_t buf_bytes,
                        void* stream) {
  return swap_common(geom, (void*)k_arena, (void*)v_arena, ids, n, buf, buf_bytes, false,
                     stream);
}

pkv_status pkv_swap_in(const pkv_geom* geom, void* k_arena, void* v_arena, const int32_t* ids,
                       int32_t n, const void* buf, size_t buf_bytes, void* stream) {
  return swap_common(geom, k_arena, v_arena, ids, n, (void*)buf, buf_bytes, true, stream);
}

pkv_status pkv_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink) return PKV_ERR_NULL;
  if (bytes % 16 != 0 || ((uintptr_t)src & 15) != 0) return PKV_ERR_RANGE;
  return hip_status(pkv::launch_stream_read(src, bytes, sink, (hipStream_t)stream));
}

}  // extern "C"
