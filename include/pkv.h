/*
 * pkv.h — C ABI of libpkv: attention over a block-arena ("paged") KV cache with
 * grouped-query heads, for AMD MI355X (gfx950).
 *
 * Method: the Kshipra blog series, part 3 (blog/kshipra-3).  Section 1
 * "Block-Arena KV Cache": KV memory is reserved once as an arena of
 * fixed-size blocks handed out by a LIFO free list; no allocation per token.
 * Section 3 "Radix-Tree Prefix Cache": shared blocks are kept alive by
 * reference counts and a block that diverges is copied before it is written.
 * Section 4 "Chunked Prefill": attention over a chunk runs an online softmax
 * across KV blocks read in place from the arena; RoPE uses absolute positions
 * (a chunk after P cached tokens is rotated at P, P+1, ...); the causal mask
 * covers the chunk; the result equals dense masked attention.  Part 2
 * (blog/kshipra-2) section 1 "KV-Caching": a decode step appends the new token's
 * K/V and attends over the whole cache, the new token included.
 *
 * Conventions (every entry point):
 *   - Return value: PKV_OK, or an error code after host-side validation of
 *     pointers, geometry, dtypes, sizes and workspace.  Nothing is launched
 *     when an error is returned.  A failed kernel launch returns PKV_ERR_HIP.
 *   - Device pointers are owned by the caller.  The library never allocates or
 *     frees device memory, never synchronises the device, and launches only on
 *     `stream` (a hipStream_t; NULL = the default stream).  Calls are
 *     asynchronous with respect to the host unless stated otherwise.
 *   - Device-resident tables (block ids, lengths, positions) are the caller's
 *     contract and are not read by the host.  Kernels clamp every index they
 *     derive from them so that a bad table cannot address memory outside the
 *     buffers described here; the results for such rows are then unspecified.
 *     pkv_validate_tables() checks host copies of the tables.
 *   - Layouts (row-major, innermost index last), x = 16 / sizeof(element)
 *     (8 for fp16, 4 for fp32):
 *       K arena  [num_blocks][num_kv_heads][head_dim/x][16][x]  element d of the
 *                key in slot s at [d/x][s][d%x]: the 16 keys' 16-byte pieces of
 *                one head-dim range are contiguous
 *       V arena  [num_blocks][num_kv_heads][head_dim][16]       head-dim-major
 *     Position `pos` of a sequence whose block-table row is `bt` lives in
 *     physical block bt[pos / 16], slot pos % 16.  Query head h reads KV head
 *     h / (num_q_heads / num_kv_heads).
 *   - Positions are absolute and start at 0 for each sequence's first token
 *     (part 2, section 2 "Static Batching & the Left-Padding Position Bug").
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 1
#define PKV_BLOCK_SIZE 16

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,       /* a required pointer is NULL */
  PKV_ERR_SHAPE = 2,      /* geometry or size not supported / inconsistent */
  PKV_ERR_DTYPE = 3,      /* unsupported storage or output dtype */
  PKV_ERR_RANGE = 4,      /* an id, count or position out of range */
  PKV_ERR_WORKSPACE = 5,  /* workspace missing or smaller than required */
  PKV_ERR_NOMEM = 6,      /* block pool exhausted */
  PKV_ERR_REFCOUNT = 7,   /* reference count misuse (block not allocated) */
  PKV_ERR_HIP = 8         /* a HIP runtime call or kernel launch failed */
} pkv_status;

/* PKV_I8KV: q, k, v (inputs) and the rotated q are fp16; the arenas hold the
 * K and V of every (token, KV head) vector as INT8 codes with one fp16 scale
 * (part 3 section 2's group codec with group = one head vector of head_dim
 * values: s = fp16(fp32(max |x|) / 127), floored at 2^-24; code =
 * round-half-even(fp32(x) / fp32(s)); x_hat = code * s, |x - x_hat| <= s/2),
 * x being the value an fp16 arena would hold.  Tile of one (block, head):
 * 16 * head_dim + 32 bytes rounded up to a multiple of 128 (2176 at head_dim
 * 128), so every tile starts on a 128-byte line:
 *   K  int8 codes [head_dim/16][16][16] (16-byte pieces of 16 dims, the 16
 *      keys of a piece contiguous; the key of slot s sits at position s with
 *      bits 2 and 3 exchanged: positions 0..7 hold slots 0-3 and 8-11,
 *      positions 8..15 slots 4-7 and 12-15), then fp16 scales [16] (slot
 *      order), then padding
 *   V  int8 codes [head_dim][16] (slot order), then fp16 scales [16], then
 *      padding
 * Padding bytes are never written or read.  head_dim must be a multiple of 16.
 *
 * PKV_I4KV: the same with 4-bit codes (s = fp16(fp32(max |x|) / 7), codes in
 * [-7, 7], stored as their two's-complement low 4 bits, two per byte, low
 * nibble first).  Tile of one (block, head): 8 * head_dim codes bytes + 32,
 * rounded up to a multiple of 128 (1152 at head_dim 128):
 *   K  [head_dim/16 pieces][16 records][8 bytes]: the key of slot s has record
 *      2 r + u, r = 4 ((s >> 3) & 1) + (s & 3), u = (s >> 2) & 1; byte i of a
 *      record holds dims 16p + i (low) and 16p + 8 + i (high); then fp16
 *      scales [16] (slot order), then padding
 *   V  head dims in groups of 64 (the last of 32 if head_dim is not a
 *      multiple of 64); group j (G = 4 blocks of 16 dims, or 2) holds
 *      [half h][dim & 15][block (dim >> 4) & 3] words of 4 bytes at
 *      512 j + 4 ((16 h + (dim & 15)) G + ((dim >> 4) & 3)); byte i of the word
 *      of half h holds slots 8h + i (low) and 8h + 4 + i (high); then fp16
 *      scales [16], then padding
 * head_dim must be a multiple of 32. */
typedef enum pkv_dtype { PKV_F16 = 0, PKV_F32 = 1, PKV_I8KV = 2, PKV_I4KV = 3 } pkv_dtype;

/* Geometry of one layer's arena.  block_size must be 16; head_dim a multiple of
 * x (8 for fp16, 4 for fp32, 16 for PKV_I8KV, 32 for PKV_I4KV) and <= 256;
 * num_q_heads a multiple of num_kv_heads; dtype is the storage dtype of q, k,
 * v and both arenas (IEEE binary16 or binary32), or PKV_I8KV / PKV_I4KV (fp16
 * q/k/v, INT8 / INT4 arenas). */
typedef struct pkv_geom {
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t dtype; /* pkv_dtype */
} pkv_geom;

const char* pkv_status_string(pkv_status s);
int32_t pkv_abi_version(void);
/* SHA-256 (64 lowercase hex digits, NUL-terminated, static storage) of the
 * sources and compiler flags this library was built from: every file of the
 * kernel source folder, this header, and the flag set.  Bindings compare it
 * with a hash of the sources beside them and refuse a library built from
 * other sources. */
const char* pkv_source_hash(void);

/* ---------------------------------------------------------------------------
 * RoPE table (part 3, section 4: RoPE at absolute positions).
 * Rotate-half RoPE: element i pairs with i + D/2, angle pos * theta^(-2i/D).
 * Table layout: fp64 [max_pos][head_dim/2][2] = (cos, sin), computed on the host
 * in fp64 with the C library's pow/cos/sin.
 * ------------------------------------------------------------------------- */
pkv_status pkv_rope_table_bytes(int32_t head_dim, int32_t max_pos, size_t* bytes);
/* Fills a host buffer of pkv_rope_table_bytes() bytes. */
pkv_status pkv_rope_table_host(double* cos_sin, double theta, int32_t head_dim,
                               int32_t max_pos);
/* Fills a device buffer: builds the table on the host and copies it with a
 * synchronous copy on `stream` (set-up call, blocks the host until done). */
pkv_status pkv_rope_table_init(void* d_cos_sin, double theta, int32_t head_dim,
                               int32_t max_pos, void* stream);

/* ---------------------------------------------------------------------------
 * kv_append_rope — append new tokens to the arena (part 3 sections 1 and 4).
 * For every new token t of sequence b at absolute position
 *   pos = chunk_start[b] + (t - cu_q_lens[b]):
 *   q[t][h][:] (all query heads) and k (all KV heads) are rotated by RoPE at
 *   pos in fp64 (products and sums, no fused multiply-add) and rounded once,
 *   round-to-nearest-even, to the storage dtype; the rotated q goes to q_out;
 *   rotated k goes to the K arena, block bt[b][pos/16], slot pos%16, and v,
 *   unchanged, to the V arena, same block and slot.
 * q            device [num_tokens][Hq][D], read; may be NULL (cache fill
 *              without queries).
 * q_out        device [num_tokens][Hq][D] for the rotated queries; NULL or
 *              equal to q rotates q in place (no other overlap allowed).
 * k, v         device [num_tokens][Hkv][D], read only.
 * block_table  device int32 [num_seqs][max_blocks_per_seq].
 * cu_q_lens    device int32 [num_seqs+1], cu_q_lens[0] = 0, nondecreasing,
 *              cu_q_lens[num_seqs] = num_tokens (empty sequences allowed).
 * chunk_start  device int32 [num_seqs], first new position P_b of each sequence.
 * rope_table   device table of pkv_rope_table_init() for >= rope_max_pos
 *              positions.  Tokens whose position is >= rope_max_pos or past the
 *              block table are skipped (caller contract violation).
 * num_tokens == 0 or num_seqs == 0 is a no-op.
 * ------------------------------------------------------------------------- */
pkv_status kv_append_rope(const pkv_geom* geom, void* q, void* q_out, const void* k,
                          const void* v, void* k_arena, void* v_arena,
                          const int32_t* block_table,
                          int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                          const int32_t* chunk_start, int32_t num_seqs, int32_t num_tokens,
                          const void* rope_table, int32_t rope_max_pos, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_decode — one query token per sequence (part 2 section 1;
 * part 3 section 4's online-softmax merge over blocks read in place).
 * For sequence b with context length L = context_lens[b] (the new token,
 * already appended at position L-1, included) and each query head h:
 *   out[b][h][:] = softmax_j((q[b][h] . k_j) * scale) @ V,  j = 0 .. L-1.
 * Split-KV: each sequence's keys are cut into fixed 384-token splits processed
 * in parallel; splits are merged by their log-sum-exp.  The split size never
 * depends on the batch, so a sequence's result does not either.
 * out          device fp32 [num_seqs][Hq][D]  (out_dtype must be PKV_F32).
 * q            device [num_seqs][Hq][D], already rotated (kv_append_rope).
 * context_lens device int32 [num_seqs], 1 <= L <= max_context_len
 *              (rows with L <= 0 are written as zeros).
 * max_context_len  host upper bound of context_lens (sizes the grid and the
 *              workspace); must be <= max_blocks_per_seq * 16.
 * workspace    device scratch of paged_attention_decode_workspace_bytes()
 *              bytes (split partials); may be NULL when that size is 0.
 * scale        softmax scale, normally 1/sqrt(head_dim).
 * ------------------------------------------------------------------------- */
pkv_status paged_attention_decode_workspace_bytes(const pkv_geom* geom, int32_t num_seqs,
                                                  int32_t max_context_len, size_t* bytes);
pkv_status paged_attention_decode(const pkv_geom* geom, void* out, int32_t out_dtype,
                                  const void* q, const void* k_arena, const void* v_arena,
                                  const int32_t* block_table, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t max_context_len, float scale, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_decode_append — one decode step's append and attention in
 * one call (part 3 sections 1 and 4): for every sequence b, its new token at
 * position L - 1, L = context_lens[b], is appended as kv_append_rope does
 * (q[b] and k[b] rotated by RoPE at L - 1 in fp64 and rounded once to fp16;
 * the rotated q to q_out[b]; the rotated k and v[b] to the arena at block
 * bt[b][(L-1)/16], slot (L-1)%16, quantized with their scales for INT8 / INT4
 * arenas), and out[b] is paged_attention_decode's
 * result over positions 0 .. L-1 with the rotated q.  Outputs, q_out and the
 * arena bytes are bit for bit those of kv_append_rope (cu_q_lens = 0..num_seqs,
 * chunk_start = L - 1) followed by paged_attention_decode.
 * Arguments as kv_append_rope and paged_attention_decode, with q, k, v of one
 * token per sequence: q [num_seqs][Hq][D], k, v [num_seqs][Hkv][D], read only;
 * q_out [num_seqs][Hq][D] must not overlap q (PKV_ERR_RANGE).  The workspace
 * is paged_attention_decode's (paged_attention_decode_workspace_bytes()).
 * fp16, INT8 and INT4 arenas with head_dim 128 and 4 query heads per KV
 * head only (PKV_ERR_DTYPE for fp32 arenas, PKV_ERR_SHAPE for other shapes).
 * A position at or past
 * rope_max_pos skips the append and leaves q unrotated for the attention.
 * ------------------------------------------------------------------------- */
pkv_status paged_attention_decode_append(const pkv_geom* geom, void* out, int32_t out_dtype,
                                         const void* q, void* q_out, const void* k, const void* v,
                                         void* k_arena, void* v_arena, const int32_t* block_table,
                                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                                         int32_t num_seqs, int32_t max_context_len, float scale,
                                         const void* rope_table, int32_t rope_max_pos,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_decode_noalloc — paged_attention_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, result and
 * kernels as paged_attention_decode, without the workspace: the split
 * partials live in a static device array of PKV_DECODE_SCRATCH_BYTES inside
 * the library (one per GPU, held until the process ends; its address is
 * looked up on the first call on each device).  The call allocates nothing.
 * Returns PKV_ERR_WORKSPACE when paged_attention_decode_workspace_bytes() for
 * (num_seqs, max_context_len) exceeds PKV_DECODE_SCRATCH_BYTES (32 MiB: for
 * example 64 sequences of 32 query heads up to 11,904 tokens each).  Every
 * call on one GPU shares that array: calls that overlap on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 * ------------------------------------------------------------------------- */
#define PKV_DECODE_SCRATCH_BYTES (32u << 20)
pkv_status paged_attention_decode_noalloc(const pkv_geom* geom, void* out, int32_t out_dtype,
                                          const void* q, const void* k_arena,
                                          const void* v_arena, const int32_t* block_table,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t max_context_len, float scale, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_decode_shared — paged_attention_decode for a batch in which
 * groups of rows share a cached prefix (part 3 section 3: requests that share
 * a prefix reuse its blocks, kept alive by reference counts).  The shared
 * splits are read once for up to 4 rows at a time instead of once per row;
 * the result is bit for bit that of paged_attention_decode.
 * group_start  device int32 [num_groups+1], nondecreasing within
 *              [0, num_seqs]: group i is rows group_start[i] .. [i+1]-1.
 * row_skip     device int32 [num_seqs]: s_i for every row of group i, 0 for
 *              rows in no group.  Contract: the rows of group i have the same
 *              block-table entries for logical blocks 0 .. 24*s_i - 1 (the
 *              first s_i 384-token splits) and context lengths > 384*s_i.
 * max_skip     host bound of row_skip; max_group_size host bound of a group's
 *              row count.  Other arguments as for paged_attention_decode.
 * num_groups == 0 is plain paged_attention_decode.  Arenas other than fp16
 * with head_dim 128 and 4 query heads per KV head, and 3, 5, 6 or 7 KV heads
 * (whose workgroup of one wave per KV head holds 3, 5, 6 or 7 waves), compute
 * every split per row (same result).
 * ------------------------------------------------------------------------- */
pkv_status paged_attention_decode_shared(
    const pkv_geom* geom, void* out, int32_t out_dtype, const void* q, const void* k_arena,
    const void* v_arena, const int32_t* block_table, int32_t max_blocks_per_seq,
    const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len, float scale,
    const int32_t* group_start, const int32_t* row_skip, int32_t num_groups, int32_t max_skip,
    int32_t max_group_size, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_chunk — prefill chunks (part 3 section 4).
 * Sequence b has C_b = cu_q_lens[b+1] - cu_q_lens[b] new rows at absolute
 * positions P_b .. P_b + C_b - 1 (P_b = chunk_start[b]); its cached prefix and
 * the chunk itself are already in the arena (kv_append_rope).  Row i sees keys
 * j <= P_b + i: the whole prefix and the chunk up to and including itself.
 *   out[t][h][:] = softmax_j((q[t][h] . k_j) * scale) @ V over those keys.
 * out          device fp32 [num_tokens][Hq][D]  (out_dtype must be PKV_F32).
 * q            device [num_tokens][Hq][D], already rotated.
 * max_q_len    host upper bound of C_b; max_context_len host upper bound of
 *              P_b + C_b, <= max_blocks_per_seq * 16.
 * workspace    device memory of paged_attention_chunk_workspace_bytes()
 *              bytes (the schedule of the tuned kernel: one int32 per
 *              (sequence, 64-row tile); for a split call also the parts'
 *              partials, fp32 [parts][num_tokens][Hq][D + 2]);
 *              PKV_ERR_WORKSPACE if missing or short.
 * A call with fewer than 512 (64-row tile, KV head) work units (its rows
 * packed in whole tiles) splits every tile's keys into `parts` even ranges
 * (up to 8, each at least 768 keys of the longest context) and merges them by
 * log-sum-exp, so that small batches with long prefixes fill the chip.  Rows
 * of a split call then round differently (same tolerance) from an unsplit
 * one; paged_attention_chunk_parts() reports the number of parts the tuned
 * path uses for a call's sizes (1: not split; always 1 off the tuned path).
 * The tuned path takes fp16, INT8 and INT4 arenas at head_dim 128 with 4 query
 * heads per KV head, and scale > 0; other calls run the generic kernel
 * (fp32 arithmetic, one workgroup per row and query head, no workspace use).
 * ------------------------------------------------------------------------- */
pkv_status paged_attention_chunk_workspace_bytes(const pkv_geom* geom, int32_t num_seqs,
                                                 int32_t num_tokens, int32_t max_context_len,
                                                 size_t* bytes);
pkv_status paged_attention_chunk_parts(const pkv_geom* geom, int32_t num_seqs,
                                      int32_t num_tokens, int32_t max_context_len,
                                      int32_t* parts);
pkv_status paged_attention_chunk(const pkv_geom* geom, void* out, int32_t out_dtype,
                                 const void* q, const void* k_arena, const void* v_arena,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* cu_q_lens, const int32_t* chunk_start,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                                 int32_t max_context_len, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* paged_attention_chunk in two halves, for a step that runs the same batch
 * through several layers (part 3 section 5: a step's batch is fixed before
 * its layers run).  paged_attention_chunk_plan writes the tuned kernel's
 * schedule (the longest-first order of the (sequence, 64-row tile) items; it
 * orders work only and changes no result) into the workspace; it reads
 * cu_q_lens and chunk_start and takes the same sizes and checks as
 * paged_attention_chunk.  paged_attention_chunk_run takes
 * paged_attention_chunk's arguments and computes exactly what it computes
 * (bit for bit), over the schedule found in the workspace: it must follow a
 * plan call on the same stream with the same workspace, cu_q_lens,
 * chunk_start (contents too), num_seqs, num_tokens, max_q_len and
 * max_blocks_per_seq; q, the arenas, the block table's entries, out and scale
 * may change between runs.  A run over a schedule of another batch gives
 * undefined output rows, never an access outside the arguments' ranges
 * (entries outside the item range are skipped).  Off the tuned path the plan
 * does nothing and the run is the generic kernel.  Errors as for
 * paged_attention_chunk (the plan does not check q, out, the arenas or the
 * block table). */
pkv_status paged_attention_chunk_plan(const pkv_geom* geom, int32_t max_blocks_per_seq,
                                      const int32_t* cu_q_lens, const int32_t* chunk_start,
                                      int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                                      int32_t max_context_len, void* workspace,
                                      size_t workspace_bytes, void* stream);
pkv_status paged_attention_chunk_run(const pkv_geom* geom, void* out, int32_t out_dtype,
                                     const void* q, const void* k_arena, const void* v_arena,
                                     const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* cu_q_lens, const int32_t* chunk_start,
                                     int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                                     int32_t max_context_len, float scale, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * paged_attention_mixed — one continuous-batching step (part 3 section 5: each
 * step mixes prefill chunks and decode tokens under a token budget) in one
 * attention launch.  Arguments, layouts and result are those of
 * paged_attention_chunk; a sequence with C_b = 1 is a decode (its row sees
 * keys 0 .. P_b, computed in 384-token splits exactly as
 * paged_attention_decode computes a row of context P_b + 1), a sequence with
 * C_b >= 2 a prefill chunk (computed exactly as paged_attention_chunk does
 * without splitting keys).  Results are bit for bit those of the two
 * stand-alone calls whenever paged_attention_chunk_parts() is 1 for the
 * chunk call.
 * workspace    device memory of paged_attention_mixed_workspace_bytes()
 *              bytes: the schedule and the decode partials.  Sized from
 *              num_seqs, num_tokens and max_context_len; PKV_ERR_WORKSPACE if
 *              missing or short.
 * Other shapes (not fp16, INT8 or INT4 storage / head_dim 128 / 4 query heads
 * per KV head) run the generic kernel over every row, as paged_attention_chunk
 * does.
 * ------------------------------------------------------------------------- */
pkv_status paged_attention_mixed_workspace_bytes(const pkv_geom* geom, int32_t num_seqs,
                                                 int32_t num_tokens, int32_t max_context_len,
                                                 size_t* bytes);
pkv_status paged_attention_mixed(const pkv_geom* geom, void* out, int32_t out_dtype,
                                 const void* q, const void* k_arena, const void* v_arena,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* cu_q_lens, const int32_t* chunk_start,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_q_len,
                                 int32_t max_context_len, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_copy_blocks — the copy of copy-on-write (part 3 section 3): for each
 * pair i, block src_dst[2i] is copied bit for bit onto block src_dst[2i+1] in
 * both arenas (all KV heads, all 16 slots).  src_dst: device int32 [n][2];
 * pairs whose ids are out of range are skipped.  Destinations must be distinct
 * and must not be sources of other pairs in the same call.
 * ------------------------------------------------------------------------- */
pkv_status pkv_copy_blocks(const pkv_geom* geom, void* k_arena, void* v_arena,
                           const int32_t* src_dst, int32_t n, void* stream);

/* ---------------------------------------------------------------------------
 * pkv_swap_out / pkv_swap_in — preemption by swapping (part 3 section 5: when
 * memory is short a running sequence is preempted; recomputing its KV cache
 * is too expensive, so its blocks are swapped out of the arena and restored
 * later).
 * pkv_swap_out copies, bit for bit, block ids[i]'s K tile and V tile (all KV
 * heads, all 16 slots) to buf at byte offset i * 2T (K tile) and
 * i * 2T + T (V tile), T = num_kv_heads * 16 * head_dim * element size;
 * pkv_swap_in copies them back into block ids[i] of the arenas.  The arena
 * layouts are unchanged, so a sequence restored into different blocks is the
 * same sequence once its block-table row names the new ids.
 * ids        device int32 [n]; ids outside [0, num_blocks) are skipped (their
 *            buf slots are left unchanged / their tiles are not written).
 *            Swap-in ids must be distinct.
 * buf        device-accessible memory of pkv_swap_bytes(n) bytes, 16-byte
 *            aligned: pinned host memory (hipHostMalloc) for a swap to the
 *            host, or device memory.  buf_bytes is its size.
 * PKV_ERR_WORKSPACE if buf_bytes is too small; PKV_ERR_RANGE if buf is not
 * 16-byte aligned.  Asynchronous on `stream`; the caller synchronises before
 * reading buf on the host or reusing the swapped-out blocks.
 * ------------------------------------------------------------------------- */
pkv_status pkv_swap_bytes(const pkv_geom* geom, int32_t n, size_t* bytes);
pkv_status pkv_swap_out(const pkv_geom* geom, const void* k_arena, const void* v_arena,
                        const int32_t* ids, int32_t n, void* buf, size_t buf_bytes,
                        void* stream);
pkv_status pkv_swap_in(const pkv_geom* geom, void* k_arena, void* v_arena, const int32_t* ids,
                       int32_t n, const void* buf, size_t buf_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Host block pool (part 3 sections 1 and 3).  The free list starts as
 * [0, 1, ..., N-1]; allocation pops from its end (highest id first); a block
 * whose count drops to 0 is pushed on the end and is the next one allocated.
 * Not thread-safe; owned by the caller.
 * ------------------------------------------------------------------------- */
typedef struct pkv_pool pkv_pool;
pkv_pool* pkv_pool_create(int32_t num_blocks);          /* NULL if num_blocks < 1 */
void pkv_pool_destroy(pkv_pool* pool);
pkv_status pkv_pool_alloc(pkv_pool* pool, int32_t* id); /* count := 1; NOMEM if empty */
/* n allocations in a row; all-or-nothing (NOMEM leaves the pool unchanged). */
pkv_status pkv_pool_alloc_n(pkv_pool* pool, int32_t n, int32_t* ids);
pkv_status pkv_pool_incref(pkv_pool* pool, int32_t id); /* share one more time */
pkv_status pkv_pool_decref(pkv_pool* pool, int32_t id); /* at 0: back on the free list */
/* Copy-on-write decision: if id is shared (count > 1) a fresh block is popped
 * (*out_id), one reference to id is dropped and *copied = 1 — the caller then
 * copies the data (pkv_copy_blocks); otherwise *out_id = id, *copied = 0. */
pkv_status pkv_pool_cow(pkv_pool* pool, int32_t id, int32_t* out_id, int32_t* copied);
int32_t pkv_pool_num_free(const pkv_pool* pool);
int32_t pkv_pool_refcount(const pkv_pool* pool, int32_t id); /* -1 if out of range */
/* Copies the free list, bottom first, into out[0..cap); *n = its length. */
pkv_status pkv_pool_free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n);
/* Admission rule of continuous batching (part 3 section 5): a new sequence
 * needing new_need blocks is admitted only if
 *   free + evictable >= active_reserved + new_need,
 * free = the pool's free blocks, evictable = blocks the prefix cache could
 * release, active_reserved = blocks the running sequences still have to
 * allocate to finish.  Returns 1 (admit), 0 (do not), -1 (NULL pool or a
 * negative count). */
int32_t pkv_pool_can_admit(const pkv_pool* pool, int64_t evictable, int64_t active_reserved,
                           int64_t new_need);

/* ---------------------------------------------------------------------------
 * Radix-tree prefix cache over the pool's blocks (part 3 section 3: KV blocks
 * live in a radix tree keyed by token blocks; a new request reuses every
 * matching block; reference counts keep shared blocks alive; under memory
 * pressure the least recently used leaf is evicted, the tree being re-scanned
 * on every iteration so a parent that becomes a leaf is considered).
 * A node is one full block of 16 token ids; the tree owns one reference to
 * its block.  Host-only, not thread-safe; the pool must outlive the tree.
 * ------------------------------------------------------------------------- */
typedef struct pkv_radix pkv_radix;
pkv_radix* pkv_radix_create(pkv_pool* pool);  /* NULL if pool is NULL */
void pkv_radix_destroy(pkv_radix* r);          /* drops the tree's references */
/* Longest cached prefix of whole blocks of tokens[0..n): writes up to cap of
 * its block ids to blocks and returns its length in blocks (-1 on bad
 * arguments).  Marks the matched nodes as used now; takes no reference (a
 * request adopting the blocks increfs them). */
int32_t pkv_radix_match(pkv_radix* r, const int32_t* tokens, int32_t n, int32_t* blocks,
                        int32_t cap);
/* Caches the n / 16 whole blocks of tokens[0..n), held in blocks[i] (live
 * pool blocks): each block not yet in the tree becomes a node and the tree
 * increfs it; existing nodes keep their block.  All-or-nothing on
 * PKV_ERR_RANGE / PKV_ERR_REFCOUNT (a new block id out of range or free). */
pkv_status pkv_radix_insert(pkv_radix* r, const int32_t* tokens, int32_t n,
                            const int32_t* blocks);
/* Frees up to target blocks, one least recently used evictable leaf at a time
 * (a leaf whose block the tree alone holds; ties: older node first); returns
 * how many were freed (-1 on bad arguments). */
int32_t pkv_radix_evict(pkv_radix* r, int32_t target);
/* Blocks repeated eviction could free: nodes the tree alone holds whose
 * whole subtree is evictable (the "evictable" of pkv_pool_can_admit). */
int32_t pkv_radix_evictable(const pkv_radix* r);
int32_t pkv_radix_num_nodes(const pkv_radix* r);

/* Host check of table copies: every row with length L > 0 needs
 * ceil(L/16) <= max_blocks_per_seq entries, each in [0, num_blocks). */
pkv_status pkv_validate_tables(const pkv_geom* geom, const int32_t* h_block_table,
                               int32_t max_blocks_per_seq, const int32_t* h_lens,
                               int32_t num_seqs);

/* The library's fp64 -> fp16 rounding (round-to-nearest-even, subnormals,
 * overflow to infinity), the same routine kv_append_rope uses on the device,
 * run on the host: n values from x to out (IEEE binary16 bit patterns). */
pkv_status pkv_f64_to_f16_host(const double* x, uint16_t* out, int64_t n);

/* ---------------------------------------------------------------------------
 * Measurement helper (not a step of the attention path): reads `bytes` of the
 * device buffer `src` once with the 16-byte non-temporal loads the decode
 * kernels use for K/V, on `stream`, so a benchmark can time the achievable
 * HBM read rate beside their rooflines.  src: device, 16-byte aligned;
 * bytes: a multiple of 16; sink: device, at least 4 bytes, written only for
 * one data-dependent value (it keeps the loads live).  Returns PKV_ERR_NULL /
 * PKV_ERR_RANGE on bad arguments, PKV_ERR_HIP on a launch failure.
 * ------------------------------------------------------------------------- */
pkv_status pkv_stream_read(const void* src, size_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */
