// paged_attention_decode: one query token per sequence over its block-arena
// KV cache (Kshipra part 2, section 1: decode attends over the cache holding
// the new token too; part 3, section 4: online-softmax merge over KV blocks read
// in place through the block table, out = o / l).
//
// Tuned path (fp16 storage, head_dim 128, 4 query heads per KV head — the
// Llama-3-8B layer shape):
//   * split-KV: the keys of each sequence are cut into fixed 384-token splits
//     (24 arena blocks); one 64-lane wavefront per (sequence, KV head, split)
//     serves all 4 query heads of the group, so each K/V byte is read once;
//     the waves of all KV heads of one (sequence, split) form one workgroup;
//   * per pair of blocks (32 tokens) the two small contractions, S = q . K^T
//     ([4 heads x 128] . [128 x 32]) and o += P . V, run on the fp16 matrix
//     cores (v_mfma_f32_16x16x32_f16, fp32 accumulation).  This is not to
//     reach matrix-core throughput (4 of the 16 MFMA columns carry heads): it
//     takes the multiply-adds, fp16 conversions and cross-lane traffic off the
//     vector ALUs and LDS, which otherwise sit at ~50% busy at full HBM rate;
//   * K and V tiles go from HBM straight into operand registers with
//     non-temporal loads: per instruction the wave reads 1 KiB contiguous of a
//     K tile (the arena keeps K in 16-byte pieces grouped by piece) and 512 B
//     contiguous of a head-dim-major V tile; the next pair is in flight while
//     the current one is computed, and the split's block-table entries are
//     fetched once into a register up front;
//   * the grid's split dimension is padded to an odd width so that a given
//     split index is not pinned to the same XCDs (workgroups are dealt to the
//     8 XCDs round-robin by linear id): otherwise the XCDs that always draw
//     split 0 carry far more work than those drawing high split indices;
//   * online softmax in fp32 on scores in log2 units; accumulators are
//     rescaled only when some head's running max moved; P is rounded to fp16
//     for the second product and the denominator sums those rounded values;
//   * a split writes its unnormalised (o, m, l); a second kernel merges the
//     splits of each (sequence, head) by their log-sum-exp.  A sequence that
//     fits one split is normalised and written by the split kernel directly.
//     (Merging inside the split kernel — the last split to finish, found with
//     an atomic counter — needs device-scope release/acquire fences, which on
//     this multi-XCD part write back and invalidate the L2 per wave; measured
//     4x slower than the second launch.)
// Other shapes run the generic kernel.
#include <mutex>

#include "decode_core.h"
#include "decode_q_core.h"
#include "lds_dma.h"

namespace pkv {
namespace {

__global__ __launch_bounds__(64 * kDecodeWavesPerWG, PKV_DECODE_WAVES_PER_SIMD) void decode_split_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q,
    const _Float16* __restrict__ k_arena, const _Float16* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ context_lens, float scale_log2, int Hkv, int nsplit_max,
    int num_blocks) {
  const int split = blockIdx.x, b = blockIdx.y;
  const int g = blockIdx.z * kDecodeWavesPerWG + (threadIdx.x >> 6);
  if (g >= Hkv) return;
  decode_split_unit(out, ws_o, ws_ml, q, k_arena, v_arena, block_table, max_blocks, b, b,
                    context_lens, 0, scale_log2, Hkv, nsplit_max, num_blocks, split, g);
}

// The same split units with the step's append fused in (fp16 arenas): each
// wave rotates its query and the new key at position L - 1 itself, split 0
// writes the rotated queries, and the last split writes the new key and value
// to the arena and takes them from registers for its last pair.
__global__ __launch_bounds__(64 * kDecodeWavesPerWG, PKV_DECODE_WAVES_PER_SIMD) void decode_split_append_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ context_lens, float scale_log2, int Hkv, int nsplit_max,
    int num_blocks, DecodeAppend app) {
  const int split = blockIdx.x, b = blockIdx.y;
  const int g = blockIdx.z * kDecodeWavesPerWG + (threadIdx.x >> 6);
  if (g >= Hkv) return;
  decode_split_unit<true, true>(out, ws_o, ws_ml, nullptr, app.k_arena, app.v_arena, block_table,
                                max_blocks, b, b, context_lens, 0, scale_log2, Hkv, nsplit_max,
                                num_blocks, split, g, app);
}

// ---- splits shared by several sequences ---------------------------------------
// Kshipra part 3, section 3: sequences that share a cached prefix share its
// physical blocks.  For a group of rows whose first `skip` splits are the same
// blocks, decode_shared_kernel reads each of those splits once for up to 4
// rows at a time: the 16 columns of the first product, of which the per-row
// kernel fills 4 (one row's 4 query heads), carry 4 rows x 4 heads.  Column
// ln is row 4 * quad + (ln >> 2), head ln & 3.  Every column is computed with
// the same instructions, operand layouts and order as the per-row kernel, so
// the partials -- and the merged output -- are bit for bit those of
// paged_attention_decode.  All keys of a shared split are real (a member's
// own token comes after the shared prefix), so there is no mask.
//
// A shared workgroup serves kHeads KV heads x kQuads quads of one shared split
// (kWaves = kHeads * kQuads waves; wave w: head slot w / kQuads, quad slot
// w % kQuads).  Each pair of blocks of its heads travels once from memory into
// a kStages-deep LDS ring (direct-to-LDS loads, kDma per wave and pair) and
// every quad's wave reads its operands from there, into the registers and
// layouts the per-row kernel loads them to; the quads of a head share one
// read from L2 instead of each fetching it.  Stage layout, per head slot:
// the K tiles of blocks A and B as in the arena, then the V tiles of A and B
// as [16-dim group][8-key half][dim & 15] (16-byte units), so that a wave's
// 8-byte V reads (keys 4 lq .. 4 lq + 3 of dims 16 db + ln) cover 256
// contiguous bytes per 32 lanes.
template <int kWaves>
struct SharedGeom {
  static constexpr int kQuads = kWaves < 4 ? kWaves : 4;
  static constexpr int kHeads = kWaves / kQuads;
  static constexpr int kTile = kBlock * kD * 2;  // one (block, KV head) K or V tile
  static constexpr int kStage = kHeads * 4 * kTile;
  static constexpr int kStages = kWaves >= 4 ? 4 : 3;
  static constexpr int kLds = kStages * kStage;
  static constexpr int kDma = kStage / 1024 / kWaves;  // 1 KiB per load instruction
  static_assert(kDma * 1024 * kWaves == kStage, "whole loads per wave");
  static_assert(kLds <= 160 * 1024, "fits a CU's LDS");
};

// LDS byte offset, within a stage, of the V unit (dim, half) of tile slot t
// (4 * head slot + 2 + block); the load side places source unit
// 2 * dim + half there.
__host__ __device__ constexpr int shared_v_unit(int dim, int half) {
  return ((dim >> 4) * 32 + half * 16 + (dim & 15)) * 16;
}

// Every staged load lands inside the LDS array, and every operand read of a
// stage stays inside the tile it means to read.
template <int kWaves>
constexpr bool shared_lds_in_bounds() {
  using SG = SharedGeom<kWaves>;
  for (int st = 0; st < SG::kStages; ++st)
    for (int w = 0; w < kWaves; ++w)
      for (int e = 0; e < SG::kDma; ++e) {
        const int n = w * SG::kDma + e, t = n >> 2;
        if (t >= 4 * SG::kHeads) return false;
        const int at = st * SG::kStage + t * SG::kTile + (n & 3) * 1024;
        if (at < 0 || at + 64 * 16 > SG::kLds) return false;
      }
  for (int lq = 0; lq < 4; ++lq)
    for (int ln = 0; ln < 16; ++ln) {
      for (int kd = 0; kd < 4; ++kd) {
        const int off = ((4 * kd + lq) * kBlock + ln) * 16;
        if (off < 0 || off + 16 > SG::kTile) return false;
      }
      for (int db = 0; db < 8; ++db) {
        const int off = shared_v_unit(16 * db + ln, lq >> 1) + 8 * (lq & 1);
        if (off < 0 || off + 8 > SG::kTile) return false;
      }
    }
  return true;
}
static_assert(shared_lds_in_bounds<1>() && shared_lds_in_bounds<2>() &&
                  shared_lds_in_bounds<4>() && shared_lds_in_bounds<8>(),
              "shared decode LDS layout");

template <int kWaves>
__device__ __forceinline__ void decode_shared_unit(
    u32x4* __restrict__ lds, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const _Float16* __restrict__ k_arena,
    const _Float16* __restrict__ v_arena, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ group_start, const int32_t* __restrict__ row_skip,
    float scale_log2, int Hkv, int nsplit_max, int num_blocks, int hgroups, int num_seqs,
    int nshared, int qgroups, int u) {
  using SG = SharedGeom<kWaves>;
  // Unit u = ((group * hgroups + hgroup) * nshared + split) * qgroups + qgroup:
  // the workgroups of a split are consecutive units (the kernel deals them to
  // one or two XCDs, whose L2s then fetch the split's blocks once each).
  const int qg = u % qgroups;
  u /= qgroups;
  const int split = u % nshared;
  u /= nshared;
  const int hg = u % hgroups, gi = u / hgroups;
  // rows of the group, clamped to the batch (a bad table cannot address
  // memory outside the buffers); the group's skip is the same for all waves
  const int r0 = max(0, group_start[gi]), r1 = min(num_seqs, group_start[gi + 1]);
  if (r0 >= r1) return;
  const int skip = min(row_skip[r0], nsplit_max);
  if (split >= skip) return;
  // From here on every wave runs the whole loop (it holds barriers); a wave
  // whose head or rows do not exist computes on clamped inputs and stores
  // nothing.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hs = wave / SG::kQuads, quad = qg * SG::kQuads + wave % SG::kQuads;
  const int g = hg * SG::kHeads + hs;
  const bool head_ok = g < Hkv;
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, lq = lane >> 4;
  const int Hq = Hkv * kG;
  const int blk0 = split * kSB;
  const int first = r0 + 4 * quad;
  const int row = first + (ln >> 2);  // this column's sequence
  const bool col_ok = head_ok && row < r1;
  int my_blk = 0;
  if (lane < kSB && blk0 + lane < max_blocks)
    my_blk = block_table[(size_t)r0 * max_blocks + blk0 + lane];  // the group's shared blocks
  if (my_blk < 0 || my_blk >= num_blocks) my_blk = 0;
  half8_t qb[4];
#pragma unroll
  for (int kd = 0; kd < 4; ++kd)
    qb[kd] = col_ok ? *(const half8_t*)(q + ((size_t)row * Hq + g * kG + (ln & 3)) * kD + 32 * kd + 8 * lq)
                    : (half8_t)(_Float16)0.f;
  // the queries and block ids are in before the first tile load (the
  // compiler does not see those loads; its waits would otherwise cover them)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  constexpr int npairs = kSB / 2;  // a shared split is whole

  // Loads of pair p into stage p % kStages: load n of the stage (1 KiB) is
  // quarter n & 3 of tile slot n >> 2 (head slot t >> 2; K A, K B, V A, V B);
  // wave w issues loads w * kDma .. +kDma.
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4*)lds;
  auto issue = [&](int p) {
    const int stage = p % SG::kStages;
    const int ba = __builtin_amdgcn_readlane(my_blk, 2 * p), bb = __builtin_amdgcn_readlane(my_blk, 2 * p + 1);
#pragma unroll
    for (int e = 0; e < SG::kDma; ++e) {
      const int n = wave * SG::kDma + e;
      const int t = n >> 2, quarter = n & 3;
      const int gl = min(hg * SG::kHeads + (t >> 2), Hkv - 1);  // clamped head of the slot
      const int kind = t & 3;
      const int blk = (kind & 1) ? bb : ba;
      const _Float16* tile = (kind < 2 ? k_arena : v_arena) + ((size_t)blk * Hkv + gl) * (kBlock * kD);
      const int pos = quarter * 64 + lane;  // 16-byte unit of the staged tile
      int src = pos;                        // K: as in the arena
      if (kind >= 2) {                      // V: [dim group][half][dim & 15]
        const int dim = (pos >> 5) * 16 + (pos & 15), half = (pos >> 4) & 1;
        src = 2 * dim + half;
      }
      dma16(tile + 8 * src,
            __builtin_amdgcn_readfirstlane(lds_base + stage * SG::kStage + t * SG::kTile + quarter * 1024));
    }
  };

  f32x4 o[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) o[db] = (f32x4)0.f;
  float m_run = -INFINITY, l_run = 0.f;

  auto compute = [&](const Pair& pr) {
    f32x4 s[2];
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
      s[u2] = (f32x4)0.f;
#pragma unroll
      for (int kd = 0; kd < 4; ++kd)
        s[u2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pr.k[u2][kd], qb[kd], s[u2], 0, 0, 0);
    }
    // same rounding steps as decode_split_kernel: max of raw scores scaled
    // once, exponent fma(score, scale_log2, -m)
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, s[e >> 2][e & 3]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
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
      const _Float16 ph =
          (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[e >> 2][e & 3], scale_log2, -m_new));
      pb[e] = ph;
      lsum += (float)ph;
    }
    l_run += lsum;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pr.v[db], pb, o[db], 0, 0, 0);
  };

  // The operands of pair p from its stage, in load_pair's registers and order.
  auto read_pair = [&](int p) {
    const char* st = (const char*)lds + (p % SG::kStages) * SG::kStage + 4 * hs * SG::kTile;
    Pair pr;
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) {
      const int off = ((4 * kd + lq) * kBlock + ln) * 16;
      pr.k[0][kd] = *(const half8_t*)(st + off);
      pr.k[1][kd] = *(const half8_t*)(st + SG::kTile + off);
    }
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int off = shared_v_unit(16 * db + ln, lq >> 1) + 8 * (lq & 1);
      const u32x2 lo = *(const u32x2*)(st + 2 * SG::kTile + off);
      const u32x2 hi = *(const u32x2*)(st + 3 * SG::kTile + off);
      pr.v[db] = __builtin_bit_cast(half8_t, u32x4{lo.x, lo.y, hi.x, hi.y});
    }
    return pr;
  };

#pragma unroll
  for (int p = 0; p < SG::kStages - 1; ++p)
    if (p < npairs) issue(p);
#pragma unroll
  for (int p = 0; p < npairs; ++p) {
    // this wave's loads of pair p are in (pairs p + 1 .. p + kStages - 2 may
    // be in flight); after the barrier every wave's are, and every wave is
    // done reading pair p - 1, whose stage the next load reuses
    constexpr int kAhead = SG::kStages - 2;
    const int inflight = min(kAhead, npairs - 1 - p);
    if (inflight >= 2) wait_vm<2 * SG::kDma>();
    else if (inflight == 1) wait_vm<SG::kDma>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (p + SG::kStages - 1 < npairs) issue(p + SG::kStages - 1);
    compute(read_pair(p));
  }

  float l_row = l_run;
  l_row += __shfl_xor(l_row, 16);
  l_row += __shfl_xor(l_row, 32);
  if (col_ok) {
    const size_t part = ((size_t)row * nsplit_max + split) * Hq + g * kG + (ln & 3);
    float* dst = ws_o + part * kD + 4 * lq;
#pragma unroll
    for (int db = 0; db < 8; ++db) *(f32x4*)(dst + 16 * db) = o[db];
    if (lq == 0) {
      ws_ml[2 * part] = m_run;
      ws_ml[2 * part + 1] = l_row;
    }
  }
}

// One launch for a batch with shared splits: the shared units
// (decode_shared_unit) and every row's own splits (those from its skip on),
// run as decode_split_kernel runs them.  Both kinds run side by side: either
// alone is a chain of up to 12 dependent pairs per wave with little of the
// chip busy when groups are few.  Every unit runs the code of the separate
// kernels, so partials and outputs are those of paged_attention_decode.  All
// its K/V loads are cached (the split kernel streams): the shared units of a
// split and the rows' own splits that still hold the end of the shared prompt
// read the same blocks close in time.
//
// Grid order.  Workgroups are handed out in linear-id order, id i to XCD
// i mod 8, and an XCD with no free compute unit holds up the hand-out of
// every later workgroup (measured: with the shared units' XCD set to
// split mod 8, the two XCDs drawing two splits each were full, and every
// own-split workgroup, ids after them, started only when their shared units
// ended, serialising the two kinds).  So:
//   * the first nsplit_max * n0 workgroups (n0 = num_seqs * zheads) take the
//     rows' own splits: own split k of row b for KV-head group z in the order
//     (k, z, b), b fastest (all rows' first own splits, then second ones, ...;
//     k past a row's splits only exits);
//   * the last 8 per (per = ceil(n_shared / 8)) take the shared units, the
//     i-th of them unit (i mod 8) * per + i / 8: each XCD runs a run of
//     consecutive units, i.e. an even share, and a split's workgroups fall
//     on one or two XCDs.
// When the units outnumber the compute units, the ones left waiting are
// shared units, all of one length, and they start as a row's short last
// split ends (measured on the shared workload, 160 shared and ~126 own
// units: with the shared units before the rows' later splits, long later
// splits waited for free compute units and ended at ~40 us; 8 of the 10 us
// of that tail go with this order).
template <int kWaves>
__global__ __launch_bounds__(64 * kWaves, PKV_DECODE_WAVES_PER_SIMD) void decode_shared_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const _Float16* __restrict__ k_arena,
    const _Float16* __restrict__ v_arena, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ group_start,
    const int32_t* __restrict__ row_skip, float scale_log2, int Hkv, int nsplit_max,
    int num_blocks, int zheads, int num_seqs, int nshared, int hgroups, int qgroups,
    int n_shared, int per) {
  __shared__ u32x4 lds[SharedGeom<kWaves>::kLds / 16];
  const int n_own = nsplit_max * num_seqs * zheads;
  const int j = blockIdx.x;
  if (j >= n_own) {
    const int i = j - n_own;
    const int u = (i & 7) * per + (i >> 3);
    if (u < n_shared)
      decode_shared_unit<kWaves>(lds, ws_o, ws_ml, q, k_arena, v_arena, block_table, max_blocks,
                                 group_start, row_skip, scale_log2, Hkv, nsplit_max, num_blocks,
                                 hgroups, num_seqs, nshared, qgroups, u);
    return;
  }
  const int b = j % num_seqs, rest = j / num_seqs;
  const int z = rest % zheads, k = rest / zheads;
  const int g = z * kWaves + (threadIdx.x >> 6);
  const int split = min(max(row_skip[b], 0), nsplit_max) + k;
  if (g >= Hkv || split >= nsplit_max) return;
  decode_split_unit<false>(out, ws_o, ws_ml, q, k_arena, v_arena, block_table, max_blocks, b, b,
                    context_lens, 0, scale_log2, Hkv, nsplit_max, num_blocks, split, g);
}

// ---- INT8 arenas (PKV_I8KV) -------------------------------------------------
// Same split-KV structure for arenas holding INT8 codes with one fp16 scale per
// (token, KV head) vector (tile: codes, then 16 scales).  Half the bytes per
// token, so twice the tokens per second at the same HBM rate.
//   * K rows of the first product are permuted: row m of MFMA u is token
//     8((m >> 2) & 1) + 4u + (m & 3) of block A (m < 8) or B (m >= 8), so a
//     lane's 8 scores for head ln are 8 consecutive tokens of one block -- one
//     8-byte load of V codes per head dim.  The head dims of the contraction
//     are permuted too (MFMA kd, lane group lq: dims 16(4(kd >> 1) + lq) +
//     8(kd & 1) .. +8), so one 16-byte load of K codes feeds two MFMAs; the
//     queries are loaded in the same order.  The arena stores the tokens an
//     MFMA reads together contiguously (i8_kpos) and pads tiles to whole
//     128-byte lines, so every load instruction reads whole lines (measured
//     16% faster than the unpadded slot-order layout).
//   * codes become fp16 exactly (byte b: fp16 bits 0x6400 | (b ^ 0x80) =
//     1024 + b + 128, minus 1152), the K scale multiplies the score, and the V
//     scale is folded into the probability: P^T holds fp16(p * s_v * boost),
//     the boost keeping small weights out of fp16 subnormals (undone at the
//     end).  With p <= 1 and s_v <= 65504 / qmax the product stays below
//     fp16's largest finite value: boost 2^6 for INT8 (s_v <= 516), 2^2 for
//     INT4 (s_v <= 9358).
__global__ __launch_bounds__(64 * kI8WavesPerWG, PKV_DECODE_I8_WAVES_PER_SIMD) void decode_split_i8_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const uint8_t* __restrict__ k_arena,
    const uint8_t* __restrict__ v_arena, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ context_lens, float scale_log2, int Hkv, int nsplit_max,
    int num_blocks) {
  const int g = blockIdx.z * kI8WavesPerWG + (threadIdx.x >> 6);
  if (g >= Hkv) return;
  decode_split_q_unit<CodesI8>(out, ws_o, ws_ml, q, k_arena, v_arena, block_table, max_blocks,
                               blockIdx.y, blockIdx.y, context_lens, 0, scale_log2, Hkv,
                               nsplit_max, num_blocks, blockIdx.x, g);
}

__global__ __launch_bounds__(64 * kI8WavesPerWG, PKV_DECODE_I4_WAVES_PER_SIMD) void decode_split_i4_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    const _Float16* __restrict__ q, const uint8_t* __restrict__ k_arena,
    const uint8_t* __restrict__ v_arena, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ context_lens, float scale_log2, int Hkv, int nsplit_max,
    int num_blocks) {
  const int g = blockIdx.z * kI8WavesPerWG + (threadIdx.x >> 6);
  if (g >= Hkv) return;
  decode_split_q_unit<CodesI4>(out, ws_o, ws_ml, q, k_arena, v_arena, block_table, max_blocks,
                               blockIdx.y, blockIdx.y, context_lens, 0, scale_log2, Hkv,
                               nsplit_max, num_blocks, blockIdx.x, g);
}

// The fused decode step over INT8 / INT4 arenas: the same split units, each
// wave rotating its query at L - 1 (split 0 writing it out), the last split's
// wave quantizing the new key and value into the arena before it reads its
// pairs (decode_split_q_unit with kAppend).
__global__ __launch_bounds__(64 * kI8WavesPerWG, PKV_DECODE_I8_WAVES_PER_SIMD) void decode_split_append_i8_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    uint8_t* k_arena, uint8_t* v_arena, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ context_lens, float scale_log2, int Hkv, int nsplit_max,
    int num_blocks, DecodeAppend app) {
  const int g = blockIdx.z * kI8WavesPerWG + (threadIdx.x >> 6);
  if (g >= Hkv) return;
  decode_split_q_unit<CodesI8, true>(out, ws_o, ws_ml, nullptr, k_arena, v_arena, block_table,
                                     max_blocks, blockIdx.y, blockIdx.y, context_lens, 0,
                                     scale_log2, Hkv, nsplit_max, num_blocks, blockIdx.x, g, app);
}

__global__ __launch_bounds__(64 * kI8WavesPerWG, PKV_DECODE_I4_WAVES_PER_SIMD) void decode_split_append_i4_kernel(
    float* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
    uint8_t* k_arena, uint8_t* v_arena, const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ context_lens, float scale_log2, int Hkv, int nsplit_max,
    int num_blocks, DecodeAppend app) {
  const int g = blockIdx.z * kI8WavesPerWG + (threadIdx.x >> 6);
  if (g >= Hkv) return;
  decode_split_q_unit<CodesI4, true>(out, ws_o, ws_ml, nullptr, k_arena, v_arena, block_table,
                                     max_blocks, blockIdx.y, blockIdx.y, context_lens, 0,
                                     scale_log2, Hkv, nsplit_max, num_blocks, blockIdx.x, g, app);
}

// Log-sum-exp merge of the splits of one (sequence b, query head h):
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.
// One wave per query head (the 4 heads of KV head g form a workgroup), each
// lane 2 head dims.  Lane i holds the (m, l) of splits i, i + 64, ...; M and
// the denominator are wave reductions, and each split's weight reaches every
// lane through a lane read (no LDS, no barrier).  The (m, l) of the first 64
// splits and the partial o of the first kPre splits are requested before the
// context length arrives (the workspace holds nsplit_max splits per sequence,
// so these reads stay inside it; slots past a sequence's own splits are never
// used).  kPre = kCombineChunk suits small batches (one memory round trip per
// row of up to that many splits); for batches whose partials are large the
// launcher takes kPre = 2, every merged row having at least two splits, so
// unused slots are not fetched.
constexpr int kCombineThreads = 64 * kG;
constexpr int kCombineChunk = 16;
// partial bytes of a batch above which the combine prefetches 2 splits only
constexpr size_t kCombineEagerBytes = (size_t)64 << 20;

// Sequence b's output row is b and its context context_lens[b]; with a varlen
// batch (cu_q_lens != nullptr) only sequences of one row are decodes, their
// output row is cu_q_lens[b] and context_lens holds chunk starts (context
// chunk_start[b] + 1).
template <int kPre>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(
    float* __restrict__ out, const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
    const int32_t* __restrict__ context_lens, int max_blocks, int Hq, int nsplit_max,
    const int32_t* __restrict__ cu_q_lens, int num_tokens) {
  static_assert(kPre >= 1 && kPre <= kCombineChunk, "prefetch within the first batch");
  const int g = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int hh = tid >> 6, d = 2 * lane;  // head within the group, 2 dims
  // partial (b, split s, head h) sits at ((b * nsplit_max + s) * Hq + h)
  const size_t part0 = (size_t)b * nsplit_max * Hq + g * kG + hh;
  const float* ml = ws_ml + 2 * part0;
  const float* po = ws_o + part0 * kD + d;
  float2 ml0 = make_float2(-INFINITY, 0.f);
  if (lane < nsplit_max) ml0 = *(const float2*)(ml + (size_t)2 * lane * Hq);
  float2 ov[kCombineChunk];
#pragma unroll
  for (int s = 0; s < kPre; ++s)
    if (s < nsplit_max) ov[s] = *(const float2*)(po + (size_t)s * Hq * kD);
  int row = b, len = 0;
  if (cu_q_lens != nullptr) {
    row = cu_q_lens[b];
    if (min(cu_q_lens[b + 1], num_tokens) - row != 1) return;
    len = context_lens[b] + 1;
  } else {
    len = context_lens[b];
  }
  const int L = min(min(len, max_blocks * kBlock), nsplit_max * kDecodeSplit);
  const int nsplit = (L + kDecodeSplit - 1) / kDecodeSplit;
  if (nsplit <= 1) return;
#pragma unroll
  for (int s = kPre; s < kCombineChunk; ++s)
    if (s < nsplit) ov[s] = *(const float2*)(po + (size_t)s * Hq * kD);

  float M = lane < nsplit ? ml0.x : -INFINITY;
  for (int s = lane + 64; s < nsplit; s += 64) M = fmaxf(M, ml[(size_t)2 * s * Hq]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float w0 = lane < nsplit ? exp2f(ml0.x - M) : 0.f;
  float den = lane < nsplit ? w0 * ml0.y : 0.f;
  for (int s = lane + 64; s < nsplit; s += 64)
    den += exp2f(ml[(size_t)2 * s * Hq] - M) * ml[(size_t)2 * s * Hq + 1];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);

  float a0 = 0.f, a1 = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += 64) {
    // this lane's weight in the 64 splits from c0 (split c0 + lane)
    const float wc = c0 == 0 ? w0
                     : (c0 + lane < nsplit ? exp2f(ml[(size_t)2 * (c0 + lane) * Hq] - M) : 0.f);
    const int nc = min(64, nsplit - c0);
    for (int j0 = 0; j0 < nc; j0 += kCombineChunk) {
      if (c0 + j0 > 0) {
#pragma unroll
        for (int s = 0; s < kCombineChunk; ++s)
          if (j0 + s < nc) ov[s] = *(const float2*)(po + (size_t)(c0 + j0 + s) * Hq * kD);
      }
#pragma unroll
      for (int s = 0; s < kCombineChunk; ++s) {
        if (j0 + s < nc) {
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wc), j0 + s));
          a0 += w * ov[s].x;
          a1 += w * ov[s].y;
        }
      }
    }
  }
  const float inv = 1.f / den;
  float* dst = out + ((size_t)row * Hq + g * kG + hh) * kD + d;
  *(float2*)dst = make_float2(a0 * inv, a1 * inv);
}

}  // namespace

// ---- allocation-free decode ------------------------------------------------
// The split partials of paged_attention_decode_noalloc live in this file-scope
// device array (each GPU the library runs on holds its own copy until the
// process ends).  Its device address is looked up once per device, with that
// device current, and kept; the array's name is only a host-side stand-in.
static __device__ __align__(256) unsigned char scratch[PKV_DECODE_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

bool decode_fast_path(const pkv_geom& g) {
  return (g.dtype == PKV_F16 || g.dtype == PKV_I8KV || g.dtype == PKV_I4KV) && g.head_dim == kD &&
         g.num_q_heads == kG * g.num_kv_heads;
}

// Workspace: [partial o: S x nsplit x Hq x D floats][partial (m, l): S x nsplit x
// Hq x 2 floats], nsplit = ceil(max_context_len / kDecodeSplit); split-major,
// so the waves of one workgroup write one contiguous range.
static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t decode_workspace_bytes(const pkv_geom& g, int num_seqs, int max_context_len) {
  if (!decode_fast_path(g)) return 0;
  const size_t nsplit = (size_t)(max_context_len + kDecodeSplit - 1) / kDecodeSplit;
  if (nsplit <= 1) return 0;
  const size_t parts = (size_t)num_seqs * g.num_q_heads * nsplit;
  return align256(parts * kD * sizeof(float)) + parts * 2 * sizeof(float);
}

hipError_t launch_decode(const pkv_geom& g, float* out, const void* q, const void* k_arena,
                         const void* v_arena, const int32_t* block_table, int max_blocks,
                         const int32_t* context_lens, int num_seqs, int max_context_len,
                         float scale, void* workspace, size_t workspace_bytes,
                         hipStream_t stream, const DecodeGroups* groups) {
  if (!decode_fast_path(g))
    return launch_attend_generic(g, out, q, k_arena, v_arena, block_table, max_blocks,
                                 context_lens, nullptr, nullptr, num_seqs, num_seqs, scale,
                                 stream);
  const int nsplit = (max_context_len + kDecodeSplit - 1) / kDecodeSplit;
  (void)workspace_bytes;
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (nsplit > 1) {
    const size_t parts = (size_t)num_seqs * g.num_q_heads * nsplit;
    ws_o = (float*)workspace;
    ws_ml = (float*)((char*)workspace + align256(parts * kD * sizeof(float)));
  }
  const float scale_log2 = scale * 1.4426950408889634f;
  const int wpg = g.num_kv_heads < kDecodeWavesPerWG ? g.num_kv_heads : kDecodeWavesPerWG;
  const int zg = (g.num_kv_heads + kDecodeWavesPerWG - 1) / kDecodeWavesPerWG;
  // Workgroups are dealt to the 8 XCDs round-robin by linear id, and the id
  // is split + gx * sequence.  With an even gx a split index would always land
  // on the same XCDs — the low splits (present in every sequence) on some, the
  // high ones (long sequences only) on others.  An odd gx rotates each split
  // index across all XCDs; the extra column of workgroups exits at once.
  const int gx = nsplit | 1;
  const dim3 grid(gx, num_seqs, zg);
  // shared splits (fp16 arenas whose workgroup holds 1, 2, 4 or 8 KV heads;
  // other dtypes and widths compute every split per row, the same result)
  const bool shared = groups != nullptr && g.dtype == PKV_F16 && nsplit > 1 &&
                      groups->num_groups > 0 && groups->max_skip > 0 &&
                      groups->max_group_size > 0 && (wpg == 1 || wpg == 2 || wpg == 4 || wpg == 8);
  if (shared) {
    const int quads = (groups->max_group_size + 3) / 4;
    const int nshared = min(groups->max_skip, nsplit);
    // a shared workgroup: kHeads KV heads x kQuads quads (SharedGeom<wpg>)
    const int wq = wpg < 4 ? wpg : 4, wh = wpg / wq;
    const int hgroups = (g.num_kv_heads + wh - 1) / wh, qgroups = (quads + wq - 1) / wq;
    const long n_shared = (long)nshared * qgroups * hgroups * groups->num_groups;
    const long per = (n_shared + 7) / 8;
    const long nwg = 8 * per + (long)nsplit * num_seqs * zg;
    if (nwg > 0x7fffffffL) return hipErrorInvalidValue;
    auto kernel = wpg == 8   ? decode_shared_kernel<8>
                  : wpg == 4 ? decode_shared_kernel<4>
                  : wpg == 2 ? decode_shared_kernel<2>
                             : decode_shared_kernel<1>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)nwg), dim3(64 * wpg), 0, stream, out,
                       ws_o, ws_ml, (const _Float16*)q, (const _Float16*)k_arena,
                       (const _Float16*)v_arena, block_table, max_blocks, context_lens,
                       groups->group_start, groups->row_skip, scale_log2, g.num_kv_heads, nsplit,
                       g.num_blocks, zg, num_seqs, nshared, hgroups, qgroups, (int)n_shared,
                       (int)per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_combine(g, out, ws_o, ws_ml, context_lens, nullptr, 0, max_blocks,
                                 num_seqs, nsplit, stream);
  }
  if (g.dtype == PKV_I8KV || g.dtype == PKV_I4KV) {
    const int wpg8 = g.num_kv_heads < kI8WavesPerWG ? g.num_kv_heads : kI8WavesPerWG;
    const dim3 grid8(gx, num_seqs, (g.num_kv_heads + kI8WavesPerWG - 1) / kI8WavesPerWG);
    hipLaunchKernelGGL(g.dtype == PKV_I8KV ? decode_split_i8_kernel : decode_split_i4_kernel,
                       grid8, dim3(64 * wpg8), 0, stream,
                       out, ws_o, ws_ml, (const _Float16*)q, (const uint8_t*)k_arena,
                       (const uint8_t*)v_arena, block_table, max_blocks, context_lens,
                       scale_log2, g.num_kv_heads, nsplit, g.num_blocks);
  } else {
    hipLaunchKernelGGL(decode_split_kernel, grid, dim3(64 * wpg), 0, stream,
                       out, ws_o, ws_ml, (const _Float16*)q, (const _Float16*)k_arena,
                       (const _Float16*)v_arena, block_table, max_blocks, context_lens,
                       scale_log2, g.num_kv_heads, nsplit, g.num_blocks);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit <= 1) return e;
  return launch_decode_combine(g, out, ws_o, ws_ml, context_lens, nullptr, 0, max_blocks, num_seqs,
                               nsplit, stream);
}

hipError_t launch_decode_append(const pkv_geom& g, float* out, const void* q, void* q_out,
                                const void* k, const void* v, void* k_arena, void* v_arena,
                                const int32_t* block_table, int max_blocks,
                                const int32_t* context_lens, int num_seqs, int max_context_len,
                                float scale, const void* rope_table, int rope_max_pos,
                                void* workspace, hipStream_t stream) {
  const int nsplit = (max_context_len + kDecodeSplit - 1) / kDecodeSplit;
  float* ws_o = nullptr;
  float* ws_ml = nullptr;
  if (nsplit > 1) {
    const size_t parts = (size_t)num_seqs * g.num_q_heads * nsplit;
    ws_o = (float*)workspace;
    ws_ml = (float*)((char*)workspace + align256(parts * kD * sizeof(float)));
  }
  DecodeAppend app;
  app.q = (const _Float16*)q;
  app.q_out = (_Float16*)q_out;
  app.k = (const _Float16*)k;
  app.v = (const _Float16*)v;
  app.k_arena = (_Float16*)k_arena;
  app.v_arena = (_Float16*)v_arena;
  app.rope = (const double2*)rope_table;
  app.rope_max_pos = rope_max_pos;
  const float scale_log2 = scale * 1.4426950408889634f;
  if (g.dtype == PKV_I8KV || g.dtype == PKV_I4KV) {
    const int wpg8 = g.num_kv_heads < kI8WavesPerWG ? g.num_kv_heads : kI8WavesPerWG;
    const dim3 grid8(nsplit | 1, num_seqs, (g.num_kv_heads + kI8WavesPerWG - 1) / kI8WavesPerWG);
    hipLaunchKernelGGL(g.dtype == PKV_I8KV ? decode_split_append_i8_kernel
                                           : decode_split_append_i4_kernel,
                       grid8, dim3(64 * wpg8), 0, stream, out, ws_o, ws_ml, (uint8_t*)k_arena,
                       (uint8_t*)v_arena, block_table, max_blocks, context_lens, scale_log2,
                       g.num_kv_heads, nsplit, g.num_blocks, app);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nsplit <= 1) return e;
    return launch_decode_combine(g, out, ws_o, ws_ml, context_lens, nullptr, 0, max_blocks,
                                 num_seqs, nsplit, stream);
  }
  const int wpg = g.num_kv_heads < kDecodeWavesPerWG ? g.num_kv_heads : kDecodeWavesPerWG;
  const int zg = (g.num_kv_heads + kDecodeWavesPerWG - 1) / kDecodeWavesPerWG;
  const dim3 grid(nsplit | 1, num_seqs, zg);  // odd width: see launch_decode
  hipLaunchKernelGGL(decode_split_append_kernel, grid, dim3(64 * wpg), 0, stream, out, ws_o,
                     ws_ml, block_table, max_blocks, context_lens, scale_log2, g.num_kv_heads,
                     nsplit, g.num_blocks, app);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit <= 1) return e;
  return launch_decode_combine(g, out, ws_o, ws_ml, context_lens, nullptr, 0, max_blocks, num_seqs,
                               nsplit, stream);
}

hipError_t launch_decode_combine(const pkv_geom& g, float* out, const float* ws_o,
                                 const float* ws_ml, const int32_t* lens,
                                 const int32_t* cu_q_lens, int num_tokens, int max_blocks,
                                 int num_seqs, int nsplit_max, hipStream_t stream) {
  const size_t partial_bytes =
      (size_t)num_seqs * g.num_q_heads * nsplit_max * (kD + 2) * sizeof(float);
  if (partial_bytes <= kCombineEagerBytes)
    hipLaunchKernelGGL(decode_combine_kernel<kCombineChunk>, dim3(g.num_kv_heads, num_seqs),
                       dim3(kCombineThreads), 0, stream, out, ws_o, ws_ml, lens, max_blocks,
                       g.num_q_heads, nsplit_max, cu_q_lens, num_tokens);
  else
    hipLaunchKernelGGL(decode_combine_kernel<2>, dim3(g.num_kv_heads, num_seqs),
                       dim3(kCombineThreads), 0, stream, out, ws_o, ws_ml, lens, max_blocks,
                       g.num_q_heads, nsplit_max, cu_q_lens, num_tokens);
  return hipGetLastError();
}

}  // namespace pkv
