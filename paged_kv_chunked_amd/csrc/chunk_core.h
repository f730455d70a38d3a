// Core of the tuned chunk prefill: one (sequence, 64-row tile, KV head) unit,
// used by paged_attention_chunk and by the mixed-batch kernel (the design is
// described at the top of chunk.hip).  A workgroup of kThreads runs one unit;
// the unit owns the workgroup's LDS, one array laid out by ChunkLds<kQ> and
// declared by the kernel.
#pragma once

#include <type_traits>

#include "fp16_shape.h"
#include "lds_dma.h"
#include "quant_codes.h"

namespace pkv {
namespace {

#ifndef PKV_CHUNK_RB
#define PKV_CHUNK_RB 2
#endif
constexpr int kRB = PKV_CHUNK_RB;  // 16-row blocks per wave
constexpr int kBM = 16 * kRB;      // rows per wave
constexpr int kRows = 64;          // chunk rows per workgroup
constexpr int kRowGroups = kRows / kBM;  // waves per query head in a workgroup
constexpr int kBN = 64;            // keys per tile (4 arena blocks)
constexpr int kWaves = kG * kRowGroups;
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerTile = 2 * 16 / kWaves;  // direct-to-LDS loads per wave per tile
constexpr int kStages = 4;         // LDS ring depth (tiles)
constexpr int kUnitsPerBlock = kBlock * kD * 2 / 16;  // 16-byte units in one (block, head) tile
constexpr int kStageUnits = 2 * 4 * kUnitsPerBlock;    // K and V of 4 blocks

// Reductions over the four lanes {l, l^16, l^32, l^48} that hold one row,
// through the gfx950 cross-row lane swaps (no LDS round trip).
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Three-way maximum as one v_max3_f32.  fmaxf would first quiet each operand
// (the compiler cannot tell that matrix-core results are never signalling
// NaNs), doubling the instruction count of the row maximum.
__device__ inline float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// How far (log2 units) a row's running maximum may lag the true maximum before
// the accumulator is rescaled (fp16 arenas): probabilities stay <= 2^8, well
// inside fp16.  Quantized arenas keep the exact running maximum (slack 0), so
// probabilities stay <= 1 and a tile's largest one is exactly 1 (QGeom).
constexpr float kSlack = 8.f;

// Work of row tile rt of sequence b, in 64-key tiles (0 if the tile is empty).
// The same arithmetic decides the tile loop of the attention kernel.
__device__ inline int chunk_item_cost(const int32_t* __restrict__ cu_q_lens,
                                      const int32_t* __restrict__ chunk_start, int b, int rt,
                                      int max_blocks, int num_tokens) {
  const int row0 = cu_q_lens[b];
  const int C = min(cu_q_lens[b + 1], num_tokens) - row0;
  if (rt * kRows >= C) return 0;
  const int P = chunk_start[b];
  const int Lc = min(P + C, max_blocks * kBlock);
  if (Lc <= 0) return 0;
  const int kend = min(Lc, P + min(C, rt * kRows + kRows));
  return max(1, (kend + kBN - 1) / kBN);
}

// Zero the halves of a 16-byte V unit (8 consecutive keys key0..key0+7) whose
// key is >= limit.
__device__ inline u32x4 mask_unit(u32x4 x, int key0, int limit) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int k = key0 + 2 * c;
    uint32_t w = x[c];
    if (k >= limit) w = 0u;
    else if (k + 1 >= limit) w &= 0xFFFFu;
    x[c] = w;
  }
  return x;
}

// Quantized arenas (head dim 128): each (block, KV head) tile holds the codes,
// then 16 fp16 scales at byte kCodeBlk.  The codes of 3 key tiles are staged in
// LDS ([K codes of 4 blocks][V codes of 4 blocks][K scales][V scales]); every
// thread then turns its share of one tile's codes into fp16 (exactly: every
// code is a small integer) in a 2-stage fp16 ring laid out as the fp16 unit's,
// so the matrix-core loop is the same, and 128 threads put the tile's scales
// into a 2-stage fp32 scale ring.  The scales are applied where the codec's
// decoded value code * scale enters exactly: the K scale multiplies the fp32
// score of its key, the V scale the key's probability before it is rounded to
// fp16 for the second product (as the quantized decode unit does).  Rounding
// code * scale to fp16 instead would add a second rounding the codec does not
// have.
constexpr int kCodeStages = 3;
template <int kQ>
struct QGeom;
template <>
struct QGeom<0> {  // fp16 arena: tiles land in the fp16 ring directly
  static constexpr int kFp16Stages = kStages;
  static constexpr int kStageBytes = 0;
  static constexpr int kCodeStageCount = 0;
  static constexpr int kScaleStages = 0;
  static constexpr float kPvScale = 1.f;
  static constexpr float kRowSlack = kSlack;
};
template <>
struct QGeom<1> {  // INT8: 3 loads per wave per tile (K codes, V codes, scales)
  static constexpr int kCodeBlk = kBlock * kD;
  static constexpr int kTile = (int)i8_tile_bytes(kD);
  static constexpr int kLoads = 3;
  static constexpr int kStageBytes = 8 * kCodeBlk + 256;
  static constexpr int kFp16Stages = 2;
  static constexpr int kCodeStageCount = kCodeStages;
  static constexpr int kScaleStages = 2;
  // p * s_v * kPvScale must stay finite in fp16: p <= 1 (exact running
  // maximum) and an INT8 scale is at most fp16(65504 / 127) = 515.5, so
  // 515.5 * 2^6 = 32992; the factor keeps small weights out of fp16's
  // subnormal range, where their rounding would grow
  static constexpr float kPvScale = 64.f;
  static constexpr float kRowSlack = 0.f;
};
template <>
struct QGeom<2> {  // INT4: 2 loads per wave per tile (K or V codes, scales)
  static constexpr int kCodeBlk = kBlock * kD / 2;
  static constexpr int kTile = (int)i4_tile_bytes(kD);
  static constexpr int kLoads = 2;
  static constexpr int kStageBytes = 8 * kCodeBlk + 256;
  static constexpr int kFp16Stages = 2;
  static constexpr int kCodeStageCount = kCodeStages;
  static constexpr int kScaleStages = 2;
  // INT4 scales reach fp16(65504 / 7) = 9360: 9360 * 2^2 = 37440
  static constexpr float kPvScale = 4.f;
  static constexpr float kRowSlack = 0.f;
};

// Scale ring stage (fp32): 64 K scales, 64 V scales times kPvScale, and their
// reciprocals.
constexpr int kScaleStageFloats = 3 * kBN;

// The unit's LDS, one array, byte offsets of its regions:
//   [fp16 ring: kFp16Stages x kStageUnits 16-byte units (K of 4 blocks, V of 4)]
//   [scale ring: kScaleStages x kScaleStageFloats fp32]
//   [code ring: kCodeStageCount x kStageBytes]
//   [slot: 16 bytes for the persistent mixed kernel's unit index]
template <int kQ>
struct ChunkLds {
  using QG = QGeom<kQ>;
  static constexpr int kFp16 = 0;
  static constexpr int kScale = kFp16 + QG::kFp16Stages * kStageUnits * 16;
  static constexpr int kCode = kScale + QG::kScaleStages * kScaleStageFloats * 4;
  static constexpr int kSlot = kCode + QG::kCodeStageCount * QG::kStageBytes;
  static constexpr int kBytes = kSlot + 16;
  static constexpr int kUnits = kBytes / 16;  // size of the u32x4 array
  static_assert(kScale % 16 == 0 && kCode % 16 == 0 && kSlot % 16 == 0, "16-byte regions");
  static_assert(kBytes <= 160 * 1024, "fits the 160 KiB of LDS of a gfx950 CU");
};

// ---- where every LDS write of a unit lands (host-checkable) ---------------
// The same functions give the kernel its addresses and the compile-time check
// below its cases, so the check covers the code that runs.

// fp16 arenas, direct-to-LDS tile load: byte address (relative to the LDS
// array) of lane `lane`'s 16 bytes for quarter j of wave `wave`, K (kv = 0)
// or V (kv = 1), in fp16 stage `stage`.
__host__ __device__ constexpr int tile_dma_byte(int stage, int wave, int j, int kv, int lane) {
  constexpr int kQuarters = 16 / kWaves;
  const int dma_blk = (wave * kQuarters) >> 2;
  const int qq = (wave * kQuarters + j) & 3;
  return stage * kStageUnits * 16 + kv * 4 * kUnitsPerBlock * 16 +
         (dma_blk * kUnitsPerBlock + qq * 64) * 16 + 16 * lane;
}

// Quantized arenas, direct-to-LDS code loads into code stage `cstage`:
// which = 0: the K codes (INT8) or the codes (INT4) of wave `wave`; 1: the V
// codes (INT8 only); 2: the scale run (lanes 0-1 only).
template <int kQ>
__host__ __device__ constexpr int code_dma_byte(int cstage, int wave, int which, int lane) {
  using QG = QGeom<kQ>;
  const int st = ChunkLds<kQ>::kCode + cstage * QG::kStageBytes;
  if (which == 2) return st + 8 * QG::kCodeBlk + 32 * wave + 16 * lane;
  return st + (which == 1 ? 4 * QG::kCodeBlk : 0) + 1024 * wave + 16 * lane;
}

// Conversion of one code tile: thread tid writes fp16 units tid + 512 j of the
// K half (kv = 0) and of the V half (kv = 1) of fp16 stage `stage`; threads
// below 2 kBN write one scale each.
template <int kQ>
__host__ __device__ constexpr int conv_unit_byte(int stage, int kv, int tid, int j) {
  return ChunkLds<kQ>::kFp16 + stage * kStageUnits * 16 +
         (kv * 4 * kUnitsPerBlock + tid + 512 * j) * 16;
}
template <int kQ>
__host__ __device__ constexpr int conv_scale_byte(int stage, int tid) {
  return ChunkLds<kQ>::kScale + (stage * kScaleStageFloats + tid) * 4;
}

// Offsets (bytes, within one code stage) the conversion reads for thread tid's
// unit tid + 512 j: K codes, K scale, V codes, V scale.
template <int kQ>
__host__ __device__ constexpr int conv_kcode_off(int tid, int j) {
  using QG = QGeom<kQ>;
  const int u = tid + 512 * j;
  const int a = u >> 8, pos = u & 255, p8 = pos >> 4;
  const int sl = (pos & 15) ^ (4 * (a & 1));
  if (kQ == 1) return a * QG::kCodeBlk + (p8 >> 1) * 256 + i8_kpos(sl) * 16 + 8 * (p8 & 1);
  return a * QG::kCodeBlk + (p8 >> 1) * 128 + i4_krec(sl) * 8;
}
template <int kQ>
__host__ __device__ constexpr int conv_vcode_off(int tid, int j) {
  using QG = QGeom<kQ>;
  const int u = tid + 512 * j;
  const int a = u >> 8, pos = u & 255;
  const int unit = (pos - 16 * (a & 1)) & 255, d = unit >> 1, hs = unit & 1;
  if (kQ == 1) return 4 * QG::kCodeBlk + a * QG::kCodeBlk + 8 * unit;
  return 4 * QG::kCodeBlk + a * QG::kCodeBlk + i4_vbyte(d, 8 * hs, kD);
}
// Scale of key `key` of the tile (K: kv = 0, V: kv = 1) within a code stage.
template <int kQ>
__host__ __device__ constexpr int conv_scale_off(int kv, int key) {
  return 8 * QGeom<kQ>::kCodeBlk + 128 * kv + 32 * (key >> 4) + 2 * (key & 15);
}

// Every write of the unit stays inside its own region (and so never reaches
// another region or the slot), and every conversion read stays inside the
// part of the code stage it means to read.
template <int kQ>
constexpr bool chunk_lds_writes_in_bounds() {
  using L = ChunkLds<kQ>;
  using QG = QGeom<kQ>;
  auto inside = [](int lo, int n, int at, int hi) { return at >= lo && at + n <= hi; };
  if constexpr (kQ == 0) {
    for (int st = 0; st < QG::kFp16Stages; ++st)
      for (int w = 0; w < kWaves; ++w)
        for (int j = 0; j < 16 / kWaves; ++j)
          for (int kv = 0; kv < 2; ++kv)
            for (int ln = 0; ln < 64; ++ln) {
              const int lo = st * kStageUnits * 16 + kv * 4 * kUnitsPerBlock * 16;
              if (!inside(lo, 16, tile_dma_byte(st, w, j, kv, ln), lo + 4 * kUnitsPerBlock * 16))
                return false;
            }
    // zeroing of V past the sequence: units tid + e kThreads of the V half
    for (int st = 0; st < QG::kFp16Stages; ++st)
      for (int u = 0; u < 2 * kThreads; ++u)
        if (u >= 4 * kUnitsPerBlock) return false;
    return L::kSlot == QG::kFp16Stages * kStageUnits * 16;
  } else {
    for (int cs = 0; cs < QG::kCodeStageCount; ++cs) {
      const int lo = L::kCode + cs * QG::kStageBytes;
      for (int w = 0; w < kWaves; ++w)
        for (int ln = 0; ln < 64; ++ln) {
          // codes: K (and for INT8 V) regions of the stage
          if (!inside(lo, 16, code_dma_byte<kQ>(cs, w, 0, ln),
                      lo + (kQ == 1 ? 4 : 8) * QG::kCodeBlk))
            return false;
          if (kQ == 1 && !inside(lo + 4 * QG::kCodeBlk, 16, code_dma_byte<kQ>(cs, w, 1, ln),
                                 lo + 8 * QG::kCodeBlk))
            return false;
          if (ln < 2 && !inside(lo + 8 * QG::kCodeBlk, 16, code_dma_byte<kQ>(cs, w, 2, ln),
                                lo + QG::kStageBytes))
            return false;
        }
    }
    for (int st = 0; st < QG::kFp16Stages; ++st)
      for (int tid = 0; tid < kThreads; ++tid)
        for (int j = 0; j < 2; ++j)
          for (int kv = 0; kv < 2; ++kv) {
            const int lo = st * kStageUnits * 16 + kv * 4 * kUnitsPerBlock * 16;
            if (!inside(lo, 16, conv_unit_byte<kQ>(st, kv, tid, j), lo + 4 * kUnitsPerBlock * 16))
              return false;
          }
    for (int st = 0; st < QG::kScaleStages; ++st)
      for (int tid = 0; tid < kScaleStageFloats; ++tid) {
        const int lo = L::kScale + st * kScaleStageFloats * 4;
        if (!inside(lo, 4, conv_scale_byte<kQ>(st, tid), lo + kScaleStageFloats * 4))
          return false;
      }
    // conversion reads: codes in the K / V code regions, scales in the scale runs
    for (int tid = 0; tid < kThreads; ++tid)
      for (int j = 0; j < 2; ++j) {
        if (!inside(0, 8, conv_kcode_off<kQ>(tid, j), 4 * QG::kCodeBlk)) return false;
        if (!inside(4 * QG::kCodeBlk, kQ == 1 ? 8 : 4, conv_vcode_off<kQ>(tid, j),
                    8 * QG::kCodeBlk))
          return false;
      }
    for (int key = 0; key < kBN; ++key)
      for (int kv = 0; kv < 2; ++kv)
        if (!inside(8 * QG::kCodeBlk + 128 * kv, 2, conv_scale_off<kQ>(kv, key),
                    8 * QG::kCodeBlk + 128 * kv + 128))
          return false;
    return L::kSlot == L::kCode + QG::kCodeStageCount * QG::kStageBytes;
  }
}
static_assert(kWaves == 8 && kThreads == 512,
              "the quantized load and conversion maps assume 8 waves of 64 lanes");
static_assert(chunk_lds_writes_in_bounds<0>(), "fp16 unit LDS layout");
static_assert(chunk_lds_writes_in_bounds<1>(), "INT8 unit LDS layout");
static_assert(chunk_lds_writes_in_bounds<2>(), "INT4 unit LDS layout");

// Row tile rt of sequence b for KV head g.  With parts > 1 the unit covers
// part `part` of the tile's key tiles (an even share, possibly empty) and
// writes the unnormalised O, the running maximum (log2 units) and the
// denominator of every row to part_o / part_ml, [part][row][head], for
// chunk_combine_kernel to merge.  kQ: arena storage, 0 fp16, 1 INT8, 2 INT4.
// lds: the workgroup's LDS array of ChunkLds<kQ>::kUnits 16-byte units.
template <int kQ = 0>
__device__ __forceinline__ void chunk_tile_unit(
    u32x4* __restrict__ lds, float* __restrict__ out, const _Float16* __restrict__ q,
    const void* __restrict__ k_arena, const void* __restrict__ v_arena,
    const int32_t* __restrict__ block_table, int max_blocks,
    const int32_t* __restrict__ cu_q_lens, const int32_t* __restrict__ chunk_start,
    float scale_log2, int Hkv, int num_blocks, int num_tokens, int b, int rt, int g,
    int part = 0, int parts = 1, float* __restrict__ part_o = nullptr,
    float* __restrict__ part_ml = nullptr) {
  using QG = QGeom<kQ>;
  using LY = ChunkLds<kQ>;
  const int row0 = cu_q_lens[b];
  const int C = min(cu_q_lens[b + 1], num_tokens) - row0;
  if (rt * kRows >= C) return;
  const int P = chunk_start[b];
  const int Lc = min(P + C, max_blocks * kBlock);  // keys that exist
  if (Lc <= 0) return;
  // the wave index is made visibly uniform, so block-table reads indexed by
  // it are scalar loads (they must not add to the vector-memory count)
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int Hq = Hkv * kG;
  const int h = g * kG + (wave & 3);
  const int wrow0 = rt * kRows + kBM * (wave >> 2);  // first chunk row of this wave

  // fp16 stages of (K: 4 blocks x 256 units, then V: 4 blocks x 256 units):
  // 4 for fp16 arenas (128 KiB), else 2, then the scale and code stages
  u32x4* const ring = lds + LY::kFp16 / 16;
  float* const scale_ring = (float*)(lds + LY::kScale / 16);

  const int row_hi = min(C, rt * kRows + kRows);
  const int kend = min(Lc, P + row_hi);  // keys [0, kend) are visible to some row
  const int ntiles = (kend + kBN - 1) / kBN;
  const int tb = (int)((long)part * ntiles / parts), te = (int)((long)(part + 1) * ntiles / parts);
  const int nblk_seq = (Lc + kBlock - 1) / kBlock;
  const int32_t* bt = block_table + (size_t)b * max_blocks;

  // Tile loads.  Each block's K and V tiles are 4 quarters of 1 KiB; wave w
  // moves quarters w * kQuarters .. +kQuarters-1 of the 16 (block = index / 4);
  // a lane's unit goes to position pos of the block's 256 units:
  //   K: pos = piece * 16 + slot', fetched from slot' ^ 4 in odd blocks, so
  //      the two blocks an operand read touches use disjoint banks;
  //   V: pos = (dim * 2 + half + 16 (block & 1)) mod 256: the odd blocks'
  //      units are rotated by 16, so the two blocks an operand read touches
  //      use disjoint banks (measured conflict-free on gfx950).
  // Past the sequence's last block the id of that last block is used (its
  // contents never reach the output: scores masked, V zeroed).
  constexpr int kQuarters = 16 / kWaves;  // 1 KiB quarters of block tiles per wave
  const int dma_blk = (wave * kQuarters) >> 2;
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) u32x4*)lds;
  auto issue_tile = [&](int t) {
    int blk = bt[min(t * 4 + dma_blk, nblk_seq - 1)];
    blk = (blk < 0 || blk >= num_blocks) ? 0 : blk;
    const u32x4* kt = (const u32x4*)k_arena + ((size_t)blk * Hkv + g) * kUnitsPerBlock;
    const u32x4* vt = (const u32x4*)v_arena + ((size_t)blk * Hkv + g) * kUnitsPerBlock;
    const int stage = t % kStages;
#pragma unroll
    for (int j = 0; j < kQuarters; ++j) {
      const int qq = (wave * kQuarters + j) & 3;
      const int pos = qq * 64 + lane;
      // lane 0's address; lane i lands 16 i bytes further
      dma16(kt + (pos ^ (4 * (dma_blk & 1))),
            __builtin_amdgcn_readfirstlane(lds_base + tile_dma_byte(stage, wave, j, 0, 0)));
      dma16(vt + ((pos - 16 * (dma_blk & 1)) & (kUnitsPerBlock - 1)),
            __builtin_amdgcn_readfirstlane(lds_base + tile_dma_byte(stage, wave, j, 1, 0)));
    }
  };

  // Quantized arenas: code tile t goes to code stage t % kCodeStages.  INT8:
  // wave w moves half w & 1 of block w >> 1's K and V codes; INT4: waves 0-3
  // move the K codes of block w, waves 4-7 the V codes of block w - 4; and
  // lanes 0-1 of wave w the K (w < 4) or V scales of block w & 3.
  auto issue_codes = [&](int t) {
    if constexpr (kQ != 0) {
      const uint8_t* ka8 = (const uint8_t*)k_arena;
      const uint8_t* va8 = (const uint8_t*)v_arena;
      const int cs = t % kCodeStages;
      int sblk = bt[min(t * 4 + (wave & 3), nblk_seq - 1)];
      sblk = (sblk < 0 || sblk >= num_blocks) ? 0 : sblk;
      const size_t stile = ((size_t)sblk * Hkv + g) * QG::kTile;
      const uint8_t* sarena = wave < 4 ? ka8 : va8;
      if constexpr (kQ == 1) {
        int blk = bt[min(t * 4 + (wave >> 1), nblk_seq - 1)];
        blk = (blk < 0 || blk >= num_blocks) ? 0 : blk;
        const size_t src = ((size_t)blk * Hkv + g) * QG::kTile + 16 * (64 * (wave & 1) + lane);
        dma16(ka8 + src, __builtin_amdgcn_readfirstlane(lds_base + code_dma_byte<kQ>(cs, wave, 0, 0)));
        dma16(va8 + src, __builtin_amdgcn_readfirstlane(lds_base + code_dma_byte<kQ>(cs, wave, 1, 0)));
      } else {
        dma16(sarena + stile + 16 * lane,
              __builtin_amdgcn_readfirstlane(lds_base + code_dma_byte<kQ>(cs, wave, 0, 0)));
      }
      if (lane < 2)
        dma16(sarena + stile + QG::kCodeBlk + 16 * lane,
              __builtin_amdgcn_readfirstlane(lds_base + code_dma_byte<kQ>(cs, wave, 2, 0)));
    }
  };
  auto issue = [&](int t) {
    if constexpr (kQ == 0) issue_tile(t);
    else issue_codes(t);
  };

  // Conversion of code tile t into fp16 stage t & 1 and scale stage t & 1:
  // thread tid writes units tid and tid + 512 of the K half and of the V half
  // of the fp16 stage, in the fp16 unit's order (K: piece p * 16 + slot',
  // slot' = slot ^ 4 in odd blocks; V: (2 dim + half + 16 (block & 1)) mod
  // 256), holding the codes as exact fp16 integers.  Threads 0-63 write the
  // K scale of key tid as fp32, threads 64-127 the V scale of key tid - 64
  // times kPvScale, threads 128-191 the reciprocal of that.  Keys past the
  // sequence get 0 for all three (their scale bytes are not data; their codes
  // are finite).
  [[maybe_unused]] int kc_off[2], vc_off[2], k_sh[2];
  [[maybe_unused]] int sc_off = 0, sc_key = 0;
  [[maybe_unused]] float sc_mul = 1.f;
  [[maybe_unused]] bool sc_recip = false;
  if constexpr (kQ != 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      kc_off[j] = conv_kcode_off<kQ>(tid, j);
      vc_off[j] = conv_vcode_off<kQ>(tid, j);
      k_sh[j] = 4 * ((((tid + 512 * j) & 255) >> 4) & 1);
    }
    sc_key = tid & (kBN - 1);
    sc_off = conv_scale_off<kQ>(min(tid >> 6, 1), sc_key);
    sc_mul = tid >= kBN ? QG::kPvScale : 1.f;
    sc_recip = tid >= 2 * kBN;
  }
  // (masked: the tile reaches past the sequence; keys >= lim get scale 0)
  auto convert_tile = [&](int t, auto masked) {
    if constexpr (kQ != 0) {
      const uint8_t* cs = (const uint8_t*)lds + LY::kCode + (t % kCodeStages) * QG::kStageBytes;
      u32x4* fs = ring + (t & 1) * kStageUnits;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint2 c = *(const uint2*)(cs + kc_off[j]);
        half8_t hk;
        if constexpr (kQ == 1) hk = codes_to_half(c.x, c.y);
        else hk = nibbles_to_half(c.x >> k_sh[j], c.y >> k_sh[j]);
        fs[tid + 512 * j] = __builtin_bit_cast(u32x4, hk);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        half8_t hv;
        if constexpr (kQ == 1) {
          const uint2 c = *(const uint2*)(cs + vc_off[j]);
          hv = codes_to_half(c.x, c.y);
        } else {
          const uint32_t w = *(const uint32_t*)(cs + vc_off[j]);
          hv = nibbles_to_half(w, w >> 4);
        }
        fs[4 * kUnitsPerBlock + tid + 512 * j] = __builtin_bit_cast(u32x4, hv);
      }
      if (tid < kScaleStageFloats) {
        float sc = (float)*(const _Float16*)(cs + sc_off) * sc_mul;
        if (sc_recip) sc = 1.f / sc;  // scales are at least the smallest positive fp16
        if (masked && sc_key >= Lc - t * kBN) sc = 0.f;
        scale_ring[(t & 1) * kScaleStageFloats + tid] = sc;
      }
    }
  };
  auto convert = [&](int t) {
    if (t * kBN + kBN > Lc) convert_tile(t, std::true_type{});
    else convert_tile(t, std::false_type{});
  };

  // The first three tiles' loads go out before the queries', so all their
  // latencies overlap; then everything is waited for (the compiler, which
  // does not see the tile loads, must see the queries complete before the
  // loop, or it waits for all loads at their first use in every tile).
  if (tb < te) issue(tb);
  if (tb + 1 < te) issue(tb + 1);
  if (tb + 2 < te) issue(tb + 2);
  // Q^T as the B operand: qf[rb][kd] = Q[row wrow0 + 16rb + lr][dims 32kd + 8lq .. +8]
  half8_t qf[kRB][4];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const int r = wrow0 + 16 * rb + lr;
#pragma unroll
    for (int kd = 0; kd < 4; ++kd) {
      if (r < C) {
        qf[rb][kd] = __builtin_bit_cast(
            half8_t, *(const u32x4*)(q + ((size_t)(row0 + r) * Hq + h) * kD + 32 * kd + 8 * lq));
      } else {
        qf[rb][kd] = (half8_t)(_Float16)0.f;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  if constexpr (kQ != 0) {
    if (tb < te) {
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      convert(tb);
    }
  }

  // absolute positions of this lane's two rows (rows past the chunk borrow the
  // last valid position so they stay finite; they are never stored)
  int prow[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) prow[rb] = min(P + wrow0 + 16 * rb + lr, Lc - 1);
  const int first_pos = P + wrow0;  // smallest row position of this wave

  f32x4 oacc[8][kRB];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) oacc[db][rb] = (f32x4)0.f;
  // Per row: running maximum of the raw scores, the raw score above which
  // the accumulator must be rescaled, -max * scale_log2, and the denominator.
  float m_raw[kRB], m_lim[kRB], m_off[kRB], l_run[kRB];
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    m_raw[rb] = -INFINITY;
    m_lim[rb] = -INFINITY;
    m_off[rb] = 0.f;
    l_run[rb] = 0.f;
  }
  const float slack_raw = QG::kRowSlack / scale_log2;
  const half2_t ones = {(_Float16)1.f, (_Float16)1.f};

  // Operand addresses (16-byte units within a stage).  K fragment of MFMA kb,
  // dim piece 4kd + lq: MFMA row m = lr holds key slot
  // 8((m >> 2) & 1) + 4(kb & 1) + (m & 3) of block 2(kb >> 1) + (m >> 3).
  const int ka = lr >> 3;  // block offset within the pair of blocks
  const int kslot0 = 8 * ((lr >> 2) & 1) + (lr & 3);
  // V fragment of dims block db for the keys of MFMA u: 16-byte unit
  // (2 (16db + lr) + (lq & 1) + 16 (lq >> 1)) mod 256 of block 2u + (lq >> 1)
  const int vunit = 2 * lr + (lq & 1) + 16 * (lq >> 1);
  // This lane's scores (kb, i) are keys key_u + 4 (kb & 1) + i of the tile,
  // u = kb >> 1, key_u = 32 u + key_u0, its probabilities pb[u][..][e] and its
  // V fragments of MFMA u keys key_u + e.
  const int key_u0 = 16 * (lq >> 1) + 8 * (lq & 1);

  // ---- the steps of one key tile -----------------------------------------
  // Zero V of keys past the sequence in tile t (its last tile; fp16 arenas:
  // p = 0 there, but 0 * NaN would not be 0), 2 units per thread.
  auto zero_v_tail = [&](int t) {
    u32x4* vw = ring + (t % kStages) * kStageUnits + 4 * kUnitsPerBlock;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int unit = tid + e * kThreads;  // [block][dim][half']
      const int a = unit >> 8, hs = unit & 1;  // block, half (8 keys) of the unit
      const int key0 = t * kBN + 16 * a + 8 * hs;
      if (key0 + 8 > Lc) vw[unit] = mask_unit(vw[unit], key0, Lc);
    }
  };
  auto k_stage = [&](int t) { return ring + (kQ == 0 ? t % kStages : t & 1) * kStageUnits; };
  auto read_v = [&](int t, int db, half8_t* f) {
    const u32x4* vl = k_stage(t) + 4 * kUnitsPerBlock;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int a = 2 * u + (lq >> 1);
      f[u] = __builtin_bit_cast(half8_t, vl[a * kUnitsPerBlock + ((32 * db + vunit) & (kUnitsPerBlock - 1))]);
    }
  };

  // S^T[key][row] = K . Q^T (raw scores) of tile t; the K fragments of MFMA
  // kb + 1 are read while kb's products run, and the first two V fragment
  // pairs of the tile are requested at the end (read during the softmax).
  auto qk = [&](int t, f32x4 (&sacc)[4][kRB], half8_t (&vf)[3][2], bool prefetch_v = true) {
    const u32x4* kl = k_stage(t);
    // Quantized arenas: the K scales of this lane's 16 keys (requested here,
    // used after the first product)
    [[maybe_unused]] f32x4 ksc[2][2];
    if constexpr (kQ != 0) {
      const float* sl = scale_ring + (t & 1) * kScaleStageFloats;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) ksc[u][hh] = *(const f32x4*)(sl + key_u0 + 32 * u + 4 * hh);
    }
    half8_t kf[2][4];
    auto read_k = [&](int kb, half8_t* f) {
      const int a = 2 * (kb >> 1) + ka;
      const int s = (kslot0 + 4 * (kb & 1)) ^ (4 * (a & 1));
#pragma unroll
      for (int kd = 0; kd < 4; ++kd)
        f[kd] = __builtin_bit_cast(half8_t, kl[a * kUnitsPerBlock + (4 * kd + lq) * 16 + s]);
    };
    read_k(0, kf[0]);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb < 3) read_k(kb + 1, kf[(kb + 1) & 1]);
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) sacc[kb][rb] = (f32x4)0.f;
#pragma unroll
      for (int kd = 0; kd < 4; ++kd)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[kb & 1][kd], qf[rb][kd], sacc[kb][rb], 0, 0, 0);
    }
    if (prefetch_v) {
      read_v(t, 0, vf[0]);
      read_v(t, 1, vf[1]);
    }
    // Instruction order of this block: each LDS read is issued about two
    // products ahead of the first product that needs it, so the read latency
    // hides behind matrix-core work (the scheduler would otherwise place
    // every read right before its use).
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, kRB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    // Quantized arenas: the product of the codes with q times the key's scale
    // is the score of the decoded key (code * scale, exact)
    if constexpr (kQ != 0) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) sacc[kb][rb] *= ksc[kb >> 1][kb & 1];
    }
  };

  // Masks, online softmax and P^T of tile t's scores (pb[u][rb]: B operand
  // of the second product, keys 8(lq & 1) .. +7 of block 2u + (lq >> 1) =
  // scores (kb = 2u, i = 0..3), (kb = 2u + 1, i = 0..3)).
  auto softmax = [&](int t, f32x4 (&sacc)[4][kRB], half8_t (&pb)[2][kRB]) {
    // Causal mask (and keys past the sequence) only where the tile reaches
    // past this wave's smallest row position.  Score (kb, i) of this lane is
    // key 16(2(kb >> 1) + (lq >> 1)) + 8(lq & 1) + 4(kb & 1) + i of the tile.
    if (t * kBN + kBN - 1 > first_pos || t * kBN + kBN > Lc) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int key0 = t * kBN + 16 * (2 * (kb >> 1) + (lq >> 1)) + 8 * (lq & 1) + 4 * (kb & 1);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (key0 + i > prow[rb]) sacc[kb][rb][i] = -INFINITY;
      }
    }

    // online softmax per row (this lane: rows 16rb + lr, 16 keys each).  A
    // row's running maximum is only raised when one of its scores exceeds it
    // by more than the slack (kSlack for fp16 arenas, 0 for quantized ones);
    // both the numerator and the denominator use the same (possibly stale)
    // maximum, so the quotient is unchanged.  The decision is
    // each row's own (rows whose maximum stays get alpha = 1 exactly), so a
    // row's arithmetic does not depend on which rows share its wave.
    float mloc[kRB];
    bool raise = false;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const f32x4 s0 = sacc[0][rb], s1 = sacc[1][rb], s2 = sacc[2][rb], s3 = sacc[3][rb];
      const float a0 = max3f(s0[0], s0[1], s0[2]), a1 = max3f(s0[3], s1[0], s1[1]);
      const float a2 = max3f(s1[2], s1[3], s2[0]), a3 = max3f(s2[1], s2[2], s2[3]);
      const float a4 = max3f(s3[0], s3[1], s3[2]);
      mloc[rb] = max3f(max3f(a0, a1, a2), max3f(a3, a4, s3[3]), a0);
      raise = raise || mloc[rb] > m_lim[rb];
    }
    if (__any(raise)) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        const float mx = max_xor16(max_xor32(mloc[rb]));
        // finite when raised: key 0 is in tile 0 for every row
        const float m_new = mx > m_lim[rb] ? mx : m_raw[rb];
        const float alpha =
            mx > m_lim[rb] ? __builtin_amdgcn_exp2f((m_raw[rb] - m_new) * scale_log2) : 1.f;
        m_raw[rb] = m_new;
        m_lim[rb] = m_new + slack_raw;
        // a row that has seen no key yet (only in a later part of its keys)
        // keeps m_off = 0: its scores are all -inf, so P = 0
        m_off[rb] = m_new == -INFINITY ? 0.f : -m_new * scale_log2;
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[db][rb] *= alpha;
      }
    }

    if constexpr (kQ == 0) {
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; i += 2) {
            const half2_t ph = {
                (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][rb][i], scale_log2, m_off[rb])),
                (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][rb][i + 1], scale_log2, m_off[rb]))};
            lsum = __builtin_amdgcn_fdot2(ph, ones, lsum, false);
            pb[kb >> 1][rb][4 * (kb & 1) + i] = ph[0];
            pb[kb >> 1][rb][4 * (kb & 1) + i + 1] = ph[1];
          }
        l_run[rb] += lsum;
      }
    } else {
      // The V scale (times kPvScale) multiplies the fp32 probability, which
      // is then rounded once to fp16: w = fp16(p * s_v * kPvScale) is the
      // weight the second product gives the exact codes.  The denominator
      // adds w / (s_v * kPvScale), i.e. the same rounded weight in
      // probability units, so numerator and denominator agree key by key
      // (a single dominant key returns its decoded value code * s_v exactly).
      f32x4 vsc[2][2], rsc[2][2];
      const float* sl = scale_ring + (t & 1) * kScaleStageFloats + kBN;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          vsc[u][hh] = *(const f32x4*)(sl + key_u0 + 32 * u + 4 * hh);
          rsc[u][hh] = *(const f32x4*)(sl + kBN + key_u0 + 32 * u + 4 * hh);
        }
#pragma unroll
      for (int rb = 0; rb < kRB; ++rb) {
        float lsum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pe =
                __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][rb][i], scale_log2, m_off[rb]));
            const _Float16 w = (_Float16)(pe * vsc[kb >> 1][kb & 1][i]);
            lsum = __builtin_fmaf((float)w, rsc[kb >> 1][kb & 1][i], lsum);
            pb[kb >> 1][rb][4 * (kb & 1) + i] = w;
          }
        l_run[rb] += lsum;
      }
    }
  };

  // O^T[dim][row] += V^T[dim][key] . P^T[key][row] for tile t.  The V
  // fragments of dims block db + 2 are read before block db's four products
  // (scheduling barriers keep that order).
  auto pv = [&](int t, half8_t (&pb)[2][kRB], half8_t (&vf)[3][2]) {
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      if (db + 2 < 8) read_v(t, db + 2, vf[(db + 2) % 3]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          oacc[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf[db % 3][u], pb[u][rb], oacc[db][rb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int t = tb; t < te; ++t) {
    if constexpr (kQ == 0) {
      // tile t's loads (this wave's) are done; then every wave's, and every
      // wave has finished tile t - 1, whose stage the next load reuses
      if (t + 2 < te) wait_vm<2 * kLoadsPerTile>();
      else if (t + 1 < te) wait_vm<kLoadsPerTile>();
      else wait_vm<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + 3 < te) issue_tile(t + 3);
    } else {
      // code tile t + 1 is in LDS (this wave's loads, then every wave's);
      // after the barrier fp16 and scale stage t & 1 are complete, every wave
      // is done with stage (t + 1) & 1 and with code stage t % 3, which the
      // next load reuses
      if (t + 2 < te) wait_vm<QG::kLoads>();
      else wait_vm<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + 3 < te) issue_codes(t + 3);
      if (t + 1 < te) convert(t + 1);
    }
    if (kQ == 0 && t * kBN + kBN > Lc) {
      zero_v_tail(t);
      __syncthreads();
    }
    f32x4 sacc[4][kRB];
    half8_t vf[3][2];
    half8_t pb[2][kRB];
    qk(t, sacc, vf);
    softmax(t, sacc, pb);
    pv(t, pb, vf);
  }

  // the quantized products carry the V scales times kPvScale
  constexpr float unscale = 1.f / QG::kPvScale;
#pragma unroll
  for (int rb = 0; rb < kRB; ++rb) {
    const float l = sum_xor16(sum_xor32(l_run[rb]));
    const int r = wrow0 + 16 * rb + lr;
    if (r >= C) continue;
    if (parts == 1) {
      const float inv = kQ == 0 ? 1.f / l : unscale / l;
      float* dst = out + ((size_t)(row0 + r) * Hq + h) * kD + 4 * lq;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const f32x4 v = oacc[db][rb] * inv;
        *(f32x4*)(dst + 16 * db) = v;
      }
    } else {
      const size_t pr = ((size_t)part * num_tokens + row0 + r) * Hq + h;
      float* dst = part_o + pr * kD + 4 * lq;
#pragma unroll
      for (int db = 0; db < 8; ++db)
        *(f32x4*)(dst + 16 * db) = kQ == 0 ? oacc[db][rb] : oacc[db][rb] * unscale;
      if (lq == 0) {
        part_ml[2 * pr] = m_raw[rb] == -INFINITY ? -INFINITY : m_raw[rb] * scale_log2;
        part_ml[2 * pr + 1] = l;
      }
    }
  }
}


}  // namespace
}  // namespace pkv
