// prefill.hip -- causal attention of prefill chunks over the paged cache,
// on the matrix cores (v_mfma_f32_16x16x32_f16).
//
// A prefilling sequence asks, in a pass, for the rest of its prompt capped
// by the per-pass token budget, and shares the pass with the decoding
// sequences (deepconcepts.dev, "Continuous Batching Is Not a Bigger Batch",
// section "What the scheduler does on one step": chunked prefill, no
// separate prefill phase).  Its n new tokens were just appended behind the
// ctx - n cached ones; query row k sits at position ctx - n + k and attends
// positions 0 .. ctx - n + k.  Unlike decode, this is a dense contraction
// (n query rows against every key), so it runs on MFMA.
//
// Work-group = 4 waves = 64 query rows of one query head; wave w owns rows
// 16w .. 16w+15.  Per tile of KV_TILE context tokens (gathered from the
// paged pools through the block table into LDS by the whole work-group):
//   S^T = K Q^T     A = K tile rows (LDS), B = the wave's Q rows (registers),
//                   so each lane ends with scores of ONE query row (lane%16)
//                   for 4 tokens per 16-token sub-tile;
//   online softmax  per query row, base 2, row max over the 4 lanes sharing
//                   the row; the O rescale needs no cross-lane traffic since
//                   every lane's O values belong to its own query row;
//   O^T += V^T P^T  B = P straight from the S^T registers (token order chosen
//                   to match), A = V^T read from an LDS copy of the V tile
//                   stored transposed ([d][token]), written with in-register
//                   4x8 transposes while staging.
// Tokens past the tile's last row position are zero-filled in LDS, so stale
// or NaN slots never reach the MFMA accumulators; per-row causal masking is
// a select to -inf on the scores.
//
// Packed rows (PACK): a short chunk -- a few query tokens per sequence, as
// when a decoding sequence verifies several drafted tokens in one pass --
// would fill a 64-row tile of one head with a handful of rows and read the
// same K/V once per query head.  When every chunk has n <= 64 / G tokens,
// one work-group takes all G heads of one KV group instead: tile row
// r = k G + hh is query token k of head g G + hh, so each K/V tile leaves
// HBM once per KV head and the tile holds n G of its 64 rows.
#include <algorithm>
#include <climits>

#include "device_util.h"
#include "fp8_util.h"
#include "kernels.h"
#include "merge.h"

namespace pkv {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;    // query rows per work-group (16 per wave)
constexpr int64_t kCUs = 256;
// work-groups resident per CU (the kernel's occupancy: 3 or 2 waves per SIMD)
constexpr int64_t kGroupsPerCU128 = 3;
constexpr int64_t kGroupsPerCU256 = 2;
constexpr uint32_t kXcds = 8;
using merge::kMaxPrefillSplits;
constexpr int64_t kPackedRounds = 2;  // packed rows: target rounds of resident work-groups
// long-chunk kernels at d = 128 (fp16 and fp8 caches): 256 rows per
// work-group, one per CU, counted in 128-row groups, two per CU
constexpr int64_t kWideRows = 128;
constexpr int64_t kWideGroupsPerCU = 2;
constexpr float kRescaleSlack = 8.f;  // lazy max (base 2): rescale only past m + 8
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int D>
struct PrefillShape {
  static constexpr int KT = D == 128 ? 64 : 32;  // context tokens per tile
  static constexpr int NT = KT / 16;             // 16-token sub-tiles
  static constexpr int KC = D / 32;              // 32-wide d chunks (S^T reduction)
  static constexpr int DT = D / 16;              // 16-row d tiles of O^T
  // K rows: 16-byte fragment reads by 8 lanes of 8 consecutive rows touch
  // all 32 banks once with a row stride of 4 (mod 32) dwords; V^T rows:
  // 8-byte reads by 16 lanes of 16 consecutive rows need 2 (mod 32).
  static constexpr int KSTRIDE = D + 8;          // K tile row stride (fp16)
  static constexpr int VSTRIDE = KT + 4;         // V^T row stride (fp16)
  static constexpr int LDS_BYTES = (KT * KSTRIDE + D * VSTRIDE) * 2;
  static constexpr int kIdTiles = 64;            // tiles whose block ids are staged in LDS
};

// One thread's share of a K/V tile in flight.  fp16 cache: 4 K chunks of 8
// values, and 4 tokens x 8 d values of V (one 4x8 group per thread).  fp8
// cache: the same tokens and columns as codes (2 K chunks of 16, 4 x 8 V
// codes), and one row scale (threads 0 .. KT-1: K of token tid, KT .. 2KT-1:
// V of token tid - KT).
template <bool FP8>
struct TileRegs {
  uint4 k[4];
  uint4 v[4];
};
template <>
struct TileRegs<true> {
  uint4 k[2];
  uint2 v[4];
  float sc;
};

// HPW query heads of one KV group per wave (its 16 rows of each): every K
// and V^T fragment read from LDS feeds HPW MFMAs.  Measured on MI355X, HPW = 2
// needs ~350 registers (one wave per SIMD) and runs slower than HPW = 1 at
// three waves per SIMD, whose waves hide each other's MFMA, LDS and exp
// latencies; only HPW = 1 is launched.
template <int D, int HPW, bool PACK, bool FP8>
__global__ __launch_bounds__(256, HPW == 1 ? (D == 128 ? kGroupsPerCU128 : kGroupsPerCU256) : 1) void prefill_chunk_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k_pool_raw,
    const void* __restrict__ v_pool_raw, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int64_t num_blocks, int32_t num_kv_heads,
    int32_t num_q_heads, const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
    int32_t first_seq, int32_t ctx_clamp, int32_t num_splits, int32_t split_tiles,
    float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml) {
  using S = PrefillShape<D>;
  constexpr int KT = S::KT, NT = S::NT, KC = S::KC, DT = S::DT;
  static_assert(KT * (D / 8) == 4 * 256 && (KT / 4) * (D / 8) == 256, "tile split over 256 threads");
  static_assert(!PACK || HPW == 1, "packed rows carry their own head");
  __shared__ __attribute__((aligned(16))) uint16_t lds[S::LDS_BYTES / 2];
  __shared__ int64_t s_tile_base[S::kIdTiles * (KT / 16)];  // pool offsets of staged blocks
  // fp8: the tile's row scales, K then V (0 for tokens past pos_hi)
  __shared__ __attribute__((aligned(16))) float s_scale[FP8 ? 2 * KT : 4];
  const uint16_t* __restrict__ k_pool = static_cast<const uint16_t*>(k_pool_raw);
  const uint16_t* __restrict__ v_pool = static_cast<const uint16_t*>(v_pool_raw);
  const uint8_t* __restrict__ k_codes = static_cast<const uint8_t*>(k_pool_raw);
  const uint8_t* __restrict__ v_codes = static_cast<const uint8_t*>(v_pool_raw);
  uint16_t* k_lds = lds;                         // [KT][KSTRIDE]
  uint16_t* vt_lds = lds + KT * S::KSTRIDE;      // [D][VSTRIDE]

  const int i = first_seq + blockIdx.z;
  const int G = num_q_heads / num_kv_heads;
  // heads h0 .. h0 + HPW - 1 of one KV group; PACK: all G heads of group y
  const int h0 = PACK ? blockIdx.y * G : blockIdx.y * HPW;
  const int g = h0 / G;
  // PACK: the highest split first -- only long contexts have high splits, so
  // the longest work starts first and short sequences fill in behind it
  const int split = PACK ? num_splits - 1 - (int)(blockIdx.x % num_splits)
                         : (int)(blockIdx.x % num_splits);
  const int tile_row0 = (blockIdx.x / num_splits) * kRows;  // x past the last tile: exits below
  const int row_base = query_start_loc[i];
  const int n = query_start_loc[i + 1] - row_base;
  const int ctx = min(context_lens[i], ctx_clamp);
  const int rows = PACK ? n * G : n;                 // rows of this sequence's row space
  if (n <= 0 || tile_row0 >= rows || ctx < n) return;  // uniform over the work-group
  if (PACK && rows > kRows) return;  // a chunk longer than the host hint (broken contract)
  const int p0 = ctx - n;                            // position of the chunk's first row
  // last position this tile needs (PACK: the tile holds every token of the chunk)
  const int pos_hi = PACK ? ctx - 1 : p0 + min(tile_row0 + kRows, n) - 1;
  const int num_kv_tiles = pos_hi / KT + 1;
  // KV tiles per split: a fixed count (split_tiles > 0: short sequences use
  // fewer splits), or the context cut into num_splits even ranges
  const int per_split =
      split_tiles > 0 ? split_tiles : (num_kv_tiles + num_splits - 1) / num_splits;
  const int kt_begin = split * per_split;
  const int kt_end = min(kt_begin + per_split, num_kv_tiles);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // the same in all its lanes
  const int lrow = lane & 15, lgrp = lane >> 4;
  // This lane's query row (rows past the chunk end reuse the last row; not
  // written): token my_row of the chunk, for heads my_head + hh.
  const int my_row_raw = tile_row0 + 16 * wave + lrow;
  const bool row_valid = my_row_raw < rows;
  const bool wave_live = tile_row0 + 16 * wave < rows;  // the same in all lanes of the wave
  const int my_rr = row_valid ? my_row_raw : rows - 1;
  const int my_row = PACK ? my_rr / G : my_rr;
  const int my_head = PACK ? h0 + (my_rr - my_row * G) : h0;
  const int my_pos = p0 + my_row;
  if (kt_begin >= kt_end) {
    // an empty split (short context, fixed tiles per split): the merge reads
    // only its weight l = 0
    if (row_valid && lgrp == 0) {
      const int64_t first_row = query_start_loc[first_seq];
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) {
        const int64_t pidx =
            ((row_base + my_row - first_row) * num_q_heads + my_head + hh) * num_splits + split;
        part_ml[pidx * 2] = -__builtin_huge_valf();
        part_ml[pidx * 2 + 1] = 0.f;
      }
    }
    return;  // uniform over the work-group
  }

  // Q^T fragments: B operands, lane = query row lrow, 8 d values per 32-wide chunk.
  f16x8 qb[HPW][KC];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const uint16_t* qrow = q + ((int64_t)(row_base + my_row) * num_q_heads + my_head + hh) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qb[hh][c] = *reinterpret_cast<const f16x8*>(qrow + 32 * c + 8 * lgrp);
  }

  f32x4 o[HPW][DT];
  float m_row[HPW], l_row[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
    for (int t = 0; t < DT; ++t) o[hh][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_row[hh] = -__builtin_huge_valf();
    l_row[hh] = 0.f;
  }

  const int32_t* bt_row = block_tables + (int64_t)i * max_blocks_per_seq;
  const int64_t tile_elems = (int64_t)16 * D;
  const int64_t head_off = (int64_t)g * tile_elems;
  const int64_t block_stride = (int64_t)num_kv_heads * tile_elems;
  const int used_blocks = (pos_hi >> 4) + 1;  // table entries this tile range may read
  // Pool offsets of the blocks of this work-group's first kIdTiles tiles,
  // staged once (block ids clamped into the pool); later tiles read the
  // table directly.
  auto block_base = [&](int j) -> int64_t {
    const uint32_t id = j < used_blocks ? (uint32_t)bt_row[j] : 0u;
    return (int64_t)(id < (uint64_t)num_blocks ? id : num_blocks - 1) * block_stride + head_off;
  };
  for (int e = tid; e < S::kIdTiles * (KT / 16); e += 256) {
    const int j = kt_begin * (KT / 16) + e;
    if (j < kt_end * (KT / 16)) s_tile_base[e] = block_base(j);
  }
  __syncthreads();
  // Global -> registers for tile kt; tokens past pos_hi are zeros.
  auto load_tile = [&](TileRegs<FP8>& r, int kt) {
    const int tok0 = kt * KT;
    int64_t tile_base[KT / 16];
#pragma unroll
    for (int b = 0; b < KT / 16; ++b) {
      const int e = (kt - kt_begin) * (KT / 16) + b;
      tile_base[b] = e < S::kIdTiles * (KT / 16) ? s_tile_base[e] : block_base(kt * (KT / 16) + b);
    }
    if constexpr (FP8) {
      // codes: element offsets are byte offsets; a row's scale sits at its
      // element offset / D
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int idx = tid + 256 * j;
        const int tok = idx / (D / 16), ch = idx % (D / 16);
        r.k[j] = uint4{0u, 0u, 0u, 0u};
        if (tok0 + tok <= pos_hi)
          r.k[j] = *reinterpret_cast<const uint4*>(k_codes + tile_base[tok >> 4] +
                                                   (tok & 15) * D + 16 * ch);
      }
      const int tq = tid % (KT / 4), dg = tid / (KT / 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tok = 4 * tq + t;
        r.v[t] = uint2{0u, 0u};
        if (tok0 + tok <= pos_hi)
          r.v[t] = *reinterpret_cast<const uint2*>(v_codes + tile_base[tok >> 4] +
                                                   (tok & 15) * D + 8 * dg);
      }
      r.sc = 0.f;
      const int stok = tid % KT;
      if (tid < 2 * KT && tok0 + stok <= pos_hi)
        r.sc = (tid < KT ? k_scale : v_scale)[tile_base[stok >> 4] / D + (stok & 15)];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 256 * j;
        const int tok = idx / (D / 8), ch = idx % (D / 8);
        r.k[j] = uint4{0u, 0u, 0u, 0u};
        if (tok0 + tok <= pos_hi)
          r.k[j] = *reinterpret_cast<const uint4*>(k_pool + tile_base[tok >> 4] +
                                                   (tok & 15) * D + 8 * ch);
      }
      const int tq = tid % (KT / 4), dg = tid / (KT / 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tok = 4 * tq + t;
        r.v[t] = uint4{0u, 0u, 0u, 0u};
        if (tok0 + tok <= pos_hi)
          r.v[t] = *reinterpret_cast<const uint4*>(v_pool + tile_base[tok >> 4] + (tok & 15) * D +
                                                   8 * dg);
      }
    }
  };
  // Registers -> LDS: K row-major, V transposed to [d][token] (4x8 transpose).
  // fp8: codes are turned into fp16 here (exact), so the tiles in LDS and
  // the MFMAs are those of the fp16 cache; the row scales go to s_scale.
  auto store_tile = [&](const TileRegs<FP8>& r) {
    uint4 vh[4];
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int idx = tid + 256 * j;
        const int tok = idx / (D / 16), ch = idx % (D / 16);
        uint4 lo, hi;
        fp8x16_to_h16(r.k[j], lo, hi);
        *reinterpret_cast<uint4*>(k_lds + tok * S::KSTRIDE + 16 * ch) = lo;
        *reinterpret_cast<uint4*>(k_lds + tok * S::KSTRIDE + 16 * ch + 8) = hi;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) vh[t] = fp8x8_to_h8(r.v[t]);
      if (tid < 2 * KT) s_scale[tid] = r.sc;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 256 * j;
        const int tok = idx / (D / 8), ch = idx % (D / 8);
        *reinterpret_cast<uint4*>(k_lds + tok * S::KSTRIDE + 8 * ch) = r.k[j];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) vh[t] = r.v[t];
    }
    const int tq = tid % (KT / 4), dg = tid / (KT / 4);
    const uint32_t w0[4] = {vh[0].x, vh[0].y, vh[0].z, vh[0].w};
    const uint32_t w1[4] = {vh[1].x, vh[1].y, vh[1].z, vh[1].w};
    const uint32_t w2[4] = {vh[2].x, vh[2].y, vh[2].z, vh[2].w};
    const uint32_t w3[4] = {vh[3].x, vh[3].y, vh[3].z, vh[3].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int w = j >> 1;
      uint2 col;
      if (j & 1) {
        col.x = (w0[w] >> 16) | (w1[w] & 0xffff0000u);
        col.y = (w2[w] >> 16) | (w3[w] & 0xffff0000u);
      } else {
        col.x = (w0[w] & 0xffffu) | (w1[w] << 16);
        col.y = (w2[w] & 0xffffu) | (w3[w] << 16);
      }
      *reinterpret_cast<uint2*>(vt_lds + (8 * dg + j) * S::VSTRIDE + 4 * tq) = col;
    }
  };

  // fp8: O is kept in units of vref, the largest V row scale of the current
  // tile (a power of two; O is rescaled, exactly, when the next tile's
  // differs), so that every fp16 weight p 2^(e_t) / vref stays <= p and
  // loses range only against the rows of its own tile
  float vref = 0.f, inv_vref = 0.f;
  TileRegs<FP8> next;
  if (kt_begin < kt_end) load_tile(next, kt_begin);
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int tok0 = kt * KT;
    __syncthreads();  // the previous tile's LDS reads are done
    store_tile(next);
    if (kt + 1 < kt_end) load_tile(next, kt + 1);  // in flight during this tile's math
    __syncthreads();
    // A wave whose 16 rows are all past the row space (packed short chunks:
    // n G rows of the 64) only stages tiles: no fragment reads, no math.
    if (!wave_live) continue;

    // S^T = K Q^T: s[hh][t][e] = score of head h0+hh, query row lrow, with
    // token tok0 + 16t + 4*lgrp + e.  Each K fragment feeds HPW MFMAs.
    f32x4 s[HPW][NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int hh = 0; hh < HPW; ++hh) s[hh][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(k_lds + (16 * t + lrow) * S::KSTRIDE +
                                                         32 * c + 8 * lgrp);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) s[hh][t] = mfma16(a, qb[hh][c], s[hh][t]);
      }
    }
    // fp8: scores times the K row scales (exact: powers of two); the V row
    // scales of this lane's tokens relative to vref
    float vrel[NT][4];
    if constexpr (FP8) {
      float vmax = 0.f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4 ks = *reinterpret_cast<const float4*>(s_scale + 16 * t + 4 * lgrp);
        const float4 vs = *reinterpret_cast<const float4*>(s_scale + KT + 16 * t + 4 * lgrp);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          s[hh][t][0] *= ks.x;
          s[hh][t][1] *= ks.y;
          s[hh][t][2] *= ks.z;
          s[hh][t][3] *= ks.w;
        }
        vrel[t][0] = vs.x;
        vrel[t][1] = vs.y;
        vrel[t][2] = vs.z;
        vrel[t][3] = vs.w;
        vmax = fmaxf(fmaxf(vmax, fmaxf(vs.x, vs.y)), fmaxf(vs.z, vs.w));
      }
      // lanes of one lgrp hold the same tokens; the four groups cover the tile
      vmax = max_of_rows(vmax);
      if (vmax != vref) {  // the same in every lane and wave
        const float ratio = vref / vmax;  // exact: powers of two (0 before the first tile)
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
          for (int t = 0; t < DT; ++t) o[hh][t] *= ratio;
        vref = vmax;
        inv_vref = 1.f / vmax;
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) vrel[t][e] *= inv_vref;
    }

    // Online softmax per (head, row), base 2.  Off the diagonal every token
    // is visible and the scale goes into the exp's argument (one FMA per
    // score, extreme taken on raw scores); on tiles that cross the diagonal
    // of this work-group's rows the scores are scaled first and masked to
    // -inf.  P^T as B operands: chunk c2 covers sub-tiles 2*c2 (elements
    // 0..3) and 2*c2+1 (4..7), converted in pairs; l sums exactly the
    // rounded weights.
    const bool diagonal = tok0 + KT - 1 > p0 + (PACK ? 0 : tile_row0);
    f16x8 pb[HPW][NT / 2];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      float sc = scale_log2;
      if (diagonal) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = s[hh][t][e] * scale_log2;
            s[hh][t][e] = tok0 + 16 * t + 4 * lgrp + e > my_pos ? -__builtin_huge_valf() : x;
          }
        sc = 1.f;
      }
      float ext = s[hh][0][0];
      if (sc >= 0.f) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) ext = fmaxf(ext, s[hh][t][e]);
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) ext = fminf(ext, s[hh][t][e]);
      }
      float tile_max = ext * sc;
      tile_max = max_of_rows(tile_max);
      // Lazy max: the reference only moves when a score passes it by more
      // than kRescaleSlack (weights stay <= 2^8, exact in fp16 range), so
      // after the first tiles the O rescale is skipped by the whole wave.
      if (__any(tile_max > m_row[hh] + kRescaleSlack)) {
        const float m_new = tile_max > m_row[hh] + kRescaleSlack ? tile_max : m_row[hh];
        // A row that has seen no visible token keeps weight 0 (no -inf - -inf).
        const float alpha = m_new == -__builtin_huge_valf() ? 1.f : fast_exp2(m_row[hh] - m_new);
        m_row[hh] = m_new;
        l_row[hh] *= alpha;
#pragma unroll
        for (int t = 0; t < DT; ++t) o[hh][t] *= alpha;
      }
      const float neg_ref = m_row[hh] == -__builtin_huge_valf() ? 0.f : -m_row[hh];
#pragma unroll
      for (int c2 = 0; c2 < NT / 2; ++c2) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4& sv = s[hh][2 * c2 + j / 2];
          const float p0 = fast_exp2(__builtin_fmaf(sv[2 * (j % 2)], sc, neg_ref));
          const float p1 = fast_exp2(__builtin_fmaf(sv[2 * (j % 2) + 1], sc, neg_ref));
          w[j] = pack_h2_rtz(p0, p1);
          l_row[hh] = dot2(w[j], kOnesH2, l_row[hh]);
          if constexpr (FP8)  // the same rounded weights, times 2^(e_t) / vref
            w[j] = pack_h2_rtz(p0 * vrel[2 * c2 + j / 2][2 * (j % 2)],
                               p1 * vrel[2 * c2 + j / 2][2 * (j % 2) + 1]);
        }
        pb[hh][c2] = __builtin_bit_cast(f16x8, uint4{w[0], w[1], w[2], w[3]});
      }
    }

    // O^T += V^T P^T; A lane = d row 16*dt + lrow, tokens matching pb's order;
    // each V^T fragment feeds HPW MFMAs.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int c2 = 0; c2 < NT / 2; ++c2) {
        const uint16_t* vrow = vt_lds + (16 * dt + lrow) * S::VSTRIDE + 32 * c2 + 4 * lgrp;
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        const uint4 packed = {lo.x, lo.y, hi.x, hi.y};
        const f16x8 a = __builtin_bit_cast(f16x8, packed);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) o[hh][dt] = mfma16(a, pb[hh][c2], o[hh][dt]);
      }
  }

#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    l_row[hh] = sum_of_rows(l_row[hh]);
  }
  if (!row_valid) return;
  const int64_t first_row = query_start_loc[first_seq];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float inv = l_row[hh] > 0.f ? (FP8 ? vref : 1.f) / l_row[hh] : 0.f;
    const int64_t row_head = (int64_t)(row_base + my_row) * num_q_heads + my_head + hh;
    if (num_splits == 1) {
      uint16_t* dst = out + row_head * D + 4 * lgrp;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint2 w;
        w.x = pack_h2_rne(o[hh][dt][0] * inv, o[hh][dt][1] * inv);
        w.y = pack_h2_rne(o[hh][dt][2] * inv, o[hh][dt][3] * inv);
        *reinterpret_cast<uint2*>(dst + 16 * dt) = w;
      }
      continue;
    }
    // Partial of this split: (o / l, m, l); l = 0 when no position was visible.
    const int64_t pidx =
        ((row_base + my_row - first_row) * num_q_heads + my_head + hh) * num_splits + split;
    float* dst = part_o + pidx * D + 4 * lgrp;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[hh][dt] * inv;
    if (lane < 16) {
      part_ml[pidx * 2] = m_row[hh];
      part_ml[pidx * 2 + 1] = l_row[hh];
    }
  }
}

// Merge of the splits of every (prefill row, query head): one wave each.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ query_start_loc, int32_t first_seq, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_splits, int64_t max_row_heads, uint16_t* __restrict__ out) {
  merge::chunk_merge_row_head<D>(part_o, part_ml, query_start_loc, first_seq, num_seqs,
                                 num_q_heads, num_splits, max_row_heads, out,
                                 (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6));
}

// The step's combined merge: the decode part's merge left by its launch (work-
// groups 0 .. dm.groups - 1: partition grid rows or schedule pieces) and the
// chunks' merge (the rest, four (row, head) pairs each) in one launch after
// the prefill kernel.  They write different rows of `out`.
template <int D>
__global__ __launch_bounds__(256) void step_merge_kernel(
    DecodeMerge dm, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ query_start_loc, int32_t first_seq, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_splits, int64_t max_row_heads, uint16_t* __restrict__ out) {
  const int64_t w = blockIdx.x;
  if (w < dm.groups) {  // uniform over the work-group
    if (dm.pieces)
      merge::piece_merge_unit<D>(dm.sched, dm.units, dm.sched_groups, dm.num_kv_heads, dm.group,
                                 dm.part_o, dm.part_ml, out, (int32_t)(w / dm.group),
                                 (int32_t)(w % dm.group));
    else
      merge::lse_merge_row<D>(dm.part_o, dm.part_ml, dm.context_lens, dm.ctx_clamp,
                              dm.partition_blocks, dm.max_parts, dm.num_q_heads, out, (int)w);
    return;
  }
  merge::chunk_merge_row_head<D>(part_o, part_ml, query_start_loc, first_seq, num_seqs,
                                 num_q_heads, num_splits, max_row_heads, out,
                                 (w - dm.groups) * 4 + (threadIdx.x >> 6));
}

}  // namespace

PrefillPlan plan_prefill(int32_t num_prefill_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t max_context_len, int32_t max_query_len,
                         int32_t kv_partition_tokens) {
  PrefillPlan plan{};
  plan.splits = 1;
  if (num_prefill_seqs <= 0) return plan;
  const int32_t kt = head_dim == 128 ? PrefillShape<128>::KT : PrefillShape<256>::KT;
  // every chunk's G n rows fit one tile: one work-group per (sequence, KV head)
  plan.packed = (int64_t)max_query_len * (num_q_heads / num_kv_heads) <= kRows;
  const int64_t groups =
      plan.packed ? (int64_t)num_prefill_seqs * num_kv_heads
                  : (int64_t)num_prefill_seqs * ((max_query_len + kRows - 1) / kRows) * num_q_heads;
  const int64_t kv_tiles = (max_context_len + kt - 1) / kt;
  const int64_t resident = kCUs * (head_dim == 128 ? kGroupsPerCU128 : kGroupsPerCU256);
  if (plan.packed) {
    // A fixed number of KV tiles per split, so that a long context gets more
    // splits than a short one: about kPackedRounds rounds of resident
    // work-groups if every context had the longest length.
    int64_t per = kv_partition_tokens > 0
                      ? std::max<int64_t>(1, kv_partition_tokens / kt)
                      : (groups * kv_tiles + kPackedRounds * resident - 1) / (kPackedRounds * resident);
    per = std::max<int64_t>(std::max<int64_t>(per, 1),
                            (kv_tiles + kMaxPrefillSplits - 1) / kMaxPrefillSplits);
    plan.splits = (int32_t)((kv_tiles + per - 1) / per);
    plan.split_tiles = plan.splits > 1 ? (int32_t)per : 0;
  } else if (head_dim == 128) {
    // long chunks at d = 128 (prefill_wide.hip): splits for one round of
    // resident work-groups, counted in 128-row groups, two per CU
    plan.wide = true;
    const int64_t wide_groups =
        (int64_t)num_prefill_seqs * ((max_query_len + kWideRows - 1) / kWideRows) * num_q_heads;
    int64_t splits = kCUs * kWideGroupsPerCU / wide_groups;
    splits = std::min<int64_t>(std::min<int64_t>(splits, kMaxPrefillSplits), kv_tiles);
    plan.splits = (int32_t)std::max<int64_t>(splits, 1);
    plan.split_tiles = 0;
  } else {
    // as many splits as fit in one round of resident work-groups (no tail round)
    int64_t splits = resident / groups;
    splits = std::min<int64_t>(std::min<int64_t>(splits, kMaxPrefillSplits), kv_tiles);
    plan.splits = (int32_t)std::max<int64_t>(splits, 1);
    plan.split_tiles = 0;
  }
  plan.max_row_heads = (int64_t)num_prefill_seqs * max_query_len * num_q_heads;
  plan.partial_bytes =
      plan.splits > 1 ? (size_t)plan.max_row_heads * plan.splits * (head_dim + 2) * sizeof(float)
                      : 0;
  return plan;
}

// The chunks' merge (when split), with the decode part's merge folded in when
// its launch left one.
template <int D>
static hipError_t launch_chunk_merges(const PrefillPlan& plan, const float* part_o,
                                      const float* part_ml, const int32_t* query_start_loc,
                                      int32_t first_seq, int32_t num_prefill_seqs,
                                      int32_t num_q_heads, void* out, const DecodeMerge* fold,
                                      hipStream_t stream) {
  const int64_t chunk_groups = plan.splits > 1 ? (plan.max_row_heads + 3) / 4 : 0;
  const int64_t dec_groups = fold ? fold->groups : 0;
  if (chunk_groups + dec_groups == 0) return hipSuccess;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  if (dec_groups == 0)
    hipLaunchKernelGGL(prefill_merge_kernel<D>, dim3((uint32_t)chunk_groups), dim3(256), 0,
                       stream, part_o, part_ml, query_start_loc, first_seq,
                       first_seq + num_prefill_seqs, num_q_heads, plan.splits,
                       plan.max_row_heads, static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL(step_merge_kernel<D>, dim3((uint32_t)(dec_groups + chunk_groups)),
                       dim3(256), 0, stream, *fold, part_o, part_ml, query_start_loc, first_seq,
                       first_seq + num_prefill_seqs, num_q_heads, plan.splits,
                       plan.max_row_heads, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

template <int D, bool FP8>
static hipError_t launch_prefill_d(const void* q, const void* k_pool, const void* v_pool,
                                   const float* k_scale, const float* v_scale, int64_t num_blocks, int32_t num_kv_heads, int32_t num_q_heads,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, const int32_t* query_start_loc,
                                   int32_t first_seq, int32_t num_prefill_seqs,
                                   int32_t max_query_len, float scale, const PrefillPlan& plan,
                                   void* out, void* workspace, hipStream_t stream,
                                   const DecodeMerge* fold) {
  const int32_t ctx_clamp =
      (int32_t)std::min<int64_t>((int64_t)max_blocks_per_seq * 16, INT32_MAX);
  float* part_o = static_cast<float*>(workspace);
  float* part_ml = part_o ? part_o + (size_t)plan.max_row_heads * plan.splits * D : nullptr;
  hipError_t err;
  if (plan.wide) {
    err = launch_prefill_wide(q, k_pool, v_pool, k_scale, v_scale, num_blocks, num_kv_heads,
                              num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                              query_start_loc, first_seq, num_prefill_seqs, max_query_len, scale,
                              plan.splits, out, part_o, part_ml, stream);
    if (err != hipSuccess) return err;
    return launch_chunk_merges<D>(plan, part_o, part_ml, query_start_loc, first_seq,
                                  num_prefill_seqs, num_q_heads, out, fold, stream);
  }
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  if (plan.packed) {
    // x = split, y = KV head: each work-group holds all heads of its group
    const dim3 grid((uint32_t)plan.splits, num_kv_heads, num_prefill_seqs);
    hipLaunchKernelGGL((prefill_chunk_kernel<D, 1, true, FP8>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), k_pool, v_pool, k_scale, v_scale,
                       num_blocks, num_kv_heads,
                       num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                       query_start_loc, first_seq, ctx_clamp, plan.splits, plan.split_tiles,
                       scale * kLog2e,
                       static_cast<uint16_t*>(out), part_o, part_ml);
  } else {
    // x = (query tile, split), padded to a multiple of the 8 XCDs: work-groups
    // are dealt round-robin over the XCDs, so every head of one (tile, split)
    // -- in particular the G heads sharing one KV head -- runs on one XCD and
    // reads the K/V tiles through the same L2.
    const uint32_t x = ((max_query_len + kRows - 1) / kRows) * plan.splits;
    const dim3 grid((x + kXcds - 1) / kXcds * kXcds, num_q_heads, num_prefill_seqs);
    hipLaunchKernelGGL((prefill_chunk_kernel<D, 1, false, FP8>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), k_pool, v_pool, k_scale, v_scale,
                       num_blocks, num_kv_heads,
                       num_q_heads, block_tables, max_blocks_per_seq, context_lens,
                       query_start_loc, first_seq, ctx_clamp, plan.splits, plan.split_tiles,
                       scale * kLog2e,
                       static_cast<uint16_t*>(out), part_o, part_ml);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_chunk_merges<D>(plan, part_o, part_ml, query_start_loc, first_seq,
                                num_prefill_seqs, num_q_heads, out, fold, stream);
}

hipError_t launch_prefill(const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scale, const float* v_scale, int64_t num_blocks,
                          int32_t num_kv_heads, int32_t num_q_heads, int32_t head_dim,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, const int32_t* query_start_loc,
                          int32_t first_seq, int32_t num_prefill_seqs, int32_t max_query_len,
                          float scale, const PrefillPlan& plan, void* out, void* workspace,
                          hipStream_t stream, const DecodeMerge* fold) {
  if (num_prefill_seqs <= 0) return hipSuccess;
  const bool fp8 = k_scale != nullptr;
#define PKV_PREFILL_ARGS                                                                      \
  q, k_pool, v_pool, k_scale, v_scale, num_blocks, num_kv_heads, num_q_heads, block_tables,  \
      max_blocks_per_seq, context_lens, query_start_loc, first_seq, num_prefill_seqs,         \
      max_query_len, scale, plan, out, workspace, stream, fold
  if (head_dim == 128)
    return fp8 ? launch_prefill_d<128, true>(PKV_PREFILL_ARGS)
               : launch_prefill_d<128, false>(PKV_PREFILL_ARGS);
  if (head_dim == 256)
    return fp8 ? launch_prefill_d<256, true>(PKV_PREFILL_ARGS)
               : launch_prefill_d<256, false>(PKV_PREFILL_ARGS);
#undef PKV_PREFILL_ARGS
  return hipErrorInvalidValue;
}

}  // namespace pkv
