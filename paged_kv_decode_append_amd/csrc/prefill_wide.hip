// prefill_wide.hip -- causal attention of long prefill chunks (head_dim 128)
// on the matrix cores with 32 query rows per wave (v_mfma_f32_32x32x16_f16).
//
// A prefilling sequence shares the pass with the decoding ones and brings
// up to the per-pass token budget of its prompt (deepconcepts.dev,
// "Continuous Batching Is Not a Bigger Batch", section "What the scheduler
// does on one step"); query row k of a chunk of n rows sits at position
// ctx - n + k and attends positions 0 .. ctx - n + k.
//
// Both kernels here give each wave 32 query rows, so one 32x32x16 product
// consumes a 1 KiB K or V fragment for twice the flops of a 16-row wave:
// half the LDS bytes per flop, which with the exps is what bounds the
// contraction on CDNA4 (measured per SIMD: a 32x32x16 product ~42 cycles, a
// wave64 v_exp_f32 ~13, a 1 KiB ds_read_b128 ~20 and a 512-byte transposing
// ds_read_b64_tr_b16 ~18, and they overlap only in part).
//
// Per tile of 64 context tokens, in both:
//   S^T = K Q^T     A = K rows (LDS), B = the wave's Q rows (registers); lane
//                   l ends with query row l % 32 for 16 of each 32 tokens
//                   (tokens 8 (r / 4) + 4 (l / 32) + r % 4 in register r);
//   online softmax  per query row, base 2, lazy max; a row's scores sit in
//                   lanes l and l ^ 32 (one exchange);
//   O^T += V^T P^T  B = P straight from the S^T registers (registers 8h ..
//                   8h + 7 of a sub-tile are one 16-token product step), A =
//                   V^T in the same token order (two 4-token reads);
//                   O^T tile dt holds d = 32 dt + 8 (r / 4) + 4 (l / 32) +
//                   r % 4 of row l % 32 in register r.
// Causal masking is a select to -inf.
//
// prefill_wide_kernel (fp8 cache): work-group = 4 waves = 128 rows of one
// query head, two per CU.  The tile is gathered from the paged pools into
// registers by the whole work-group one tile ahead, the codes turned into
// fp16 (exact), and stored to LDS, K row-major and V transposed to
// [d][token]; tokens past the tile's last row position are zero-filled.  The
// K row scales multiply the scores and the V row scales the weights
// (relative to vref, the tile's largest V scale; O is kept in units of
// vref), as in the 16-row kernel.
//
// prefill_wide_dma_kernel (fp16 cache): work-group = 8 waves = 256 rows of
// one query head, one per CU; the tiles go from the pools straight into
// 4-deep LDS rings three tiles ahead (described with the kernel).
#include <algorithm>
#include <climits>

#include "device_util.h"
#include "fp8_util.h"
#include "kernels.h"

namespace pkv {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int kWideRows = 128;      // query rows per work-group (32 per wave)
constexpr int KT = 64;              // context tokens per tile
constexpr int KSTRIDE = kD + 8;     // K tile row stride (fp16): 16-byte reads of 8 rows conflict-free
constexpr int VSTRIDE = KT + 4;     // V^T row stride (fp16): 8-byte reads of 16 rows conflict-free
constexpr int kIdTiles = 64;        // tiles whose block offsets are staged in LDS
constexpr float kRescaleSlack = 8.f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <bool FP8>
struct WideTile {
  uint4 k[4];  // token idx / 16, 8 values at column 8 (idx % 16), idx = tid + 256 j
  uint4 v[4];  // tokens 4 (tid % 16) + t, 8 values at column 8 (tid / 16)
};
template <>
struct WideTile<true> {
  uint4 k[2];  // token idx / 8, 16 codes at column 16 (idx % 8)
  uint2 v[4];
  float sc;    // threads 0 .. 63: K scale of token tid, 64 .. 127: V scale of token tid - 64
};

template <bool FP8>
__global__ __launch_bounds__(256, 2) void prefill_wide_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ k_pool_raw,
    const void* __restrict__ v_pool_raw, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int64_t num_blocks, int32_t num_kv_heads,
    int32_t num_q_heads, const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
    int32_t first_seq, int32_t ctx_clamp, int32_t num_splits, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[KT * KSTRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[kD * VSTRIDE];
  __shared__ int64_t s_tile_base[kIdTiles * (KT / 16)];
  __shared__ __attribute__((aligned(16))) float s_scale[FP8 ? 2 * KT : 4];
  const uint16_t* __restrict__ k_pool = static_cast<const uint16_t*>(k_pool_raw);
  const uint16_t* __restrict__ v_pool = static_cast<const uint16_t*>(v_pool_raw);
  const uint8_t* __restrict__ k_codes = static_cast<const uint8_t*>(k_pool_raw);
  const uint8_t* __restrict__ v_codes = static_cast<const uint8_t*>(v_pool_raw);

  const int i = first_seq + blockIdx.z;
  const int G = num_q_heads / num_kv_heads;
  const int head = blockIdx.y;
  const int g = head / G;
  const int split = (int)(blockIdx.x % num_splits);
  const int tile_row0 = (blockIdx.x / num_splits) * kWideRows;  // past the last tile: exits
  const int row_base = query_start_loc[i];
  const int n = query_start_loc[i + 1] - row_base;
  const int ctx = min(context_lens[i], ctx_clamp);
  if (n <= 0 || tile_row0 >= n || ctx < n) return;  // uniform over the work-group
  const int p0 = ctx - n;
  const int pos_hi = p0 + min(tile_row0 + kWideRows, n) - 1;
  const int num_kv_tiles = pos_hi / KT + 1;
  const int per_split = (num_kv_tiles + num_splits - 1) / num_splits;
  const int kt_begin = split * per_split;
  const int kt_end = min(kt_begin + per_split, num_kv_tiles);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int my_row_raw = tile_row0 + 32 * wave + lrow;
  const bool row_valid = my_row_raw < n;
  const bool wave_live = tile_row0 + 32 * wave < n;  // the same in all lanes of the wave
  const int my_row = row_valid ? my_row_raw : n - 1;
  const int my_pos = p0 + my_row;
  const int64_t first_row = query_start_loc[first_seq];
  if (kt_begin >= kt_end) {
    // an empty split: the merge reads only its weight l = 0
    if (row_valid && lgrp == 0) {
      const int64_t pidx =
          ((row_base + my_row - first_row) * num_q_heads + head) * num_splits + split;
      part_ml[pidx * 2] = -__builtin_huge_valf();
      part_ml[pidx * 2 + 1] = 0.f;
    }
    return;  // uniform over the work-group
  }

  // Q^T fragments (B operands): row my_row, d = 16 c + 8 lgrp .. +7
  f16x8 qb[kD / 16];
  {
    const uint16_t* qrow = q + ((int64_t)(row_base + my_row) * num_q_heads + head) * kD;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c)
      qb[c] = *reinterpret_cast<const f16x8*>(qrow + 16 * c + 8 * lgrp);
  }
  f32x16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_row = -__builtin_huge_valf(), l_row = 0.f;

  const int32_t* bt_row = block_tables + (int64_t)i * max_blocks_per_seq;
  const int64_t tile_elems = (int64_t)16 * kD;
  const int64_t head_off = (int64_t)g * tile_elems;
  const int64_t block_stride = (int64_t)num_kv_heads * tile_elems;
  const int used_blocks = (pos_hi >> 4) + 1;
  auto block_base = [&](int j) -> int64_t {
    const uint32_t id = j < used_blocks ? (uint32_t)bt_row[j] : 0u;
    return (int64_t)(id < (uint64_t)num_blocks ? id : num_blocks - 1) * block_stride + head_off;
  };
  for (int e = tid; e < kIdTiles * (KT / 16); e += 256) {
    const int j = kt_begin * (KT / 16) + e;
    if (j < kt_end * (KT / 16)) s_tile_base[e] = block_base(j);
  }
  __syncthreads();

  // Global -> registers for tile kt; tokens past pos_hi are zeros.
  auto load_tile = [&](WideTile<FP8>& r, int kt) {
    const int tok0 = kt * KT;
    int64_t tile_base[KT / 16];
#pragma unroll
    for (int b = 0; b < KT / 16; ++b) {
      const int e = (kt - kt_begin) * (KT / 16) + b;
      tile_base[b] = e < kIdTiles * (KT / 16) ? s_tile_base[e] : block_base(kt * (KT / 16) + b);
    }
    const int tq = tid % (KT / 4), dg = tid / (KT / 4);
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int idx = tid + 256 * j;
        const int tok = idx / (kD / 16), ch = idx % (kD / 16);
        r.k[j] = uint4{0u, 0u, 0u, 0u};
        if (tok0 + tok <= pos_hi)
          r.k[j] = *reinterpret_cast<const uint4*>(k_codes + tile_base[tok >> 4] +
                                                   (tok & 15) * kD + 16 * ch);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tok = 4 * tq + t;
        r.v[t] = uint2{0u, 0u};
        if (tok0 + tok <= pos_hi)
          r.v[t] = *reinterpret_cast<const uint2*>(v_codes + tile_base[tok >> 4] +
                                                   (tok & 15) * kD + 8 * dg);
      }
      r.sc = 0.f;
      const int stok = tid % KT;
      if (tid < 2 * KT && tok0 + stok <= pos_hi)
        r.sc = (tid < KT ? k_scale : v_scale)[tile_base[stok >> 4] / kD + (stok & 15)];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 256 * j;
        const int tok = idx / (kD / 8), ch = idx % (kD / 8);
        r.k[j] = uint4{0u, 0u, 0u, 0u};
        if (tok0 + tok <= pos_hi)
          r.k[j] = *reinterpret_cast<const uint4*>(k_pool + tile_base[tok >> 4] +
                                                   (tok & 15) * kD + 8 * ch);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int tok = 4 * tq + t;
        r.v[t] = uint4{0u, 0u, 0u, 0u};
        if (tok0 + tok <= pos_hi)
          r.v[t] = *reinterpret_cast<const uint4*>(v_pool + tile_base[tok >> 4] +
                                                   (tok & 15) * kD + 8 * dg);
      }
    }
  };
  // Registers -> LDS: K row-major, V transposed to [d][token] (4x8 transposes).
  auto store_tile = [&](const WideTile<FP8>& r) {
    uint4 vh[4];
    if constexpr (FP8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int idx = tid + 256 * j;
        const int tok = idx / (kD / 16), ch = idx % (kD / 16);
        uint4 lo, hi;
        fp8x16_to_h16(r.k[j], lo, hi);
        *reinterpret_cast<uint4*>(k_lds + tok * KSTRIDE + 16 * ch) = lo;
        *reinterpret_cast<uint4*>(k_lds + tok * KSTRIDE + 16 * ch + 8) = hi;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) vh[t] = fp8x8_to_h8(r.v[t]);
      if (tid < 2 * KT) s_scale[tid] = r.sc;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = tid + 256 * j;
        const int tok = idx / (kD / 8), ch = idx % (kD / 8);
        *reinterpret_cast<uint4*>(k_lds + tok * KSTRIDE + 8 * ch) = r.k[j];
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
      *reinterpret_cast<uint2*>(vt_lds + (8 * dg + j) * VSTRIDE + 4 * tq) = col;
    }
  };

  float vref = 0.f, inv_vref = 0.f;
  WideTile<FP8> next;
  load_tile(next, kt_begin);
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    const int tok0 = kt * KT;
    __syncthreads();  // the previous tile's LDS reads are done
    store_tile(next);
    if (kt + 1 < kt_end) load_tile(next, kt + 1);  // in flight during this tile's math
    __syncthreads();
    if (!wave_live) continue;  // rows all past the chunk: stage only

    // S^T = K Q^T for the tile's two 32-token sub-tiles
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
#pragma unroll
      for (int c = 0; c < kD / 16; ++c) {
        const f16x8 a = *reinterpret_cast<const f16x8*>(k_lds + (32 * st + lrow) * KSTRIDE +
                                                         16 * c + 8 * lgrp);
        s[st] = mfma32(a, qb[c], s[st]);
      }
    }
    // token of register r of sub-tile st (relative to tok0)
    auto tok_of = [&](int st, int r) { return 32 * st + 8 * (r >> 2) + 4 * lgrp + (r & 3); };
    if constexpr (FP8) {
      float vmax = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int t0 = 32 * st + 8 * qq + 4 * lgrp;
          const float4 ks = *reinterpret_cast<const float4*>(s_scale + t0);
          const float4 vs = *reinterpret_cast<const float4*>(s_scale + KT + t0);
          s[st][4 * qq + 0] *= ks.x;
          s[st][4 * qq + 1] *= ks.y;
          s[st][4 * qq + 2] *= ks.z;
          s[st][4 * qq + 3] *= ks.w;
          vmax = fmaxf(fmaxf(vmax, fmaxf(vs.x, vs.y)), fmaxf(vs.z, vs.w));
        }
      vmax = fmaxf(vmax, __shfl_xor(vmax, 32));  // the two lane halves cover the tile
      if (vmax != vref) {  // the same in every lane and wave
        const float ratio = vref / vmax;  // exact: powers of two (0 before the first tile)
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) o[dt] *= ratio;
        vref = vmax;
        inv_vref = 1.f / vmax;
      }
    }

    // Online softmax of row my_row, base 2 (as in the 16-row kernel: off the
    // diagonal the scale goes into the exp's argument, on tiles crossing the
    // diagonal the scores are scaled first and masked).
    const bool diagonal = tok0 + KT - 1 > p0 + tile_row0;
    float sc = scale_log2;
    if (diagonal) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = s[st][r] * scale_log2;
          s[st][r] = tok0 + tok_of(st, r) > my_pos ? -__builtin_huge_valf() : x;
        }
      sc = 1.f;
    }
    float ext = s[0][0];
    if (sc >= 0.f) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) ext = fmaxf(ext, s[st][r]);
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) ext = fminf(ext, s[st][r]);
    }
    float tile_max = ext * sc;
    tile_max = fmaxf(tile_max, __shfl_xor(tile_max, 32));
    if (__any(tile_max > m_row + kRescaleSlack)) {
      const float m_new = tile_max > m_row + kRescaleSlack ? tile_max : m_row;
      const float alpha = m_new == -__builtin_huge_valf() ? 1.f : fast_exp2(m_row - m_new);
      m_row = m_new;
      l_row *= alpha;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) o[dt] *= alpha;
    }
    const float neg_ref = m_row == -__builtin_huge_valf() ? 0.f : -m_row;
    // P^T as B operands: product step (st, hf) takes registers 8 hf .. 8 hf + 7
    f16x8 pb[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 8 * hf + 2 * j;
          const float e0 = fast_exp2(__builtin_fmaf(s[st][r], sc, neg_ref));
          const float e1 = fast_exp2(__builtin_fmaf(s[st][r + 1], sc, neg_ref));
          w[j] = pack_h2_rtz(e0, e1);
          l_row = dot2(w[j], kOnesH2, l_row);
          if constexpr (FP8) {  // the same rounded weights, times 2^(e_t) / vref
            const float2 vs =
                *reinterpret_cast<const float2*>(s_scale + KT + tok_of(st, r));
            w[j] = pack_h2_rtz(e0 * (vs.x * inv_vref), e1 * (vs.y * inv_vref));
          }
        }
        pb[st][hf] = __builtin_bit_cast(f16x8, uint4{w[0], w[1], w[2], w[3]});
      }

    // O^T += V^T P^T: A lane = d row 32 dt + lrow, tokens in pb's order
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint16_t* vrow =
              vt_lds + (32 * dt + lrow) * VSTRIDE + 32 * st + 16 * hf + 4 * lgrp;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          const f16x8 a = __builtin_bit_cast(f16x8, uint4{lo.x, lo.y, hi.x, hi.y});
          o[dt] = mfma32(a, pb[st][hf], o[dt]);
        }
  }

  l_row += __shfl_xor(l_row, 32);
  if (!row_valid) return;
  const float inv = l_row > 0.f ? (FP8 ? vref : 1.f) / l_row : 0.f;
  const int64_t row_head = (int64_t)(row_base + my_row) * num_q_heads + head;
  if (num_splits == 1) {
    uint16_t* dst = out + row_head * kD + 4 * lgrp;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        uint2 w;
        w.x = pack_h2_rne(o[dt][4 * qq] * inv, o[dt][4 * qq + 1] * inv);
        w.y = pack_h2_rne(o[dt][4 * qq + 2] * inv, o[dt][4 * qq + 3] * inv);
        *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * qq) = w;
      }
    return;
  }
  // Partial of this split: (o / l, m, l); l = 0 when no position was visible.
  const int64_t pidx = ((row_base + my_row - first_row) * num_q_heads + head) * num_splits + split;
  float* dst = part_o + pidx * kD + 4 * lgrp;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      *reinterpret_cast<float4*>(dst + 32 * dt + 8 * qq) =
          float4{o[dt][4 * qq] * inv, o[dt][4 * qq + 1] * inv, o[dt][4 * qq + 2] * inv,
                 o[dt][4 * qq + 3] * inv};
  if (lgrp == 0) {
    part_ml[pidx * 2] = m_row;
    part_ml[pidx * 2 + 1] = l_row;
  }
}


// ---------------------------------------------------------------------------
// fp16 cache: the tiles go from the pools straight into LDS
// (global_load_lds_dwordx4: lane l's 16 bytes land at the wave's LDS base +
// 16 l), so staging needs no registers and no VALU work, and the loads of a
// tile are in flight for a whole tile of math.  K and V have two buffers
// each; at tile kt a wave reads K(kt + 1) (the next scores) and V(kt) (this
// tile's O update) while K(kt + 2) and V(kt + 1) are loading.  Rows are
// 256 bytes, unpadded; their 16-byte chunks are swizzled so that the
// matrix-core operand reads hit distinct LDS banks:
//   K: chunk c of token t at slot c ^ (t & 15)     (16 rows per 128-bit read)
//   V: chunk c of token t at slot c ^ 4 (t & 3)    (4 rows x 4 chunks per
//                                                   transposing read)
// V^T fragments come from ds_read_b64_tr_b16: within each 16 lanes, lane a
// points at token t0 + a / 4, d0 + 4 (a % 4) .. +3, and lane i receives
// V[t0 + e][d0 + i] for e = 0 .. 3 -- four tokens of one d, the A-operand
// layout of the 32x32x16 product.
// Tokens past the tile's last row position are loaded from that position's
// row instead (finite data; their scores are masked, their weights 0).
typedef __fp16 h4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) h4_t* lds_h4_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int kRowBytes = kD * 2;           // 256
constexpr int kTileBytes = KT * kRowBytes;  // 16 KiB
constexpr int kIdPages = 256;               // pages whose pool offsets are staged in LDS
constexpr int kDmaWaves = 8;                // one work-group per CU, two waves per SIMD
constexpr int kDmaRows = 32 * kDmaWaves;    // query rows per work-group

constexpr int kStages = 4;                  // LDS ring depth of K and V
constexpr int kAhead = kStages - 1;         // tiles loaded ahead of the O update
// Per wave and tile: 2 loads of K + 2 of V (half a page each).
constexpr int kLoadsPerTile = 4;
static_assert(kLoadsPerTile * (kAhead - 1) == 8, "the wait below allows 8 loads in flight");
// s_waitcnt immediates (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8); only vmcnt is waited for.  The builtin, unlike an
// asm wait, is seen by the compiler's own wait insertion.
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm8 = 0x0F78;
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(kWaitVm0); }
// 16 bytes per lane from global memory into LDS at lds_base + 16 * lane
// (lds_base: the wave's LDS byte address, uniform).  Written as inline asm
// so that the compiler does not track these LDS writes: it would make every
// LDS read wait for all loads in flight (it cannot tell the ring's buffers
// apart), and so would __syncthreads(), whose fence also orders global
// memory.  The tiles a step reads are waited for explicitly before it
// (vmcnt counts these loads in issue order), and the barrier below orders
// the work-group's LDS accesses.
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_loads_but_newest() { __builtin_amdgcn_s_waitcnt(kWaitVm8); }

__global__ __launch_bounds__(64 * kDmaWaves) void prefill_wide_dma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, int64_t num_blocks, int32_t num_kv_heads,
    int32_t num_q_heads, const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
    int32_t first_seq, int32_t ctx_clamp, int32_t num_splits, int32_t row_tiles,
    int32_t num_units, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  // rings of kStages tiles: K(t) in k_lds<t % kStages>, V(t) in v_lds<t % kStages>
  // (t counted from the split's first tile)
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds3[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds2[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds3[kTileBytes];
  __shared__ int64_t s_page[kIdPages];

  // Work-group -> (sequence, row tile, split, KV head g, query head of g):
  // work-groups are dealt round-robin over the 8 XCDs, so unit u = (sequence,
  // row tile, split, g) goes to XCD u % 8 with all G query heads of g (they
  // read the same K/V tiles through that XCD's L2), and every XCD gets the
  // same number of units (one work-group per CU: no XCD runs a second round
  // while another idles).
  const int G = num_q_heads / num_kv_heads;
  const int unit = (int)(blockIdx.x & 7) + 8 * (int)((blockIdx.x >> 3) / G);
  if (unit >= num_units) return;  // padding of the last round of units
  const int g = unit % num_kv_heads;
  const int tile_row0 = (unit / num_kv_heads % row_tiles) * kDmaRows;
  const int split = unit / num_kv_heads / row_tiles % num_splits;
  const int i = first_seq + unit / num_kv_heads / row_tiles / num_splits;
  const int head = g * G + (int)((blockIdx.x >> 3) % G);
  const int row_base = query_start_loc[i];
  const int n = query_start_loc[i + 1] - row_base;
  const int ctx = min(context_lens[i], ctx_clamp);
  if (n <= 0 || tile_row0 >= n || ctx < n) return;  // uniform over the work-group
  const int p0 = ctx - n;
  const int pos_hi = p0 + min(tile_row0 + kDmaRows, n) - 1;
  const int num_kv_tiles = pos_hi / KT + 1;
  const int per_split = (num_kv_tiles + num_splits - 1) / num_splits;
  const int kt_begin = split * per_split;
  const int kt_end = min(kt_begin + per_split, num_kv_tiles);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int my_row_raw = tile_row0 + 32 * wave + lrow;
  const bool row_valid = my_row_raw < n;
  const bool wave_live = tile_row0 + 32 * wave < n;  // the same in all lanes of the wave
  const int my_row = row_valid ? my_row_raw : n - 1;
  const int my_pos = p0 + my_row;
  const int64_t first_row = query_start_loc[first_seq];
  if (kt_begin >= kt_end) {
    // an empty split: the merge reads only its weight l = 0
    if (row_valid && lgrp == 0) {
      const int64_t pidx =
          ((row_base + my_row - first_row) * num_q_heads + head) * num_splits + split;
      part_ml[pidx * 2] = -__builtin_huge_valf();
      part_ml[pidx * 2 + 1] = 0.f;
    }
    return;  // uniform over the work-group
  }

  // pool offset (elements) of page pg of this sequence, head g
  const int32_t* bt_row = block_tables + (int64_t)i * max_blocks_per_seq;
  const int64_t block_stride = (int64_t)num_kv_heads * 16 * kD;
  const int64_t head_off = (int64_t)g * 16 * kD;
  const int last_pg = pos_hi >> 4;
  auto block_off = [&](int pg) -> int64_t {
    const uint32_t id = (uint32_t)bt_row[pg];
    return (int64_t)(id < (uint64_t)num_blocks ? id : num_blocks - 1) * block_stride + head_off;
  };
  // Q^T fragments (B operands): row my_row, d = 16 c + 8 lgrp .. +7; loaded
  // beside the block-table reads, both waited for by the barrier below
  // (later waits count only the tile loads)
  f16x8 qb[kD / 16];
  {
    const uint16_t* qrow = q + ((int64_t)(row_base + my_row) * num_q_heads + head) * kD;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c)
      qb[c] = *reinterpret_cast<const f16x8*>(qrow + 16 * c + 8 * lgrp);
  }
  const int pg_begin = kt_begin * (KT / 16);
  const int pg_end = min(kt_end * (KT / 16) - 1, last_pg) + 1;
  for (int e = tid; e < kIdPages; e += 64 * kDmaWaves)
    if (pg_begin + e < pg_end) s_page[e] = block_off(pg_begin + e);
#pragma unroll
  for (int c = 0; c < kD / 16; ++c) asm volatile("" ::"v"(qb[c]));  // Q in before the barrier
  __syncthreads();

  // Wave w loads half of page w % 4 of a tile (tokens 16 (w % 4) + 8 (w / 4)
  // .. +7) as two 1 KiB rows-of-four, lane l -> token 16 (w % 4) + 8 (w / 4)
  // + 4 j + l / 16, LDS slot l % 16.
  const int dma_sub = lane >> 4, dma_slot = lane & 15;
  const int dma_page = wave & 3, dma_half = wave >> 2;
  auto dma_tile = [&](const uint16_t* __restrict__ pool, unsigned char* buf, int kt, bool is_v) {
    const int pg = min(kt * (KT / 16) + dma_page, last_pg);  // uniform
    const int rmax = pg == last_pg ? (pos_hi & 15) : 15;
    const int e = pg - pg_begin;
    const int64_t base = e < kIdPages ? s_page[e] : block_off(pg);
#pragma unroll
    for (int j = 2 * dma_half; j < 2 * dma_half + 2; ++j) {
      const int r = 4 * j + dma_sub;
      const int c = is_v ? (dma_slot ^ (4 * (r & 3))) : (dma_slot ^ r);
      const uint16_t* src = pool + base + min(r, rmax) * kD + 8 * c;
      load_lds16(src, (uint32_t)(uintptr_t)(lds_void_ptr)(buf + (16 * dma_page + 4 * j) * kRowBytes));
    }
  };

  f32x16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_row = -__builtin_huge_valf(), l_row = 0.f;

  // K fragment (c, st): token 32 st + lrow, chunk 2 c + lgrp at slot
  // (2 c + lgrp) ^ (lrow & 15) = address k_xor ^ (32 c) (+ 8 KiB for st = 1).
  const uint32_t k_xor = lrow * kRowBytes + 32 * ((lrow & 15) >> 1) + 16 * (lgrp ^ (lrow & 1));
  // V^T fragment (dt, st, hf): lane block b = lane / 16 covers d = 32 dt +
  // 16 (b & 1) + 0 .. 15 and tokens 32 st + 16 hf + 4 (b >> 1) + {0..3, 8..11}.
  const int va = lane & 15, vb = lane >> 4;
  const uint32_t v_base = (4 * (vb >> 1) + (va >> 2)) * kRowBytes + 64 * (va >> 2) +
                          16 * (2 * (vb & 1) + ((va & 3) >> 1)) + 8 * (va & 1);

  auto tok_of = [&](int st, int r) { return 32 * st + 8 * (r >> 2) + 4 * lgrp + (r & 3); };
  // First half of the online softmax of tile kt's scores (base 2, lazy max;
  // as in the 16-row kernel): scale and mask on tiles crossing the diagonal,
  // the row maximum, the rescale of l and O when it moves past m + slack.
  // Returns the factor of the exp's argument (scale_log2, or 1 when the
  // scores were scaled here).
  auto softmax_max = [&](f32x16 (&sc)[2], int kt) -> float {
    const int tok0 = kt * KT;
    const bool diagonal = tok0 + KT - 1 > p0 + tile_row0;
    float scl = scale_log2;
    if (diagonal) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = sc[st][r] * scale_log2;
          sc[st][r] = tok0 + tok_of(st, r) > my_pos ? -__builtin_huge_valf() : x;
        }
      scl = 1.f;
    }
    float ext = sc[0][0];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) ext = fmaxf(ext, sc[st][r]);
    float tile_max = ext * scl;
    tile_max = fmaxf(tile_max, __shfl_xor(tile_max, 32));
    if (__any(tile_max > m_row + kRescaleSlack)) {
      const float m_new = tile_max > m_row + kRescaleSlack ? tile_max : m_row;
      const float alpha = m_new == -__builtin_huge_valf() ? 1.f : fast_exp2(m_row - m_new);
      m_row = m_new;
      l_row *= alpha;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) o[dt] *= alpha;
    }
    return scl;
  };

  // Prologue: K(kt_begin), then, in the order the steps would have issued
  // them, K(kt_begin + 1 + a) and V(kt_begin + a) for a < kAhead, all issued
  // at once; K(kt_begin) waited for (the later loads stay in flight: the
  // first step's K(kt_begin + 1) arrives with it) and its scores computed.
  dma_tile(k_pool, k_lds0, kt_begin, false);
  if (kt_begin + 1 < kt_end) dma_tile(k_pool, k_lds1, kt_begin + 1, false);
  dma_tile(v_pool, v_lds0, kt_begin, true);
  if (kt_begin + 2 < kt_end) dma_tile(k_pool, k_lds2, kt_begin + 2, false);
  if (kt_begin + 1 < kt_end) dma_tile(v_pool, v_lds1, kt_begin + 1, true);
  if (kt_begin + 3 < kt_end) dma_tile(k_pool, k_lds3, kt_begin + 3, false);
  if (kt_begin + 2 < kt_end) dma_tile(v_pool, v_lds2, kt_begin + 2, true);
  {
    // this wave's loads issued after K(kt_begin): 2 per tile
    static_assert(kLoadsPerTile == 4, "2 loads per wave and tile of K, 2 of V");
    const int later = 2 * (1 + 2 * (kt_begin + 1 < kt_end) + 2 * (kt_begin + 2 < kt_end) +
                           (kt_begin + 3 < kt_end));
    if (later >= 12)
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | 12);
    else if (later >= 10)
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | 10);
    else if (later >= 6)
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | 6);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | 2);
  }
  lds_barrier();  // every wave's share of K(kt_begin) landed
  f32x16 s[2];
  if (wave_live) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[st][r] = 0.f;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
      const unsigned char* p = k_lds0 + (k_xor ^ (32u * c));
      s[0] = mfma32(*reinterpret_cast<const f16x8*>(p), qb[c], s[0]);
      s[1] = mfma32(*reinterpret_cast<const f16x8*>(p + 32 * kRowBytes), qb[c], s[1]);
    }
  }

  // One step: tile kt's scores in s, K(kt + 1) in kn, V(kt) in vc; K(kt + 4)
  // goes to kc (K(kt)'s buffer), V(kt + 3) to vn (V(kt - 1)'s).  The loads
  // of K(kt + 1) and V(kt) were issued three steps earlier; the two later
  // steps' loads may still be in flight.  After the row maximum,
  // one block of straight-line code, software-pipelined: eight stages each
  // issue the next K fragment pair, two products of the next tile's scores
  // and one eighth of this tile's exps (4 scores -> 2 packed weight pairs);
  // then the 16 products of the O update, their transposing reads issued
  // ahead.  The matrix cores work on the next scores while the VALU turns
  // this tile's scores into weights.
  auto step = [&](int kt, const unsigned char* kn, unsigned char* kc, const unsigned char* vc,
                  unsigned char* vn) {
    // this wave's share of K(kt + 1) and V(kt): all but the two later steps'
    // loads (fewer were issued near the end: then wait for all)
    if (kt + kAhead < kt_end)
      wait_loads_but_newest();
    else
      wait_all_loads();
    lds_barrier();  // every share landed; every wave is done with K(kt) and V(kt - 1)
    if (kt + 1 + kAhead < kt_end) dma_tile(k_pool, kc, kt + 1 + kAhead, false);
    if (kt + kAhead < kt_end) dma_tile(v_pool, vn, kt + kAhead, true);
    if (!wave_live) return;  // rows all past the chunk: load only
    const float scl = softmax_max(s, kt);
    const float neg_ref = m_row == -__builtin_huge_valf() ? 0.f : -m_row;

    f32x16 sn[2];  // the next tile's scores (past the last tile: a stale buffer's, unused)
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) sn[st][r] = 0.f;
    uint32_t w[2][8];  // packed weights: w[st][4 hf + j] = registers 8 hf + 2 j, +1
    f16x8 ka[2][2];
    ka[0][0] = *reinterpret_cast<const f16x8*>(kn + k_xor);
    ka[0][1] = *reinterpret_cast<const f16x8*>(kn + k_xor + 32 * kRowBytes);
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
      if (c + 1 < kD / 16) {
        const unsigned char* p = kn + (k_xor ^ (32u * (c + 1)));
        ka[(c + 1) & 1][0] = *reinterpret_cast<const f16x8*>(p);
        ka[(c + 1) & 1][1] = *reinterpret_cast<const f16x8*>(p + 32 * kRowBytes);
      }
      sn[0] = mfma32(ka[c & 1][0], qb[c], sn[0]);
      sn[1] = mfma32(ka[c & 1][1], qb[c], sn[1]);
      // exps of registers 4 q .. 4 q + 3 of s[st], st = c / 4, q = c % 4
      const int st = c >> 2, q = c & 3;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 4 * q + 2 * h;
        const float e0 = fast_exp2(__builtin_fmaf(s[st][r], scl, neg_ref));
        const float e1 = fast_exp2(__builtin_fmaf(s[st][r + 1], scl, neg_ref));
        w[st][2 * q + h] = pack_h2_rtz(e0, e1);
        l_row = dot2(w[st][2 * q + h], kOnesH2, l_row);
      }
    }
    // O^T += V^T P^T; product (st, hf) x dt, reads issued two products ahead
    constexpr int kPv = 16;
    auto pv_read = [&](int k) -> f16x8 {
      const int st = k >> 3, hf = (k >> 2) & 1, dt = k & 3;
      const unsigned char* p = vc + (v_base ^ (64u * dt)) + (32 * st + 16 * hf) * kRowBytes;
      const h4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4_ptr)p);
      const h4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_h4_ptr)(p + 8 * kRowBytes));
      return __builtin_bit_cast(
          f16x8, uint4{__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                       __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y});
    };
    f16x8 va_[3];
    va_[0] = pv_read(0);
    va_[1] = pv_read(1);
#pragma unroll
    for (int k = 0; k < kPv; ++k) {
      if (k + 2 < kPv) va_[(k + 2) % 3] = pv_read(k + 2);
      const int st = k >> 3, hf = (k >> 2) & 1, dt = k & 3;
      const f16x8 pb = __builtin_bit_cast(
          f16x8, uint4{w[st][4 * hf], w[st][4 * hf + 1], w[st][4 * hf + 2], w[st][4 * hf + 3]});
      o[dt] = mfma32(va_[k % 3], pb, o[dt]);
    }
    // instruction order of the block: 2 K reads; 8 x (2 K reads, 2 products,
    // 12 VALU); 4 V reads; 16 x (2 V reads, 1 product)
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int c = 0; c + 1 < kD / 16; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k + 2 < kPv; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
#pragma unroll
    for (int st = 0; st < 2; ++st) s[st] = sn[st];
  };
  for (int kt = kt_begin; kt < kt_end; kt += kStages) {
    step(kt, k_lds1, k_lds0, v_lds0, v_lds3);
    if (kt + 1 < kt_end) step(kt + 1, k_lds2, k_lds1, v_lds1, v_lds0);
    if (kt + 2 < kt_end) step(kt + 2, k_lds3, k_lds2, v_lds2, v_lds1);
    if (kt + 3 < kt_end) step(kt + 3, k_lds0, k_lds3, v_lds3, v_lds2);
  }

  l_row += __shfl_xor(l_row, 32);
  if (!row_valid) return;
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  const int64_t row_head = (int64_t)(row_base + my_row) * num_q_heads + head;
  if (num_splits == 1) {
    uint16_t* dst = out + row_head * kD + 4 * lgrp;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        uint2 w;
        w.x = pack_h2_rne(o[dt][4 * qq] * inv, o[dt][4 * qq + 1] * inv);
        w.y = pack_h2_rne(o[dt][4 * qq + 2] * inv, o[dt][4 * qq + 3] * inv);
        *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * qq) = w;
      }
    return;
  }
  const int64_t pidx = ((row_base + my_row - first_row) * num_q_heads + head) * num_splits + split;
  float* dst = part_o + pidx * kD + 4 * lgrp;
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      *reinterpret_cast<float4*>(dst + 32 * dt + 8 * qq) =
          float4{o[dt][4 * qq] * inv, o[dt][4 * qq + 1] * inv, o[dt][4 * qq + 2] * inv,
                 o[dt][4 * qq + 3] * inv};
  if (lgrp == 0) {
    part_ml[pidx * 2] = m_row;
    part_ml[pidx * 2 + 1] = l_row;
  }
}

}  // namespace

hipError_t launch_prefill_wide(const void* q, const void* k_pool, const void* v_pool,
                               const float* k_scale, const float* v_scale, int64_t num_blocks,
                               int32_t num_kv_heads, int32_t num_q_heads,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               int32_t first_seq, int32_t num_prefill_seqs,
                               int32_t max_query_len, float scale, int32_t splits, void* out,
                               float* part_o, float* part_ml, hipStream_t stream) {
  const int32_t ctx_clamp =
      (int32_t)std::min<int64_t>((int64_t)max_blocks_per_seq * 16, INT32_MAX);
  // x = (query tile, split), padded to a multiple of the 8 XCDs: work-groups
  // are dealt round-robin over the XCDs, so every head of one (tile, split)
  // -- the G heads sharing one KV head in particular -- runs on one XCD and
  // reads the K/V tiles through the same L2.
  constexpr uint32_t kXcds = 8;
  const uint32_t x = ((max_query_len + kWideRows - 1) / kWideRows) * splits;
  const dim3 grid((x + kXcds - 1) / kXcds * kXcds, num_q_heads, num_prefill_seqs);
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  if (k_scale != nullptr)
    hipLaunchKernelGGL((prefill_wide_kernel<true>), grid, dim3(256), 0, stream,
                       static_cast<const uint16_t*>(q), k_pool, v_pool, k_scale, v_scale,
                       num_blocks, num_kv_heads, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, query_start_loc, first_seq, ctx_clamp, splits,
                       scale * kLog2e, static_cast<uint16_t*>(out), part_o, part_ml);
  else {
    const int32_t row_tiles = (max_query_len + kDmaRows - 1) / kDmaRows;
    const int64_t units = (int64_t)num_prefill_seqs * row_tiles * splits * num_kv_heads;
    const int64_t G = num_q_heads / num_kv_heads;
    const int64_t wgs = (units + kXcds - 1) / kXcds * kXcds * G;
    if (units > INT32_MAX || wgs > UINT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(prefill_wide_dma_kernel, dim3((uint32_t)wgs), dim3(64 * kDmaWaves), 0,
                       stream, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k_pool), static_cast<const uint16_t*>(v_pool),
                       num_blocks, num_kv_heads, num_q_heads, block_tables, max_blocks_per_seq,
                       context_lens, query_start_loc, first_seq, ctx_clamp, splits, row_tiles,
                       (int32_t)units, scale * kLog2e, static_cast<uint16_t*>(out), part_o,
                       part_ml);
  }
  return hipGetLastError();
}

}  // namespace pkv
