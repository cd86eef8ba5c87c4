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
// 32 flop per LDS byte, which at the LDS's ~128 bytes per clock per CU is
// the matrix cores' own rate -- LDS reads, not the products, bound the
// contraction on CDNA4 once the exps and the tile loads share the time.
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
// prefill_wide_dma_kernel (fp16 cache): work-group = 8 waves = 256 rows of
// one query head, one per CU; the tiles go from the pools straight into
// 4-deep LDS rings three tiles ahead (described with the kernel).
// prefill_wide_dma8_kernel (fp8 cache): the same work-groups; the codes and
// row scales go into LDS rings and the work-group turns each tile into
// fp16 tiles for the same reads and products (described with the kernel).
#include <algorithm>
#include <climits>

#include "device_util.h"
#include "kernels.h"

namespace pkv {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 128;
constexpr int KT = 64;              // context tokens per tile
constexpr float kRescaleSlack = 8.f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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
    tile_max = max_of_halves(tile_max);
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
  f32x16 s0[2], s1[2];  // scores of the current and next tile, alternating
  if (wave_live) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[st][r] = 0.f;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
      const unsigned char* p = k_lds0 + (k_xor ^ (32u * c));
      s0[0] = mfma32(*reinterpret_cast<const f16x8*>(p), qb[c], s0[0]);
      s0[1] = mfma32(*reinterpret_cast<const f16x8*>(p + 32 * kRowBytes), qb[c], s0[1]);
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
  auto step = [&](int kt, f32x16 (&s)[2], f32x16 (&sn)[2], const unsigned char* kn,
                  unsigned char* kc, const unsigned char* vc, unsigned char* vn) {
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

    // sn: the next tile's scores (past the last tile: a stale buffer's, unused)
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
  };
  for (int kt = kt_begin; kt < kt_end; kt += kStages) {
    step(kt, s0, s1, k_lds1, k_lds0, v_lds0, v_lds3);
    if (kt + 1 < kt_end) step(kt + 1, s1, s0, k_lds2, k_lds1, v_lds1, v_lds0);
    if (kt + 2 < kt_end) step(kt + 2, s0, s1, k_lds3, k_lds2, v_lds2, v_lds1);
    if (kt + 3 < kt_end) step(kt + 3, s1, s0, k_lds0, k_lds3, v_lds3, v_lds2);
  }

  l_row = sum_of_halves(l_row);
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


// ---------------------------------------------------------------------------
// fp8 cache on the work-groups of the kernel above.  The DMA brings each
// tile's codes (8 KiB of K, 8 KiB of V: token-major 128-byte rows, in order)
// and its row scales into LDS rings; in each step the whole work-group turns
// the K tile of the next step's scores and the V tile of the next step's O
// update into fp16 tiles laid out and swizzled as above, each value being
// code x 2^(e - 1) for its row's scale 2^e -- half the dequantized value --
// so the steps run the fp16 kernel's fragment reads and products, with the
// factor 2 in the scores' scale and in the output's normalisation.  With
// the row exponents the quantizing append writes (e <= 8, from fp16 rows)
// no value overflows fp16 (448 x 2^7 = 57344); the values are exact for e
// >= -14 and otherwise off by at most 2^-24 (fp16's subnormal spacing, in
// the dequantized units).  (A reference taken per tile instead, the largest
// row scale, costs three wave reductions per step.)
// Load schedule: step kt issues the K codes and K scales of tile kt + 4 and
// the V codes and V scales of tile kt + 3 (four loads per wave); it converts
// K(kt + 2) and V(kt + 1); so at its start everything but the previous
// step's loads has to be in.
constexpr int kCodeTileBytes = KT * kD;  // 8 KiB of codes per tile
constexpr int kDma8LoadsPerStep = 4;     // per wave: K codes, K scales, V codes, V scales

// 4 bytes per active lane from global memory into LDS at lds_base + 4 * lane
__device__ __forceinline__ void load_lds4(const void* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(lds_base)
               : "memory", "m0");
}
// all of this wave's loads but the newest n (n = 0, 2 or 4, wave-uniform)
__device__ __forceinline__ void wait_loads_but4(int n) {
  if (n >= 4)
    __builtin_amdgcn_s_waitcnt(kWaitVm0 | 4);
  else if (n >= 2)
    __builtin_amdgcn_s_waitcnt(kWaitVm0 | 2);
  else
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
}

__global__ __launch_bounds__(64 * kDmaWaves) void prefill_wide_dma8_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ k_codes,
    const uint8_t* __restrict__ v_codes, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int64_t num_blocks, int32_t num_kv_heads,
    int32_t num_q_heads, const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
    int32_t first_seq, int32_t ctx_clamp, int32_t num_splits, int32_t row_tiles,
    int32_t num_units, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  // code rings (slot (t - kt_begin) % 4), fp16 tiles (slot (t - kt_begin) % 2),
  // row-scale rings (slot (t - kt_begin) % 4)
  __shared__ __attribute__((aligned(1024))) unsigned char kc_lds0[kCodeTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kc_lds1[kCodeTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kc_lds2[kCodeTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char kc_lds3[kCodeTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vc_lds0[kCodeTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vc_lds1[kCodeTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vc_lds2[kCodeTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char vc_lds3[kCodeTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k16_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char k16_lds1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v16_lds0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v16_lds1[kTileBytes];
  __shared__ __attribute__((aligned(16))) float ks_lds[4][KT];
  __shared__ __attribute__((aligned(16))) float vs_lds[4][KT];
  __shared__ int64_t s_page[kIdPages];

  // work-group -> (sequence, row tile, split, KV head g, query head of g), as
  // in the fp16 kernel above
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

  // byte offset of page pg's codes (this sequence, head g); its row scales
  // start at that offset / d
  const int32_t* bt_row = block_tables + (int64_t)i * max_blocks_per_seq;
  const int64_t block_stride = (int64_t)num_kv_heads * 16 * kD;
  const int64_t head_off = (int64_t)g * 16 * kD;
  const int last_pg = pos_hi >> 4;
  auto block_off = [&](int pg) -> int64_t {
    const uint32_t id = (uint32_t)bt_row[pg];
    return (int64_t)(id < (uint64_t)num_blocks ? id : num_blocks - 1) * block_stride + head_off;
  };
  // Q^T fragments (B operands): row my_row, d = 16 c + 8 lgrp .. +7
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

  // Wave w loads tokens 8 w .. 8 w + 7 of a tile (rows 8 (w & 1) .. +7 of page
  // w / 2): codes lane l -> token 8 w + l / 8, 16-byte chunk l % 8 (LDS byte
  // 16 (64 w + l)); row scales lanes 0 .. 7.  Tokens past the tile's last
  // row position load that position's row.
  auto dma_codes = [&](const uint8_t* __restrict__ codes, unsigned char* buf, int kt) {
    const int pg = min(kt * (KT / 16) + (wave >> 1), last_pg);  // uniform
    const int rmax = pg == last_pg ? (pos_hi & 15) : 15;
    const int e = pg - pg_begin;
    const int64_t base = e < kIdPages ? s_page[e] : block_off(pg);
    const int r = 8 * (wave & 1) + (lane >> 3);
    load_lds16(codes + base + min(r, rmax) * kD + 16 * (lane & 7),
               (uint32_t)(uintptr_t)(lds_void_ptr)(buf + 1024 * wave));
  };
  auto dma_scales = [&](const float* __restrict__ scales, float* buf, int kt) {
    const int pg = min(kt * (KT / 16) + (wave >> 1), last_pg);
    const int rmax = pg == last_pg ? (pos_hi & 15) : 15;
    const int e = pg - pg_begin;
    const int64_t base = e < kIdPages ? s_page[e] : block_off(pg);
    if (lane < 8)
      load_lds4(scales + base / kD + min(8 * (wave & 1) + lane, rmax),
                (uint32_t)(uintptr_t)(lds_void_ptr)(buf + 8 * wave));
  };
  // Codes of a tile (slot in, row scales sc) to fp16 (slot out): value =
  // code x scale / 2.  Thread t takes token t / 8 and, with j = t % 8, the
  // fp16 chunks j and j + 8 of its row (codes 8 j .. +7 and 64 + 8 j .. +7),
  // odd tokens the upper chunk first: so that each read and write
  // instruction spreads its lanes over all LDS banks (addresses differ per
  // lane, the data path does not).  K and V swizzled as in the fp16 kernel.
  auto convert_tile = [&](const unsigned char* in, const float* sc, unsigned char* out_tile,
                          bool is_v) {
    const int tt = tid >> 3, j = tid & 7;
    const float f = 0.5f * sc[tt];  // a power of two: exact
    const int x = is_v ? 4 * (tt & 3) : (tt & 15);
    const int ca = j + 8 * (tt & 1), cb = j + 8 * (~tt & 1);  // fp16 chunks, in order
    const uint2 qa = *reinterpret_cast<const uint2*>(in + tt * kD + 8 * ca);
    const uint2 qb2 = *reinterpret_cast<const uint2*>(in + tt * kD + 8 * cb);
    auto h4 = [&](const uint2& c) {
      return uint4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.x, f, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, f, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c.y, f, true))};
    };
    *reinterpret_cast<uint4*>(out_tile + tt * kRowBytes + 16 * (ca ^ x)) = h4(qa);
    *reinterpret_cast<uint4*>(out_tile + tt * kRowBytes + 16 * (cb ^ x)) = h4(qb2);
  };

  f32x16 o[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_row = -__builtin_huge_valf(), l_row = 0.f;
  const float scale_k = 2.f * scale_log2;  // the scores are in units of 2 (K tiles hold K / 2)

  const uint32_t k_xor = lrow * kRowBytes + 32 * ((lrow & 15) >> 1) + 16 * (lgrp ^ (lrow & 1));
  const int va = lane & 15, vb = lane >> 4;
  const uint32_t v_base = (4 * (vb >> 1) + (va >> 2)) * kRowBytes + 64 * (va >> 2) +
                          16 * (2 * (vb & 1) + ((va & 3) >> 1)) + 8 * (va & 1);

  auto tok_of = [&](int st, int r) { return 32 * st + 8 * (r >> 2) + 4 * lgrp + (r & 3); };
  // The first half of the online softmax of tile kt's scores, as in the
  // fp16 kernel with the scale doubled.
  auto softmax_max = [&](f32x16 (&sc)[2], int kt) -> float {
    const int tok0 = kt * KT;
    const bool diagonal = tok0 + KT - 1 > p0 + tile_row0;
    float scl = scale_k;
    if (diagonal) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = sc[st][r] * scale_k;
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
    tile_max = max_of_halves(tile_max);
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

  // loads this wave issued at step j (j >= kt_begin - 4)
  auto loads_of_step = [&](int j) {
    const bool k4 = j + 4 < kt_end, t3 = j + 3 >= kt_begin && j + 3 < kt_end;
    return 2 * (int)k4 + 2 * (int)t3;
  };
  // Prologue: the loads of steps kt_begin - 4 .. kt_begin - 1, in their
  // order; then K(kt_begin), K(kt_begin + 1) and V(kt_begin) converted and
  // the scores of tile kt_begin computed.
  {
    unsigned char* kc[4] = {kc_lds0, kc_lds1, kc_lds2, kc_lds3};
    unsigned char* vc[4] = {vc_lds0, vc_lds1, vc_lds2, vc_lds3};
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if (kt_begin + a < kt_end) {
        dma_codes(k_codes, kc[a], kt_begin + a);
        dma_scales(k_scale, ks_lds[a], kt_begin + a);
      }
      if (a >= 1 && kt_begin + a - 1 < kt_end) {
        dma_codes(v_codes, vc[a - 1], kt_begin + a - 1);
        dma_scales(v_scale, vs_lds[a - 1], kt_begin + a - 1);
      }
    }
  }
  {
    // all but the loads of steps kt_begin - 2 and kt_begin - 1 (8, 6, 2 or 0)
    const int later = loads_of_step(kt_begin - 2) + loads_of_step(kt_begin - 1);
    if (later >= 8)
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | 8);
    else if (later >= 6)
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | 6);
    else if (later >= 2)
      __builtin_amdgcn_s_waitcnt(kWaitVm0 | 2);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
  }
  lds_barrier();
  convert_tile(kc_lds0, ks_lds[0], k16_lds0, false);
  convert_tile(vc_lds0, vs_lds[0], v16_lds0, true);
  if (kt_begin + 1 < kt_end) convert_tile(kc_lds1, ks_lds[1], k16_lds1, false);
  lds_barrier();
  f32x16 s0[2], s1[2];  // scores of the current and next tile, alternating
  if (wave_live) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) s0[st][r] = 0.f;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
      const unsigned char* p = k16_lds0 + (k_xor ^ (32u * c));
      s0[0] = mfma32(*reinterpret_cast<const f16x8*>(p), qb[c], s0[0]);
      s0[1] = mfma32(*reinterpret_cast<const f16x8*>(p + 32 * kRowBytes), qb[c], s0[1]);
    }
  }

  // One step at tile kt (slots for r = kt - kt_begin): its scores in s, K(kt
  // + 1) in fp16 at kn, V(kt) in fp16 at vcur; issues K codes and scales
  // (kt + 4) to kdst / ksdst, V codes and scales (kt + 3) to vdst / vsdst;
  // converts K(kt + 2) (kcin, scales kcs -> kconv) and V(kt + 1) (vcin,
  // scales vcs -> vconv).
  auto step = [&](int kt, f32x16 (&s)[2], f32x16 (&sn)[2], const unsigned char* kn,
                  const unsigned char* vcur,
                  unsigned char* kdst, float* ksdst, unsigned char* vdst, float* vsdst,
                  const unsigned char* kcin, const float* kcs, unsigned char* kconv,
                  const unsigned char* vcin, const float* vcs, unsigned char* vconv) {
    wait_loads_but4(loads_of_step(kt - 1));
    lds_barrier();  // every share landed; every wave is done with the slots reused below
    if (kt + 4 < kt_end) {
      dma_codes(k_codes, kdst, kt + 4);
      dma_scales(k_scale, ksdst, kt + 4);
    }
    if (kt + 3 < kt_end) {
      dma_codes(v_codes, vdst, kt + 3);
      dma_scales(v_scale, vsdst, kt + 3);
    }
    // the conversions of K(kt + 2) and V(kt + 1) (their codes are in: waited
    // for above; their fp16 slots were last read in the previous step) come
    // at the end of the step, under the O update's products
    auto convert_next = [&]() {
      if (kt + 2 < kt_end) convert_tile(kcin, kcs, kconv, false);
      if (kt + 1 < kt_end) convert_tile(vcin, vcs, vconv, true);
    };
    if (!wave_live) {  // rows all past the chunk: load and convert only
      convert_next();
      return;
    }
    const float scl = softmax_max(s, kt);
    const float neg_ref = m_row == -__builtin_huge_valf() ? 0.f : -m_row;

    // sn: the next tile's scores (past the last tile: a stale buffer's, unused)
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
      const int st = c >> 2, qq = c & 3;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 4 * qq + 2 * h;
        const float e0 = fast_exp2(__builtin_fmaf(s[st][r], scl, neg_ref));
        const float e1 = fast_exp2(__builtin_fmaf(s[st][r + 1], scl, neg_ref));
        w[st][2 * qq + h] = pack_h2_rtz(e0, e1);
        l_row = dot2(w[st][2 * qq + h], kOnesH2, l_row);
      }
    }
    constexpr int kPv = 16;
    auto pv_read = [&](int k) -> f16x8 {
      const int st = k >> 3, hf = (k >> 2) & 1, dt = k & 3;
      const unsigned char* p = vcur + (v_base ^ (64u * dt)) + (32 * st + 16 * hf) * kRowBytes;
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
    // instruction order: 2 K reads; 8 x (2 K reads, 2 products, 12 VALU);
    // 4 V reads; 16 x (2 V reads, 1 product)
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
    convert_next();
  };
  // slots for r = kt - kt_begin: codes (K kt + 4 -> r % 4; V kt + 3 ->
  // (r + 3) % 4), scales (tile t -> (t - kt_begin) % 4), fp16 (K kt + 1 ->
  // (r + 1) % 2; V kt -> r % 2; K kt + 2 -> r % 2; V kt + 1 -> (r + 1) % 2)
  for (int kt = kt_begin; kt < kt_end; kt += 4) {
    step(kt, s0, s1, k16_lds1, v16_lds0, kc_lds0, ks_lds[0], vc_lds3, vs_lds[3], kc_lds2, ks_lds[2],
         k16_lds0, vc_lds1, vs_lds[1], v16_lds1);
    if (kt + 1 < kt_end)
      step(kt + 1, s1, s0, k16_lds0, v16_lds1, kc_lds1, ks_lds[1], vc_lds0, vs_lds[0], kc_lds3,
           ks_lds[3], k16_lds1, vc_lds2, vs_lds[2], v16_lds0);
    if (kt + 2 < kt_end)
      step(kt + 2, s0, s1, k16_lds1, v16_lds0, kc_lds2, ks_lds[2], vc_lds1, vs_lds[1], kc_lds0,
           ks_lds[0], k16_lds0, vc_lds3, vs_lds[3], v16_lds1);
    if (kt + 3 < kt_end)
      step(kt + 3, s1, s0, k16_lds0, v16_lds1, kc_lds3, ks_lds[3], vc_lds2, vs_lds[2], kc_lds1,
           ks_lds[1], k16_lds1, vc_lds0, vs_lds[0], v16_lds0);
  }

  l_row = sum_of_halves(l_row);
  if (!row_valid) return;
  const float inv = l_row > 0.f ? 2.f / l_row : 0.f;  // O was in units of 2 (V tiles hold V / 2)
  const int64_t row_head = (int64_t)(row_base + my_row) * num_q_heads + head;
  if (num_splits == 1) {
    uint16_t* dst = out + row_head * kD + 4 * lgrp;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        uint2 wv;
        wv.x = pack_h2_rne(o[dt][4 * qq] * inv, o[dt][4 * qq + 1] * inv);
        wv.y = pack_h2_rne(o[dt][4 * qq + 2] * inv, o[dt][4 * qq + 3] * inv);
        *reinterpret_cast<uint2*>(dst + 32 * dt + 8 * qq) = wv;
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
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  {
    const int32_t row_tiles = (max_query_len + kDmaRows - 1) / kDmaRows;
    const int64_t units = (int64_t)num_prefill_seqs * row_tiles * splits * num_kv_heads;
    const int64_t G = num_q_heads / num_kv_heads;
    const int64_t wgs = (units + kXcds - 1) / kXcds * kXcds * G;
    if (units > INT32_MAX || wgs > UINT32_MAX) return hipErrorInvalidValue;
    if (k_scale != nullptr)
      hipLaunchKernelGGL(prefill_wide_dma8_kernel, dim3((uint32_t)wgs), dim3(64 * kDmaWaves), 0,
                         stream, static_cast<const uint16_t*>(q),
                         static_cast<const uint8_t*>(k_pool), static_cast<const uint8_t*>(v_pool),
                         k_scale, v_scale, num_blocks, num_kv_heads, num_q_heads, block_tables,
                         max_blocks_per_seq, context_lens, query_start_loc, first_seq, ctx_clamp,
                         splits, row_tiles, (int32_t)units, scale * kLog2e,
                         static_cast<uint16_t*>(out), part_o, part_ml);
    else
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
