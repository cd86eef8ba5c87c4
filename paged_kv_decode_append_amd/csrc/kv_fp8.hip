// kv_fp8.hip -- the quantized (fp8, OCP E4M3) KV cache: the append that
// quantizes each new K/V row, and paged decode attention reading the codes.
//
// Why: decode reads the whole cache every step and is bound by HBM, and the
// raw KV of a window halves at 8 bits ("8 GiB at 8-bit ... before scales"
// for a 262,144-token window -- a8q9.cn, "An advertised batch limit proves
// nothing until sampled"; quantizing the cache is one of the remedies when
// memory caps the batch -- deepconcepts.dev, "Continuous Batching Is Not a
// Bigger Batch", "Checking it on a real system").
//
// Format (the pages fix none; the reading taken): codes are OCP E4M3 bytes in
// the same [block][KV head][16][d] layout as the fp16 pools; every (token, KV
// head) row carries one fp32 scale 2^e, the smallest power of two with
// max|x| <= 448 x 2^e, so scaling is exact and the codes are x / 2^e rounded
// to nearest (ties to even) by v_cvt_pk_fp8_f32.  The row value is code x 2^e.
//
// Decode works like the fp16 kernel (decode.hip): grid (sequence, KV head,
// partition), 4 waves dealt the partition's blocks round-robin, the G query
// heads of the group applied to each K/V byte once, base-2 online softmax
// with a lazy maximum, masking by select, and the same partials and merge.
// Per block and wave:
//   K: the scores are S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_f16,
//     the G query heads as columns): lane l loads 16 codes of token row
//     l % 16 and turns them into the A fragments of two 32-wide chunks with
//     v_cvt_scalef32_pk_f16_fp8 (exact: every E4M3 value is an fp16 value);
//     the query fragments are read from LDS in the same column order.  Each
//     lane ends with the scores of head l % 16 for 4 tokens, times the rows'
//     K scales.
//   V: P.V is O = P V on the matrix cores too (v_mfma_f32_16x16x16_f16,
//     heads as rows, one 16-column tile of d per product): the scores'
//     output layout (head l % 16, tokens 4 (l / 16) .. +3 in lane l) is
//     already P's A fragment, so the weights never leave registers.  Lane l
//     loads those four tokens' codes at columns (d / 16)(l % 16) .. +d/16-1
//     (one 8- or 16-byte load per token); a 4 x 4 byte transpose with
//     v_perm_b32 gives each column tile's B fragment, converted to fp16
//     (exact).  The row scales 2^e_t enter the weights: each weight is
//     scaled by 2^(e_t - e_max) (e_max the block's largest, so weights stay
//     within fp16), and the O tiles are kept in units of 2^e_max, rescaled
//     when it changes from one block to the next; the softmax denominator
//     sums the unscaled weights.
// On MI355X this kernel is bound by its per-block arithmetic more than by
// bytes in flight: with P.V as packed fp16 dot products over weights passed
// through LDS it ran 40% slower at B = 256, ctx 512 than with P.V removed
// altogether.
#include <algorithm>
#include <climits>

#include "device_util.h"
#include "fp8_util.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kBlockSize = 16;
constexpr int kWaves = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.f;  // lazy max (base 2)
// Unused dynamic LDS of a d = 128 decode work-group: by itself more than a
// third of the CU's 160 KiB (whatever the group size G makes the static
// part), so at most two work-groups are resident per CU (two waves per
// SIMD) whatever the register count.  Measured: at three per CU the ragged
// grid's work-groups pack onto fewer CUs and the ragged batch slows by ~15%.
constexpr size_t kResidencyPadBytes = 54 << 10;

// Smallest e with amax <= 448 x 2^e (0 for amax = 0).  amax is a finite fp16
// value, a normal fp32 number: amax = 1.f x 2^k; 448 = 1.75 x 2^8, so
// e = k - 8, plus 1 when the fraction f exceeds 0.75.
__device__ __forceinline__ int row_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  const uint32_t b = __float_as_uint(amax);
  const int k = (int)((b >> 23) & 0xFF) - 127;
  return k - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
}

// 2^e as fp32 for |e| <= 126.
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// ---------------------------------------------------------------- append ---

// One fp16 row of D values quantized by one wave (lane l holds values
// EPL*l .. EPL*l + EPL-1, EPL = D/64): returns the lane's EPL codes (byte k
// of the word = value k) and sets e (the row's scale is 2^e).
template <int D>
__device__ __forceinline__ uint32_t quantize_row_wave(const uint16_t* __restrict__ row, int lane,
                                                      int& e) {
  constexpr int EPL = D / 64;
  const uint16_t* src = row + EPL * lane;
  float x[EPL];
  if constexpr (EPL == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
    x[0] = (float)__builtin_bit_cast(f16, (uint16_t)(w & 0xffffu));
    x[1] = (float)__builtin_bit_cast(f16, (uint16_t)(w >> 16));
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(src);
    x[0] = (float)__builtin_bit_cast(f16, (uint16_t)(w.x & 0xffffu));
    x[1] = (float)__builtin_bit_cast(f16, (uint16_t)(w.x >> 16));
    x[2] = (float)__builtin_bit_cast(f16, (uint16_t)(w.y & 0xffffu));
    x[3] = (float)__builtin_bit_cast(f16, (uint16_t)(w.y >> 16));
  }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < EPL; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  e = row_exponent(amax);
  const float inv = exp2i(-e);  // exact scaling: |x * inv| <= 448
  int c = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[1] * inv, 0, false);
  if constexpr (EPL == 4) c = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * inv, x[3] * inv, c, true);
  return (uint32_t)c;
}

// Stores a lane's EPL codes (EPL = 2: two bytes; 4: four).
template <int D>
__device__ __forceinline__ void store_codes(uint8_t* dst, uint32_t c) {
  if constexpr (D == 128)
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(c & 0xffffu);
  else
    *reinterpret_cast<uint32_t*>(dst) = c;
}

// Quantizes row r of K (is_v false) or V of the new tokens ([tokens][Hkv][D]
// fp16, row r = token r / Hkv, KV head r % Hkv) into its slot: one wave,
// lane l quantizing values EPL*l .. EPL*l + EPL-1.
template <int D>
__device__ __forceinline__ void append_row_fp8(
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes, float* __restrict__ k_scale,
    float* __restrict__ v_scale, int64_t num_blocks, int32_t num_kv_heads,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, int64_t r, bool is_v, int lane) {
  constexpr int EPL = D / 64;
  const int64_t t = r / num_kv_heads;
  const int g = (int)(r - t * num_kv_heads);
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;  // padding: nothing to write
  const int64_t b = slot / kBlockSize;
  if (b >= num_blocks) return;  // beyond the pool (a broken contract): skipped
  const int o = (int)(slot % kBlockSize);
  int e;
  const uint32_t c = quantize_row_wave<D>((is_v ? v_new : k_new) + r * D, lane, e);
  const int64_t row = ((b * num_kv_heads + g) * kBlockSize + o);
  store_codes<D>((is_v ? v_codes : k_codes) + row * D + EPL * lane, c);
  if (lane == 0) (is_v ? v_scale : k_scale)[row] = exp2i(e);
}

// One wave per (token, KV head) row of K (grid.y = 0) or V (grid.y = 1),
// four rows per work-group.
template <int D>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes, float* __restrict__ k_scale,
    float* __restrict__ v_scale, int64_t num_blocks, int32_t num_kv_heads,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  append_row_fp8<D>(k_codes, v_codes, k_scale, v_scale, num_blocks, num_kv_heads, k_new, v_new,
                    slot_mapping, r, blockIdx.y == 1, threadIdx.x & 63);
}

// ---------------------------------------------------------------- decode ---

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// V in the matrix cores' B layout (P.V as O = P V, 16 x 16 x 16 tiles): lane
// l holds the codes of tokens 4 (l / 16) .. +3 of a block at columns
// VB (l % 16) .. +VB-1 (VB = d / 16: one 8- or 16-byte load per token).
// Column tile ct of the product takes byte ct of each of those four chunks,
// so output column n of tile ct is d = VB n + ct.
template <int D>
struct V8Layout {
  static constexpr int VB = D / 16;  // codes per token per lane = column tiles
  static constexpr int VW = VB / 4;  // their 32-bit words
};

// K in the matrix cores' A layout: lane l holds 16 codes of token row l % 16
// at columns 64 c2 + 16 (l / 16) .. +15, the fragments of chunks 2 c2 and
// 2 c2 + 1 (the query fragments are read with the same column order).
template <int D>
struct KV8Regs {
  static constexpr int K16 = D / 64;  // 16-code loads per lane
  uint4 k[K16];
  float4 ks;                          // K scales of tokens 4 (l / 16) .. +3
  float4 vs;                          // their V scales
  uint32_t v[4][V8Layout<D>::VW];     // V codes of those 4 tokens (B layout)
};

template <int D, int G>
struct Wave8 {
  float m;                   // running max of this lane's head (lane % 16), base 2
  float l;                   // sum of its weights over this lane's tokens
  float vref;                // acc is in units of this V row scale (wave-uniform; 0 at the start)
  f32x4 acc[D / 16];         // O tiles: heads 4 (l / 16) + i, column (ct, l % 16)
};

// The same block through raw buffer resources (codes of K and V, 16 row
// scales each); resources of 0 bytes read nothing and give zeros, so the
// loop issues its prefetch unconditionally, without a branch or a re-read.
struct Block8Rsrc {
  __amdgpu_buffer_rsrc_t k, v, ks, vs;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc8(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int D>
__device__ __forceinline__ void load8(KV8Regs<D>& r, const Block8Rsrc& t, int lane) {
  constexpr int VB = V8Layout<D>::VB;
  const int row = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int c2 = 0; c2 < KV8Regs<D>::K16; ++c2)
    r.k[c2] = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(t.k, row * D + 64 * c2 + 16 * grp, 0, 0));
  r.ks = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(t.ks, 16 * grp, 0, 0));
  r.vs = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(t.vs, 16 * grp, 0, 0));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int off = (4 * grp + e) * D + VB * row;
    if constexpr (VB == 8) {
      const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(t.v, off, 0, kLoadNonTemporal));
      r.v[e][0] = x.x;
      r.v[e][1] = x.y;
    } else {
      const uint4 x = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t.v, off, 0, kLoadNonTemporal));
      r.v[e][0] = x.x;
      r.v[e][1] = x.y;
      r.v[e][2] = x.z;
      r.v[e][3] = x.w;
    }
  }
}

template <int D, int G>
__device__ __forceinline__ void wave8_init(Wave8<D, G>& st) {
  st.m = -__builtin_huge_valf();
  st.l = 0.f;
  st.vref = 0.f;
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) st.acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// Scores on the matrix cores (codes converted to fp16 pairs, exact), the K
// row scales, lazy-max online softmax; the weights times the V row scales
// over the block's largest, as fp16 pairs in pw: the A fragment of P.V (the
// scores' output layout puts head l % 16 and tokens 4 (l / 16) .. +3 in lane
// l, which is what the A operand asks for).  Returns the block's largest V
// scale (wave-uniform) for block_pv8.
// knew: when not null, the codes of the K row appended in this step for
// position ctx - 1 (LDS), with its K and V scales ksnew, vsnew; they replace
// that row of the block holding ctx - 1.
template <int D, int G>
__device__ __forceinline__ float block_scores8(KV8Regs<D>& r, const uint16_t* qs,
                                               Wave8<D, G>& st, int tok0, int ctx,
                                               float scale_log2, uint2& pw,
                                               const uint8_t* knew, float ksnew, float vsnew,
                                               int lane) {
  static_assert(G <= 16, "one MFMA column per query head");
  const int row = lane & 15, grp = lane >> 4;
  const float kNegInf = -__builtin_huge_valf();
  asm volatile("" ::: "memory");  // re-read the query fragments from LDS every block
  if (knew != nullptr && tok0 + 16 >= ctx) {
    const int tn = ctx - 1 - tok0;
    if (row == tn) {
#pragma unroll
      for (int c2 = 0; c2 < KV8Regs<D>::K16; ++c2)
        r.k[c2] = *reinterpret_cast<const uint4*>(knew + 64 * c2 + 16 * grp);
    }
    if (grp == (tn >> 2)) {
      const int i = tn & 3;
      if (i == 0) { r.ks.x = ksnew; r.vs.x = vsnew; }
      if (i == 1) { r.ks.y = ksnew; r.vs.y = vsnew; }
      if (i == 2) { r.ks.z = ksnew; r.vs.z = vsnew; }
      if (i == 3) { r.ks.w = ksnew; r.vs.w = vsnew; }
    }
  }
  const int hq = row < G ? row : 0;  // columns past G repeat head 0; masked below
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c2 = 0; c2 < KV8Regs<D>::K16; ++c2) {
    const uint4 w = r.k[c2];
    const uint4 a0 = {fp8x2_to_h2<false>(w.x), fp8x2_to_h2<true>(w.x),
                      fp8x2_to_h2<false>(w.y), fp8x2_to_h2<true>(w.y)};
    const uint4 a1 = {fp8x2_to_h2<false>(w.z), fp8x2_to_h2<true>(w.z),
                      fp8x2_to_h2<false>(w.w), fp8x2_to_h2<true>(w.w)};
    const uint16_t* qp = qs + hq * D + 64 * c2 + 16 * grp;
    const uint4 q0 = *reinterpret_cast<const uint4*>(qp);
    const uint4 q1 = *reinterpret_cast<const uint4*>(qp + 8);
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a0),
                                               __builtin_bit_cast(f16x8, q0), s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a1),
                                               __builtin_bit_cast(f16x8, q1), s, 0, 0, 0);
  }
  const float ks[4] = {r.ks.x, r.ks.y, r.ks.z, r.ks.w};
  const float vs[4] = {r.vs.x, r.vs.y, r.vs.z, r.vs.w};
  float x[4], vsv[4];
  bool grow = false;
  float vmax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool valid = tok0 + 4 * grp + i < ctx;
    // select, not multiply: a stale row's scale or codes may be anything
    x[i] = row < G && valid ? s[i] * (ks[i] * scale_log2) : kNegInf;
    grow |= x[i] > st.m + kRescaleSlack;
    vsv[i] = valid ? vs[i] : 0.f;
    vmax = fmaxf(vmax, vsv[i]);
  }
  vmax = max_of_rows(vmax);  // over the four lane groups' tokens
  if (__any(grow)) {
    const float bm = max_of_rows(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const float mn = fmaxf(st.m, bm);
    const float alpha = mn == kNegInf ? 1.f : fast_exp2(st.m - mn);
    st.l *= alpha;
    st.m = mn;
    // O rows are heads 4 (l / 16) + i here: their factors from the lanes
    // that hold those heads' scores (alpha is 1 for heads past G)
    float a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __shfl(alpha, 4 * grp + i);
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[ct][i] *= a[i];
  }
  // vmax is a power of two (or 0): 1 / vmax = 2 x 2^-k for vmax = 0.5 x 2^k,
  // exact, without a division
  const float inv_vmax =
      vmax > 0.f ? __builtin_ldexpf(2.f, -__builtin_amdgcn_frexp_expf(vmax)) : 0.f;
  const float neg_m = st.m == kNegInf ? 0.f : -st.m;
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(x[i] + neg_m);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  pw.x = pack_h2_rtz(p[0] * (vsv[0] * inv_vmax), p[1] * (vsv[1] * inv_vmax));
  pw.y = pack_h2_rtz(p[2] * (vsv[2] * inv_vmax), p[3] * (vsv[3] * inv_vmax));
  return vmax;
}

// P.V on the matrix cores: O (heads x d) += P (heads x 16 tokens) V (16
// tokens x d), one 16 x 16 x 16 product per column tile.  The B fragment of
// tile ct is byte ct of each of the lane's four token chunks: a 4 x 4 byte
// transpose (v_perm_b32) of one 32-bit word per token gives four tiles'
// codes, each converted to four fp16 values (exact).
// vnew: when not null, the codes of the V row appended for position ctx - 1.
template <int D, int G>
__device__ __forceinline__ void block_pv8(KV8Regs<D>& r, Wave8<D, G>& st, int tok0, int ctx,
                                          const uint2& pw, float vmax, const uint8_t* vnew,
                                          int lane) {
  constexpr int VB = V8Layout<D>::VB, VW = V8Layout<D>::VW;
  const int row = lane & 15, grp = lane >> 4;
  if (vnew != nullptr && tok0 + 16 >= ctx) {
    const int tn = ctx - 1 - tok0 - 4 * grp;  // this lane's token holding ctx - 1 (may be outside)
    if (tn >= 0 && tn < 4) {
      uint32_t nv[VW];
#pragma unroll
      for (int w = 0; w < VW; ++w) nv[w] = reinterpret_cast<const uint32_t*>(vnew + VB * row)[w];
      // constant indices keep r.v in registers
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e == tn)
#pragma unroll
          for (int w = 0; w < VW; ++w) r.v[e][w] = nv[w];
    }
  }
  // code 0 = +0 for rows past the context: stale rows never leak (a select on
  // every block, no branch: a branch around the buffer's registers would make
  // the compiler copy them and wait for every load in flight)
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bool valid = tok0 + 4 * grp + e < ctx;
#pragma unroll
    for (int w = 0; w < VW; ++w) r.v[e][w] = valid ? r.v[e][w] : 0u;
  }
  // acc moves to units of this block's largest V scale when it differs from
  // the last block's (a power-of-two ratio for scales the append writes:
  // exact); the weights are already relative to it.
  if (vmax > 0.f && vmax != st.vref) {  // the same in every lane
    const float ratio = st.vref / vmax;
#pragma unroll
    for (int ct = 0; ct < D / 16; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[ct][i] *= ratio;
    st.vref = vmax;
  }
  const f16x4 a = __builtin_bit_cast(f16x4, pw);
#pragma unroll
  for (int w = 0; w < VW; ++w) {
    // bytes {t0.c, t1.c, ...} of words x0..x3 (tokens 0..3), c = 0..3
    const uint32_t x0 = r.v[0][w], x1 = r.v[1][w], x2 = r.v[2][w], x3 = r.v[3][w];
    const uint32_t lo01 = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // t0.0 t1.0 t0.1 t1.1
    const uint32_t hi01 = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // t0.2 t1.2 t0.3 t1.3
    const uint32_t lo23 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
    const uint32_t col[4] = {__builtin_amdgcn_perm(lo23, lo01, 0x05040100u),
                             __builtin_amdgcn_perm(lo23, lo01, 0x07060302u),
                             __builtin_amdgcn_perm(hi23, hi01, 0x05040100u),
                             __builtin_amdgcn_perm(hi23, hi01, 0x07060302u)};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint2 b = {fp8x2_to_h2<false>(col[c]), fp8x2_to_h2<true>(col[c])};
      st.acc[4 * w + c] = __builtin_amdgcn_mfma_f32_16x16x16f16(
          a, __builtin_bit_cast(f16x4, b), st.acc[4 * w + c], 0, 0, 0);
    }
  }
}

// APPEND: the step's decode tokens are quantized and appended by this kernel
// (as the fp16 kernel does): row i of k_new / v_new ([Hkv][D] fp16, one token
// of sequence i) belongs at position ctx_i - 1.  The work-group whose
// partition holds that position quantizes the rows into LDS at its start
// (waves 0 and 1), uses them in place of the pool's row when slot_mapping[i]
// is the table's slot of ctx_i - 1, and writes codes and scales to
// slot_mapping[i] at its end (nothing when the slot is negative or beyond the
// pool) -- the same result as the append kernel followed by the attention.
template <int D, int G, bool APPEND>
__global__ __launch_bounds__(64 * kWaves, D == 128 ? 2 : 1) void paged_decode_fp8_kernel(
    const uint16_t* __restrict__ q, uint8_t* __restrict__ k_codes,
    uint8_t* __restrict__ v_codes, float* __restrict__ k_scale,
    float* __restrict__ v_scale, int64_t num_blocks, int32_t num_kv_heads,
    const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, int32_t ctx_clamp, int32_t partition_blocks,
    int32_t max_parts, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ part_o,
    float* __restrict__ part_ml, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int64_t* __restrict__ slot_mapping,
    int32_t num_tokens) {
  constexpr int EPL = D / 64;
  // Blocks in flight per wave (4 KiB each at d = 128, 8 KiB at d = 256).
  // Measured on MI355X: at d = 128 two per wave at two waves per SIMD beat
  // three or four (and one block at four waves per SIMD, which loses on
  // ragged batches); at d = 256 the 16 O tiles leave room for two blocks
  // only at one wave per SIMD, which beats one block at two.
  constexpr int NBUF = 2;
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_newc[2][APPEND ? D : 16];  // K, V codes
  __shared__ float s_news[2];                                                // their scales

  if (APPEND && (int)blockIdx.z >= max_parts) {
    // the z slices past the partitions (dispatched last): prefill rows, one
    // wave per (token, KV head) row of K or V
    const int64_t nxy = (int64_t)gridDim.x * gridDim.y;
    const int64_t w = (blockIdx.z - max_parts) * nxy + blockIdx.y * gridDim.x + blockIdx.x;
    const int64_t nw = (gridDim.z - max_parts) * nxy;
    const int64_t r0 = (int64_t)gridDim.x * num_kv_heads;  // past the decode rows
    const int64_t n = 2 * ((int64_t)num_tokens * num_kv_heads - r0);
    for (int64_t k = w * kWaves + (threadIdx.x >> 6); k < n; k += nw * kWaves)
      append_row_fp8<D>(k_codes, v_codes, k_scale, v_scale, num_blocks, num_kv_heads, k_new,
                        v_new, slot_mapping, r0 + (k >> 1), (k & 1) != 0, threadIdx.x & 63);
    return;
  }
  const int i = blockIdx.x, g = blockIdx.y;
  const int part = max_parts - 1 - (int)blockIdx.z;  // highest partitions dispatch first
  const int num_q_heads = num_kv_heads * G;
  // the wave index is the same in all its lanes (kept in scalar registers)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b0 = part * partition_blocks;
  const int32_t* bt_row = block_tables + (int64_t)i * max_blocks_per_seq;

  uint32_t raw_bid = 0;
  {
    const int e = b0 + wave + kWaves * lane;
    if (wave + kWaves * lane < partition_blocks && e < max_blocks_per_seq)
      raw_bid = (uint32_t)bt_row[e];
  }
  const uint4* qsrc =
      reinterpret_cast<const uint4*>(q + ((int64_t)i * num_q_heads + (int64_t)g * G) * D);
  constexpr int QCH = G * D / 8;
  uint4 qstage[(QCH + 255) / 256];
#pragma unroll
  for (int k = 0; k < (QCH + 255) / 256; ++k)
    if (tid + 256 * k < QCH) qstage[k] = qsrc[tid + 256 * k];
  int64_t slot = -1;
  if constexpr (APPEND) slot = slot_mapping[i];

  const int ctx = min(context_lens[i], ctx_clamp);
  const int nblk = (ctx + 15) >> 4;
  if (ctx <= 0 || b0 >= nblk) return;  // uniform over the work-group
  const int b1 = min(b0 + partition_blocks, nblk);
  const int nparts = (nblk + partition_blocks - 1) / partition_blocks;

  const int nbw = (b1 - b0 - wave + kWaves - 1) / kWaves;
  const int my_bid =
      lane < nbw ? (int)(raw_bid < (uint64_t)num_blocks ? raw_bid : (uint32_t)(num_blocks - 1))
                 : 0;
  const int64_t tile = (int64_t)16 * D;           // bytes of one block of one head
  const int64_t head_off = (int64_t)g * tile;
  const int64_t block_stride = (int64_t)num_kv_heads * tile;
  // Loads are issued unconditionally, through buffer resources that are
  // empty past the wave's last block: a load under a branch makes the
  // compiler merge the buffer registers at the join and wait for all loads.
  auto load_block = [&](KV8Regs<D>& r, int k) {
    const bool valid = k < nbw;
    const int64_t bid = __builtin_amdgcn_readlane(my_bid, valid ? k : 0);
    const int64_t o = bid * block_stride + head_off;
    const int64_t so = (bid * num_kv_heads + g) * 16;
    const uint32_t cb = valid ? (uint32_t)tile : 0u, sb = valid ? 64u : 0u;
    const Block8Rsrc t{rsrc8(k_codes + o, cb), rsrc8(v_codes + o, cb), rsrc8(k_scale + so, sb),
                       rsrc8(v_scale + so, sb)};
    load8<D>(r, t, lane);
  };

  // The first blocks' loads in the same order as the loop issues them (the
  // scheduler may not move one across another block's): the wait counts at
  // the loop top hold for both ways in, and stay deep.
  KV8Regs<D> buf[NBUF];
#pragma unroll
  for (int j = 0; j < NBUF; ++j) {
    load_block(buf[j], j);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int k = 0; k < (QCH + 255) / 256; ++k)
    if (tid + 256 * k < QCH) reinterpret_cast<uint4*>(s_q)[tid + 256 * k] = qstage[k];
  // The appended token sits in block nblk - 1; this partition holds it when
  // nblk <= b1: its K (wave 0) and V (wave 1) rows quantized into LDS.
  const bool owner = APPEND && nblk <= b1;
  if constexpr (APPEND) {
    if (owner && wave < 2) {
      int e;
      const uint32_t c = quantize_row_wave<D>(
          (wave == 0 ? k_new : v_new) + ((int64_t)i * num_kv_heads + g) * D, lane, e);
      store_codes<D>(&s_newc[wave][EPL * lane], c);
      if (lane == 0) s_news[wave] = exp2i(e);
    }
  }
  __syncthreads();

  // the wave that reads that block substitutes the rows
  const uint8_t* knew = nullptr;
  const uint8_t* vnew = nullptr;
  float ksnew = 0.f, vsnew = 0.f;
  if constexpr (APPEND) {
    const int kl = nblk - 1 - b0 - wave;  // multiple of kWaves when this wave reads it
    if (owner && kl >= 0 && kl % kWaves == 0 && slot >= 0) {
      const uint32_t raw_last = (uint32_t)__builtin_amdgcn_readlane((int)raw_bid, kl / kWaves);
      if (raw_last < (uint64_t)num_blocks &&
          slot == (int64_t)raw_last * 16 + ((ctx - 1) & 15)) {
        knew = s_newc[0];
        vnew = s_newc[1];
        ksnew = s_news[0];
        vsnew = s_news[1];
      }
    }
  }

  Wave8<D, G> st;
  wave8_init(st);
  auto tok_of = [&](int kk) { return (b0 + wave + kWaves * kk) * 16; };
  // NBUF blocks per trip with no exit in its middle (with one, the compiler
  // sinks loads into the continuing path and the wait counts at the top of
  // the loop drain the prefetch); the last 1 .. NBUF blocks after it.  The
  // appended row can only be in the wave's last block, so only the blocks
  // after the loop carry the substitution (fewer registers in the loop).
  int k = 0;
  for (; k + NBUF < nbw; k += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      uint2 pw;
      const float vmax = block_scores8<D, G>(buf[j], s_q, st, tok_of(k + j), ctx, scale_log2,
                                             pw, nullptr, 0.f, 0.f, lane);
      block_pv8<D, G>(buf[j], st, tok_of(k + j), ctx, pw, vmax, nullptr, lane);
      load_block(buf[j], k + j + NBUF);
    }
  }
#pragma unroll
  for (int j = 0; j < NBUF; ++j) {
    if (k + j < nbw) {
      uint2 pw;
      const float vmax = block_scores8<D, G>(buf[j], s_q, st, tok_of(k + j), ctx, scale_log2,
                                             pw, knew, ksnew, vsnew, lane);
      block_pv8<D, G>(buf[j], st, tok_of(k + j), ctx, pw, vmax, vnew, lane);
    }
  }

  // The wave's per-head totals to LDS (O tiles back to absolute units and
  // to d = VB n + ct); then merge the 4 waves.
  float lw = st.l;
  lw += __shfl_xor(lw, 16);
  lw += __shfl_xor(lw, 32);
  if (lane < G) {
    s_m[wave][lane] = st.m;
    s_l[wave][lane] = lw;
  }
  {
    constexpr int VB = V8Layout<D>::VB;
    const int row = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * grp + i;
      if (h < G)
#pragma unroll
        for (int ct = 0; ct < VB; ++ct) s_acc[wave][h][VB * row + ct] = st.acc[ct][i] * st.vref;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 64 * kWaves) {
    const int h = idx / D, e = idx - h * D;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (s_l[w][h] > 0.f) {
        const float wt = fast_exp2(s_m[w][h] - M);
        L += wt * s_l[w][h];
        O += wt * s_acc[w][h][e];
      }
    }
    const int64_t row_head = (int64_t)i * num_q_heads + g * G + h;
    if (nparts == 1) {
      out[row_head * D + e] = __builtin_bit_cast(uint16_t, (f16)(O / L));
    } else {
      const int64_t pidx = row_head * max_parts + part;
      part_o[pidx * D + e] = O / L;
      if (e == 0) {
        part_ml[pidx * 2] = M;
        part_ml[pidx * 2 + 1] = L;
      }
    }
  }

  // The appended rows to their slot (only this work-group reads the block
  // that holds them, and it is done with it).
  if constexpr (APPEND) {
    if (owner && slot >= 0 && (slot >> 4) < num_blocks && wave < 2) {
      const int64_t rowi = ((slot >> 4) * num_kv_heads + g) * 16 + (slot & 15);
      const uint32_t c = EPL == 2 ? *reinterpret_cast<const uint16_t*>(&s_newc[wave][EPL * lane])
                                  : *reinterpret_cast<const uint32_t*>(&s_newc[wave][EPL * lane]);
      store_codes<D>((wave == 0 ? k_codes : v_codes) + rowi * D + EPL * lane, c);
      if (lane == 0) (wave == 0 ? k_scale : v_scale)[rowi] = s_news[wave];
    }
  }
}

template <int D, int G, bool APPEND>
hipError_t launch_decode_fp8_dg(const void* q, void* k_codes, void* v_codes, float* k_scale,
                                float* v_scale, int64_t num_blocks,
                                int32_t num_kv_heads, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_decode_seqs, float scale, const DecodePlan& plan,
                                const DecodeAppend& app, void* out, void* workspace,
                                hipStream_t stream, DecodeMerge* defer) {
  const int32_t num_q_heads = num_kv_heads * G;
  const int64_t clamp64 = std::min<int64_t>((int64_t)max_blocks_per_seq * 16,
                                            (int64_t)plan.max_parts * plan.partition_blocks * 16);
  const int32_t ctx_clamp = (int32_t)std::min<int64_t>(clamp64, INT32_MAX);
  float* part_o = static_cast<float*>(workspace);
  float* part_ml =
      part_o ? part_o + (size_t)num_decode_seqs * num_q_heads * plan.max_parts * D : nullptr;
  // prefill rows of the step (rows past the decode rows) get z slices of
  // their own after the partitions
  const int64_t xy = (int64_t)num_decode_seqs * num_kv_heads;
  const int32_t app_z =
      APPEND ? (int32_t)((append_groups(app.num_tokens - num_decode_seqs) + xy - 1) / xy) : 0;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  hipLaunchKernelGGL((paged_decode_fp8_kernel<D, G, APPEND>),
                     dim3(num_decode_seqs, num_kv_heads, plan.max_parts + app_z), dim3(64 * kWaves),
                     D == 128 ? kResidencyPadBytes : 0,
                     stream, static_cast<const uint16_t*>(q), static_cast<uint8_t*>(k_codes),
                     static_cast<uint8_t*>(v_codes), k_scale, v_scale, num_blocks,
                     num_kv_heads, block_tables, max_blocks_per_seq, context_lens, ctx_clamp,
                     plan.partition_blocks, plan.max_parts, scale * kLog2e,
                     static_cast<uint16_t*>(out), part_o, part_ml,
                     static_cast<const uint16_t*>(app.k_new),
                     static_cast<const uint16_t*>(app.v_new), app.slot_mapping,
                     app.num_tokens);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.max_parts <= 1) return err;
  if (defer) {
    *defer = grid_merge(part_o, part_ml, context_lens, ctx_clamp, plan, num_decode_seqs,
                        num_q_heads);
    return hipSuccess;
  }
  return launch_decode_merge(part_o, part_ml, context_lens, ctx_clamp, plan, num_decode_seqs,
                             num_q_heads, D, out, stream);
}

template <int D>
hipError_t launch_decode_fp8_d(int32_t group, const void* q, void* kc, void* vc, float* ks,
                               float* vs, int64_t num_blocks, int32_t num_kv_heads,
                               const int32_t* bt, int32_t maxblk, const int32_t* ctx,
                               int32_t nseq, float scale, const DecodePlan& plan,
                               const DecodeAppend& app, void* out, void* ws,
                               hipStream_t stream, DecodeMerge* defer) {
  const bool fused = app.k_new != nullptr;
#define PKV_CASE(GG)                                                                          \
  case GG:                                                                                   \
    return fused ? launch_decode_fp8_dg<D, GG, true>(q, kc, vc, ks, vs, num_blocks,          \
                                                     num_kv_heads, bt, maxblk, ctx, nseq,    \
                                                     scale, plan, app, out, ws, stream,      \
                                                     defer)                                  \
                 : launch_decode_fp8_dg<D, GG, false>(q, kc, vc, ks, vs, num_blocks,         \
                                                      num_kv_heads, bt, maxblk, ctx, nseq,   \
                                                      scale, plan, app, out, ws, stream,     \
                                                      defer);
  switch (group) {
    PKV_CASE(1) PKV_CASE(2) PKV_CASE(3) PKV_CASE(4)
    PKV_CASE(5) PKV_CASE(6) PKV_CASE(7) PKV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef PKV_CASE
}

}  // namespace

hipError_t launch_kv_append_fp8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                                int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, int32_t num_tokens,
                                hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int64_t rows = (int64_t)num_tokens * num_kv_heads;
  const dim3 grid((uint32_t)((rows + 3) / 4), 2);
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  if (head_dim == 128)
    hipLaunchKernelGGL(kv_append_fp8_kernel<128>, grid, dim3(256), 0, stream,
                       static_cast<uint8_t*>(k_codes), static_cast<uint8_t*>(v_codes), k_scale,
                       v_scale, num_blocks, num_kv_heads, static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), slot_mapping, rows);
  else if (head_dim == 256)
    hipLaunchKernelGGL(kv_append_fp8_kernel<256>, grid, dim3(256), 0, stream,
                       static_cast<uint8_t*>(k_codes), static_cast<uint8_t*>(v_codes), k_scale,
                       v_scale, num_blocks, num_kv_heads, static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), slot_mapping, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_paged_decode_fp8(const void* q, void* k_codes, void* v_codes, float* k_scale,
                                   float* v_scale, int64_t num_blocks, int32_t num_kv_heads,
                                   int32_t num_q_heads, int32_t head_dim,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_decode_seqs,
                                   float scale, const DecodePlan& plan, const DecodeAppend& app,
                                   void* out, void* workspace, hipStream_t stream,
                                   DecodeMerge* defer) {
  if (num_decode_seqs == 0) return hipSuccess;
  const int32_t group = num_q_heads / num_kv_heads;
  if (head_dim == 128)
    return launch_decode_fp8_d<128>(group, q, k_codes, v_codes, k_scale, v_scale, num_blocks,
                                    num_kv_heads, block_tables, max_blocks_per_seq,
                                    context_lens, num_decode_seqs, scale, plan, app, out,
                                    workspace, stream, defer);
  if (head_dim == 256)
    return launch_decode_fp8_d<256>(group, q, k_codes, v_codes, k_scale, v_scale, num_blocks,
                                    num_kv_heads, block_tables, max_blocks_per_seq,
                                    context_lens, num_decode_seqs, scale, plan, app, out,
                                    workspace, stream, defer);
  return hipErrorInvalidValue;
}

}  // namespace pkv
