// decode_block.h -- per-block pieces of paged decode attention shared by the
// decode kernels (decode.hip, decode_sched.hip): the register layout of one
// 16-token K/V block of one KV head, its loads, the q.k scores with the
// lazy-max online softmax, and the P.V accumulation.
//
// Scores on the matrix cores: with grouped-query attention the G query heads
// of a KV head read the same keys, so the scores of a block are a small dense
// product S^T = K Q^T (16 tokens x d times d x G), one
// v_mfma_f32_16x16x32_f16 per 32 values of d.  K is the A operand loaded
// straight from the block (lane l holds 8 values of token row l % 16 at
// column 32c + 8 (l / 16)); Q^T is the B operand read from LDS (column n =
// query head n of the group; columns n >= G hold some head's query and their
// scores are masked).  The result gives lane l the scores of head l % 16 for
// tokens 4 (l / 16) .. +3.
// Online softmax, base 2: scores are scaled by scale*log2(e); each lane keeps
//   the running max m of its head and only raises it when a score passes it
//   by more than kRescaleSlack (a wave vote; then the head's accumulators are
//   rescaled), so weights p = 2^(s-m) stay in (0, 256] and the common case
//   needs no cross-lane traffic at all.
// P.V at d = 128 on the matrix cores too: O = P V with heads as rows, one
//   v_mfma_f32_16x16x16_f16 per 16-column tile of d.  The scores' layout
//   (head l % 16, tokens 4 (l / 16) .. +3 in lane l) is P's A fragment as it
//   stands, so the weights stay in registers.  Lane l loads V of tokens
//   4 (l / 16) .. +3 at columns 8 (l % 16) .. +7 (one 16-byte load per
//   token), and one v_perm_b32 per token pair builds a column tile's B
//   fragment: output column n of tile ct is d = 8 n + ct.
// At d = 256 (16 such tiles would need 64 more registers): every lane owns
//   d/64 output elements of all 16 tokens, the weights travel from the score
//   layout to all lanes through a small per-wave LDS buffer as fp16 pairs of
//   consecutive tokens, and P.V is v_dot2_f32_f16 over those pairs.
// Masking is by select: positions >= ctx get score -inf and their V rows are
//   zeroed before use, so stale or NaN-poisoned slots never leak.
#pragma once

#include "device_util.h"

namespace pkv {
namespace decode_block {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kRescaleSlack = 8.f;  // lazy max: rescale only past m + 8 (base 2)

template <int D> struct VFrag;
template <> struct VFrag<256> { typedef uint2 T; };

template <int D>
struct KVRegs {
  static constexpr int KC = D / 32;  // 32-wide chunks of d (MFMA K)
  uint4 k[KC];                       // token row lane % 16, columns 32c + 8 (lane / 16) .. +7
  typename VFrag<D>::T v[16];
};
template <>
struct KVRegs<128> {
  static constexpr int KC = 4;
  uint4 k[KC];
  uint4 v[4];  // tokens 4 (lane / 16) + e, columns 8 (lane % 16) .. +7
};

template <int D, int G>
struct WaveState {
  float m;              // running max of this lane's head (lane % 16), base 2
  float l;              // sum of its weights over this lane's tokens
  float acc[G][D / 64]; // sum of weight * v over this lane's output elements
};
template <int G>
struct WaveState<128, G> {
  float m;
  float l;
  f32x4 acc[8];  // O tiles: heads 4 (lane / 16) + i, column (ct, lane % 16): d = 8 (lane % 16) + ct
  uint2 pw;      // this block's weights (P's A fragment)
};

template <int D, int G>
__device__ __forceinline__ void wave_init(WaveState<D, G>& st) {
  st.m = -__builtin_huge_valf();
  st.l = 0.f;
  if constexpr (D == 128) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) st.acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < D / 64; ++e) st.acc[h][e] = 0.f;
  }
}

// The wave's partial (per head: max, weight sum, weighted V columns) into
// per-wave LDS rows: s_acc_w[G][D], s_m_w[G], s_l_w[G].
template <int D, int G>
__device__ __forceinline__ void wave_store(const WaveState<D, G>& st, float (&s_acc_w)[G][D],
                                           float (&s_m_w)[G], float (&s_l_w)[G], int lane) {
  constexpr int EPL = D / 64;
  float l = st.l;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);  // the head's 16 tokens per block, over the 4 lane groups
  const int row = lane & 15;
  if (lane < 16 && row < G) {
    s_m_w[row] = st.m;
    s_l_w[row] = l;
  }
  if constexpr (D == 128) {
    const int grp = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * grp + i;
      if (h < G)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) s_acc_w[h][8 * row + ct] = st.acc[ct][i];
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc_w[h][EPL * lane + e] = st.acc[h][e];
  }
}

template <int D>
__device__ __forceinline__ void load_k(KVRegs<D>& r, const uint16_t* __restrict__ ktile, int lane) {
#pragma unroll
  for (int c = 0; c < KVRegs<D>::KC; ++c)
    r.k[c] = *reinterpret_cast<const uint4*>(ktile + (lane & 15) * D + 32 * c + 8 * (lane >> 4));
}

template <int D>
__device__ __forceinline__ void load_v(KVRegs<D>& r, const uint16_t* __restrict__ vtile, int lane) {
  if constexpr (D == 128) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r.v[e] = *reinterpret_cast<const uint4*>(vtile + (4 * (lane >> 4) + e) * D + 8 * (lane & 15));
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t)
      r.v[t] = *reinterpret_cast<const typename VFrag<D>::T*>(vtile + t * D + (D / 64) * lane);
  }
}

// The same loads through a raw buffer resource over one tile (4 KiB at
// d = 128): a resource of 0 bytes reads nothing and gives zeros, so a loop
// can issue its prefetch every trip without a branch (a load under a branch
// makes the compiler merge the buffer registers at the join, which waits for
// the load right after issuing it).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* tile, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(tile), (short)0, (int)bytes,
                                           0x00020000);
}

template <int D>
__device__ __forceinline__ void load_k(KVRegs<D>& r, __amdgpu_buffer_rsrc_t ktile, int lane) {
  const int base = ((lane & 15) * D + 8 * (lane >> 4)) * 2;
#pragma unroll
  for (int c = 0; c < KVRegs<D>::KC; ++c)
    r.k[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ktile, base + 64 * c, 0, 0));
}

template <int D>
__device__ __forceinline__ void load_v(KVRegs<D>& r, __amdgpu_buffer_rsrc_t vtile, int lane) {
  if constexpr (D == 128) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int off = ((4 * (lane >> 4) + e) * D + 8 * (lane & 15)) * 2;
      r.v[e] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(vtile, off, 0, kLoadNonTemporal));
    }
  } else {
    const int base = (D / 64) * lane * 2;
#pragma unroll
    for (int t = 0; t < 16; ++t)
      r.v[t] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(vtile, base + t * D * 2, 0, kLoadNonTemporal));
  }
}

// P.V over one token pair for one packed dword of V per token:
// lo element pair (a.lo, b.lo), hi element pair (a.hi, b.hi).
template <int G>
__device__ __forceinline__ void pv_dword(float (&acc)[G][2], const uint32_t (&pr)[G], uint32_t a,
                                         uint32_t b) {
  const uint32_t lo = (a & 0xffffu) | (b << 16);
  const uint32_t hi = (a >> 16) | (b & 0xffff0000u);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc[h][0] = dot2(pr[h], lo, acc[h][0]);
    acc[h][1] = dot2(pr[h], hi, acc[h][1]);
  }
}

// One 16-token block, first half: scores on the matrix cores, lazy-max online
// softmax, weights to st.pw (d = 128) or to the wave's LDS buffer (d = 256;
// pair pi = tokens 2pi, 2pi + 1).
// After it returns the K registers are free (the next K load may target them).
// tok0 = logical position of the block's first token.
// qs = the segment's G query rows in LDS ([G][D] fp16).
// knew: when not null, the K row appended in this step for position ctx - 1
// ([D] fp16 in LDS); it replaces that row of the block holding ctx - 1.
template <int D, int G>
__device__ __forceinline__ void block_scores(KVRegs<D>& r, const uint16_t* qs,
                                             WaveState<D, G>& st, int tok0, int ctx,
                                             float scale_log2, uint32_t* __restrict__ p_lds,
                                             const uint16_t* knew, int lane) {
  constexpr int KC = KVRegs<D>::KC;
  constexpr int GP = (G + 3) & ~3;
  static_assert(G <= 16, "one MFMA column per query head");
  const int row = lane & 15, grp = lane >> 4;
  const float kNegInf = -__builtin_huge_valf();
  asm volatile("" ::: "memory");  // re-read the query fragments from LDS every block
  if (knew != nullptr && tok0 + 16 >= ctx && row == ctx - 1 - tok0) {
#pragma unroll
    for (int c = 0; c < KC; ++c)
      r.k[c] = *reinterpret_cast<const uint4*>(knew + 32 * c + 8 * grp);
  }

  // S^T = K Q^T: s[i] = score of head `row` with token 4 grp + i
  const int hq = row < G ? row : 0;  // columns past G repeat head 0; masked below
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    const uint4 qv = *reinterpret_cast<const uint4*>(qs + hq * D + 32 * c + 8 * grp);
    s = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, r.k[c]),
                                               __builtin_bit_cast(f16x8, qv), s, 0, 0, 0);
  }
  float x[4];
  bool grow = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = row < G && tok0 + 4 * grp + i < ctx;
    x[i] = ok ? s[i] * scale_log2 : kNegInf;
    grow |= x[i] > st.m + kRescaleSlack;
  }
  if (__any(grow)) {
    // the head's block maximum over its 16 tokens (4 lane groups)
    float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(st.m, bm);
    // a lane of no head (row >= G) stays at -inf with weight 0
    const float alpha = mn == kNegInf ? 1.f : fast_exp2(st.m - mn);
    st.l *= alpha;
    st.m = mn;
    if constexpr (D == 128) {
      // O rows are heads 4 grp + i: their factors from the lanes holding them
      float a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = __shfl(alpha, 4 * grp + i);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[ct][i] *= a[i];
    } else {
      // head h's factor lives in lane h
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ah = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
#pragma unroll
        for (int e = 0; e < D / 64; ++e) st.acc[h][e] *= ah;
      }
    }
  }
  const float neg_m = st.m == kNegInf ? 0.f : -st.m;
  const uint32_t pp0 = pack_h2_rtz(fast_exp2(x[0] + neg_m), fast_exp2(x[1] + neg_m));
  const uint32_t pp1 = pack_h2_rtz(fast_exp2(x[2] + neg_m), fast_exp2(x[3] + neg_m));
  // l sums exactly the rounded weights that P.V uses
  st.l = dot2(pp0, kOnesH2, st.l);
  st.l = dot2(pp1, kOnesH2, st.l);
  if constexpr (D == 128) {
    st.pw = uint2{pp0, pp1};
  } else {
    if (row < G) {
      p_lds[(2 * grp) * GP + row] = pp0;
      p_lds[(2 * grp + 1) * GP + row] = pp1;
    }
    wave_fence();
  }
}

// Second half: P.V from the V registers and the weights.  Rows of positions
// >= ctx are zeroed first (select), so stale slots never leak; vnew, when not
// null, is the V row appended for position ctx - 1 (LDS).
template <int D, int G>
__device__ __forceinline__ void block_pv(KVRegs<D>& r, WaveState<D, G>& st, int tok0, int ctx,
                                         const uint32_t* __restrict__ p_lds,
                                         const uint16_t* vnew, int lane) {
  if constexpr (D == 128) {
    const int row = lane & 15, grp = lane >> 4;
    // The appended row and the rows past the context by select only: a
    // branch around the buffer's registers makes the compiler wait for every
    // load in flight.
    uint4 nv = {0u, 0u, 0u, 0u};
    int tn = -1;  // this lane's token (0..3) holding ctx - 1, if any
    if (vnew != nullptr && tok0 + 16 >= ctx) {
      tn = ctx - 1 - tok0 - 4 * grp;
      nv = *reinterpret_cast<const uint4*>(vnew + 8 * row);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint4 x = e == tn ? nv : r.v[e];
      r.v[e] = tok0 + 4 * grp + e < ctx ? x : uint4{0u, 0u, 0u, 0u};
    }
    // O += P V: tile ct takes the low (even ct) or high half of word ct / 2
    // of each token's 8 columns
    const f16x4 a = __builtin_bit_cast(f16x4, st.pw);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      const int w = ct >> 1;
      const uint32_t sel = (ct & 1) ? 0x07060302u : 0x05040100u;
      auto word = [&](const uint4& v) {
        return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
      };
      const uint2 b = {__builtin_amdgcn_perm(word(r.v[1]), word(r.v[0]), sel),
                       __builtin_amdgcn_perm(word(r.v[3]), word(r.v[2]), sel)};
      st.acc[ct] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, __builtin_bit_cast(f16x4, b),
                                                         st.acc[ct], 0, 0, 0);
    }
  } else {
    constexpr int GP = (G + 3) & ~3;
    if (vnew != nullptr && tok0 + 16 >= ctx) {
      // one bit per token row, tested with constant t: keeps r.v in registers
      const uint32_t hit = 1u << (ctx - 1 - tok0);
      const typename VFrag<D>::T nv =
          *reinterpret_cast<const typename VFrag<D>::T*>(vnew + (D / 64) * lane);
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (hit & (1u << t)) r.v[t] = nv;
    }
    if (tok0 + 16 > ctx) {
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (tok0 + t >= ctx) r.v[t] = typename VFrag<D>::T{};
    }
    // P.V: pair pi holds tokens 2pi and 2pi + 1.
#pragma unroll
    for (int pi = 0; pi < 8; ++pi) {
      const int ta = 2 * pi, tb = ta + 1;
      uint32_t pr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pr[h] = p_lds[pi * GP + h];
      float lo[G][2], hi[G][2];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        lo[h][0] = st.acc[h][0]; lo[h][1] = st.acc[h][1];
        hi[h][0] = st.acc[h][2]; hi[h][1] = st.acc[h][3];
      }
      pv_dword<G>(lo, pr, r.v[ta].x, r.v[tb].x);
      pv_dword<G>(hi, pr, r.v[ta].y, r.v[tb].y);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        st.acc[h][0] = lo[h][0]; st.acc[h][1] = lo[h][1];
        st.acc[h][2] = hi[h][0]; st.acc[h][3] = hi[h][1];
      }
    }
    wave_fence();
  }
}

// Prefill rows appended by extra work-groups of a decode launch: rows
// r_begin .. r_end - 1 of k_new / v_new ([rows][Hkv][D] fp16) go to their
// slots (slot_mapping[row]; negative, or past the pool: skipped), one 16-byte
// chunk per thread and pass; work-group w of nw takes every nw-th pass.
// Their slots lie in blocks that only their own (prefill) sequence lists, so
// the decode work-groups of the same launch never read them.
template <int D>
__device__ __forceinline__ void append_rows(uint16_t* __restrict__ k_pool,
                                            uint16_t* __restrict__ v_pool, int64_t num_blocks,
                                            int num_kv_heads, const uint16_t* __restrict__ k_new,
                                            const uint16_t* __restrict__ v_new,
                                            const int64_t* __restrict__ slot_mapping,
                                            int64_t r_begin, int64_t r_end, int64_t w,
                                            int64_t nw, int tid, int threads) {
  constexpr int RCH = D / 8;  // 16-byte chunks of one head's row
  const int per_pool = num_kv_heads * RCH;
  const int64_t total = (r_end - r_begin) * 2 * per_pool;
  for (int64_t idx = w * threads + tid; idx < total; idx += nw * threads) {
    const int64_t t = r_begin + idx / (2 * per_pool);
    int c = (int)(idx % (2 * per_pool));
    const bool is_v = c >= per_pool;
    c -= is_v ? per_pool : 0;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot / 16 >= num_blocks) continue;
    const int g = c / RCH, ch = c - g * RCH;
    const uint4 val =
        reinterpret_cast<const uint4*>((is_v ? v_new : k_new) + (t * num_kv_heads + g) * D)[ch];
    reinterpret_cast<uint4*>((is_v ? v_pool : k_pool) +
                             (((slot / 16) * num_kv_heads + g) * 16 + slot % 16) * D)[ch] = val;
  }
}

}  // namespace decode_block
}  // namespace pkv
