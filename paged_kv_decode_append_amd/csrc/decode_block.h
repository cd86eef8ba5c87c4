// decode_block.h -- per-block pieces of paged decode attention shared by the
// decode kernels (decode.hip, decode_sched.hip): the register layout of one
// 16-token K/V block of one KV head, its loads, the q.k scores with the
// lazy-max online softmax, and the P.V accumulation.
//
// K layout: D/16 lanes share one token row, each lane holding 16 of its d
//   values (two 16-byte chunks), so a K load instruction reads whole 128-byte
//   runs of rows.  q.k is 8 packed fp16 dot products (v_dot2_f32_f16, fp32
//   accumulate) per head with the query fragments read from LDS, then a DPP
//   butterfly inside the lane group.
// Online softmax, base 2: scores are scaled by scale*log2(e); the running max
//   m is wave-uniform and only raised when a score exceeds it by more than
//   kRescaleSlack (then the accumulators are rescaled), so weights
//   p = 2^(s-m) stay in (0, 256] and the common case does no rescale.
// V layout: every lane owns d/64 output elements of all 16 tokens, so the
//   P.V accumulation needs no cross-lane reduction.  The weights travel from
//   the K layout to all lanes through a small per-wave LDS buffer as fp16
//   pairs of tokens, and P.V is again v_dot2_f32_f16 over those pairs.
// Masking is by select: positions >= ctx get score -inf and their V rows are
//   zeroed before use, so stale or NaN-poisoned slots never leak.
#pragma once

#include "device_util.h"

namespace pkv {
namespace decode_block {

constexpr float kRescaleSlack = 8.f;  // lazy max: rescale only past m + 8 (base 2)

template <int D> struct VFrag;
template <> struct VFrag<128> { typedef uint32_t T; };
template <> struct VFrag<256> { typedef uint2 T; };

template <int D>
struct KVRegs {
  static constexpr int LPT = D / 16;    // lanes sharing one K row
  static constexpr int TPS = 64 / LPT;  // tokens covered by one wave-wide K load
  static constexpr int SPB = 16 / TPS;  // K loads (steps) per 16-token block
  uint4 k[SPB][2];
  typename VFrag<D>::T v[16];
};

template <int D, int G>
struct WaveState {
  float m[G];           // running max of base-2 scores (wave-uniform)
  float l[G];           // sum of weights over this lane group's tokens
  float acc[G][D / 64]; // sum of weight * v over this lane's output elements
};

template <int D>
__device__ __forceinline__ void load_k(KVRegs<D>& r, const uint16_t* __restrict__ ktile, int lane) {
  constexpr int LPT = KVRegs<D>::LPT, TPS = KVRegs<D>::TPS, SPB = KVRegs<D>::SPB;
  const int tl = lane / LPT, c = lane % LPT;
#pragma unroll
  for (int s = 0; s < SPB; ++s)
#pragma unroll
    for (int ch = 0; ch < 2; ++ch)
      r.k[s][ch] =
          *reinterpret_cast<const uint4*>(ktile + (tl + TPS * s) * D + 8 * (c + LPT * ch));
}

template <int D>
__device__ __forceinline__ void load_v(KVRegs<D>& r, const uint16_t* __restrict__ vtile, int lane) {
#pragma unroll
  for (int t = 0; t < 16; ++t)
    r.v[t] = *reinterpret_cast<const typename VFrag<D>::T*>(vtile + t * D + (D / 64) * lane);
}

__device__ __forceinline__ float dot16(const uint32_t (&q)[8], const uint4& a, const uint4& b) {
  float s = 0.f;
  s = dot2(q[0], a.x, s);
  s = dot2(q[1], a.y, s);
  s = dot2(q[2], a.z, s);
  s = dot2(q[3], a.w, s);
  s = dot2(q[4], b.x, s);
  s = dot2(q[5], b.y, s);
  s = dot2(q[6], b.z, s);
  s = dot2(q[7], b.w, s);
  return s;
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

// One 16-token block, first half: scores from the K registers, lazy-max
// online softmax, weights to the wave's LDS buffer.  After it returns the K
// registers are free (the next K load may target them).
// tok0 = logical position of the block's first token.
// qs = the segment's G query rows in LDS ([G][D] fp16); each lane reads its
// 16-value fragments per block instead of holding them in registers.
// knew: when not null, the K row appended in this step for position ctx - 1
// ([D] fp16 in LDS); it replaces that row of the block holding ctx - 1.
template <int D, int G>
__device__ __forceinline__ void block_scores(KVRegs<D>& r, const uint16_t* qs,
                                             WaveState<D, G>& st, int tok0, int ctx,
                                             float scale_log2, uint32_t* __restrict__ p_lds,
                                             const uint16_t* knew, int lane) {
  constexpr int LPT = KVRegs<D>::LPT, TPS = KVRegs<D>::TPS, SPB = KVRegs<D>::SPB;
  constexpr int GP = (G + 3) & ~3;
  const int tl = lane / LPT, c = lane % LPT;
  const bool tail = tok0 + 16 > ctx;
  const float kNegInf = -__builtin_huge_valf();
  asm volatile("" ::: "memory");  // re-read the query fragments from LDS every block
  if (knew != nullptr && tok0 + 16 >= ctx) {
    const int row = ctx - 1 - tok0;
    const uint4 n0 = *reinterpret_cast<const uint4*>(knew + 8 * c);
    const uint4 n1 = *reinterpret_cast<const uint4*>(knew + 8 * (c + LPT));
#pragma unroll
    for (int s = 0; s < SPB; ++s)
      if (tl + TPS * s == row) {
        r.k[s][0] = n0;
        r.k[s][1] = n1;
      }
  }

  // Scores of this lane group's SPB tokens (tl + TPS*s) for every head.
  float x[SPB][G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 qa = *reinterpret_cast<const uint4*>(qs + h * D + 8 * c);
    const uint4 qb = *reinterpret_cast<const uint4*>(qs + h * D + 8 * (c + LPT));
    const uint32_t qh[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
    for (int s = 0; s < SPB; ++s)
      x[s][h] = group_sum<LPT>(dot16(qh, r.k[s][0], r.k[s][1])) * scale_log2;
  }
  if (tail) {
#pragma unroll
    for (int s = 0; s < SPB; ++s) {
      const bool valid = tok0 + tl + TPS * s < ctx;
#pragma unroll
      for (int h = 0; h < G; ++h) x[s][h] = valid ? x[s][h] : kNegInf;
    }
  }

  // Raise the running max only when a score passes it by the slack.
  bool grow = false;
#pragma unroll
  for (int s = 0; s < SPB; ++s)
#pragma unroll
    for (int h = 0; h < G; ++h) grow |= x[s][h] > st.m[h] + kRescaleSlack;
  if (__any(grow)) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = x[0][h];
#pragma unroll
      for (int s = 1; s < SPB; ++s) bm = fmaxf(bm, x[s][h]);
#pragma unroll
      for (int off = LPT; off < 64; off <<= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
      const float mn = fmaxf(st.m[h], bm);
      const float alpha = fast_exp2(st.m[h] - mn);
      st.l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < D / 64; ++e) st.acc[h][e] *= alpha;
      st.m[h] = mn;
    }
  }

  // Weights as fp16 pairs of tokens (tl + 2j*TPS, tl + (2j+1)*TPS); l sums
  // exactly the rounded weights that P.V uses.
  uint32_t pp[SPB / 2][G];
#pragma unroll
  for (int j = 0; j < SPB / 2; ++j)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      pp[j][h] = pack_h2_rtz(fast_exp2(x[2 * j][h] - st.m[h]),
                             fast_exp2(x[2 * j + 1][h] - st.m[h]));
      st.l[h] = dot2(pp[j][h], kOnesH2, st.l[h]);
    }
  // Pair index pi = j*TPS + tl; one writer lane per group.
  if (c == 0) {
#pragma unroll
    for (int j = 0; j < SPB / 2; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) p_lds[(j * TPS + tl) * GP + h] = pp[j][h];
  }
  wave_fence();
}

// Second half: P.V from the V registers and the weights in LDS.  Rows of
// positions >= ctx are zeroed first (select), so stale slots never leak;
// vnew, when not null, is the V row appended for position ctx - 1 (LDS).
template <int D, int G>
__device__ __forceinline__ void block_pv(KVRegs<D>& r, WaveState<D, G>& st, int tok0, int ctx,
                                         const uint32_t* __restrict__ p_lds,
                                         const uint16_t* vnew, int lane) {
  constexpr int TPS = KVRegs<D>::TPS;
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

  // P.V: pair pi holds tokens ta = pi%TPS + 2*TPS*(pi/TPS) and tb = ta + TPS.
#pragma unroll
  for (int pi = 0; pi < 8; ++pi) {
    const int ta = pi % TPS + 2 * TPS * (pi / TPS), tb = ta + TPS;
    uint32_t pr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) pr[h] = p_lds[pi * GP + h];
    if constexpr (D == 128) {
      pv_dword<G>(reinterpret_cast<float(&)[G][2]>(st.acc), pr, r.v[ta], r.v[tb]);
    } else {
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
  }
  wave_fence();
}


}  // namespace decode_block
}  // namespace pkv
