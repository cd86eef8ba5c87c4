// merge.h -- the log-sum-exp merges of split attention, as device functions
// of one work-group (or one wave), shared by the merge kernels of the decode
// partitions (decode.hip), of the balanced schedule's pieces
// (decode_sched.hip) and of the prefill splits (prefill.hip), and by the
// step's combined merge (prefill.hip), which runs the decode part's merge
// and the prefill chunks' in one launch.
#pragma once

#include "device_util.h"
#include "sched_layout.h"

namespace pkv {
namespace merge {

using sched::sched_um_offset;

constexpr int64_t kMaxPrefillSplits = 16;  // splits of a prefill row: one lane each

// Merge of the partitions of one (sequence, query head) row, one 256-thread
// work-group (rows with a single partition return at once):
//   M = max_p m_p,  w_p = l_p 2^(m_p - M),  O = sum_p w_p o_p / sum_p w_p.
// The merge sits between two kernels on the step's critical path, so its
// memory round trips are what it costs: the context length and the (m, l)
// pairs are requested together (thread p holds pair p; pairs past the
// sequence's partition count are stale and selected away), and the first
// kMergeUnroll partitions of each wave's o vectors (wave w takes every 4th
// partition from w) are in flight while M is reduced.
constexpr int kMergeUnroll = 4;

template <int D>
__device__ __forceinline__ void lse_merge_row(const float* __restrict__ part_o,
                                              const float* __restrict__ part_ml,
                                              const int32_t* __restrict__ context_lens,
                                              int32_t ctx_clamp, int32_t partition_blocks,
                                              int32_t max_parts, int32_t num_q_heads,
                                              uint16_t* __restrict__ out, int row_head) {
  constexpr int EPL = D / 64;
  constexpr int kStride = 4 * kMergeUnroll;  // partitions per round of the 4 waves
  __shared__ float s_max[4];
  __shared__ float s_w[256];
  __shared__ float s_wsum[4];
  __shared__ float s_acc[4][D];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int i = row_head / num_q_heads;
  const float* ml = part_ml + (int64_t)row_head * max_parts * 2;
  const float* po = part_o + (int64_t)row_head * max_parts * D + EPL * lane;
  const int ctx = context_lens[i];
  float2 own = {-__builtin_huge_valf(), 0.f};
  if (tid < max_parts) own = *reinterpret_cast<const float2*>(ml + 2 * tid);
  const int nblk = (min(ctx, ctx_clamp) + 15) >> 4;
  const int np = (nblk + partition_blocks - 1) / partition_blocks;
  if (np <= 1) return;  // written directly by the decode kernel

  // Every partition p < np holds at least one position: m_p is finite,
  // l_p > 0, o_p written.  Loads of p >= np re-read partition np - 1.
  float v[kMergeUnroll][EPL];
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const int pc = min(wave + 4 * u, np - 1);
#pragma unroll
    for (int e = 0; e < EPL; ++e) v[u][e] = po[(int64_t)pc * D + e];
  }

  float M = tid < np ? own.x : -__builtin_huge_valf();
  for (int p = tid + 256; p < np; p += 256) M = fmaxf(M, ml[2 * p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_max[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  s_w[tid] = tid < np ? own.y * fast_exp2(own.x - M) : 0.f;
  __syncthreads();
  auto weight = [&](int p) -> float {
    if (p >= np) return 0.f;
    if (p < 256) return s_w[p];
    return ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
  };

  float W = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int u = 0; u < kMergeUnroll; ++u) {
    const float w = weight(wave + 4 * u);
    W += w;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += w * v[u][e];
  }
  // more partitions than one round holds (long contexts)
  for (int p0 = wave + kStride; p0 < np; p0 += kStride) {
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int pc = min(p0 + 4 * u, np - 1);
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[u][e] = po[(int64_t)pc * D + e];
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const float w = weight(p0 + 4 * u);
      W += w;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += w * v[u][e];
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[wave][EPL * lane + e] = acc[e];
  if (lane == 0) s_wsum[wave] = W;
  __syncthreads();
  if (tid < D) {
    const float total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    const float o = s_acc[0][tid] + s_acc[1][tid] + s_acc[2][tid] + s_acc[3][tid];
    out[(int64_t)row_head * D + tid] = __builtin_bit_cast(uint16_t, (f16)(o / total));
  }
}

// Merge of the pieces of a split unit: one 4-wave work-group per (unit, query
// head of its group); pieces w = wf .. wf + np - 1 at slots u + w (work-groups
// with an empty cost range hold none).  Each wave merges its pieces in one
// pass (running log-sum-exp), then the 4 waves combine through LDS.
template <int D>
__device__ __forceinline__ void piece_merge_unit(const int32_t* __restrict__ sched, int32_t U,
                                                 int32_t nwg, int32_t num_kv_heads, int32_t G,
                                                 const float* __restrict__ part_o,
                                                 const float* __restrict__ part_ml,
                                                 uint16_t* __restrict__ out, int32_t u,
                                                 int32_t h) {
  constexpr int EPL = D / 64;
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[4][D];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (u >= U) return;
  const int32_t W = sched[0];
  const int2 um = reinterpret_cast<const int2*>(sched + sched_um_offset(U, nwg))[u];
  const int32_t wf = max(0, min(nwg - 1, um.x));
  const int32_t np = min(um.y, nwg - wf);
  if (np <= 1 || W <= 0) return;  // whole: written by the decode kernel
  float M = -__builtin_huge_valf(), L = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int p = wave; p < np; p += 4) {
    const int32_t ww = wf + p;
    if ((int64_t)(ww + 1) * W / nwg <= (int64_t)ww * W / nwg) continue;  // empty range
    const int64_t pidx = ((int64_t)u + ww) * G + h;
    const float mp = part_ml[pidx * 2], lp = part_ml[pidx * 2 + 1];
    float op[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) op[e] = part_o[pidx * D + EPL * lane + e];
    if (!(lp > 0.f)) continue;
    const float Mn = fmaxf(M, mp);
    const float a = fast_exp2(M - Mn), b = lp * fast_exp2(mp - Mn);
    L = L * a + b;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * a + b * op[e];
    M = Mn;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[wave][EPL * lane + e] = acc[e];
  if (lane == 0) {
    s_m[wave] = M;
    s_l[wave] = L;
  }
  __syncthreads();
  if (tid < D) {
    const float Mt = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float Lt = 0.f, o = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      if (s_l[ww] > 0.f) {
        const float a = fast_exp2(s_m[ww] - Mt);
        Lt += a * s_l[ww];
        o += a * s_acc[ww][tid];
      }
    }
    const int i = u / num_kv_heads, g = u - i * num_kv_heads;
    const int64_t row_head = (int64_t)i * num_kv_heads * G + g * G + h;
    out[row_head * D + tid] = __builtin_bit_cast(uint16_t, (f16)(o / Lt));
  }
}

// Merge of the splits of one (prefill row, query head) rh: one wave.
//   M = max m_s over splits with l_s > 0, w_s = l_s 2^(m_s - M),
//   O = sum_s w_s o_s / sum_s w_s.
// Lane s holds split s's (m, l), so the weights take one round of loads and
// two wave reductions; every split's o is then requested at once (a split
// that saw no position -- l = 0 -- may have left o unwritten: its value is
// read but selected away, never multiplied).
template <int D>
__device__ __forceinline__ void chunk_merge_row_head(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ query_start_loc, int32_t first_seq, int32_t num_seqs,
    int32_t num_q_heads, int32_t num_splits, int64_t max_row_heads, uint16_t* __restrict__ out,
    int64_t rh) {
  constexpr int EPL = D / 64;
  static_assert(kMaxPrefillSplits <= 64, "one lane per split");
  const int lane = threadIdx.x & 63;
  const int64_t first_row = query_start_loc[first_seq];
  const int64_t rows = (int64_t)query_start_loc[num_seqs] - first_row;
  if (rh >= rows * num_q_heads || rh >= max_row_heads) return;
  const float* ml = part_ml + rh * num_splits * 2;
  float m = -__builtin_huge_valf(), l = 0.f;
  if (lane < num_splits) {
    m = ml[2 * lane];
    l = ml[2 * lane + 1];
  }
  // Every split's o is requested before the weights are known (one memory
  // round trip, not two); loads of splits past num_splits re-read the last
  // one (in bounds) and get weight 0.
  const float* src = part_o + rh * num_splits * D + EPL * lane;
  float o[kMaxPrefillSplits][EPL];
#pragma unroll
  for (int s = 0; s < kMaxPrefillSplits; ++s) {
    const int sc = min(s, num_splits - 1);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[s][e] = src[(int64_t)sc * D + e];
  }
  float M = l > 0.f ? m : -__builtin_huge_valf();
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float w = l > 0.f ? l * fast_exp2(m - M) : 0.f;
  float W = w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) W += __shfl_xor(W, off);
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxPrefillSplits; ++s) {
    const float ws = s < num_splits ? __shfl(w, s) : 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += ws > 0.f ? ws * o[s][e] : 0.f;
  }
  uint16_t* dst = out + (first_row * num_q_heads + rh) * D + EPL * lane;
  const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) dst[e] = __builtin_bit_cast(uint16_t, (f16)(acc[e] * inv));
}

}  // namespace merge
}  // namespace pkv
