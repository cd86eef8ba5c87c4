// decode.hip -- paged decode attention with split-KV partitions, and the
// log-sum-exp merge of partitions.
//
// Each decode sequence attends its one new query token over its whole
// context, read through its block table (deepconcepts.dev, "Continuous
// Batching Is Not a Bigger Batch": the batch is re-formed every pass and
// its cache is allocated in fixed 16-token blocks; danielfleming.xyz,
// "Static batching", section "Ragged batches": a paged layout stores only
// real tokens, so a ragged mix does not pay for its widest member).
//
// Work decomposition (gfx950, wave64):
//   grid = (sequence, KV head, partition of the context); a work-group of 4
//   waves reads the partition's blocks of ONE KV head once and applies them
//   to all G query heads of that group (grouped-query attention), so every
//   K/V byte leaves HBM once per step.  Work-groups are dispatched highest
//   partition first: only long contexts have high partitions, so the
//   longest work starts first and short sequences fill the gaps behind it
//   (longest-first list scheduling by the hardware dispatcher).
//   Blocks of a partition are dealt round-robin to its waves; each wave
//   fetches all its block ids with one vector load and keeps about 16 KiB of
//   K/V in flight: at d = 128 block f+8 is loaded into block f's registers
//   in two halves (K once f's scores are done, V after f's P.V), at d = 256
//   one block (16 KiB) is loaded ahead into a second buffer.
//
// Per block (16 tokens x d) and wave:
//   K layout: D/16 lanes share one token row, each lane holding 16 of its
//     d values (two 16-byte chunks), so a K load instruction reads whole
//     128-byte runs of rows.  q.k is 8 packed fp16 dot products
//     (v_dot2_f32_f16, fp32 accumulate) per head with the query fragments
//     read from LDS, then a DPP butterfly inside the lane group.
//   Online softmax, base 2: scores are scaled by scale*log2(e); the running
//     max m is wave-uniform and only raised when a score exceeds it by more
//     than 8 (then the accumulators are rescaled), so weights p = 2^(s-m)
//     stay in (0, 256] and the common case does no rescale.
//   V layout: every lane owns d/64 output elements of all 16 tokens, so the
//     P.V accumulation needs no cross-lane reduction.  The weights travel
//     from the K layout to all lanes through a small per-wave LDS buffer as
//     fp16 pairs of tokens (the two tokens a lane group scores in
//     consecutive K steps), and P.V is again v_dot2_f32_f16 over those pairs.
//   Masking is by select: positions >= ctx get score -inf and their V rows
//   are zeroed before use, so stale or NaN-poisoned slots never leak.
// At the end the 4 waves' (m, l, acc) merge through LDS; a sequence with a
// single partition writes fp16 output directly, otherwise the partition
// writes (o / l, m, l) and the merge kernel combines partitions:
//   M = max_p m_p, w_p = l_p 2^(m_p - M), O = sum_p w_p o_p / sum_p w_p.
#include <algorithm>
#include <climits>

#include "device_util.h"
#include "kernels.h"

namespace pkv {

namespace {

constexpr int kWaves = 4;                 // waves per work-group
constexpr int kMaxBlocksPerWave = 64;     // one block id per lane
constexpr int kMaxPartitionBlocks = kWaves * kMaxBlocksPerWave;
constexpr int32_t kResidentGroups = 512;  // 256 CUs x 2 work-groups of 4 waves
constexpr int32_t kTargetItems = 1024;    // work-groups to aim for when contexts must be cut
constexpr int32_t kMinPartitionBlocks = 16;
constexpr float kRescaleSlack = 8.f;      // lazy max: rescale only past m + 8 (base 2)
constexpr float kLog2e = 1.4426950408889634f;

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


// APPEND: the step's decode tokens are appended by this kernel (fused
// append): k_new / v_new row i (one token of sequence i, [Hkv][D]) belongs
// at position ctx_i - 1.  The work-group whose partition holds that position
// stages the row in LDS, uses it in place of the pool's old row when
// slot_mapping[i] is the table's slot of ctx_i - 1, and writes it to
// slot_mapping[i] at the end (nothing when the slot is negative or beyond
// the pool), so the result equals an append followed by the attention.
template <int D, int G, bool APPEND>
__global__ __launch_bounds__(64 * kWaves) void paged_decode_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ k_pool,
    uint16_t* __restrict__ v_pool, int64_t num_blocks, int32_t num_kv_heads,
    const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, int32_t ctx_clamp, int32_t partition_blocks,
    int32_t max_parts, float scale_log2, uint16_t* __restrict__ out, float* __restrict__ part_o,
    float* __restrict__ part_ml, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const int64_t* __restrict__ slot_mapping) {
  constexpr int LPT = D / 16, EPL = D / 64, GP = (G + 3) & ~3;
  // d = 128: two blocks (16 KiB) in flight per wave by refilling a buffer as
  // soon as each half is consumed; d = 256: one block is already 16 KiB, and
  // the plain two-buffer scheme keeps registers under 256 (2 waves per SIMD).
  constexpr bool kEarlyRefill = D == 128;
  constexpr int RCH = D / 8;  // 16-byte chunks of one appended row
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ uint32_t s_p[kWaves][8 * GP];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_new[APPEND ? 2 * D : 8];  // K row, V row

  const int i = blockIdx.x, g = blockIdx.y;
  const int part = max_parts - 1 - (int)blockIdx.z;  // highest partitions dispatch first
  const int num_q_heads = num_kv_heads * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b0 = part * partition_blocks;
  const int32_t* bt_row = block_tables + (int64_t)i * max_blocks_per_seq;

  // Everything that does not depend on the context length is requested
  // first, so that the length, the block ids, the query rows and the
  // appended rows arrive together: block ids of this wave's blocks
  // b0 + wave + kWaves*k (one per lane, k < the partition's share; entries
  // past the context are never used) ...
  uint32_t raw_bid = 0;
  {
    const int e = b0 + wave + kWaves * lane;
    if (wave + kWaves * lane < partition_blocks && e < max_blocks_per_seq)
      raw_bid = (uint32_t)bt_row[e];
  }
  // ... the query rows of the G heads (to LDS after the first K/V loads) ...
  const uint4* qsrc =
      reinterpret_cast<const uint4*>(q + ((int64_t)i * num_q_heads + (int64_t)g * G) * D);
  constexpr int QCH = G * D / 8;
  uint4 qstage[(QCH + 255) / 256];
#pragma unroll
  for (int k = 0; k < (QCH + 255) / 256; ++k)
    if (tid + 256 * k < QCH) qstage[k] = qsrc[tid + 256 * k];
  // ... and the appended rows with their slot.
  uint4 nstage{};
  int64_t slot = -1;
  if constexpr (APPEND) {
    slot = slot_mapping[i];
    const int64_t row = ((int64_t)i * num_kv_heads + g) * D;
    if (tid < RCH)
      nstage = reinterpret_cast<const uint4*>(k_new + row)[tid];
    else if (tid >= 64 && tid < 64 + RCH)
      nstage = reinterpret_cast<const uint4*>(v_new + row)[tid - 64];
  }

  // A length beyond the table row or the planned partitions breaks the
  // caller contract; clamp so that it can only give wrong numbers.
  const int ctx = min(context_lens[i], ctx_clamp);
  const int nblk = (ctx + 15) >> 4;
  if (ctx <= 0 || b0 >= nblk) return;  // uniform over the work-group
  const int b1 = min(b0 + partition_blocks, nblk);
  const int nparts = (nblk + partition_blocks - 1) / partition_blocks;

  // Block ids clamped into the pool.
  const int nbw = (b1 - b0 - wave + kWaves - 1) / kWaves;
  const int my_bid =
      lane < nbw ? (int)(raw_bid < (uint64_t)num_blocks ? raw_bid : (uint32_t)(num_blocks - 1))
                 : 0;
  const int64_t tile_elems = (int64_t)16 * D;
  const int64_t head_off = (int64_t)g * tile_elems;
  const int64_t block_stride = (int64_t)num_kv_heads * tile_elems;
  auto tile_off = [&](int k) -> int64_t {
    return (int64_t)__builtin_amdgcn_readlane(my_bid, k) * block_stride + head_off;
  };

  KVRegs<D> A, B;
  if (nbw > 0) {
    const int64_t o = tile_off(0);
    load_k<D>(A, k_pool + o, lane);
    load_v<D>(A, v_pool + o, lane);
  }
  if (kEarlyRefill && nbw > 1) {
    const int64_t o = tile_off(1);
    load_k<D>(B, k_pool + o, lane);
    load_v<D>(B, v_pool + o, lane);
  }
#pragma unroll
  for (int k = 0; k < (QCH + 255) / 256; ++k)
    if (tid + 256 * k < QCH) reinterpret_cast<uint4*>(s_q)[tid + 256 * k] = qstage[k];
  if constexpr (APPEND) {
    if (tid < RCH)
      reinterpret_cast<uint4*>(s_new)[tid] = nstage;
    else if (tid >= 64 && tid < 64 + RCH)
      reinterpret_cast<uint4*>(s_new + D)[tid - 64] = nstage;
  }
  __syncthreads();

  // The appended token sits in block nblk - 1; this partition holds it when
  // nblk <= b1, and the wave that reads that block substitutes the rows.
  const bool owner = APPEND && nblk <= b1;
  const uint16_t* knew = nullptr;
  const uint16_t* vnew = nullptr;
  if constexpr (APPEND) {
    const int kl = nblk - 1 - b0 - wave;  // multiple of kWaves when this wave reads it
    if (owner && kl >= 0 && kl % kWaves == 0 && slot >= 0) {
      const uint32_t raw_last = (uint32_t)__builtin_amdgcn_readlane((int)raw_bid, kl / kWaves);
      if (raw_last < (uint64_t)num_blocks &&
          slot == (int64_t)raw_last * 16 + ((ctx - 1) & 15)) {
        knew = s_new;
        vnew = s_new + D;
      }
    }
  }

  WaveState<D, G> st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    st.m[h] = -__builtin_huge_valf();
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.acc[h][e] = 0.f;
  }

  // Blocks k (in A) and k+1 (in B) per trip, buffer roles fixed so both stay
  // in registers.
  auto tok_of = [&](int kk) { return (b0 + wave + kWaves * kk) * 16; };
  for (int k = 0; k < nbw; k += 2) {
    if constexpr (kEarlyRefill) {
      // block k+2 goes into A (K after the scores, V after P.V), k+3 into B
      const int64_t oa = k + 2 < nbw ? tile_off(k + 2) : 0;
      block_scores<D, G>(A, s_q, st, tok_of(k), ctx, scale_log2, s_p[wave], knew, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 2 < nbw) load_k<D>(A, k_pool + oa, lane);
      block_pv<D, G>(A, st, tok_of(k), ctx, s_p[wave], vnew, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 2 < nbw) load_v<D>(A, v_pool + oa, lane);
      if (k + 1 >= nbw) break;
      const int64_t ob = k + 3 < nbw ? tile_off(k + 3) : 0;
      block_scores<D, G>(B, s_q, st, tok_of(k + 1), ctx, scale_log2, s_p[wave], knew, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 3 < nbw) load_k<D>(B, k_pool + ob, lane);
      block_pv<D, G>(B, st, tok_of(k + 1), ctx, s_p[wave], vnew, lane);
      __builtin_amdgcn_sched_barrier(0);
      if (k + 3 < nbw) load_v<D>(B, v_pool + ob, lane);
    } else {
      // block k+1 goes into B before A is computed, k+2 into A before B
      if (k + 1 < nbw) {
        const int64_t o = tile_off(k + 1);
        load_k<D>(B, k_pool + o, lane);
        load_v<D>(B, v_pool + o, lane);
      }
      block_scores<D, G>(A, s_q, st, tok_of(k), ctx, scale_log2, s_p[wave], knew, lane);
      block_pv<D, G>(A, st, tok_of(k), ctx, s_p[wave], vnew, lane);
      if (k + 1 >= nbw) break;
      if (k + 2 < nbw) {
        const int64_t o = tile_off(k + 2);
        load_k<D>(A, k_pool + o, lane);
        load_v<D>(A, v_pool + o, lane);
      }
      block_scores<D, G>(B, s_q, st, tok_of(k + 1), ctx, scale_log2, s_p[wave], knew, lane);
      block_pv<D, G>(B, st, tok_of(k + 1), ctx, s_p[wave], vnew, lane);
    }
  }

  // Lane groups' weight sums -> wave totals; then merge the 4 waves.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float lw = st.l[h];
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) lw += __shfl_xor(lw, off);
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[wave][h][EPL * lane + e] = st.acc[h][e];
    if (lane == 0) {
      s_m[wave][h] = st.m[h];
      s_l[wave][h] = lw;
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

  // The appended rows go to their slot (only this work-group reads the
  // block that holds them, and it is done with it).
  if constexpr (APPEND) {
    if (owner && slot >= 0 && (slot >> 4) < num_blocks) {
      const int64_t dst = (((slot >> 4) * num_kv_heads + g) * 16 + (slot & 15)) * D;
      if (tid < RCH)
        reinterpret_cast<uint4*>(k_pool + dst)[tid] = reinterpret_cast<const uint4*>(s_new)[tid];
      else if (tid >= 64 && tid < 64 + RCH)
        reinterpret_cast<uint4*>(v_pool + dst)[tid - 64] =
            reinterpret_cast<const uint4*>(s_new + D)[tid - 64];
    }
  }
}

// One work-group per (sequence, query head) with more than one partition:
// the 4 waves take every 4th partition, then combine through LDS.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ context_lens, int32_t ctx_clamp, int32_t partition_blocks,
    int32_t max_parts, int32_t num_q_heads, uint16_t* __restrict__ out) {
  constexpr int EPL = D / 64;
  __shared__ float s_max[4];
  __shared__ float s_w[4];
  __shared__ float s_acc[4][D];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row_head = blockIdx.x;
  const int i = row_head / num_q_heads;
  const int nblk = (min(context_lens[i], ctx_clamp) + 15) >> 4;
  const int np = (nblk + partition_blocks - 1) / partition_blocks;
  if (np <= 1) return;  // written directly by the decode kernel
  const float* ml = part_ml + (int64_t)row_head * max_parts * 2;
  const float* po = part_o + (int64_t)row_head * max_parts * D + EPL * lane;

  float M = -__builtin_huge_valf();
  for (int p = tid; p < np; p += 256) M = fmaxf(M, ml[2 * p]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) s_max[wave] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));

  float W = 0.f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll 4
  for (int p = wave; p < np; p += 4) {
    const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
    W += w;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += w * po[(int64_t)p * D + e];
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) s_acc[wave][EPL * lane + e] = acc[e];
  if (lane == 0) s_w[wave] = W;
  __syncthreads();
  if (tid < D) {
    const float total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
    const float o = s_acc[0][tid] + s_acc[1][tid] + s_acc[2][tid] + s_acc[3][tid];
    out[(int64_t)row_head * D + tid] = __builtin_bit_cast(uint16_t, (f16)(o / total));
  }
}

template <int D, int G, bool APPEND>
hipError_t launch_decode_dga(const void* q, void* k_pool, void* v_pool, int64_t num_blocks,
                             int32_t num_kv_heads, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t num_decode_seqs, float scale, const DecodePlan& plan,
                             const DecodeAppend& app, void* out, void* workspace,
                             hipStream_t stream) {
  const int32_t num_q_heads = num_kv_heads * G;
  const int64_t clamp64 = std::min<int64_t>((int64_t)max_blocks_per_seq * 16,
                                            (int64_t)plan.max_parts * plan.partition_blocks * 16);
  const int32_t ctx_clamp = (int32_t)std::min<int64_t>(clamp64, INT32_MAX);
  float* part_o = static_cast<float*>(workspace);
  float* part_ml =
      part_o ? part_o + (size_t)num_decode_seqs * num_q_heads * plan.max_parts * D : nullptr;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  hipLaunchKernelGGL((paged_decode_kernel<D, G, APPEND>),
                     dim3(num_decode_seqs, num_kv_heads, plan.max_parts), dim3(64 * kWaves), 0,
                     stream, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(k_pool),
                     static_cast<uint16_t*>(v_pool), num_blocks, num_kv_heads, block_tables,
                     max_blocks_per_seq, context_lens, ctx_clamp, plan.partition_blocks,
                     plan.max_parts, scale * kLog2e, static_cast<uint16_t*>(out), part_o,
                     part_ml, static_cast<const uint16_t*>(app.k_new),
                     static_cast<const uint16_t*>(app.v_new), app.slot_mapping);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.max_parts <= 1) return err;
  const int32_t rows = num_decode_seqs * num_q_heads;
  hipLaunchKernelGGL((lse_merge_kernel<D>), dim3(rows), dim3(256), 0, stream, part_o, part_ml,
                     context_lens, ctx_clamp, plan.partition_blocks, plan.max_parts, num_q_heads,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(int32_t group, const void* q, void* k_pool, void* v_pool,
                           int64_t num_blocks, int32_t num_kv_heads, const int32_t* bt,
                           int32_t maxblk, const int32_t* ctx, int32_t nseq, float scale,
                           const DecodePlan& plan, const DecodeAppend& app, void* out, void* ws,
                           hipStream_t stream) {
  const bool fused = app.k_new != nullptr;
#define PKV_CASE(GG)                                                                         \
  case GG:                                                                                  \
    return fused ? launch_decode_dga<D, GG, true>(q, k_pool, v_pool, num_blocks,            \
                                                  num_kv_heads, bt, maxblk, ctx, nseq,      \
                                                  scale, plan, app, out, ws, stream)        \
                 : launch_decode_dga<D, GG, false>(q, k_pool, v_pool, num_blocks,           \
                                                   num_kv_heads, bt, maxblk, ctx, nseq,     \
                                                   scale, plan, app, out, ws, stream);
  switch (group) {
    PKV_CASE(1) PKV_CASE(2) PKV_CASE(3) PKV_CASE(4)
    PKV_CASE(5) PKV_CASE(6) PKV_CASE(7) PKV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef PKV_CASE
}

}  // namespace

DecodePlan plan_decode(int32_t num_decode_seqs, int32_t num_kv_heads, int32_t num_q_heads,
                       int32_t head_dim, int32_t max_context_len, int32_t kv_partition_tokens) {
  DecodePlan plan{};
  const int32_t max_blocks = (max_context_len + 15) / 16;
  const int32_t units = num_decode_seqs * num_kv_heads > 0 ? num_decode_seqs * num_kv_heads : 1;
  int32_t pb;
  if (kv_partition_tokens > 0) {
    pb = kv_partition_tokens / 16;
  } else if (units >= kResidentGroups && max_blocks <= kMaxPartitionBlocks) {
    pb = max_blocks;  // enough (sequence, KV head) pairs to fill the GPU: no split, no merge
  } else {
    // cut the longest context so that there are about kTargetItems work-groups
    // if every context were that long; shorter ones get fewer partitions
    const int32_t splits = (kTargetItems + units - 1) / units;
    pb = std::max((max_blocks + splits - 1) / splits, kMinPartitionBlocks);
  }
  pb = (pb + kWaves - 1) / kWaves * kWaves;
  if (pb > kMaxPartitionBlocks) pb = kMaxPartitionBlocks;
  if (pb < kWaves) pb = kWaves;
  plan.partition_blocks = pb;
  plan.max_parts = max_blocks > 0 ? (max_blocks + pb - 1) / pb : 1;
  plan.partial_bytes = plan.max_parts > 1 ? (size_t)num_decode_seqs * num_q_heads *
                                                plan.max_parts * (head_dim + 2) * sizeof(float)
                                          : 0;
  return plan;
}

hipError_t launch_paged_decode(const void* q, void* k_pool, void* v_pool, int64_t num_blocks,
                               int32_t num_kv_heads, int32_t num_q_heads, int32_t head_dim,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_decode_seqs, float scale,
                               const DecodePlan& plan, const DecodeAppend& app, void* out,
                               void* workspace, hipStream_t stream) {
  if (num_decode_seqs == 0) return hipSuccess;
  const int32_t group = num_q_heads / num_kv_heads;
  if (head_dim == 128)
    return launch_decode_d<128>(group, q, k_pool, v_pool, num_blocks, num_kv_heads,
                                block_tables, max_blocks_per_seq, context_lens, num_decode_seqs,
                                scale, plan, app, out, workspace, stream);
  if (head_dim == 256)
    return launch_decode_d<256>(group, q, k_pool, v_pool, num_blocks, num_kv_heads,
                                block_tables, max_blocks_per_seq, context_lens, num_decode_seqs,
                                scale, plan, app, out, workspace, stream);
  return hipErrorInvalidValue;
}

}  // namespace pkv
