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
//   fetches all its block ids with one vector load and keeps two blocks
//   (16 KiB) in flight: at d = 128 block k+2 is loaded into block k's
//   registers in two halves (K once k's scores are done, V after its P.V),
//   at d = 256 one block is loaded ahead into a second buffer.
//
// Per block (16 tokens x d) and wave (decode_block.h):
//   Scores S^T = K Q^T on the matrix cores: K straight from the block as the
//     A operand, the G query rows from LDS as B; lane l gets head l % 16 for
//     4 tokens.
//   Online softmax, base 2: scores are scaled by scale*log2(e); each head's
//     running max m is only raised when a score exceeds it by more than 8
//     (then its accumulators are rescaled), so weights p = 2^(s-m) stay in
//     (0, 256] and the common case does no rescale.
//   P.V: at d = 128 on the matrix cores as well (P straight from the
//     scores' registers, V loaded in the B layout); at d = 256 as packed
//     fp16 dot products with the weights passed through a per-wave LDS
//     buffer.
//   Masking is by select: positions >= ctx get score -inf and their V rows
//   are zeroed before use, so stale or NaN-poisoned slots never leak.
// At the end the 4 waves' (m, l, acc) merge through LDS; a sequence with a
// single partition writes fp16 output directly, otherwise the partition
// writes (o / l, m, l) and the merge kernel combines partitions:
//   M = max_p m_p, w_p = l_p 2^(m_p - M), O = sum_p w_p o_p / sum_p w_p.
#include <algorithm>
#include <climits>

#include "decode_block.h"
#include "device_util.h"
#include "kernels.h"
#include "merge.h"

namespace pkv {

namespace {

using namespace decode_block;

constexpr int kWaves = 4;                 // waves per work-group
constexpr int kMaxBlocksPerWave = 64;     // one block id per lane
constexpr int kMaxPartitionBlocks = kWaves * kMaxBlocksPerWave;
constexpr int32_t kResidentGroups = 512;  // 256 CUs x 2 work-groups of 4 waves
constexpr int32_t kTargetItems = 1024;    // work-groups to aim for when contexts must be cut
constexpr int32_t kMinPartitionBlocks = 16;
constexpr float kLog2e = 1.4426950408889634f;

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
    const uint16_t* __restrict__ v_new, const int64_t* __restrict__ slot_mapping,
    int32_t num_tokens) {
  constexpr int GP = (G + 3) & ~3;
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

  if (APPEND && (int)blockIdx.z >= max_parts) {
    // the z slices past the partitions (dispatched last): prefill rows
    const int64_t nxy = (int64_t)gridDim.x * gridDim.y;
    decode_block::append_rows<D>(k_pool, v_pool, num_blocks, num_kv_heads, k_new, v_new,
                                 slot_mapping, gridDim.x, num_tokens,
                                 (blockIdx.z - max_parts) * nxy + blockIdx.y * gridDim.x + blockIdx.x,
                                 (gridDim.z - max_parts) * nxy, (int)threadIdx.x, 64 * kWaves);
    return;
  }
  const int i = blockIdx.x, g = blockIdx.y;
  const int part = max_parts - 1 - (int)blockIdx.z;  // highest partitions dispatch first
  const int num_q_heads = num_kv_heads * G;
  // the wave index is the same in all its lanes: say so, so that what derives
  // from it (block counts, buffer resources) stays in scalar registers
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Tile k of this wave as a buffer resource; past the wave's blocks an empty
  // one (the loads below are issued unconditionally and read nothing then).
  constexpr uint32_t kTileBytes = 16 * D * 2;
  auto k_tile = [&](int kk) {
    const bool valid = kk < nbw;
    return tile_rsrc(k_pool + tile_off(valid ? kk : 0), valid ? kTileBytes : 0u);
  };
  auto v_tile = [&](int kk) {
    const bool valid = kk < nbw;
    return tile_rsrc(v_pool + tile_off(valid ? kk : 0), valid ? kTileBytes : 0u);
  };

  KVRegs<D> A, B;
  if constexpr (kEarlyRefill) {
    load_k<D>(A, k_tile(0), lane);
    load_v<D>(A, v_tile(0), lane);
    load_k<D>(B, k_tile(1), lane);
    load_v<D>(B, v_tile(1), lane);
  } else if (nbw > 0) {
    const int64_t o = tile_off(0);
    load_k<D>(A, k_pool + o, lane);
    load_v<D>(A, v_pool + o, lane);
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
  wave_init(st);

  auto tok_of = [&](int kk) { return (b0 + wave + kWaves * kk) * 16; };
  if constexpr (kEarlyRefill) {
    // Blocks k (in A) and k+1 (in B) per trip, buffer roles fixed so both
    // stay in registers; block k+2 goes into A (K after the scores, V after
    // P.V), k+3 into B, through buffer resources that are empty past the
    // wave's blocks; an odd last block (in A) after the loop.  The trip has
    // no branch around a load and no exit in its middle: with either, the
    // compiler merges buffer registers or sinks loads into one path, and
    // the wait counts it then assumes at the top of the loop drain the
    // prefetch.
    int k = 0;
    for (; k + 1 < nbw; k += 2) {
      const auto ka = k_tile(k + 2), va = v_tile(k + 2);
      const auto kb = k_tile(k + 3), vb = v_tile(k + 3);
      block_scores<D, G>(A, s_q, st, tok_of(k), ctx, scale_log2, s_p[wave], knew, lane);
      __builtin_amdgcn_sched_barrier(0);
      load_k<D>(A, ka, lane);
      block_pv<D, G>(A, st, tok_of(k), ctx, s_p[wave], vnew, lane);
      __builtin_amdgcn_sched_barrier(0);
      load_v<D>(A, va, lane);
      block_scores<D, G>(B, s_q, st, tok_of(k + 1), ctx, scale_log2, s_p[wave], knew, lane);
      __builtin_amdgcn_sched_barrier(0);
      load_k<D>(B, kb, lane);
      block_pv<D, G>(B, st, tok_of(k + 1), ctx, s_p[wave], vnew, lane);
      __builtin_amdgcn_sched_barrier(0);
      load_v<D>(B, vb, lane);
    }
    if (k < nbw) {
      block_scores<D, G>(A, s_q, st, tok_of(k), ctx, scale_log2, s_p[wave], knew, lane);
      block_pv<D, G>(A, st, tok_of(k), ctx, s_p[wave], vnew, lane);
    }
  } else {
    // d = 256 (one block is 16 KiB): block k+1 goes into B before A is
    // computed, k+2 into A before B.
    for (int k = 0; k < nbw; k += 2) {
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

  // Each wave's per-head totals to LDS; then merge the 4 waves.
  wave_store<D, G>(st, s_acc[wave], s_m[wave], s_l[wave], lane);
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

// One work-group per (sequence, query head) with more than one partition.
template <int D>
__global__ __launch_bounds__(256) void lse_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const int32_t* __restrict__ context_lens, int32_t ctx_clamp, int32_t partition_blocks,
    int32_t max_parts, int32_t num_q_heads, uint16_t* __restrict__ out) {
  merge::lse_merge_row<D>(part_o, part_ml, context_lens, ctx_clamp, partition_blocks, max_parts,
                          num_q_heads, out, (int)blockIdx.x);
}

template <int D, int G, bool APPEND>
hipError_t launch_decode_dga(const void* q, void* k_pool, void* v_pool, int64_t num_blocks,
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
  hipLaunchKernelGGL((paged_decode_kernel<D, G, APPEND>),
                     dim3(num_decode_seqs, num_kv_heads, plan.max_parts + app_z), dim3(64 * kWaves), 0,
                     stream, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(k_pool),
                     static_cast<uint16_t*>(v_pool), num_blocks, num_kv_heads, block_tables,
                     max_blocks_per_seq, context_lens, ctx_clamp, plan.partition_blocks,
                     plan.max_parts, scale * kLog2e, static_cast<uint16_t*>(out), part_o,
                     part_ml, static_cast<const uint16_t*>(app.k_new),
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
hipError_t launch_decode_d(int32_t group, const void* q, void* k_pool, void* v_pool,
                           int64_t num_blocks, int32_t num_kv_heads, const int32_t* bt,
                           int32_t maxblk, const int32_t* ctx, int32_t nseq, float scale,
                           const DecodePlan& plan, const DecodeAppend& app, void* out, void* ws,
                           hipStream_t stream, DecodeMerge* defer) {
  const bool fused = app.k_new != nullptr;
#define PKV_CASE(GG)                                                                         \
  case GG:                                                                                  \
    return fused ? launch_decode_dga<D, GG, true>(q, k_pool, v_pool, num_blocks,            \
                                                  num_kv_heads, bt, maxblk, ctx, nseq,      \
                                                  scale, plan, app, out, ws, stream, defer) \
                 : launch_decode_dga<D, GG, false>(q, k_pool, v_pool, num_blocks,           \
                                                   num_kv_heads, bt, maxblk, ctx, nseq,     \
                                                   scale, plan, app, out, ws, stream, defer);
  switch (group) {
    PKV_CASE(1) PKV_CASE(2) PKV_CASE(3) PKV_CASE(4)
    PKV_CASE(5) PKV_CASE(6) PKV_CASE(7) PKV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef PKV_CASE
}

}  // namespace

hipError_t launch_decode_merge(const float* part_o, const float* part_ml,
                               const int32_t* context_lens, int32_t ctx_clamp,
                               const DecodePlan& plan, int32_t num_decode_seqs,
                               int32_t num_q_heads, int32_t head_dim, void* out,
                               hipStream_t stream) {
  const int32_t rows = num_decode_seqs * num_q_heads;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  if (head_dim == 128)
    hipLaunchKernelGGL((lse_merge_kernel<128>), dim3(rows), dim3(256), 0, stream, part_o,
                       part_ml, context_lens, ctx_clamp, plan.partition_blocks, plan.max_parts,
                       num_q_heads, static_cast<uint16_t*>(out));
  else if (head_dim == 256)
    hipLaunchKernelGGL((lse_merge_kernel<256>), dim3(rows), dim3(256), 0, stream, part_o,
                       part_ml, context_lens, ctx_clamp, plan.partition_blocks, plan.max_parts,
                       num_q_heads, static_cast<uint16_t*>(out));
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

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
                               void* workspace, hipStream_t stream, DecodeMerge* defer) {
  if (num_decode_seqs == 0) return hipSuccess;
  const int32_t group = num_q_heads / num_kv_heads;
  if (head_dim == 128)
    return launch_decode_d<128>(group, q, k_pool, v_pool, num_blocks, num_kv_heads,
                                block_tables, max_blocks_per_seq, context_lens, num_decode_seqs,
                                scale, plan, app, out, workspace, stream, defer);
  if (head_dim == 256)
    return launch_decode_d<256>(group, q, k_pool, v_pool, num_blocks, num_kv_heads,
                                block_tables, max_blocks_per_seq, context_lens, num_decode_seqs,
                                scale, plan, app, out, workspace, stream, defer);
  return hipErrorInvalidValue;
}

}  // namespace pkv
