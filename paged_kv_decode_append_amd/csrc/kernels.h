// kernels.h -- host-side launchers of the HIP kernels, called by the C ABI
// in api.hip.  Each returns hipSuccess or the launch error.  Arguments are
// validated by the caller.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Keeps a HIP error for pkv_last_hip_error on this thread (api.hip).
void record_hip_error(hipError_t e);

hipError_t launch_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               int32_t num_seqs, int32_t num_tokens, int64_t* slot_mapping,
                               hipStream_t stream);

hipError_t launch_kv_append(void* k_pool, void* v_pool, int64_t num_blocks,
                            int32_t num_kv_heads, int32_t head_dim, const void* k_new,
                            const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                            hipStream_t stream);

// Split-KV plan of the decode part of a step, made from host hints only.
struct DecodePlan {
  int32_t partition_blocks;  // KV blocks per partition (multiple of the waves per group)
  int32_t max_parts;         // partitions of the longest context
  size_t partial_bytes;      // workspace for the partials (0 when no split)
};

DecodePlan plan_decode(int32_t num_decode_seqs, int32_t num_kv_heads, int32_t num_q_heads,
                       int32_t head_dim, int32_t max_context_len, int32_t kv_partition_tokens);

// The step's new rows to append inside the decode launch: row t of k_new /
// v_new [num_tokens][Hkv][d] goes to slot_mapping[t]; the decode rows
// (t < num_decode_seqs) by the work-group that attends that position, the
// prefill chunks' rows after them by extra work-groups.  All null (and
// num_tokens 0) for attention only.
struct DecodeAppend {
  const void* k_new;
  const void* v_new;
  const int64_t* slot_mapping;
  int32_t num_tokens;
};

// Work-groups a decode launch adds for appending `rows` prefill rows.
inline int32_t append_groups(int64_t rows) {
  return rows <= 0 ? 0 : (int32_t)std::min<int64_t>((rows + 7) / 8, 128);
}

// A decode launch's merge of its split attention left for the step's
// combined merge (launch_prefill with `fold`): the partition grid's partials
// (one work-group per (sequence, query head)) or the balanced schedule's
// pieces (one per (unit, query head)).
struct DecodeMerge {
  int32_t groups = 0;  // work-groups of the merge (0: none left)
  bool pieces = false;
  const float* part_o = nullptr;
  const float* part_ml = nullptr;
  // partition grid
  const int32_t* context_lens = nullptr;
  int32_t ctx_clamp = 0, partition_blocks = 0, max_parts = 0, num_q_heads = 0;
  // schedule pieces
  const int32_t* sched = nullptr;
  int32_t units = 0, sched_groups = 0, num_kv_heads = 0, group = 0;
};

// The merge of the partition grid's partials, as launch_decode_merge runs it.
inline DecodeMerge grid_merge(const float* part_o, const float* part_ml,
                              const int32_t* context_lens, int32_t ctx_clamp,
                              const DecodePlan& plan, int32_t num_decode_seqs,
                              int32_t num_q_heads) {
  DecodeMerge m;
  m.groups = num_decode_seqs * num_q_heads;
  m.part_o = part_o;
  m.part_ml = part_ml;
  m.context_lens = context_lens;
  m.ctx_clamp = ctx_clamp;
  m.partition_blocks = plan.partition_blocks;
  m.max_parts = plan.max_parts;
  m.num_q_heads = num_q_heads;
  return m;
}

// With `defer` set, a merge the launch needs is described there instead of
// launched (the decode launchers below).
hipError_t launch_paged_decode(const void* q, void* k_pool, void* v_pool, int64_t num_blocks,
                               int32_t num_kv_heads, int32_t num_q_heads, int32_t head_dim,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_decode_seqs, float scale,
                               const DecodePlan& plan, const DecodeAppend& app, void* out,
                               void* workspace, hipStream_t stream, DecodeMerge* defer = nullptr);

// Log-sum-exp merge of the split-KV partitions written by a decode kernel
// (partials [rows][max_parts] of (o / l) and (m, l)); rows with a single
// partition were written by the decode kernel and are skipped.
hipError_t launch_decode_merge(const float* part_o, const float* part_ml,
                               const int32_t* context_lens, int32_t ctx_clamp,
                               const DecodePlan& plan, int32_t num_decode_seqs,
                               int32_t num_q_heads, int32_t head_dim, void* out,
                               hipStream_t stream);

// fp8 (OCP E4M3) cache (kv_fp8.hip): the quantizing append, and paged decode
// over the codes with the same plan, partials and merge as the fp16 kernel.
hipError_t launch_kv_append_fp8(void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                                int64_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                const void* k_new, const void* v_new,
                                const int64_t* slot_mapping, int32_t num_tokens,
                                hipStream_t stream);

// With app.k_new set, the decode tokens are quantized and appended inside the
// decode kernel (as with fp16).
hipError_t launch_paged_decode_fp8(const void* q, void* k_codes, void* v_codes, float* k_scale,
                                   float* v_scale, int64_t num_blocks, int32_t num_kv_heads,
                                   int32_t num_q_heads, int32_t head_dim,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t num_decode_seqs,
                                   float scale, const DecodePlan& plan, const DecodeAppend& app,
                                   void* out, void* workspace, hipStream_t stream,
                                   DecodeMerge* defer = nullptr);

// Balanced decode schedule (decode_sched.hip): made once per step on the
// device from the context lengths, read by every layer's decode launch.
struct DecodeSchedulePlan {
  int32_t num_groups;     // decode work-groups (0: not schedulable, use the partition path)
  size_t schedule_bytes;  // size of the schedule buffer
  size_t partial_bytes;   // workspace for the pieces of split units
};

DecodeSchedulePlan plan_decode_schedule(int32_t num_decode_seqs, int32_t num_kv_heads,
                                        int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_context_len);

hipError_t launch_decode_schedule(const int32_t* context_lens, int32_t num_decode_seqs,
                                  int32_t num_kv_heads, int32_t ctx_clamp,
                                  const DecodeSchedulePlan& plan, void* schedule,
                                  hipStream_t stream);

hipError_t launch_paged_decode_scheduled(const void* q, void* k_pool, void* v_pool,
                                         int64_t num_blocks, int32_t num_kv_heads,
                                         int32_t num_q_heads, int32_t head_dim,
                                         const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, int32_t num_decode_seqs,
                                         float scale, const DecodeSchedulePlan& plan,
                                         const void* schedule, const DecodeAppend& app,
                                         void* out, void* workspace, hipStream_t stream,
                                         DecodeMerge* defer = nullptr);

// Split-KV plan of the prefill chunks: each 64-row query tile is cut into
// `splits` ranges of context tiles, merged by log-sum-exp when splits > 1.
struct PrefillPlan {
  int32_t splits;
  bool packed;             // every chunk's G x n rows fit one tile (short chunks)
  bool wide;               // long chunks at head_dim 128: 32 rows per wave (prefill_wide.hip)
  int32_t split_tiles;     // KV tiles per split (packed; 0: even ranges of the context)
  int64_t max_row_heads;   // bound on (prefill rows x query heads)
  size_t partial_bytes;
};

PrefillPlan plan_prefill(int32_t num_prefill_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t max_context_len, int32_t max_query_len,
                         int32_t kv_partition_tokens);

// The long-chunk kernels at head_dim 128 (prefill_wide.hip): 32 query rows
// per wave; the partials and their merge are the 16-row kernel's.
hipError_t launch_prefill_wide(const void* q, const void* k_pool, const void* v_pool,
                               const float* k_scale, const float* v_scale, int64_t num_blocks,
                               int32_t num_kv_heads, int32_t num_q_heads,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               int32_t first_seq, int32_t num_prefill_seqs,
                               int32_t max_query_len, float scale, int32_t splits, void* out,
                               float* part_o, float* part_ml, hipStream_t stream);

// Causal attention of the prefill chunks (sequences first_seq ..
// first_seq + num_prefill_seqs - 1) on the matrix cores.  With k_scale set
// the pools hold fp8 (E4M3) codes and k_scale / v_scale their row scales.
// With `fold` holding a decode merge left by the decode launch, that merge
// runs in the same launch as the chunks' merge (or alone, when the chunks
// need none), after the prefill kernel; the decode partials must then lie
// outside `workspace`.
hipError_t launch_prefill(const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scale, const float* v_scale, int64_t num_blocks,
                          int32_t num_kv_heads, int32_t num_q_heads, int32_t head_dim,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, const int32_t* query_start_loc,
                          int32_t first_seq, int32_t num_prefill_seqs, int32_t max_query_len,
                          float scale, const PrefillPlan& plan, void* out, void* workspace,
                          hipStream_t stream, const DecodeMerge* fold = nullptr);

}  // namespace pkv
