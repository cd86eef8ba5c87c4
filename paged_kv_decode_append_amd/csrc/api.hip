// api.hip -- the extern "C" entry points of libpkv.so declared in include/pkv.h.
//
// Every entry point checks its host scalars and pointers first and returns
// an error before touching the GPU, so argument errors are reported on a
// machine without one.  Device arrays are never read from the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pkv.h"
#include "kernels.h"

namespace {

constexpr int32_t kBlockSize = 16;
constexpr int32_t kMaxGroup = 8;
constexpr int32_t kMaxGridYZ = 65535;

bool supported_head_dim(int32_t d) { return d == 128 || d == 256; }

int check_cache(const pkv_kv_cache* cache) {
  if (!cache || !cache->k_pool || !cache->v_pool) return PKV_ERR_INVALID_ARG;
  if (cache->kv_dtype != PKV_KV_FP16 && cache->kv_dtype != PKV_KV_FP8_E4M3)
    return PKV_ERR_UNSUPPORTED;
  if (cache->kv_dtype == PKV_KV_FP8_E4M3 && (!cache->k_scale || !cache->v_scale))
    return PKV_ERR_INVALID_ARG;
  if (cache->num_blocks <= 0 || cache->num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (cache->block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (!supported_head_dim(cache->head_dim)) return PKV_ERR_UNSUPPORTED;
  if (cache->num_kv_heads > kMaxGridYZ) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// Host-hint checks shared by the workspace query and the step.
int check_step_shape(int32_t num_seqs, int32_t num_decode_seqs, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, int32_t max_context_len,
                     int32_t max_query_len, int32_t kv_partition_tokens) {
  if (num_seqs < 0 || num_decode_seqs < 0 || num_decode_seqs > num_seqs)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return PKV_ERR_INVALID_ARG;
  if (num_q_heads / num_kv_heads > kMaxGroup) return PKV_ERR_UNSUPPORTED;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs > 0 && (max_context_len < 1 || max_query_len < 1)) return PKV_ERR_INVALID_ARG;
  if (kv_partition_tokens < 0 || kv_partition_tokens % 64 != 0 || kv_partition_tokens > 4096)
    return PKV_ERR_INVALID_ARG;
  if (max_query_len > (1 << 30) / 64) return PKV_ERR_UNSUPPORTED;
  return PKV_OK;
}

// Workspace: the decode partials and then, over the same bytes, the prefill
// partials -- the decode kernel and its merge are done with theirs (stream
// order) before the prefill kernel writes.
// Workspace of a step: the decode part's partials at its start; the prefill
// chunks' after them when the step has both, since the decode merge then
// runs in the step's combined merge after the prefill kernel (otherwise the
// chunks reuse the same bytes: the decode merge is done before they write).
size_t chunk_partial_offset(const pkv::DecodePlan& d, const pkv::PrefillPlan& p) {
  return d.partial_bytes > 0 && p.partial_bytes > 0 ? (d.partial_bytes + 255) / 256 * 256 : 0;
}
size_t workspace_layout(const pkv::DecodePlan& d, const pkv::PrefillPlan& p) {
  const size_t off = chunk_partial_offset(d, p);
  return off > 0 ? off + p.partial_bytes : std::max(d.partial_bytes, p.partial_bytes);
}

thread_local hipError_t t_last_hip_error = hipSuccess;

int from_hip(hipError_t e) {
  if (e == hipSuccess) return PKV_OK;
  t_last_hip_error = e;
  return PKV_ERR_HIP;
}

}  // namespace

namespace pkv {
void record_hip_error(hipError_t e) { t_last_hip_error = e; }
}  // namespace pkv

extern "C" {

int pkv_version(void) { return PKV_VERSION; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_CONTRACT: return "PKV_ERR_CONTRACT";
    default: return "PKV_ERR_UNKNOWN";
  }
}

int pkv_last_hip_error(const char** name) {
  if (name) *name = t_last_hip_error == hipSuccess ? "hipSuccess" : hipGetErrorName(t_last_hip_error);
  return (int)t_last_hip_error;
}

int pkv_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start_loc,
                     int32_t num_seqs, int32_t num_tokens, int32_t block_size,
                     int64_t* slot_mapping, void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (block_size != kBlockSize) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!query_start_loc && num_tokens != num_seqs) return PKV_ERR_INVALID_ARG;
  return from_hip(pkv::launch_slot_mapping(block_tables, max_blocks_per_seq, context_lens,
                                           query_start_loc, num_seqs, num_tokens, slot_mapping,
                                           static_cast<hipStream_t>(stream)));
}

int pkv_kv_append(const pkv_kv_cache* cache, const void* k_new, const void* v_new,
                  const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if (num_tokens < 0) return PKV_ERR_INVALID_ARG;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (cache->kv_dtype == PKV_KV_FP8_E4M3)
    return from_hip(pkv::launch_kv_append_fp8(
        cache->k_pool, cache->v_pool, static_cast<float*>(cache->k_scale),
        static_cast<float*>(cache->v_scale), cache->num_blocks, cache->num_kv_heads,
        cache->head_dim, k_new, v_new, slot_mapping, num_tokens,
        static_cast<hipStream_t>(stream)));
  return from_hip(pkv::launch_kv_append(cache->k_pool, cache->v_pool, cache->num_blocks,
                                        cache->num_kv_heads, cache->head_dim, k_new, v_new,
                                        slot_mapping, num_tokens,
                                        static_cast<hipStream_t>(stream)));
}

int pkv_attention_workspace_size(int32_t num_seqs, int32_t num_decode_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t max_query_len, int32_t kv_partition_tokens,
                                 size_t* bytes) {
  if (!bytes) return PKV_ERR_INVALID_ARG;
  int rc = check_step_shape(num_seqs, num_decode_seqs, num_q_heads, num_kv_heads, head_dim,
                            max_context_len, max_query_len, kv_partition_tokens);
  if (rc != PKV_OK) return rc;
  pkv::DecodePlan plan = pkv::plan_decode(num_decode_seqs, num_kv_heads, num_q_heads, head_dim,
                                          max_context_len, kv_partition_tokens);
  if (plan.max_parts > kMaxGridYZ) return PKV_ERR_UNSUPPORTED;
  const pkv::DecodeSchedulePlan splan = pkv::plan_decode_schedule(
      num_decode_seqs, num_kv_heads, num_q_heads, head_dim, max_context_len);
  if (kv_partition_tokens == 0)  // either decode path may run
    plan.partial_bytes = std::max(plan.partial_bytes, splan.partial_bytes);
  const pkv::PrefillPlan pplan = pkv::plan_prefill(num_seqs - num_decode_seqs, num_q_heads,
                                                   num_kv_heads, head_dim, max_context_len,
                                                   max_query_len, kv_partition_tokens);
  *bytes = workspace_layout(plan, pplan);
  return PKV_OK;
}

int pkv_decode_schedule_size(int32_t num_decode_seqs, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_context_len, size_t* bytes) {
  if (!bytes || num_decode_seqs < 0 || num_kv_heads <= 0 || max_context_len < 0)
    return PKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  *bytes = pkv::plan_decode_schedule(num_decode_seqs, num_kv_heads, num_kv_heads, head_dim,
                                     max_context_len).schedule_bytes;
  return PKV_OK;
}

int pkv_decode_schedule(const int32_t* context_lens, int32_t num_decode_seqs,
                        int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                        int32_t max_context_len, void* schedule, size_t schedule_bytes,
                        void* stream) {
  if (num_decode_seqs < 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0)
    return PKV_ERR_INVALID_ARG;
  if (!supported_head_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlockSize)
    return PKV_ERR_INVALID_ARG;
  const pkv::DecodeSchedulePlan splan = pkv::plan_decode_schedule(
      num_decode_seqs, num_kv_heads, num_kv_heads, head_dim, max_context_len);
  if (splan.num_groups == 0) return PKV_OK;  // nothing to schedule (partition path)
  if (!context_lens || !schedule) return PKV_ERR_INVALID_ARG;
  if (schedule_bytes < splan.schedule_bytes) return PKV_ERR_WORKSPACE;
  const int32_t ctx_clamp =
      (int32_t)std::min<int64_t>((int64_t)max_blocks_per_seq * kBlockSize, INT32_MAX);
  return from_hip(pkv::launch_decode_schedule(context_lens, num_decode_seqs, num_kv_heads,
                                              ctx_clamp, splan, schedule,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Attention of one layer; with k_new non-null the new tokens' append is done
// here too: the decode tokens' inside the decode kernel, the prefill tokens'
// by extra work-groups of the decode launch (by the append kernel when the
// step has no decode sequence), both ahead of the prefill kernel.  With
// check_only, every check (arguments, plans, workspace and schedule sizes,
// grid limits) runs and nothing is launched.
int attention_step(bool check_only, const pkv_kv_cache* cache, const void* k_new,
                   const void* v_new,
                   const int64_t* slot_mapping, int32_t num_tokens, const void* q, void* out,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, const int32_t* query_start_loc,
                   int32_t num_seqs, int32_t num_decode_seqs, int32_t num_q_heads, float scale,
                   int32_t max_context_len, int32_t max_query_len, int32_t kv_partition_tokens,
                   const void* schedule, size_t schedule_bytes, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  rc = check_step_shape(num_seqs, num_decode_seqs, num_q_heads, cache->num_kv_heads,
                        cache->head_dim, max_context_len, max_query_len, kv_partition_tokens);
  if (rc != PKV_OK) return rc;
  if (!std::isfinite(scale)) return PKV_ERR_INVALID_ARG;
  const bool fused = k_new != nullptr;
  if (fused) {
    if (!v_new || !slot_mapping || num_tokens < num_decode_seqs) return PKV_ERR_INVALID_ARG;
    if (!query_start_loc && num_tokens != num_seqs) return PKV_ERR_INVALID_ARG;
  }
  if (num_seqs == 0) return PKV_OK;
  if (!q || !out || !block_tables || !context_lens || max_blocks_per_seq <= 0)
    return PKV_ERR_INVALID_ARG;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * kBlockSize)
    return PKV_ERR_INVALID_ARG;
  const int32_t num_prefill = num_seqs - num_decode_seqs;
  if (num_prefill > 0 && !query_start_loc) return PKV_ERR_INVALID_ARG;
  if (num_prefill > kMaxGridYZ || num_q_heads > kMaxGridYZ) return PKV_ERR_UNSUPPORTED;
  pkv::DecodePlan plan = pkv::plan_decode(num_decode_seqs, cache->num_kv_heads, num_q_heads,
                                          cache->head_dim, max_context_len, kv_partition_tokens);
  // with the append, a step with decode sequences appends the prefill rows
  // in work-groups of the decode launch: up to append_groups more z slices
  const bool rows_in_decode = fused && num_decode_seqs > 0 && num_tokens > num_decode_seqs;
  const int32_t extra_z = rows_in_decode ? pkv::append_groups(num_tokens - num_decode_seqs) : 0;
  if (plan.max_parts > kMaxGridYZ - extra_z) return PKV_ERR_UNSUPPORTED;
  const pkv::DecodeSchedulePlan splan = pkv::plan_decode_schedule(
      num_decode_seqs, cache->num_kv_heads, num_q_heads, cache->head_dim, max_context_len);
  // The balanced schedule replaces the partition grid whenever the latter
  // would cut contexts (and was not forced by kv_partition_tokens); when
  // every (sequence, KV head) fits one work-group of a single round, the
  // partition grid needs no merge and is kept.
  const bool scheduled = schedule != nullptr && splan.num_groups > 0 &&
                         kv_partition_tokens == 0 && plan.max_parts > 1;
  if (scheduled && schedule_bytes < splan.schedule_bytes) return PKV_ERR_WORKSPACE;
  if (kv_partition_tokens == 0) plan.partial_bytes = std::max(plan.partial_bytes, splan.partial_bytes);
  const pkv::PrefillPlan pplan = pkv::plan_prefill(num_prefill, num_q_heads, cache->num_kv_heads,
                                                   cache->head_dim, max_context_len,
                                                   max_query_len, kv_partition_tokens);
  const size_t need = workspace_layout(plan, pplan);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  if (check_only) return PKV_OK;
  void* prefill_ws = need > 0 ? static_cast<char*>(workspace) + chunk_partial_offset(plan, pplan)
                              : nullptr;
  // a decode merge is left to the step's combined merge when the chunks are
  // split too (one launch fewer)
  pkv::DecodeMerge dm;
  pkv::DecodeMerge* const defer =
      num_prefill > 0 && pplan.splits > 1 && chunk_partial_offset(plan, pplan) > 0 ? &dm
                                                                                   : nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (cache->kv_dtype == PKV_KV_FP8_E4M3) {
    // quantized cache (partition grid only): with the append, the prefill
    // rows are quantized by the append kernel ahead of the attention, and
    // the decode kernel quantizes and appends the decode rows itself
    float* k_scale = static_cast<float*>(cache->k_scale);
    float* v_scale = static_cast<float*>(cache->v_scale);
    if (fused && num_tokens > num_decode_seqs && !rows_in_decode) {
      const size_t row_bytes = (size_t)cache->num_kv_heads * cache->head_dim * 2;
      rc = from_hip(pkv::launch_kv_append_fp8(
          cache->k_pool, cache->v_pool, k_scale, v_scale, cache->num_blocks,
          cache->num_kv_heads, cache->head_dim,
          static_cast<const char*>(k_new) + (size_t)num_decode_seqs * row_bytes,
          static_cast<const char*>(v_new) + (size_t)num_decode_seqs * row_bytes,
          slot_mapping + num_decode_seqs, num_tokens - num_decode_seqs, s));
      if (rc != PKV_OK) return rc;
    }
    const pkv::DecodeAppend app8{k_new, v_new, fused ? slot_mapping : nullptr,
                                 fused ? num_tokens : 0};
    rc = from_hip(pkv::launch_paged_decode_fp8(
        q, cache->k_pool, cache->v_pool, k_scale, v_scale, cache->num_blocks,
        cache->num_kv_heads, num_q_heads, cache->head_dim, block_tables, max_blocks_per_seq,
        context_lens, num_decode_seqs, scale, plan, app8, out, workspace, s, defer));
    if (rc != PKV_OK) return rc;
    return from_hip(pkv::launch_prefill(q, cache->k_pool, cache->v_pool, k_scale, v_scale,
                                        cache->num_blocks, cache->num_kv_heads, num_q_heads,
                                        cache->head_dim, block_tables, max_blocks_per_seq,
                                        context_lens, query_start_loc, num_decode_seqs,
                                        num_prefill, max_query_len, scale, pplan, out,
                                        prefill_ws, s, defer));
  }
  if (fused && num_tokens > num_decode_seqs && !rows_in_decode) {
    // rows of the prefill chunks follow the decode rows
    const size_t row_bytes = (size_t)cache->num_kv_heads * cache->head_dim * 2;
    rc = from_hip(pkv::launch_kv_append(
        cache->k_pool, cache->v_pool, cache->num_blocks, cache->num_kv_heads, cache->head_dim,
        static_cast<const char*>(k_new) + (size_t)num_decode_seqs * row_bytes,
        static_cast<const char*>(v_new) + (size_t)num_decode_seqs * row_bytes,
        slot_mapping + num_decode_seqs, num_tokens - num_decode_seqs, s));
    if (rc != PKV_OK) return rc;
  }
  const pkv::DecodeAppend app{k_new, v_new, fused ? slot_mapping : nullptr,
                             fused ? num_tokens : 0};
  if (scheduled)
    rc = from_hip(pkv::launch_paged_decode_scheduled(
        q, cache->k_pool, cache->v_pool, cache->num_blocks, cache->num_kv_heads, num_q_heads,
        cache->head_dim, block_tables, max_blocks_per_seq, num_decode_seqs, scale, splan,
        schedule, app, out, workspace, s, defer));
  else
    rc = from_hip(pkv::launch_paged_decode(
        q, cache->k_pool, cache->v_pool, cache->num_blocks, cache->num_kv_heads, num_q_heads,
        cache->head_dim, block_tables, max_blocks_per_seq, context_lens, num_decode_seqs, scale,
        plan, app, out, workspace, s, defer));
  if (rc != PKV_OK) return rc;
  return from_hip(pkv::launch_prefill(q, cache->k_pool, cache->v_pool, nullptr, nullptr,
                                      cache->num_blocks, cache->num_kv_heads, num_q_heads,
                                      cache->head_dim, block_tables, max_blocks_per_seq,
                                      context_lens, query_start_loc, num_decode_seqs,
                                      num_prefill, max_query_len, scale, pplan, out,
                                      prefill_ws, s, defer));
}

}  // namespace

extern "C" {

int pkv_paged_attention_step(const pkv_kv_cache* cache, const void* q, void* out,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, const int32_t* query_start_loc,
                             int32_t num_seqs, int32_t num_decode_seqs,
                             int32_t num_q_heads, float scale,
                             int32_t max_context_len, int32_t max_query_len,
                             int32_t kv_partition_tokens, const void* schedule,
                             size_t schedule_bytes, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return attention_step(false, cache, nullptr, nullptr, nullptr, 0, q, out, block_tables,
                        max_blocks_per_seq, context_lens, query_start_loc, num_seqs,
                        num_decode_seqs, num_q_heads, scale, max_context_len, max_query_len,
                        kv_partition_tokens, schedule, schedule_bytes, workspace,
                        workspace_bytes, stream);
}

int pkv_append_attention_step(const pkv_kv_cache* cache, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping, int32_t num_tokens, const void* q,
                              void* out, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              const int32_t* query_start_loc, int32_t num_seqs,
                              int32_t num_decode_seqs, int32_t num_q_heads, float scale,
                              int32_t max_context_len, int32_t max_query_len,
                              int32_t kv_partition_tokens, const void* schedule,
                              size_t schedule_bytes, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!k_new) return PKV_ERR_INVALID_ARG;
  return attention_step(false, cache, k_new, v_new, slot_mapping, num_tokens, q, out, block_tables,
                        max_blocks_per_seq, context_lens, query_start_loc, num_seqs,
                        num_decode_seqs, num_q_heads, scale, max_context_len, max_query_len,
                        kv_partition_tokens, schedule, schedule_bytes, workspace,
                        workspace_bytes, stream);
}

int pkv_append_attention_layers(const pkv_kv_cache* caches, int32_t num_layers,
                                const void* const* k_new, const void* const* v_new,
                                const int64_t* slot_mapping, int32_t num_tokens,
                                const void* const* q, void* const* out,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, const int32_t* query_start_loc,
                                int32_t num_seqs, int32_t num_decode_seqs, int32_t num_q_heads,
                                float scale, int32_t max_context_len, int32_t max_query_len,
                                int32_t kv_partition_tokens, const void* schedule,
                                size_t schedule_bytes, void* workspace, size_t workspace_bytes,
                                void* stream) {
  if (num_layers < 0) return PKV_ERR_INVALID_ARG;
  if (num_layers == 0) return PKV_OK;
  if (!caches || !k_new || !v_new || !q || !out) return PKV_ERR_INVALID_ARG;
  // every layer's descriptor, pointers and plans (workspace and schedule
  // sizes, grid limits, which depend on its heads and head_dim) before the
  // first launch
  for (int32_t l = 0; l < num_layers; ++l) {
    if (!k_new[l]) return PKV_ERR_INVALID_ARG;
    const int rc = attention_step(true, &caches[l], k_new[l], v_new[l], slot_mapping, num_tokens,
                                  q[l], out[l], block_tables, max_blocks_per_seq, context_lens,
                                  query_start_loc, num_seqs, num_decode_seqs, num_q_heads, scale,
                                  max_context_len, max_query_len, kv_partition_tokens, schedule,
                                  schedule_bytes, workspace, workspace_bytes, stream);
    if (rc != PKV_OK) return rc;
  }
  for (int32_t l = 0; l < num_layers; ++l) {
    const int rc = attention_step(false, &caches[l], k_new[l], v_new[l], slot_mapping,
                                  num_tokens, q[l],
                                  out[l], block_tables, max_blocks_per_seq, context_lens,
                                  query_start_loc, num_seqs, num_decode_seqs, num_q_heads, scale,
                                  max_context_len, max_query_len, kv_partition_tokens, schedule,
                                  schedule_bytes, workspace, workspace_bytes, stream);
    if (rc != PKV_OK) return rc;
  }
  return PKV_OK;
}

int pkv_validate_step(const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, const int32_t* query_start_loc,
                      int32_t num_seqs, int32_t num_decode_seqs, int64_t num_blocks,
                      int32_t block_size, const int64_t* slot_mapping, int32_t num_tokens,
                      int32_t max_context_len, int32_t max_query_len,
                      int32_t* bad_what, int64_t* bad_index) {
  if (!bad_what || !bad_index) return PKV_ERR_INVALID_ARG;
  *bad_what = 0;
  *bad_index = -1;
  if (num_seqs < 0 || num_decode_seqs < 0 || num_decode_seqs > num_seqs || num_tokens < 0 ||
      max_blocks_per_seq <= 0 || num_blocks <= 0 || block_size <= 0)
    return PKV_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PKV_ERR_INVALID_ARG;
  auto fail = [&](int32_t what, int64_t index) {
    *bad_what = what;
    *bad_index = index;
    return (int)PKV_ERR_CONTRACT;
  };
  if (query_start_loc && query_start_loc[0] != 0) return fail(3, 0);
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int32_t ctx = context_lens[i];
    const int32_t n = query_start_loc ? query_start_loc[i + 1] - query_start_loc[i] : 1;
    if (ctx < 1) return fail(1, i);
    if ((int64_t)ctx > (int64_t)max_blocks_per_seq * block_size) return fail(2, i);
    if (n < 0 || ctx < n) return fail(3, i);
    if (i < num_decode_seqs && n != 1) return fail(5, i);
    if (ctx > max_context_len || n > max_query_len) return fail(8, i);
    const int64_t used = ((int64_t)ctx + block_size - 1) / block_size;
    for (int64_t j = 0; j < used; ++j) {
      const int64_t b = block_tables[(int64_t)i * max_blocks_per_seq + j];
      if (b < 0 || b >= num_blocks) return fail(4, i);
    }
  }
  if (query_start_loc && query_start_loc[num_seqs] != num_tokens) return fail(3, num_seqs);
  if (!query_start_loc && num_tokens != num_seqs) return fail(3, num_seqs);
  if (slot_mapping) {
    std::unordered_set<int64_t> seen;
    seen.reserve((size_t)num_tokens * 2);
    for (int32_t t = 0; t < num_tokens; ++t) {
      const int64_t s = slot_mapping[t];
      if (s < 0) continue;
      if (s >= num_blocks * block_size) return fail(6, t);
      if (!seen.insert(s).second) return fail(7, t);
    }
    // every non-negative slot is the table's slot of its token's position
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int32_t first = query_start_loc ? query_start_loc[i] : i;
      const int32_t n = query_start_loc ? query_start_loc[i + 1] - first : 1;
      for (int32_t k = 0; k < n; ++k) {
        const int64_t s = slot_mapping[first + k];
        if (s < 0) continue;
        const int64_t p = (int64_t)context_lens[i] - n + k;
        const int64_t b = block_tables[(int64_t)i * max_blocks_per_seq + p / block_size];
        if (s != b * block_size + p % block_size) return fail(9, first + k);
      }
    }
    // a block that receives a new token is listed by no other sequence's
    // context (the fused step appends while other work-groups read)
    std::unordered_map<int64_t, int32_t> owner;
    std::unordered_set<int64_t> shared;
    for (int32_t i = 0; i < num_seqs; ++i) {
      const int64_t used = ((int64_t)context_lens[i] + block_size - 1) / block_size;
      for (int64_t j = 0; j < used; ++j) {
        const int64_t b = block_tables[(int64_t)i * max_blocks_per_seq + j];
        const auto it = owner.emplace(b, i).first;
        if (it->second != i) shared.insert(b);
      }
    }
    for (int32_t t = 0; t < num_tokens; ++t) {
      const int64_t s = slot_mapping[t];
      if (s >= 0 && shared.count(s / block_size)) return fail(10, t);
    }
  }
  return PKV_OK;
}

}  // extern "C"
