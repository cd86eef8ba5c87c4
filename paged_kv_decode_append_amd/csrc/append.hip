// append.hip -- slot mapping and slot-mapped KV append kernels.
//
// Slot mapping: new token k of sequence i sits on top of the tokens already
// computed, at logical position ctx_i - n_i + k, inside the sequence's own
// 16-token blocks (deepconcepts.dev, "Continuous Batching Is Not a Bigger
// Batch", sections "What the scheduler does on one step" and "The allocator
// is the other half").
//
// Append: each new token's K and V rows are copied into their slot, one
// 16-byte chunk per thread: a [T][Hkv][d] fp16 source row of one KV head is
// d*2 contiguous bytes, and so is its destination row inside the block, so
// every wave stores whole 16-byte chunks of contiguous rows.
#include "device_util.h"
#include "kernels.h"

namespace pkv {

constexpr int kBlockSize = 16;

// One work-group of 64 threads per sequence; threads stride over its new tokens.
__global__ __launch_bounds__(64) void slot_mapping_kernel(
    const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ query_start_loc,
    int32_t num_tokens, int64_t* __restrict__ slot_mapping) {
  const int32_t i = blockIdx.x;
  const int32_t first = query_start_loc ? query_start_loc[i] : i;
  const int32_t n = query_start_loc ? query_start_loc[i + 1] - first : 1;
  const int32_t ctx = context_lens[i];
  const int32_t* row = block_tables + (int64_t)i * max_blocks_per_seq;
  for (int32_t k = threadIdx.x; k < n; k += blockDim.x) {
    if (first + k < 0 || first + k >= num_tokens) break;  // inconsistent offsets: write nothing
    const int32_t p = ctx - n + k;
    const int32_t logical_block = p / kBlockSize;
    int64_t slot = -1;
    if (p >= 0 && logical_block < max_blocks_per_seq)
      slot = (int64_t)row[logical_block] * kBlockSize + p % kBlockSize;
    slot_mapping[first + k] = slot;
  }
}

hipError_t launch_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, const int32_t* query_start_loc,
                               int32_t num_seqs, int32_t num_tokens, int64_t* slot_mapping,
                               hipStream_t stream) {
  if (num_seqs == 0 || num_tokens == 0) return hipSuccess;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(num_seqs), dim3(64), 0, stream, block_tables,
                     max_blocks_per_seq, context_lens, query_start_loc, num_tokens, slot_mapping);
  return hipGetLastError();
}

// grid.y selects the pool (0 = K, 1 = V); x covers num_tokens * Hkv * (d / 8) chunks.
__global__ __launch_bounds__(256) void kv_append_kernel(
    uint4* __restrict__ k_pool, uint4* __restrict__ v_pool, int64_t num_blocks,
    int32_t chunks_per_token, int32_t chunks_per_row, const uint4* __restrict__ k_new,
    const uint4* __restrict__ v_new, const int64_t* __restrict__ slot_mapping,
    int64_t total_chunks) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const int64_t t = idx / chunks_per_token;
  const int32_t rest = (int32_t)(idx - t * chunks_per_token);  // head * chunks_per_row + chunk
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;
  const int64_t block = slot / kBlockSize;
  if (block >= num_blocks) return;
  const int32_t offset = (int32_t)(slot % kBlockSize);
  const int32_t head = rest / chunks_per_row;
  const int32_t chunk = rest - head * chunks_per_row;
  const int32_t num_kv_heads = chunks_per_token / chunks_per_row;
  const int64_t dst =
      ((block * num_kv_heads + head) * kBlockSize + offset) * chunks_per_row + chunk;
  if (blockIdx.y == 0)
    k_pool[dst] = k_new[idx];
  else
    v_pool[dst] = v_new[idx];
}

hipError_t launch_kv_append(void* k_pool, void* v_pool, int64_t num_blocks,
                            int32_t num_kv_heads, int32_t head_dim, const void* k_new,
                            const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                            hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int32_t chunks_per_row = head_dim / 8;  // 16-byte chunks of one head's row
  const int32_t chunks_per_token = num_kv_heads * chunks_per_row;
  const int64_t total = (int64_t)num_tokens * chunks_per_token;
  const int64_t blocks = (total + 255) / 256;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  hipLaunchKernelGGL(kv_append_kernel, dim3((uint32_t)blocks, 2), dim3(256), 0, stream,
                     static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), num_blocks,
                     chunks_per_token, chunks_per_row, static_cast<const uint4*>(k_new),
                     static_cast<const uint4*>(v_new), slot_mapping, total);
  return hipGetLastError();
}

}  // namespace pkv
