// noalloc.hip -- pkv_append_attention_step_noalloc: the fused append +
// attention step with its partials in a scratch array that lives in the
// library's device code, for callers that cannot allocate device memory
// (code under HIP graph capture, serving loops that forbid allocation).
//
// The scratch is one file-scope __device__ array per GPU (each device that
// loads the library holds its own copy until the process ends).  Its device
// address is looked up once per device, with that device current, and every
// later call passes that address to the same kernels the workspace version
// runs.  Nothing here allocates: no hipMalloc, no library call that does.
// No kernel of the step needs the scratch to start at zero (every partial
// is written before it is read), so it is never cleared.  Calls that
// overlap on one GPU (two streams, or two host threads) share the array and
// race; calls in stream order do not.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/pkv.h"
#include "kernels.h"

namespace {

static __device__ __attribute__((aligned(256))) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];

// Device address of this device's copy of `scratch` (looked up on the first
// call made with the device current), or null with the HIP error recorded
// for pkv_last_hip_error.
void* device_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    pkv::record_hip_error(e != hipSuccess ? e : hipErrorInvalidDevice);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      pkv::record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int pkv_append_attention_step_noalloc(const pkv_kv_cache* cache, const void* k_new,
                                      const void* v_new, const int64_t* slot_mapping,
                                      int32_t num_tokens, const void* q, void* out,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens,
                                      const int32_t* query_start_loc, int32_t num_seqs,
                                      int32_t num_decode_seqs, int32_t num_q_heads, float scale,
                                      int32_t max_context_len, int32_t max_query_len,
                                      int32_t kv_partition_tokens, const void* schedule,
                                      size_t schedule_bytes, void* stream) {
  if (!cache || !k_new) return PKV_ERR_INVALID_ARG;
  // The scratch's limit first, from the host hints alone, so that a step
  // too large for it is refused before any HIP call.
  size_t need = 0;
  int rc = pkv_attention_workspace_size(num_seqs, num_decode_seqs, num_q_heads,
                                        cache->num_kv_heads, cache->head_dim, max_context_len,
                                        max_query_len, kv_partition_tokens, &need);
  if (rc != PKV_OK) return rc;
  if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = device_scratch();
    if (ws == nullptr) return PKV_ERR_HIP;
  }
  return pkv_append_attention_step(cache, k_new, v_new, slot_mapping, num_tokens, q, out,
                                   block_tables, max_blocks_per_seq, context_lens,
                                   query_start_loc, num_seqs, num_decode_seqs, num_q_heads,
                                   scale, max_context_len, max_query_len, kv_partition_tokens,
                                   schedule, schedule_bytes, ws,
                                   need > 0 ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"
