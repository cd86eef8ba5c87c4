// probe.hip -- HBM read-rate probe: reads a list of whole tiles of a buffer
// once, in the listed order, and nothing else.  With 4 KiB (d = 128) or
// 8 KiB (d = 256) tiles in a random order it is the paged decode's memory
// access pattern (one KV head's block of K or V is one contiguous tile,
// blocks scattered through the pool) without any of its arithmetic, so its
// rate is what HBM gives that pattern: the measured denominator beside the
// 8 TB/s specification.  The pages report read rates as a share of the
// card's peak bandwidth (danielfleming.xyz, "Static batching", section
// "Where scaling stops, and why the prediction missed").
//
// Each thread reads 16-byte chunks; a wave's load covers 1 KiB of one tile
// (64 lanes x 16 bytes, one contiguous run), kUnroll chunks per thread are
// in flight, and the grid strides over the chunks of the whole list.  The
// loaded words are folded with XOR into one word per work-group (the sink),
// so no load can be dropped.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/pkv.h"
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 128 bytes in flight per thread

__global__ __launch_bounds__(kThreads) void read_tiles_kernel(
    const uint8_t* __restrict__ base, int64_t num_base_tiles, const int32_t* __restrict__ tile_ids,
    int64_t num_tiles, int32_t chunk_shift, int32_t tile_bytes, uint32_t* __restrict__ sink) {
  const int64_t total = num_tiles << chunk_shift;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  const int64_t chunk_mask = ((int64_t)1 << chunk_shift) - 1;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; c0 < total;
       c0 += stride * kUnroll) {
    // all ids first, then all data loads, without branches (a load under a
    // branch is waited for at once): chunks past the end re-read the last
    // chunk and are dropped
    int32_t raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = min(c0 + stride * u, total - 1);
      raw[u] = tile_ids[c >> chunk_shift];
    }
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = min(c0 + stride * u, total - 1);
      // ids outside the buffer are clamped into it: a wrong list gives a
      // wrong rate, never a read outside the buffer
      const int64_t id = raw[u] < 0 ? 0 : (raw[u] >= num_base_tiles ? num_base_tiles - 1 : raw[u]);
      v[u] = *reinterpret_cast<const uint4*>(base + id * tile_bytes + ((c & chunk_mask) << 4));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (c0 + stride * u < total) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // fold: within the wave by lane exchanges, then the 4 waves' words
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  __shared__ uint32_t s_acc[kThreads / 64];
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int k = 0; k < kThreads / 64; ++k) x ^= s_acc[k];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

extern "C" int pkv_hbm_read_probe(const void* base, size_t base_bytes, const int32_t* tile_ids,
                                  int64_t num_tiles, int32_t tile_bytes, int32_t launches,
                                  uint32_t* sink, void* stream) {
  if (num_tiles < 0 || launches < 0) return PKV_ERR_INVALID_ARG;
  if (tile_bytes < 1024 || tile_bytes > 65536 || (tile_bytes & (tile_bytes - 1)) != 0)
    return PKV_ERR_INVALID_ARG;
  if (num_tiles == 0 || launches == 0) return PKV_OK;
  if (!base || !tile_ids || !sink || base_bytes < (size_t)tile_bytes) return PKV_ERR_INVALID_ARG;
  if (num_tiles > (int64_t)1 << 40 || launches > 4096) return PKV_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  // back-to-back launches from here: one host call for all of them, so that
  // the host cost of a call does not leave the GPU idle between launches
  for (int32_t k = 0; k < launches; ++k) {
    hipLaunchKernelGGL(read_tiles_kernel, dim3(PKV_PROBE_SINK_WORDS), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(base),
                       (int64_t)(base_bytes / (size_t)tile_bytes), tile_ids + k * num_tiles,
                       num_tiles, __builtin_ctz((unsigned)tile_bytes) - 4, tile_bytes, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      pkv::record_hip_error(e);
      return PKV_ERR_HIP;
    }
  }
  return PKV_OK;
}
