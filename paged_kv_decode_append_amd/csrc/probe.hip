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
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void read_tiles_kernel(
    const uint8_t* __restrict__ base, int64_t num_base_tiles, const int32_t* __restrict__ tile_ids,
    int64_t num_tiles, int32_t chunk_shift, int32_t tile_bytes, uint32_t* __restrict__ sink) {
  const int64_t total = num_tiles << chunk_shift;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  for (int64_t c0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; c0 < total;
       c0 += stride * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t c = c0 + stride * u;
      v[u] = uint4{0u, 0u, 0u, 0u};
      if (c < total) {
        const int64_t t = c >> chunk_shift;
        const int32_t raw = tile_ids[t];
        // ids outside the buffer are clamped into it: a wrong list gives a
        // wrong rate, never a read outside the buffer
        const int64_t id = raw < 0 ? 0 : (raw >= num_base_tiles ? num_base_tiles - 1 : raw);
        v[u] = *reinterpret_cast<const uint4*>(base + id * tile_bytes +
                                               ((c - (t << chunk_shift)) << 4));
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t s_acc[kThreads];
  s_acc[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int k = 0; k < kThreads; ++k) x ^= s_acc[k];
    sink[blockIdx.x] = x;
  }
}

}  // namespace

extern "C" int pkv_hbm_read_probe(const void* base, size_t base_bytes, const int32_t* tile_ids,
                                  int64_t num_tiles, int32_t tile_bytes, uint32_t* sink,
                                  void* stream) {
  if (num_tiles < 0) return PKV_ERR_INVALID_ARG;
  if (tile_bytes < 1024 || tile_bytes > 65536 || (tile_bytes & (tile_bytes - 1)) != 0)
    return PKV_ERR_INVALID_ARG;
  if (num_tiles == 0) return PKV_OK;
  if (!base || !tile_ids || !sink || base_bytes < (size_t)tile_bytes) return PKV_ERR_INVALID_ARG;
  if (num_tiles > (int64_t)1 << 40) return PKV_ERR_UNSUPPORTED;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  hipLaunchKernelGGL(read_tiles_kernel, dim3(PKV_PROBE_SINK_WORDS), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint8_t*>(base),
                     (int64_t)(base_bytes / (size_t)tile_bytes), tile_ids, num_tiles,
                     __builtin_ctz((unsigned)tile_bytes) - 4, tile_bytes, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    pkv::record_hip_error(e);
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}
