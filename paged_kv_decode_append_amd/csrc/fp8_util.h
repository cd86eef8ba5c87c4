// fp8_util.h -- OCP E4M3 decoding shared by the kernels that read an fp8 KV
// cache (decode in kv_fp8.hip, prefill chunks in prefill.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Two E4M3 codes (bytes 0-1 of w when HI is false, bytes 2-3 when true) to an
// fp16 pair; exact, since every E4M3 value is an fp16 value.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_h2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Sixteen codes to sixteen fp16 values (two 8-value halves, in order).
__device__ __forceinline__ void fp8x16_to_h16(const uint4& c, uint4& lo, uint4& hi) {
  lo = uint4{fp8x2_to_h2<false>(c.x), fp8x2_to_h2<true>(c.x), fp8x2_to_h2<false>(c.y),
             fp8x2_to_h2<true>(c.y)};
  hi = uint4{fp8x2_to_h2<false>(c.z), fp8x2_to_h2<true>(c.z), fp8x2_to_h2<false>(c.w),
             fp8x2_to_h2<true>(c.w)};
}

// Eight codes to eight fp16 values, in order.
__device__ __forceinline__ uint4 fp8x8_to_h8(const uint2& c) {
  return uint4{fp8x2_to_h2<false>(c.x), fp8x2_to_h2<true>(c.x), fp8x2_to_h2<false>(c.y),
               fp8x2_to_h2<true>(c.y)};
}

}  // namespace pkv
