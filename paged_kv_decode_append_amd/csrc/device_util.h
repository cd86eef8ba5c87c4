// device_util.h -- small gfx950 device helpers shared by the HIP kernels of
// libpkv.so (fp16 packing, packed dot products, DPP lane exchanges).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Cache-policy operand of a raw buffer load that carries the non-temporal
// hint (nt).  The decode kernels put it on their V loads: measured on MI355X,
// it makes the decode launches 2-9% faster (long_context at d = 256 over an
// fp16 cache: no change), while the same hint on the K loads, which the
// scores wait for first, slows the ragged batches by 3-5%.
constexpr int kLoadNonTemporal = 2;

// 1.0 in both halves of a packed fp16 pair.
constexpr uint32_t kOnesH2 = 0x3C003C00u;

__device__ __forceinline__ f16x2 as_h2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }

// a.lo*b.lo + a.hi*b.hi + c, fp16 products accumulated in fp32 (v_dot2_f32_f16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// Two fp32 values packed into one fp16 pair (lo = a, hi = b), rounding toward zero.
__device__ __forceinline__ uint32_t pack_h2_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Two fp32 values packed into one fp16 pair (lo = a, hi = b), round to nearest even.
__device__ __forceinline__ uint32_t pack_h2_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(f16)a, (f16)b});
}

// 2^x with the hardware v_exp_f32 (exp2(-inf) = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane exchange inside a row of 16 lanes; every lane must have a source.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within each 16

// Sum over each aligned group of N lanes (N = 8 or 16); every lane of the
// group ends with the group's total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp<kDppMirror>(x);
  return x;
}

// v_permlane32_swap: lanes 32..63 of a trade places with lanes 0..31 of b;
// v_permlane16_swap: rows 1 and 3 of a (16 lanes each) with rows 0 and 2 of
// b.  Inline asm: hipcc's builtins for them lose one of the two results when
// both operands hold the same value.  The s_nop gives the two wait states the
// swaps need after a VALU write of their operands.
__device__ __forceinline__ void permlane32_swap(uint32_t& a, uint32_t& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void permlane16_swap(uint32_t& a, uint32_t& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// The maximum / sum of this lane's value and lane l ^ 32's, the same bits in
// both lanes (the halves exchanged in registers, no LDS round trip; the sum
// adds the lower lane's value first).
__device__ __forceinline__ float max_of_halves(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane32_swap(a, b);  // a: lane l % 32's value, b: lane 32 + l % 32's
  return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float sum_of_halves(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane32_swap(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// The maximum / sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the wave's four
// 16-lane rows), the same bits in all four: rows 0-1 and 2-3 are paired
// first, then the halves; the sum is (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float max_of_rows(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane16_swap(a, b);  // a: the even row's value, b: the odd row's
  return max_of_halves(fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
}
__device__ __forceinline__ float sum_of_rows(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  permlane16_swap(a, b);
  return sum_of_halves(__builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
}

// Keeps the compiler from moving LDS accesses across this point (no instruction).
__device__ __forceinline__ void wave_fence() { __builtin_amdgcn_wave_barrier(); }

}  // namespace pkv
