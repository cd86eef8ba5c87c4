// sched_layout.h -- word layout of the balanced decode schedule buffer,
// shared by the schedule kernel, the decode kernel that walks it and the
// merge of the units it splits (decode_sched.hip, merge.h).
#pragma once

#include <stdint.h>

namespace pkv {
namespace sched {

constexpr int kInlineSegs = 4;  // segment descriptors inside the record

// Layout of the schedule buffer (int32 words):
//   [0] W (total cost)  [1] NWG  [2] U  [3] unused
//   P[U]       inclusive prefix of the unit costs (pad to 4 words)
//   rec[NWG]   per work-group: int4 head {n, overflow base, 0, 0},
//              int4 desc[kInlineSegs]
//   ovf[...]   descriptors k >= kInlineSegs, dense (capacity U + NWG)
//   um[U]      per unit: int2 {first work-group with a piece, work-groups
//              spanned} (the merge of split units)
// A descriptor is {u, jb, je, ctx}: unit u, its blocks [jb, je), context
// length of u's sequence (clamped).
constexpr int kRecWords = 4 + 4 * kInlineSegs;

__host__ __device__ inline int64_t sched_p_offset() { return 4; }
__host__ __device__ inline int64_t sched_rec_offset(int32_t U) { return 4 + (((int64_t)U + 3) & ~3LL); }
__host__ __device__ inline int64_t sched_ovf_offset(int32_t U, int32_t nwg) {
  return sched_rec_offset(U) + (int64_t)nwg * kRecWords;
}
// Overflow descriptors: at most one per (unit, work-group) piece beyond the
// inline ones, and pieces number at most U + NWG.
// Per unit: {first work-group holding a piece, work-groups spanned}.
__host__ __device__ inline int64_t sched_um_offset(int32_t U, int32_t nwg) {
  return sched_ovf_offset(U, nwg) + 4 * ((int64_t)U + nwg);
}
__host__ __device__ inline int64_t sched_words(int32_t U, int32_t nwg) {
  return sched_um_offset(U, nwg) + 2 * (int64_t)U;
}

}  // namespace sched
}  // namespace pkv
