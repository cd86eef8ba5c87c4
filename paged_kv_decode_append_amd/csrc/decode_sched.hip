// decode_sched.hip -- paged decode attention over a balanced per-step
// schedule, for batches whose context lengths differ (deepconcepts.dev,
// "Continuous Batching Is Not a Bigger Batch": the batch is re-formed every
// pass and mixes sequences at every stage of generation; danielfleming.xyz,
// "Static batching", section "Ragged batches": a paged layout stores only
// real tokens, so a ragged mix should cost only its real tokens).
//
// The unit of work is one (sequence, KV head): ceil(ctx / 16) blocks read
// once and applied to the G query heads of the group.  In a ragged batch the
// units differ by two orders of magnitude, so one work-group per unit (or per
// fixed-size piece of a unit) leaves most of the GPU idle behind the longest
// ones.  Here the units are laid end to end, each costing its blocks plus
// kSegCost (the fixed work of a segment: query rows, merge of the waves,
// output), and the total cost is cut into equal ranges, one per work-group of
// a single resident round.  A work-group's range is a list of segments: the
// tail of one unit, whole short units, the head of a long one.  Short units
// are packed together; only units longer than a range are split, and their
// pieces -- one per work-group, at slot u + w (unique: the ranges are
// contiguous) -- are merged by log-sum-exp afterwards.
//
// The schedule depends only on the context lengths, so it is computed once
// per step (decode_schedule_kernel, one work-group) and read by every layer's
// decode kernel with one scalar load of its 64-byte record.
//
// Inside a work-group the 4 waves take the blocks of each segment round-robin;
// every wave streams its blocks of consecutive segments with the two-buffer
// register prefetch running across segment boundaries, so a segment's first
// blocks are already in flight when the previous segment is merged.
#include <algorithm>
#include <climits>

#include "decode_block.h"
#include "device_util.h"
#include "kernels.h"
#include "merge.h"
#include "sched_layout.h"

namespace pkv {

namespace {

using namespace decode_block;
using namespace sched;

constexpr int kWaves = 4;
constexpr int32_t kSegCost = 2;          // fixed cost of a segment, in blocks
constexpr int kMaxSegs = 128;            // segments per work-group (host-enforced bound)
constexpr int kMaxWgBlocks = 2048;       // blocks per work-group (host-enforced bound)
constexpr int kSchedThreads = 1024;
constexpr int32_t kMaxSchedUnits = 16384;
constexpr float kLog2e = 1.4426950408889634f;


// Work-group of the block at cost position c (ranges [C_w, C_w+1),
// C_w = floor(w W / NWG)).
__device__ __forceinline__ int32_t wg_of(int64_t c, int64_t W, int32_t nwg) {
  return (int32_t)(((c + 1) * nwg + W - 1) / W) - 1;
}

__global__ __launch_bounds__(kSchedThreads) void decode_schedule_kernel(
    const int32_t* __restrict__ context_lens, int32_t num_seqs, int32_t num_kv_heads,
    int32_t ctx_clamp, int32_t nwg, int32_t* __restrict__ sched) {
  __shared__ int32_t s_p[kMaxSchedUnits];
  __shared__ int32_t s_wave[kSchedThreads / 64];
  __shared__ int32_t s_carry;
  __shared__ int32_t s_ovf_total;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t U = num_seqs * num_kv_heads;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  // inclusive prefix of the unit costs, 1024 units at a time
  for (int32_t base = 0; base < U; base += kSchedThreads) {
    const int32_t u = base + tid;
    int32_t c = 0;
    if (u < U) {
      const int32_t ctx = min(context_lens[u / num_kv_heads], ctx_clamp);
      c = ctx > 0 ? ((ctx + 15) >> 4) + kSegCost : 0;
    }
    int32_t x = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int32_t before = s_carry;
    for (int w2 = 0; w2 < wave; ++w2) before += s_wave[w2];
    x += before;
    if (u < U) s_p[u] = x;
    __syncthreads();
    if (tid == kSchedThreads - 1) s_carry = x;
    __syncthreads();
  }
  const int32_t W = U > 0 ? s_p[U - 1] : 0;
  int32_t* P = sched + sched_p_offset();
  int2* um = reinterpret_cast<int2*>(sched + sched_um_offset(U, nwg));
  for (int32_t u = tid; u < U; u += kSchedThreads) {
    P[u] = s_p[u];
    const int32_t prev = u > 0 ? s_p[u - 1] : 0;
    const int64_t b0 = (int64_t)prev + kSegCost, b1 = (int64_t)s_p[u] - 1;
    int2 m{0, 0};
    if (b1 >= b0 && W > 0) {
      m.x = wg_of(b0, W, nwg);
      m.y = wg_of(b1, W, nwg) - m.x + 1;
    }
    um[u] = m;
  }
  if (tid == 0) {
    sched[0] = W;
    sched[1] = nwg;
    sched[2] = U;
    sched[3] = 0;
  }

  // Per work-group: its segments (non-empty intersections of its cost range
  // with the units' block ranges [P[u-1] + kSegCost, P[u])).
  auto lower_bound = [&](int32_t key) {  // first u with P[u] >= key (U if none)
    int32_t lo = 0, hi = U;
    while (lo < hi) {
      const int32_t mid = (lo + hi) >> 1;
      if (s_p[mid] < key) lo = mid + 1; else hi = mid;
    }
    return lo;
  };
  auto count_and_emit = [&](int32_t w, bool emit, int32_t ovf_base) -> int32_t {
    const int64_t c0 = W > 0 ? (int64_t)w * W / nwg : 0;
    const int64_t c1 = W > 0 ? (int64_t)(w + 1) * W / nwg : 0;
    if (c1 <= c0) return 0;
    const int32_t uf = lower_bound((int32_t)c0 + 1);
    const int32_t ul = min(lower_bound((int32_t)c1), U - 1);
    int32_t n = 0;
    for (int32_t u = uf; u <= ul; ++u) {
      const int32_t prev = u > 0 ? s_p[u - 1] : 0;
      const int32_t b0 = prev + kSegCost;     // cost position of block 0
      const int32_t nb = s_p[u] - b0;         // blocks of the unit (<= 0: empty)
      if (nb <= 0) continue;
      const int32_t jb = (int32_t)max<int64_t>(0, c0 - b0);
      const int32_t je = (int32_t)min<int64_t>(nb, c1 - b0);
      if (je <= jb) continue;
      if (emit) {
        const int32_t ctx = min(context_lens[u / num_kv_heads], ctx_clamp);
        int4 d{u, jb, je, ctx};
        int32_t* dst = n < kInlineSegs
                           ? sched + sched_rec_offset(U) + (int64_t)w * kRecWords + 4 + 4 * n
                           : sched + sched_ovf_offset(U, nwg) + 4 * (int64_t)(ovf_base + n - kInlineSegs);
        *reinterpret_cast<int4*>(dst) = d;
      }
      ++n;
    }
    return n;
  };
  // overflow bases: exclusive prefix over work-groups of max(0, n_w - kInlineSegs)
  if (tid == 0) s_ovf_total = 0;
  __syncthreads();
  for (int32_t base = 0; base < nwg; base += kSchedThreads) {
    const int32_t w = base + tid;
    const int32_t n = w < nwg ? count_and_emit(w, false, 0) : 0;
    int32_t x = max(0, n - kInlineSegs);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int32_t before = s_ovf_total;
    for (int w2 = 0; w2 < wave; ++w2) before += s_wave[w2];
    const int32_t incl = before + x;
    if (w < nwg) {
      const int32_t ob = incl - max(0, n - kInlineSegs);
      count_and_emit(w, true, ob);
      int4 head{n, ob, 0, 0};
      *reinterpret_cast<int4*>(sched + sched_rec_offset(U) + (int64_t)w * kRecWords) = head;
    }
    __syncthreads();
    if (tid == kSchedThreads - 1) s_ovf_total = incl;
    __syncthreads();
  }
}

// Stream position of a wave: its blocks of segment s are j = jb + wave + 4k,
// k < nbw(s); every segment takes an even number of positions (a trailing
// empty slot when nbw is odd) so that its first block always lands in
// buffer A, and the refills of one segment's last blocks request the next
// segments' first ones.
struct SegInfo {
  int32_t u, jb, je, ctx;
};

template <int D, int G, bool APPEND>
__global__ __launch_bounds__(64 * kWaves, 2) void paged_decode_sched_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ k_pool,
    uint16_t* __restrict__ v_pool, int64_t num_blocks, int32_t num_kv_heads,
    const int32_t* __restrict__ block_tables, int32_t max_blocks_per_seq,
    const int32_t* __restrict__ sched, int32_t U, int32_t nwg, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int64_t* __restrict__ slot_mapping, int32_t num_decode_seqs, int32_t num_tokens) {
  constexpr int GP = (G + 3) & ~3, RCH = D / 8;
  constexpr bool kEarlyRefill = D == 128;
  constexpr int QCH = G * D / 8;
  constexpr int QPT = (QCH + 255) / 256;  // query chunks per thread
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ uint32_t s_p[kWaves][8 * GP];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[2][G * D];   // current, next segment
  __shared__ __attribute__((aligned(16))) uint16_t s_new[2][APPEND ? 2 * D : 8];
  __shared__ int32_t s_subst[2];
  __shared__ SegInfo s_seg[kMaxSegs];
  __shared__ int32_t s_fstart[kMaxSegs + 1];   // first staged block of each segment
  __shared__ int32_t s_bid[kMaxWgBlocks];      // raw block ids of the work-group's blocks

  // the wave index is the same in all its lanes: say so, so that what derives
  // from it (block counts, buffer resources) stays in scalar registers
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w = blockIdx.x;
  if (APPEND && w >= nwg) {
    // the work-groups past the schedule's (dispatched last): prefill rows
    append_rows<D>(k_pool, v_pool, num_blocks, num_kv_heads, k_new, v_new, slot_mapping,
                   num_decode_seqs, num_tokens, w - nwg, (int)gridDim.x - nwg, tid, 64 * kWaves);
    return;
  }
  const int32_t* rec = sched + sched_rec_offset(U) + (int64_t)w * kRecWords;
  // the whole 80-byte record at once (16-byte aligned): head + 4 descriptors
  int4 rv[1 + kInlineSegs];
#pragma unroll
  for (int k = 0; k <= kInlineSegs; ++k) rv[k] = reinterpret_cast<const int4*>(rec)[k];
  const int32_t nseg = rv[0].x;
  const int32_t ob = rv[0].y;
  // A schedule not made by the schedule kernel for this step breaks the
  // caller contract: every read it drives is range-checked, so it can only
  // give wrong numbers (> kMaxSegs is excluded by the plan).
  if (nseg <= 0 || nseg > kMaxSegs || ob < 0 ||
      (int64_t)ob + max(0, nseg - kInlineSegs) > (int64_t)U + nwg)
    return;  // uniform over the work-group
  const int num_q_heads = num_kv_heads * G;
  const int64_t tile_elems = (int64_t)16 * D;
  const int64_t block_stride = (int64_t)num_kv_heads * tile_elems;

  const int32_t ctx_cap = (int32_t)min<int64_t>((int64_t)max_blocks_per_seq * 16, INT32_MAX);
  auto checked = [&](int4 d) -> SegInfo {
    SegInfo sg{d.x, d.y, d.z, min(max(d.w, 1), ctx_cap)};
    // keep a corrupt descriptor inside the tables: an empty segment of unit 0
    const int32_t nb = (sg.ctx + 15) >> 4;
    if (sg.u < 0 || sg.u >= U || sg.jb < 0 || sg.je > nb || sg.je <= sg.jb)
      sg = SegInfo{0, 0, 0, 1};
    return sg;
  };
  // descriptor k >= kInlineSegs (the inline ones are in rv)
  auto seg_from_record = [&](int k) -> SegInfo {
    return checked(reinterpret_cast<const int4*>(
        sched + sched_ovf_offset(U, nwg) + 4 * (int64_t)(ob + k - kInlineSegs))[0]);
  };
  // a segment descriptor read from LDS, as scalars (the same for every lane)
  auto seg_at = [&](int k) -> SegInfo {
    const SegInfo sg = s_seg[k];
    return SegInfo{__builtin_amdgcn_readfirstlane(sg.u), __builtin_amdgcn_readfirstlane(sg.jb),
                   __builtin_amdgcn_readfirstlane(sg.je), __builtin_amdgcn_readfirstlane(sg.ctx)};
  };
  auto nbw_of = [&](const SegInfo& sg) {
    return max(0, (sg.je - sg.jb - wave + kWaves - 1) / kWaves);
  };
  auto clamp_bid = [&](int32_t raw) -> int64_t {
    return (uint32_t)raw < (uint64_t)num_blocks ? (int64_t)raw : num_blocks - 1;
  };
  // Per-segment side data for the append: the new K/V rows of the unit (one
  // 16-byte chunk per thread) and whether they replace the pool's rows.
  struct NewRows {
    uint4 kc, vc;  // this thread's 16-byte chunk of the K row / of the V row
    int32_t subst;
  };
  auto fetch_new = [&](const SegInfo& sg) -> NewRows {
    NewRows r{uint4{0u, 0u, 0u, 0u}, uint4{0u, 0u, 0u, 0u}, 0};
    if constexpr (APPEND) {
      const int i = sg.u / num_kv_heads, g = sg.u - i * num_kv_heads;
      const int nblk_u = (sg.ctx + 15) >> 4;
      if (sg.je != nblk_u) return r;  // not the piece that holds the new token
      const int64_t row = ((int64_t)i * num_kv_heads + g) * D;
      // separate destinations: no load waits for the other's register
      if (tid < RCH) r.kc = reinterpret_cast<const uint4*>(k_new + row)[tid];
      if (tid >= 64 && tid < 64 + RCH)
        r.vc = reinterpret_cast<const uint4*>(v_new + row)[tid - 64];
      const int64_t slot = slot_mapping[i];
      const int32_t raw_last = block_tables[(int64_t)i * max_blocks_per_seq + nblk_u - 1];
      r.subst = slot >= 0 && (uint32_t)raw_last < (uint64_t)num_blocks &&
                slot == (int64_t)raw_last * 16 + ((sg.ctx - 1) & 15);
    }
    return r;
  };
  auto stage_new = [&](const NewRows& r, int buf) {
    if constexpr (APPEND) {
      if (tid < RCH)
        reinterpret_cast<uint4*>(s_new[buf])[tid] = r.kc;
      else if (tid >= 64 && tid < 64 + RCH)
        reinterpret_cast<uint4*>(s_new[buf] + D)[tid - 64] = r.vc;
      if (tid == 0) s_subst[buf] = r.subst;
    }
  };
  auto fetch_q = [&](const SegInfo& sg, uint4 (&qr)[QPT]) {
    const int i = sg.u / num_kv_heads, g = sg.u - i * num_kv_heads;
    const uint4* qsrc =
        reinterpret_cast<const uint4*>(q + ((int64_t)i * num_q_heads + (int64_t)g * G) * D);
#pragma unroll
    for (int k = 0; k < QPT; ++k)
      if (tid + 256 * k < QCH) qr[k] = qsrc[tid + 256 * k];
  };
  auto stage_q = [&](const uint4 (&qr)[QPT], int buf) {
#pragma unroll
    for (int k = 0; k < QPT; ++k)
      if (tid + 256 * k < QCH) reinterpret_cast<uint4*>(s_q[buf])[tid + 256 * k] = qr[k];
  };

  // ---- startup.  The small loads go first -- the block ids of the
  // segments described in the record (one per thread), segment 0's query and
  // appended rows, this wave's first two block ids -- and this wave's first
  // two blocks of K/V after them: in the other order they would queue behind
  // the first 32 MiB of K/V that the whole GPU requests at once.
  const int ninl = min(nseg, kInlineSegs);
  SegInfo inl[kInlineSegs];
  int32_t inl_f[kInlineSegs + 1];
  inl_f[0] = 0;
#pragma unroll
  for (int k = 0; k < kInlineSegs; ++k) {
    inl[k] = k < ninl ? checked(rv[1 + k]) : SegInfo{0, 0, 0, 1};
    inl_f[k + 1] = inl_f[k] + (k < ninl ? inl[k].je - inl[k].jb : 0);
  }
  const SegInfo seg0 = inl[0];
  const int n0 = nbw_of(seg0);
  const int i0 = seg0.u / num_kv_heads, g0 = seg0.u - i0 * num_kv_heads;
  const int32_t* bt0 = block_tables + (int64_t)i0 * max_blocks_per_seq;
  // the wave index as a scalar: the first two block ids are scalar loads
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int32_t first_a = n0 > 0 ? bt0[seg0.jb + wv] : 0;
  const int32_t first_b = n0 > 1 ? bt0[seg0.jb + wv + kWaves] : 0;
  constexpr int kIdsPerThread = kMaxWgBlocks / (64 * kWaves);
  int32_t ids[kIdsPerThread];
  const int32_t inl_blocks = min(inl_f[kInlineSegs], kMaxWgBlocks);
#pragma unroll
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int32_t f = tid + 64 * kWaves * r;
    ids[r] = 0;
    if (f < inl_blocks) {
      // segment of flat block f among the inline ones (selects, no indexing)
      SegInfo sg = inl[0];
      int32_t f0 = 0;
#pragma unroll
      for (int kk = 1; kk < kInlineSegs; ++kk)
        if (f >= inl_f[kk]) {
          sg = inl[kk];
          f0 = inl_f[kk];
        }
      ids[r] = block_tables[(int64_t)(sg.u / num_kv_heads) * max_blocks_per_seq + sg.jb +
                            (f - f0)];
    }
  }
  uint4 q0[QPT];
  fetch_q(seg0, q0);
  const NewRows r0 = fetch_new(seg0);
  // This wave's first two blocks of K/V, requested unconditionally (block 0
  // of the pool stands in for one it does not have) so that the number of
  // loads in flight is fixed and the LDS stores below wait only for the
  // small loads above.
  KVRegs<D> A, B;
  __builtin_amdgcn_sched_barrier(0);  // nothing that uses the loads above moves up here
  {
    const int64_t oa = (n0 > 0 ? clamp_bid(first_a) * block_stride : 0) + (int64_t)g0 * tile_elems;
    load_k<D>(A, k_pool + oa, lane);
    load_v<D>(A, v_pool + oa, lane);
    if constexpr (kEarlyRefill) {
      const int64_t ob2 =
          (n0 > 1 ? clamp_bid(first_b) * block_stride : 0) + (int64_t)g0 * tile_elems;
      load_k<D>(B, k_pool + ob2, lane);
      load_v<D>(B, v_pool + ob2, lane);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  if (tid < ninl) {
    SegInfo my_seg = inl[0];
#pragma unroll
    for (int k = 1; k < kInlineSegs; ++k)
      if (tid == k) my_seg = inl[k];
    s_seg[tid] = my_seg;
  }
#pragma unroll
  for (int r = 0; r < kIdsPerThread; ++r) {
    const int32_t f = tid + 64 * kWaves * r;
    if (f < inl_blocks) s_bid[f] = ids[r];
  }
#pragma unroll
  for (int k = 0; k <= kInlineSegs; ++k)
    if (tid == k && k <= ninl) s_fstart[k] = inl_f[k];
  stage_q(q0, 0);
  stage_new(r0, 0);
  __syncthreads();
  if (nseg > kInlineSegs) {
    // more segments than the record holds: their descriptors, offsets and
    // block ids now
    if (tid >= kInlineSegs && tid < nseg) s_seg[tid] = seg_from_record(tid);
    __syncthreads();
    if (tid == 0) {
      int32_t f = inl_f[kInlineSegs];
      for (int k = kInlineSegs; k < nseg; ++k) {
        s_fstart[k] = f;
        f += s_seg[k].je - s_seg[k].jb;
      }
      s_fstart[nseg] = f;
    }
    __syncthreads();
    // more blocks than staged only with a context longer than the planned
    // maximum (a broken contract): give up on this range rather than read
    // past the staging buffer
    if (s_fstart[nseg] > kMaxWgBlocks) return;  // uniform over the work-group
    for (int32_t f = inl_f[kInlineSegs] + tid; f < s_fstart[nseg]; f += 64 * kWaves) {
      int k = kInlineSegs;
      while (k + 1 < nseg && s_fstart[k + 1] <= f) ++k;
      const SegInfo sg = s_seg[k];
      s_bid[f] = block_tables[(int64_t)(sg.u / num_kv_heads) * max_blocks_per_seq + sg.jb +
                              (f - s_fstart[k])];
    }
    __syncthreads();
  } else if (inl_f[kInlineSegs] > kMaxWgBlocks) {
    return;  // as above (uniform)
  }

  // Pool offset of this wave's k-th block of segment s (a scalar).
  auto tile_off = [&](int s, int k) -> int64_t {
    const int g = __builtin_amdgcn_readfirstlane(s_seg[s].u % num_kv_heads);
    const int32_t f = __builtin_amdgcn_readfirstlane(s_fstart[s]) + wave + kWaves * k;
    return clamp_bid(__builtin_amdgcn_readfirstlane(s_bid[f])) * block_stride +
           (int64_t)g * tile_elems;
  };
  // Tile (cs, kk) as buffer resources; empty when the cursor has no block
  // there (the loads are issued unconditionally and read nothing then).
  constexpr uint32_t kTileBytes = 16 * D * 2;
  auto k_rsrc = [&](bool valid, int64_t o) {
    return tile_rsrc(k_pool + (valid ? o : 0), valid ? kTileBytes : 0u);
  };
  auto v_rsrc = [&](bool valid, int64_t o) {
    return tile_rsrc(v_pool + (valid ? o : 0), valid ? kTileBytes : 0u);
  };
  // Refill cursor: the stream pair (cs, ck), (cs, ck + 1) that A and B load
  // next (ck even; every segment has an even number of positions).
  int cs = 0, ck = 0, cn = n0;
  auto cursor_skip = [&]() {  // move past exhausted segments
    while (cs < nseg && ck >= ((cn + 1) & ~1)) {
      ck -= (cn + 1) & ~1;
      ++cs;
      cn = cs < nseg ? nbw_of(seg_at(cs)) : 0;
    }
  };
  auto cursor_advance = [&]() {
    ck += 2;
    cursor_skip();
  };
  // The first pair of segment 0 (loaded above); a wave without blocks there
  // starts with the next segment's first pair.
  if (n0 == 0) {
    cursor_skip();
    if constexpr (kEarlyRefill) {
      const bool ra = cs < nseg && ck < cn, rb = cs < nseg && ck + 1 < cn;
      const int64_t oa = ra ? tile_off(cs, ck) : 0, obb = rb ? tile_off(cs, ck + 1) : 0;
      load_k<D>(A, k_rsrc(ra, oa), lane);
      load_v<D>(A, v_rsrc(ra, oa), lane);
      load_k<D>(B, k_rsrc(rb, obb), lane);
      load_v<D>(B, v_rsrc(rb, obb), lane);
    } else if (cs < nseg && ck < cn) {
      const int64_t o = tile_off(cs, ck);
      load_k<D>(A, k_pool + o, lane);
      load_v<D>(A, v_pool + o, lane);
    }
  }
  cursor_advance();  // the cursor now points at the pair after the first one

  WaveState<D, G> st;
  for (int s = 0; s < nseg; ++s) {
    const SegInfo sg = seg_at(s);
    const int i = sg.u / num_kv_heads, g = sg.u - i * num_kv_heads;
    const int ctx = sg.ctx;
    const int nblk_u = (ctx + 15) >> 4;
    const bool whole = sg.jb == 0 && sg.je == nblk_u;
    const int buf = s & 1;
    const uint16_t* qs = s_q[buf];
    const bool owner = APPEND && sg.je == nblk_u;
    const bool subst = owner && s_subst[buf];
    const uint16_t* knew = subst ? s_new[buf] : nullptr;
    const uint16_t* vnew = subst ? s_new[buf] + D : nullptr;
    // the next segment's query and appended rows travel during this one
    uint4 qnext[QPT];
    NewRows rnext{uint4{0u, 0u, 0u, 0u}, uint4{0u, 0u, 0u, 0u}, 0};
    if (s + 1 < nseg) {
      const SegInfo sn = seg_at(s + 1);
      fetch_q(sn, qnext);
      rnext = fetch_new(sn);
    }

    wave_init(st);
    const int nbw = nbw_of(sg);
    auto tok_of = [&](int kk) { return (sg.jb + wave + kWaves * kk) * 16; };
    if constexpr (kEarlyRefill) {
      // Block k of this segment is in A, k + 1 in B; the cursor names the
      // pair they are refilled with (possibly in a following segment),
      // through buffer resources that are empty where it has no block.  No
      // branch around a load and no exit in the middle of a trip (either
      // makes the compiler drain the prefetch at the top of the loop); an
      // odd last block after the loop, with B refilled there.
      int k = 0;
      for (; k + 1 < nbw; k += 2) {
        const bool ra = cs < nseg && ck < cn;
        const bool rb = cs < nseg && ck + 1 < cn;
        const int64_t oa = ra ? tile_off(cs, ck) : 0;
        const int64_t obb = rb ? tile_off(cs, ck + 1) : 0;
        cursor_advance();
        const auto ka = k_rsrc(ra, oa), va = v_rsrc(ra, oa);
        const auto kb = k_rsrc(rb, obb), vb = v_rsrc(rb, obb);
        block_scores<D, G>(A, qs, st, tok_of(k), ctx, scale_log2, s_p[wave], knew, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_k<D>(A, ka, lane);
        block_pv<D, G>(A, st, tok_of(k), ctx, s_p[wave], vnew, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_v<D>(A, va, lane);
        block_scores<D, G>(B, qs, st, tok_of(k + 1), ctx, scale_log2, s_p[wave], knew, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_k<D>(B, kb, lane);
        block_pv<D, G>(B, st, tok_of(k + 1), ctx, s_p[wave], vnew, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_v<D>(B, vb, lane);
      }
      if (k < nbw) {
        // odd count: position k + 1 is this segment's empty slot
        const bool ra = cs < nseg && ck < cn;
        const bool rb = cs < nseg && ck + 1 < cn;
        const int64_t oa = ra ? tile_off(cs, ck) : 0;
        const int64_t obb = rb ? tile_off(cs, ck + 1) : 0;
        cursor_advance();
        const auto ka = k_rsrc(ra, oa), va = v_rsrc(ra, oa);
        const auto kb = k_rsrc(rb, obb), vb = v_rsrc(rb, obb);
        block_scores<D, G>(A, qs, st, tok_of(k), ctx, scale_log2, s_p[wave], knew, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_k<D>(A, ka, lane);
        block_pv<D, G>(A, st, tok_of(k), ctx, s_p[wave], vnew, lane);
        __builtin_amdgcn_sched_barrier(0);
        load_v<D>(A, va, lane);
        load_k<D>(B, kb, lane);
        load_v<D>(B, vb, lane);
      }
    } else {
      for (int k = 0; k < nbw; k += 2) {
        const bool ra = cs < nseg && ck < cn;
        const int64_t oa = ra ? tile_off(cs, ck) : 0;
        cursor_advance();
        // B takes block k + 1 (this pair) before A is computed; A takes the
        // cursor's first position before B is computed
        if (k + 1 < nbw) {
          const int64_t o = tile_off(s, k + 1);
          load_k<D>(B, k_pool + o, lane);
          load_v<D>(B, v_pool + o, lane);
        }
        block_scores<D, G>(A, qs, st, tok_of(k), ctx, scale_log2, s_p[wave], knew, lane);
        block_pv<D, G>(A, st, tok_of(k), ctx, s_p[wave], vnew, lane);
        if (ra) {
          load_k<D>(A, k_pool + oa, lane);
          load_v<D>(A, v_pool + oa, lane);
        }
        if (k + 1 >= nbw) break;
        block_scores<D, G>(B, qs, st, tok_of(k + 1), ctx, scale_log2, s_p[wave], knew, lane);
        block_pv<D, G>(B, st, tok_of(k + 1), ctx, s_p[wave], vnew, lane);
      }
    }

    // merge the 4 waves of this segment
    wave_store<D, G>(st, s_acc[wave], s_m[wave], s_l[wave], lane);
    if (s + 1 < nseg) {
      stage_q(qnext, buf ^ 1);
      stage_new(rnext, buf ^ 1);
    }
    __syncthreads();
    const int64_t piece = (int64_t)sg.u + w;  // slot of a split unit's piece
    for (int idx = tid; idx < G * D; idx += 64 * kWaves) {
      const int h = idx / D, e = idx - h * D;
      float M = -__builtin_huge_valf();
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) {
        if (s_l[ww][h] > 0.f) {
          const float wt = fast_exp2(s_m[ww][h] - M);
          L += wt * s_l[ww][h];
          O += wt * s_acc[ww][h][e];
        }
      }
      if (whole) {
        const int64_t row_head = (int64_t)i * num_q_heads + g * G + h;
        out[row_head * D + e] = __builtin_bit_cast(uint16_t, (f16)(O / L));
      } else {
        const int64_t pidx = piece * G + h;
        part_o[pidx * D + e] = O / L;
        if (e == 0) {
          part_ml[pidx * 2] = M;
          part_ml[pidx * 2 + 1] = L;
        }
      }
    }
    if constexpr (APPEND) {
      // the appended rows go to their slot (only this piece reads the block)
      if (owner) {
        const int64_t slot = slot_mapping[i];
        if (slot >= 0 && (slot >> 4) < num_blocks) {
          const int64_t dst = (((slot >> 4) * num_kv_heads + g) * 16 + (slot & 15)) * D;
          if (tid < RCH)
            reinterpret_cast<uint4*>(k_pool + dst)[tid] =
                reinterpret_cast<const uint4*>(s_new[buf])[tid];
          else if (tid >= 64 && tid < 64 + RCH)
            reinterpret_cast<uint4*>(v_pool + dst)[tid - 64] =
                reinterpret_cast<const uint4*>(s_new[buf] + D)[tid - 64];
        }
      }
    }
    __syncthreads();  // s_acc / s_m / s_l reused by the next segment
  }
}

// Merge of the pieces of split units: one 4-wave work-group per (unit, query
// head of its group).
template <int D, int G>
__global__ __launch_bounds__(256) void piece_merge_kernel(
    const int32_t* __restrict__ sched, int32_t U, int32_t nwg, int32_t num_kv_heads,
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    uint16_t* __restrict__ out) {
  merge::piece_merge_unit<D>(sched, U, nwg, num_kv_heads, G, part_o, part_ml, out,
                             (int32_t)blockIdx.x, (int32_t)blockIdx.y);
}

template <int D, int G, bool APPEND>
hipError_t launch_sched_dga(const void* q, void* k_pool, void* v_pool, int64_t num_blocks,
                            int32_t num_kv_heads, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, int32_t num_decode_seqs, float scale,
                            const DecodeSchedulePlan& plan, const void* schedule,
                            const DecodeAppend& app, void* out, void* workspace,
                            hipStream_t stream, DecodeMerge* defer) {
  const int32_t* sched = static_cast<const int32_t*>(schedule);
  float* part_o = static_cast<float*>(workspace);
  const int64_t pieces = (int64_t)num_decode_seqs * num_kv_heads + plan.num_groups;
  float* part_ml = part_o + (size_t)pieces * G * D;
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  const int32_t U = num_decode_seqs * num_kv_heads;
  const int32_t app_groups = APPEND ? append_groups(app.num_tokens - num_decode_seqs) : 0;
  hipLaunchKernelGGL((paged_decode_sched_kernel<D, G, APPEND>), dim3(plan.num_groups + app_groups),
                     dim3(64 * kWaves), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), num_blocks,
                     num_kv_heads, block_tables, max_blocks_per_seq, sched, U, plan.num_groups,
                     scale * kLog2e,
                     static_cast<uint16_t*>(out), part_o, part_ml,
                     static_cast<const uint16_t*>(app.k_new),
                     static_cast<const uint16_t*>(app.v_new), app.slot_mapping, num_decode_seqs,
                     app.num_tokens);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (defer) {
    DecodeMerge m;
    m.groups = U * G;
    m.pieces = true;
    m.part_o = part_o;
    m.part_ml = part_ml;
    m.sched = sched;
    m.units = U;
    m.sched_groups = plan.num_groups;
    m.num_kv_heads = num_kv_heads;
    m.group = G;
    *defer = m;
    return hipSuccess;
  }
  hipLaunchKernelGGL((piece_merge_kernel<D, G>),
                     dim3((uint32_t)U, G), dim3(256), 0, stream, sched, U, plan.num_groups,
                     num_kv_heads, part_o, part_ml, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

template <int D>
hipError_t launch_sched_d(int32_t group, const void* q, void* k_pool, void* v_pool,
                          int64_t num_blocks, int32_t num_kv_heads, const int32_t* bt,
                          int32_t maxblk, int32_t nseq, float scale,
                          const DecodeSchedulePlan& plan, const void* schedule,
                          const DecodeAppend& app, void* out, void* ws, hipStream_t stream,
                          DecodeMerge* defer) {
  const bool fused = app.k_new != nullptr;
#define PKV_CASE(GG)                                                                         \
  case GG:                                                                                  \
    return fused ? launch_sched_dga<D, GG, true>(q, k_pool, v_pool, num_blocks, num_kv_heads, \
                                                 bt, maxblk, nseq, scale, plan, schedule,   \
                                                 app, out, ws, stream, defer)               \
                 : launch_sched_dga<D, GG, false>(q, k_pool, v_pool, num_blocks,            \
                                                  num_kv_heads, bt, maxblk, nseq, scale,    \
                                                  plan, schedule, app, out, ws, stream,     \
                                                  defer);
  switch (group) {
    PKV_CASE(1) PKV_CASE(2) PKV_CASE(3) PKV_CASE(4)
    PKV_CASE(5) PKV_CASE(6) PKV_CASE(7) PKV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef PKV_CASE
}

}  // namespace

DecodeSchedulePlan plan_decode_schedule(int32_t num_decode_seqs, int32_t num_kv_heads,
                                        int32_t num_q_heads, int32_t head_dim,
                                        int32_t max_context_len) {
  DecodeSchedulePlan plan{};
  const int32_t U = num_decode_seqs * num_kv_heads;
  // d = 256 keeps the partition grid: its long contexts already stream near
  // the memory's rate there, and the kernel would not fit 2 waves per SIMD
  if (head_dim != 128) return plan;
  if (U <= 0 || U > kMaxSchedUnits) return plan;  // not schedulable: partition path
  const int64_t max_blocks = (max_context_len + 15) / 16;
  const int64_t w_max = (int64_t)U * (max_blocks + kSegCost);
  if (w_max >= INT32_MAX / 2) return plan;
  // one resident round of 4-wave work-groups, more when a range would hold
  // more blocks than the kernel stages, or more segments than it tracks
  // A range of R = ceil(W / NWG) cost units meets at most R / (kSegCost + 1)
  // + 2 units and holds at most R blocks.
  int64_t nwg = 512;
  nwg = std::max<int64_t>(nwg, (w_max + kMaxWgBlocks - 2) / (kMaxWgBlocks - 1));
  nwg = std::max<int64_t>(nwg, (w_max + (kMaxSegs - 3) * (kSegCost + 1) - 1) /
                                   ((kMaxSegs - 3) * (kSegCost + 1)));
  if (nwg > INT32_MAX / 4) return plan;
  plan.num_groups = (int32_t)nwg;
  plan.schedule_bytes = (size_t)sched_words(U, plan.num_groups) * sizeof(int32_t);
  plan.partial_bytes = (size_t)(U + nwg) * (num_q_heads / num_kv_heads) * (head_dim + 2) *
                       sizeof(float);
  return plan;
}

hipError_t launch_decode_schedule(const int32_t* context_lens, int32_t num_decode_seqs,
                                  int32_t num_kv_heads, int32_t ctx_clamp,
                                  const DecodeSchedulePlan& plan, void* schedule,
                                  hipStream_t stream) {
  (void)hipGetLastError();  // drop errors left by earlier runtime calls
  hipLaunchKernelGGL(decode_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream,
                     context_lens, num_decode_seqs, num_kv_heads, ctx_clamp, plan.num_groups,
                     static_cast<int32_t*>(schedule));
  return hipGetLastError();
}

hipError_t launch_paged_decode_scheduled(const void* q, void* k_pool, void* v_pool,
                                         int64_t num_blocks, int32_t num_kv_heads,
                                         int32_t num_q_heads, int32_t head_dim,
                                         const int32_t* block_tables,
                                         int32_t max_blocks_per_seq, int32_t num_decode_seqs,
                                         float scale, const DecodeSchedulePlan& plan,
                                         const void* schedule, const DecodeAppend& app,
                                         void* out, void* workspace, hipStream_t stream,
                                         DecodeMerge* defer) {
  if (num_decode_seqs == 0) return hipSuccess;
  const int32_t group = num_q_heads / num_kv_heads;
  if (head_dim == 128)
    return launch_sched_d<128>(group, q, k_pool, v_pool, num_blocks, num_kv_heads,
                               block_tables, max_blocks_per_seq, num_decode_seqs, scale, plan,
                               schedule, app, out, workspace, stream, defer);
  return hipErrorInvalidValue;
}

}  // namespace pkv
