/*
 * pkv.h -- C ABI of libpkv.so: paged KV append + paged attention step for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  A continuous-batching engine re-forms its
 * batch before every forward pass: each running sequence brings its
 * num_new_tokens (one for a decoding sequence, a chunk of the prompt for a
 * prefilling one) on top of num_computed_tokens, and the cache manager
 * allocates cache slots for them before the pass runs (deepconcepts.dev,
 * "Continuous Batching Is Not a Bigger Batch", section "What the scheduler
 * does on one step").  The KV cache is held in fixed 16-token blocks
 * (same page, section "The allocator is the other half"), so a sequence's
 * cache is a list of physical blocks in logical order -- its block table --
 * and a paged cache stores only real tokens (danielfleming.xyz, "Static
 * batching", section "Ragged batches").  Every sequence carries one key and
 * one value vector per token per layer ("Continuous Batching Is Not a Bigger
 * Batch", introduction), with fewer KV heads than query heads (grouped-query
 * attention, section "Where the batch size actually comes from").
 *
 * One step of one layer is:
 *   0. pkv_decode_schedule -- balanced split of the decode work over the
 *      GPU (optional; shared by all layers of the step);
 *   1. pkv_slot_mapping  -- pool slot of every new token (shared by all layers);
 *   2. pkv_kv_append     -- write each new token's K/V rows into its slot;
 *   3. pkv_paged_attention_step -- every new query token attends its own
 *      context through the block table: decode sequences (one token each)
 *      over their whole context, prefill chunks causally.
 * pkv_append_attention_step does 2 and 3 in one call with the same result,
 * appending the decode tokens inside the decode kernel (one launch fewer
 * per layer).
 *
 * Conventions shared by every entry point.
 *   - "device" pointers are GPU memory (hipMalloc / torch CUDA tensors),
 *     "host" pointers are CPU memory.  The caller owns every buffer; the
 *     library allocates nothing and keeps no per-call state.
 *   - fp16 is IEEE binary16.  Integer arrays are little-endian, C order.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every GPU
 *     entry point only enqueues work on `stream` and returns; it never
 *     synchronises and never reads device memory from the host.
 *   - Entry points validate their host-side scalars and pointers and return
 *     a pkv_status; on any error nothing is enqueued.  They never abort and
 *     never print.  Contents of device arrays (block ids, lengths, slots)
 *     are a caller contract, checked only by pkv_validate_step; kernels
 *     clamp block ids into the pool so that a broken contract gives wrong
 *     numbers, not a memory fault.
 *   - Context lengths include this step's new tokens: the append runs
 *     first, then the attention reads the just-written tokens.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ABI version.  2: a mixed step's workspace holds the chunks' partials after
 * the decode part's (pkv_attention_workspace_size grew accordingly), and
 * pkv_validate_step reports code 10. */
#define PKV_VERSION 2

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shapes      */
  PKV_ERR_UNSUPPORTED = -2, /* block_size != 16, head_dim not 128/256, group > 8     */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required          */
  PKV_ERR_HIP = -4,         /* a HIP launch or runtime call failed                 */
  PKV_ERR_CONTRACT = -5     /* pkv_validate_step found a device-content violation  */
} pkv_status;

/* Element type of a KV cache (pkv_kv_cache.kv_dtype). */
enum {
  PKV_KV_FP16 = 0,     /* IEEE binary16 values */
  PKV_KV_FP8_E4M3 = 1  /* 8-bit codes + one fp32 scale per (token, KV head) row */
};

/*
 * One layer's paged KV cache.  k_pool and v_pool are device arrays of shape
 * [num_blocks][num_kv_heads][block_size][head_dim]: one block of one KV head
 * is block_size * head_dim contiguous values (4 KiB at d = 128 in fp16).
 * Physical block b of KV head g holds the rows of block_size consecutive
 * token positions of whichever sequence owns b.  Owned by the caller.
 *
 * kv_dtype PKV_KV_FP8_E4M3 (a quantized cache: 8-bit KV halves the bytes of
 * a window, "before scales" -- a8q9.cn, "An advertised batch limit proves
 * nothing until sampled"): the pools hold OCP FP8 E4M3 codes (1 byte per
 * value: sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite
 * 448), and k_scale / v_scale are device fp32 arrays [num_blocks]
 * [num_kv_heads][block_size]: row (b, g, o) stands for code value x
 * scale[b][g][o].  pkv_kv_append writes each new row with the smallest
 * power-of-two scale 2^e such that max|x| <= 448 x 2^e (1 for a zero row)
 * and codes x / 2^e rounded to nearest, ties to even.  For fp16 caches
 * kv_dtype is 0 and the scale pointers are ignored.
 */
typedef struct {
  void* k_pool;
  void* v_pool;
  int64_t num_blocks;
  int32_t block_size;   /* must be 16 */
  int32_t num_kv_heads; /* >= 1 */
  int32_t head_dim;     /* 128 or 256 */
  int32_t kv_dtype;     /* PKV_KV_FP16 or PKV_KV_FP8_E4M3 */
  void* k_scale;        /* fp8: fp32 [num_blocks][num_kv_heads][block_size] */
  void* v_scale;
} pkv_kv_cache;

/* Library version (PKV_VERSION of the build). */
int pkv_version(void);

/* Static string naming a pkv_status value ("PKV_OK", ...). */
const char* pkv_status_string(int status);

/*
 * The HIP runtime error (hipError_t value) behind the most recent
 * PKV_ERR_HIP returned on the calling thread, 0 if none; when `name` is not
 * NULL it receives the runtime's static error string.  Host only.
 */
int pkv_last_hip_error(const char** name);

/*
 * Slot of every new token of the step (deepconcepts.dev, "Continuous
 * Batching Is Not a Bigger Batch", "What the scheduler does on one step":
 * new tokens sit on top of the computed ones, in blocks the cache manager
 * allocated).  For sequence i with n_i new tokens and context length ctx_i,
 * new token k is at logical position p = ctx_i - n_i + k and its slot is
 *     block_tables[i][p / block_size] * block_size + p % block_size.
 *
 *   block_tables     device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens     device int32 [num_seqs], ctx_i >= n_i
 *   query_start_loc  device int32 [num_seqs + 1], row of sequence i's first
 *                    new token; n_i = qsl[i+1] - qsl[i].  NULL: every
 *                    sequence has exactly one new token in row i.
 *   slot_mapping     device int64 [num_tokens] (output); a position that
 *                    falls outside its table row gets slot -1 (skipped by
 *                    pkv_kv_append).
 *   num_tokens       total new tokens (= qsl[num_seqs], or num_seqs when
 *                    query_start_loc is NULL).
 * Errors: PKV_ERR_INVALID_ARG (null pointer, negative size),
 * PKV_ERR_UNSUPPORTED (block_size != 16), PKV_ERR_HIP.
 */
int pkv_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, const int32_t* query_start_loc,
                     int32_t num_seqs, int32_t num_tokens, int32_t block_size,
                     int64_t* slot_mapping, void* stream);

/*
 * KV append: for every token t with slot_mapping[t] >= 0, copy the
 * num_kv_heads x head_dim values of k_new[t] into
 * k_pool[slot / block_size][g][slot % block_size][:] for every KV head g,
 * and v_new[t] into v_pool likewise.  Bit-exact copy; slots < 0 are
 * padding and are skipped; slots beyond the pool are skipped too (a broken
 * contract, reported by pkv_validate_step).  Duplicate slots race.
 *
 *   cache         the layer's pools (device)
 *   k_new, v_new  device fp16 [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping  device int64 [num_tokens]
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP.
 */
int pkv_kv_append(const pkv_kv_cache* cache, const void* k_new, const void* v_new,
                  const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/*
 * Bytes of device workspace pkv_paged_attention_step needs for a step of
 * this shape (written to *bytes).  The same host-side hints must be passed
 * to the step.  Pure host function: touches no GPU.
 *
 *   num_seqs, num_decode_seqs   sequences in the step; the first
 *                               num_decode_seqs have one new token each
 *   num_q_heads, num_kv_heads, head_dim
 *   max_context_len             >= every ctx_i
 *   max_query_len               >= every n_i (1 for a pure decode step)
 *   kv_partition_tokens         0 = automatic; otherwise force this many
 *                               context tokens per split-KV partition of
 *                               the decode sequences and of packed short
 *                               chunks (multiple of 64)
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED.
 */
int pkv_attention_workspace_size(int32_t num_seqs, int32_t num_decode_seqs,
                                 int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t max_query_len, int32_t kv_partition_tokens,
                                 size_t* bytes);

/*
 * Bytes of the per-step decode schedule buffer for these host hints (0 when
 * the step is not schedulable: head_dim 256 (which keeps the partition
 * grid), more than 16,384 (sequence, KV head) units, or no decode
 * sequence).  Pure host function.
 */
int pkv_decode_schedule_size(int32_t num_decode_seqs, int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_context_len, size_t* bytes);

/*
 * Balanced schedule of the decode work of one step (danielfleming.xyz,
 * "Static batching", section "Ragged batches": a ragged mix should cost only
 * its real tokens).  Every (decode sequence, KV head) pair is a unit of
 * ceil(ctx_i / 16) blocks; the units are laid end to end and cut into equal
 * shares, one per decode work-group, so that short contexts are packed
 * together and only long ones are split (and merged by log-sum-exp).  It
 * depends only on the context lengths, so one schedule serves every layer
 * of the step: build it once per step (after the context lengths are final,
 * on the same stream), pass it to pkv_paged_attention_step /
 * pkv_append_attention_step with the same num_decode_seqs, num_kv_heads,
 * head_dim and max_context_len.
 *
 *   context_lens   device int32 [num_decode_seqs] (the step's, including the
 *                  new token); read on the device only
 *   schedule       device buffer of pkv_decode_schedule_size bytes (written)
 * One launch of one work-group.  Does nothing when the size is 0.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_WORKSPACE (buffer too small),
 * PKV_ERR_HIP.
 */
int pkv_decode_schedule(const int32_t* context_lens, int32_t num_decode_seqs,
                        int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                        int32_t max_context_len, void* schedule, size_t schedule_bytes,
                        void* stream);

/*
 * Paged attention over one layer for every new token of the step.
 *
 * Query row r of sequence i (row r = qsl[i] + k, k < n_i) sits at position
 * pos = ctx_i - n_i + k and, for query head h, computes
 *     out[r][h] = softmax_p( scale * q[r][h] . K_i[p][g] ) V_i[p][g],
 *                 p = 0 .. pos,  g = h / (num_q_heads / num_kv_heads),
 * where K_i[p] / V_i[p] are read from the pools through block_tables[i]
 * (position p in table entry p / 16 at offset p % 16).  Decode sequences
 * (the first num_decode_seqs, one token each) attend their whole context;
 * the others are prefill chunks, attended causally.  Context positions at or
 * beyond ctx_i, and table entries past ceil(ctx_i / 16), are never used,
 * whatever they hold (NaN included).
 *
 *   cache            the layer's pools (device)
 *   q                device fp16 [num_tokens][num_q_heads][head_dim]
 *   out              device fp16 [num_tokens][num_q_heads][head_dim], written
 *                    with round-to-nearest-even from fp32 accumulation
 *   block_tables     device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens     device int32 [num_seqs]
 *   query_start_loc  device int32 [num_seqs + 1], or NULL when every
 *                    sequence is a decode sequence (row i = sequence i)
 *   num_seqs, num_decode_seqs, num_q_heads, scale
 *   max_context_len, max_query_len, kv_partition_tokens
 *                    host hints, as for pkv_attention_workspace_size; the
 *                    split-KV plan is made from these alone (no device read)
 *   schedule, schedule_bytes
 *                    the step's pkv_decode_schedule buffer, or NULL / 0.  With
 *                    a schedule, decode contexts that would be cut into
 *                    partitions run on the balanced schedule instead; when
 *                    every (sequence, KV head) fits one work-group the plain
 *                    grid is used either way.  Ignored when
 *                    kv_partition_tokens forces a partition size.
 *   workspace        device buffer of at least the size that
 *                    pkv_attention_workspace_size reports (may be NULL when
 *                    that size is 0); contents need not be initialised and
 *                    are undefined afterwards.  Calls that share one
 *                    workspace must be ordered on one stream.
 * Launches: the decode kernel (grid over sequence x KV head x partition, or
 * one work-group per schedule share), the log-sum-exp merge of partitions or
 * pieces when any context is split, and the MFMA prefill kernel (+ its merge)
 * when prefill chunks are present -- short chunks (max_query_len x
 * num_q_heads / num_kv_heads <= 64, e.g. a decoding sequence verifying a few
 * drafted tokens) with all query heads of a KV head packed into one
 * work-group; all on `stream`.
 * Over an fp8 cache the decode part always uses the partition grid (the
 * schedule is ignored), and the prefill kernel turns the codes it stages
 * into fp16 (exact) and applies the row scales to the scores (K) and to the
 * softmax weights (V); the result is attention over the dequantized cache.
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE,
 * PKV_ERR_HIP.
 */
int pkv_paged_attention_step(const pkv_kv_cache* cache, const void* q, void* out,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, const int32_t* query_start_loc,
                             int32_t num_seqs, int32_t num_decode_seqs,
                             int32_t num_q_heads, float scale,
                             int32_t max_context_len, int32_t max_query_len,
                             int32_t kv_partition_tokens, const void* schedule,
                             size_t schedule_bytes, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * pkv_kv_append(cache, k_new, v_new, slot_mapping, num_tokens) followed by
 * pkv_paged_attention_step(cache, q, out, ...) in one call, with the same
 * result in the pools and in `out`.  A step's tokens are written into the
 * cache before they are attended (deepconcepts.dev, "Continuous Batching Is
 * Not a Bigger Batch", "What the scheduler does on one step"), and the many
 * small GPU launches of a pass are a cost of their own, paid per pass
 * (danielfleming.xyz, "Static batching", section "What changed").
 *
 * The decode tokens (rows 0 .. num_decode_seqs-1) are appended by the
 * decode kernel itself: the work-group that reads the block holding
 * position ctx_i - 1 takes the new row from k_new / v_new instead of the
 * pool and writes it to slot_mapping[i] at its end.  Prefill tokens (rows
 * num_decode_seqs .. num_tokens-1) are appended by extra work-groups of the
 * same decode launch (by the append kernel when num_decode_seqs is 0), before
 * the prefill kernel runs.  Since the decode work-groups read the pools
 * meanwhile, a new token's slot must lie in a block that no other sequence's
 * context lists, as the block manager of pkv_sched.h hands them out
 * (pkv_validate_step code 10).  Over an fp8 cache both quantize the rows as
 * pkv_kv_append does.
 *
 *   k_new, v_new   device fp16 [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping   device int64 [num_tokens]; as for pkv_kv_append.  The
 *                  fused decode append assumes each decode token's slot is
 *                  either negative (skipped: the attention then reads the
 *                  pool's current row) or the slot that the block table
 *                  gives position ctx_i - 1 (what pkv_slot_mapping writes;
 *                  pkv_validate_step code 9); a slot elsewhere is written,
 *                  but the attention does not see it.
 *   num_tokens     rows of k_new / v_new / q (= qsl[num_seqs], or num_seqs
 *                  when query_start_loc is NULL); >= num_decode_seqs
 *   other arguments exactly as for pkv_paged_attention_step (schedule
 *                  included), with the same workspace size
 *                  (pkv_attention_workspace_size).
 * The rows of a sequence whose ctx_i < 1 are not written.
 * Errors: PKV_ERR_INVALID_ARG (also: k_new, v_new or slot_mapping NULL,
 * num_tokens inconsistent), PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE,
 * PKV_ERR_HIP.
 */
int pkv_append_attention_step(const pkv_kv_cache* cache, const void* k_new, const void* v_new,
                              const int64_t* slot_mapping, int32_t num_tokens, const void* q,
                              void* out, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              const int32_t* query_start_loc, int32_t num_seqs,
                              int32_t num_decode_seqs, int32_t num_q_heads, float scale,
                              int32_t max_context_len, int32_t max_query_len,
                              int32_t kv_partition_tokens, const void* schedule,
                              size_t schedule_bytes, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * pkv_append_attention_step for every layer of one step, in one call: for
 * l = 0 .. num_layers-1, in that order on `stream`, exactly
 *   pkv_append_attention_step(&caches[l], k_new[l], v_new[l], slot_mapping,
 *       num_tokens, q[l], out[l], block_tables, ...)
 * with the arguments after out[l] shared by all layers (block tables,
 * context lengths and slots are per step; the pools, new rows, queries and
 * outputs are per layer).  A step issues two to four small launches per
 * layer and the host cost of a layer's call is paid once per launch
 * (danielfleming.xyz, "Static batching", section "What changed": the kernel
 * launches of a pass cost more host time than the GPU spends); this entry
 * point leaves one call per step.
 *
 *   caches                  host array [num_layers] of cache descriptors
 *   k_new, v_new, q, out    host arrays [num_layers] of device pointers
 *   num_layers              >= 0 (0: nothing is launched)
 *   other arguments         as for pkv_append_attention_step; the one
 *                           workspace serves every layer (stream order).
 * Every argument is checked before the first launch: all layers'
 * descriptors and pointers, and each layer's plan (workspace and schedule
 * sizes, grid limits -- they depend on its heads and head_dim), so an
 * argument error enqueues nothing.  The first launch error stops the loop
 * and is returned (the layers before it are enqueued).
 * Errors: as for pkv_append_attention_step.
 */
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
                                void* stream);

/*
 * Bytes of the device scratch array behind pkv_append_attention_step_noalloc
 * (one copy per GPU the library runs on, held until the process ends).
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * pkv_append_attention_step without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * or harnesses that forbid hipMalloc.  The split-KV and prefill partials go
 * to a scratch array of PKV_NOALLOC_SCRATCH_BYTES inside the library's
 * device code instead of a caller-owned workspace; the kernels, the result
 * and every other argument are those of pkv_append_attention_step.  The
 * call allocates nothing.
 *
 *   all arguments   as for pkv_append_attention_step, without workspace and
 *                   workspace_bytes; the scratch of the current device is
 *                   used, so `stream` must belong to the current device.
 * Limit: a step whose pkv_attention_workspace_size (same hints) exceeds
 * PKV_NOALLOC_SCRATCH_BYTES is refused with PKV_ERR_WORKSPACE before any HIP
 * call.  Every call on one GPU shares that GPU's scratch, which keeps the
 * last call's partials: calls in stream order are safe, calls that overlap
 * on one GPU (other streams, other host threads) race.  The first call on a
 * device looks up that device's copy of the array; a failure there returns
 * PKV_ERR_HIP (pkv_last_hip_error names it).
 * Errors: as for pkv_append_attention_step.
 */
int pkv_append_attention_step_noalloc(const pkv_kv_cache* cache, const void* k_new,
                                      const void* v_new, const int64_t* slot_mapping,
                                      int32_t num_tokens, const void* q, void* out,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens,
                                      const int32_t* query_start_loc, int32_t num_seqs,
                                      int32_t num_decode_seqs, int32_t num_q_heads, float scale,
                                      int32_t max_context_len, int32_t max_query_len,
                                      int32_t kv_partition_tokens, const void* schedule,
                                      size_t schedule_bytes, void* stream);

/*
 * Work-groups of pkv_hbm_read_probe: the sink holds one word per work-group.
 */
#define PKV_PROBE_SINK_WORDS 4096

/*
 * HBM read-rate probe (measurement only; not part of a step).  Runs
 * `launches` launches back to back on `stream`; launch k reads tiles
 * tile_ids[k * num_tiles .. (k + 1) * num_tiles - 1] of `base` (tile t =
 * bytes [t * tile_bytes, (t + 1) * tile_bytes)) once each, in the listed
 * order, and folds the words it read into `sink`, one word per work-group.  With the block size of one
 * KV head as tile_bytes (4 KiB at head_dim 128, 8 KiB at 256) and the ids in
 * a random order over a buffer much larger than the last-level cache, it is
 * the paged decode's access pattern without its arithmetic: timed around
 * the launches, it gives the read rate HBM sustains for that pattern at
 * that launch size (each launch pays its own ramp and drain), the
 * measured denominator beside the 8 TB/s specification (danielfleming.xyz,
 * "Static batching", section "Where scaling stops, and why the prediction
 * missed": read rates reported as a share of peak).
 *
 *   base, base_bytes   device buffer (any content), >= tile_bytes
 *   tile_ids           device int32 [launches * num_tiles]; ids outside
 *                      [0, base_bytes / tile_bytes) are clamped into it
 *   tile_bytes         a power of two in [1024, 65536]
 *   launches           0 .. 4096
 *   sink               device uint32 [PKV_PROBE_SINK_WORDS], overwritten
 * Asynchronous on `stream`.  Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED,
 * PKV_ERR_HIP.
 */
int pkv_hbm_read_probe(const void* base, size_t base_bytes, const int32_t* tile_ids,
                       int64_t num_tiles, int32_t tile_bytes, int32_t launches, uint32_t* sink,
                       void* stream);

/*
 * Debug validator (host, synchronous, no GPU): checks on host copies of
 * the step's index arrays every device-content contract the hot path
 * assumes.  Returns PKV_OK, or PKV_ERR_CONTRACT with *bad_what set to one
 * of the codes below and *bad_index to the first offending sequence (or
 * token) index.  query_start_loc and slot_mapping may be NULL.
 *   1  ctx_i < 1
 *   2  ctx_i > max_blocks_per_seq * block_size
 *   3  ctx_i < n_i, or query_start_loc not non-decreasing / inconsistent
 *   4  a used block id (table entry < ceil(ctx_i / block_size)) outside
 *      [0, num_blocks)
 *   5  a decode sequence (i < num_decode_seqs) with n_i != 1
 *   6  a slot outside [0, num_blocks * block_size) (negative = skipped)
 *   7  two new tokens with the same non-negative slot
 *   8  max_context_len or max_query_len smaller than an actual length
 *   9  a non-negative slot that is not the table's slot of its token's
 *      position (ctx_i - n_i + k)
 *  10  a non-negative slot in a block that another sequence's context also
 *      lists (shared blocks are read-only: new tokens go to blocks that
 *      belong to one sequence)
 */
int pkv_validate_step(const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, const int32_t* query_start_loc,
                      int32_t num_seqs, int32_t num_decode_seqs, int64_t num_blocks,
                      int32_t block_size, const int64_t* slot_mapping, int32_t num_tokens,
                      int32_t max_context_len, int32_t max_query_len,
                      int32_t* bad_what, int64_t* bad_index);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
