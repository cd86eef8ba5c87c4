/*
 * pkv_sched.h -- C ABI of the host-side block manager and per-pass scheduler
 * in libpkv.so: the step before the attention path, which decides for every
 * forward pass which sequences run, how many new tokens each brings, and in
 * which cache blocks those tokens live -- the block tables, context lengths,
 * query offsets and slot mapping that pkv_paged_attention_step and
 * pkv_append_attention_step (pkv.h) consume.
 *
 * What it follows (deepconcepts.dev, "Continuous Batching Is Not a Bigger
 * Batch"):
 *   - section "What the scheduler does on one step": membership is decided
 *     again before every pass.  Phase one walks the running requests in
 *     arrival order; each asks for its next tokens -- one when decoding, the
 *     rest of its prompt capped by the pass's token budget when prefilling
 *     (chunked prefill) -- and the cache manager allocates the blocks those
 *     tokens need.  When an allocation fails the newest running request is
 *     preempted: its blocks are freed, its computed-token count goes back to
 *     zero (it will prefill again, prompt and generated tokens alike) and it
 *     goes to the front of the waiting queue; if the request being scheduled
 *     is itself the newest, it is the one preempted.  Phase two admits
 *     waiting requests in order while the token budget lasts and the running
 *     count is below max_num_seqs -- and only in a pass that preempted
 *     nobody.  max_num_seqs is read nowhere else: a ceiling on admission.
 *   - section "The allocator is the other half": cache is allocated in fixed
 *     16-token blocks on demand (a request holds ceil(tokens / 16) blocks),
 *     or, with PKV_ALLOC_RESERVE, reserved up front for the prompt plus the
 *     declared maximum output at admission (never preempts).
 *   - section "Where the batch size actually comes from": the pool is a
 *     whole number of blocks; what fits is the arithmetic of blocks held.
 *   - prefix caching ("What the scheduler does on one step", the note on
 *     recompute): requests that declare the same prefix id share the full
 *     blocks of their common prefix while any of them is resident (the
 *     blocks are reference-counted and aliased in every sharer's table; a
 *     sharer starts with those tokens computed).  A shared block is never
 *     appended to: new tokens always land past the shared full blocks.
 *
 * Everything here is host memory and host code; nothing touches a GPU.  The
 * scheduler owns its state and the arrays of its last plan; the caller owns
 * nothing it passes in beyond the call.  Not thread-safe: one scheduler per
 * thread, or external locking.  Errors are return codes (pkv_status of
 * pkv.h); nothing aborts or prints.
 */
#ifndef PKV_SCHED_H
#define PKV_SCHED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_scheduler pkv_scheduler;

enum { PKV_ALLOC_ON_DEMAND = 0, PKV_ALLOC_RESERVE = 1 };

typedef struct {
  int64_t num_blocks;          /* blocks in the pool (>= 1) */
  int32_t block_size;          /* must be 16 */
  int32_t max_num_seqs;        /* admission ceiling on running requests (>= 1) */
  int32_t max_num_batched_tokens; /* token budget of one pass (>= 1) */
  int32_t max_blocks_per_seq;  /* width of the block tables the plan returns; a
                                  request needing more is rejected at add */
  int32_t alloc_policy;        /* PKV_ALLOC_ON_DEMAND or PKV_ALLOC_RESERVE */
} pkv_sched_config;

/*
 * The plan of one pass.  Arrays are owned by the scheduler and stay valid
 * until the next pkv_sched_schedule or pkv_sched_destroy.  Scheduled
 * sequences are ordered as the attention step wants them: the ones with one
 * new token first (decodes, and prefills with one prompt token left), then
 * the chunks, each group in running order.
 */
typedef struct {
  int32_t num_seqs;            /* sequences in the pass (B) */
  int32_t num_decode_seqs;     /* the first num_decode_seqs have one new token */
  int32_t num_tokens;          /* T = sum of new tokens */
  int32_t max_context_len;     /* max context_lens (0 when B = 0) */
  int32_t max_query_len;       /* max new tokens of a sequence (0 when B = 0) */
  const int64_t* request_ids;  /* [B] */
  const int32_t* context_lens; /* [B] computed + new tokens (after this pass's append) */
  const int32_t* query_start_loc; /* [B+1] */
  const int32_t* block_tables; /* [B][max_blocks_per_seq]; entries past
                                  ceil(ctx / 16) are 0 */
  const int64_t* slot_mapping; /* [T] slot of every new token */
  /* what the pass did */
  int32_t num_preempted;       /* requests preempted in this pass */
  int32_t num_admitted;        /* requests admitted from the waiting queue */
  int64_t recomputed_tokens;   /* computed tokens discarded by this pass's preemptions */
  int64_t prefix_hit_tokens;   /* tokens admitted as already computed via shared prefixes */
} pkv_sched_plan;

/* Cumulative counters and the pool's state. */
typedef struct {
  int64_t passes;
  int64_t preemptions;
  int64_t recomputed_tokens;
  int64_t prefix_hit_tokens;
  int64_t generated_tokens;
  int32_t peak_running;
  int32_t num_running;
  int32_t num_waiting;
  int32_t num_finished;
  int64_t free_blocks;
} pkv_sched_stats;

/*
 * New scheduler; NULL on invalid configuration (or out of host memory).
 *   free_order   host int32 [num_blocks], a permutation of 0 .. num_blocks-1:
 *                the initial order of the free-block queue (blocks are taken
 *                from its front, freed blocks join its back); NULL = 0, 1, ...
 *                Copied; not a permutation -> NULL is returned.
 */
pkv_scheduler* pkv_sched_create(const pkv_sched_config* config, const int32_t* free_order);
void pkv_sched_destroy(pkv_scheduler* s);

/*
 * Queue a request (it arrives after every request added before it).
 *   prompt_len       >= 1 prompt tokens
 *   max_new_tokens   >= 1 tokens to generate before it finishes
 *   prefix_id        < 0: none; otherwise requests with the same id share the
 *                    first prefix_len tokens of their prompt
 *   prefix_len       0 .. prompt_len - 1 (only whole 16-token blocks are shared)
 * Errors: PKV_ERR_INVALID_ARG (bad lengths, duplicate id, the request could
 * never fit the table width or the pool).
 */
int pkv_sched_add_request(pkv_scheduler* s, int64_t request_id, int32_t prompt_len,
                          int32_t max_new_tokens, int64_t prefix_id, int32_t prefix_len);

/*
 * Plan the next pass.  *plan receives the pass (num_seqs = 0 when nothing
 * can run).  Must be followed by pkv_sched_complete before the next
 * pkv_sched_schedule.  Errors: PKV_ERR_INVALID_ARG (NULL, or a plan still
 * outstanding).
 */
int pkv_sched_schedule(pkv_scheduler* s, pkv_sched_plan* plan);

/*
 * The planned pass has run: every scheduled sequence has its new tokens
 * computed; a sequence whose computed tokens reach its total (prompt plus
 * tokens generated so far) samples one more token, and one that has
 * generated max_new_tokens finishes and frees its blocks.
 * Errors: PKV_ERR_INVALID_ARG (no plan outstanding).
 */
int pkv_sched_complete(pkv_scheduler* s);

int pkv_sched_get_stats(const pkv_scheduler* s, pkv_sched_stats* stats);

/*
 * Blocks currently held by a request (in logical order) into out[cap];
 * returns the count (may exceed cap), or -1 when the id is unknown or the
 * request holds nothing.  For tests and inspection.
 */
int64_t pkv_sched_request_blocks(const pkv_scheduler* s, int64_t request_id, int32_t* out,
                                 int64_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PKV_SCHED_H */
