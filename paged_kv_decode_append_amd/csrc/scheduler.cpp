// scheduler.cpp -- host-side block manager and per-pass scheduler
// (include/pkv_sched.h): decides every pass's sequences, their new tokens
// and the cache blocks those tokens live in, and hands the attention step its
// block tables, context lengths, query offsets and slot mapping.
//
// Rules (deepconcepts.dev, "Continuous Batching Is Not a Bigger Batch"):
//   "What the scheduler does on one step" -- two phases per pass.  Running
//     requests, in arrival order, ask for one token (decode) or the rest of
//     the prompt capped by the token budget (chunked prefill); a failed block
//     allocation preempts the newest running request (blocks freed, computed
//     tokens reset to zero, back to the front of the waiting queue), possibly
//     the requester itself.  Waiting requests are admitted only in a pass that
//     preempted nobody, while the budget lasts and the running count is below
//     max_num_seqs (the only place that setting is read).
//   "The allocator is the other half" -- fixed 16-token blocks allocated on
//     demand, or reserved up front for prompt + declared maximum output.
//   prefix caching (same section's note on recompute) -- full blocks of a
//     declared common prefix are shared, reference-counted, while resident.
// Free blocks are a FIFO queue (a freed block goes to the back; a request's
// blocks are freed last block first), initially in the caller's order (a
// permutation of the pool scatters the tables over it).
#include <stdint.h>

#include <algorithm>
#include <deque>
#include <new>
#include <numeric>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_sched.h"

namespace {

constexpr int32_t kBlockSize = 16;

int64_t blocks_for(int64_t tokens) { return (tokens + kBlockSize - 1) / kBlockSize; }

struct Request {
  int64_t id = 0;
  int32_t prompt_len = 0;
  int32_t max_new_tokens = 0;
  int64_t prefix_id = -1;
  int32_t prefix_len = 0;
  int32_t num_generated = 0;   // tokens sampled so far
  int64_t num_computed = 0;    // tokens whose K/V are in the cache
  std::vector<int32_t> blocks; // logical order
  bool finished = false;
  int64_t num_tokens() const { return (int64_t)prompt_len + num_generated; }
};

struct Scheduled {
  Request* req;
  int32_t num_new;
};

}  // namespace

struct pkv_scheduler {
  pkv_sched_config cfg{};
  std::vector<Request*> all;                      // arrival order (owned)
  std::unordered_map<int64_t, Request*> by_id;
  std::deque<Request*> waiting;
  std::vector<Request*> running;                  // admission order
  std::deque<int32_t> free_blocks;
  std::vector<int32_t> refcount;                  // per block
  std::unordered_map<int64_t, std::vector<int32_t>> prefix_blocks;  // prefix id -> shared full blocks
  std::vector<int64_t> block_prefix;              // per block: prefix id of its entry, or -1
  // the outstanding plan
  bool outstanding = false;
  std::vector<Scheduled> sched;
  std::vector<int64_t> p_ids;
  std::vector<int32_t> p_ctx, p_qsl, p_bt;
  std::vector<int64_t> p_slots;
  pkv_sched_stats stats{};

  ~pkv_scheduler() {
    for (Request* r : all) delete r;
  }

  // ---- block pool ----
  int32_t take_block() {
    const int32_t b = free_blocks.front();
    free_blocks.pop_front();
    refcount[b] = 1;
    return b;
  }
  void drop_prefix_entry(int64_t pid) {
    auto it = prefix_blocks.find(pid);
    if (it == prefix_blocks.end()) return;
    for (int32_t b : it->second) block_prefix[b] = -1;
    prefix_blocks.erase(it);
  }
  void release(Request* r) {  // last block first
    for (auto it = r->blocks.rbegin(); it != r->blocks.rend(); ++it) {
      const int32_t b = *it;
      if (--refcount[b] == 0) {
        if (block_prefix[b] >= 0) drop_prefix_entry(block_prefix[b]);
        free_blocks.push_back(b);
      }
    }
    r->blocks.clear();
  }
  // On-demand growth to hold num_computed + n tokens; all or nothing.
  bool allocate(Request* r, int64_t n) {
    const int64_t need = blocks_for(r->num_computed + n) - (int64_t)r->blocks.size();
    if (need <= 0) return true;
    if (need > (int64_t)free_blocks.size()) return false;
    for (int64_t k = 0; k < need; ++k) r->blocks.push_back(take_block());
    return true;
  }
  void preempt(Request* r) {
    stats.recomputed_tokens += r->num_computed;
    release(r);
    r->num_computed = 0;
    waiting.push_front(r);
    ++stats.preemptions;
  }
  // Shared full prefix blocks a waiting request can alias now.
  int64_t prefix_hit_blocks(const Request* r) const {
    if (r->prefix_id < 0) return 0;
    auto it = prefix_blocks.find(r->prefix_id);
    if (it == prefix_blocks.end()) return 0;
    // whole blocks of its own prefix, and at least one token left to compute
    int64_t hit = std::min<int64_t>((int64_t)it->second.size(), r->prefix_len / kBlockSize);
    hit = std::min<int64_t>(hit, (r->num_tokens() - 1) / kBlockSize);
    return hit;
  }
  // After a pass: blocks of a request's prefix that are full and computed
  // become shareable (an entry grows only from a holder of all its blocks).
  void register_prefix(Request* r) {
    if (r->prefix_id < 0) return;
    const int64_t full = std::min<int64_t>(r->num_computed, r->prefix_len) / kBlockSize;
    if (full <= 0) return;
    auto it = prefix_blocks.find(r->prefix_id);
    if (it == prefix_blocks.end()) {
      std::vector<int32_t> v(r->blocks.begin(), r->blocks.begin() + full);
      for (int32_t b : v) block_prefix[b] = r->prefix_id;
      prefix_blocks.emplace(r->prefix_id, std::move(v));
      return;
    }
    std::vector<int32_t>& v = it->second;
    if ((int64_t)v.size() >= full) return;
    if (!std::equal(v.begin(), v.end(), r->blocks.begin())) return;
    for (int64_t k = (int64_t)v.size(); k < full; ++k) {
      v.push_back(r->blocks[k]);
      block_prefix[r->blocks[k]] = r->prefix_id;
    }
  }

  // ---- one pass ----
  void plan_pass(pkv_sched_plan* plan) {
    sched.clear();
    int64_t budget = cfg.max_num_batched_tokens;
    int32_t preempted = 0, admitted = 0;
    const int64_t recomputed0 = stats.recomputed_tokens;
    int64_t hits = 0;

    // Phase one: the running requests, in admission (arrival) order.
    size_t i = 0;
    while (i < running.size() && budget > 0) {
      Request* r = running[i];
      const int64_t n = std::min<int64_t>(r->num_tokens() - r->num_computed, budget);
      if (n <= 0) {
        ++i;
        continue;
      }
      bool scheduled = true;
      while (!allocate(r, n)) {
        Request* victim = running.back();  // the newest
        running.pop_back();
        preempt(victim);
        ++preempted;
        if (victim == r) {
          scheduled = false;
          break;
        }
      }
      if (!scheduled) break;  // the requester was the newest: nothing after it
      sched.push_back({r, (int32_t)n});
      budget -= n;
      ++i;
    }

    // Phase two: admission, only in a pass that preempted nobody.
    if (preempted == 0) {
      while (!waiting.empty() && budget > 0) {
        if ((int32_t)running.size() >= cfg.max_num_seqs) break;
        Request* r = waiting.front();
        const int64_t hit = prefix_hit_blocks(r);
        const int64_t computed = hit * kBlockSize;
        const int64_t n = std::min<int64_t>(r->num_tokens() - computed, budget);
        const int64_t total_blocks = cfg.alloc_policy == PKV_ALLOC_RESERVE
                                         ? blocks_for((int64_t)r->prompt_len + r->max_new_tokens)
                                         : blocks_for(computed + n);
        if (total_blocks - hit > (int64_t)free_blocks.size()) break;  // stays first in line
        waiting.pop_front();
        if (hit > 0) {
          const std::vector<int32_t>& shared = prefix_blocks[r->prefix_id];
          for (int64_t k = 0; k < hit; ++k) {
            r->blocks.push_back(shared[k]);
            ++refcount[shared[k]];
          }
        }
        r->num_computed = computed;
        for (int64_t k = hit; k < total_blocks; ++k) r->blocks.push_back(take_block());
        hits += computed;
        running.push_back(r);
        ++admitted;
        sched.push_back({r, (int32_t)n});
        budget -= n;
      }
    }

    // The plan, one-token sequences first.
    std::stable_partition(sched.begin(), sched.end(),
                          [](const Scheduled& s) { return s.num_new == 1; });
    const int32_t B = (int32_t)sched.size();
    const int32_t W = cfg.max_blocks_per_seq;
    p_ids.assign(B, 0);
    p_ctx.assign(B, 0);
    p_qsl.assign(B + 1, 0);
    p_bt.assign((size_t)B * W, 0);
    p_slots.clear();
    int32_t ndec = 0, max_ctx = 0, max_q = 0;
    for (int32_t k = 0; k < B; ++k) {
      const Request* r = sched[k].req;
      const int32_t n = sched[k].num_new;
      const int64_t ctx = r->num_computed + n;
      p_ids[k] = r->id;
      p_ctx[k] = (int32_t)ctx;
      p_qsl[k + 1] = p_qsl[k] + n;
      std::copy(r->blocks.begin(), r->blocks.end(), p_bt.begin() + (size_t)k * W);
      for (int64_t p = r->num_computed; p < ctx; ++p)
        p_slots.push_back((int64_t)r->blocks[p / kBlockSize] * kBlockSize + p % kBlockSize);
      if (n == 1 && ndec == k) ++ndec;
      max_ctx = std::max<int32_t>(max_ctx, (int32_t)ctx);
      max_q = std::max(max_q, n);
    }
    stats.prefix_hit_tokens += hits;
    ++stats.passes;
    stats.peak_running = std::max<int32_t>(stats.peak_running, (int32_t)running.size());

    plan->num_seqs = B;
    plan->num_decode_seqs = ndec;
    plan->num_tokens = p_qsl[B];
    plan->max_context_len = max_ctx;
    plan->max_query_len = max_q;
    plan->request_ids = p_ids.data();
    plan->context_lens = p_ctx.data();
    plan->query_start_loc = p_qsl.data();
    plan->block_tables = p_bt.data();
    plan->slot_mapping = p_slots.data();
    plan->num_preempted = preempted;
    plan->num_admitted = admitted;
    plan->recomputed_tokens = stats.recomputed_tokens - recomputed0;
    plan->prefix_hit_tokens = hits;
  }

  void complete_pass() {
    for (const Scheduled& s : sched) {
      Request* r = s.req;
      r->num_computed += s.num_new;
      register_prefix(r);
      if (r->num_computed == r->num_tokens()) {
        ++r->num_generated;  // caught up: the pass sampled its next token
        ++stats.generated_tokens;
        if (r->num_generated >= r->max_new_tokens) {
          r->finished = true;
          release(r);
          running.erase(std::find(running.begin(), running.end(), r));
          ++stats.num_finished;
        }
      }
    }
    sched.clear();
  }
};

extern "C" {

pkv_scheduler* pkv_sched_create(const pkv_sched_config* c, const int32_t* free_order) {
  if (!c || c->num_blocks < 1 || c->num_blocks > INT32_MAX || c->block_size != kBlockSize ||
      c->max_num_seqs < 1 || c->max_num_batched_tokens < 1 || c->max_blocks_per_seq < 1 ||
      (c->alloc_policy != PKV_ALLOC_ON_DEMAND && c->alloc_policy != PKV_ALLOC_RESERVE))
    return nullptr;
  pkv_scheduler* s = new (std::nothrow) pkv_scheduler();
  if (!s) return nullptr;
  s->cfg = *c;
  std::vector<int32_t> order((size_t)c->num_blocks);
  if (free_order) {
    std::vector<char> seen((size_t)c->num_blocks, 0);
    for (size_t k = 0; k < order.size(); ++k) {
      const int32_t b = free_order[k];
      if (b < 0 || b >= c->num_blocks || seen[(size_t)b]) {
        delete s;
        return nullptr;
      }
      seen[(size_t)b] = 1;
      order[k] = b;
    }
  } else {
    std::iota(order.begin(), order.end(), 0);
  }
  s->free_blocks.assign(order.begin(), order.end());
  s->refcount.assign((size_t)c->num_blocks, 0);
  s->block_prefix.assign((size_t)c->num_blocks, -1);
  return s;
}

void pkv_sched_destroy(pkv_scheduler* s) { delete s; }

int pkv_sched_add_request(pkv_scheduler* s, int64_t request_id, int32_t prompt_len,
                          int32_t max_new_tokens, int64_t prefix_id, int32_t prefix_len) {
  if (!s || prompt_len < 1 || max_new_tokens < 1) return PKV_ERR_INVALID_ARG;
  if (prefix_len < 0 || (prefix_id >= 0 && prefix_len >= prompt_len)) return PKV_ERR_INVALID_ARG;
  if (s->by_id.count(request_id)) return PKV_ERR_INVALID_ARG;
  const int64_t most = blocks_for((int64_t)prompt_len + max_new_tokens);
  if (most > s->cfg.max_blocks_per_seq || most > s->cfg.num_blocks) return PKV_ERR_INVALID_ARG;
  Request* r = new (std::nothrow) Request();
  if (!r) return PKV_ERR_INVALID_ARG;
  r->id = request_id;
  r->prompt_len = prompt_len;
  r->max_new_tokens = max_new_tokens;
  r->prefix_id = prefix_id < 0 ? -1 : prefix_id;
  r->prefix_len = prefix_id < 0 ? 0 : prefix_len;
  s->all.push_back(r);
  s->by_id.emplace(request_id, r);
  s->waiting.push_back(r);
  return PKV_OK;
}

int pkv_sched_schedule(pkv_scheduler* s, pkv_sched_plan* plan) {
  if (!s || !plan || s->outstanding) return PKV_ERR_INVALID_ARG;
  s->plan_pass(plan);
  s->outstanding = true;
  return PKV_OK;
}

int pkv_sched_complete(pkv_scheduler* s) {
  if (!s || !s->outstanding) return PKV_ERR_INVALID_ARG;
  s->complete_pass();
  s->outstanding = false;
  return PKV_OK;
}

int pkv_sched_get_stats(const pkv_scheduler* s, pkv_sched_stats* st) {
  if (!s || !st) return PKV_ERR_INVALID_ARG;
  *st = s->stats;
  st->num_running = (int32_t)s->running.size();
  st->num_waiting = (int32_t)s->waiting.size();
  st->free_blocks = (int64_t)s->free_blocks.size();
  return PKV_OK;
}

int64_t pkv_sched_request_blocks(const pkv_scheduler* s, int64_t request_id, int32_t* out,
                                 int64_t cap) {
  if (!s) return -1;
  auto it = s->by_id.find(request_id);
  if (it == s->by_id.end() || it->second->blocks.empty()) return -1;
  const std::vector<int32_t>& b = it->second->blocks;
  for (int64_t k = 0; k < (int64_t)b.size() && k < cap; ++k) out[k] = b[k];
  return (int64_t)b.size();
}

}  // extern "C"
