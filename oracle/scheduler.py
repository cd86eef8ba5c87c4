"""Plain-Python model of the per-pass scheduler and its block pool.

TEST INFRASTRUCTURE ONLY (as the rest of ``oracle/``): the C++ scheduler in
libpkv.so is checked against it pass by pass; the product never imports it,
and it shares no code with the C++ (different language, written from the
page, not from the C++).

Follows deepconcepts.dev, "Continuous Batching Is Not a Bigger Batch":

* section "What the scheduler does on one step" -- a pass has two phases.
  Phase one: the running requests, in arrival (admission) order, each ask
  for their next tokens: a decoding request wants one; a prefilling request
  wants the rest of its prompt, capped by what is left of the pass's token
  budget.  The cache manager allocates the blocks for them; when that fails,
  the last request of the running list (the newest) is preempted -- its
  blocks freed, its computed tokens reset to zero, put at the front of the
  waiting queue -- and allocation is tried again; if the preempted one is the
  requester itself, phase one ends.  Phase two, only when nothing was
  preempted in this pass: waiting requests in order are admitted while the
  budget is positive and fewer than max_num_seqs requests run; one that
  cannot get its blocks stays at the head of the queue and admission stops.
* section "The allocator is the other half": 16-token blocks, allocated on
  demand (a request holds ceil(tokens / 16) of them), or -- the reserving
  design -- the blocks for prompt + declared maximum output at admission.
* prefix caching (the note on recompute in the first section): requests
  declaring the same prefix share its full, computed blocks while any of
  them holds those blocks.

Readings where the page is silent (listed with the design notes): a request
samples its next token in the pass that brings its computed tokens level
with its total (prompt + tokens generated so far), and finishes when it has
generated max_new_tokens, freeing its blocks; the last generated token is
never appended.  Free blocks form a FIFO queue (taken from the front; a
request's blocks are freed last block first and join the back).  A pass's
sequences are reported one-token sequences first (the attention step's
order), each group in running order.  The parity of this model with the
C++ is exact (integers); the page's own simulation numbers (peak batch 83,
38 preemptions, 49,535 recomputed tokens) come from a workload the page does
not give, so they are context, not pins.
"""
from __future__ import annotations

BLOCK = 16


def _blocks(tokens: int) -> int:
    return -(-tokens // BLOCK)


class _Req:
    def __init__(self, rid, prompt, max_new, prefix_id, prefix_len):
        self.rid = rid
        self.prompt = prompt
        self.max_new = max_new
        self.prefix_id = prefix_id if prefix_id is not None and prefix_id >= 0 else -1
        self.prefix_len = prefix_len if self.prefix_id >= 0 else 0
        self.generated = 0
        self.computed = 0
        self.blocks = []

    def total(self):
        return self.prompt + self.generated


class SchedulerModel:
    def __init__(self, num_blocks, max_num_seqs, max_num_batched_tokens, max_blocks_per_seq,
                 reserve=False, free_order=None):
        self.max_num_seqs = max_num_seqs
        self.budget_per_pass = max_num_batched_tokens
        self.width = max_blocks_per_seq
        self.reserve = reserve
        self.free = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        self.ref = [0] * num_blocks
        self.waiting = []      # front = index 0
        self.running = []      # admission order
        self.shared = {}       # prefix id -> list of shared full blocks
        self.planned = None
        self.stats = {"preemptions": 0, "recomputed_tokens": 0, "prefix_hit_tokens": 0,
                      "generated_tokens": 0, "peak_running": 0, "finished": 0}

    # ------------------------------------------------------------ pool ---
    def _take(self):
        b = self.free.pop(0)
        self.ref[b] = 1
        return b

    def _free_request_blocks(self, r):
        for b in reversed(r.blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                for pid in [p for p, bl in self.shared.items() if b in bl]:
                    del self.shared[pid]
                self.free.append(b)
        r.blocks = []

    def _grow(self, r, n):
        need = _blocks(r.computed + n) - len(r.blocks)
        if need > len(self.free):
            return False
        for _ in range(max(need, 0)):
            r.blocks.append(self._take())
        return True

    # -------------------------------------------------------- requests ---
    def add_request(self, rid, prompt, max_new, prefix_id=-1, prefix_len=0):
        self.waiting.append(_Req(rid, prompt, max_new, prefix_id, prefix_len))

    def _hit(self, r):
        if r.prefix_id < 0 or r.prefix_id not in self.shared:
            return 0
        return min(len(self.shared[r.prefix_id]), r.prefix_len // BLOCK, (r.total() - 1) // BLOCK)

    # ------------------------------------------------------------ pass ---
    def schedule(self):
        budget = self.budget_per_pass
        chosen = []            # (request, new tokens) in scheduling order
        preempted = admitted = 0
        recomputed = hits = 0

        i = 0
        while i < len(self.running) and budget > 0:
            r = self.running[i]
            n = min(r.total() - r.computed, budget)
            requester_lost = False
            while not self._grow(r, n):
                victim = self.running.pop()
                recomputed += victim.computed
                self._free_request_blocks(victim)
                victim.computed = 0
                self.waiting.insert(0, victim)
                preempted += 1
                if victim is r:
                    requester_lost = True
                    break
            if requester_lost:
                break
            chosen.append((r, n))
            budget -= n
            i += 1

        if preempted == 0:
            while self.waiting and budget > 0 and len(self.running) < self.max_num_seqs:
                r = self.waiting[0]
                hit = self._hit(r)
                n = min(r.total() - hit * BLOCK, budget)
                want = _blocks(r.prompt + r.max_new) if self.reserve else _blocks(hit * BLOCK + n)
                if want - hit > len(self.free):
                    break
                self.waiting.pop(0)
                r.blocks = []
                for b in (self.shared[r.prefix_id][:hit] if hit else []):
                    r.blocks.append(b)
                    self.ref[b] += 1
                r.computed = hit * BLOCK
                for _ in range(want - hit):
                    r.blocks.append(self._take())
                hits += hit * BLOCK
                self.running.append(r)
                admitted += 1
                chosen.append((r, n))
                budget -= n

        self.stats["preemptions"] += preempted
        self.stats["recomputed_tokens"] += recomputed
        self.stats["prefix_hit_tokens"] += hits
        self.stats["peak_running"] = max(self.stats["peak_running"], len(self.running))

        order = [c for c in chosen if c[1] == 1] + [c for c in chosen if c[1] != 1]
        self.planned = order
        plan = {"request_ids": [], "context_lens": [], "new_tokens": [], "block_tables": [],
                "slot_mapping": [], "num_decode_seqs": sum(1 for c in order if c[1] == 1),
                "num_preempted": preempted, "num_admitted": admitted,
                "recomputed_tokens": recomputed, "prefix_hit_tokens": hits}
        for r, n in order:
            plan["request_ids"].append(r.rid)
            plan["context_lens"].append(r.computed + n)
            plan["new_tokens"].append(n)
            plan["block_tables"].append(r.blocks + [0] * (self.width - len(r.blocks)))
            for p in range(r.computed, r.computed + n):
                plan["slot_mapping"].append(r.blocks[p // BLOCK] * BLOCK + p % BLOCK)
        return plan

    def _register(self, r):
        if r.prefix_id < 0:
            return
        full = min(r.computed, r.prefix_len) // BLOCK
        if full <= 0:
            return
        if r.prefix_id not in self.shared:
            self.shared[r.prefix_id] = list(r.blocks[:full])
            return
        have = self.shared[r.prefix_id]
        if len(have) < full and r.blocks[:len(have)] == have:
            have.extend(r.blocks[len(have):full])

    def complete(self):
        for r, n in self.planned:
            r.computed += n
            self._register(r)
            if r.computed == r.total():
                r.generated += 1
                self.stats["generated_tokens"] += 1
                if r.generated >= r.max_new:
                    self._free_request_blocks(r)
                    self.running.remove(r)
                    self.stats["finished"] += 1
        self.planned = None

    def done(self):
        return not self.running and not self.waiting
