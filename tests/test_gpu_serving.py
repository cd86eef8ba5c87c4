"""A run of the per-pass scheduler driving the GPU attention step.

40 requests through a 160-block pool (tight enough to preempt, with chunked
prefill under a 256-token budget and two groups sharing a 48-token prefix):
every pass, the scheduler's plan (block tables, context lengths, query
offsets) goes to the HIP path exactly as the benchmark runs it -- slot
mapping, then one pkv_append_attention_step -- over one persistent pool.
Each pass checks
  * the GPU slot mapping against the scheduler's, bit for bit;
  * the cache content of every scheduled sequence, read back through its
    table for all positions of its context, against the rows the run defines
    for (request or shared prefix, position) -- after preemptions, recompute
    and prefix aliasing, bit for bit;
  * the attention output against the CPU oracle (tolerance of the path).
The K/V rows of a token are a pure function of (key, position), so a
recomputed token and a shared-prefix token have the same rows.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_append_amd as pkv
import workloads
from paged_kv_decode_append_amd.scheduler import Scheduler
from paged_kv_decode_append_amd.step import Step
from parity import assert_close, host_bits

pytestmark = pytest.mark.gpu

HQ, HKV, D = 12, 2, 128
NUM_BLOCKS, WIDTH, PREFIX = 160, 64, 48
GROUP_KEY = 1 << 40  # K/V key of a shared prefix group (request ids are small)


def test_scheduler_driven_passes_on_the_gpu():
    prompts, outputs, groups = workloads.serving_requests(
        seed=7, num_requests=40, prompt_range=(16, 300), output_range=(4, 40),
        prefix_groups=2, shared_prefix=PREFIX)
    groups = np.where(np.arange(40) % 2 == 0, groups, -1)
    sched = Scheduler(NUM_BLOCKS, 32, 256, WIDTH,
                      free_order=workloads.free_block_order(NUM_BLOCKS, seed=7))
    for rid in range(40):
        g = int(groups[rid])
        sched.add_request(rid, int(prompts[rid]), int(outputs[rid]), g, PREFIX if g >= 0 else 0)

    rows = {}  # (key, position) -> [2, Hkv, d] fp16

    def key_of(rid, pos):
        g = int(groups[rid])
        return GROUP_KEY + g if g >= 0 and pos < PREFIX else rid

    def kv(rid, pos):
        k = (key_of(rid, pos), pos)
        if k not in rows:
            rows[k] = workloads.token_kv_rows(k[0], [pos], HKV, D, seed=11)[0]
        return rows[k]

    nan = float("nan")
    k_pool = torch.full((NUM_BLOCKS, HKV, 16, D), nan, dtype=torch.float16, device="cuda")
    v_pool = torch.full_like(k_pool, nan)
    cache = pkv.KVCache(k_pool, v_pool)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    scale = 1.0 / np.sqrt(D)
    passes = preempting = worst = 0

    while not sched.done():
        plan = sched.schedule()
        if plan.num_seqs == 0:
            sched.complete()
            continue
        # this pass's new K/V rows, in plan order
        new = np.stack([kv(int(plan.request_ids[k]), p)
                        for k in range(plan.num_seqs)
                        for p in range(int(plan.context_lens[k] - plan.new_tokens[k]),
                                       int(plan.context_lens[k]))])
        k_new = torch.from_numpy(np.ascontiguousarray(new[:, 0])).cuda()
        v_new = torch.from_numpy(np.ascontiguousarray(new[:, 1])).cuda()
        q = torch.randn(plan.num_tokens, HQ, D, generator=gen, device="cuda",
                        dtype=torch.float16)
        out = torch.full_like(q, nan)
        step = Step(plan.block_tables, plan.context_lens, plan.new_tokens,
                    plan.num_decode_seqs, HQ, HKV, D, scale)
        step.plan()
        step.layer(cache, q, k_new, v_new, out)
        torch.cuda.synchronize()

        assert np.array_equal(step.slot_mapping[: plan.num_tokens].cpu().numpy(),
                              plan.slot_mapping), f"pass {passes}: slot mapping"
        kp, vp = host_bits(k_pool), host_bits(v_pool)
        for k in range(plan.num_seqs):
            rid, ctx = int(plan.request_ids[k]), int(plan.context_lens[k])
            want = np.stack([kv(rid, p) for p in range(ctx)]).view(np.uint16)
            tb = plan.block_tables[k]
            got_k = np.stack([kp[tb[p // 16], :, p % 16] for p in range(ctx)])
            got_v = np.stack([vp[tb[p // 16], :, p % 16] for p in range(ctx)])
            assert np.array_equal(got_k, want[:, 0]), f"pass {passes}: K of request {rid}"
            assert np.array_equal(got_v, want[:, 1]), f"pass {passes}: V of request {rid}"
        qsl = plan.query_start_loc if plan.num_decode_seqs < plan.num_seqs else None
        ref = oracle.paged_attention(host_bits(q), kp, vp, plan.block_tables, plan.context_lens,
                                     qsl, scale)
        err = assert_close(out.cpu().numpy(), ref, f"pass {passes}")
        worst = max(worst, err[0])
        preempting += plan.num_preempted > 0
        sched.complete()
        passes += 1

    st = sched.stats()
    print(f"[serving] passes={passes} preemptions={st['preemptions']} "
          f"recomputed={st['recomputed_tokens']} prefix_hits={st['prefix_hit_tokens']} "
          f"peak={st['peak_running']} max_abs={worst:.2e}", flush=True)
    assert st["num_finished"] == 40 and st["free_blocks"] == NUM_BLOCKS
    assert preempting > 0 and st["prefix_hit_tokens"] > 0
