"""pkv_append_attention_step_noalloc on the GPU: the no-allocation step (its
partials in the library's own device scratch) gives the same bits as
pkv_append_attention_step with a caller-owned workspace -- outputs and both
pools -- on two calls in a row, the second on a smaller step, so that the
second call runs over the first call's stale partials; and both are within
the attention tolerance of the oracle.  Every call goes through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_append_amd as pkv
import workloads
from paged_kv_decode_append_amd.step import Step
from parity import assert_close, host_bits

pytestmark = pytest.mark.gpu


FP16_POOLS = ("k_pool", "v_pool")
FP8_POOLS = ("k_codes", "v_codes", "k_scale", "v_scale")


def _both_ways(wl, layer, part=0, fp8=False):
    """The step's layer run once with the workspace and once without, on two
    copies of the same inputs; returns the two results, the inputs and the
    step."""
    pools = FP8_POOLS if fp8 else FP16_POOLS
    make = workloads.layer_tensors_fp8 if fp8 else workloads.layer_tensors
    t = make(wl, layer, device="cuda")
    t2 = {k: v.clone() for k, v in t.items()}
    step = Step.from_workload(wl, kv_partition_tokens=part)
    step.plan()
    qsl = step.query_start_loc if wl.num_decode_seqs < wl.num_seqs else None
    host_in = {k: host_bits(v) if v.dtype == torch.float16 else v.cpu().numpy()
               for k, v in t.items()}
    outs = []
    for tensors, noalloc in ((t, False), (t2, True)):
        cache = pkv.KVCache(*(tensors[n] for n in pools))
        out = torch.full_like(tensors["q"], float("nan"))
        args = (cache, tensors["k_new"], tensors["v_new"], step.slot_mapping, tensors["q"], out,
                step.block_tables, step.context_lens, qsl, wl.num_decode_seqs, wl.scale,
                step.max_context_len, step.max_query_len)
        if noalloc:
            pkv.append_attention_step_noalloc(*args, kv_partition_tokens=part,
                                              schedule=step.schedule)
        else:
            pkv.append_attention_step(*args, workspace=step.workspace, kv_partition_tokens=part,
                                      schedule=step.schedule)
        outs.append(out)
    torch.cuda.synchronize()
    return t, t2, outs, host_in


def _check(wl, layer, part=0):
    t, t2, (o_ws, o_na), host_in = _both_ways(wl, layer, part)
    assert np.array_equal(host_bits(o_ws), host_bits(o_na)), "outputs differ"
    assert np.array_equal(host_bits(t["k_pool"]), host_bits(t2["k_pool"])), "K pools differ"
    assert np.array_equal(host_bits(t["v_pool"]), host_bits(t2["v_pool"])), "V pools differ"
    qsl = wl.query_start_loc if wl.num_decode_seqs < wl.num_seqs else None
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, qsl, wl.block_size)
    kp, vp = oracle.kv_append(host_in["k_pool"], host_in["v_pool"], host_in["k_new"],
                              host_in["v_new"], slots)
    assert np.array_equal(host_bits(t2["k_pool"]), kp), "K pool after append"
    assert np.array_equal(host_bits(t2["v_pool"]), vp), "V pool after append"
    ref = oracle.paged_attention(host_in["q"], kp, vp, wl.block_tables, wl.context_lens, qsl,
                                 wl.scale)
    errs = assert_close(o_na.cpu().numpy(), ref, wl.name)
    print(f"[parity] noalloc {wl.name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}", flush=True)


def test_noalloc_step_matches_the_workspace_step_twice():
    # first call: decodes split over several partitions plus a prefill chunk
    # (decode and prefill partials both in the scratch)
    big = workloads.custom("noalloc_big", [4100, 9000, 300, 17, 2600], [1, 1, 1, 1, 200], 4,
                           12, 2, 128, seed=71)
    _check(big, 0)
    # second call, smaller: its partials land over the first call's
    small = workloads.custom("noalloc_small", [700, 33, 1500], [1, 1, 1], 3, 12, 2, 128, seed=73)
    _check(small, 0, part=256)


def test_noalloc_step_long_context_shape():
    # d = 256, G = 4, contexts long enough for 64-block partitions
    wl = workloads.custom("noalloc_d256", [20000, 9000, 100], [1, 1, 1], 3, 16, 4, 256, seed=79)
    _check(wl, 0)


def test_noalloc_step_fp8_cache_twice():
    # an fp8 cache: a mixed step (split decodes, a chunk), then a smaller
    # decode-only step over the first one's scratch contents
    from oracle import fp8 as ofp8
    for wl, part in ((workloads.custom("noalloc_fp8_big", [4100, 9000, 300, 2600], [1, 1, 1, 150],
                                       3, 12, 2, 128, seed=81), 0),
                     (workloads.custom("noalloc_fp8_small", [700, 33, 1500], [1, 1, 1], 3, 16, 4,
                                       256, seed=83), 256)):
        t, t2, (o_ws, o_na), host_in = _both_ways(wl, 0, part, fp8=True)
        assert np.array_equal(host_bits(o_ws), host_bits(o_na)), "outputs differ"
        for n in FP8_POOLS:
            assert np.array_equal(t[n].cpu().numpy().view(np.uint8),
                                  t2[n].cpu().numpy().view(np.uint8)), f"{n} differs"
        qsl = wl.query_start_loc if wl.num_decode_seqs < wl.num_seqs else None
        slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, qsl, wl.block_size)
        after = ofp8.kv_append(*(host_in[n] for n in FP8_POOLS), host_in["k_new"],
                               host_in["v_new"], slots)
        for n, want in zip(FP8_POOLS, after):
            assert np.array_equal(t2[n].cpu().numpy().view(np.uint8), want.view(np.uint8)), n
        ref = oracle.paged_attention_fp8(host_in["q"], *after, wl.block_tables, wl.context_lens,
                                         qsl, wl.scale)
        errs = assert_close(o_na.cpu().numpy(), ref, wl.name)
        print(f"[parity] noalloc fp8 {wl.name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}",
              flush=True)
