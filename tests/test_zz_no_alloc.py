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


def _both_ways(wl, layer, part=0):
    """The step's layer run once with the workspace and once without, on two
    copies of the same inputs; returns the two results, the inputs and the
    step."""
    t = workloads.layer_tensors(wl, layer, device="cuda")
    t2 = {k: v.clone() for k, v in t.items()}
    step = Step.from_workload(wl, kv_partition_tokens=part)
    step.plan()
    qsl = step.query_start_loc if wl.num_decode_seqs < wl.num_seqs else None
    host_in = {k: host_bits(v) for k, v in t.items()}
    outs = []
    for tensors, noalloc in ((t, False), (t2, True)):
        cache = pkv.KVCache(tensors["k_pool"], tensors["v_pool"])
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
