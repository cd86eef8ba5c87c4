"""GPU edge cases of the step: empty inputs, a context that fills its whole
block-table row, a step whose every slot is padding, and the largest query
group the library takes, each through the C ABI and checked against the
oracle (pools bit-exact, attention within tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_append_amd as pkv
import workloads
from parity import assert_close, host_bits, run_layer_and_check

pytestmark = pytest.mark.gpu


def test_empty_step_and_empty_append_write_nothing():
    wl = workloads.custom("empty_ref", [40], [1], 1, 12, 2, 128, seed=71)
    t = workloads.layer_tensors(wl, 0, device="cuda")
    cache = pkv.KVCache(t["k_pool"], t["v_pool"])
    kp0, vp0 = host_bits(t["k_pool"]), host_bits(t["v_pool"])
    f16 = dict(dtype=torch.float16, device="cuda")
    i32 = dict(dtype=torch.int32, device="cuda")
    pkv.kv_append(cache, torch.empty(0, 2, 128, **f16), torch.empty(0, 2, 128, **f16),
                  torch.empty(0, dtype=torch.int64, device="cuda"))
    q = torch.empty(0, 12, 128, **f16)
    out = torch.empty(0, 12, 128, **f16)
    pkv.paged_attention_step(cache, q, out, torch.zeros(0, 4, **i32), torch.zeros(0, **i32), None,
                             0, wl.scale, 0, 0)
    sentinel = torch.full((3, 12, 128), 7.0, **f16)
    pkv.paged_attention_step(cache, q, sentinel[:0], torch.zeros(0, 4, **i32),
                             torch.zeros(0, **i32), torch.zeros(1, **i32), 0, wl.scale, 0, 0)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(t["k_pool"]), kp0)
    assert np.array_equal(host_bits(t["v_pool"]), vp0)
    assert bool((sentinel == 7.0).all())


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("d,hq,hkv", [(128, 12, 2), (256, 16, 4)])
def test_context_filling_its_whole_table_row(d, hq, hkv, fused):
    """Every sequence's context reaches the last slot of its table row (the
    row is exactly ceil(ctx / 16) wide for the longest one), with the new
    token in the row's last slot."""
    ctx = [16 * 40, 16 * 40 - 1, 17, 16 * 40]
    wl = workloads.custom("full_row", ctx, [1] * len(ctx), len(ctx), hq, hkv, d, seed=73)
    assert wl.block_tables.shape[1] == 40
    _, _, errs = run_layer_and_check(wl, fused=fused)
    print(f"[parity] full table row d={d} fused={fused}: max_abs={errs[0]:.2e}", flush=True)


def test_step_whose_every_slot_is_padding():
    """slot -1 for every decode token: nothing is written, and each sequence
    attends the pool's current row at ctx - 1."""
    from paged_kv_decode_append_amd.step import Step

    ctx = [20, 33, 300, 1025]
    wl = workloads.custom("all_pad", ctx, [1] * 4, 4, 12, 2, 128, seed=79)
    t = workloads.layer_tensors(wl, 0, device="cuda")
    kp0, vp0 = host_bits(t["k_pool"]), host_bits(t["v_pool"])
    step = Step.from_workload(wl)
    step.plan()
    slots = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    out = torch.full_like(t["q"], float("nan"))
    pkv.append_attention_step(pkv.KVCache(t["k_pool"], t["v_pool"]), t["k_new"], t["v_new"], slots,
                              t["q"], out, step.block_tables, step.context_lens,
                              step.query_start_loc, wl.num_decode_seqs, wl.scale,
                              step.max_context_len, step.max_query_len, workspace=step.workspace,
                              schedule=step.schedule)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(t["k_pool"]), kp0)
    assert np.array_equal(host_bits(t["v_pool"]), vp0)
    ref = oracle.paged_attention(host_bits(t["q"]), kp0, vp0, wl.block_tables, wl.context_lens,
                                 None, wl.scale)
    assert_close(out.cpu().numpy(), ref, "all-padding step")


@pytest.mark.parametrize("d", [128, 256])
def test_largest_query_group_with_one_kv_head(d):
    """G = 8 query heads on a single KV head, decodes and a chunk together."""
    ctx = [1, 16, 17, 500, 2000, 300]
    new = [1, 1, 1, 1, 1, 40]
    wl = workloads.custom("g8", ctx, new, 5, 8, 1, d, seed=83 + d)
    _, _, errs = run_layer_and_check(wl)
    print(f"[parity] G=8 Hkv=1 d={d}: max_abs={errs[0]:.2e}", flush=True)


# (context lengths, new tokens, decodes, query heads, KV heads, head size):
# short chunks, and one chunk longer than the decode launch's extra
# work-groups take in one row each (more than 128 x 8 rows)
PADDED_STEPS = {
    "short": ([300, 40, 1025, 700, 130], [1, 1, 1, 200, 65], 3, 12, 2),
    "long": ([900, 75, 1700], [1, 1, 1500], 2, 4, 1),
}


@pytest.mark.parametrize("kv,use_schedule,d,shape", [
    ("fp16", False, 128, "short"), ("fp16", True, 128, "short"), ("fp8", False, 128, "short"),
    ("fp16", False, 256, "short"), ("fp8", False, 256, "short"),
    ("fp16", False, 128, "long"), ("fp16", True, 128, "long"), ("fp8", False, 256, "long")])
def test_mixed_step_with_padded_prefill_rows(kv, use_schedule, d, shape):
    """A fused step of decodes and chunks where every third prefill row has
    slot -1: the decode launch's extra work-groups write the other prefill
    rows and skip those, whose positions keep the pool's row, which the
    chunk then attends (pools bit-exact against the oracle's append replay)."""
    from paged_kv_decode_append_amd.step import Step

    ctx, new, n_dec, hq, hkv = PADDED_STEPS[shape]
    print(f"[parity] padded prefill rows {shape} {kv} d={d} schedule={use_schedule}", flush=True)
    wl = workloads.custom("pad_chunks", ctx, new, n_dec, hq, hkv, d, seed=83)
    step = Step.from_workload(wl, use_schedule=use_schedule)
    step.plan()
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, wl.query_start_loc, 16)
    slots[n_dec::3] = -1                   # every third prefill row (decode rows come first)
    slots_t = torch.from_numpy(slots).cuda()
    if kv == "fp16":
        t = workloads.layer_tensors(wl, 0, device="cuda")
        cache = pkv.KVCache(t["k_pool"], t["v_pool"])
        before = [host_bits(t["k_pool"]), host_bits(t["v_pool"])]
    else:
        t = workloads.layer_tensors_fp8(wl, 0, device="cuda")
        cache = pkv.KVCache(t["k_codes"], t["v_codes"], t["k_scale"], t["v_scale"])
        before = [t[k].cpu().numpy() for k in ("k_codes", "v_codes", "k_scale", "v_scale")]
    out = torch.full_like(t["q"], float("nan"))
    pkv.append_attention_step(cache, t["k_new"], t["v_new"], slots_t, t["q"], out,
                              step.block_tables, step.context_lens, step.query_start_loc,
                              wl.num_decode_seqs, wl.scale, step.max_context_len,
                              step.max_query_len, workspace=step.workspace,
                              schedule=step.schedule)
    torch.cuda.synchronize()
    kn, vn, q = host_bits(t["k_new"]), host_bits(t["v_new"]), host_bits(t["q"])
    if kv == "fp16":
        kref, vref = oracle.kv_append(before[0], before[1], kn, vn, slots)
        assert np.array_equal(host_bits(t["k_pool"]), kref)
        assert np.array_equal(host_bits(t["v_pool"]), vref)
        ref = oracle.paged_attention(q, kref, vref, wl.block_tables, wl.context_lens,
                                     wl.query_start_loc, wl.scale)
    else:
        from oracle import fp8 as ofp8
        after = ofp8.kv_append(*before, kn, vn, slots)
        for name, want in zip(("k_codes", "v_codes", "k_scale", "v_scale"), after):
            assert np.array_equal(t[name].cpu().numpy(), want), name
        ref = oracle.paged_attention_fp8(q, *after, wl.block_tables, wl.context_lens,
                                         wl.query_start_loc, wl.scale)
    assert_close(out.cpu().numpy(), ref, f"padded prefill rows {shape} {kv} d={d} "
                 f"schedule={use_schedule}")
