"""GPU parity of the decode path (slot mapping, KV append, paged decode
attention with split-KV + log-sum-exp merge) against the CPU oracle.

Every case runs the HIP path through the C ABI exactly as the benchmark
does, then checks: slot mapping bit-exact, whole pools after the append
bit-exact, attention within max|diff| <= 2e-3 and per-row norm-relative
<= 1e-2 of the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_append_amd as pkv
import workloads
from parity import assert_close, host_bits, poison_stale, run_layer_and_check

pytestmark = pytest.mark.gpu


def _report(name, errs):
    print(f"[parity] {name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}", flush=True)


FUSED = [pytest.param(True, id="fused"), pytest.param(False, id="separate")]


@pytest.mark.parametrize("fused", FUSED)
def test_small_b4_workload(fused):
    wl = workloads.small_b4()
    _, _, errs = run_layer_and_check(wl, fused=fused)
    _report(f"small_b4 fused={fused}", errs)


EDGE_CTX = [1, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 255, 256, 257, 1000]


@pytest.mark.parametrize("fused", FUSED)
@pytest.mark.parametrize("d,hq,hkv", [(128, 12, 2), (256, 16, 4)])
def test_block_edge_context_lengths(d, hq, hkv, fused):
    wl = workloads.custom("edges", EDGE_CTX, [1] * len(EDGE_CTX), len(EDGE_CTX), hq, hkv, d, seed=1)
    _, _, errs = run_layer_and_check(wl, fused=fused)
    _report(f"edges d={d} fused={fused}", errs)


@pytest.mark.parametrize("d,hq,hkv", [(128, 2, 2), (128, 4, 2), (128, 6, 2), (128, 8, 2),
                                      (128, 10, 2), (128, 14, 2), (128, 16, 2), (128, 8, 8),
                                      (256, 4, 4), (256, 8, 4), (256, 12, 2), (256, 24, 3)])
def test_query_group_sizes(d, hq, hkv):
    ctx = [7, 40, 129, 700]
    wl = workloads.custom("groups", ctx, [1] * 4, 4, hq, hkv, d, seed=hq + d)
    _, _, errs = run_layer_and_check(wl)
    _report(f"G={hq // hkv} d={d}", errs)


@pytest.mark.parametrize("fused", FUSED)
@pytest.mark.parametrize("part", [64, 128, 256, 1024, 4096])
def test_split_kv_partitions(part, fused):
    ctx = [1, 63, 64, 65, 300, 1024, 3000, 5000]
    wl = workloads.custom("split", ctx, [1] * len(ctx), len(ctx), 12, 2, 128, seed=5)
    _, _, errs = run_layer_and_check(wl, kv_partition_tokens=part, fused=fused)
    _report(f"partition {part} fused={fused}", errs)


@pytest.mark.parametrize("fused", FUSED)
def test_single_token_context_returns_the_new_value_bit_exactly(fused):
    wl = workloads.custom("ctx1", [1, 1, 1], [1, 1, 1], 3, 12, 2, 128, seed=9)
    got, _, _ = run_layer_and_check(wl, fused=fused)
    vn = workloads.layer_tensors(wl, 0, device="cuda")["v_new"]
    vbits = host_bits(vn)
    gbits = got.view(np.uint16)
    for h in range(12):
        assert np.array_equal(gbits[:, h], vbits[:, h // 6])


def _run_plain(wl, tensors, part=0, fused=True):
    from paged_kv_decode_append_amd.step import Step
    step = Step.from_workload(wl, kv_partition_tokens=part)
    step.plan()
    out = torch.empty_like(tensors["q"])
    step.layer(pkv.KVCache(tensors["k_pool"], tensors["v_pool"]), tensors["q"], tensors["k_new"],
               tensors["v_new"], out, fused=fused)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("fused", FUSED)
@pytest.mark.parametrize("part", [0, 256])
def test_block_placement_and_poison_are_invisible_bit_exactly(part, fused):
    """Relabelling physical blocks, and NaN in every stale slot, leave the
    GPU output bit-identical."""
    ctx = [5, 33, 300, 777]
    wl = workloads.custom("perm", ctx, [1] * 4, 4, 12, 2, 128, seed=11, pool_factor=2.0)
    t = workloads.layer_tensors(wl, 0, device="cuda")
    base = _run_plain(wl, {k: v.clone() for k, v in t.items()}, part, fused)

    # relabel: physical block b -> perm[b]
    perm = np.random.default_rng(3).permutation(wl.num_blocks)
    inv = torch.from_numpy(np.argsort(perm)).cuda()
    t2 = {k: v.clone() for k, v in t.items()}
    t2["k_pool"] = t["k_pool"][inv].contiguous()
    t2["v_pool"] = t["v_pool"][inv].contiguous()
    wl2 = workloads.custom("perm", ctx, [1] * 4, 4, 12, 2, 128, seed=11, pool_factor=2.0)
    wl2.block_tables = perm[wl.block_tables].astype(np.int32)
    assert np.array_equal(_run_plain(wl2, t2, part, fused), base)

    # poison every stale slot and the unused table entries
    t3 = {k: v.clone() for k, v in t.items()}
    wl3 = workloads.custom("perm", ctx, [1] * 4, 4, 12, 2, 128, seed=11, pool_factor=2.0)
    poison_stale(wl3, t3)
    assert np.array_equal(_run_plain(wl3, t3, part, fused), base)


def test_append_skips_padding_slots_and_touches_nothing_else():
    wl = workloads.custom("pad", [20, 40, 60], [1, 1, 1], 3, 12, 2, 128, seed=13)
    t = workloads.layer_tensors(wl, 0, device="cuda")
    kp0, vp0 = host_bits(t["k_pool"]), host_bits(t["v_pool"])
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, None, 16)
    slots[1] = -1
    cache = pkv.KVCache(t["k_pool"], t["v_pool"])
    pkv.kv_append(cache, t["k_new"], t["v_new"], torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kref, vref = oracle.kv_append(kp0, vp0, host_bits(t["k_new"]), host_bits(t["v_new"]), slots)
    assert np.array_equal(host_bits(t["k_pool"]), kref)
    assert np.array_equal(host_bits(t["v_pool"]), vref)


def test_slot_mapping_with_prefill_chunks():
    wl = workloads.custom("chunks", [17, 40, 100, 33], [1, 1, 60, 16], 2, 12, 2, 128, seed=17)
    out = torch.full((wl.num_tokens,), -7, dtype=torch.int64, device="cuda")
    pkv.slot_mapping(torch.from_numpy(wl.block_tables).cuda(), torch.from_numpy(wl.context_lens).cuda(),
                     torch.from_numpy(wl.query_start_loc).cuda(), wl.num_tokens, out)
    torch.cuda.synchronize()
    ref = oracle.slot_mapping(wl.block_tables, wl.context_lens, wl.query_start_loc, 16)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_random_ragged_shapes():
    rng = np.random.default_rng(21)
    for trial in range(6):
        d = int(rng.choice([128, 256]))
        hkv = int(rng.integers(1, 5))
        g = int(rng.integers(1, 9))
        B = int(rng.integers(1, 40))
        ctx = rng.integers(1, 3000, size=B)
        wl = workloads.custom("rand", ctx, [1] * B, B, hkv * g, hkv, d, seed=100 + trial)
        part = int(rng.choice([0, 64, 192, 512]))
        fused = bool(trial % 2)
        _, _, errs = run_layer_and_check(wl, kv_partition_tokens=part, fused=fused)
        _report(f"rand d={d} G={g} Hkv={hkv} B={B} part={part} fused={fused}", errs)


@pytest.mark.parametrize("d,hq,hkv,part", [(128, 12, 2, 0), (128, 12, 2, 128), (256, 16, 4, 0),
                                           (128, 8, 1, 64), (256, 8, 8, 256)])
def test_fused_and_separate_append_give_identical_bits(d, hq, hkv, part):
    """pkv_append_attention_step leaves the same pools and the same output
    bits as pkv_kv_append followed by pkv_paged_attention_step."""
    ctx = [1, 2, 15, 16, 17, 32, 33, 200, 513, 1025]
    wl = workloads.custom("fused_eq", ctx, [1] * len(ctx), len(ctx), hq, hkv, d, seed=d + hq + part)
    t = workloads.layer_tensors(wl, 0, device="cuda")
    t_sep = {k: v.clone() for k, v in t.items()}
    out_f = _run_plain(wl, t, part, fused=True)
    out_s = _run_plain(wl, t_sep, part, fused=False)
    assert np.array_equal(out_f, out_s)
    assert np.array_equal(host_bits(t["k_pool"]), host_bits(t_sep["k_pool"]))
    assert np.array_equal(host_bits(t["v_pool"]), host_bits(t_sep["v_pool"]))


def _fused_call(wl, t, slots, part=0):
    from paged_kv_decode_append_amd.step import Step
    step = Step.from_workload(wl, kv_partition_tokens=part)
    step.plan()  # the decode schedule (the slot mapping it also writes is not used)
    out = torch.empty_like(t["q"])
    pkv.append_attention_step(pkv.KVCache(t["k_pool"], t["v_pool"]), t["k_new"], t["v_new"],
                              torch.from_numpy(slots).cuda(), t["q"], out, step.block_tables,
                              step.context_lens, step.query_start_loc, wl.num_decode_seqs,
                              wl.scale, step.max_context_len, step.max_query_len,
                              workspace=step.workspace, kv_partition_tokens=part,
                              schedule=step.schedule)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("part", [0, 64])
def test_fused_append_skips_a_padding_slot(part):
    """A decode token with slot -1 is not written, and its sequence attends
    the pool's current row at ctx - 1 -- as with the separate calls."""
    ctx = [20, 40, 60, 300]
    wl = workloads.custom("pad_fused", ctx, [1] * 4, 4, 12, 2, 128, seed=19)
    t = workloads.layer_tensors(wl, 0, device="cuda")
    kp0, vp0 = host_bits(t["k_pool"]), host_bits(t["v_pool"])
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, None, 16)
    slots[1] = -1
    slots[3] = -1
    out = _fused_call(wl, t, slots, part)
    kref, vref = oracle.kv_append(kp0, vp0, host_bits(t["k_new"]), host_bits(t["v_new"]), slots)
    assert np.array_equal(host_bits(t["k_pool"]), kref)
    assert np.array_equal(host_bits(t["v_pool"]), vref)
    ref = oracle.paged_attention(host_bits(t["q"]), kref, vref, wl.block_tables, wl.context_lens,
                                 None, wl.scale)
    assert_close(out.cpu().numpy(), ref, "padding slot, fused")
