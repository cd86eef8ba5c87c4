"""GPU parity of chunked prefill (causal query chunks on the MFMA kernel),
alone and sharing a step with decode sequences, against the CPU oracle."""
import numpy as np
import pytest

import workloads
from parity import run_layer_and_check

pytestmark = pytest.mark.gpu


def _report(name, errs):
    print(f"[parity] {name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}", flush=True)


@pytest.mark.parametrize("fused", [pytest.param(True, id="fused"),
                                   pytest.param(False, id="separate")])
def test_tiny_chunks_across_block_edges(fused):
    # decode sequences first, then chunks of 1..8 rows whose contexts cross 16/32
    ctx = [15, 16, 17, 31, 32, 33, 40, 16, 17, 33, 8]
    new = [1, 1, 1, 1, 1, 1, 8, 8, 3, 5, 8]
    wl = workloads.custom("tiny_chunks", ctx, new, 6, 12, 2, 128, seed=31)
    _, _, errs = run_layer_and_check(wl, fused=fused)
    _report(f"tiny chunks fused={fused}", errs)


@pytest.mark.parametrize("d,hq,hkv", [(128, 12, 2), (128, 8, 8), (128, 16, 2), (256, 16, 4),
                                      (256, 4, 4), (256, 24, 3)])
def test_chunks_spanning_query_tiles(d, hq, hkv):
    # chunks longer than one 64-row tile, with and without a cached prefix
    ctx = [300, 100, 64, 65, 500]
    new = [1, 100, 64, 65, 130]
    wl = workloads.custom("chunks", ctx, new, 1, hq, hkv, d, seed=hq * d)
    _, _, errs = run_layer_and_check(wl)
    _report(f"chunks d={d} G={hq // hkv}", errs)


def test_prefill_only_step():
    wl = workloads.custom("prefill_only", [40, 200, 129], [40, 70, 129], 0, 12, 2, 128, seed=37)
    _, _, errs = run_layer_and_check(wl)
    _report("prefill only", errs)


def test_qwen_mixed_full_size():
    """64 decodes + a 512-row chunk over an 8,192-token prefix, 28-layer shapes:
    every decode sequence and every row of the chunk checked."""
    wl = workloads.qwen_mixed()
    _, _, errs = run_layer_and_check(wl, 5, poison=False)
    _report("qwen_mixed layer 5 (64 decodes, all 512 chunk rows)", errs)


@pytest.mark.parametrize("hq,hkv", [(12, 2), (8, 8), (16, 2)])
def test_chunks_of_several_row_tiles_over_short_contexts(hq, hkv):
    """Chunks of 257 .. 700 rows (two or three 256-row tiles of the d = 128
    kernel) with little or no cached prefix: splits of one or two 64-token
    tiles, empty splits, and the loads' tail waits from the first step on;
    every row checked."""
    ctx = [1, 600, 700, 257, 520]
    new = [1, 600, 520, 257, 513]
    wl = workloads.custom("row_tiles", ctx, new, 1, hq, hkv, 128, seed=hq + 17 * hkv)
    _, _, errs = run_layer_and_check(wl)
    _report(f"several row tiles G={hq // hkv}", errs)


def test_long_chunk_over_long_context_splits_past_staged_pages():
    """A 2,048-row chunk over a 20,000-token context: 2 splits of ~157 KV
    tiles each, so the kernel's pages past the first 256 of a split take
    their pool offsets from the block table directly (not from the copy
    staged in LDS).  Sampled rows across the row tiles, checked each as the
    query that attends positions [0, its position]."""
    wl = workloads.custom("long_split", [20000], [2048], 0, 12, 2, 128, seed=71)
    rows = [0, 1, 127, 128, 255, 256, 1000, 1023, 1024, 1791, 2046, 2047]
    _, _, errs = run_layer_and_check(wl, seq_subset=[], row_samples={0: rows}, poison=False)
    _report("2,048-row chunk over 20,000 tokens (sampled rows)", errs)


def test_fused_chunk_append_matches_separate_calls_with_odd_slots():
    """A step with chunks, some of whose rows are skipped (slot -1: the
    pool's current row is attended) and one written to a slot outside its
    table position (written there, not attended): the fused call gives the
    same bits as pkv_kv_append followed by pkv_paged_attention_step, in the
    output and in both pools."""
    import torch
    import oracle
    import paged_kv_decode_append_amd as pkv
    from paged_kv_decode_append_amd.step import Step
    from parity import host_bits, poison_stale

    ctx, new = [40, 300, 129, 90], [1, 70, 129, 6]
    wl = workloads.custom("odd_slots", ctx, new, 1, 12, 2, 128, seed=61, pool_factor=2.0)
    qsl = wl.query_start_loc
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, qsl, 16).copy()
    used = set(slots.tolist())
    free = next(s for s in range(wl.num_blocks * 16) if s not in used and s // 16 not in
                set(wl.block_tables.ravel().tolist()))
    slots[qsl[1] + 3] = -1                 # long chunk: a padding row
    slots[qsl[2] + 64] = -1                # second row tile of the 129-row chunk
    slots[qsl[3] + 5] = -1                 # packed-size chunk, last row
    slots[qsl[1] + 10] = free              # written elsewhere, not attended
    outs, pools = [], []
    for fused in (True, False):
        t = workloads.layer_tensors(wl, 0, device="cuda")
        poison_stale(wl, t, poison_new=False)
        step = Step.from_workload(wl)
        step.plan()                         # the step's decode schedule (slots given below)
        sm = torch.from_numpy(slots).cuda()
        out = torch.full_like(t["q"], float("nan"))
        cache = pkv.KVCache(t["k_pool"], t["v_pool"])
        if fused:
            pkv.append_attention_step(cache, t["k_new"], t["v_new"], sm, t["q"], out,
                                      step.block_tables, step.context_lens, step.query_start_loc,
                                      wl.num_decode_seqs, wl.scale, step.max_context_len,
                                      step.max_query_len, workspace=step.workspace,
                                      schedule=step.schedule)
        else:
            pkv.kv_append(cache, t["k_new"], t["v_new"], sm)
            pkv.paged_attention_step(cache, t["q"], out, step.block_tables, step.context_lens,
                                     step.query_start_loc, wl.num_decode_seqs, wl.scale,
                                     step.max_context_len, step.max_query_len,
                                     workspace=step.workspace, schedule=step.schedule)
        torch.cuda.synchronize()
        outs.append(host_bits(out))
        pools.append((host_bits(t["k_pool"]), host_bits(t["v_pool"])))
    assert np.array_equal(outs[0], outs[1]), "output"
    assert np.array_equal(pools[0][0], pools[1][0]) and np.array_equal(pools[0][1], pools[1][1])
    assert not np.isnan(outs[0].view(np.float16).astype(np.float32)).any()
