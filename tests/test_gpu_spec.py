"""GPU parity of multi-token decode: sequences that bring a few query tokens
each (the last sampled token plus drafted ones to verify), attended causally
over their whole context.  When every such chunk's G x n rows fit one 64-row
tile, the step packs all G query heads of a KV group into one work-group
(each K/V tile read once per KV head); larger chunks take the per-head
path.  Checked against the CPU oracle."""
import numpy as np
import pytest

import workloads
from parity import run_layer_and_check

pytestmark = pytest.mark.gpu


def _report(name, errs):
    print(f"[parity] {name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}", flush=True)


@pytest.mark.parametrize("fused", [pytest.param(True, id="fused"),
                                   pytest.param(False, id="separate")])
@pytest.mark.parametrize("d,hq,hkv,qmax", [(128, 12, 2, 8), (128, 8, 1, 8), (256, 16, 4, 16),
                                           (128, 8, 8, 64), (256, 24, 3, 8)])
def test_multi_token_decode(d, hq, hkv, qmax, fused):
    # contexts across block edges and up to a few thousand tokens; n in 2..qmax
    rng = np.random.default_rng(d + hq + qmax)
    ctx = np.array([2, 15, 16, 17, 31, 33, 64, 100, 700, 3000, 4100], dtype=np.int32)
    new = np.minimum(rng.integers(2, qmax, size=len(ctx), endpoint=True), ctx).astype(np.int32)
    new[-1] = qmax  # the longest chunk the packing allows
    wl = workloads.custom("multi_token", ctx, new, 0, hq, hkv, d, seed=hq * d + qmax)
    _, _, errs = run_layer_and_check(wl, fused=fused)
    _report(f"multi-token d={d} G={hq // hkv} n<={qmax} fused={fused}", errs)


def test_decodes_then_multi_token_decodes():
    # single-token decodes first (decode kernel), then 2..8-token chunks (packed kernel)
    ctx = [512, 17, 1000, 33, 16, 250, 4096, 9]
    new = [1, 1, 1, 8, 2, 5, 7, 3]
    wl = workloads.custom("decode_then_multi", ctx, new, 3, 12, 2, 128, seed=41)
    _, _, errs = run_layer_and_check(wl)
    _report("decodes then multi-token", errs)


def test_chunk_just_past_the_packing_limit():
    # G = 8 and n = 9: 72 rows > 64, so every chunk takes the per-head path
    ctx = [40, 9, 300]
    new = [9, 9, 2]
    wl = workloads.custom("past_packing", ctx, new, 0, 16, 2, 128, seed=43)
    _, _, errs = run_layer_and_check(wl)
    _report("n=9, G=8 (per-head path)", errs)


def test_qwen_spec_full_size():
    """64 sequences x 4 query tokens over contexts in [256, 4096], 28-layer
    shapes: one layer, all sequences checked."""
    wl = workloads.qwen_spec()
    _, _, errs = run_layer_and_check(wl, 11, poison=False)
    _report("qwen_spec layer 11", errs)


@pytest.mark.parametrize("fused", [pytest.param(True, id="fused"),
                                   pytest.param(False, id="separate")])
@pytest.mark.parametrize("hq,hkv,qmax", [(12, 2, 5), (12, 2, 2), (8, 1, 4), (16, 2, 4), (8, 8, 32),
                                         (8, 8, 16), (4, 4, 8), (6, 2, 10), (2, 2, 1)])
def test_short_chunks_of_up_to_32_rows(hq, hkv, qmax, fused):
    """n G <= 32 rows per KV head (packed, half a row tile or less):
    contexts across block edges and up to a few thousand tokens, chunks of
    1..qmax tokens, the longest one at qmax."""
    rng = np.random.default_rng(hq * 7 + qmax)
    ctx = np.array([1, 2, 15, 16, 17, 31, 33, 64, 100, 700, 3000, 4100], dtype=np.int32)
    new = np.minimum(rng.integers(1, qmax, size=len(ctx), endpoint=True), ctx).astype(np.int32)
    new[-1] = qmax
    wl = workloads.custom("short_chunks", ctx, new, 0, hq, hkv, 128, seed=hq * 131 + qmax)
    _, _, errs = run_layer_and_check(wl, fused=fused)
    _report(f"short chunks G={hq // hkv} n<={qmax} fused={fused}", errs)


@pytest.mark.parametrize("part", [64, 128, 256, 1024, 4096])
def test_short_chunk_splits(part):
    """The same with the context cut into fixed splits (some empty for the
    short contexts), merged by log-sum-exp; 4096: each context (up to 4,096
    tokens) in one split, no merge."""
    ctx = [1, 16, 100, 700, 1500, 3000, 4096]
    new = [1, 4, 4, 3, 4, 2, 4]
    wl = workloads.custom("short_chunk_splits", ctx, new, 0, 12, 2, 128, seed=part)
    _, _, errs = run_layer_and_check(wl, kv_partition_tokens=part)
    _report(f"short chunks part={part}", errs)


def test_decodes_then_short_chunks():
    """Single-token decodes (decode kernel) then short packed chunks."""
    ctx = [512, 17, 1000, 33, 16, 250, 4096, 9]
    new = [1, 1, 1, 5, 2, 5, 4, 3]
    wl = workloads.custom("decode_then_short", ctx, new, 3, 12, 2, 128, seed=47)
    _, _, errs = run_layer_and_check(wl)
    _report("decodes then short chunks", errs)
