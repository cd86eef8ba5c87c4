"""GPU parity of multi-token decode: sequences that bring a few query tokens
each (the last sampled token plus drafted ones to verify), attended causally
over their whole context.  When every such chunk's G x n rows fit one 64-row
tile, the step packs all G query heads of a KV group into one work-group
(each K/V tile read once per KV head); larger chunks take the per-head path.
Checked against the CPU oracle."""
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
