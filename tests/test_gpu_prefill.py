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
    decode sequences sampled, chunk rows sampled across all 8 row tiles."""
    wl = workloads.qwen_mixed()
    chunk_seq = wl.num_seqs - 1
    rows = [0, 1, 15, 16, 63, 64, 127, 200, 255, 256, 300, 383, 448, 500, 510, 511]
    _, _, errs = run_layer_and_check(wl, 5, poison=False, seq_subset=[0, 17, 40, 63],
                                     row_samples={chunk_seq: rows})
    _report("qwen_mixed layer 5", errs)
