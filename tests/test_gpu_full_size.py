"""Parity at the benchmark's full workload sizes, in the launch configuration
bench.py times (paged_kv_decode_append_amd.step.Step, automatic split-KV
plan): slot mapping and pools bit-exact, attention checked on sampled
sequences the oracle computes one by one."""
import numpy as np
import pytest

import workloads
from parity import run_layer_and_check

pytestmark = pytest.mark.gpu


def _report(name, errs):
    print(f"[parity] {name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}", flush=True)


@pytest.mark.parametrize("layer", [0, 27])
def test_qwen_uniform_b256_ctx512(layer):
    wl = workloads.qwen_uniform()
    _, _, errs = run_layer_and_check(wl, layer, poison=False, seq_subset=[0, 1, 128, 255])
    _report(f"qwen_uniform layer {layer}", errs)


def test_qwen_ragged_b83():
    wl = workloads.qwen_ragged()
    ctx = wl.context_lens
    # one sequence from each prompt class, plus the longest and the shortest
    picks = {int(np.argmax(ctx)), int(np.argmin(ctx))}
    for lo, hi in ((16, 272), (64, 320), (256, 512), (1024, 1280), (4096, 4352)):
        idx = np.nonzero((ctx >= lo) & (ctx <= hi))[0]
        if len(idx):
            picks.add(int(idx[0]))
    _, _, errs = run_layer_and_check(wl, 3, poison=False, seq_subset=sorted(picks))
    _report("qwen_ragged layer 3", errs)


def test_long_context_b4_262k():
    wl = workloads.long_context()
    _, _, errs = run_layer_and_check(wl, 0, poison=False, seq_subset=[0, 3])
    _report("long_context layer 0", errs)
