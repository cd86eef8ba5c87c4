"""Parity at the benchmark's full workload sizes, in the launch configuration
bench.py times (paged_kv_decode_append_amd.step.Step, automatic split-KV
plan): slot mapping and pools bit-exact, attention of every sequence
checked against the oracle."""
import pytest

import workloads
from parity import run_layer_and_check

pytestmark = pytest.mark.gpu


def _report(name, errs):
    print(f"[parity] {name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}", flush=True)


@pytest.mark.parametrize("layer", [0, 27])
def test_qwen_uniform_b256_ctx512(layer):
    wl = workloads.qwen_uniform()
    _, _, errs = run_layer_and_check(wl, layer, poison=False)
    _report(f"qwen_uniform layer {layer} (all 256 sequences)", errs)


def test_qwen_ragged_b83():
    wl = workloads.qwen_ragged()
    _, _, errs = run_layer_and_check(wl, 3, poison=False)
    _report("qwen_ragged layer 3 (all 83 sequences)", errs)


def test_long_context_b4_262k():
    wl = workloads.long_context()
    _, _, errs = run_layer_and_check(wl, 0, poison=False)
    _report("long_context layer 0 (all 4 sequences)", errs)
