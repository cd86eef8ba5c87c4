"""pkv_append_attention_layers (every layer of a step in one call) against
the per-layer pkv_append_attention_step calls it stands for: the outputs and
the pools after the step must be the same bits, on fp16 and fp8 caches, for
decode steps with split contexts and for steps with prefill chunks."""
import numpy as np
import pytest
import torch

import paged_kv_decode_append_amd as pkv
import workloads
from paged_kv_decode_append_amd.step import Step
from parity import host_bits

pytestmark = pytest.mark.gpu

LAYERS = 3
CASES = {
    # decodes only, contexts cut into partitions (merge launches)
    "decode": ([1, 17, 300, 1025, 2500, 4100], [1] * 6, 6),
    # decodes + long chunks (prefill kernel + its merge, chunk append)
    "mixed": ([40, 700, 3000, 200, 1300], [1, 1, 1, 130, 70], 3),
    # multi-token decodes (packed rows)
    "spec": ([64, 500, 2000, 3300], [4, 4, 4, 4], 0),
}


def _tensors(wl, kv_dtype):
    if kv_dtype == "fp8":
        ts = [workloads.layer_tensors_fp8(wl, l, device="cuda") for l in range(LAYERS)]
        caches = [pkv.KVCache(t["k_codes"], t["v_codes"], t["k_scale"], t["v_scale"]) for t in ts]
        pools = ("k_codes", "v_codes", "k_scale", "v_scale")
    else:
        ts = [workloads.layer_tensors(wl, l, device="cuda") for l in range(LAYERS)]
        caches = [pkv.KVCache(t["k_pool"], t["v_pool"]) for t in ts]
        pools = ("k_pool", "v_pool")
    outs = [torch.full_like(t["q"], float("nan")) for t in ts]
    return ts, caches, outs, pools


def _bits(t):
    return host_bits(t) if t.dtype == torch.float16 else t.cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
@pytest.mark.parametrize("case", list(CASES))
def test_layers_call_equals_per_layer_calls(case, kv_dtype):
    ctx, new, ndec = CASES[case]
    wl = workloads.custom(f"layers_{case}", ctx, new, ndec, 12, 2, 128, layers=LAYERS, seed=43)
    ta, ca, oa, pools = _tensors(wl, kv_dtype)
    tb, cb, ob, _ = _tensors(wl, kv_dtype)
    step = Step.from_workload(wl)
    step.plan()
    for c, t, o in zip(ca, ta, oa):
        step.layer(c, t["q"], t["k_new"], t["v_new"], o, fused=True)
    run = step.prepare_layers([(c, t["q"], t["k_new"], t["v_new"], o)
                               for c, t, o in zip(cb, tb, ob)])
    run()
    torch.cuda.synchronize()
    for l in range(LAYERS):
        assert np.array_equal(host_bits(oa[l]), host_bits(ob[l])), f"out of layer {l}"
        assert not np.isnan(oa[l].float().cpu().numpy()).any()
        for n in pools:
            assert np.array_equal(_bits(ta[l][n]), _bits(tb[l][n])), f"{n} of layer {l}"
    print(f"[layers] {case} {kv_dtype}: {LAYERS} layers in one call, same bits", flush=True)
