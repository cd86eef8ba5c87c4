"""HIP-graph capture of a whole step (Step.capture): every replay gives the
same bits as the eager step, in the outputs and in the pools after the
append (fp16 pools, or fp8 codes and row scales), with eager work and
synchronisations between the replays."""
import numpy as np
import pytest
import torch

import paged_kv_decode_append_amd as pkv
import workloads
from paged_kv_decode_append_amd.step import Step

pytestmark = pytest.mark.gpu


def _cases():
    rng = np.random.default_rng(11)
    ragged = (rng.choice([16, 64, 256, 1024], 21) + rng.integers(0, 40, 21)).tolist()
    return {
        "small_b4": (workloads.small_b4(layers=3), {}),
        "ragged_split": (workloads.custom("ragged", ragged, [1] * 21, 21, 12, 2, 128, layers=3,
                                          seed=5), {}),
        "forced_partitions": (workloads.custom("parts", [700, 33, 1500], [1] * 3, 3, 8, 1, 128,
                                               layers=2, seed=6), {"kv_partition_tokens": 128}),
        "mixed_scheduled": (workloads.custom("mixed", [300, 900, 45, 1200], [1, 1, 1, 200], 3,
                                             12, 2, 128, layers=3, seed=7), {}),
        "d256": (workloads.custom("d256", [500, 2100, 17], [1] * 3, 3, 16, 4, 256, layers=2,
                                  seed=8), {}),
        # fp8 caches: codes and row scales written by the replays' appends
        "ragged_split_fp8": (workloads.custom("ragged8", ragged, [1] * 21, 21, 12, 2, 128,
                                              layers=3, seed=5), {}),
        "mixed_fp8": (workloads.custom("mixed8", [300, 900, 45, 1200], [1, 1, 1, 200], 3, 12, 2,
                                       128, layers=3, seed=7), {}),
        "d256_fp8": (workloads.custom("d256_8", [500, 2100, 17, 700], [1, 1, 1, 90], 3, 16, 4,
                                      256, layers=2, seed=8), {}),
    }


FP16_POOLS = ("k_pool", "v_pool")
FP8_POOLS = ("k_codes", "v_codes", "k_scale", "v_scale")


def _bits(t):
    """A tensor's raw bits, so that NaN compares equal to itself."""
    return t.view({torch.float16: torch.int16, torch.float32: torch.int32}.get(t.dtype, t.dtype))


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", list(_cases()))
def test_graph_replays_match_the_eager_step(name, fused):
    wl, kw = _cases()[name]
    L = wl.num_layers
    fp8 = name.endswith("_fp8")
    pools = FP8_POOLS if fp8 else FP16_POOLS
    make = workloads.layer_tensors_fp8 if fp8 else workloads.layer_tensors
    ts = [make(wl, l, device="cuda") for l in range(L)]
    saved = [{n: t[n].clone() for n in pools} for t in ts]
    caches = [pkv.KVCache(*(t[n] for n in pools)) for t in ts]
    outs = [torch.empty_like(t["q"]) for t in ts]
    step = Step.from_workload(wl, **kw)
    if name == "mixed_scheduled":
        assert step.schedule is not None

    def restore():
        for l in range(L):
            for n in pools:
                ts[l][n].copy_(saved[l][n])
            outs[l].fill_(float("nan"))

    restore()
    step.plan()
    for c, t, o in zip(caches, ts, outs):
        step.layer(c, t["q"], t["k_new"], t["v_new"], o, fused=fused)
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in outs]
    ref_pools = [{n: t[n].clone() for n in pools} for t in ts]
    assert all(torch.isfinite(o.float()).all() for o in ref_out)

    restore()
    graph = step.capture([(c, t["q"], t["k_new"], t["v_new"], o)
                          for c, t, o in zip(caches, ts, outs)], fused=fused)
    for rep in range(3):
        restore()
        if rep == 1:
            # unrelated eager library work between replays
            other = workloads.small_b4()
            ot = workloads.layer_tensors(other, 0, device="cuda")
            os_ = Step.from_workload(other)
            os_.plan()
            os_.layer(pkv.KVCache(ot["k_pool"], ot["v_pool"]), ot["q"], ot["k_new"], ot["v_new"],
                      torch.empty_like(ot["q"]))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for l in range(L):
            assert torch.equal(outs[l].view(torch.int16), ref_out[l].view(torch.int16)), \
                f"replay {rep} layer {l}: output differs from the eager step"
            for n in pools:
                assert torch.equal(_bits(ts[l][n]), _bits(ref_pools[l][n])), \
                    f"replay {rep} layer {l}: {n} differs from the eager step"
        print(f"[graph] {name} fused={fused} replay {rep}: identical to eager", flush=True)
