"""HIP-graph capture of a whole step (Step.capture): every replay gives the
same bits as the eager step, in the outputs and in the pools after the
append, with eager work and synchronisations between the replays."""
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
    }


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("name", list(_cases()))
def test_graph_replays_match_the_eager_step(name, fused):
    wl, kw = _cases()[name]
    L = wl.num_layers
    ts = [workloads.layer_tensors(wl, l, device="cuda") for l in range(L)]
    k0 = [t["k_pool"].clone() for t in ts]
    v0 = [t["v_pool"].clone() for t in ts]
    caches = [pkv.KVCache(t["k_pool"], t["v_pool"]) for t in ts]
    outs = [torch.empty_like(t["q"]) for t in ts]
    step = Step.from_workload(wl, **kw)
    if name == "mixed_scheduled":
        assert step.schedule is not None

    def restore():
        for l in range(L):
            ts[l]["k_pool"].copy_(k0[l])
            ts[l]["v_pool"].copy_(v0[l])
            outs[l].fill_(float("nan"))

    restore()
    step.plan()
    for c, t, o in zip(caches, ts, outs):
        step.layer(c, t["q"], t["k_new"], t["v_new"], o, fused=fused)
    torch.cuda.synchronize()
    ref_out = [o.clone() for o in outs]
    ref_k = [t["k_pool"].clone() for t in ts]
    ref_v = [t["v_pool"].clone() for t in ts]
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
            assert torch.equal(ts[l]["k_pool"].view(torch.int16), ref_k[l].view(torch.int16))
            assert torch.equal(ts[l]["v_pool"].view(torch.int16), ref_v[l].view(torch.int16))
        print(f"[graph] {name} fused={fused} replay {rep}: identical to eager", flush=True)
