"""GPU tests of the balanced decode schedule (pkv_decode_schedule) and of the
decode kernel that runs on it: the schedule covers every block of every
(sequence, KV head) exactly once, and attention on it matches the CPU
oracle for shapes that stress the packing (many tiny contexts, one huge
context among tiny ones, contexts of one token)."""
import numpy as np
import pytest
import torch

import paged_kv_decode_append_amd as pkv
import workloads
from parity import run_layer_and_check

pytestmark = pytest.mark.gpu

SEG_COST = 2       # fixed cost of a segment in the schedule, in blocks
INLINE = 4         # descriptors inside a work-group's record
REC_WORDS = 4 + 4 * INLINE


def _report(name, errs):
    print(f"[parity] {name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}", flush=True)


def _schedule(ctx, hkv, max_blocks):
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    B = len(ctx)
    nbytes = pkv.decode_schedule_size(B, hkv, 128, int(max(ctx)))
    assert nbytes > 0
    buf = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    pkv.decode_schedule(ctx_t, B, hkv, 128, max_blocks, int(max(ctx)), buf)
    torch.cuda.synchronize()
    return buf.cpu().numpy().view(np.int32)


@pytest.mark.parametrize("case", ["ragged", "tiny_many", "huge_and_tiny", "uniform_short"])
def test_schedule_covers_every_block_once(case):
    rng = np.random.default_rng(7)
    if case == "ragged":
        ctx = (rng.choice([16, 64, 256, 1024, 4096], 83) + rng.integers(0, 257, 83)).tolist()
    elif case == "tiny_many":
        ctx = rng.integers(1, 40, 3000).tolist()
    elif case == "huge_and_tiny":
        ctx = [100_000] + rng.integers(1, 30, 500).tolist()
    else:
        ctx = [17] * 64
    hkv = 2
    max_blocks = -(-max(ctx) // 16)
    words = _schedule(ctx, hkv, max_blocks)
    W, nwg, U = int(words[0]), int(words[1]), int(words[2])
    assert U == len(ctx) * hkv
    nb = np.repeat(-(-np.array(ctx) // 16), hkv)
    cost = nb + SEG_COST
    P = words[4:4 + U].astype(np.int64)
    assert np.array_equal(P, np.cumsum(cost)) and W == P[-1]
    rec0 = 4 + ((U + 3) & ~3)
    ovf0 = rec0 + nwg * REC_WORDS
    covered = [np.zeros(n, np.int32) for n in nb]
    slots = set()
    for w in range(nwg):
        rec = words[rec0 + w * REC_WORDS: rec0 + (w + 1) * REC_WORDS]
        n, ob = int(rec[0]), int(rec[1])
        assert 0 <= n <= 128
        for k in range(n):
            d = rec[4 + 4 * k: 8 + 4 * k] if k < INLINE else \
                words[ovf0 + 4 * (ob + k - INLINE): ovf0 + 4 * (ob + k - INLINE) + 4]
            u, jb, je, c = (int(x) for x in d)
            assert 0 <= jb < je <= nb[u] and c == ctx[u // hkv]
            covered[u][jb:je] += 1
            if not (jb == 0 and je == nb[u]):
                assert (u + w) not in slots
                slots.add(u + w)
        # this work-group's blocks are its share of the cost line
        c0, c1 = w * W // nwg, (w + 1) * W // nwg
        assert c1 - c0 <= 2048
    for u in range(U):
        assert (covered[u] == 1).all(), f"unit {u} coverage {covered[u]}"
    # per-unit merge metadata: first work-group holding a piece, work-groups spanned
    um = words[ovf0 + 4 * (U + nwg): ovf0 + 4 * (U + nwg) + 2 * U].reshape(U, 2)
    wg_of = lambda c: -(-(c + 1) * nwg // W) - 1
    for u in range(U):
        b0 = (P[u - 1] if u else 0) + SEG_COST
        b1 = P[u] - 1
        assert um[u, 0] == wg_of(b0) and um[u, 1] == wg_of(b1) - wg_of(b0) + 1


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("hq,hkv", [(12, 2), (8, 1), (4, 2), (12, 3), (16, 4)])
def test_many_tiny_contexts(hq, hkv, fused):
    rng = np.random.default_rng(hq * 10 + hkv)
    ctx = rng.integers(1, 48, 300).tolist() + [700, 2000]
    wl = workloads.custom("tiny", ctx, [1] * len(ctx), len(ctx), hq, hkv, 128, seed=hq + hkv,
                          pool_factor=1.3)
    _, _, errs = run_layer_and_check(wl, fused=fused, use_schedule=True)
    _report(f"tiny contexts G={hq // hkv} Hkv={hkv} fused={fused}", errs)


@pytest.mark.parametrize("fused", [True, False])
def test_one_huge_context_among_tiny_ones(fused):
    rng = np.random.default_rng(3)
    ctx = [30_000] + rng.integers(1, 30, 60).tolist() + [4096, 1, 16, 17]
    wl = workloads.custom("huge_tiny", ctx, [1] * len(ctx), len(ctx), 12, 2, 128, seed=29,
                          pool_factor=1.1)
    _, _, errs = run_layer_and_check(wl, fused=fused, use_schedule=True)
    _report(f"huge + tiny fused={fused}", errs)


def test_single_token_contexts_on_the_schedule():
    ctx = [1] * 700
    wl = workloads.custom("ones", ctx, [1] * 700, 700, 12, 2, 128, seed=31)
    _, _, errs = run_layer_and_check(wl, use_schedule=True)
    _report("700 x ctx 1", errs)


def test_schedule_and_partition_grid_agree():
    """The same ragged step on the balanced schedule and on the partition
    grid: both within tolerance of the oracle (checked in each run) and of
    each other."""
    ctx = [5, 40, 300, 1000, 2500, 4300, 17, 64, 65, 129] * 3
    outs = []
    for use in (True, False):
        wl = workloads.custom("agree", ctx, [1] * len(ctx), len(ctx), 12, 2, 128, seed=37)
        t = workloads.layer_tensors(wl, 0, device="cuda")
        from paged_kv_decode_append_amd.step import Step
        step = Step.from_workload(wl, use_schedule=use)
        assert (step.schedule is not None) == use
        step.plan()
        out = torch.empty_like(t["q"])
        step.layer(pkv.KVCache(t["k_pool"], t["v_pool"]), t["q"], t["k_new"], t["v_new"], out)
        torch.cuda.synchronize()
        outs.append(out.float().cpu().numpy())
    assert np.abs(outs[0] - outs[1]).max() <= 2e-3


def test_pieces_merge_ignores_empty_work_groups():
    """A tiny step has fewer cost units than work-groups, so some work-groups
    between a unit's first and last piece hold nothing: the merge must not
    read their (here NaN-filled) workspace slots."""
    from paged_kv_decode_append_amd.step import Step
    ctx = [7, 40, 129, 700]
    wl = workloads.custom("tiny_w", ctx, [1] * 4, 4, 2, 2, 128, seed=2 + 128)
    t = workloads.layer_tensors(wl, 0, device="cuda")
    step = Step.from_workload(wl, use_schedule=True)
    assert step.schedule is not None
    step.workspace.view(torch.float16).fill_(float("nan")) if step.workspace.numel() % 2 == 0 else None
    _, _, errs = run_layer_and_check(wl, tensors=t, step=step)
    _report("fewer cost units than work-groups", errs)


def test_default_uses_the_schedule_only_with_prefill_chunks():
    from paged_kv_decode_append_amd.step import Step
    dec = workloads.custom("dec", [300, 40], [1, 1], 2, 12, 2, 128)
    mix = workloads.custom("mix", [300, 40, 700], [1, 1, 64], 2, 12, 2, 128)
    assert Step.from_workload(dec).schedule is None
    assert Step.from_workload(mix).schedule is not None
    assert Step.from_workload(dec, use_schedule=True).schedule is not None
