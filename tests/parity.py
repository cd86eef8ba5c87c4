"""Helpers for the GPU parity tests: run the HIP path exactly as the bench
does (paged_kv_decode_append_amd.step.Step) and compare with the oracle.

Expected values come only from ``oracle`` applied to the generator's
inputs (read back as exact fp16 bits); nothing the HIP path computes is fed
to the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import paged_kv_decode_append_amd as pkv
from paged_kv_decode_append_amd.step import Step

# Attention tolerance for fp16 inputs with fp32 accumulation: max |diff|
# <= 2e-3 elementwise AND, per (row, head) vector, ||diff||_2 <= 1e-2 ||ref||_2.
ATOL = 2e-3
RTOL_NORM = 1e-2


def errors(got_fp16: np.ndarray, ref: np.ndarray):
    g = got_fp16.astype(np.float64)
    diff = g - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    num = np.linalg.norm(diff, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    rel = float((num / np.maximum(den, 1e-300)).max()) if diff.size else 0.0
    return max_abs, rel


def assert_close(got_fp16: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.isfinite(got_fp16.astype(np.float64)).all(), f"{what}: non-finite output"
    max_abs, rel = errors(got_fp16, ref)
    assert max_abs <= ATOL and rel <= RTOL_NORM, f"{what}: max_abs={max_abs:.3e} norm_rel={rel:.3e}"
    return max_abs, rel


def all_position_slots(wl, tables=None):
    """Pool slots of every context position [0, ctx_i) of every sequence
    (the oracle's slot arithmetic applied to a query covering whole contexts)."""
    tables = wl.block_tables if tables is None else tables
    qsl = np.concatenate([[0], np.cumsum(wl.context_lens)]).astype(np.int32)
    return oracle.slot_mapping(tables, wl.context_lens, qsl, wl.block_size)


def poison_stale(wl, tensors, poison_table_tail=True, poison_new=True):
    """NaN (0x7E00) in every pool slot outside the sequences' contexts, and
    point table entries past ceil(ctx/16) at a poisoned free block.  With
    poison_new, the slots the step's new tokens are appended to hold NaN too
    before the step: an attention that read one of them before (or instead
    of) its append would give NaN."""
    live = np.zeros(wl.num_blocks * wl.block_size, bool)
    live[all_position_slots(wl)] = True
    if poison_new:
        qsl = wl.query_start_loc if wl.num_decode_seqs < wl.num_seqs else None
        new_slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, qsl, wl.block_size)
        live[new_slots[new_slots >= 0]] = False
    dead = torch.from_numpy(np.nonzero(~live)[0]).to(tensors["k_pool"].device)
    for name in ("k_pool", "v_pool"):
        view = tensors[name].transpose(1, 2)          # [NB, 16, Hkv, d] view of the pool
        view[dead // wl.block_size, dead % wl.block_size] = float("nan")
    if poison_table_tail and len(wl.free_blocks):
        used = -(-wl.context_lens // wl.block_size)
        for i, u in enumerate(used):
            wl.block_tables[i, u:] = wl.free_blocks[0]


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def run_layer_and_check(wl, layer: int = 0, kv_partition_tokens: int = 0, poison: bool = True,
                        seq_subset=None, tensors=None, row_samples=None, fused: bool = True,
                        step=None, use_schedule=None):
    """One layer of one step on the GPU, checked against the oracle.

    fused: the layer runs as pkv_append_attention_step (the benchmark's
    path), else as pkv_kv_append followed by pkv_paged_attention_step.

    Checks: slot mapping bit-exact; whole pools after the append bit-exact
    (canaries and NaN poison included); attention within tolerance for the
    sequences in seq_subset (all when None), and for row_samples
    {sequence: [chunk rows]} of long prefill chunks, each sampled row checked
    as the query that attends positions [0, its position] through the same
    block table.  Returns (out_fp16, ref, errors).
    """
    t = workloads_tensors(wl, layer) if tensors is None else tensors
    if poison:
        poison_stale(wl, t)
    kp0, vp0 = host_bits(t["k_pool"]), host_bits(t["v_pool"])
    q, kn, vn = host_bits(t["q"]), host_bits(t["k_new"]), host_bits(t["v_new"])

    if step is None:
        step = Step.from_workload(wl, kv_partition_tokens=kv_partition_tokens,
                                  use_schedule=use_schedule)
    step.plan()
    cache = pkv.KVCache(t["k_pool"], t["v_pool"])
    out = torch.full_like(t["q"], float("nan"))
    step.layer(cache, t["q"], t["k_new"], t["v_new"], out, fused=fused)
    torch.cuda.synchronize()

    qsl = wl.query_start_loc if wl.num_decode_seqs < wl.num_seqs else None
    slots_ref = oracle.slot_mapping(wl.block_tables, wl.context_lens, qsl, wl.block_size)
    assert np.array_equal(step.slot_mapping[: wl.num_tokens].cpu().numpy(), slots_ref), "slot mapping"

    kp_ref, vp_ref = oracle.kv_append(kp0, vp0, kn, vn, slots_ref)
    assert np.array_equal(host_bits(t["k_pool"]), kp_ref), "K pool after append"
    assert np.array_equal(host_bits(t["v_pool"]), vp_ref), "V pool after append"

    got = out.cpu().numpy()
    ref = None
    errs = (0.0, 0.0)
    if seq_subset is None or len(seq_subset):
        ref = oracle.paged_attention(q, kp_ref, vp_ref, wl.block_tables, wl.context_lens, qsl,
                                     wl.scale, seq_subset=seq_subset)
        rows = rows_of(wl, seq_subset)
        errs = assert_close(got[rows], ref[rows], wl.name)
    for seq, sample in (row_samples or {}).items():
        sample = np.asarray(sample)
        n, ctx, r0 = wl.new_tokens[seq], wl.context_lens[seq], wl.query_start_loc[seq]
        sub_ctx = (ctx - n + sample + 1).astype(np.int32)
        sub_bt = np.repeat(wl.block_tables[seq:seq + 1], len(sample), axis=0)
        sub_ref = oracle.paged_attention(q[r0 + sample], kp_ref, vp_ref, sub_bt, sub_ctx, None,
                                         wl.scale)
        e2 = assert_close(got[r0 + sample], sub_ref, f"{wl.name} rows of sequence {seq}")
        errs = (max(errs[0], e2[0]), max(errs[1], e2[1]))
    return got, ref, errs


def rows_of(wl, seq_subset):
    if seq_subset is None:
        return np.arange(wl.num_tokens)
    qsl = wl.query_start_loc
    return np.concatenate([np.arange(qsl[i], qsl[i + 1]) for i in seq_subset])


def workloads_tensors(wl, layer):
    import workloads
    return workloads.layer_tensors(wl, layer, device="cuda")
