"""Step orchestration: one continuous-batching step over all layers.

The batch is re-formed before every pass (deepconcepts.dev, "Continuous
Batching Is Not a Bigger Batch", section "What the scheduler does on one
step"), so block tables, context lengths and query offsets are step-level
metadata shared by every layer, while the pools are per layer.  Per step:

    pkv_decode_schedule                   (once, when the step uses the balanced
                                           split of the decode work)
    pkv_slot_mapping                      (once)
    for every layer:
        pkv_append_attention_step         (this layer's new K/V into its pool,
                                           decode + merge [+ prefill chunks])
    or, with fused=False, the two halves as separate calls:
        pkv_kv_append ; pkv_paged_attention_step

all enqueued on one stream; append precedes attention within a layer.
`Step.capture` records that whole sequence once as a HIP graph, so a step
costs one graph launch on the host instead of 1 + L (or 2 + 2L) library
calls ([SB] "What changed": per-pass launch overhead is what grows with the
number of launches).  The library's calls only enqueue kernels (no
allocation, no memset, no synchronisation), which is what makes them
capturable; the graph keeps the buffers' addresses, so a replay reads and
writes the same tensors, whose contents the caller refreshes between steps.

The balanced schedule is used by default only in steps that carry prefill
chunks.  There the one context-length hint of the attention call covers the
chunk's context, so the fixed partition grid would be cut for a context longer
than any decode has and would leave much of the GPU idle; the schedule is cut
from the actual context lengths on the device.  In pure decode steps the grid
is cut from the true longest context, and on the measured workloads it is the
faster of the two.
"""
from __future__ import annotations

import numpy as np

from . import (AttentionLayers, KVCache, append_attention_step, attention_workspace_size,
               decode_schedule, decode_schedule_size, kv_append, paged_attention_step,
               slot_mapping)


class Step:
    def __init__(self, block_tables, context_lens, new_tokens, num_decode_seqs: int,
                 num_q_heads: int, num_kv_heads: int, head_dim: int, scale: float,
                 kv_partition_tokens: int = 0, device="cuda", use_schedule: bool | None = None):
        import torch

        bt = np.ascontiguousarray(block_tables, dtype=np.int32)
        ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
        new = np.ascontiguousarray(new_tokens, dtype=np.int32)
        self.num_seqs = int(ctx.shape[0])
        self.num_decode_seqs = int(num_decode_seqs)
        self.num_tokens = int(new.sum())
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.scale = float(scale)
        self.max_context_len = int(ctx.max()) if self.num_seqs else 1
        self.max_query_len = int(new.max()) if self.num_seqs else 1
        self.kv_partition_tokens = int(kv_partition_tokens)
        self.block_tables = torch.from_numpy(bt).to(device)
        self.context_lens = torch.from_numpy(ctx).to(device)
        pure_decode = self.num_decode_seqs == self.num_seqs
        qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
        self.query_start_loc = None if pure_decode else torch.from_numpy(qsl).to(device)
        self.slot_mapping = torch.empty(max(self.num_tokens, 1), dtype=torch.int64, device=device)
        ws = attention_workspace_size(self.num_seqs, self.num_decode_seqs, num_q_heads,
                                      num_kv_heads, head_dim, self.max_context_len,
                                      self.max_query_len, self.kv_partition_tokens)
        self.workspace_bytes = ws
        self.workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
        self.max_blocks_per_seq = int(bt.shape[1])
        if use_schedule is None:
            use_schedule = not pure_decode
        sb = decode_schedule_size(self.num_decode_seqs, num_kv_heads, head_dim,
                                  self.max_context_len) if use_schedule else 0
        self.schedule = torch.empty(sb, dtype=torch.uint8, device=device) if sb else None

    @classmethod
    def from_workload(cls, wl, kv_partition_tokens: int = 0, device="cuda",
                      use_schedule: bool | None = None):
        return cls(wl.block_tables, wl.context_lens, wl.new_tokens, wl.num_decode_seqs,
                   wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.scale,
                   kv_partition_tokens=kv_partition_tokens, device=device,
                   use_schedule=use_schedule)

    def plan(self, stream=None):
        """Per-step work shared by all layers: the balanced decode schedule
        (when the step has one) and the slot of every new token."""
        if self.schedule is not None:
            decode_schedule(self.context_lens, self.num_decode_seqs, self.num_kv_heads,
                            self.head_dim, self.max_blocks_per_seq, self.max_context_len,
                            self.schedule, stream=stream)
        slot_mapping(self.block_tables, self.context_lens, self.query_start_loc, self.num_tokens,
                     self.slot_mapping, stream=stream)

    def capture(self, layers, fused: bool = True):
        """One HIP graph of the whole step: plan() then every layer's call.

        layers: per layer (cache, q, k_new, v_new, out).  Returns a
        torch.cuda.CUDAGraph; graph.replay() enqueues the step on the current
        stream.  Nothing is allocated during capture."""
        import torch
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=side):
            self.plan()
            for cache, q, k_new, v_new, out in layers:
                self.layer(cache, q, k_new, v_new, out, fused=fused)
        torch.cuda.current_stream().wait_stream(side)
        return graph

    def prepare_layers(self, layers):
        """One library call per step for all layers (pkv_append_attention_layers).

        layers: per layer (cache, q, k_new, v_new, out), tensors that stay
        allocated.  Returns run(stream=None): plan() then every layer's
        append + attention, as plan() followed by layer(..., fused=True) per
        layer."""
        caches, qs, ks, vs, outs = (list(x) for x in zip(*layers))
        batch = AttentionLayers(caches, ks, vs, qs, outs)

        def attend(stream=None):
            batch(self.slot_mapping, self.block_tables, self.context_lens, self.query_start_loc,
                  self.num_decode_seqs, self.scale, self.max_context_len, self.max_query_len,
                  workspace=self.workspace, kv_partition_tokens=self.kv_partition_tokens,
                  stream=stream, schedule=self.schedule)

        def run(stream=None):
            self.plan(stream=stream)
            attend(stream)
        run.attend = attend  # the layers' call alone (plan() already done)
        return run

    def layer(self, cache: KVCache, q, k_new, v_new, out, stream=None, fused: bool = True):
        """Append this layer's new K/V, then attend (one call when fused)."""
        if fused:
            return append_attention_step(
                cache, k_new, v_new, self.slot_mapping, q, out, self.block_tables,
                self.context_lens, self.query_start_loc, self.num_decode_seqs, self.scale,
                self.max_context_len, self.max_query_len, workspace=self.workspace,
                kv_partition_tokens=self.kv_partition_tokens, stream=stream,
                schedule=self.schedule)
        kv_append(cache, k_new, v_new, self.slot_mapping, stream=stream)
        paged_attention_step(cache, q, out, self.block_tables, self.context_lens,
                             self.query_start_loc, self.num_decode_seqs, self.scale,
                             self.max_context_len, self.max_query_len,
                             workspace=self.workspace,
                             kv_partition_tokens=self.kv_partition_tokens, stream=stream,
                             schedule=self.schedule)
        return out
