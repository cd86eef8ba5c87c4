"""Binding of the host block manager and per-pass scheduler in libpkv.so
(include/pkv_sched.h): argument marshalling only, the decisions are made in
the C++ code.

    s = Scheduler(num_blocks=7281, max_num_seqs=256, max_num_batched_tokens=8192,
                  max_blocks_per_seq=512)
    s.add_request(rid, prompt_len, max_new_tokens)
    while not s.done():
        plan = s.schedule()         # Plan: numpy copies of the pass's arrays
        ...                         # run the pass (append + attention per layer)
        s.complete()

The plan's arrays are what the attention step consumes: block_tables,
context_lens, query_start_loc (decode sequences first) and slot_mapping.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import PKV_OK, PkvError, lib

ALLOC_ON_DEMAND = 0
ALLOC_RESERVE = 1

SCHED_EXPORTED = (
    "pkv_sched_create", "pkv_sched_destroy", "pkv_sched_add_request", "pkv_sched_schedule",
    "pkv_sched_complete", "pkv_sched_get_stats", "pkv_sched_request_blocks",
)


class _Config(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("max_num_seqs", ctypes.c_int32), ("max_num_batched_tokens", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("alloc_policy", ctypes.c_int32)]


class _Plan(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_decode_seqs", ctypes.c_int32),
                ("num_tokens", ctypes.c_int32), ("max_context_len", ctypes.c_int32),
                ("max_query_len", ctypes.c_int32),
                ("request_ids", ctypes.POINTER(ctypes.c_int64)),
                ("context_lens", ctypes.POINTER(ctypes.c_int32)),
                ("query_start_loc", ctypes.POINTER(ctypes.c_int32)),
                ("block_tables", ctypes.POINTER(ctypes.c_int32)),
                ("slot_mapping", ctypes.POINTER(ctypes.c_int64)),
                ("num_preempted", ctypes.c_int32), ("num_admitted", ctypes.c_int32),
                ("recomputed_tokens", ctypes.c_int64), ("prefix_hit_tokens", ctypes.c_int64)]


class _Stats(ctypes.Structure):
    _fields_ = [("passes", ctypes.c_int64), ("preemptions", ctypes.c_int64),
                ("recomputed_tokens", ctypes.c_int64), ("prefix_hit_tokens", ctypes.c_int64),
                ("generated_tokens", ctypes.c_int64), ("peak_running", ctypes.c_int32),
                ("num_running", ctypes.c_int32), ("num_waiting", ctypes.c_int32),
                ("num_finished", ctypes.c_int32), ("free_blocks", ctypes.c_int64)]


def _setup():
    P = ctypes.c_void_p
    lib.pkv_sched_create.argtypes = [ctypes.POINTER(_Config), P]
    lib.pkv_sched_create.restype = P
    lib.pkv_sched_destroy.argtypes = [P]
    lib.pkv_sched_destroy.restype = None
    lib.pkv_sched_add_request.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_int64, ctypes.c_int32]
    lib.pkv_sched_schedule.argtypes = [P, ctypes.POINTER(_Plan)]
    lib.pkv_sched_complete.argtypes = [P]
    lib.pkv_sched_get_stats.argtypes = [P, ctypes.POINTER(_Stats)]
    lib.pkv_sched_request_blocks.argtypes = [P, ctypes.c_int64, P, ctypes.c_int64]
    lib.pkv_sched_request_blocks.restype = ctypes.c_int64
    for name in ("pkv_sched_add_request", "pkv_sched_schedule", "pkv_sched_complete",
                 "pkv_sched_get_stats"):
        getattr(lib, name).restype = ctypes.c_int


_setup()


@dataclass
class Plan:
    """One pass (numpy copies; decode sequences first)."""
    request_ids: np.ndarray       # int64 [B]
    context_lens: np.ndarray      # int32 [B]
    new_tokens: np.ndarray        # int32 [B]
    query_start_loc: np.ndarray   # int32 [B+1]
    block_tables: np.ndarray      # int32 [B, max_blocks_per_seq]
    slot_mapping: np.ndarray      # int64 [T]
    num_decode_seqs: int
    num_preempted: int
    num_admitted: int
    recomputed_tokens: int
    prefix_hit_tokens: int

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])


class Scheduler:
    def __init__(self, num_blocks: int, max_num_seqs: int, max_num_batched_tokens: int,
                 max_blocks_per_seq: int, alloc_policy: int = ALLOC_ON_DEMAND,
                 free_order=None, block_size: int = 16):
        """free_order: initial order of the free-block queue (a permutation of
        the pool, e.g. a seeded one so that tables scatter), default 0..N-1."""
        cfg = _Config(num_blocks, block_size, max_num_seqs, max_num_batched_tokens,
                      max_blocks_per_seq, alloc_policy)
        order = None if free_order is None else np.ascontiguousarray(free_order, dtype=np.int32)
        if order is not None and order.shape != (num_blocks,):
            raise ValueError("free_order must list every block once")
        h = lib.pkv_sched_create(ctypes.byref(cfg), None if order is None else order.ctypes.data)
        if not h:
            raise ValueError("invalid scheduler configuration")
        self._h = ctypes.c_void_p(h)
        self.max_blocks_per_seq = max_blocks_per_seq

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and lib is not None:  # (lib is None during interpreter shutdown)
            lib.pkv_sched_destroy(h)
            self._h = None

    def add_request(self, request_id: int, prompt_len: int, max_new_tokens: int,
                    prefix_id: int = -1, prefix_len: int = 0):
        rc = lib.pkv_sched_add_request(self._h, request_id, prompt_len, max_new_tokens,
                                       prefix_id, prefix_len)
        if rc != PKV_OK:
            raise PkvError(rc, "pkv_sched_add_request")

    def schedule(self) -> Plan:
        p = _Plan()
        rc = lib.pkv_sched_schedule(self._h, ctypes.byref(p))
        if rc != PKV_OK:
            raise PkvError(rc, "pkv_sched_schedule")
        B, T, W = p.num_seqs, p.num_tokens, self.max_blocks_per_seq

        def arr(ptr, n, dtype):
            if n == 0:
                return np.zeros(0, dtype)
            return np.ctypeslib.as_array(ptr, shape=(n,)).astype(dtype, copy=True)

        qsl = arr(p.query_start_loc, B + 1, np.int32)
        return Plan(request_ids=arr(p.request_ids, B, np.int64),
                    context_lens=arr(p.context_lens, B, np.int32),
                    new_tokens=np.diff(qsl).astype(np.int32),
                    query_start_loc=qsl,
                    block_tables=arr(p.block_tables, B * W, np.int32).reshape(B, W),
                    slot_mapping=arr(p.slot_mapping, T, np.int64),
                    num_decode_seqs=p.num_decode_seqs, num_preempted=p.num_preempted,
                    num_admitted=p.num_admitted, recomputed_tokens=p.recomputed_tokens,
                    prefix_hit_tokens=p.prefix_hit_tokens)

    def complete(self):
        rc = lib.pkv_sched_complete(self._h)
        if rc != PKV_OK:
            raise PkvError(rc, "pkv_sched_complete")

    def stats(self) -> dict:
        st = _Stats()
        rc = lib.pkv_sched_get_stats(self._h, ctypes.byref(st))
        if rc != PKV_OK:
            raise PkvError(rc, "pkv_sched_get_stats")
        return {name: int(getattr(st, name)) for name, _ in _Stats._fields_}

    def request_blocks(self, request_id: int) -> np.ndarray | None:
        cap = self.max_blocks_per_seq
        out = np.zeros(cap, np.int32)
        n = lib.pkv_sched_request_blocks(self._h, request_id, out.ctypes.data, cap)
        return None if n < 0 else out[:n].copy()

    def done(self) -> bool:
        st = self.stats()
        return st["num_running"] == 0 and st["num_waiting"] == 0
