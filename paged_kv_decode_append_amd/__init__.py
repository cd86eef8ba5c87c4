"""Python binding of libpkv.so (paged KV append + paged attention for MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libpkv.so; torch supplies device memory and the stream.  The names follow
the C ABI in include/pkv.h without the ``pkv_`` prefix:

    slot_mapping, kv_append, attention_workspace_size, decode_schedule_size,
    decode_schedule, paged_attention_step, append_attention_step,
    append_attention_step_noalloc, validate_step, hbm_read_probe, status_string,
    last_hip_error, version

There is no fallback: importing this package without a built libpkv.so
raises, and every call raises PkvError on a non-OK status.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the same library (e.g. one whose host
# code is built with sanitizers); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
PKV_ERR_CONTRACT = -5

# every symbol include/pkv.h declares
EXPORTED = (
    "pkv_version", "pkv_status_string", "pkv_last_hip_error", "pkv_slot_mapping", "pkv_kv_append",
    "pkv_attention_workspace_size", "pkv_decode_schedule_size", "pkv_decode_schedule",
    "pkv_paged_attention_step", "pkv_append_attention_step", "pkv_append_attention_layers",
    "pkv_append_attention_step_noalloc", "pkv_validate_step", "pkv_hbm_read_probe",
)

# work-groups of pkv_hbm_read_probe (words of its sink)
PROBE_SINK_WORDS = 4096

# bytes of the device scratch behind pkv_append_attention_step_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20


class PkvError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = f"{what}: {status_string(status)} ({status})"
        if status == PKV_ERR_HIP:
            code, name = last_hip_error()
            msg += f" [HIP error {code}: {name}]"
        super().__init__(msg)
        self.status = status


PKV_KV_FP16 = 0
PKV_KV_FP8_E4M3 = 1


class _Cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p)]


def _load():
    # torch ships its own libamdhip64.so.7 with the same soname as the
    # system one; importing torch first makes libpkv.so bind to the HIP
    # runtime torch already uses, so one runtime owns the device, the
    # memory and the streams in this process.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python paged_kv_decode_append_amd/build.py` "
                          "or __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pkv_version.restype = ctypes.c_int
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_last_hip_error.argtypes = [ctypes.POINTER(ctypes.c_char_p)]
    lib.pkv_slot_mapping.argtypes = [P, i32, P, P, i32, i32, i32, P, P]
    lib.pkv_kv_append.argtypes = [ctypes.POINTER(_Cache), P, P, P, i32, P]
    lib.pkv_attention_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32,
                                                 ctypes.POINTER(ctypes.c_size_t)]
    sz = ctypes.c_size_t
    lib.pkv_decode_schedule_size.argtypes = [i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.pkv_decode_schedule.argtypes = [P, i32, i32, i32, i32, i32, P, sz, P]
    lib.pkv_paged_attention_step.argtypes = [ctypes.POINTER(_Cache), P, P, P, i32, P, P, i32, i32,
                                             i32, ctypes.c_float, i32, i32, i32, P, sz, P, sz, P]
    lib.pkv_append_attention_step.argtypes = [ctypes.POINTER(_Cache), P, P, P, i32, P, P, P, i32,
                                              P, P, i32, i32, i32, ctypes.c_float, i32, i32, i32,
                                              P, sz, P, sz, P]
    lib.pkv_append_attention_step_noalloc.argtypes = [
        ctypes.POINTER(_Cache), P, P, P, i32, P, P, P, i32, P, P, i32, i32, i32, ctypes.c_float,
        i32, i32, i32, P, sz, P]
    lib.pkv_append_attention_layers.argtypes = [ctypes.POINTER(_Cache), i32, P, P, P, i32, P, P,
                                                P, i32, P, P, i32, i32, i32, ctypes.c_float, i32,
                                                i32, i32, P, sz, P, sz, P]
    lib.pkv_hbm_read_probe.argtypes = [P, sz, P, i64, i32, i32, P, P]
    lib.pkv_validate_step.argtypes = [P, i32, P, P, i32, i32, i64, i32, P, i32, i32, i32,
                                      ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    for name in EXPORTED:
        getattr(lib, name).restype = getattr(lib, name).restype or ctypes.c_int
    return lib


lib = _load()


def version() -> int:
    return int(lib.pkv_version())


def status_string(status: int) -> str:
    return lib.pkv_status_string(int(status)).decode()


def last_hip_error():
    """(hipError_t code, name) behind the last PKV_ERR_HIP on this thread."""
    name = ctypes.c_char_p()
    code = lib.pkv_last_hip_error(ctypes.byref(name))
    return int(code), (name.value or b"").decode()


def _check(rc: int, what: str):
    if rc != PKV_OK:
        raise PkvError(rc, what)


def _ptr(t):
    """Device (or host) address of a tensor / numpy array, or None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class KVCache:
    """One layer's pools: k_pool, v_pool [num_blocks, num_kv_heads, 16, head_dim],
    fp16 values, or (with k_scale / v_scale fp32 [num_blocks, num_kv_heads, 16])
    uint8 fp8-E4M3 codes of a quantized cache."""

    def __init__(self, k_pool, v_pool, k_scale=None, v_scale=None):
        import torch
        fp8 = k_scale is not None or v_scale is not None
        dt = torch.uint8 if fp8 else torch.float16
        _need(k_pool, dt, "k_pool")
        _need(v_pool, dt, "v_pool")
        if k_pool.shape != v_pool.shape or k_pool.dim() != 4:
            raise ValueError("k_pool and v_pool must share a 4-d shape")
        self.k_pool, self.v_pool = k_pool, v_pool
        nb, hkv, bs, d = k_pool.shape
        self.k_scale, self.v_scale = k_scale, v_scale
        if fp8:
            _need(k_scale, torch.float32, "k_scale")
            _need(v_scale, torch.float32, "v_scale")
            if tuple(k_scale.shape) != (nb, hkv, bs) or tuple(v_scale.shape) != (nb, hkv, bs):
                raise ValueError("scales must be [num_blocks, num_kv_heads, block_size]")
            self._c = _Cache(k_pool.data_ptr(), v_pool.data_ptr(), nb, bs, hkv, d,
                             PKV_KV_FP8_E4M3, k_scale.data_ptr(), v_scale.data_ptr())
        else:
            self._c = _Cache(k_pool.data_ptr(), v_pool.data_ptr(), nb, bs, hkv, d,
                             PKV_KV_FP16, None, None)

    @property
    def is_fp8(self):
        return self._c.kv_dtype == PKV_KV_FP8_E4M3

    @property
    def num_blocks(self):
        return self._c.num_blocks

    @property
    def num_kv_heads(self):
        return self._c.num_kv_heads

    @property
    def head_dim(self):
        return self._c.head_dim

    @property
    def block_size(self):
        return self._c.block_size


def slot_mapping(block_tables, context_lens, query_start_loc, num_tokens: int, out,
                 block_size: int = 16, stream=None):
    """pkv_slot_mapping: int64 slot of every new token into `out` [num_tokens]."""
    import torch
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if query_start_loc is not None:
        _need(query_start_loc, torch.int32, "query_start_loc")
    _need(out, torch.int64, "out")
    if out.numel() < num_tokens:
        raise ValueError("out is smaller than num_tokens")
    rc = lib.pkv_slot_mapping(_ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                              _ptr(query_start_loc), context_lens.shape[0], num_tokens,
                              block_size, _ptr(out), _stream(stream))
    _check(rc, "pkv_slot_mapping")
    return out


def kv_append(cache: KVCache, k_new, v_new, slot_mapping_t, stream=None):
    """pkv_kv_append: write k_new/v_new [T, Hkv, d] rows into their slots."""
    import torch
    _need(k_new, torch.float16, "k_new")
    _need(v_new, torch.float16, "v_new")
    _need(slot_mapping_t, torch.int64, "slot_mapping")
    T = k_new.shape[0]
    if v_new.shape != k_new.shape or k_new.shape[1:] != (cache.num_kv_heads, cache.head_dim):
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    if slot_mapping_t.numel() < T:
        raise ValueError("slot_mapping shorter than the token count")
    rc = lib.pkv_kv_append(ctypes.byref(cache._c), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping_t),
                           T, _stream(stream))
    _check(rc, "pkv_kv_append")


def attention_workspace_size(num_seqs, num_decode_seqs, num_q_heads, num_kv_heads, head_dim,
                             max_context_len, max_query_len, kv_partition_tokens=0) -> int:
    out = ctypes.c_size_t(0)
    rc = lib.pkv_attention_workspace_size(num_seqs, num_decode_seqs, num_q_heads, num_kv_heads,
                                          head_dim, max_context_len, max_query_len,
                                          kv_partition_tokens, ctypes.byref(out))
    _check(rc, "pkv_attention_workspace_size")
    return int(out.value)


def decode_schedule_size(num_decode_seqs, num_kv_heads, head_dim, max_context_len) -> int:
    """pkv_decode_schedule_size: bytes of the per-step decode schedule (0: not used)."""
    out = ctypes.c_size_t(0)
    rc = lib.pkv_decode_schedule_size(num_decode_seqs, num_kv_heads, head_dim, max_context_len,
                                      ctypes.byref(out))
    _check(rc, "pkv_decode_schedule_size")
    return int(out.value)


def decode_schedule(context_lens, num_decode_seqs: int, num_kv_heads: int, head_dim: int,
                    max_blocks_per_seq: int, max_context_len: int, schedule, stream=None):
    """pkv_decode_schedule: balanced split of the step's decode work into `schedule`
    (uint8 device tensor of decode_schedule_size bytes)."""
    import torch
    _need(context_lens, torch.int32, "context_lens")
    nbytes = 0
    if schedule is not None:
        _need(schedule, torch.uint8, "schedule")
        nbytes = schedule.numel()
    rc = lib.pkv_decode_schedule(_ptr(context_lens), num_decode_seqs, num_kv_heads, head_dim,
                                 max_blocks_per_seq, max_context_len, _ptr(schedule), nbytes,
                                 _stream(stream))
    _check(rc, "pkv_decode_schedule")
    return schedule


def _schedule_args(schedule):
    import torch
    if schedule is None:
        return None, 0
    _need(schedule, torch.uint8, "schedule")
    return _ptr(schedule), schedule.numel()


def paged_attention_step(cache: KVCache, q, out, block_tables, context_lens, query_start_loc,
                         num_decode_seqs: int, scale: float, max_context_len: int,
                         max_query_len: int, workspace=None, kv_partition_tokens: int = 0,
                         stream=None, schedule=None):
    """pkv_paged_attention_step over one layer; q/out fp16 [T, Hq, d]."""
    import torch
    _need(q, torch.float16, "q")
    _need(out, torch.float16, "out")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if query_start_loc is not None:
        _need(query_start_loc, torch.int32, "query_start_loc")
    if out.shape != q.shape or q.dim() != 3 or q.shape[2] != cache.head_dim:
        raise ValueError("q and out must be [T, num_q_heads, head_dim]")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    sched_ptr, sched_bytes = _schedule_args(schedule)
    rc = lib.pkv_paged_attention_step(
        ctypes.byref(cache._c), _ptr(q), _ptr(out), _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), _ptr(query_start_loc), context_lens.shape[0], num_decode_seqs,
        q.shape[1], float(scale), int(max_context_len), int(max_query_len),
        int(kv_partition_tokens), sched_ptr, sched_bytes, _ptr(workspace), ws_bytes,
        _stream(stream))
    _check(rc, "pkv_paged_attention_step")
    return out


def append_attention_step(cache: KVCache, k_new, v_new, slot_mapping_t, q, out, block_tables,
                          context_lens, query_start_loc, num_decode_seqs: int, scale: float,
                          max_context_len: int, max_query_len: int, workspace=None,
                          kv_partition_tokens: int = 0, stream=None, schedule=None):
    """pkv_append_attention_step: kv_append then paged_attention_step in one
    call, the decode tokens appended inside the decode kernel."""
    import torch
    for t, name in ((k_new, "k_new"), (v_new, "v_new"), (q, "q"), (out, "out")):
        _need(t, torch.float16, name)
    _need(slot_mapping_t, torch.int64, "slot_mapping")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if query_start_loc is not None:
        _need(query_start_loc, torch.int32, "query_start_loc")
    T = k_new.shape[0]
    if v_new.shape != k_new.shape or k_new.shape[1:] != (cache.num_kv_heads, cache.head_dim):
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    if out.shape != q.shape or q.dim() != 3 or q.shape[0] != T or q.shape[2] != cache.head_dim:
        raise ValueError("q and out must be [T, num_q_heads, head_dim]")
    if slot_mapping_t.numel() < T:
        raise ValueError("slot_mapping shorter than the token count")
    ws_bytes = 0
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    rc = lib.pkv_append_attention_step(
        ctypes.byref(cache._c), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping_t), T, _ptr(q),
        _ptr(out), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        _ptr(query_start_loc), context_lens.shape[0], num_decode_seqs, q.shape[1], float(scale),
        int(max_context_len), int(max_query_len), int(kv_partition_tokens),
        *_schedule_args(schedule), _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc, "pkv_append_attention_step")
    return out


def append_attention_step_noalloc(cache: KVCache, k_new, v_new, slot_mapping_t, q, out,
                                  block_tables, context_lens, query_start_loc,
                                  num_decode_seqs: int, scale: float, max_context_len: int,
                                  max_query_len: int, kv_partition_tokens: int = 0, stream=None,
                                  schedule=None):
    """pkv_append_attention_step_noalloc: append_attention_step with the
    partials in the library's own device scratch (no workspace argument; the
    call allocates nothing)."""
    import torch
    for t, name in ((k_new, "k_new"), (v_new, "v_new"), (q, "q"), (out, "out")):
        _need(t, torch.float16, name)
    _need(slot_mapping_t, torch.int64, "slot_mapping")
    _need(block_tables, torch.int32, "block_tables")
    _need(context_lens, torch.int32, "context_lens")
    if query_start_loc is not None:
        _need(query_start_loc, torch.int32, "query_start_loc")
    T = k_new.shape[0]
    if v_new.shape != k_new.shape or k_new.shape[1:] != (cache.num_kv_heads, cache.head_dim):
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    if out.shape != q.shape or q.dim() != 3 or q.shape[0] != T or q.shape[2] != cache.head_dim:
        raise ValueError("q and out must be [T, num_q_heads, head_dim]")
    if slot_mapping_t.numel() < T:
        raise ValueError("slot_mapping shorter than the token count")
    rc = lib.pkv_append_attention_step_noalloc(
        ctypes.byref(cache._c), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping_t), T, _ptr(q),
        _ptr(out), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        _ptr(query_start_loc), context_lens.shape[0], num_decode_seqs, q.shape[1], float(scale),
        int(max_context_len), int(max_query_len), int(kv_partition_tokens),
        *_schedule_args(schedule), _stream(stream))
    _check(rc, "pkv_append_attention_step_noalloc")
    return out


class AttentionLayers:
    """Every layer of a step in one call (pkv_append_attention_layers).

    Built once from the per-layer caches and tensors, which must stay
    allocated (their addresses are kept); calling it enqueues
    pkv_append_attention_step for each layer in order with the step's shared
    arguments, in one call into the library."""

    def __init__(self, caches, k_new, v_new, q, out):
        import torch
        L = len(caches)
        if not (len(k_new) == len(v_new) == len(q) == len(out) == L):
            raise ValueError("one cache, k_new, v_new, q and out per layer")
        for i in range(L):
            for t, name in ((k_new[i], "k_new"), (v_new[i], "v_new"), (q[i], "q"), (out[i], "out")):
                _need(t, torch.float16, name)
            if v_new[i].shape != k_new[i].shape or q[i].shape != q[0].shape or \
                    out[i].shape != q[0].shape or k_new[i].shape != k_new[0].shape:
                raise ValueError("every layer's tensors must have the same shapes")
            c = caches[i]
            if k_new[i].dim() != 3 or k_new[i].shape[1:] != (c.num_kv_heads, c.head_dim):
                raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
            if q[i].dim() != 3 or q[i].shape[0] != k_new[i].shape[0] or q[i].shape[2] != c.head_dim:
                raise ValueError("q and out must be [T, num_q_heads, head_dim]")
        self.num_layers = L
        self.num_tokens = int(k_new[0].shape[0]) if L else 0
        self.num_q_heads = int(q[0].shape[1]) if L else 0
        self._keep = (list(caches), list(k_new), list(v_new), list(q), list(out))
        self._caches = (_Cache * max(L, 1))(*[c._c for c in caches])
        vp = ctypes.c_void_p
        self._k = (vp * max(L, 1))(*[t.data_ptr() for t in k_new])
        self._v = (vp * max(L, 1))(*[t.data_ptr() for t in v_new])
        self._q = (vp * max(L, 1))(*[t.data_ptr() for t in q])
        self._o = (vp * max(L, 1))(*[t.data_ptr() for t in out])

    def __call__(self, slot_mapping_t, block_tables, context_lens, query_start_loc,
                 num_decode_seqs: int, scale: float, max_context_len: int, max_query_len: int,
                 workspace=None, kv_partition_tokens: int = 0, stream=None, schedule=None):
        if slot_mapping_t.numel() < self.num_tokens:
            raise ValueError("slot_mapping shorter than the token count")
        rc = lib.pkv_append_attention_layers(
            self._caches, self.num_layers, self._k, self._v, _ptr(slot_mapping_t),
            self.num_tokens, self._q, self._o, _ptr(block_tables), block_tables.shape[1],
            _ptr(context_lens), _ptr(query_start_loc), context_lens.shape[0], num_decode_seqs,
            self.num_q_heads, float(scale), int(max_context_len), int(max_query_len),
            int(kv_partition_tokens), *_schedule_args(schedule), _ptr(workspace),
            0 if workspace is None else workspace.numel(), _stream(stream))
        _check(rc, "pkv_append_attention_layers")


def validate_step(block_tables, context_lens, query_start_loc, num_decode_seqs: int,
                  num_blocks: int, slot_mapping_arr=None, max_context_len=None,
                  max_query_len=None, block_size: int = 16):
    """pkv_validate_step on host (numpy) arrays; returns (what, index), (0, -1) when valid."""
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    ctx = np.ascontiguousarray(context_lens, dtype=np.int32)
    qsl = None if query_start_loc is None else np.ascontiguousarray(query_start_loc, dtype=np.int32)
    sm = None if slot_mapping_arr is None else np.ascontiguousarray(slot_mapping_arr, dtype=np.int64)
    B = ctx.shape[0]
    T = int(qsl[-1]) if qsl is not None else B
    if sm is not None:
        T = sm.shape[0]
    mcl = int(ctx.max()) if max_context_len is None else int(max_context_len)
    mql = (int(np.diff(qsl).max()) if qsl is not None else 1) if max_query_len is None else int(max_query_len)
    what = ctypes.c_int32(0)
    idx = ctypes.c_int64(-1)
    rc = lib.pkv_validate_step(_ptr(bt), bt.shape[1], _ptr(ctx), _ptr(qsl), B, num_decode_seqs,
                               num_blocks, block_size, _ptr(sm), T, mcl, mql,
                               ctypes.byref(what), ctypes.byref(idx))
    if rc not in (PKV_OK, PKV_ERR_CONTRACT):
        raise PkvError(rc, "pkv_validate_step")
    return int(what.value), int(idx.value)


def hbm_read_probe(base, tile_ids, tile_bytes: int, sink, launches: int = 1, stream=None):
    """pkv_hbm_read_probe: `launches` launches back to back, launch k reading
    tiles tile_ids[k n .. (k + 1) n) (int32 device tensor, n = its length /
    launches) of `base` (uint8 device tensor) once each, in that order; `sink`
    is a uint32-sized (int32) device tensor of PROBE_SINK_WORDS words.
    Measurement only."""
    import torch
    _need(base, torch.uint8, "base")
    _need(tile_ids, torch.int32, "tile_ids")
    _need(sink, torch.int32, "sink")
    if sink.numel() < PROBE_SINK_WORDS:
        raise ValueError("sink must hold PROBE_SINK_WORDS words")
    if launches < 1 or tile_ids.numel() % launches:
        raise ValueError("tile_ids must hold launches equal windows")
    rc = lib.pkv_hbm_read_probe(_ptr(base), base.numel(), _ptr(tile_ids),
                                tile_ids.numel() // launches, int(tile_bytes), int(launches),
                                _ptr(sink), _stream(stream))
    _check(rc, "pkv_hbm_read_probe")
