"""CPU oracle for the paged KV append + paged attention step.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The product path never
imports this package.  It shares no code with the HIP kernels: the C part
(``oracle.c``) is compiled with the host C compiler into its own
``liboracle.so``; the numpy part (``dense.py``) is a dense brute force that
knows nothing of block tables.

Functions (each cites what it follows in the C source):
  slot_mapping, kv_append, paged_attention, paged_attention_fp8,
  paged_attention_f64,
  attention_partial, lse_merge, half_to_float64.
Submodules: ``fp8`` (E4M3 codes and the per-row quantization of an fp8
cache), ``scheduler`` (plain model of the per-pass scheduler), ``dense``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_LIBRARY names another build of oracle.c (e.g. with sanitizers).
_LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB_PATH,
          sanitize: bool = False) -> str:
    """Compile oracle.c with gcc into liboracle.so (plain -O2, no fast-math).

    src / out: another source (a test's mutated copy) or output path.
    sanitize: build with clang's AddressSanitizer and UndefinedBehaviorSanitizer
    (clang, so that the process holds one sanitizer runtime with the
    library's sanitized host code; load it with that runtime preloaded)."""
    if sanitize:
        cmd = [os.environ.get("SAN_CC", "/opt/rocm/llvm/bin/clang"), "-O1", "-g",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", "-shared-libsan", "-std=c11", "-fopenmp", "-fPIC",
               "-shared", src, "-o", out, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", src, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = f64
    lib.oracle_half_array_to_double.argtypes = [P, P, i64]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_slot_mapping.argtypes = [P, i32, P, P, i32, i32, P]
    lib.oracle_kv_append.argtypes = [P, P, i64, i32, i32, i32, P, P, P, i32]
    lib.oracle_paged_attention.argtypes = [P, P, P, i64, i32, i32, i32, P, i32, P, P, i32,
                                           i32, f64, P, P, P, i32]
    lib.oracle_paged_attention_f64.argtypes = [P, P, P, i64, i32, i32, i32, P, i32, P, P, i32,
                                               i32, f64, P, P, i32]
    lib.oracle_attention_partial.argtypes = [P, P, P, i32, i32, i32, f64, P, P, P]
    lib.oracle_lse_merge.argtypes = [P, P, P, i32, i32, P]
    lib.oracle_attention_contiguous.argtypes = [P, P, P, i32, i32, f64, P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _bits(a) -> np.ndarray:
    """fp16 values (numpy float16 or uint16 bit patterns) as contiguous uint16 bits."""
    a = np.asarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return np.ascontiguousarray(a)


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def half_to_float64(bits) -> np.ndarray:
    """Decode fp16 bit patterns to float64 from the binary16 definition."""
    b = _bits(bits)
    out = np.empty(b.shape, dtype=np.float64)
    _load().oracle_half_array_to_double(_ptr(b), _ptr(out), b.size)
    return out


def slot_mapping(block_tables, context_lens, query_start_loc, block_size: int) -> np.ndarray:
    """Pool slot of every new token (int64 [T]); query_start_loc None => one token each."""
    bt = _c(block_tables, np.int32)
    ctx = _c(context_lens, np.int32)
    qsl = None if query_start_loc is None else _c(query_start_loc, np.int32)
    B = ctx.shape[0]
    T = B if qsl is None else int(qsl[-1])
    out = np.full(T, -(2 ** 62), dtype=np.int64)
    rc = _load().oracle_slot_mapping(_ptr(bt), bt.shape[1], _ptr(ctx), _ptr(qsl), B,
                                     block_size, _ptr(out))
    _check(rc, "oracle_slot_mapping")
    return out


def kv_append(k_pool, v_pool, k_new, v_new, slots) -> tuple[np.ndarray, np.ndarray]:
    """Return copies of the pools after the append replay (inputs untouched).

    k_pool/v_pool: [NB, Hkv, bs, d] fp16 (or uint16 bits); k_new/v_new: [T, Hkv, d].
    """
    kp = _bits(k_pool).copy()
    vp = _bits(v_pool).copy()
    kn, vn = _bits(k_new), _bits(v_new)
    s = _c(slots, np.int64)
    NB, Hkv, bs, d = kp.shape
    rc = _load().oracle_kv_append(_ptr(kp), _ptr(vp), NB, Hkv, bs, d, _ptr(kn), _ptr(vn),
                                  _ptr(s), s.shape[0])
    _check(rc, "oracle_kv_append")
    return kp, vp


def paged_attention(q, k_pool, v_pool, block_tables, context_lens, query_start_loc,
                    scale: float, seq_subset=None, want_lse: bool = False):
    """fp64 attention output [T, Hq, d] (rows of sequences outside seq_subset are NaN)."""
    qb = _bits(q)
    kp, vp = _bits(k_pool), _bits(v_pool)
    bt = _c(block_tables, np.int32)
    ctx = _c(context_lens, np.int32)
    qsl = None if query_start_loc is None else _c(query_start_loc, np.int32)
    T, Hq, d = qb.shape
    NB, Hkv, bs, d2 = kp.shape
    assert d2 == d
    out = np.full((T, Hq, d), np.nan, dtype=np.float64)
    lse = np.full((T, Hq), np.nan, dtype=np.float64) if want_lse else None
    sub = None if seq_subset is None else _c(seq_subset, np.int32)
    rc = _load().oracle_paged_attention(
        _ptr(qb), _ptr(kp), _ptr(vp), NB, Hkv, bs, d, _ptr(bt), bt.shape[1], _ptr(ctx),
        _ptr(qsl), ctx.shape[0], Hq, float(scale), _ptr(out), _ptr(lse), _ptr(sub),
        0 if sub is None else sub.shape[0])
    _check(rc, "oracle_paged_attention")
    return (out, lse) if want_lse else out


def paged_attention_fp8(q, k_codes, v_codes, k_scales, v_scales, block_tables, context_lens,
                        query_start_loc, scale: float, seq_subset=None):
    """fp64 attention [T, Hq, d] over an fp8 cache: the pools are dequantized
    (oracle.fp8.dequantize, exact) and attended as in paged_attention."""
    from . import fp8
    kd = fp8.dequantize(k_codes, k_scales)
    vd = fp8.dequantize(v_codes, v_scales)
    return paged_attention_f64(q, kd, vd, block_tables, context_lens, query_start_loc, scale,
                               seq_subset=seq_subset)


def paged_attention_f64(q, k_pool, v_pool, block_tables, context_lens, query_start_loc,
                        scale: float, seq_subset=None):
    """fp64 attention [T, Hq, d] over pools already held as float64
    [NB, Hkv, bs, d] (a dequantized fp8 cache): the same gather-then-attend
    as paged_attention, with fp16 queries."""
    qb = _bits(q)
    kd = _c(k_pool, np.float64)
    vd = _c(v_pool, np.float64)
    bt = _c(block_tables, np.int32)
    ctx = _c(context_lens, np.int32)
    qsl = None if query_start_loc is None else _c(query_start_loc, np.int32)
    T, Hq, d = qb.shape
    NB, Hkv, bs, d2 = kd.shape
    assert d2 == d
    out = np.full((T, Hq, d), np.nan, dtype=np.float64)
    sub = None if seq_subset is None else _c(seq_subset, np.int32)
    rc = _load().oracle_paged_attention_f64(
        _ptr(qb), _ptr(kd), _ptr(vd), NB, Hkv, bs, d, _ptr(bt), bt.shape[1], _ptr(ctx),
        _ptr(qsl), ctx.shape[0], Hq, float(scale), _ptr(out), _ptr(sub),
        0 if sub is None else sub.shape[0])
    _check(rc, "oracle_paged_attention_f64")
    return out


def attention_partial(q, K, V, lo: int, hi: int, scale: float):
    """(o_part[d], m_part, l_part) of one fp64 query row over contiguous rows [lo, hi)."""
    q, K, V = _c(q, np.float64), _c(K, np.float64), _c(V, np.float64)
    d = q.shape[0]
    o = np.empty(d, dtype=np.float64)
    m = np.zeros(1, dtype=np.float64)
    l = np.zeros(1, dtype=np.float64)
    _load().oracle_attention_partial(_ptr(q), _ptr(K), _ptr(V), lo, hi, d, float(scale),
                                     _ptr(o), _ptr(m), _ptr(l))
    return o, float(m[0]), float(l[0])


def attention_contiguous(q, K, V, scale: float) -> np.ndarray:
    q, K, V = _c(q, np.float64), _c(K, np.float64), _c(V, np.float64)
    out = np.empty(q.shape[0], dtype=np.float64)
    _load().oracle_attention_contiguous(_ptr(q), _ptr(K), _ptr(V), K.shape[0], q.shape[0],
                                        float(scale), _ptr(out))
    return out


def lse_merge(o_parts, m_parts, l_parts) -> np.ndarray:
    """Merge partials [P, d], [P], [P] into one output row [d] (fp64)."""
    o = _c(o_parts, np.float64)
    m = _c(m_parts, np.float64)
    l = _c(l_parts, np.float64)
    out = np.empty(o.shape[1], dtype=np.float64)
    _load().oracle_lse_merge(_ptr(o), _ptr(m), _ptr(l), o.shape[0], o.shape[1], _ptr(out))
    return out
