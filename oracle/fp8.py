"""fp8 (OCP E4M3) KV cache: encode, decode, per-row quantization, append.

TEST INFRASTRUCTURE ONLY (as the rest of ``oracle/``); numpy, fp64, written
from the format's definition, sharing nothing with the HIP kernels.

Why a quantized cache: the raw KV of a long window halves at 8 bits ("8 GiB
at 8-bit ... before scales" for the 262,144-token window -- a8q9.cn, "An
advertised batch limit proves nothing until sampled"), and quantizing the
cache is one of the remedies when memory caps the batch (deepconcepts.dev,
"Continuous Batching Is Not a Bigger Batch", "Checking it on a real system").
The pages give no format or scale granularity; the reading taken here:

* codes: OCP 8-bit floating point E4M3 -- 1 sign bit, 4 exponent bits (bias
  7), 3 mantissa bits; exponent field 0 is zero / subnormal (M x 2^-9); the
  pattern S.1111.111 is NaN; no infinities; largest finite 448 (S.1111.110).
* one fp32 scale per (token, KV head) row, a power of two 2^e: the smallest
  e with max|x| <= 448 x 2^e (e = 0 for an all-zero row).  Dividing by it is
  exact, so a row's codes are its values divided by 2^e rounded to the
  nearest E4M3 value, ties to even mantissa, sign kept (-0 -> 0x80); no value
  can overflow.
* dequantized value = E4M3 value x scale (exact in fp64).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
MIN_NORMAL = 2.0 ** -6
MIN_SUBNORMAL = 2.0 ** -9


def e4m3_to_float64(codes) -> np.ndarray:
    """Decode E4M3 codes (uint8) from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    E = (c >> 3) & 0xF
    M = c & 0x7
    sub = M * MIN_SUBNORMAL
    norm = (1.0 + M / 8.0) * np.exp2(E.astype(np.float64) - 7.0)
    v = np.where(E == 0, sub, norm)
    v = np.where((E == 15) & (M == 7), np.nan, v)
    return sign * v


def float64_to_e4m3(y) -> np.ndarray:
    """Round finite values with |y| <= 448 to the nearest E4M3 code (ties to
    even mantissa, sign kept)."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > E4M3_MAX):
        raise ValueError("E4M3 encode needs finite |y| <= 448")
    a = np.abs(y)
    sign = np.signbit(y).astype(np.int64) << 7
    # exponent of the binade (subnormals share the smallest normal's spacing)
    with np.errstate(divide="ignore"):
        E_unb = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    E_unb = np.maximum(E_unb, -6.0)
    # log2 rounding can be off by one at binade edges: correct against 2^E
    E_unb = np.where(np.exp2(E_unb) > a, np.maximum(E_unb - 1, -6.0), E_unb)
    E_unb = np.where(np.exp2(E_unb + 1) <= a, E_unb + 1, E_unb)
    ulp = np.exp2(E_unb - 3.0)
    n = np.rint(a / ulp)            # a / ulp is exact; rint rounds halves to even
    q = n * ulp                      # the rounded magnitude (may be 2^(E_unb + 1))
    out = np.zeros(a.shape, dtype=np.int64)
    is_sub = q < MIN_NORMAL
    out = np.where(is_sub, np.rint(q / MIN_SUBNORMAL).astype(np.int64), out)
    with np.errstate(divide="ignore"):
        Eq = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    Eq = np.where(np.exp2(Eq) > q, Eq - 1, Eq)
    Eq = np.where(np.exp2(Eq + 1) <= q, Eq + 1, Eq)
    Mq = np.rint((q / np.exp2(Eq) - 1.0) * 8.0).astype(np.int64)
    normal_code = ((Eq.astype(np.int64) + 7) << 3) | Mq
    out = np.where(is_sub, out, normal_code)
    return (out | sign).astype(np.uint8)


def row_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 x 2^e (0 where amax == 0).
    With amax = m 2^k, m in [0.5, 1) and 448 = 0.875 x 2^9: e = k - 9, plus 1
    when m > 0.875."""
    a = np.asarray(amax, dtype=np.float64)
    m, k = np.frexp(a)
    e = k.astype(np.int64) - 9 + (m > 0.875)
    return np.where(a > 0, e, 0).astype(np.int64)


def quantize_rows(x_bits) -> tuple[np.ndarray, np.ndarray]:
    """fp16 rows (bits or float16, last axis = the row) -> (codes uint8 of the
    same shape, scales float32 of the shape without the last axis)."""
    x = np.asarray(x_bits)
    if x.dtype == np.uint16:
        x = x.view(np.float16)
    x = x.astype(np.float64)
    e = row_exponent(np.abs(x).max(axis=-1))
    scales = np.ldexp(1.0, e)
    y = np.ldexp(x, -e[..., None])        # exact: a power-of-two scaling
    return float64_to_e4m3(y), scales.astype(np.float32)


def dequantize(codes, scales) -> np.ndarray:
    """fp64 values of a quantized pool or row set: code value x row scale."""
    return e4m3_to_float64(codes) * np.asarray(scales, dtype=np.float64)[..., None]


def kv_append(k_codes, v_codes, k_scales, v_scales, k_new, v_new, slots):
    """Append replay on an fp8 cache (copies returned, inputs untouched).

    Pools: codes [NB, Hkv, 16, d] uint8, scales [NB, Hkv, 16] float32; new
    rows [T, Hkv, d] fp16 (bits).  Token t with slot >= 0 writes the
    quantized rows of every KV head at block slot // 16, offset slot % 16."""
    kc, vc = np.array(k_codes, copy=True), np.array(v_codes, copy=True)
    ks, vs = np.array(k_scales, copy=True), np.array(v_scales, copy=True)
    qk, sk = quantize_rows(k_new)
    qv, sv = quantize_rows(v_new)
    for t, slot in enumerate(np.asarray(slots, dtype=np.int64)):
        if slot < 0:
            continue
        b, o = slot // 16, slot % 16
        if b >= kc.shape[0]:
            raise IndexError("slot beyond the pool")
        kc[b, :, o], vc[b, :, o] = qk[t], qv[t]
        ks[b, :, o], vs[b, :, o] = sk[t], sv[t]
    return kc, vc, ks, vs
