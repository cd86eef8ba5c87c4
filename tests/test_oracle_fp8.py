"""Pins of the fp8 (OCP E4M3) part of the oracle, CPU only: the format's
defining values, round-to-nearest-even against a brute-force nearest-code
search, the row-scale rule, the quantization error bound, and closed forms
of attention over a quantized cache."""
import numpy as np
import pytest

import oracle
from oracle import fp8


def test_defining_values_of_the_format():
    dec = fp8.e4m3_to_float64(np.arange(256, dtype=np.uint8))
    assert dec[0x00] == 0.0 and not np.signbit(dec[0x00])
    assert dec[0x80] == 0.0 and np.signbit(dec[0x80])
    assert dec[0x01] == 2.0 ** -9          # smallest subnormal
    assert dec[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert dec[0x08] == 2.0 ** -6          # smallest normal
    assert dec[0x38] == 1.0                # exponent field 7 = bias
    assert dec[0x3C] == 1.5
    assert dec[0x77] == 240.0              # 1.875 x 2^7
    assert dec[0x78] == 256.0
    assert dec[0x7E] == 448.0              # largest finite: S.1111.110
    assert dec[0xFE] == -448.0
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert np.isnan(dec).sum() == 2
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0)        # 0x00 .. 0x7E strictly increasing


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.float64_to_e4m3(fp8.e4m3_to_float64(codes)), codes)


def test_ties_go_to_the_even_mantissa():
    assert fp8.float64_to_e4m3(2.0 ** -10) == 0x00        # half the smallest subnormal
    assert fp8.float64_to_e4m3(np.nextafter(2.0 ** -10, 1)) == 0x01
    assert fp8.float64_to_e4m3(1.5 * 2.0 ** -9) == 0x02   # between 0x01 and 0x02
    assert fp8.float64_to_e4m3(2.5 * 2.0 ** -9) == 0x02   # between 0x02 and 0x03
    assert fp8.float64_to_e4m3(1.0625) == 0x38            # between 1 and 1.125
    assert fp8.float64_to_e4m3(1.1875) == 0x3A            # between 1.125 and 1.25
    assert fp8.float64_to_e4m3(-1.1875) == 0xBA
    assert fp8.float64_to_e4m3(-0.0) == 0x80
    assert fp8.float64_to_e4m3(432.0) == 0x7E             # between 416 and 448: even is 448


def test_rounding_matches_a_brute_force_nearest_code():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-448, 448, 4000),
                        rng.uniform(-1, 1, 4000) * 2.0 ** rng.integers(-12, 0, 4000),
                        fp8.e4m3_to_float64(rng.integers(0, 0x7F, 2000)) * 1.0])
    codes = fp8.float64_to_e4m3(y)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.e4m3_to_float64(finite)
    for yy, c in zip(y, codes):
        dist = np.abs(vals - yy)
        best = finite[dist == dist.min()]
        best = best[np.sign(fp8.e4m3_to_float64(best)) != -np.sign(yy)] if yy != 0 else best
        if len(best) > 1:   # a tie: the even mantissa wins
            best = best[(best & 1) == 0]
        assert fp8.e4m3_to_float64(c) == fp8.e4m3_to_float64(best[0]), (yy, c, best)


def test_row_exponent_is_the_smallest_that_fits():
    assert fp8.row_exponent(448.0) == 0
    assert fp8.row_exponent(448.25) == 1
    assert fp8.row_exponent(224.0) == -1
    assert fp8.row_exponent(224.125) == 0
    assert fp8.row_exponent(1.0) == -8
    assert fp8.row_exponent(0.0) == 0
    rng = np.random.default_rng(2)
    a = rng.uniform(0, 1, 5000) * 2.0 ** rng.integers(-24, 16, 5000)
    a = a.astype(np.float16).astype(np.float64)
    a = a[a > 0]
    e = fp8.row_exponent(a)
    assert np.all(a <= 448 * np.exp2(e.astype(float)))
    assert np.all(a > 448 * np.exp2(e.astype(float) - 1))


def test_quantization_error_bound():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((300, 128)) * 2.0 ** rng.integers(-10, 10, (300, 1))).astype(np.float16)
    codes, scales = fp8.quantize_rows(x)
    deq = fp8.dequantize(codes, scales)
    xd = x.astype(np.float64)
    # half an E4M3 spacing: 2^-4 of the value's binade, 2^-10 x scale below the normals
    bound = np.maximum(np.abs(xd) * 2.0 ** -4, 2.0 ** -10 * scales[:, None].astype(np.float64))
    assert np.all(np.abs(deq - xd) <= bound)
    assert np.all(np.abs(codes.astype(np.int64) & 0x7F) <= 0x7E)  # never NaN
    amax = np.abs(xd).max(axis=1)
    assert np.all(np.abs(deq).max(axis=1) <= 448 * scales)
    assert np.all(amax > 224 * scales)     # the scale is the smallest that fits


def test_append_writes_quantized_rows_at_their_slots():
    rng = np.random.default_rng(4)
    NB, Hkv, d = 8, 2, 128
    kc = rng.integers(0, 256, (NB, Hkv, 16, d)).astype(np.uint8)
    vc = kc.copy()
    ks = np.ones((NB, Hkv, 16), np.float32)
    vs = ks.copy()
    kn = rng.standard_normal((3, Hkv, d)).astype(np.float16)
    vn = rng.standard_normal((3, Hkv, d)).astype(np.float16)
    slots = np.array([5, -1, 77])
    k2, v2, ks2, vs2 = fp8.kv_append(kc, vc, ks, vs, kn, vn, slots)
    qk, sk = fp8.quantize_rows(kn)
    assert np.array_equal(k2[0, :, 5], qk[0]) and ks2[0, 0, 5] == sk[0, 0]
    assert np.array_equal(k2[4, :, 13], qk[2])
    changed = (k2 != kc).any(axis=(1, 3))
    assert set(zip(*np.nonzero(changed))) <= {(0, 5), (4, 13)}


def test_attention_over_a_quantized_cache_closed_forms():
    rng = np.random.default_rng(5)
    NB, Hkv, d, Hq = 6, 2, 128, 12
    v = rng.standard_normal((1, Hkv, d)).astype(np.float16)
    codes, scales = fp8.quantize_rows(v)
    kc = np.zeros((NB, Hkv, 16, d), np.uint8)
    vc = np.zeros_like(kc)
    ks = np.ones((NB, Hkv, 16), np.float32)
    vs = ks.copy()
    vc[3, :, 0], vs[3, :, 0] = codes[0], scales[0]
    q = rng.standard_normal((1, Hq, d)).astype(np.float16)
    out = oracle.paged_attention_fp8(q, kc, vc, ks, vs, np.array([[3]]), np.array([1]), None,
                                     d ** -0.5)
    deq = fp8.dequantize(codes, scales)[0]
    for h in range(Hq):
        assert np.array_equal(out[0, h], deq[h // 6])        # one position: its value
    # equal keys everywhere: the mean of the dequantized values
    vrows = rng.standard_normal((20, Hkv, d)).astype(np.float16)
    c2, s2 = fp8.quantize_rows(vrows)
    bt = np.array([[1, 4]])
    for p in range(20):
        vc[bt[0, p // 16], :, p % 16], vs[bt[0, p // 16], :, p % 16] = c2[p], s2[p]
    out = oracle.paged_attention_fp8(q, kc, vc, ks, vs, bt, np.array([20]), None, d ** -0.5)
    mean = fp8.dequantize(c2, s2).mean(axis=0)
    for h in range(Hq):
        assert np.allclose(out[0, h], mean[h // 6], rtol=0, atol=1e-12)
