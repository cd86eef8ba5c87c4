"""GPU parity of the fp8 (OCP E4M3) KV cache against the CPU oracle:
the quantizing append bit for bit (codes and scales, on rows that together
hold every finite fp16 value, so every rounding the hardware conversion
makes is checked), and paged decode over fp8 pools within the attention
tolerance of the fp16 path (the oracle attends the exactly dequantized
cache, so the same rounding budget applies)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_decode_append_amd as pkv
import workloads
from oracle import fp8 as ofp8
from paged_kv_decode_append_amd.step import Step
from parity import assert_close, host_bits

pytestmark = pytest.mark.gpu


def _report(name, errs):
    print(f"[parity] {name}: max_abs={errs[0]:.2e} norm_rel={errs[1]:.2e}", flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def _all_finite_fp16_rows(d):
    """Every finite fp16 value once, sorted by magnitude and cut into rows of
    d (a row's values are close in size, so its codes span the format), plus
    the same values shuffled into rows (a row's small values meet its large
    scale)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16)
    finite = bits[np.isfinite(vals)]
    order = np.argsort(np.abs(finite.view(np.float16).astype(np.float64)), kind="stable")
    sorted_bits = finite[order]
    shuffled = np.random.default_rng(3).permutation(finite)
    allrows = np.concatenate([sorted_bits, shuffled])
    pad = (-len(allrows)) % d
    allrows = np.concatenate([allrows, np.zeros(pad, np.uint16)])
    return allrows.reshape(-1, d)


@pytest.mark.parametrize("d", [128, 256])
def test_append_quantizes_every_fp16_value_bit_exactly(d):
    hkv = 2
    rows = _all_finite_fp16_rows(d)                    # [R, d]
    T = len(rows) // hkv
    rows = rows[: T * hkv].reshape(T, hkv, d)
    NB = (T + 15) // 16 + 3
    rng = np.random.default_rng(d)
    kc0 = rng.integers(0, 256, (NB, hkv, 16, d), dtype=np.uint8)
    vc0 = rng.integers(0, 256, (NB, hkv, 16, d), dtype=np.uint8)
    ks0 = rng.standard_normal((NB, hkv, 16)).astype(np.float32)
    vs0 = rng.standard_normal((NB, hkv, 16)).astype(np.float32)
    slots = rng.permutation(NB * 16)[:T].astype(np.int64)
    slots[::97] = -1                                    # padding tokens are skipped
    k_new = rows
    v_new = rows[::-1].copy()
    dev = {n: torch.from_numpy(np.ascontiguousarray(a)).cuda()
           for n, a in (("kc", kc0), ("vc", vc0), ("ks", ks0), ("vs", vs0))}
    cache = pkv.KVCache(dev["kc"], dev["vc"], dev["ks"], dev["vs"])
    kn = torch.from_numpy(k_new.view(np.float16)).cuda()
    vn = torch.from_numpy(np.ascontiguousarray(v_new).view(np.float16)).cuda()
    pkv.kv_append(cache, kn, vn, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kc, vc, ks, vs = ofp8.kv_append(kc0, vc0, ks0, vs0, k_new, v_new, slots)
    assert np.array_equal(_np(dev["kc"]), kc), "K codes"
    assert np.array_equal(_np(dev["vc"]), vc), "V codes"
    assert np.array_equal(_np(dev["ks"]).view(np.uint32), ks.view(np.uint32)), "K scales"
    assert np.array_equal(_np(dev["vs"]).view(np.uint32), vs.view(np.uint32)), "V scales"


def _fp8_cache(wl, layer=0, poison=True, scale_exp=(-6, -2), v_scale_exp=None):
    t = workloads.layer_tensors_fp8(wl, layer, device="cuda", scale_exp=scale_exp,
                                    v_scale_exp=v_scale_exp)
    if poison:
        # stale rows (outside every context) hold NaN codes and NaN scales
        qsl = np.concatenate([[0], np.cumsum(wl.context_lens)]).astype(np.int32)
        live = np.zeros(wl.num_blocks * 16, bool)
        live[oracle.slot_mapping(wl.block_tables, wl.context_lens, qsl, 16)] = True
        dead = torch.from_numpy(np.nonzero(~live)[0]).cuda()
        for n in ("k_codes", "v_codes"):
            t[n].transpose(1, 2)[dead // 16, dead % 16] = 0x7F
        for n in ("k_scale", "v_scale"):
            t[n].transpose(1, 2)[dead // 16, dead % 16] = float("nan")
    return t


def _run(wl, t, part=0, fused=False):
    step = Step.from_workload(wl, kv_partition_tokens=part)
    step.plan()
    cache = pkv.KVCache(t["k_codes"], t["v_codes"], t["k_scale"], t["v_scale"])
    out = torch.full_like(t["q"], float("nan"))
    step.layer(cache, t["q"], t["k_new"], t["v_new"], out, fused=fused)
    torch.cuda.synchronize()
    return step, out


def _ref(wl, t, q=None, seq_subset=None):
    return oracle.paged_attention_fp8(host_bits(t["q"]) if q is None else q, _np(t["k_codes"]),
                                      _np(t["v_codes"]), _np(t["k_scale"]), _np(t["v_scale"]),
                                      wl.block_tables, wl.context_lens, None, wl.scale,
                                      seq_subset=seq_subset)


@pytest.mark.parametrize("d,hq,hkv", [(128, 12, 2), (128, 8, 8), (128, 8, 1), (128, 24, 3),
                                      (256, 16, 4), (256, 8, 8), (256, 12, 2), (256, 24, 3)])
@pytest.mark.parametrize("part", [0, 64, 256])
def test_decode_over_an_fp8_cache(d, hq, hkv, part):
    ctx = [1, 2, 15, 16, 17, 31, 33, 64, 65, 300, 1025, 2500]
    wl = workloads.custom("fp8", ctx, [1] * len(ctx), len(ctx), hq, hkv, d, seed=hq * d + part)
    t = _fp8_cache(wl)
    # attention only: the decode tokens' rows are already in the cache
    step = Step.from_workload(wl, kv_partition_tokens=part)
    cache = pkv.KVCache(t["k_codes"], t["v_codes"], t["k_scale"], t["v_scale"])
    out = torch.full_like(t["q"], float("nan"))
    pkv.paged_attention_step(cache, t["q"], out, step.block_tables, step.context_lens, None,
                             wl.num_decode_seqs, wl.scale, step.max_context_len, 1,
                             workspace=step.workspace, kv_partition_tokens=part)
    torch.cuda.synchronize()
    errs = assert_close(out.cpu().numpy(), _ref(wl, t), f"fp8 d={d} G={hq // hkv} part={part}")
    _report(f"fp8 decode d={d} G={hq // hkv} part={part}", errs)


@pytest.mark.parametrize("d", [128, 256])
def test_single_position_returns_the_dequantized_value(d):
    wl = workloads.custom("fp8_ctx1", [1, 1, 1], [1, 1, 1], 3, 2 * (d // 64), 2, d, seed=d)
    t = _fp8_cache(wl, poison=False)
    step = Step.from_workload(wl)
    cache = pkv.KVCache(t["k_codes"], t["v_codes"], t["k_scale"], t["v_scale"])
    out = torch.empty_like(t["q"])
    pkv.paged_attention_step(cache, t["q"], out, step.block_tables, step.context_lens, None, 3,
                             wl.scale, 1, 1, workspace=step.workspace)
    torch.cuda.synchronize()
    deq = ofp8.dequantize(_np(t["v_codes"]), _np(t["v_scale"]))   # exact, fits fp16
    G = wl.num_q_heads // wl.num_kv_heads
    got = out.cpu().numpy()
    for i in range(3):
        b = wl.block_tables[i, 0]
        for h in range(wl.num_q_heads):
            want = deq[b, h // G, 0].astype(np.float16)
            assert np.array_equal(got[i, h].view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("fused", [True, False])
def test_step_appends_quantized_rows_then_attends(fused):
    """The step's new tokens: quantized into their slots (bit-exact against
    the oracle's append replay), then attended with the rest of the cache."""
    ctx = [5, 16, 17, 100, 513, 2049]
    wl = workloads.custom("fp8_step", ctx, [1] * len(ctx), len(ctx), 12, 2, 128, seed=29)
    t = _fp8_cache(wl)
    kc0, vc0, ks0, vs0 = (_np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale"))
    step, out = _run(wl, t, fused=fused)
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, None, 16)
    kc, vc, ks, vs = ofp8.kv_append(kc0, vc0, ks0, vs0, host_bits(t["k_new"]),
                                    host_bits(t["v_new"]), slots)
    assert np.array_equal(_np(t["k_codes"]), kc) and np.array_equal(_np(t["v_codes"]), vc)
    assert np.array_equal(_np(t["k_scale"]).view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(_np(t["v_scale"]).view(np.uint32), vs.view(np.uint32))
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, None, wl.scale)
    _report(f"fp8 step fused={fused}", assert_close(out.cpu().numpy(), ref, "fp8 step"))


def _append_ref(wl, t0, t):
    """The oracle's append replay of the step's rows over the pre-step pools
    t0 (host copies); checks the GPU pools (codes and scales) bit for bit."""
    qsl = wl.query_start_loc if wl.num_decode_seqs < wl.num_seqs else None
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, qsl, 16)
    kc, vc, ks, vs = ofp8.kv_append(t0["k_codes"], t0["v_codes"], t0["k_scale"], t0["v_scale"],
                                    host_bits(t["k_new"]), host_bits(t["v_new"]), slots)
    assert np.array_equal(_np(t["k_codes"]), kc) and np.array_equal(_np(t["v_codes"]), vc)
    assert np.array_equal(_np(t["k_scale"]).view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(_np(t["v_scale"]).view(np.uint32), vs.view(np.uint32))
    return kc, vc, ks, vs, qsl


FP8_CHUNKS = {
    # decodes, then short chunks whose G x n rows fit one tile (packed rows),
    # crossing block edges, one over a long cached context
    "short": ([15, 16, 17, 33, 40, 16, 17, 33, 8, 300, 1500], [1, 1, 1, 1, 8, 8, 3, 5, 8, 4, 2], 4),
    # chunks longer than a 64-row tile, with and without a cached prefix
    "long": ([300, 100, 64, 65, 500, 2100], [1, 100, 64, 65, 130, 200], 1),
}


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("kind", ["short", "long"])
@pytest.mark.parametrize("d,hq,hkv", [(128, 12, 2), (128, 8, 8), (256, 16, 4), (256, 24, 3)])
def test_chunks_over_an_fp8_cache(d, hq, hkv, kind, fused):
    """Prefill chunks (and decodes) in one step over an fp8 cache: the rows
    quantized into their slots bit-exactly, then every query row within
    tolerance of the oracle over the dequantized cache."""
    ctx, new, ndec = FP8_CHUNKS[kind]
    wl = workloads.custom(f"fp8_{kind}", ctx, new, ndec, hq, hkv, d, seed=hq * d + len(kind))
    t = _fp8_cache(wl)
    t0 = {n: _np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    _, out = _run(wl, t, fused=fused)
    kc, vc, ks, vs, qsl = _append_ref(wl, t0, t)
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, qsl, wl.scale)
    errs = assert_close(out.cpu().numpy(), ref, f"fp8 {kind} chunks d={d} G={hq // hkv}")
    _report(f"fp8 {kind} chunks d={d} G={hq // hkv} fused={fused}", errs)


@pytest.mark.parametrize("part", [64, 256])
def test_short_chunk_splits_over_an_fp8_cache(part):
    """Packed short chunks with the context cut into fixed splits (merged by
    log-sum-exp), some splits empty for the short contexts."""
    ctx = [16, 100, 700, 1500, 3000]
    wl = workloads.custom("fp8_spec", ctx, [4] * len(ctx), 0, 12, 2, 128, seed=part)
    t = _fp8_cache(wl)
    t0 = {n: _np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    _, out = _run(wl, t, part=part, fused=True)
    kc, vc, ks, vs, qsl = _append_ref(wl, t0, t)
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, qsl, wl.scale)
    _report(f"fp8 short chunks part={part}",
            assert_close(out.cpu().numpy(), ref, f"fp8 short chunks part={part}"))


def test_qwen_mixed_full_size_fp8():
    """64 decodes + a 512-row chunk over an 8,192-token prefix over an fp8
    cache: every decode sequence and every row of the chunk checked."""
    wl = workloads.qwen_mixed()
    t = _fp8_cache(wl, layer=5, poison=False)
    t0 = {n: _np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    _, out = _run(wl, t, fused=True)
    kc, vc, ks, vs, qsl = _append_ref(wl, t0, t)
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, qsl, wl.scale)
    errs = assert_close(out.cpu().numpy(), ref, "qwen_mixed fp8")
    _report("qwen_mixed fp8 layer 5 (64 decodes, all 512 chunk rows)", errs)


@pytest.mark.parametrize("hq,hkv", [(12, 2), (8, 8), (16, 2)])
def test_fp8_chunks_of_several_row_tiles_over_short_contexts(hq, hkv):
    """Chunks of 257 .. 700 rows (two or three 256-row tiles of the d = 128
    kernel) with little or no cached prefix over an fp8 cache: splits of one
    or two 64-token tiles, empty splits, the prologue's and the last steps'
    load counts, and the tiles converted from codes in the first step; every
    row checked."""
    ctx = [1, 600, 700, 257, 520]
    new = [1, 600, 520, 257, 513]
    wl = workloads.custom("fp8_row_tiles", ctx, new, 1, hq, hkv, 128, seed=hq + 19 * hkv)
    t = _fp8_cache(wl)
    t0 = {n: _np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    _, out = _run(wl, t, fused=True)
    kc, vc, ks, vs, qsl = _append_ref(wl, t0, t)
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, qsl, wl.scale)
    errs = assert_close(out.cpu().numpy(), ref, f"fp8 several row tiles G={hq // hkv}")
    _report(f"fp8 several row tiles G={hq // hkv}", errs)


def test_fp8_long_chunk_over_long_context_splits_past_staged_pages():
    """A 2,048-row chunk over a 20,000-token context over an fp8 cache: 2
    splits of ~157 KV tiles each, so the codes and row scales of pages past
    the first 256 of a split come by pool offsets read from the block table
    directly.  Sampled rows across the row tiles, each checked as the query
    that attends positions [0, its position] of the appended cache."""
    n, ctx = 2048, 20000
    wl = workloads.custom("fp8_long_split", [ctx], [n], 0, 12, 2, 128, seed=73)
    t = _fp8_cache(wl, poison=False)
    t0 = {k: _np(t[k]) for k in ("k_codes", "v_codes", "k_scale", "v_scale")}
    _, out = _run(wl, t, fused=True)
    kc, vc, ks, vs, _ = _append_ref(wl, t0, t)
    q = host_bits(t["q"])
    got = out.cpu().numpy()
    worst = (0.0, 0.0)
    for r in [0, 1, 127, 128, 255, 256, 1000, 1023, 1024, 1791, 2046, 2047]:
        ref = oracle.paged_attention_fp8(q[r:r + 1], kc, vc, ks, vs, wl.block_tables[:1],
                                         np.array([ctx - n + r + 1], np.int32), None, wl.scale)
        e = assert_close(got[r:r + 1], ref, f"fp8 long chunk row {r}")
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    _report("fp8 2,048-row chunk over 20,000 tokens (sampled rows)", worst)


@pytest.mark.parametrize("kind", ["decode", "short", "long"])
def test_row_scales_spanning_a_wide_range(kind):
    """K row scales from 2^-11 to 2^7 move the logits over many orders of
    magnitude (saturated softmax rows included); V row scales from 2^-4 to
    2^3 make the per-block (decode) and per-tile (prefill) reference scale
    change from block to block.  The V range is kept to 2^8: the weights are
    fp16, so the error of an output element scales with sum_t w_t |v_t|, and
    a much wider V range makes rows whose output is a small difference of
    large terms (relative error grows with that ratio, in any fp16-weight
    kernel).  The result stays within the tolerance of the oracle over the
    exactly dequantized cache."""
    if kind == "decode":
        ctx, new, ndec = [1, 16, 17, 300, 1025, 2500], [1] * 6, 6
    else:
        ctx, new, ndec = FP8_CHUNKS[kind]
    wl = workloads.custom(f"fp8_wide_{kind}", ctx, new, ndec, 12, 2, 128, seed=53)
    t = _fp8_cache(wl, scale_exp=(-11, 8), v_scale_exp=(-4, 4))
    t0 = {n: _np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    _, out = _run(wl, t, fused=True)
    kc, vc, ks, vs, qsl = _append_ref(wl, t0, t)
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, qsl, wl.scale)
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    # The 2e-3 bound is stated for unit-scale values; here rows reach ~10^3
    # and fp16 output rounding alone is 2^-11 of the value, so the
    # elementwise bound is taken relative to each row's largest |value|
    # (at least 1); the norm-relative bound is unchanged.
    r = ref.reshape(-1, ref.shape[-1])
    d = np.abs(got.reshape(r.shape) - r)
    row_scale = np.maximum(1.0, np.abs(r).max(axis=1))
    scaled = float((d.max(axis=1) / row_scale).max())
    norm_rel = float((np.linalg.norm(d, axis=1) / np.maximum(np.linalg.norm(r, axis=1), 1e-30)).max())
    assert scaled <= 2e-3 and norm_rel <= 1e-2, f"scaled max_abs={scaled:.2e} norm_rel={norm_rel:.2e}"
    _report(f"fp8 wide scales {kind} (row-scaled)", (scaled, norm_rel))


@pytest.mark.parametrize("name", ["qwen_uniform", "qwen_ragged", "qwen_spec"])
def test_full_size_fp8(name):
    """One layer of the 28-layer workloads over an fp8 cache (qwen_spec:
    64 sequences verifying 4 tokens each, on the packed-row kernel), every
    sequence against the oracle."""
    wl = workloads.WORKLOADS[name]()
    t = _fp8_cache(wl, layer=3, poison=False)
    t0 = {n: _np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    _, out = _run(wl, t, fused=True)
    kc, vc, ks, vs, qsl = _append_ref(wl, t0, t)
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, qsl, wl.scale)
    errs = assert_close(out.cpu().numpy(), ref, name)
    _report(f"{name} fp8 layer 3 (all {wl.num_seqs} sequences)", errs)


def _dequantized_sequence(wl, i, kc, vc, ks, vs):
    """Sequence i's blocks of an fp8 cache, dequantized (the oracle's E4M3
    decoding, applied through a table of its 256 code values) into a compact
    pool in table order, with the table that reads them there: block
    relabelling leaves attention unchanged, and the whole 4 GiB-per-layer
    pool would not fit in fp64."""
    nb = -(-int(wl.context_lens[i]) // wl.block_size)
    ids = wl.block_tables[i, :nb]
    lut = ofp8.e4m3_to_float64(np.arange(256, dtype=np.uint8))
    kd = lut[kc[ids]] * ks[ids].astype(np.float64)[..., None]
    vd = lut[vc[ids]] * vs[ids].astype(np.float64)[..., None]
    table = np.arange(nb, dtype=np.int32)[None, :]
    return kd, vd, table


def test_long_context_full_size_fp8():
    """long_context (4 x 262,144 tokens, d = 256, 16/4 heads) over an fp8
    cache at the plan the benchmark runs (256-block partitions: 64 blocks per
    wave, a block id in every lane), the decode tokens' quantizing append
    fused: codes and scales bit-exact, all 4 sequences against the oracle."""
    wl = workloads.long_context()
    t = _fp8_cache(wl, layer=2, poison=False)
    t0 = {n: _np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    step, out = _run(wl, t, fused=True)
    assert step.kv_partition_tokens == 0
    kc, vc, ks, vs, _ = _append_ref(wl, t0, t)
    del t0
    got, q = out.cpu().numpy(), host_bits(t["q"])
    worst = (0.0, 0.0)
    for i in range(wl.num_seqs):
        kd, vd, table = _dequantized_sequence(wl, i, kc, vc, ks, vs)
        ctx = wl.context_lens[i:i + 1]
        ref = oracle.paged_attention_f64(q[i:i + 1], kd, vd, table, ctx, None, wl.scale)
        e = assert_close(got[i:i + 1], ref, f"long_context fp8 sequence {i}")
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        del kd, vd
    _report("long_context fp8 layer 2 (all 4 sequences)", worst)


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("d,hq,hkv", [(128, 12, 2), (128, 8, 1), (256, 16, 4), (256, 24, 3)])
def test_long_partitions_over_an_fp8_cache(d, hq, hkv, fused):
    """4,096-token partitions (256 blocks: 64 per wave, a block id in every
    lane) over contexts of 4,097 to 9,000 tokens, next to short ones: the
    partition sizes the long-context plan picks, at contexts the oracle
    attends in full."""
    ctx = [4100, 8200, 9000, 5000, 17, 4096, 4097, 8192]
    wl = workloads.custom("fp8_long_part", ctx, [1] * len(ctx), len(ctx), hq, hkv, d,
                          seed=hq * d + fused)
    t = _fp8_cache(wl)
    t0 = {n: _np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale")}
    _, out = _run(wl, t, part=4096, fused=fused)
    kc, vc, ks, vs, qsl = _append_ref(wl, t0, t)
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, qsl, wl.scale)
    errs = assert_close(out.cpu().numpy(), ref, f"fp8 part=4096 d={d} G={hq // hkv}")
    _report(f"fp8 part=4096 d={d} G={hq // hkv} fused={fused}", errs)


@pytest.mark.parametrize("part", [0, 64])
def test_fused_fp8_append_skips_a_padding_slot(part):
    """A decode token with slot -1 is not written, and its sequence attends
    the pool's current row at ctx - 1 -- as with the separate calls."""
    ctx = [20, 40, 60, 300]
    wl = workloads.custom("fp8_pad", ctx, [1] * 4, 4, 12, 2, 128, seed=37)
    t = _fp8_cache(wl, poison=False)
    kc0, vc0, ks0, vs0 = (_np(t[n]) for n in ("k_codes", "v_codes", "k_scale", "v_scale"))
    slots = oracle.slot_mapping(wl.block_tables, wl.context_lens, None, 16)
    slots[1] = -1
    slots[3] = -1
    step = Step.from_workload(wl, kv_partition_tokens=part)
    cache = pkv.KVCache(t["k_codes"], t["v_codes"], t["k_scale"], t["v_scale"])
    out = torch.empty_like(t["q"])
    pkv.append_attention_step(cache, t["k_new"], t["v_new"], torch.from_numpy(slots).cuda(),
                              t["q"], out, step.block_tables, step.context_lens, None, 4,
                              wl.scale, step.max_context_len, 1, workspace=step.workspace,
                              kv_partition_tokens=part)
    torch.cuda.synchronize()
    kc, vc, ks, vs = ofp8.kv_append(kc0, vc0, ks0, vs0, host_bits(t["k_new"]),
                                    host_bits(t["v_new"]), slots)
    assert np.array_equal(_np(t["k_codes"]), kc) and np.array_equal(_np(t["v_codes"]), vc)
    assert np.array_equal(_np(t["k_scale"]).view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(_np(t["v_scale"]).view(np.uint32), vs.view(np.uint32))
    ref = oracle.paged_attention_fp8(host_bits(t["q"]), kc, vc, ks, vs, wl.block_tables,
                                     wl.context_lens, None, wl.scale)
    _report(f"fp8 padding slot part={part}", assert_close(out.cpu().numpy(), ref, "fp8 pad"))
