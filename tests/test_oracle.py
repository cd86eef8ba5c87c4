"""Pins for the CPU oracle: closed forms, invariants, a dense brute force that
knows nothing of paging, and the pages' worked sizing numbers.

Each test pins the oracle to something other than itself, so that a dropped
term, a wrong index, a wrong sign or a transposed operand in ``oracle.c``
fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads
from oracle.dense import dense_attention

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")


# ----------------------------------------------------------------- helpers ---

def _rand_half(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


def _scatter_dense_into_pool(K_seqs, V_seqs, tables, num_blocks, bs=16, fill=np.nan):
    """Write each sequence's contiguous K/V [ctx, Hkv, d] into a fresh pool
    through its table row, by enumerating (block, offset) pairs in order --
    a construction independent of the oracle's div/mod indexing."""
    Hkv, d = K_seqs[0].shape[1:]
    kp = np.full((num_blocks, Hkv, bs, d), fill, dtype=np.float16)
    vp = np.full((num_blocks, Hkv, bs, d), fill, dtype=np.float16)
    for i, (K, V) in enumerate(zip(K_seqs, V_seqs)):
        positions = [(b, o) for b in tables[i] for o in range(bs)]
        for p in range(K.shape[0]):
            b, o = positions[p]
            kp[b, :, o, :] = K[p]
            vp[b, :, o, :] = V[p]
    return kp, vp


def _random_case(rng, ctx, new, hq, hkv, d, extra_blocks=3, dup_block_edges=False):
    """Dense per-sequence data plus a scattered pool and tables."""
    ctx = np.asarray(ctx, np.int32)
    new = np.asarray(new, np.int32)
    nb = [-(-int(c) // 16) for c in ctx]
    num_blocks = sum(nb) + extra_blocks
    perm = rng.permutation(num_blocks)
    maxblk = max(nb)
    tables = np.zeros((len(ctx), maxblk), np.int32)
    pos = 0
    for i, n in enumerate(nb):
        tables[i, :n] = perm[pos:pos + n]
        pos += n
    K_seqs = [_rand_half(rng, (int(c), hkv, d)) for c in ctx]
    V_seqs = [_rand_half(rng, (int(c), hkv, d)) for c in ctx]
    kp, vp = _scatter_dense_into_pool(K_seqs, V_seqs, tables, num_blocks)
    q = _rand_half(rng, (int(new.sum()), hq, d))
    qsl = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    return dict(ctx=ctx, new=new, tables=tables, kp=kp, vp=vp, q=q, qsl=qsl,
                K_seqs=K_seqs, V_seqs=V_seqs, num_blocks=num_blocks)


def _dense_reference(case, scale):
    outs = []
    for i in range(len(case["ctx"])):
        r0, r1 = case["qsl"][i], case["qsl"][i + 1]
        outs.append(dense_attention(case["q"][r0:r1], case["K_seqs"][i], case["V_seqs"][i], scale))
    return np.concatenate(outs, axis=0)


# --------------------------------------------------------- fp16 decoding ---

def test_half_decoding_matches_numpy_on_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_float64(bits)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


# ------------------------------------------------------- page arithmetic ---

def test_page_sizing_numbers():
    g = json.load(open(GOLDEN))
    a = g["qwen3_8b_bytes_per_token"]
    assert workloads.kv_bytes_per_token(a["layers"], a["kv_heads"], a["head_dim"],
                                        a["bytes_per_elem"]) == a["bytes_per_token"]
    b = g["qwen3_8b_16gib_pool"]
    blocks = workloads.pool_blocks_for_bytes(b["pool_bytes"], b["bytes_per_token"])
    assert blocks == b["blocks"] and blocks * 16 == b["tokens"]
    c = g["qwen3_8b_request_blocks"]
    nb = workloads.blocks_for_tokens(c["prompt_tokens"] + c["generated_tokens"])
    assert nb == c["blocks"]
    assert b["blocks"] // nb == c["sequences_at_final_size"]
    d = g["qwen25_1p5b_bytes_per_token"]
    assert workloads.kv_bytes_per_token(d["layers"], d["kv_heads"], d["head_dim"],
                                        d["bytes_per_elem"]) == d["bytes_per_token"]
    e = g["qwen25_1p5b_cache_p1024_b256"]
    cache = e["batch"] * (e["prompt_tokens"] + e["budget_tokens"]) * e["bytes_per_token"]
    assert cache == e["cache_gib"] * 2 ** 30
    f = g["long_window_kv"]
    for key, bpe in (("gib_fp16", 2), ("gib_8bit", 1), ("gib_4bit", 0.5)):
        per_tok = workloads.kv_bytes_per_token(f["kv_layers"], f["kv_heads"], f["head_dim"], bpe)
        assert per_tok * f["window_tokens"] == f[key] * 2 ** 30


def test_page_request_block_count_bounds_slot_mapping():
    """A 1,368 + 256 token sequence holds 102 blocks: its last token maps into
    table entry 101, and a 101-entry table is too short for it."""
    ctx = 1368 + 256
    table = np.arange(1000, 1102, dtype=np.int32)[None, :]         # 102 entries
    slots = oracle.slot_mapping(table, [ctx], None, 16)
    assert slots[0] == table[0, 101] * 16 + (ctx - 1) % 16
    with pytest.raises(oracle.OracleError):
        oracle.slot_mapping(table[:, :101], [ctx], None, 16)


# ---------------------------------------------------------- slot mapping ---

def test_slot_mapping_matches_enumeration():
    rng = np.random.default_rng(3)
    ctx = np.array([1, 15, 16, 17, 33, 40, 100], np.int32)
    new = np.array([1, 1, 1, 1, 5, 8, 1], np.int32)
    case = _random_case(rng, ctx, new, 2, 1, 8)
    slots = oracle.slot_mapping(case["tables"], ctx, case["qsl"], 16)
    expect = []
    for i, c in enumerate(ctx):
        slot_of_position = [b * 16 + o for b in case["tables"][i] for o in range(16)]
        expect += [slot_of_position[p] for p in range(c - new[i], c)]
    assert slots.tolist() == expect


def test_slot_mapping_identity_table_is_position():
    ctx = np.array([5, 16, 31], np.int32)
    table = np.tile(np.arange(2, dtype=np.int32), (3, 1))
    slots = oracle.slot_mapping(table, ctx, None, 16)
    assert slots.tolist() == [4, 15, 30]


# ----------------------------------------------------------------- append ---

def test_append_writes_exactly_the_slots_and_nothing_else():
    rng = np.random.default_rng(5)
    NB, Hkv, d = 6, 2, 16
    kp = np.arange(NB * Hkv * 16 * d, dtype=np.uint32).astype(np.uint16).reshape(NB, Hkv, 16, d)
    vp = (kp ^ 0x5555).astype(np.uint16)
    slots = np.array([17, -1, 95, 0], np.int64)
    kn = rng.integers(0, 65536, size=(4, Hkv, d)).astype(np.uint16)
    vn = rng.integers(0, 65536, size=(4, Hkv, d)).astype(np.uint16)
    k2, v2 = oracle.kv_append(kp, vp, kn, vn, slots)
    touched = np.zeros((NB, 16), bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, off = divmod(int(s), 16)
        touched[blk, off] = True
        assert np.array_equal(k2[blk, :, off, :], kn[t]) and np.array_equal(v2[blk, :, off, :], vn[t])
    mask = np.broadcast_to(touched[:, None, :, None], kp.shape)
    assert np.array_equal(k2[~mask], kp[~mask]) and np.array_equal(v2[~mask], vp[~mask])
    # the padding token (slot -1) was written nowhere: its row appears nowhere new
    assert not any(np.array_equal(k2[b, g, o], kn[1][g])
                   for b in range(NB) for g in range(Hkv) for o in range(16))


def test_append_then_attend_single_token_returns_the_new_value():
    """Append a token into an otherwise NaN pool, attend a 1-token context:
    the output must be exactly the appended V row (softmax of one score is 1)."""
    rng = np.random.default_rng(7)
    NB, Hkv, Hq, d = 4, 2, 6, 32
    kp = np.full((NB, Hkv, 16, d), np.nan, np.float16)
    vp = kp.copy()
    table = np.array([[2]], np.int32)
    slots = oracle.slot_mapping(table, [1], None, 16)
    kn, vn = _rand_half(rng, (1, Hkv, d)), _rand_half(rng, (1, Hkv, d))
    k2, v2 = oracle.kv_append(kp, vp, kn, vn, slots)
    q = _rand_half(rng, (1, Hq, d))
    out = oracle.paged_attention(q, k2, v2, table, [1], None, 0.125)
    for h in range(Hq):
        assert np.array_equal(out[0, h], vn[0, h // 3].astype(np.float64))


# -------------------------------------------------------------- attention ---

@pytest.mark.parametrize("hq,hkv", [(6, 2), (4, 4), (8, 1)])
def test_attention_matches_dense_brute_force(hq, hkv):
    rng = np.random.default_rng(11 + hq)
    ctx = [1, 15, 16, 17, 31, 32, 33, 40]
    new = [1, 1, 1, 1, 1, 1, 1, 8]          # last sequence is a causal chunk
    case = _random_case(rng, ctx, new, hq, hkv, 16)
    scale = 0.3
    got = oracle.paged_attention(case["q"], case["kp"], case["vp"], case["tables"], case["ctx"],
                                 case["qsl"], scale)
    want = _dense_reference(case, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_causal_chunk_rows_see_only_their_prefix():
    """Rows of a chunk must not depend on later keys: changing the chunk's
    last key and value changes only the last row."""
    rng = np.random.default_rng(13)
    case = _random_case(rng, [20], [6], 2, 1, 8)
    a = oracle.paged_attention(case["q"], case["kp"], case["vp"], case["tables"], case["ctx"],
                               case["qsl"], 0.5)
    blk, off = case["tables"][0, 19 // 16], 19 % 16
    kp, vp = case["kp"].copy(), case["vp"].copy()
    kp[blk, :, off, :] += np.float16(3.0)
    vp[blk, :, off, :] -= np.float16(2.0)
    b = oracle.paged_attention(case["q"], kp, vp, case["tables"], case["ctx"], case["qsl"], 0.5)
    assert np.array_equal(a[:5], b[:5])
    assert not np.allclose(a[5], b[5])


def test_equal_keys_or_zero_query_give_mean_of_values():
    rng = np.random.default_rng(17)
    case = _random_case(rng, [37], [1], 4, 2, 16)
    mean_v = case["V_seqs"][0].astype(np.float64).mean(axis=0)     # [Hkv, d]
    # equal keys
    kp = case["kp"].copy()
    for b in case["tables"][0][:3]:
        kp[b] = np.float16(0.75)
    out = oracle.paged_attention(case["q"], kp, case["vp"], case["tables"], case["ctx"], None, 0.2)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], mean_v[h // 2], rtol=1e-12, atol=1e-14)
    # zero query
    q0 = np.zeros_like(case["q"])
    out = oracle.paged_attention(q0, case["kp"], case["vp"], case["tables"], case["ctx"], None, 0.2)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], mean_v[h // 2], rtol=1e-12, atol=1e-14)


def test_constant_values_give_the_constant():
    rng = np.random.default_rng(19)
    case = _random_case(rng, [50], [1], 2, 1, 8)
    vp = np.full_like(case["vp"], np.float16(-1.25))
    out = oracle.paged_attention(case["q"], case["kp"], vp, case["tables"], case["ctx"], None, 1.0)
    np.testing.assert_allclose(out, -1.25, rtol=1e-14)


def test_dominant_key_selects_its_value_and_sign_matters():
    rng = np.random.default_rng(23)
    d = 16
    case = _random_case(rng, [30], [1], 1, 1, d)
    q = case["q"].astype(np.float64)[0, 0]
    blk, off = case["tables"][0, 9 // 16], 9
    kp = case["kp"].copy()
    kp[blk, 0, off, :] = (8.0 * q).astype(np.float16)              # key 9 aligned with q
    out = oracle.paged_attention(case["q"], kp, case["vp"], case["tables"], case["ctx"], None, 1.0)
    v9 = case["V_seqs"][0][9, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], v9, atol=1e-6)
    kp[blk, 0, off, :] = (-8.0 * q).astype(np.float16)             # anti-aligned: weight ~ 0
    out = oracle.paged_attention(case["q"], kp, case["vp"], case["tables"], case["ctx"], None, 1.0)
    assert np.abs(out[0, 0] - v9).max() > 0.1


def test_block_placement_permutation_is_invisible():
    rng = np.random.default_rng(29)
    case = _random_case(rng, [5, 40, 70], [1, 1, 1], 6, 2, 16, extra_blocks=5)
    a = oracle.paged_attention(case["q"], case["kp"], case["vp"], case["tables"], case["ctx"], None, 0.25)
    relabel = rng.permutation(case["num_blocks"])
    kp = np.empty_like(case["kp"])
    vp = np.empty_like(case["vp"])
    kp[relabel] = case["kp"]
    vp[relabel] = case["vp"]
    tables = relabel[case["tables"]].astype(np.int32)
    b = oracle.paged_attention(case["q"], kp, vp, tables, case["ctx"], None, 0.25)
    assert np.array_equal(a, b)


def test_stale_slots_are_never_read():
    """NaN everywhere outside the live positions (including the unused tail
    of each last block and the unused table entries) leaves outputs finite."""
    rng = np.random.default_rng(31)
    case = _random_case(rng, [3, 17, 33], [1, 1, 1], 2, 1, 8)
    tables = case["tables"].copy()
    tables[0, 1:] = case["num_blocks"] - 1                        # unused entries -> a NaN block
    out = oracle.paged_attention(case["q"], case["kp"], case["vp"], tables, case["ctx"], None, 0.5)
    assert np.isfinite(out).all()


def test_shift_of_every_key_along_any_vector_is_invisible():
    """Adding one vector u to every key adds q.u to every score of a head,
    which the softmax cancels.  Keys are put on a 1/8 grid so that the shifted
    keys are exact in fp16."""
    rng = np.random.default_rng(37)
    case = _random_case(rng, [45], [1], 2, 1, 8)
    kp = (np.round(case["kp"].astype(np.float64) * 8) / 8).astype(np.float16)
    u = (np.round(rng.standard_normal(8) * 4) / 8)
    shifted = (kp.astype(np.float64) + u).astype(np.float16)
    live = ~np.isnan(kp)
    assert np.array_equal(shifted.astype(np.float64)[live], (kp.astype(np.float64) + u)[live])
    a = oracle.paged_attention(case["q"], kp, case["vp"], case["tables"], case["ctx"], None, 0.5)
    b = oracle.paged_attention(case["q"], shifted, case["vp"], case["tables"], case["ctx"], None, 0.5)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-13)


def test_output_is_linear_in_values():
    rng = np.random.default_rng(41)
    case = _random_case(rng, [29], [1], 2, 2, 8)
    v1 = case["vp"]
    v2 = _rand_half(rng, v1.shape)
    f = lambda vp: oracle.paged_attention(case["q"], case["kp"], vp, case["tables"], case["ctx"], None, 0.5)
    s = (v1.astype(np.float32) + v2.astype(np.float32)).astype(np.float16)
    exact = np.array_equal(s.astype(np.float64), v1.astype(np.float64) + v2.astype(np.float64))
    if exact:
        np.testing.assert_allclose(f(s), f(v1) + f(v2), rtol=1e-10, atol=1e-12)
    else:
        # use a sum that is exact in fp16: v and v (doubling)
        np.testing.assert_allclose(f((v1.astype(np.float32) * 2).astype(np.float16)), 2 * f(v1),
                                   rtol=1e-12, atol=1e-13)


def test_heads_sharing_a_kv_head_with_equal_queries_agree():
    rng = np.random.default_rng(43)
    case = _random_case(rng, [21], [1], 6, 2, 8)
    q = case["q"].copy()
    q[0, 1] = q[0, 0]
    q[0, 2] = q[0, 0]
    out = oracle.paged_attention(q, case["kp"], case["vp"], case["tables"], case["ctx"], None, 0.5)
    assert np.array_equal(out[0, 0], out[0, 1]) and np.array_equal(out[0, 0], out[0, 2])
    assert not np.array_equal(out[0, 0], out[0, 3])       # head 3 reads the other KV head


def test_lse_of_equal_scores_is_log_count():
    rng = np.random.default_rng(47)
    case = _random_case(rng, [24], [1], 2, 1, 8)
    q0 = np.zeros_like(case["q"])
    _, lse = oracle.paged_attention(q0, case["kp"], case["vp"], case["tables"], case["ctx"], None,
                                    0.5, want_lse=True)
    np.testing.assert_allclose(lse, math.log(24), rtol=1e-14)


def test_seq_subset_computes_only_those_sequences():
    rng = np.random.default_rng(53)
    case = _random_case(rng, [5, 9, 20], [1, 1, 1], 2, 1, 8)
    full = oracle.paged_attention(case["q"], case["kp"], case["vp"], case["tables"], case["ctx"], None, 0.5)
    sub = oracle.paged_attention(case["q"], case["kp"], case["vp"], case["tables"], case["ctx"], None,
                                 0.5, seq_subset=[2])
    assert np.array_equal(sub[2], full[2]) and np.isnan(sub[:2]).all()


# --------------------------------------------------------- split + merge ---

@pytest.mark.parametrize("cuts", [[], [1], [7, 8, 30], [0, 0, 13, 64, 64]])
def test_lse_merge_of_partitions_equals_full_attention(cuts):
    rng = np.random.default_rng(59)
    ctx, d = 64, 16
    q = rng.standard_normal(d) * 2
    K = rng.standard_normal((ctx, d)) * 2
    V = rng.standard_normal((ctx, d))
    full = oracle.attention_contiguous(q, K, V, 0.4)
    edges = [0] + sorted(cuts) + [ctx]
    parts = [oracle.attention_partial(q, K, V, lo, hi, 0.4) for lo, hi in zip(edges[:-1], edges[1:])]
    merged = oracle.lse_merge(np.stack([p[0] for p in parts]), [p[1] for p in parts],
                              [p[2] for p in parts])
    np.testing.assert_allclose(merged, full, rtol=1e-12, atol=1e-14)
    # and the full attention itself against the dense formula
    want = dense_attention(q[None, None, :], K[:, None, :], V[:, None, :], 0.4)[0, 0]
    np.testing.assert_allclose(full, want, rtol=1e-12, atol=1e-14)


def test_empty_partition_contributes_nothing():
    rng = np.random.default_rng(61)
    q, K, V = rng.standard_normal(8), rng.standard_normal((10, 8)), rng.standard_normal((10, 8))
    o, m, l = oracle.attention_partial(q, K, V, 4, 4, 1.0)
    assert l == 0.0 and m == -math.inf and np.all(o == 0)
    a = oracle.attention_partial(q, K, V, 0, 10, 1.0)
    merged = oracle.lse_merge(np.stack([a[0], o]), [a[1], m], [a[2], l])
    assert np.array_equal(merged, a[0])
