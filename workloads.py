"""Seeded synthetic workloads for the paged KV append + paged attention step.

This module is the only code shared by the HIP path's callers (tests,
bench) and the oracle's callers.  It draws random things and sizes buffers;
it holds none of the method's arithmetic (no slot computation, no
attention, no softmax).

What it produces, per workload:
  * context lengths (after this step's append) and new-token counts per
    sequence, decode sequences first, then prefill chunks;
  * a block pool size and a block table per sequence, holding
    ceil(ctx / 16) physical blocks drawn from a seeded permutation of the
    pool (blocks scattered through the pool, as in a paged cache that
    stores only real tokens -- danielfleming.xyz, "Static batching",
    section "Ragged batches");
  * per layer, N(0,1) fp16 K/V pools, queries and new K/V rows, drawn with a
    seeded torch generator on the requested device.

Sizing helpers restate the pages' capacity arithmetic (deepconcepts.dev,
"Continuous Batching Is Not a Bigger Batch", section "Where the batch size
actually comes from": bytes per token = 2 x layers x kv_heads x head_dim x
bytes; blocks = tokens / 16 rounded up per sequence; pool blocks = whole
16-token blocks that fit).

Workload recipes (the five shapes the benchmark and parity tests use):
  small_b4        1 layer, B=4, 12/2 heads, d=128, ctx {16,64,256,1024},
                  128-block pool, tables = consecutive runs of a seeded
                  permutation of the pool.
  qwen_uniform    28 layers, B=256, ctx 512 each, 12/2 heads, d=128, pool
                  ceil(1.2 x needed) blocks, tables from a seeded permutation.
  qwen_ragged     28 layers, B=83, ctx = prompt + progress, prompt uniform on
                  {16,64,256,1024,4096}, progress uniform on {0..256}.
  long_context    16 layers, B=4, 16/4 heads, d=256, ctx 262,144 each, pool
                  exactly the 65,536 blocks needed.
  qwen_mixed      28 layers, 64 decode sequences with ctx uniform on
                  [256, 4096] plus one prefill chunk of 512 query tokens on an
                  8,192-token cached prefix (ctx 8,704).
  qwen_spec       28 layers, 64 sequences with ctx uniform on [256, 4096],
                  each verifying 4 query tokens (multi-token decode).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
FP16_BYTES = 2


# ---------------------------------------------------------------- sizing ---

def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bytes_per_elem: float) -> float:
    """K and V bytes one token occupies across all layers (2 x L x Hkv x d x bytes)."""
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def blocks_for_tokens(tokens: int, block_size: int = BLOCK_SIZE) -> int:
    """Whole blocks a sequence of `tokens` tokens holds."""
    return -(-int(tokens) // block_size)


def pool_blocks_for_bytes(pool_bytes: int, bytes_per_token: float, block_size: int = BLOCK_SIZE) -> int:
    """Whole blocks that fit in a pool of `pool_bytes`."""
    return int(pool_bytes // (bytes_per_token * block_size))


# -------------------------------------------------------------- workload ---

@dataclass
class Workload:
    name: str
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    context_lens: np.ndarray          # int32 [B], includes this step's new tokens
    new_tokens: np.ndarray            # int32 [B], 1 for decode sequences
    num_decode_seqs: int
    num_blocks: int                   # pool blocks per layer
    block_tables: np.ndarray          # int32 [B, max_blocks_per_seq]
    seed: int = 0
    block_size: int = BLOCK_SIZE
    free_blocks: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.new_tokens.sum())

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def query_start_loc(self) -> np.ndarray:
        """int32 [B+1]: row offset of each sequence's new tokens in the packed query."""
        return np.concatenate([[0], np.cumsum(self.new_tokens)]).astype(np.int32)

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def max_query_len(self) -> int:
        return int(self.new_tokens.max())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    # byte model of one layer of the step (the quantities the method must move)
    def kv_read_bytes_per_layer(self, decode_only: bool = False) -> int:
        ctx = self.context_lens[: self.num_decode_seqs] if decode_only else self.context_lens
        return int(ctx.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * FP16_BYTES

    def qo_bytes_per_layer(self, decode_only: bool = False) -> int:
        t = self.num_decode_seqs if decode_only else self.num_tokens
        return 2 * t * self.num_q_heads * self.head_dim * FP16_BYTES

    def prefill_flops_per_layer(self) -> int:
        """4 x d x Hq flops per (query row, attended position) of the prefill
        chunks (S = QK^T and O = PV, 2 flops per multiply-add), causal: row k
        of a chunk of n rows ending at ctx attends ctx - n + k + 1 positions."""
        ctx = self.context_lens[self.num_decode_seqs:].astype(np.int64)
        n = self.new_tokens[self.num_decode_seqs:].astype(np.int64)
        pairs = int((n * (ctx - n + 1) + n * (n - 1) // 2).sum())
        return 4 * self.head_dim * self.num_q_heads * pairs

    def short_chunk(self) -> np.ndarray:
        """bool [B]: sequences whose new tokens, times the query heads per KV
        head, fit one 64-row tile (decodes and multi-token decodes): their
        attention streams the cache rather than filling the matrix cores."""
        g = self.num_q_heads // self.num_kv_heads
        return self.new_tokens.astype(np.int64) * g <= 64

    def append_bytes_per_layer(self) -> int:
        return 2 * self.num_tokens * self.num_kv_heads * self.head_dim * FP16_BYTES


def _tables_from_permutation(perm: np.ndarray, ctx: np.ndarray, block_size: int,
                             fill_value: int) -> tuple[np.ndarray, np.ndarray]:
    """Sequences take consecutive runs of `perm`, ceil(ctx/bs) blocks each."""
    nb = np.array([blocks_for_tokens(c, block_size) for c in ctx], dtype=np.int64)
    maxblk = int(nb.max()) if len(nb) else 1
    tables = np.full((len(ctx), maxblk), fill_value, dtype=np.int32)
    pos = 0
    for i, n in enumerate(nb):
        tables[i, :n] = perm[pos:pos + n]
        pos += n
    return tables, perm[pos:].astype(np.int32)


def _build(name, layers, hq, hkv, d, ctx, new, n_dec, pool_factor, seed, pool_blocks=None):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, dtype=np.int32)
    new = np.asarray(new, dtype=np.int32)
    needed = int(sum(blocks_for_tokens(c) for c in ctx))
    nblocks = pool_blocks if pool_blocks is not None else int(math.ceil(pool_factor * needed))
    perm = rng.permutation(nblocks).astype(np.int32)
    tables, free = _tables_from_permutation(perm, ctx, BLOCK_SIZE, fill_value=0)
    return Workload(name=name, num_layers=layers, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                    context_lens=ctx, new_tokens=new, num_decode_seqs=n_dec, num_blocks=nblocks,
                    block_tables=tables, seed=seed, free_blocks=free)


def small_b4(seed: int = 0, layers: int = 1) -> Workload:
    ctx = [16, 64, 256, 1024]
    return _build("small_b4", layers, 12, 2, 128, ctx, [1] * 4, 4, None, seed, pool_blocks=128)


def qwen_uniform(seed: int = 0, batch: int = 256, ctx_len: int = 512, layers: int = 28) -> Workload:
    return _build("qwen_uniform", layers, 12, 2, 128, [ctx_len] * batch, [1] * batch, batch, 1.2, seed)


def qwen_ragged(seed: int = 0, batch: int = 83, layers: int = 28) -> Workload:
    rng = np.random.default_rng(seed + 1)
    prompts = rng.choice(np.array([16, 64, 256, 1024, 4096]), size=batch)
    progress = rng.integers(0, 256, size=batch, endpoint=True)
    ctx = (prompts + progress).astype(np.int32)
    return _build("qwen_ragged", layers, 12, 2, 128, ctx, [1] * batch, batch, 1.2, seed)


def long_context(seed: int = 0, batch: int = 4, ctx_len: int = 262144, layers: int = 16) -> Workload:
    needed = batch * blocks_for_tokens(ctx_len)
    return _build("long_context", layers, 16, 4, 256, [ctx_len] * batch, [1] * batch, batch, None,
                  seed, pool_blocks=needed)


def qwen_mixed(seed: int = 0, decodes: int = 64, chunk: int = 512, prefix: int = 8192,
               layers: int = 28) -> Workload:
    rng = np.random.default_rng(seed + 2)
    dec_ctx = rng.integers(256, 4096, size=decodes, endpoint=True)
    ctx = np.concatenate([dec_ctx, [prefix + chunk]]).astype(np.int32)
    new = np.array([1] * decodes + [chunk], dtype=np.int32)
    return _build("qwen_mixed", layers, 12, 2, 128, ctx, new, decodes, 1.2, seed)


def qwen_spec(seed: int = 0, batch: int = 64, query_len: int = 4, layers: int = 28) -> Workload:
    """Decoding sequences that each verify several tokens in one pass: the
    token sampled last pass plus query_len - 1 drafted ones (a request's
    scheduled tokens include its speculative ones -- deepconcepts.dev,
    "Continuous Batching Is Not a Bigger Batch", scheduler note on
    num_tokens_with_spec).  Contexts uniform on [256, 4096] after the step,
    as the decodes of qwen_mixed; every sequence is a short causal chunk."""
    rng = np.random.default_rng(seed + 3)
    ctx = rng.integers(256, 4096, size=batch, endpoint=True).astype(np.int32)
    new = np.full(batch, query_len, dtype=np.int32)
    return _build("qwen_spec", layers, 12, 2, 128, ctx, new, 0, 1.2, seed)


def custom(name: str, ctx, new, num_decode_seqs: int, hq: int, hkv: int, d: int, layers: int = 1,
           pool_factor: float = 1.5, seed: int = 0, pool_blocks: int | None = None) -> Workload:
    """Arbitrary small shapes for parity and edge-case tests."""
    return _build(name, layers, hq, hkv, d, ctx, new, num_decode_seqs, pool_factor, seed,
                  pool_blocks=pool_blocks)


def layer_tensors_fp8(wl: Workload, layer: int, device="cpu", scale_exp=(-6, -2),
                      v_scale_exp=None):
    """An fp8 (E4M3) cache of one layer with N(0,1)-like values, drawn
    directly as bytes: k_codes, v_codes uint8 [NB, Hkv, 16, d] with random
    sign, exponent field 4..10 and mantissa (values 2^-3 .. ~15, no NaN
    codes), k_scale, v_scale float32 [NB, Hkv, 16] random powers of two
    2^lo .. 2^(hi-1) for scale_exp = (lo, hi) (default 2^-6 .. 2^-3; V's
    from v_scale_exp when given); plus fp16 q, k_new, v_new as
    layer_tensors.  Drawn with a torch generator seeded by (seed, layer) on
    `device`."""
    import torch

    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed * 1_000_003 + layer * 7919 + 29)
    shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)

    def randint(lo, hi, shp, dtype):
        return torch.randint(lo, hi, shp, generator=gen, device=dev, dtype=dtype)

    def codes():
        c = randint(0, 2, shape, torch.uint8) << 7
        c |= randint(4, 11, shape, torch.uint8) << 3
        c |= randint(0, 8, shape, torch.uint8)
        return c

    def scales(lo, hi):
        return torch.exp2(randint(lo, hi, shape[:3], torch.int32).to(torch.float32))

    t = layer_tensors(Workload(wl.name, wl.num_layers, wl.num_q_heads, wl.num_kv_heads,
                               wl.head_dim, wl.context_lens, wl.new_tokens, wl.num_decode_seqs,
                               1, wl.block_tables, wl.seed), layer, device)
    vse = scale_exp if v_scale_exp is None else v_scale_exp
    return {"k_codes": codes(), "v_codes": codes(), "k_scale": scales(*scale_exp),
            "v_scale": scales(*vse),
            "q": t["q"], "k_new": t["k_new"], "v_new": t["v_new"]}


def serving_requests(seed: int = 0, num_requests: int = 256, prompt_range=(256, 2480),
                     output_range=(50, 781), shared_prefix: int = 0, prefix_groups: int = 0):
    """A queue of requests for the per-pass scheduler: prompt lengths uniform
    on prompt_range (mean 1,368 by default, the prompt size of the pages'
    worked example -- deepconcepts.dev, "Where the batch size actually comes
    from"), output lengths uniform on output_range (the 50- and 781-token
    requests of the same page's introduction).  With prefix_groups > 0 each
    request draws a group whose first shared_prefix prompt tokens it shares.
    Returns (prompt_lens, max_new_tokens, prefix_ids) int arrays."""
    rng = np.random.default_rng(seed + 4)
    prompts = rng.integers(prompt_range[0], prompt_range[1], size=num_requests, endpoint=True)
    outputs = rng.integers(output_range[0], output_range[1], size=num_requests, endpoint=True)
    if prefix_groups > 0:
        groups = rng.integers(0, prefix_groups, size=num_requests)
        prompts = np.maximum(prompts, shared_prefix + 1)
    else:
        groups = np.full(num_requests, -1)
    return prompts.astype(np.int64), outputs.astype(np.int64), groups.astype(np.int64)


def free_block_order(num_blocks: int, seed: int = 0) -> np.ndarray:
    """A seeded permutation of the pool: the initial order of the scheduler's
    free-block queue, so that block tables scatter through the pool."""
    return np.random.default_rng(seed + 5).permutation(num_blocks).astype(np.int32)


def token_kv_rows(key: int, positions, num_kv_heads: int, head_dim: int, layer: int = 0,
                  seed: int = 0) -> np.ndarray:
    """Deterministic N(0,1) fp16 K and V rows of tokens, a pure function of
    (key, position, layer): float16 [len(positions), 2, Hkv, d] (0 = K, 1 = V).
    A token that is computed again (after a preemption), or shared by
    requests with a common prefix (same key), gets the same rows."""
    out = np.empty((len(positions), 2, num_kv_heads, head_dim), np.float16)
    for j, p in enumerate(positions):
        rng = np.random.default_rng([seed, int(key) & 0x7FFFFFFFFFFFFFFF, int(p), layer])
        out[j] = rng.standard_normal((2, num_kv_heads, head_dim)).astype(np.float16)
    return out


WORKLOADS = {
    "small_b4": small_b4,
    "qwen_uniform": qwen_uniform,
    "qwen_ragged": qwen_ragged,
    "long_context": long_context,
    "qwen_mixed": qwen_mixed,
    "qwen_spec": qwen_spec,
}


# ------------------------------------------------------------------ data ---

def layer_tensors(wl: Workload, layer: int, device="cpu"):
    """N(0,1) fp16 tensors of one layer: k_pool, v_pool, q, k_new, v_new.

    Drawn from a torch generator seeded by (seed, layer) on `device`, so a
    layer can be regenerated on its own.
    """
    import torch

    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed * 1_000_003 + layer * 7919 + 17)
    shape_pool = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
    T = wl.num_tokens

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=dev, dtype=torch.float16)

    return {
        "k_pool": randn(*shape_pool),
        "v_pool": randn(*shape_pool),
        "q": randn(T, wl.num_q_heads, wl.head_dim),
        "k_new": randn(T, wl.num_kv_heads, wl.head_dim),
        "v_new": randn(T, wl.num_kv_heads, wl.head_dim),
    }
