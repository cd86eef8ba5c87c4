"""Dense brute force for tiny inputs (numpy, fp64).

TEST INFRASTRUCTURE ONLY.  Written independently of ``oracle.c``: it never
sees a block table, a pool or a slot.  It takes each sequence's keys and
values as plain contiguous arrays in logical order and applies the masked
softmax formula with an explicit mask matrix, the way a padded [B, length]
attention with a causal mask would (danielfleming.xyz, "Static batching",
section "What changed": a batch tensor plus a mask telling the model which
positions to ignore).

Each query row k of a sequence with n new tokens and ctx total tokens sits at
position ctx - n + k and may see positions 0 .. ctx - n + k.
"""
from __future__ import annotations

import numpy as np


def dense_attention(q_seq: np.ndarray, K_seq: np.ndarray, V_seq: np.ndarray,
                    scale: float) -> np.ndarray:
    """One sequence.

    q_seq: [n, Hq, d]; K_seq, V_seq: [ctx, Hkv, d] (logical order); returns [n, Hq, d].
    """
    q = np.asarray(q_seq, dtype=np.float64)
    K = np.asarray(K_seq, dtype=np.float64)
    V = np.asarray(V_seq, dtype=np.float64)
    n, Hq, d = q.shape
    ctx, Hkv, _ = K.shape
    G = Hq // Hkv
    rows = np.arange(n)[:, None] + (ctx - n)          # absolute position of each query row
    cols = np.arange(ctx)[None, :]
    visible = cols <= rows                            # [n, ctx] causal mask
    out = np.empty((n, Hq, d), dtype=np.float64)
    for h in range(Hq):
        kv = h // G
        S = scale * (q[:, h, :] @ K[:, kv, :].T)      # [n, ctx]
        S = np.where(visible, S, -np.inf)
        S = S - S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P = P / P.sum(axis=1, keepdims=True)
        out[:, h, :] = P @ V[:, kv, :]
    return out
