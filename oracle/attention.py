"""Oracle for the lookahead-attention call on its own -- test infrastructure only.

One decoding step's attention for one layer: every block row attends to the
whole committed KV prefix and to the block rows the lookahead mask lets it
see ([LD] §3.4 "The custom attention mask (Figure 2)"; the mask is the set
rules of oracle.lookahead.block_visible, materialised here).  Plain float64
softmax(q k^T / sqrt(hd)) v; query head h reads KV head floor(h * Hkv / H).
"""
from __future__ import annotations

import numpy as np

from .lookahead import block_mask


def lookahead_attention(q, k_prefix, v_prefix, k_block, v_block, N, W, G):
    """q [M, H, hd]; k/v_prefix [P, Hkv, hd]; k/v_block [M, Hkv, hd] (any
    float dtype, read as float64).  Returns [M, H, hd] float64."""
    q = np.asarray(q, dtype=np.float64)
    kk = np.concatenate([np.asarray(k_prefix, np.float64), np.asarray(k_block, np.float64)])
    vv = np.concatenate([np.asarray(v_prefix, np.float64), np.asarray(v_block, np.float64)])
    M, H, hd = q.shape
    P = k_prefix.shape[0]
    Hkv = kk.shape[1]
    vis = np.concatenate([np.ones((M, P), dtype=bool), block_mask(N, W, G)], axis=1)
    out = np.empty((M, H, hd))
    for h in range(H):
        kh = h * Hkv // H
        s = (q[:, h, :] @ kk[:, kh, :].T) / np.sqrt(hd)
        s = np.where(vis, s, -np.inf)
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vv[:, kh, :]
    return out
