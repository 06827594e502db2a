"""CPU oracle of the non-absorbed MLA prefill (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never does, and nothing here imports it.

"MLA & DSA 推理性能优化指南" §3.1: in prefill the latent c_t is first
decompressed into full per-head K and V and a standard multi-head attention
kernel runs over them (the non-absorbed path, §1.1 figure); §5.1: 128 heads
of d_h = 128 plus the 64-dim decoupled RoPE key shared by all heads.  So per
head the key is [W_UK[h] c_t | k_rope_t] (192 dims), the value W_UV[h] c_t
(128 dims), and the query [q_c | q_rope] (192 dims).  This oracle computes
the plain definition over given per-head Q, K, V:

    z[t, j] = scale * q[t] . k[j]        for j <= t (causal) or all j < T
    out[t]  = sum_j softmax_j(z[t]) v[j],  lse[t] = ln sum_j exp(z[t, j])

in fp64, for q [B, T, H, 192], k [B, T, H, 192], v [B, T, H, 128].
"""
from __future__ import annotations

import numpy as np


def prefill(q, k, v, scale: float, causal: bool = True):
    """(out [B, T, H, 128], lse [B, T, H]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, _ = q.shape
    out = np.zeros((B, T, H, v.shape[-1]))
    lse = np.zeros((B, T, H))
    for b in range(B):
        for h in range(H):
            z = scale * (q[b, :, h] @ k[b, :, h].T)          # [T, T]
            if causal:
                z = np.where(np.tril(np.ones((T, T), dtype=bool)), z, -np.inf)
            m = z.max(axis=1, keepdims=True)
            e = np.exp(z - m)
            s = e.sum(axis=1, keepdims=True)
            out[b, :, h] = (e / s) @ v[b, :, h]
            lse[b, :, h] = (m + np.log(s))[:, 0]
    return out, lse
