"""CPU oracle of the per-head projections around the absorbed decode
(TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never does, and nothing here imports it.

"MLA 在极长上下文下的显存带宽突围", section on absorbing the matrices at run
time: q~ = q^C W^UK, so that Score = q~ c^T + q^R k^R^T; "MLA & DSA
推理性能优化指南" §1.1 figure: W_UK and W_UV map the latent (d_c = 512) to
the heads (d_h = 128 each, §5.1).  Plain fp64 products:
  absorb_query:  q_nope[m, h, n] = sum_k q_c[m, h, k] * W_UK[h][k][n]
  project_out:   o[m, h, j]      = sum_d W_UV[h][j][d] * out[m, h, d]
W_UK is passed in the library's stored form w_uk_t[h, n, k] = W_UK[h][k][n].
"""
from __future__ import annotations

import numpy as np


def absorb_query(q_c, w_uk_t) -> np.ndarray:
    """q_c [M, H, 128], w_uk_t [H, 512, 128] -> q_nope [M, H, 512] (float64)."""
    q = np.asarray(q_c, dtype=np.float64)
    w = np.asarray(w_uk_t, dtype=np.float64)
    return np.einsum("mhk,hnk->mhn", q, w)


def project_out(out_latent, w_uv) -> np.ndarray:
    """out_latent [M, H, 512], w_uv [H, 128, 512] -> o [M, H, 128] (float64)."""
    x = np.asarray(out_latent, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    return np.einsum("hjd,mhd->mhj", w, x)
