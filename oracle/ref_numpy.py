"""NumPy fp64 oracle for weight-absorbed MLA decode (TEST INFRASTRUCTURE ONLY).

A second, independent implementation of the definition the C oracle
computes, written vectorised over tokens (gather visible latent rows into a
matrix, one matrix product for scores, one for the output).  Tiny inputs
only.  Also holds the un-absorbed (MHA-mode) computation used to pin the
absorption identity.

Sources:
  * "MLA 在极长上下文下的显存带宽突围", section "运行期矩阵吸收避免潜在张量展开":
    q~ = q^C W_UK and Score = q~ (c^KV)^T + q^R (k^R)^T.
  * "MLA & DSA 推理性能优化指南" §1.1 figure: the non-absorbed path first
    decompresses c into per-head K (W_UK) and V (W_UV), then runs standard
    MHA; the absorbed path works in the latent space.
"""
from __future__ import annotations

import numpy as np

PAGE = 64
DC = 512


def _f64(t):
    import torch
    if isinstance(t, torch.Tensor):
        if t.dtype == torch.uint8:
            t = t.view(torch.float8_e4m3fn)
        return t.detach().cpu().to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def latent_rows(inp: dict, b: int, positions) -> np.ndarray:
    """[n, 576] float64 latent rows of sequence b at logical `positions`.

    Every position must have a block-table entry (logical page below the
    table's row length); `visible_positions` only returns such positions."""
    kv = inp["kv_pages"]
    bt = inp["block_table"].numpy()
    pos = np.asarray(positions, dtype=np.int64)
    pages = bt[b, pos // PAGE].astype(np.int64)
    rows = pos % PAGE
    x = _f64(kv[pages, rows]) if pos.size else np.zeros((0, 576))
    if inp["kv_dtype"] == "fp8":
        x = x * inp["kv_scales"].numpy().astype(np.float64)[pages, rows][:, None]
    return x


def visible_positions(inp: dict, b: int, s: int) -> np.ndarray:
    L = int(inp["cache_seqlens"][b])
    P = inp["kv_pages"].shape[0]
    bt = inp["block_table"].numpy()
    if inp.get("indices") is not None:
        ix = inp["indices"][b, s].numpy().astype(np.int64)
        pos = ix[(ix >= 0) & (ix < L)]
    else:
        last = L - inp["Sq"] + s if inp["causal"] else L - 1
        pos = np.arange(0, min(last, L - 1) + 1, dtype=np.int64)
    # a logical page at or past the table's row length has no entry, and a
    # page entry outside the pool names no page: either way not resident
    pos = pos[pos // PAGE < bt.shape[1]]
    if pos.size:
        pg = bt[b, pos // PAGE]
        pos = pos[(pg >= 0) & (pg < P)]
    return pos


def attend(q576: np.ndarray, x: np.ndarray, scale: float):
    """Softmax attention of query rows q576 [R, 576] over latent rows x [n, 576].

    Returns (out [R, 512], lse [R]); n == 0 gives zeros and -inf."""
    R = q576.shape[0]
    if x.shape[0] == 0:
        return np.zeros((R, DC)), np.full((R,), -np.inf)
    z = scale * (q576 @ x.T)                       # [R, n]
    m = z.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
    p = np.exp(z - lse[:, None])
    return p @ x[:, :DC], lse


def decode(inp: dict):
    """(out [B,Sq,H,512], lse [B,Sq,H]) for every row, vectorised per (b, s)."""
    B, Sq, H = inp["B"], inp["Sq"], inp["H"]
    qn = _f64(inp["q_nope"])
    qr = _f64(inp["q_rope"])
    out = np.zeros((B, Sq, H, DC))
    lse = np.zeros((B, Sq, H))
    for b in range(B):
        for s in range(Sq):
            x = latent_rows(inp, b, visible_positions(inp, b, s))
            q = np.concatenate([qn[b, s], qr[b, s]], axis=1)  # [H, 576]
            out[b, s], lse[b, s] = attend(q, x, inp["softmax_scale"])
    return out, lse


def lse_merge(parts):
    """Merge softmax partials [(out_i [R,512] normalised, lse_i [R])] into one."""
    lses = np.stack([p[1] for p in parts])          # [n, R]
    mx = lses.max(axis=0)
    safe = np.where(np.isfinite(mx), mx, 0.0)
    w = np.exp(lses - safe)                          # exp(-inf) = 0
    tot = w.sum(axis=0)
    with np.errstate(divide="ignore"):
        lse = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    out = sum(w[i][:, None] * parts[i][0] for i in range(len(parts)))
    out = np.where(tot[:, None] > 0, out / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    return out, lse


def mha_nonabsorbed(q_c, q_rope, W_UK, W_UV, c, k_rope, scale):
    """Standard MHA over decompressed per-head K/V (MHA mode).

    q_c [H, dh], q_rope [H, 64], W_UK / W_UV [H, dh, 512], c [n, 512],
    k_rope [n, 64].  k_h = W_UK[h] c_j, v_h = W_UV[h] c_j; each head's key is
    [k_h | k_rope] and its query [q_c | q_rope].  Returns (out [H, dh], lse [H]).
    """
    H, dh = q_c.shape
    outs = np.zeros((H, dh))
    lses = np.zeros(H)
    for h in range(H):
        K = c @ W_UK[h].T                            # [n, dh]
        V = c @ W_UV[h].T                            # [n, dh]
        z = scale * (K @ q_c[h] + k_rope @ q_rope[h])
        m = z.max()
        lses[h] = m + np.log(np.exp(z - m).sum())
        outs[h] = np.exp(z - lses[h]) @ V
    return outs, lses
