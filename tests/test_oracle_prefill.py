"""Pins of the prefill oracle (CPU only).

The non-absorbed prefill ("MLA & DSA 推理性能优化指南" §3.1: decompress c into
per-head K and V, then standard MHA) must agree with the absorbed decode on
the same cache: for query position t, attention over K = [W_UK c | k_rope],
V = W_UV c of tokens 0..t equals W_UV applied to the absorbed decode's latent
output at L = t + 1, with the same lse ("MLA 在极长上下文下的显存带宽突围",
matrix absorption).  The decode side here is the C oracle, an independent
implementation, fed a bf16-exact absorbed query.  Also closed forms.
"""
import numpy as np
import torch

import oracle
from oracle import prefill as PF


def test_prefill_rows_equal_absorbed_decode():
    rng = np.random.default_rng(21)
    T, H, dh = 70, 4, 128
    scale = 1 / np.sqrt(192)
    # latent rows and rope keys exactly representable in bf16
    c = torch.randn(T, 512, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).double().numpy()
    kr = torch.randn(T, 64, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).double().numpy()
    W_UK = rng.integers(-2, 3, (H, dh, 512)) / 64.0     # small integers / 64: exact products
    W_UV = rng.standard_normal((H, dh, 512)) / np.sqrt(512)
    q_c = rng.integers(-2, 3, (T, H, dh)) / 4.0
    q_r = torch.randn(T, H, 64, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).double().numpy()
    K = np.concatenate([np.einsum("hkd,td->thk", W_UK, c), np.repeat(kr[:, None, :], H, axis=1)], axis=2)
    V = np.einsum("hkd,td->thk", W_UV, c)
    Q = np.concatenate([q_c, q_r], axis=2)
    out, lse = PF.prefill(Q[None], K[None], V[None], scale, causal=True)
    q_nope = np.einsum("thk,hkd->thd", q_c, W_UK)        # multiples of 1/256 below 2^8: exact in bf16
    for t in (0, 1, 31, 63, 64, 69):
        inp = dict(q_nope=torch.from_numpy(q_nope[t][None, None]).to(torch.bfloat16),
                   q_rope=torch.from_numpy(q_r[t][None, None]).to(torch.bfloat16),
                   kv_scales=None, kv_dtype="bf16", causal=False, indices=None, topk=0,
                   softmax_scale=scale, B=1, Sq=1, H=H)
        rows = np.concatenate([c, kr], axis=1)
        P = (T + 63) // 64
        pages = np.zeros((P * 64, 576))
        pages[:T] = rows
        inp["kv_pages"] = torch.from_numpy(pages.reshape(P, 64, 576)).to(torch.bfloat16)
        inp["block_table"] = torch.arange(P, dtype=torch.int32)[None]
        inp["cache_seqlens"] = torch.tensor([t + 1], dtype=torch.int32)
        assert np.array_equal(inp["q_nope"].double().numpy()[0, 0], q_nope[t])
        lat, dl = oracle.decode(inp)
        o = np.einsum("hkd,hd->hk", W_UV, lat[0, 0])
        assert np.max(np.abs(o - out[0, t])) < 1e-9
        assert np.max(np.abs(dl[0, 0] - lse[0, t])) < 1e-9


def test_closed_forms():
    rng = np.random.default_rng(4)
    T, H = 9, 2
    v = rng.standard_normal((1, T, H, 128))
    k = rng.standard_normal((1, T, H, 192))
    out, lse = PF.prefill(np.zeros((1, T, H, 192)), k, v, 0.1, causal=True)
    for t in range(T):                                   # zero query: running mean, lse = ln(t+1)
        assert np.allclose(out[0, t], v[0, : t + 1].mean(axis=0), atol=1e-12)
        assert np.allclose(lse[0, t], np.log(t + 1), atol=1e-12)
    q = rng.standard_normal((1, T, H, 192))
    o1, _ = PF.prefill(q, k, v, 0.1, causal=True)
    assert np.allclose(o1[0, 0], v[0, 0], atol=1e-12)   # the first row sees one token
    o2, l2 = PF.prefill(q, k, v, 0.1, causal=False)
    assert np.allclose(o2[0, T - 1], o1[0, T - 1], atol=1e-12)   # the last row sees all tokens either way
