"""Pins of the projection oracle (CPU only).

The absorbed path (absorb the query with W_UK, attend over the latent,
project the latent output with W_UV) must equal standard multi-head
attention over keys and values decompressed from the latent with the same
W_UK / W_UV ("MLA 在极长上下文下的显存带宽突围", section on absorbing the
matrices at run time; "MLA & DSA 推理性能优化指南" §1.1 figure, the two
paths).  The MHA side (`ref_numpy.mha_nonabsorbed`) builds K and V per head
and never forms the absorbed query, so a transposed weight, a wrong head or a
wrong contraction index in either projection fails this.
"""
import numpy as np

from oracle import projections as P
from oracle import ref_numpy as R


def test_absorbed_path_equals_nonabsorbed_mha():
    rng = np.random.default_rng(12)
    H, dh, n, M = 6, 128, 37, 3
    W_UK = rng.standard_normal((H, dh, 512)) / np.sqrt(512)
    W_UV = rng.standard_normal((H, dh, 512)) / np.sqrt(512)
    c = rng.standard_normal((n, 512))
    k_rope = rng.standard_normal((n, 64))
    x = np.concatenate([c, k_rope], axis=1)
    scale = 1 / np.sqrt(192)
    q_c = rng.standard_normal((M, H, dh))
    q_rope = rng.standard_normal((M, H, 64))
    q_nope = P.absorb_query(q_c, np.transpose(W_UK, (0, 2, 1)))      # stored form [H, 512, 128]
    for m in range(M):
        out_lat, lse = R.attend(np.concatenate([q_nope[m], q_rope[m]], axis=1), x, scale)
        o = P.project_out(out_lat[None], W_UV)[0]
        ref_o, ref_lse = R.mha_nonabsorbed(q_c[m], q_rope[m], W_UK, W_UV, c, k_rope, scale)
        assert np.max(np.abs(o - ref_o)) < 1e-10
        assert np.max(np.abs(lse - ref_lse)) < 1e-10


def test_a_heads_weights_reach_only_that_head():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((2, 3, 128))
    w = rng.standard_normal((3, 512, 128))
    v = rng.standard_normal((3, 128, 512))
    x = rng.standard_normal((2, 3, 512))
    for h in range(3):
        w0, v0 = w.copy(), v.copy()
        w0[h] = 0
        v0[h] = 0
        a, b = P.absorb_query(q, w0), P.project_out(x, v0)
        assert not a[:, h].any() and not b[:, h].any()
        others = [k for k in range(3) if k != h]
        assert np.array_equal(a[:, others], P.absorb_query(q, w)[:, others])
        assert np.array_equal(b[:, others], P.project_out(x, v)[:, others])
