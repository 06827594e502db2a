"""GPU parity of the DSA block top-k selection (mla_dsa_select, through the
C ABI) against the CPU oracle in oracle/dsa_select.py.

Selection is integer work: the token lists must equal the oracle's exactly.
Both sides compare the same fp32 scores (NaN as -inf) and break ties by the
lower block index, so there is one correct answer.
"""
import numpy as np
import pytest
import torch

import mla_synth as S
import oracle
from oracle import dsa_select as D

pytestmark = pytest.mark.gpu


def mla():
    import mla_latent_kv_12_amd as m
    return m


def _both(scores, L, Sq, n_select=16, n_init=1, n_local=2):
    print(f"select B={scores.shape[0]} Sq={Sq} nbk={scores.shape[2]} n={n_select}/{n_init}/{n_local}",
          flush=True)
    got = mla().dsa_select(torch.from_numpy(scores).cuda(), torch.from_numpy(L).cuda(),
                           n_select=n_select, n_init=n_init, n_local=n_local)
    torch.cuda.synchronize()
    want = D.select(scores, L, Sq, n_select, n_init, n_local)
    return got.cpu().numpy(), want


def _eq(got, want):
    bad = np.argwhere((got != want).any(axis=2))
    assert bad.size == 0, f"rows differ at (b, s) {bad[:5].tolist()}"


def test_dsa_workload_shape():
    rng = np.random.default_rng(1)
    B, nbk = 32, 1024
    sc = rng.standard_normal((B, 1, nbk)).astype(np.float32)
    L = np.full(B, 65536, dtype=np.int32)
    _eq(*_both(sc, L, 1))


def test_ties_nan_and_ragged_causal_lengths():
    rng = np.random.default_rng(2)
    B, Sq, nbk = 9, 2, 300
    sc = rng.integers(0, 3, (B, Sq, nbk)).astype(np.float32)      # heavy ties
    sc[rng.random(sc.shape) < 0.05] = np.nan
    L = np.array([0, 1, 63, 64, 65, 17 * 64, 17 * 64 + 1, 299 * 64 + 5, 400 * 64], dtype=np.int32)
    _eq(*_both(sc, L, Sq))



def test_signed_zeros_tie_at_the_threshold():
    # block 3 holds -0.0 and block 5 +0.0, the rest of the middle -1: the two
    # zeros are one score, so the tie goes to the lower block
    base = np.full(10, -1.0, dtype=np.float32)
    rows = []
    for z3, z5 in ((-0.0, 0.0), (0.0, -0.0), (0.0, 0.0), (-0.0, -0.0)):
        r = base.copy()
        r[3], r[5] = z3, z5
        rows.append(r)
    sc = np.stack(rows)[:, None, :]
    L = np.full(4, 10 * 64, dtype=np.int32)
    got, want = _both(sc, L, 1, n_select=4, n_init=1, n_local=2)
    _eq(got, want)
    for b in range(4):
        assert sorted(set((got[b, 0][got[b, 0] >= 0] // 64).tolist())) == [0, 3, 8, 9]
    # mixed signed zeros among heavy ties over a wider row
    rng = np.random.default_rng(8)
    sc = rng.integers(-1, 2, (6, 2, 200)).astype(np.float32)
    sc[sc == 0] = np.where(rng.random(int((sc == 0).sum())) < 0.5, -0.0, 0.0)
    L = rng.integers(1, 200 * 64 + 1, 6).astype(np.int32)
    _eq(*_both(sc, L, 2))

@pytest.mark.parametrize("n_select,n_init,n_local", [(16, 0, 0), (16, 8, 8), (1, 0, 1), (40, 3, 5),
                                                     (256, 1, 2)])
def test_selection_shapes(n_select, n_init, n_local):
    rng = np.random.default_rng(3 + n_select)
    B, Sq, nbk = 5, 1, 700
    sc = rng.standard_normal((B, Sq, nbk)).astype(np.float32)
    L = rng.integers(1, 700 * 64 + 1, B).astype(np.int32)
    _eq(*_both(sc, L, Sq, n_select, n_init, n_local))


def test_largest_score_rows():
    rng = np.random.default_rng(4)
    B, nbk = 2, 16384
    sc = rng.standard_normal((B, 1, nbk)).astype(np.float32)
    L = np.array([nbk * 64, nbk * 64 - 100], dtype=np.int32)
    _eq(*_both(sc, L, 1))


def test_score_row_shorter_than_the_sequence():
    rng = np.random.default_rng(5)
    sc = rng.standard_normal((3, 1, 50)).astype(np.float32)
    L = np.array([100 * 64, 50 * 64, 20 * 64], dtype=np.int32)
    _eq(*_both(sc, L, 1))


def test_select_then_sparse_decode_matches_oracle():
    from test_parity import check
    cfg = S.shrink("dsa_sparse")
    inp = S.make_inputs(cfg)
    B = inp["B"]
    nbk = int(inp["block_table"].shape[1])
    sc = np.random.default_rng(6).standard_normal((B, 1, nbk)).astype(np.float32)
    n_sel = inp["topk"] // 64
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    idx = mla().dsa_select(torch.from_numpy(sc).cuda(), g["cache_seqlens"], n_select=n_sel)
    out, lse = mla().sparse_decode(g["q_nope"], g["q_rope"], g["kv_pages"], g["block_table"],
                                   g["cache_seqlens"], idx, g["softmax_scale"])
    torch.cuda.synchronize()
    want_idx = D.select(sc, inp["cache_seqlens"].numpy(), 1, n_sel, 1, 2)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    ref_out, ref_lse = oracle.decode(inp, indices=torch.from_numpy(want_idx))
    check(out, lse, ref_out, ref_lse, what="select+sparse decode")
