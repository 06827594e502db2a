"""Pins of the DSA block-selection oracle (CPU only).

The selection ("MLA & DSA 推理性能优化指南" §1.2 figure, §6.1 table) is pinned
to: brute force (the selected middle blocks carry the largest possible total
score of any valid choice), invariance under order-preserving score changes,
the shape of the workload generator's DSA lists (independent code that draws
the blocks directly), and the sparse decode (selecting every block equals
dense attention).
"""
import itertools

import numpy as np
import pytest
import torch

import mla_synth as S
import oracle
from oracle import dsa_select as D


def test_brute_force_best_total_score():
    rng = np.random.default_rng(5)
    for trial in range(40):
        nb = int(rng.integers(6, 12))
        n_sel, n_init, n_local = 6, 1, 2
        sc = rng.standard_normal(nb).astype(np.float32)
        got = D.select_blocks(sc, nb, n_sel, n_init, n_local)
        fixed = {0, nb - 2, nb - 1}
        assert fixed <= set(got) and len(got) == n_sel and got == sorted(got)
        middle = [k for k in range(1, nb - 2)]
        best = max(sum(float(sc[k]) for k in c) for c in itertools.combinations(middle, n_sel - 3))
        assert abs(sum(float(sc[k]) for k in set(got) - fixed) - best) < 1e-9


def test_ties_take_the_lower_block_and_nan_is_lowest():
    sc = np.array([9, 1, 1, 1, 1, np.nan, 1, 0, 5, 5], dtype=np.float32)
    # fixed: 0, 8, 9; three more from 1..7: all 1.0 ties -> 1, 2, 3
    assert D.select_blocks(sc, 10, 6, 1, 2) == [0, 1, 2, 3, 8, 9]
    sc2 = np.full(10, np.nan, dtype=np.float32)
    assert D.select_blocks(sc2, 10, 6, 1, 2) == [0, 1, 2, 3, 8, 9]


def test_signed_zeros_are_one_score():
    # -0.0 and +0.0 are the same real number: at the selection threshold
    # they tie, and the tie goes to the lower block whatever the signs.
    base = np.full(10, -1.0, dtype=np.float32)
    for z3, z5 in ((-0.0, 0.0), (0.0, -0.0), (0.0, 0.0), (-0.0, -0.0)):
        sc = base.copy()
        sc[3], sc[5] = z3, z5
        assert D.select_blocks(sc, 10, 4, 1, 2) == [0, 3, 8, 9], (z3, z5)
    # two of them taken, the rest of the middle lower: both zeros selected
    sc = base.copy()
    sc[3], sc[5] = -0.0, 0.0
    assert D.select_blocks(sc, 10, 5, 1, 2) == [0, 3, 5, 8, 9]

def test_order_preserving_changes_keep_the_selection():
    rng = np.random.default_rng(9)
    sc = rng.standard_normal((2, 1, 200)).astype(np.float32)
    L = np.array([200 * 64, 150 * 64 - 17], dtype=np.int32)
    base = D.select(sc, L, 1, 16, 1, 2)
    for f in (lambda x: x + 3.0, lambda x: 2.0 * x, lambda x: np.exp(x)):
        assert np.array_equal(D.select(f(sc).astype(np.float32), L, 1, 16, 1, 2), base)


def test_reproduces_the_workload_generators_lists():
    cfg = S.shrink("dsa_sparse", B=3, lens=("fixed", 64 * 40), topk=8 * 64, sel_blocks=8)
    inp = S.make_inputs(cfg, poison=False)
    ix = inp["indices"].numpy()
    B = ix.shape[0]
    nb = 40
    sc = np.zeros((B, 1, nb), dtype=np.float32)
    for b in range(B):
        blocks = np.unique(ix[b, 0][ix[b, 0] >= 0] // 64)
        sc[b, 0, blocks] = 1.0                                # the generator's picks score high
    got = D.select(sc, inp["cache_seqlens"].numpy(), 1, 8, 1, 2)
    assert np.array_equal(got, ix)


def test_causal_lengths_and_short_sequences():
    sc = np.zeros((1, 2, 10), dtype=np.float32)
    L = np.array([130], dtype=np.int32)                       # query 0 sees 129, query 1 sees 130
    out = D.select(sc, L, 2, 16, 1, 2)
    for s, Ls in ((0, 129), (1, 130)):
        row = out[0, s]
        vis = row[row >= 0]
        assert vis.tolist() == list(range(Ls))
        assert np.all(row[Ls:] == -1)
    assert np.all(D.select(sc, np.array([0], dtype=np.int32), 2, 16, 1, 2) == -1)


def test_selecting_every_block_equals_dense_decode():
    cfg = S.shrink("dsv3_decode", B=2, lens=("fixed", 64 * 5 + 9))
    inp = S.make_inputs(cfg, poison=False)
    sc = np.random.default_rng(1).standard_normal((2, 1, 6)).astype(np.float32)
    ix = D.select(sc, inp["cache_seqlens"].numpy(), 1, 8, 1, 2)
    dense_out, dense_lse = oracle.decode(inp, indices=False)
    sp_out, sp_lse = oracle.decode(inp, indices=torch.from_numpy(ix))
    assert np.max(np.abs(dense_out - sp_out)) < 1e-12 and np.max(np.abs(dense_lse - sp_lse)) < 1e-12
