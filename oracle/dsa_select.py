"""CPU oracle of the DSA block top-k selection (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never does, and nothing here imports it.

What it computes ("MLA & DSA 推理性能优化指南" §1.2 figure: the Lightning
Indexer scores the sequence, a top-k selection keeps k << L tokens,
block-aligned; §6.1 table: selected blocks of 64 tokens, 16 per query, one
initial block and two local blocks always take part):

  * query s of sequence b sees L_s = L_b - Sq + s + 1 tokens (L_b counts the
    Sq new tokens), i.e. nb = ceil(L_s / 64) blocks, limited to the blocks
    the score row covers;
  * if nb <= n_select every block is selected;
  * otherwise the blocks [0, n_init) and [nb - n_local, nb) are always
    selected, and of the blocks between them the n_select - n_init - n_local
    with the highest score (ties: lower block index first; NaN counts as
    -inf);
  * the output row holds, for the selected blocks in ascending order, their
    64 token positions (positions >= L_s as -1), then -1 up to n_select * 64.

The indexer itself (its scoring of blocks) is not part of this: the block
scores are an input.
"""
from __future__ import annotations

import numpy as np

PAGE = 64


def select_blocks(scores_row, nb: int, n_select: int, n_init: int, n_local: int) -> list[int]:
    """Selected block ids (ascending) for one query with nb visible blocks."""
    if nb <= n_select:
        return list(range(nb))
    fixed = set(range(min(n_init, nb))) | set(range(max(nb - n_local, 0), nb))
    middle = [k for k in range(nb) if k not in fixed]
    sc = np.asarray(scores_row, dtype=np.float32)[middle].astype(np.float64)
    sc = np.where(np.isnan(sc), -np.inf, sc)
    # highest score first, then lower block id (a stable sort keeps id order)
    order = np.argsort(-sc, kind="stable")
    take = n_select - len(fixed)
    chosen = [middle[i] for i in order[:take]]
    return sorted(fixed | set(chosen))


def select(block_scores, cache_seqlens, Sq: int, n_select: int, n_init: int, n_local: int):
    """indices int32 [B, Sq, n_select * 64] from block_scores [B, Sq, nbk]."""
    scores = np.asarray(block_scores, dtype=np.float32)
    B, Sq_, nbk = scores.shape
    assert Sq_ == Sq
    out = np.full((B, Sq, n_select * PAGE), -1, dtype=np.int32)
    for b in range(B):
        for s in range(Sq):
            Ls = max(int(cache_seqlens[b]) - Sq + s + 1, 0)
            nb = min((Ls + PAGE - 1) // PAGE, nbk)
            blocks = select_blocks(scores[b, s], nb, n_select, n_init, n_local)
            for i, k in enumerate(blocks):
                tok = k * PAGE + np.arange(PAGE)
                out[b, s, i * PAGE:(i + 1) * PAGE] = np.where(tok < Ls, tok, -1)
    return out
