"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself:
numbers the pages print (tests/golden/kv_cache_constants.json), the
absorption identity against an un-absorbed MHA computed over decompressed
K/V, closed forms, invariances, a library fp8 decoder, and a second
independent (NumPy) implementation.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import mla_synth as S
import oracle
from oracle import ref_numpy as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_cache_constants.json")))


def g(name):
    return GOLD[name]["value"]


# ---------------------------------------------------------------- pages' numbers
def test_cache_bytes_match_pages():
    assert oracle.kv_bytes_per_token(2) == g("bf16_bytes_per_token_per_layer")
    assert oracle.kv_bytes_per_token(1) == g("fp8_bytes_per_token_per_layer")
    mha = g("n_heads") * g("d_head") * 2 * 2
    assert mha == g("mha_equivalent_bytes_per_token_per_layer")
    assert round(mha / oracle.kv_bytes_per_token(2)) == g("compression_ratio_fp16")
    assert round(mha / oracle.kv_bytes_per_token(1)) == g("compression_ratio_fp8")
    assert round(64 * oracle.kv_bytes_per_token(2) / 1000, 1) == g("layers_64_total_kb_per_token")
    assert S.D_C == g("d_c") and S.D_ROPE == g("d_rope") and S.PAGE == g("dsa_selected_block_tokens")


def test_sparse_read_reduction_matches_pages():
    # bytes read by sparse vs dense decode at L = 32K, k = 1024
    L, k = 32 * 1024, 1024
    red = 1 - k * oracle.kv_bytes_per_token(2) / (L * oracle.kv_bytes_per_token(2))
    assert abs(red - g("dsa_read_reduction_L32K_k1024")) < 0.005


def test_dsa_index_structure_matches_pages():
    cfg = S.config("dsa_sparse", B=3, lens=("fixed", 65536))
    inp = S.make_inputs(cfg, unselected="nan")
    ix = inp["indices"]
    nb = 65536 // 64
    for b in range(3):
        blocks = torch.unique(ix[b, 0] // 64)
        assert blocks.numel() == g("dsa_num_selected_blocks")
        assert int(blocks[0]) == 0  # initial block
        assert set(blocks[-g("dsa_local_blocks"):].tolist()) == {nb - 2, nb - 1}
        # whole blocks, ascending, distinct
        assert torch.all(ix[b, 0].view(16, 64) == blocks.view(16, 1) * 64 + torch.arange(64))


# ---------------------------------------------------------------- fp8 decoding
def test_e4m3fn_decoder_matches_library_for_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([oracle.e4m3fn_to_double(int(c)) for c in range(256)])
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(mine))
    assert np.array_equal(lib[~nan], mine[~nan])
    assert nan.sum() == 2  # 0x7f and 0xff


# ---------------------------------------------------------------- C vs NumPy
@pytest.mark.parametrize("name", list(S.CONFIGS))
def test_c_oracle_matches_numpy_oracle(name):
    inp = S.make_inputs(S.shrink(name), unselected="nan")
    out_c, lse_c = oracle.decode(inp)
    out_n, lse_n = R.decode(inp)
    assert np.all(np.isfinite(out_c))
    np.testing.assert_allclose(out_c, out_n, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_c, lse_n, rtol=1e-12, atol=1e-12)


def test_row_subset_matches_full():
    inp = S.make_inputs(S.shrink("dsv3_decode"))
    out, lse = oracle.decode(inp)
    rows = [0, 5, 200, inp["B"] * inp["H"] - 1]
    o2, l2 = oracle.decode(inp, rows=rows)
    flat_o = out.reshape(-1, 512)
    assert np.array_equal(o2, flat_o[rows]) and np.array_equal(l2, lse.reshape(-1)[rows])


# ---------------------------------------------------------------- absorption identity
def _absorption_case(weights: str, seed=11):
    """Cache from the tiny workload; random W_UK/W_UV; q^C drawn per head."""
    cfg = S.config("tiny")
    inp = S.make_inputs(cfg)
    H, dh = cfg["H"], 128
    rng = np.random.default_rng(seed)
    if weights == "gaussian":       # N(0, 1/512), as the workload specifies
        W_UK = rng.normal(0, 1 / math.sqrt(512), (H, dh, 512))
        W_UV = rng.normal(0, 1 / math.sqrt(512), (H, dh, 512))
        q_c = rng.normal(0, 1, (H, dh))
    else:                           # ternary / 16: q^C W_UK exact in bf16
        W_UK = rng.integers(-1, 2, (H, dh, 512)) / 16.0
        W_UV = rng.integers(-1, 2, (H, dh, 512)) / 16.0
        q_c = rng.integers(-1, 2, (H, dh)).astype(np.float64)
    q_nope = np.einsum("hk,hkd->hd", q_c, W_UK)      # absorbed query, fp64
    return inp, W_UK, W_UV, q_c, q_nope


def _mha_reference(inp, W_UK, W_UV, q_c):
    L = int(inp["cache_seqlens"][0])
    x = R.latent_rows(inp, 0, np.arange(L))
    q_rope = inp["q_rope"][0, 0].to(torch.float64).numpy()
    return R.mha_nonabsorbed(q_c, q_rope, W_UK, W_UV, x[:, :512], x[:, 512:], inp["softmax_scale"])


def test_absorption_identity_numpy_oracle_gaussian_weights():
    inp, W_UK, W_UV, q_c, q_nope = _absorption_case("gaussian")
    inp = dict(inp, q_nope=torch.from_numpy(q_nope).view(1, 1, *q_nope.shape))
    out_lat, lse = R.decode(inp)
    out_mha, lse_mha = _mha_reference(inp, W_UK, W_UV, q_c)
    out_abs = np.einsum("hkd,hd->hk", W_UV, out_lat[0, 0])
    np.testing.assert_allclose(lse[0, 0], lse_mha, rtol=1e-10)
    np.testing.assert_allclose(out_abs, out_mha, rtol=1e-10, atol=1e-12)


def test_absorption_identity_c_oracle_exact_weights():
    inp, W_UK, W_UV, q_c, q_nope = _absorption_case("ternary")
    qb = torch.from_numpy(q_nope).to(torch.bfloat16)
    assert np.array_equal(qb.to(torch.float64).numpy(), q_nope)  # exactly representable
    inp = dict(inp, q_nope=qb.view(1, 1, *q_nope.shape))
    out_lat, lse = oracle.decode(inp)
    out_mha, lse_mha = _mha_reference(inp, W_UK, W_UV, q_c)
    out_abs = np.einsum("hkd,hd->hk", W_UV, out_lat[0, 0])
    np.testing.assert_allclose(lse[0, 0], lse_mha, rtol=1e-10)
    np.testing.assert_allclose(out_abs, out_mha, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def _custom(B=1, Sq=1, H=4, lens=(70,), kv="bf16", seed=3, **kw):
    cfg = dict(B=B, Sq=Sq, H=H, lens=("list", lens), kv=kv, shuffle=True, causal=False, topk=0,
               name="custom")
    cfg.update(kw)
    return S.make_inputs(cfg, seed=seed)


def test_single_token_returns_its_latent():
    inp = _custom(lens=(1,), H=8)
    out, lse = oracle.decode(inp)
    x = R.latent_rows(inp, 0, [0])[0]
    q = np.concatenate([inp["q_nope"][0, 0].double().numpy(), inp["q_rope"][0, 0].double().numpy()], 1)
    assert np.array_equal(out[0, 0], np.broadcast_to(x[:512], (8, 512)))
    np.testing.assert_allclose(lse[0, 0], inp["softmax_scale"] * (q @ x), rtol=1e-13)


def test_zero_query_gives_uniform_average():
    inp = _custom(lens=(150,), H=4)
    inp["q_nope"].zero_()
    inp["q_rope"].zero_()
    out, lse = oracle.decode(inp)
    x = R.latent_rows(inp, 0, np.arange(150))
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(x[:, :512].mean(0), (4, 512)), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(150), rtol=1e-14)


def test_constant_score_shift_moves_only_lse():
    inp = _custom(lens=(130,), H=4)
    kv = inp["kv_pages"]
    kv[:, :, 512:] = 0
    out0, lse0 = oracle.decode(inp)
    r = torch.randn(64, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    kv[:, :, 512:] = r  # same rope key on every token: score shifts by q_rope . r
    out1, lse1 = oracle.decode(inp)
    shift = inp["softmax_scale"] * (inp["q_rope"][0, 0].double().numpy() @ r.double().numpy())
    np.testing.assert_allclose(out1, out0, atol=1e-13)
    np.testing.assert_allclose(lse1[0, 0] - lse0[0, 0], shift, atol=1e-12)


def test_softmax_weights_sum_to_one():
    inp = _custom(lens=(300, 77), B=2, H=8)
    inp["kv_pages"][:, :, 0] = 1.0  # one constant latent dim: out[0] = sum_j p_j
    out, _ = oracle.decode(inp)
    np.testing.assert_allclose(out[..., 0], 1.0, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- layout invariances
def _relayout(inp, perm):
    """Same logical cache stored under a different physical page order."""
    new = dict(inp)
    P = inp["kv_pages"].shape[0]
    perm = torch.as_tensor(perm)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(P)
    new["kv_pages"] = inp["kv_pages"][perm].clone()          # new page i = old page perm[i]
    if inp["kv_scales"] is not None:
        new["kv_scales"] = inp["kv_scales"][perm].clone()
    bt = inp["block_table"].clone()
    m = bt >= 0
    bt[m] = inv[bt[m].long()].to(torch.int32)
    new["block_table"] = bt
    return new


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_paged_equals_contiguous_and_permutation_invariant(kv):
    inp = _custom(B=3, lens=(200, 64, 129), kv=kv)
    P = inp["kv_pages"].shape[0]
    # contiguous: pages renumbered so each sequence's pages are in logical order
    order = torch.cat([inp["block_table"][b, : (int(L) + 63) // 64] for b, L in enumerate(inp["cache_seqlens"])])
    contig = _relayout(inp, order.long())
    nb = [(int(L) + 63) // 64 for L in inp["cache_seqlens"]]
    assert torch.equal(contig["block_table"][0, :nb[0]], torch.arange(nb[0], dtype=torch.int32))
    shuffled = _relayout(inp, torch.randperm(P, generator=torch.Generator().manual_seed(9)))
    a = oracle.decode(inp)
    for other in (contig, shuffled):
        b = oracle.decode(other)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("L", [1, 63, 64, 65, 127])
def test_poisoned_tails_never_influence(kv, L):
    cfg = dict(B=1, Sq=1, H=4, lens=("list", (L,)), kv=kv, shuffle=False, causal=False, topk=0)
    a = S.make_inputs(cfg, seed=5, poison=True)
    b = S.make_inputs(cfg, seed=5, poison=False)
    oa, la = oracle.decode(a)
    ob, lb = oracle.decode(b)
    assert np.all(np.isfinite(oa))
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_empty_sequence_gives_zero_and_minus_inf():
    inp = _custom(B=2, lens=(0, 5), H=4)
    out, lse = oracle.decode(inp)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(lse[1]))



# ---------------------------------------------------------------- the table's row length
def _narrow_table(inp, stride):
    """The same cache with each block-table row cut to `stride` entries."""
    return dict(inp, block_table=inp["block_table"][:, :stride].contiguous())


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_tokens_past_the_table_row_are_invisible_dense(kv):
    # Sequence 0 is longer than its 3-entry table row covers (192 tokens);
    # sequence 1's row follows it in memory and holds valid pages, so an
    # oracle that read past the row would pick up foreign tokens here.
    inp = _custom(B=3, lens=(300, 250, 260), H=4, kv=kv, seed=21)
    cut = _narrow_table(inp, 3)
    got = oracle.decode(cut)
    # the same as if every sequence were only as long as its table row
    short = dict(cut, cache_seqlens=torch.clamp(inp["cache_seqlens"], max=3 * 64))
    want = oracle.decode(short)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    # and not the same as the untruncated cache (the cut matters)
    full = oracle.decode(inp)
    assert not np.allclose(full[0], got[0])
    # the NumPy oracle reads the table the same way
    ref = R.decode(cut)
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1], ref[1], rtol=1e-12, atol=1e-12)


def test_tokens_past_the_table_row_are_invisible_causal():
    # Sq = 2, causal: both queries' visible sets are cut at the row's end
    cfg = dict(B=2, Sq=2, H=4, lens=("list", (200, 150)), kv="bf16", shuffle=True,
               causal=True, topk=0, name="custom")
    inp = S.make_inputs(cfg, seed=22)
    cut = _narrow_table(inp, 2)
    got = oracle.decode(cut)
    ref = R.decode(cut)
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1], ref[1], rtol=1e-12, atol=1e-12)
    # query 1 of each sequence now sees exactly tokens 0..127
    one = dict(cut, Sq=1, causal=False, q_nope=inp["q_nope"][:, 1:].contiguous(),
               q_rope=inp["q_rope"][:, 1:].contiguous(),
               cache_seqlens=torch.full((2,), 128, dtype=torch.int32))
    o1, l1 = oracle.decode(one)
    assert np.array_equal(got[0][:, 1], o1[:, 0]) and np.array_equal(got[1][:, 1], l1[:, 0])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_tokens_past_the_table_row_are_invisible_sparse(kv):
    inp = _custom(B=2, lens=(400, 300), H=4, kv=kv, seed=23)
    cut = _narrow_table(inp, 4)   # 256 tokens per sequence have a page
    topk = 96
    g_ = torch.Generator().manual_seed(24)
    ix = torch.full((2, 1, topk), -1, dtype=torch.int32)
    for b, L in enumerate((400, 300)):
        ix[b, 0] = torch.randperm(L, generator=g_)[:topk].to(torch.int32)
    assert (ix >= 256).any() and (ix < 256).any()
    got = oracle.decode(cut, indices=ix)
    # entries past the row behave exactly like the -1 padding
    want = oracle.decode(cut, indices=torch.where(ix >= 256, torch.full_like(ix, -1), ix))
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    ref = R.decode(dict(cut, indices=ix))
    np.testing.assert_allclose(got[0], ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[1], ref[1], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- sparse
def test_sparse_equals_dense_with_complement_masked():
    cfg = S.shrink("dsa_sparse")
    inp = S.make_inputs(cfg, unselected="nan")
    out_s, lse_s = oracle.decode(inp)
    # dense decode where every page holding no selected token is masked out
    masked = dict(inp, indices=None)
    bt = inp["block_table"].clone()
    for b in range(cfg["B"]):
        sel_pages = torch.unique(inp["indices"][b, 0] // 64).long()
        keep = torch.zeros(bt.shape[1], dtype=torch.bool)
        keep[sel_pages] = True
        bt[b, ~keep] = -1
    masked["block_table"] = bt
    out_d, lse_d = oracle.decode(masked, indices=False)
    np.testing.assert_allclose(out_s, out_d, atol=1e-13)
    np.testing.assert_allclose(lse_s, lse_d, atol=1e-13)


def test_sparse_all_tokens_equals_dense_and_order_free():
    inp = _custom(B=2, lens=(190, 64), H=4)
    L = inp["cache_seqlens"]
    topk = 192
    ix = torch.full((2, 1, topk), -1, dtype=torch.int32)
    g_ = torch.Generator().manual_seed(4)
    for b in range(2):
        ix[b, 0, : int(L[b])] = torch.randperm(int(L[b]), generator=g_).to(torch.int32)
    dense = oracle.decode(inp, indices=False)
    sparse = oracle.decode(inp, indices=ix)
    np.testing.assert_allclose(sparse[0], dense[0], atol=1e-13)
    np.testing.assert_allclose(sparse[1], dense[1], atol=1e-13)


def test_sparse_token_subset_matches_gathered_attention():
    inp = _custom(B=1, lens=(500,), H=4)
    pos = torch.tensor([3, 499, 17, 250, 251, 0, -1, 600, 500], dtype=torch.int32)
    ix = pos.view(1, 1, -1)
    out, lse = oracle.decode(inp, indices=ix)
    keep = [3, 499, 17, 250, 251, 0]
    x = R.latent_rows(inp, 0, keep)
    q = np.concatenate([inp["q_nope"][0, 0].double().numpy(), inp["q_rope"][0, 0].double().numpy()], 1)
    z = inp["softmax_scale"] * (q @ x.T)
    p = np.exp(z - z.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(out[0, 0], p @ x[:, :512], atol=1e-13)


# ---------------------------------------------------------------- causal, Sq > 1
def test_causal_rows_equal_single_query_decodes():
    cfg = dict(B=2, Sq=2, H=4, lens=("list", (130, 64)), kv="fp8", shuffle=True, causal=True, topk=0)
    inp = S.make_inputs(cfg, seed=8)
    out, lse = oracle.decode(inp)
    for s, delta in ((1, 0), (0, 1)):   # last query sees L tokens, first sees L-1
        one = dict(inp, Sq=1, causal=False, q_nope=inp["q_nope"][:, s:s + 1].contiguous(),
                   q_rope=inp["q_rope"][:, s:s + 1].contiguous(),
                   cache_seqlens=inp["cache_seqlens"] - delta)
        o1, l1 = oracle.decode(one)
        assert np.array_equal(out[:, s], o1[:, 0]) and np.array_equal(lse[:, s], l1[:, 0])


# ---------------------------------------------------------------- split-KV merge
def test_split_and_lse_merge_equals_unsplit():
    inp = _custom(B=1, lens=(700,), H=8)
    x = R.latent_rows(inp, 0, np.arange(700))
    q = np.concatenate([inp["q_nope"][0, 0].double().numpy(), inp["q_rope"][0, 0].double().numpy()], 1)
    whole = R.attend(q, x, inp["softmax_scale"])
    cuts = [0, 64, 65, 300, 699, 700]
    parts = [R.attend(q, x[a:b], inp["softmax_scale"]) for a, b in zip(cuts[:-1], cuts[1:])]
    parts.append(R.attend(q, x[:0], inp["softmax_scale"]))  # an empty split
    merged = R.lse_merge(parts)
    np.testing.assert_allclose(merged[0], whole[0], atol=1e-12)
    np.testing.assert_allclose(merged[1], whole[1], atol=1e-12)
    c_out, c_lse = oracle.decode(inp)
    np.testing.assert_allclose(c_out[0, 0], whole[0], atol=1e-12)
