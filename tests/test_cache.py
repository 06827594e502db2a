"""GPU parity of the cache append (mla_kv_append, through the C ABI) against
the CPU oracle in oracle/cache_append.py.

The append writes bytes, so the bar is bit-exact: every byte of the cache
and every fp8 scale after the GPU append equals the oracle's.  Both sides
compute the fp8 scale and the quotient x / scale in fp32 with correctly
rounded division, and round to e4m3fn to nearest even, so the codes are
decided in the same precision.
"""
import numpy as np
import pytest
import torch

import mla_synth as S
import oracle
from oracle import cache_append as C

pytestmark = pytest.mark.gpu


def mla():
    import mla_latent_kv_12_amd as m
    return m


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _new_rows(B, Sq, seed):
    return S._randn_bf16((B, Sq, 576), torch.Generator().manual_seed(seed))


def _append_both(inp, new, bt=None, L=None):
    """(GPU cache after the append, oracle cache after the append) as numpy."""
    fp8 = inp["kv_dtype"] == "fp8"
    bt = inp["block_table"] if bt is None else bt
    L = inp["cache_seqlens"] if L is None else L
    kv_g = inp["kv_pages"].cuda()
    sc_g = inp["kv_scales"].cuda() if fp8 else None
    print(f"append B={new.shape[0]} Sq={new.shape[1]} fp8={fp8} pages={kv_g.shape[0]}", flush=True)
    mla().kv_append(new.cuda(), kv_g, bt.cuda(), L.cuda(), kv_scales=sc_g)
    torch.cuda.synchronize()
    kv_o = inp["kv_pages"].numpy() if fp8 else _bits(inp["kv_pages"])
    sc_o = inp["kv_scales"].numpy() if fp8 else None
    want_kv, want_sc = C.kv_append(kv_o, sc_o, _bits(new), bt.numpy(), L.numpy(), fp8)
    got_kv = kv_g.cpu().numpy() if fp8 else _bits(kv_g)
    got_sc = sc_g.cpu().numpy() if fp8 else None
    return got_kv, got_sc, want_kv, want_sc


def _assert_same(got_kv, got_sc, want_kv, want_sc):
    bad = np.argwhere((got_kv != want_kv).any(axis=2))
    assert bad.size == 0, f"cache rows differ at (page, row) {bad[:5].tolist()}"
    if want_sc is not None:
        same = (got_sc.view(np.uint32) == want_sc.view(np.uint32))
        assert same.all(), f"scales differ at {np.argwhere(~same)[:5].tolist()}"


@pytest.mark.parametrize("name,kv,Sq", [("dsv3_decode", "bf16", 1), ("dsv3_decode", "fp8", 1),
                                        ("fp8_head_slice", "fp8", 2), ("long_context", "bf16", 3)])
def test_append_matches_oracle_bitwise_shrunk(name, kv, Sq):
    inp = S.make_inputs(S.shrink(name, kv=kv, Sq=Sq), poison=False)
    new = _new_rows(inp["B"], Sq, 21)
    _assert_same(*_append_both(inp, new))


@pytest.mark.parametrize("name", ["dsv3_decode", "fp8_head_slice"])
def test_append_matches_oracle_bitwise_full_size(name):
    cfg = S.config(name)
    inp = S.make_inputs(cfg, poison=False)
    new = _new_rows(inp["B"], inp["Sq"], 22)
    _assert_same(*_append_both(inp, new))


def test_fp8_rounding_of_every_bf16_value():
    """Rows whose maximum is 448 have scale 1, so every other value is
    rounded to e4m3fn as it is: all finite bf16 values in [-448, 448]."""
    vals = C.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16))
    keep = np.isfinite(vals) & (np.abs(vals) <= 448)
    bits = np.arange(65536, dtype=np.uint16)[keep]
    per = 575
    B = (bits.size + per - 1) // per
    rows = np.zeros((B, 1, 576), dtype=np.uint16)
    rows[:, 0, 0] = 0x43E0                                   # bf16 448.0
    flat = np.zeros(B * per, dtype=np.uint16)
    flat[: bits.size] = bits
    rows[:, 0, 1:] = flat.reshape(B, per)
    new = torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16)
    inp = dict(kv_pages=torch.zeros((B, 64, 576), dtype=torch.uint8),
               kv_scales=torch.zeros((B, 64), dtype=torch.float32), kv_dtype="fp8",
               block_table=torch.arange(B, dtype=torch.int32).view(B, 1),
               cache_seqlens=torch.ones(B, dtype=torch.int32))
    got_kv, got_sc, want_kv, want_sc = _append_both(inp, new)
    assert np.all(want_sc[:, 0] == 1.0)
    _assert_same(got_kv, got_sc, want_kv, want_sc)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_edges(kv):
    """All-zero row (scale 1, codes 0); L < Sq (no slot for the early rows);
    invalid and out-of-pool page entries and positions past the table (rows
    skipped, cache untouched)."""
    inp = S.make_inputs(S.shrink("dsv3_decode", B=5, kv=kv), poison=False)
    Sq = 2
    new = _new_rows(5, Sq, 23)
    new[0, 1] = 0
    L = inp["cache_seqlens"].clone()
    bt = inp["block_table"].clone()
    L[1] = 1                                   # j = -1 and 0
    bt[2, (int(L[2]) - 1) // 64] = -1
    bt[3, (int(L[3]) - 1) // 64] = inp["kv_pages"].shape[0]
    L[4] = 64 * bt.shape[1] + 2                 # both new positions past the table
    got = _append_both(inp, new, bt=bt, L=L)
    _assert_same(*got)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_then_decode_matches_oracle(kv):
    from test_parity import check
    inp = S.make_inputs(S.shrink("dsv3_decode", kv=kv), poison=False)
    new = _new_rows(inp["B"], 1, 24)
    fp8 = kv == "fp8"
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    m = mla()
    m.kv_append(new.cuda(), g["kv_pages"], g["block_table"], g["cache_seqlens"],
                kv_scales=g["kv_scales"])
    out, lse = m.decode(g["q_nope"], g["q_rope"], g["kv_pages"], g["block_table"],
                        g["cache_seqlens"], g["softmax_scale"], kv_scales=g["kv_scales"])
    torch.cuda.synchronize()
    kv_o = inp["kv_pages"].numpy() if fp8 else _bits(inp["kv_pages"])
    kv2, sc2 = C.kv_append(kv_o, inp["kv_scales"].numpy() if fp8 else None, _bits(new),
                           inp["block_table"].numpy(), inp["cache_seqlens"].numpy(), fp8)
    ref = dict(inp)
    ref["kv_pages"] = torch.from_numpy(kv2) if fp8 else torch.from_numpy(kv2.view(np.int16)).view(torch.bfloat16)
    if fp8:
        ref["kv_scales"] = torch.from_numpy(sc2)
    ref_out, ref_lse = oracle.decode(ref)
    check(out, lse, ref_out, ref_lse, what=f"append+decode {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_rows_straddling_a_page_boundary(kv):
    """Four new tokens per sequence that end past a 64-token page edge (62..65, 126..129, 61..64)."""
    inp = S.make_inputs(S.shrink("dsv3_decode", B=3, kv=kv, lens=("fixed", 200)), poison=False)
    L = torch.tensor([66, 128 + 2, 64 + 1], dtype=torch.int32)
    new = _new_rows(3, 4, 25)
    _assert_same(*_append_both(inp, new, L=L))
