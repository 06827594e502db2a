"""Pins of the cache-append oracle (CPU only).

The append ("MLA & DSA 推理性能优化指南" §4, decode-flow figure) and its
fp8 form (one e4m3fn byte per value, §4.1 / §5.3, with a per-token scale)
are pinned to: the e4m3fn format itself (every code round-trips; ties go to
the even code), a library cast (torch's float8_e4m3fn conversion, round to
nearest even), the quantiser's error bound, and the decode oracle (what the
append writes is exactly what a decode of the new position reads).
"""
import numpy as np
import pytest
import torch

import mla_synth as S
import oracle
from oracle import cache_append as C
from oracle import ref_numpy as R


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def test_every_code_value_matches_library():
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([C.e4m3fn_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(lib), np.isnan(mine))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], mine[ok])
    assert np.array_equal(np.signbit(lib[ok]), np.signbit(mine[ok]))


def test_every_finite_code_round_trips():
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = np.array([C.e4m3fn_value(c) for c in codes], dtype=np.float32)
    assert C.e4m3fn_encode(vals).tolist() == codes


def test_midpoints_go_to_the_even_code_and_neighbours_round_outward():
    pos = np.array([C.e4m3fn_value(c) for c in range(0x7F)])
    for c in range(0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)
        assert float(mid) == (pos[c] + pos[c + 1]) / 2          # exact in fp32
        want = c if c % 2 == 0 else c + 1
        assert int(C.e4m3fn_encode(mid)) == want
        assert int(C.e4m3fn_encode(-mid)) == want | 0x80
        up = np.nextafter(mid, np.float32(1e9), dtype=np.float32)
        dn = np.nextafter(mid, np.float32(-1e9), dtype=np.float32)
        assert int(C.e4m3fn_encode(up)) == c + 1
        assert int(C.e4m3fn_encode(dn)) == c


def test_encoder_matches_library_cast():
    rng = np.random.default_rng(7)
    v = np.concatenate([rng.uniform(-448, 448, 50000), rng.normal(0, 0.01, 20000),
                        rng.normal(0, 1e-4, 5000)]).astype(np.float32)
    allbf = C.bf16_bits_to_f32(np.arange(65536, dtype=np.uint16))
    allbf = allbf[np.isfinite(allbf) & (np.abs(allbf) <= 448)]
    v = np.concatenate([v, allbf])
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(C.e4m3fn_encode(v), lib)


def test_quantiser_error_bound_and_extremes():
    rng = np.random.default_rng(3)
    for scale_in in (1.0, 1e-3, 37.0):
        x = (rng.standard_normal(576) * scale_in).astype(np.float32)
        codes, sc = C.quantize_row(x)
        assert sc == np.float32(np.abs(x).max() / np.float32(448))
        dq = np.array([C.e4m3fn_value(int(c)) for c in codes]) * float(sc)
        q = np.abs(x.astype(np.float64) / float(sc))
        # half the code spacing at |q|: 2^(e-4) for normals, 2^-10 below 2^-6
        e = np.floor(np.log2(np.maximum(q, 2.0 ** -6)))
        half = np.where(q >= 2.0 ** -6, 2.0 ** (e - 4), 2.0 ** -10)
        assert np.all(np.abs(dq - x) <= float(sc) * half * (1 + 1e-6) + float(sc) * 1e-7 * q)
        i = int(np.argmax(np.abs(x)))
        assert codes[i] & 0x7F == 0x7E                         # the row's maximum codes to 448
    codes, sc = C.quantize_row(np.zeros(576, dtype=np.float32))
    assert sc == 1.0 and not codes.any()


def _case(kv, seed=11, Sq=1, B=3):
    cfg = S.config("dsv3_decode", B=B, Sq=Sq, lens=("uniform", 1, 300), kv=kv)
    inp = S.make_inputs(cfg, seed=seed, poison=False)
    g = torch.Generator().manual_seed(seed + 1)
    new = S._randn_bf16((B, Sq, 576), g)
    return inp, new


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_appended_row_is_what_decode_reads_at_the_new_position(kv):
    inp, new = _case(kv)
    fp8 = kv == "fp8"
    kvp = inp["kv_pages"].numpy() if fp8 else _bits(inp["kv_pages"])
    sc = inp["kv_scales"].numpy() if fp8 else None
    kv2, sc2 = C.kv_append(kvp, sc, _bits(new), inp["block_table"].numpy(),
                           inp["cache_seqlens"].numpy(), fp8)
    out = dict(inp)
    out["kv_pages"] = torch.from_numpy(kv2) if fp8 else torch.from_numpy(kv2.view(np.int16)).view(torch.bfloat16)
    if fp8:
        out["kv_scales"] = torch.from_numpy(sc2)
    for b in range(inp["B"]):
        L = int(inp["cache_seqlens"][b])
        got = R.latent_rows(out, b, [L - 1])[0]                  # read back through the pages
        x = C.bf16_bits_to_f32(_bits(new)[b, 0]).astype(np.float64)
        if fp8:
            codes, s = C.quantize_row(x.astype(np.float32))
            want = np.array([C.e4m3fn_value(int(c)) for c in codes]) * float(s)
            assert np.array_equal(got, want)
            # at most half the largest code step (32 at 448), plus fp32 rounding of x / scale
            assert np.max(np.abs(got - x)) <= float(s) * 16 * (1 + 1e-6)
        else:
            assert np.array_equal(got, x)
    # the C decode oracle reads the appended cache as the NumPy one does
    full_out, _ = oracle.decode(out)
    ref_out, _ = R.decode(out)
    assert np.max(np.abs(full_out - ref_out)) < 1e-9


def test_append_skips_invalid_slots_and_touches_nothing_else():
    inp, new = _case("bf16", Sq=2, B=4)
    kvp = _bits(inp["kv_pages"])
    bt = inp["block_table"].numpy().copy()
    L = inp["cache_seqlens"].numpy().copy()
    L[0] = 1                 # j = -1 for s = 0: skipped, s = 1 lands at 0
    bt[1, (int(L[1]) - 1) // 64] = -1          # invalid page entry
    bt[2, (int(L[2]) - 1) // 64] = kvp.shape[0]  # page past the pool
    kv2, _ = C.kv_append(kvp, None, _bits(new), bt, L, False)
    changed = np.argwhere((kv2 != kvp).any(axis=2))
    slots = set(map(tuple, changed.tolist()))
    want = {(int(bt[0, 0]), 0)}
    for b in (1, 2, 3):
        for s in range(2):
            j = int(L[b]) - 2 + s
            p = int(bt[b, j // 64])
            if 0 <= p < kvp.shape[0]:
                want.add((p, j % 64))
    assert slots == want
