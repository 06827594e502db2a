"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/mla.h declares, and rejects bad arguments before launching anything.

No call here gets past validation (pointers are fake), so nothing is ever
enqueued; num_wg > 0 keeps validation from querying a device.
"""
import ctypes
import os
import re

import pytest

import mla_latent_kv_12_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "mla.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, HIP = range(7)
FAKE = 1 << 20  # 256-aligned, never dereferenced


def declared():
    text = open(HDR).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(mla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert set(declared()) == set(mla.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = mla.lib()
    for name in declared():
        assert hasattr(L, name), name


def test_status_strings():
    L = mla.lib()
    for i, name in enumerate(mla.STATUS):
        assert L.mla_status_str(i).decode() == name


def test_workspace_size_rules():
    ws = mla.workspace_size
    assert ws(0, 1, 128, 0, 256) == 0 and ws(1, 0, 1, 0, 256) == 0 and ws(1, 1, 1, -1, 256) == 0
    assert ws(64, 1, 128, 0, -1) == 0
    a = ws(64, 1, 128, 0, 256)
    assert a > 0 and a % 256 == 0
    # partial buffers: (num_wg + units) * 128 rows * (512 fp16 values + fp32
    # lse and scale) at least
    assert a >= (256 + 64) * 128 * (512 * 2 + 8)
    assert ws(64, 1, 128, 0, 512) > a          # more workgroups, more splits
    assert ws(4, 2, 128, 0, 256) > ws(4, 1, 128, 0, 256)  # 256 rows -> 2 units per sequence
    assert ws(32, 1, 128, 1024, 256) > 0       # sparse


def _decode(**kw):
    L = mla.lib()
    args = dict(q_nope=FAKE, q_rope=FAKE, kv=FAKE, scales=None, dtype=0, num_pages=10, bt=FAKE,
                bt_stride=4, seqlens=FAKE, B=2, Sq=1, H=16, scale=0.1, causal=0, out=FAKE,
                lse=FAKE, ws=FAKE, ws_bytes=0, num_wg=8, planned=0)
    args.update(kw)
    return L.mla_decode(args["q_nope"], args["q_rope"], args["kv"], args["scales"], args["dtype"],
                        args["num_pages"], args["bt"], args["bt_stride"], args["seqlens"],
                        args["B"], args["Sq"], args["H"], args["scale"], args["causal"],
                        args["out"], args["lse"], args["ws"], args["ws_bytes"], args["num_wg"],
                        args["planned"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q_nope=None), NULL), (dict(kv=None), NULL), (dict(out=None), NULL),
    (dict(lse=None), NULL), (dict(bt=None), NULL), (dict(seqlens=None), NULL),
    (dict(dtype=1), NULL),                                   # fp8 without scales
    (dict(dtype=7), SHAPE), (dict(B=0), SHAPE), (dict(H=-1), SHAPE), (dict(Sq=0), SHAPE),
    (dict(num_pages=0), SHAPE), (dict(bt_stride=0), SHAPE),
    (dict(scale=float("nan")), SHAPE), (dict(scale=float("inf")), SHAPE),
    (dict(scale=0.0), SHAPE), (dict(scale=-0.1), SHAPE),
    (dict(num_wg=-3), SHAPE), (dict(num_wg=1 << 20), SHAPE),
    (dict(q_nope=FAKE + 8), ALIGN), (dict(kv=FAKE + 4), ALIGN), (dict(out=FAKE + 2), ALIGN),
    (dict(ws=None), WS), (dict(ws=FAKE + 16), ALIGN),
    (dict(ws_bytes=100), WS),                                # too small
])
def test_decode_rejects_before_launch(kw, code):
    assert _decode(**kw) == code
    assert mla.lib().mla_last_error().decode() != ""


def test_workspace_boundary_is_exact():
    need = mla.workspace_size(2, 1, 16, 0, 8)
    assert _decode(ws_bytes=need - 1) == WS


def test_sparse_rejects_bad_topk_and_missing_indices():
    L = mla.lib()
    f = lambda ind, topk: L.mla_sparse_decode(FAKE, FAKE, FAKE, None, 0, 10, FAKE, 4, FAKE, ind,
                                              topk, 2, 1, 16, 0.1, FAKE, FAKE, FAKE, 0, 8, 0, None)
    assert f(FAKE, 0) == SHAPE
    assert f(None, 64) == NULL
    assert f(FAKE, 64) == WS


def test_plan_rejects_before_launch():
    L = mla.lib()
    assert L.mla_plan(None, 2, 1, 16, 0, 8, FAKE, 1 << 30, None) == NULL
    assert L.mla_plan(FAKE, 2, 1, 16, 0, 8, None, 1 << 30, None) == WS
    assert L.mla_plan(FAKE, 0, 1, 16, 0, 8, FAKE, 1 << 30, None) == SHAPE
    assert L.mla_plan(FAKE, 2, 1, 16, 0, 8, FAKE, 16, None) == WS
    assert L.mla_plan(FAKE + 2, 2, 1, 16, 0, 8, FAKE, 1 << 30, None) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 16, 512, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mla.decode(q, torch.zeros(1, 1, 16, 64, dtype=torch.bfloat16),
                   torch.zeros(1, 64, 576, dtype=torch.bfloat16),
                   torch.zeros(1, 1, dtype=torch.int32), torch.ones(1, dtype=torch.int32), 0.1)


def _append(**kw):
    L = mla.lib()
    a = dict(new=FAKE, kv=FAKE, scales=None, dtype=0, num_pages=10, bt=FAKE, bt_stride=4,
             seqlens=FAKE, B=2, Sq=1)
    a.update(kw)
    return L.mla_kv_append(a["new"], a["kv"], a["scales"], a["dtype"], a["num_pages"], a["bt"],
                           a["bt_stride"], a["seqlens"], a["B"], a["Sq"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(new=None), NULL), (dict(kv=None), NULL), (dict(bt=None), NULL), (dict(seqlens=None), NULL),
    (dict(dtype=1), NULL),                                   # fp8 without scales
    (dict(dtype=5), SHAPE), (dict(B=0), SHAPE), (dict(Sq=0), SHAPE), (dict(num_pages=0), SHAPE),
    (dict(bt_stride=0), SHAPE), (dict(new=FAKE + 8), ALIGN), (dict(kv=FAKE + 4), ALIGN),
    (dict(dtype=1, scales=FAKE + 2), ALIGN), (dict(seqlens=FAKE + 1), ALIGN),
])
def test_append_rejects_before_launch(kw, code):
    assert _append(**kw) == code
    assert mla.lib().mla_last_error().decode() != ""


def _select(**kw):
    L = mla.lib()
    a = dict(sc=FAKE, nbk=100, sl=FAKE, B=2, Sq=1, n=16, i=1, l=2, out=FAKE)
    a.update(kw)
    return L.mla_dsa_select(a["sc"], a["nbk"], a["sl"], a["B"], a["Sq"], a["n"], a["i"], a["l"],
                            a["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(sc=None), NULL), (dict(sl=None), NULL), (dict(out=None), NULL),
    (dict(B=0), SHAPE), (dict(Sq=0), SHAPE), (dict(nbk=0), SHAPE), (dict(nbk=16385), UNSUP),
    (dict(n=0), SHAPE), (dict(n=257), SHAPE), (dict(i=-1), SHAPE), (dict(i=10, l=7), SHAPE),
    (dict(sc=FAKE + 2), ALIGN), (dict(out=FAKE + 1), ALIGN),
])
def test_select_rejects_before_launch(kw, code):
    assert _select(**kw) == code
    assert mla.lib().mla_last_error().decode() != ""


@pytest.mark.parametrize("fn", ["mla_absorb_query", "mla_project_out"])
@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, 4, 8), NULL), ((FAKE, None, FAKE, 4, 8), NULL), ((FAKE, FAKE, None, 4, 8), NULL),
    ((FAKE, FAKE, FAKE, 0, 8), SHAPE), ((FAKE, FAKE, FAKE, 4, 0), SHAPE), ((FAKE, FAKE, FAKE, 4, 70000), SHAPE),
    ((FAKE + 8, FAKE, FAKE, 4, 8), ALIGN), ((FAKE, FAKE, FAKE + 4, 4, 8), ALIGN),
])
def test_projections_reject_before_launch(fn, args, code):
    assert getattr(mla.lib(), fn)(*args, None) == code
    assert mla.lib().mla_last_error().decode() != ""


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, FAKE, 1, 64, 8, 0.1, 1, FAKE, FAKE), NULL),
    ((FAKE, FAKE, FAKE, 1, 64, 8, 0.1, 1, FAKE, None), NULL),
    ((FAKE, FAKE, FAKE, 0, 64, 8, 0.1, 1, FAKE, FAKE), SHAPE),
    ((FAKE, FAKE, FAKE, 1, 0, 8, 0.1, 1, FAKE, FAKE), SHAPE),
    ((FAKE, FAKE, FAKE, 1, 64, 0, 0.1, 1, FAKE, FAKE), SHAPE),
    ((FAKE, FAKE, FAKE, 1, 64, 8, 0.0, 1, FAKE, FAKE), SHAPE),
    ((FAKE, FAKE, FAKE, 1, 64, 8, float("nan"), 1, FAKE, FAKE), SHAPE),
    ((FAKE, FAKE, FAKE, 2, 65536, 128, 0.1, 1, FAKE, FAKE), SHAPE),   # B * T * H
    ((FAKE, FAKE, FAKE, 1, 87371, 128, 0.1, 1, FAKE, FAKE), SHAPE),   # (T + 64) * H * 384 > 2^32
    ((FAKE + 8, FAKE, FAKE, 1, 64, 8, 0.1, 1, FAKE, FAKE), ALIGN),
    ((FAKE, FAKE, FAKE, 1, 64, 8, 0.1, 1, FAKE, FAKE + 2), ALIGN),
])
def test_prefill_rejects_before_launch(args, code):
    assert mla.lib().mla_prefill(*args, None) == code
    assert mla.lib().mla_last_error().decode() != ""


def test_decode_noalloc_rejects_requests_beyond_its_scratch():
    L = mla.lib()
    f = lambda B, H, num_wg: L.mla_decode_noalloc(FAKE, FAKE, FAKE, None, 0, 10, FAKE, 4, FAKE, B,
                                                  1, H, 0.1, 0, FAKE, FAKE, num_wg, None)
    # 4096 workgroups over 64 sequences of 128 rows: about 1 GB of split partials
    assert mla.workspace_size(64, 1, 128, 0, 4096) > 96 * 1024 * 1024
    assert f(64, 128, 4096) == WS
    assert "MLA_NOALLOC_SCRATCH_BYTES" in L.mla_last_error().decode()
    assert f(64, 128, 1 << 20) == SHAPE
    assert f(0, 128, 8) == SHAPE
    # the named dense workloads fit at one workgroup per CU of a 256-CU device
    assert mla.workspace_size(64, 1, 128, 0, 256) <= 96 * 1024 * 1024
    assert mla.workspace_size(4, 1, 128, 0, 256) <= 96 * 1024 * 1024
    assert mla.workspace_size(128, 2, 16, 0, 1024) <= 96 * 1024 * 1024
