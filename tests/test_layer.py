"""GPU parity of the absorbed decode layer (mla_decode_layer, through the
C ABI): q_c -> W_UK -> dense decode -> W_UV -> o, with the split-KV schedule
run inside the absorption launch.

Reference: the oracle chain, every step from the pages' definitions --
fp64 absorption (oracle/projections.py), rounded to bf16 (the decode's q_nope
is a bf16 tensor), the C decode oracle on it, its output rounded to bf16
(the latent output is a bf16 tensor between the decode and the projection),
fp64 projection.  The layer's own roundings are the same plus fp32
accumulation, so its error is the decode's (rel-L2 <= 5e-3 on out, carried
through W_UV with rows of unit norm on average) plus one bf16 rounding of o.
Bounds: o rel-L2 <= 5e-3 over the whole tensor; per element
|o - ref| <= 2e-2 + 2^-8 |ref| (the decode's 1e-2 per element, doubled for
the sum over 512 latent dims of errors that are not independent, plus the
final rounding); lse max-abs <= 1e-3 as for the decode.

Against the same steps as separate calls (mla_absorb_query, mla_decode,
mla_project_out): the layer runs the same GEMM, scheduling, main-pass, merge
and projection code on the same inputs, so o and lse must match bit for bit.
"""
import numpy as np
import pytest
import torch

import mla_synth as S
import oracle
from oracle import projections as P

pytestmark = pytest.mark.gpu


def mla():
    import mla_latent_kv_12_amd as m
    return m


def _randn(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)


def layer_inputs(inp, seed):
    B, Sq, H = inp["B"], inp["Sq"], inp["H"]
    q_c = _randn((B, Sq, H, 128), 1.0, seed)
    w_uk_t = _randn((H, 512, 128), 512 ** -0.5, seed + 1)
    w_uv = _randn((H, 128, 512), 512 ** -0.5, seed + 2)
    return q_c, w_uk_t, w_uv


def oracle_chain(inp, q_c, w_uk_t, w_uv):
    B, Sq, H = inp["B"], inp["Sq"], inp["H"]
    qn = P.absorb_query(q_c.double().numpy().reshape(B * Sq, H, 128), w_uk_t.double().numpy())
    ref = dict(inp)
    ref["q_nope"] = _bf16(qn.reshape(B, Sq, H, 512))
    out, lse = oracle.decode(ref)
    out_b = _bf16(out).double().numpy().reshape(B * Sq, H, 512)
    o = P.project_out(out_b, w_uv.double().numpy()).reshape(B, Sq, H, 128)
    return o, lse


def check_o(o, lse, ref_o, ref_lse, what):
    got = o.float().cpu().double().numpy().reshape(-1, 128)
    ro = ref_o.reshape(-1, 128)
    gl = lse.cpu().double().numpy().reshape(-1)
    rl = ref_lse.reshape(-1)
    empty = np.isneginf(rl)
    assert np.all(np.isneginf(gl[empty])) and np.all(got[empty] == 0), f"{what}: empty rows"
    assert np.all(np.isfinite(got)), f"{what}: non-finite o"
    err = np.abs(got - ro)
    excess = (err - (2e-2 + 2.0 ** -8 * np.abs(ro))).max()
    rel = np.linalg.norm(got - ro) / max(np.linalg.norm(ro), 1e-30)
    lerr = np.abs(gl[~empty] - rl[~empty]).max() if (~empty).any() else 0.0
    print(f"{what}: rows {ro.shape[0]} o max-abs {err.max():.2e} rel-L2 {rel:.2e} lse {lerr:.2e}", flush=True)
    assert excess <= 0, f"{what}: o max-abs {err.max()} beyond the bound by {excess}"
    assert rel <= 5e-3, f"{what}: o rel-L2 {rel}"
    assert lerr <= 1e-3, f"{what}: lse max-abs {lerr}"


def run_layer(g, q_c, w_uk_t, w_uv, **kw):
    return mla().decode_layer(q_c.cuda(), w_uk_t.cuda(), g["q_rope"], w_uv.cuda(), g["kv_pages"],
                              g["block_table"], g["cache_seqlens"], g["softmax_scale"],
                              kv_scales=g["kv_scales"], causal=g["causal"], **kw)


def run_unfused(g, q_c, w_uk_t, w_uv):
    m = mla()
    q_nope = m.absorb_query(q_c.cuda(), w_uk_t.cuda())
    out, lse = m.decode(q_nope, g["q_rope"], g["kv_pages"], g["block_table"], g["cache_seqlens"],
                        g["softmax_scale"], kv_scales=g["kv_scales"], causal=g["causal"])
    return m.project_out(out, w_uv.cuda()), lse, out


def dev(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def test_layer_full_size_against_the_oracle_chain_and_unfused():
    """The dsv3_decode workload (B=64, H=128, 1K..8K tokens) at full size,
    every row; cache rows past each sequence end hold NaN."""
    inp = S.make_inputs(S.config("dsv3_decode"), unselected="nan", poison=True)
    q_c, w_uk_t, w_uv = layer_inputs(inp, 71)
    g = dev(inp)
    print("layer dsv3_decode full size", flush=True)
    o, lse = run_layer(g, q_c, w_uk_t, w_uv)
    o2, lse2, _ = run_unfused(g, q_c, w_uk_t, w_uv)
    torch.cuda.synchronize()
    assert torch.equal(lse, lse2) and torch.equal(o, o2), "layer and separate calls differ"
    ref_o, ref_lse = oracle_chain(inp, q_c, w_uk_t, w_uv)
    check_o(o, lse, ref_o, ref_lse, "layer dsv3_decode")


@pytest.mark.parametrize("kv,causal,B,Sq,H,lens,num_wg",
                         [("bf16", False, 3, 1, 128, (700, 65, 1), 0),
                          ("fp8", True, 3, 2, 20, (333, 130, 2), 0),
                          ("bf16", True, 2, 3, 64, (500, 9), 7),
                          ("bf16", False, 5, 1, 128, (0, 300, 1200, 64, 700), 300),
                          # more units than the main pass schedules itself: the
                          # schedule runs in the absorption launch
                          ("bf16", False, 2100, 1, 16, tuple((37 * i) % 150 for i in range(2100)), 0)])
def test_layer_shapes(kv, causal, B, Sq, H, lens, num_wg):
    cfg = dict(B=B, Sq=Sq, H=H, lens=("list", lens), kv=kv, shuffle=True, causal=causal, topk=0,
               name=f"layer {kv} B{B} Sq{Sq} H{H}")
    inp = S.make_inputs(cfg, seed=72, unselected="nan")
    q_c, w_uk_t, w_uv = layer_inputs(inp, 73)
    g = dev(inp)
    print(cfg["name"], f"num_wg={num_wg}", flush=True)
    o, lse = run_layer(g, q_c, w_uk_t, w_uv, num_wg=num_wg)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle_chain(inp, q_c, w_uk_t, w_uv)
    check_o(o, lse, ref_o, ref_lse, cfg["name"])


def test_layer_graph_replays_match_eager():
    inp = S.make_inputs(S.shrink("dsv3_decode"), unselected="nan")
    q_c, w_uk_t, w_uv = layer_inputs(inp, 74)
    g = dev(inp)
    m = mla()
    B, Sq, H = inp["B"], inp["Sq"], inp["H"]
    qc, wk, wv = q_c.cuda(), w_uk_t.cuda(), w_uv.cuda()
    ws = torch.empty(m.layer_workspace_size(B, Sq, H), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, Sq, H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Sq, H), dtype=torch.float32, device="cuda")

    def call():
        m.decode_layer(qc, wk, g["q_rope"], wv, g["kv_pages"], g["block_table"], g["cache_seqlens"],
                       g["softmax_scale"], o=o, lse=lse, workspace=ws)

    call()
    torch.cuda.synchronize()
    ref = (o.clone(), lse.clone())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(3):
        o.fill_(5.0)
        lse.fill_(5.0)
        m.decode(g["q_nope"], g["q_rope"], g["kv_pages"], g["block_table"], g["cache_seqlens"],
                 g["softmax_scale"])      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), f"replay {rep} differs"
