"""A whole absorbed decode layer captured as one HIP graph: query absorption,
cache append, DSA block selection, sparse decode and output projection, plus
a prefill, all through the C ABI.  None of these calls allocates,
synchronises or enqueues a memset, so they capture as they are; every replay
(with eager work and synchronisations in between) must reproduce the eager
result bit for bit, and the eager result must match the oracles.
"""
import numpy as np
import pytest
import torch

import mla_synth as S
import oracle
from oracle import cache_append as C
from oracle import dsa_select as D
from oracle import prefill as PF
from oracle import projections as P

pytestmark = pytest.mark.gpu


def mla():
    import mla_latent_kv_12_amd as m
    return m


def _rand(shape, seed, std=1.0):
    return (torch.randn(shape, generator=torch.Generator().manual_seed(seed)) * std).to(torch.bfloat16)


def test_layer_graph_replays_match_eager_and_oracles():
    from test_parity import check
    m = mla()
    inp = S.make_inputs(S.shrink("dsa_sparse"), poison=False)
    B, H = inp["B"], inp["H"]
    n_sel = inp["topk"] // 64
    nbk = int(inp["block_table"].shape[1])
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    kv0 = g["kv_pages"].clone()
    q_c = _rand((B, 1, H, 128), 61).cuda()
    w_uk_t = _rand((H, 512, 128), 62, 512 ** -0.5).cuda()
    w_uv = _rand((H, 128, 512), 63, 512 ** -0.5).cuda()
    new = _rand((B, 1, 576), 64).cuda()
    scores = torch.randn((B, 1, nbk), generator=torch.Generator().manual_seed(65)).cuda()
    pq, pk, pv = _rand((1, 100, 3, 192), 66).cuda(), _rand((1, 100, 3, 192), 67).cuda(), _rand((1, 100, 3, 128), 68).cuda()
    ws = m.alloc_workspace(B, 1, H, inp["topk"])
    q_nope = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, 1, inp["topk"]), dtype=torch.int32, device="cuda")
    out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, 1, H), dtype=torch.float32, device="cuda")
    o = torch.empty((B, 1, H, 128), dtype=torch.bfloat16, device="cuda")
    pout = torch.empty((1, 100, 3, 128), dtype=torch.bfloat16, device="cuda")
    plse = torch.empty((1, 100, 3), dtype=torch.float32, device="cuda")

    def layer():
        g["kv_pages"].copy_(kv0)          # a kernel copy (no memset): same cache every time
        m.absorb_query(q_c, w_uk_t, out=q_nope)
        m.kv_append(new, g["kv_pages"], g["block_table"], g["cache_seqlens"])
        m.dsa_select(scores, g["cache_seqlens"], n_select=n_sel, indices=idx)
        m.sparse_decode(q_nope, g["q_rope"], g["kv_pages"], g["block_table"], g["cache_seqlens"], idx,
                        g["softmax_scale"], out=out, lse=lse, workspace=ws)
        m.project_out(out, w_uv, out=o)
        m.prefill(pq, pk, pv, 1 / np.sqrt(192), out=pout, lse=plse)

    print("layer eager", flush=True)
    layer()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (q_nope, idx, out, lse, o, pout, plse)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    for rep in range(3):
        for t in (q_nope, out, o, pout):
            t.fill_(3.0)
        idx.fill_(-7)
        lse.fill_(3.0)
        plse.fill_(3.0)
        m.decode(g["q_nope"], g["q_rope"], g["kv_pages"], g["block_table"], g["cache_seqlens"],
                 g["softmax_scale"])      # eager work between replays
        torch.cuda.synchronize()
        print(f"replay {rep}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((q_nope, idx, out, lse, o, pout, plse), ref):
            assert torch.equal(a, b), f"replay {rep} differs"

    # the eager result against the oracles, step by step
    qn_ref = P.absorb_query(q_c.cpu().double().numpy().reshape(B, H, 128), w_uk_t.cpu().double().numpy())
    got = q_nope.float().cpu().double().numpy().reshape(B, H, 512)
    assert np.all(np.abs(got - qn_ref) <= 2.0 ** -8 * np.abs(qn_ref) + 1e-5)
    want_idx = D.select(scores.cpu().numpy(), inp["cache_seqlens"].numpy(), 1, n_sel, 1, 2)
    assert np.array_equal(idx.cpu().numpy(), want_idx)
    bits = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
    kv2, _ = C.kv_append(bits(inp["kv_pages"]), None, bits(new.cpu()), inp["block_table"].numpy(),
                         inp["cache_seqlens"].numpy(), False)
    dec = dict(inp)
    dec["kv_pages"] = torch.from_numpy(kv2.view(np.int16)).view(torch.bfloat16)
    dec["q_nope"] = q_nope.cpu()
    ro, rl = oracle.decode(dec, indices=torch.from_numpy(want_idx))
    check(out, lse, ro, rl, what="layer sparse decode")
    po_ref = P.project_out(out.float().cpu().double().numpy().reshape(B, H, 512), w_uv.cpu().double().numpy())
    got_o = o.float().cpu().double().numpy().reshape(B, H, 128)
    assert np.all(np.abs(got_o - po_ref) <= 2.0 ** -8 * np.abs(po_ref) + 1e-5)
    pr, pl = PF.prefill(pq.cpu().double().numpy(), pk.cpu().double().numpy(), pv.cpu().double().numpy(),
                        1 / np.sqrt(192), True)
    assert np.abs(pout.float().cpu().double().numpy() - pr).max() <= 1e-2
    assert np.abs(plse.cpu().double().numpy() - pl).max() <= 1e-3
