"""GPU parity of the per-head projections (mla_absorb_query, mla_project_out,
through the C ABI) against the fp64 oracle in oracle/projections.py.

Inputs are bf16, products are exact in fp32 and the sums are accumulated in
fp32, so the GPU result is the exact product rounded once to bf16 up to a
summation error far below that rounding: each element must be within one
bf16 step of the reference, 2^-8 |ref|, plus 1e-5 for values near zero.
"""
import numpy as np
import pytest
import torch

from oracle import projections as P

pytestmark = pytest.mark.gpu


def mla():
    import mla_latent_kv_12_amd as m
    return m


def _randn(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _close(got, ref, what):
    got = got.float().cpu().double().numpy()
    excess = np.abs(got - ref) - (2.0 ** -8 * np.abs(ref) + 1e-5)
    assert excess.max() <= 0, f"{what}: worst excess {excess.max():.3e}"


@pytest.mark.parametrize("M,H", [(64, 128), (256, 16), (77, 128), (1, 3), (130, 5)])
def test_absorb_query(M, H):
    q = _randn((M, H, 128), 1.0, 31 + M)
    w = _randn((H, 512, 128), 512 ** -0.5, 32 + H)
    print(f"absorb M={M} H={H}", flush=True)
    got = mla().absorb_query(q.cuda(), w.cuda())
    torch.cuda.synchronize()
    _close(got, P.absorb_query(q.double().numpy(), w.double().numpy()), f"absorb M={M} H={H}")


@pytest.mark.parametrize("M,H", [(64, 128), (256, 16), (77, 128), (1, 3), (130, 5)])
def test_project_out(M, H):
    x = _randn((M, H, 512), 1.0, 41 + M)
    w = _randn((H, 128, 512), 512 ** -0.5, 42 + H)
    print(f"project M={M} H={H}", flush=True)
    got = mla().project_out(x.cuda(), w.cuda())
    torch.cuda.synchronize()
    _close(got, P.project_out(x.double().numpy(), w.double().numpy()), f"project M={M} H={H}")


def test_absorbed_layer_on_the_gpu_matches_the_oracle_chain():
    """absorb -> decode -> project on the GPU against the same chain in the
    oracle (fp64 absorb, C decode oracle on the bf16-rounded q_nope the GPU
    produced, fp64 projection of the GPU's bf16 decode output)."""
    import mla_synth as S
    import oracle
    from test_parity import check
    inp = S.make_inputs(S.shrink("dsv3_decode"), poison=False)
    B, H = inp["B"], inp["H"]
    q_c = _randn((B, 1, H, 128), 1.0, 51)
    w_uk_t = _randn((H, 512, 128), 512 ** -0.5, 52)
    w_uv = _randn((H, 128, 512), 512 ** -0.5, 53)
    g = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    m = mla()
    q_nope = m.absorb_query(q_c.cuda(), w_uk_t.cuda())
    out, lse = m.decode(q_nope, g["q_rope"], g["kv_pages"], g["block_table"], g["cache_seqlens"],
                        g["softmax_scale"])
    o = m.project_out(out, w_uv.cuda())
    torch.cuda.synchronize()
    _close(q_nope, P.absorb_query(q_c.double().numpy().reshape(B, H, 128),
                                  w_uk_t.double().numpy()).reshape(B, 1, H, 512), "chain absorb")
    ref = dict(inp)
    ref["q_nope"] = q_nope.cpu()
    ref_out, ref_lse = oracle.decode(ref)
    check(out, lse, ref_out, ref_lse, what="chain decode")
    _close(o, P.project_out(out.float().cpu().double().numpy().reshape(B, H, 512),
                            w_uv.double().numpy()).reshape(B, 1, H, 128), "chain project")
