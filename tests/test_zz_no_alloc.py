"""mla_decode_noalloc (through the C ABI) against mla_decode.

The no-allocation entry point runs the same kernels with the library's static
workspace instead of a caller-supplied one, so its results must equal
mla_decode's bit for bit; they are also held to the oracle bound.  Two calls
in a row, the second on a smaller input, check that nothing a previous call
left in the shared array leaks into the next.
"""
import numpy as np
import pytest
import torch

import mla_synth as S
import oracle

pytestmark = pytest.mark.gpu


def mla():
    import mla_latent_kv_12_amd as m
    return m


def _dev(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _both(inp):
    g = _dev(inp)
    m = mla()
    args = (g["q_nope"], g["q_rope"], g["kv_pages"], g["block_table"], g["cache_seqlens"],
            g["softmax_scale"])
    kw = dict(kv_scales=g["kv_scales"], causal=g["causal"])
    ref = m.decode(*args, **kw)
    got = m.decode_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return ref, got


def _case(B, Sq, H, lens, kv, causal, seed):
    cfg = dict(B=B, Sq=Sq, H=H, lens=("list", tuple(lens)), kv=kv, shuffle=True, causal=causal,
               topk=0, name=f"noalloc B{B} Sq{Sq} H{H} {kv}")
    return S.make_inputs(cfg, seed=seed)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_equals_decode_two_calls_second_smaller(kv):
    from test_parity import check, visible_counts
    first = _case(6, 1, 128, (3000, 70, 1800, 4100, 640, 1), kv, False, 41)
    second = _case(2, 2, 16, (500, 129), kv, True, 42)
    for inp in (first, second):
        print(f"{inp['name']} lens {inp['cache_seqlens'].tolist()}", flush=True)
        (ro, rl), (go, gl) = _both(inp)
        assert torch.equal(go, ro) and torch.equal(gl, rl), "noalloc differs from mla_decode"
        want = oracle.decode(inp)
        check(go, gl, want[0], want[1], inp["name"] + " noalloc", nvis=visible_counts(inp))


@pytest.mark.parametrize("name", ["dsv3_decode", "fp8_head_slice"])
def test_noalloc_full_size_workload(name):
    inp = S.make_inputs(S.config(name))
    print(f"{name} noalloc", flush=True)
    (ro, rl), (go, gl) = _both(inp)
    assert torch.equal(go, ro) and torch.equal(gl, rl), "noalloc differs from mla_decode"


def test_noalloc_rejects_requests_beyond_the_scratch():
    m = mla()
    inp = _dev(_case(64, 1, 128, (100,) * 64, "bf16", False, 43))
    need = m.workspace_size(64, 1, 128, 0, 4096)
    assert need > 96 * 1024 * 1024
    out = torch.full((64, 1, 128, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(m.MLAError) as e:
        m.decode_noalloc(inp["q_nope"], inp["q_rope"], inp["kv_pages"], inp["block_table"],
                         inp["cache_seqlens"], inp["softmax_scale"], out=out, num_wg=4096)
    assert e.value.status == 5  # MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all()), "a rejected call must not touch out"
