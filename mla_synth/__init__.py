"""Seeded synthetic inputs for weight-absorbed MLA decode.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through its binding) and the CPU
oracle consume what it produces, so it is the one piece they share.

Shapes follow the DeepSeek-V3 MLA configuration that the pages use
("MLA & DSA 推理性能优化指南", §5.1 parameter table: d_c = 512, d_rope = 64,
128 heads): each cached token is one 576-element latent row
[c_KV (512) | k_rope (64)], stored in pages of 64 tokens.

Layout produced (all torch CPU tensors):
  q_nope        bf16  [B, Sq, H, 512]   absorbed query (q^C W_UK)
  q_rope        bf16  [B, Sq, H, 64]    decoupled-RoPE query
  kv_pages      bf16  [P, 64, 576]  or  uint8 [P, 64, 576] holding e4m3fn codes
  kv_scales     fp32  [P, 64]           one scale per token (fp8 only, else None)
  block_table   int32 [B, max_pages]    physical page of logical page; -1 pads
  cache_seqlens int32 [B]               tokens in the cache, new tokens included
  indices       int32 [B, Sq, topk]     sparse path only (else None); -1 pads
"""
from __future__ import annotations

import math

import torch

D_C = 512
D_ROPE = 64
D_LATENT = D_C + D_ROPE
PAGE = 64
E4M3_MAX = 448.0

# bf16 quiet NaN and e4m3fn NaN bit patterns used to poison unused cache rows.
BF16_NAN_BITS = 0x7FC0
E4M3_NAN_BITS = 0x7F

# The five workloads the pages' DeepSeek-V3 shapes call for (d_c 512, d_rope 64,
# 128 heads, 64-token pages).  "seed" is the default seed for each.
CONFIGS = {
    "tiny": dict(B=1, Sq=1, H=16, lens=("fixed", 256), kv="bf16", shuffle=False,
                 causal=False, topk=0, seed=1),
    "dsv3_decode": dict(B=64, Sq=1, H=128, lens=("uniform", 1024, 8192), kv="bf16",
                        shuffle=True, causal=False, topk=0, seed=2),
    "long_context": dict(B=4, Sq=1, H=128, lens=("fixed", 131072), kv="bf16",
                         shuffle=True, causal=False, topk=0, seed=3),
    "fp8_head_slice": dict(B=128, Sq=2, H=16, lens=("fixed", 4096), kv="fp8",
                           shuffle=True, causal=True, topk=0, seed=4),
    # dsv3_decode with every sequence at the 8K maximum (a supplementary size)
    "dsv3_decode_max": dict(B=64, Sq=1, H=128, lens=("fixed", 8192), kv="bf16",
                            shuffle=True, causal=False, topk=0, seed=6),
    "dsa_sparse": dict(B=32, Sq=1, H=128, lens=("fixed", 65536), kv="bf16",
                       shuffle=True, causal=False, topk=1024, seed=5,
                       sel_blocks=16, init_blocks=1, local_blocks=2),
}

DEFAULT_SCALE = 1.0 / math.sqrt(192.0)


def config(name: str, **overrides) -> dict:
    cfg = dict(CONFIGS[name])
    cfg["name"] = name
    cfg.update(overrides)
    return cfg


def _lengths(cfg: dict, g: torch.Generator) -> torch.Tensor:
    spec = cfg["lens"]
    B = cfg["B"]
    if spec[0] == "fixed":
        return torch.full((B,), int(spec[1]), dtype=torch.int32)
    if spec[0] == "uniform":  # integers uniform in [lo, hi], both ends included
        return torch.randint(int(spec[1]), int(spec[2]) + 1, (B,), generator=g,
                             dtype=torch.int64).to(torch.int32)
    if spec[0] == "list":
        t = torch.tensor(list(spec[1]), dtype=torch.int32)
        assert t.numel() == B
        return t
    raise ValueError(f"unknown length spec {spec!r}")


def _randn_bf16(shape, g: torch.Generator, chunk_rows: int = 1 << 14) -> torch.Tensor:
    """N(0,1) drawn in fp32 then rounded (RNE) to bf16, generated in row chunks."""
    out = torch.empty(shape, dtype=torch.bfloat16)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=g).to(torch.bfloat16)
    return out


def _randn_e4m3(shape, g: torch.Generator, chunk_rows: int = 1 << 12):
    """N(0,1) values stored as e4m3fn codes with one fp32 scale per token row.

    scale = max|x| / 448 over the token's 576 values (1 when the row is all
    zero); code = RNE(x / scale) after clamping to +-448.
    """
    P = shape[0]
    codes = torch.empty(shape, dtype=torch.uint8)
    scales = torch.empty((P, shape[1]), dtype=torch.float32)
    for r0 in range(0, P, chunk_rows):
        r1 = min(P, r0 + chunk_rows)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g)
        amax = x.abs().amax(dim=-1)
        sc = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
        q = (x / sc.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        codes[r0:r1] = q.view(torch.uint8)
        scales[r0:r1] = sc
    return codes, scales


def _sparse_indices(cfg: dict, lens: torch.Tensor, g: torch.Generator) -> torch.Tensor:
    """Block-aligned top-k lists shaped like the pages' DSA selection.

    Per (b, s): `sel_blocks` distinct 64-token blocks: the first
    `init_blocks` blocks, the last `local_blocks` blocks before L, and the
    rest drawn without replacement from the blocks in between; ascending.
    """
    B, Sq, topk = cfg["B"], cfg["Sq"], cfg["topk"]
    nsel = cfg.get("sel_blocks", topk // PAGE)
    n_init = cfg.get("init_blocks", 1)
    n_local = cfg.get("local_blocks", 2)
    assert nsel * PAGE == topk, "topk must be sel_blocks * 64"
    idx = torch.full((B, Sq, topk), -1, dtype=torch.int32)
    for b in range(B):
        nb = int(lens[b]) // PAGE  # whole blocks available
        for s in range(Sq):
            if nb <= nsel:
                blocks = torch.arange(nb)
            else:
                fixed = list(range(n_init)) + list(range(nb - n_local, nb))
                middle = torch.arange(n_init, nb - n_local)
                pick = middle[torch.randperm(middle.numel(), generator=g)[: nsel - len(fixed)]]
                blocks = torch.sort(torch.cat([torch.tensor(fixed), pick])).values
            tok = (blocks.view(-1, 1) * PAGE + torch.arange(PAGE).view(1, -1)).reshape(-1)
            idx[b, s, : tok.numel()] = tok.to(torch.int32)
    return idx


def make_inputs(cfg: dict, seed: int | None = None, poison: bool = True,
                unselected: str = "randn") -> dict:
    """Draw one seeded input set for `cfg` (a dict from `config`).

    poison:     rows at or past each sequence's length inside its last page
                are set to NaN (bf16 NaN, e4m3fn NaN code and NaN scale), so
                any read of them shows up in the result.
    unselected: sparse configs only. "randn" fills every page with N(0,1);
                "nan" fills only pages holding selected tokens and poisons
                the rest (much cheaper for large pools).
    """
    if seed is None:
        seed = cfg["seed"]
    g = torch.Generator().manual_seed(int(seed))
    B, Sq, H = cfg["B"], cfg["Sq"], cfg["H"]
    lens = _lengths(cfg, g)
    npages = [(int(L) + PAGE - 1) // PAGE for L in lens]
    P = sum(npages)
    maxp = max(max(npages), 1)
    perm = torch.randperm(P, generator=g) if cfg.get("shuffle", True) else torch.arange(P)
    bt = torch.full((B, maxp), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        bt[b, : npages[b]] = perm[off: off + npages[b]].to(torch.int32)
        off += npages[b]

    q_nope = _randn_bf16((B, Sq, H, D_C), g)
    q_rope = _randn_bf16((B, Sq, H, D_ROPE), g)

    topk = int(cfg.get("topk", 0))
    indices = _sparse_indices(cfg, lens, g) if topk > 0 else None

    fp8 = cfg["kv"] == "fp8"
    shape = (max(P, 1), PAGE, D_LATENT)
    if topk > 0 and unselected == "nan":
        used = torch.zeros(shape[0], dtype=torch.bool)
        for b in range(B):
            sel = indices[b][indices[b] >= 0].unique()
            used[bt[b, (sel // PAGE).long()].long()] = True
        if fp8:
            kv = torch.full(shape, E4M3_NAN_BITS, dtype=torch.uint8)
            scales = torch.full(shape[:2], float("nan"), dtype=torch.float32)
            c, s = _randn_e4m3((int(used.sum()),) + shape[1:], g)
            kv[used], scales[used] = c, s
        else:
            kv = torch.full(shape, BF16_NAN_BITS, dtype=torch.int16).view(torch.bfloat16)
            kv[used] = _randn_bf16((int(used.sum()),) + shape[1:], g)
            scales = None
    elif fp8:
        kv, scales = _randn_e4m3(shape, g)
    else:
        kv, scales = _randn_bf16(shape, g), None

    if poison:
        for b in range(B):
            L = int(lens[b])
            r = L % PAGE
            if npages[b] > 0 and r != 0:
                p = int(bt[b, npages[b] - 1])
                if fp8:
                    kv[p, r:] = E4M3_NAN_BITS
                    scales[p, r:] = float("nan")
                else:
                    kv.view(torch.int16)[p, r:] = BF16_NAN_BITS

    return dict(
        q_nope=q_nope, q_rope=q_rope, kv_pages=kv, kv_scales=scales,
        kv_dtype="fp8" if fp8 else "bf16", block_table=bt, cache_seqlens=lens,
        indices=indices, topk=topk, softmax_scale=float(cfg.get("softmax_scale", DEFAULT_SCALE)),
        causal=bool(cfg.get("causal", False)), B=B, Sq=Sq, H=H, seed=int(seed),
        name=cfg.get("name", "custom"),
    )


def shrink(name: str, **over) -> dict:
    """A small version of a named workload that the oracle finishes in seconds."""
    small = {
        "tiny": dict(),
        "dsv3_decode": dict(B=3, lens=("uniform", 1, 700)),
        "long_context": dict(B=2, lens=("fixed", 1500)),
        "fp8_head_slice": dict(B=4, lens=("fixed", 333)),
        "dsa_sparse": dict(B=2, lens=("fixed", 2048), topk=512, sel_blocks=8),
        "dsv3_decode_max": dict(B=2, lens=("fixed", 640)),
    }[name]
    small.update(over)
    return config(name, **small)
