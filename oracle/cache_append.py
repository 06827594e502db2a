"""CPU oracle of the decode step's cache append (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this module; the product path never does, and nothing here imports it.

What it computes ("MLA & DSA 推理性能优化指南" §4, decode-flow figure: the
output token is appended to the cache before attention reads it; §1.1 and
§5.1: one 576-value latent row [c_KV 512 | k_rope 64] per token; §4.1 and
§5.3: about 576 bytes per token in FP8):
  * row s of sequence b goes to logical position j = L_b - Sq + s, where L_b
    counts the new tokens, i.e. to page block_table[b, j // 64], row j % 64;
    rows whose j < 0, whose logical page is past the table, or whose page
    entry is outside the pool are skipped;
  * bf16 cache: the row is stored as it is;
  * fp8 cache: scale = max|x| / 448 (1 for an all-zero row), code = e4m3fn
    round-to-nearest-even of x / scale after clamping to +-448, every
    operation in fp32 (IEEE, correctly rounded).

The e4m3fn encoder is written from the format's definition (OCP FP8 E4M3:
1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
infinities, S.1111.111 = NaN): a value maps to the nearest finite code
value, a tie to the code whose last mantissa bit is 0.
"""
from __future__ import annotations

import numpy as np

PAGE = 64
DLAT = 576
E4M3_MAX = np.float32(448.0)


def e4m3fn_value(code: int) -> float:
    """Real value of an e4m3fn code (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# the 127 non-negative finite magnitudes, indexed by code 0x00..0x7E
_POS = np.array([e4m3fn_value(c) for c in range(0x7F)], dtype=np.float64)


def e4m3fn_encode(v) -> np.ndarray:
    """Nearest e4m3fn code of each float32 value with |v| <= 448 (ties to even).

    Brute force over the 127 magnitudes: the nearest one wins; of two equally
    near, the one with an even code (mantissa LSB 0).  The sign bit is the
    value's sign bit (so -0.0 gives 0x80)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v.astype(np.float64)).reshape(-1)
    if np.any(~np.isfinite(a)) or np.any(a > 448.0):
        raise ValueError("e4m3fn_encode expects finite values with |v| <= 448")
    d = np.abs(a[:, None] - _POS[None, :])               # [n, 127]
    best = d.min(axis=1, keepdims=True)
    cand = d == best                                     # one or two nearest codes
    codes = np.arange(0x7F)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    sign = np.signbit(v.reshape(-1)).astype(np.int64) << 7
    return (pick | sign).astype(np.uint8).reshape(v.shape)


def quantize_row(x) -> tuple[np.ndarray, np.float32]:
    """(codes uint8 [576], scale float32) of one latent row given as float32."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    scale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    q = np.clip(x / scale, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    return e4m3fn_encode(q), scale


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) as float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def kv_append(kv_pages, kv_scales, new_kv_bits, block_table, cache_seqlens, fp8: bool):
    """Cache after the append, as new arrays (inputs are left unchanged).

    kv_pages    uint16 [P, 64, 576] bf16 bits, or uint8 [P, 64, 576] codes
    kv_scales   float32 [P, 64] (fp8) or None
    new_kv_bits uint16 [B, Sq, 576] bf16 bits
    block_table int32 [B, stride]; cache_seqlens int32 [B]
    Returns (kv_pages', kv_scales')."""
    kv = np.array(kv_pages, copy=True)
    sc = None if kv_scales is None else np.array(kv_scales, copy=True)
    B, Sq, _ = new_kv_bits.shape
    P = kv.shape[0]
    stride = block_table.shape[1]
    for b in range(B):
        for s in range(Sq):
            j = int(cache_seqlens[b]) - Sq + s
            if j < 0 or j // PAGE >= stride:
                continue
            page = int(block_table[b, j // PAGE])
            if page < 0 or page >= P:
                continue
            row = j % PAGE
            if fp8:
                codes, scale = quantize_row(bf16_bits_to_f32(new_kv_bits[b, s]))
                kv[page, row] = codes
                sc[page, row] = scale
            else:
                kv[page, row] = new_kv_bits[b, s]
    return kv, sc
