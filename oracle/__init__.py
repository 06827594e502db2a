"""CPU oracle for weight-absorbed MLA decode (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never
imports, links or executes anything here, and nothing here imports the
product.

Two independent implementations of the same definition:
  * `decode`          -- C, fp64, threaded over query rows (mla_oracle.c)
  * `ref_numpy`       -- NumPy fp64, vectorised over tokens, tiny inputs only
plus NumPy helpers that pin the definition to the pages:
  * `ref_numpy.mha_nonabsorbed` -- the un-absorbed computation over
    decompressed K/V, for the absorption identity.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "mla_oracle.c")

_lib = None


def build(force: bool = False) -> str:
    """Compile mla_oracle.c into liboracle.so with gcc."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-std=c99",
                               "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_mla_decode.restype = ctypes.c_int
        L.oracle_mla_decode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_long,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.oracle_e4m3fn_to_double.restype = ctypes.c_double
        L.oracle_e4m3fn_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_kv_bytes_per_token.restype = ctypes.c_long
        L.oracle_kv_bytes_per_token.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def default_threads() -> int:
    """Worker threads for the oracle: OMP_NUM_THREADS when set (the CPU share
    a job is given), else every core this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = int(env)
    else:
        try:
            n = len(os.sched_getaffinity(0))
        except AttributeError:
            n = os.cpu_count() or 1
    return max(1, min(n, 256))


def _np(t, dtype):
    """Contiguous numpy view of a CPU tensor / array with the given raw dtype."""
    import torch
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        elif t.dtype == torch.float8_e4m3fn:
            t = t.view(torch.uint8)
        t = t.numpy()
    return np.ascontiguousarray(t).view(dtype)


def e4m3fn_to_double(code: int) -> float:
    return lib().oracle_e4m3fn_to_double(code)


def kv_bytes_per_token(bytes_per_element: int) -> int:
    return lib().oracle_kv_bytes_per_token(bytes_per_element)


def decode(inp: dict, rows=None, nthreads: int | None = None, indices=None, causal=None):
    """Oracle outputs for an input dict from `mla_synth.make_inputs`.

    rows: None for every (b, s, h) row, else an iterable of flat row ids
          b*Sq*H + s*H + h.  Returns (out, lse): out float64 [n, 512] and
          lse [n] for listed rows, or [B, Sq, H, 512] / [B, Sq, H] for all.
    indices: override of inp["indices"] (None keeps it; False forces dense).
    """
    B, Sq, H = inp["B"], inp["Sq"], inp["H"]
    if indices is None:
        indices = inp.get("indices")
    elif indices is False:
        indices = None
    causal = inp["causal"] if causal is None else causal
    qn = _np(inp["q_nope"], np.uint16)
    qr = _np(inp["q_rope"], np.uint16)
    fp8 = inp["kv_dtype"] == "fp8"
    kv = _np(inp["kv_pages"], np.uint8 if fp8 else np.uint16)
    sc = _np(inp["kv_scales"], np.float32) if fp8 else None
    bt = _np(inp["block_table"], np.int32)
    sl = _np(inp["cache_seqlens"], np.int32)
    ix = _np(indices, np.int32) if indices is not None else None
    topk = int(ix.shape[-1]) if ix is not None else 0
    if rows is None:
        r = None
        n = B * Sq * H
    else:
        r = np.ascontiguousarray(np.asarray(list(rows), dtype=np.int64))
        n = r.size
    out = np.zeros((n, 512), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    if nthreads is None:
        nthreads = default_threads()
    ptr = lambda a: None if a is None else a.ctypes.data
    rc = lib().oracle_mla_decode(
        ptr(qn), ptr(qr), ptr(kv), ptr(sc), int(fp8), int(kv.shape[0]), ptr(bt), int(bt.shape[1]),
        ptr(sl), B, Sq, H, float(inp["softmax_scale"]), int(bool(causal)), ptr(ix), topk,
        ptr(r), int(n), ptr(out), ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_mla_decode rejected its arguments")
    if rows is None:
        return out.reshape(B, Sq, H, 512), lse.reshape(B, Sq, H)
    return out, lse
